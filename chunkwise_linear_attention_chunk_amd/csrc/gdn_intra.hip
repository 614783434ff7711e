// Kernel (a): per (chunk, value head) -- chunk-local gate cumsum, gated beta*K K^T on the
// matrix cores and the exact inverse A = (I + strictLower(diag(beta)(Gamma (.) K K^T)))^{-1};
// with per-channel gates also the output's intra-chunk matrix P = scale Lower(Gamma) (.) Q K^T
// (with a scalar gate the recurrence kernel forms P itself from the Q and K tiles it holds).
//
// Sources: 06 . Flash Linear Attention, section 3 (chunk-local cumsum of log-gates, exp2 of
// pre-scaled differences) and section 4 (solve_tril: forward substitution inside 16x16
// diagonal blocks, row i absorbing the rows above it, then the exact block-triangular merge
// inv([[I+A00, 0], [A10, I+A11]]) = [[A00i, 0], [-A11i A10 A00i, A11i]] from 16 to 32 to 64);
// FlashQLA announcement (Qwen), the first step of the chunk-i forward.
//
// The inverse is computed in fp32 throughout (the pages use tf32 dots for the merges; gfx950
// has no tf32 path, so the merges run on fp32 MFMA).  With a scalar gate A is stored in the input
// dtype; with per-channel gates A and P are stored as fp16 for bf16 inputs, fp32 for fp32 inputs.
//
// One workgroup of 256 threads (4 waves) per (chunk, head); many workgroups per CU hide the
// latency of the serial 16-step substitutions.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

// Exact inverse of the unit lower triangular I + L (L strictly lower, fp32 [64][LP] in LDS) into X
// (same layout, strictly lower part only): forward substitution inside the four 16x16 diagonal
// blocks, then the block-triangular merges 16 -> 32 -> 64 on fp32 MFMA.  X may be L itself: each
// block of X is written only after every read of the L block at its place.  Called by all 256
// threads with L complete and visible; returns after a barrier, X complete.
__device__ __forceinline__ void invert_unit_lower(const float *sL, float *sX) {
    constexpr int LP = 64 + 4;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, grp = lane >> 4;
    // ---- inverses of the four 16x16 diagonal blocks, all in wave 0 (the other waves would repeat
    //      its vector work on idle lanes): lane group grp takes block grp, lane l16 its column c;
    //      row i absorbs the rows above it.  The lanes of a group read the same L element.
    if (wave == 0) {
        const float *L = sL + (16 * grp) * LP + 16 * grp;
        const int c = l16;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s = (i == c) ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < i; ++j) s -= L[i * LP + j] * x[j];
            x[i] = s;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sX[(16 * grp + i) * LP + 16 * grp + c] = x[i];
    }
    __syncthreads();

    // ---- 16 -> 32: Ai[b+1][b] = -D_{b+1} L_{b+1,b} D_b for b = 0 (wave 0) and b = 2 (wave 1)
    if (wave < 2) {
        const int b = 2 * wave;
        f32x4 tt = {0.f, 0.f, 0.f, 0.f}, oo = {0.f, 0.f, 0.f, 0.f};
        mm16_f32_lds(tt, sL + 16 * (b + 1) * LP + 16 * b, LP, sX + 16 * b * LP + 16 * b, LP);
        mm16_f32_regB(oo, sX + 16 * (b + 1) * LP + 16 * (b + 1), LP, tt);
#pragma unroll
        for (int r = 0; r < 4; ++r) sX[(16 * (b + 1) + 4 * grp + r) * LP + 16 * b + l16] = -oo[r];
    }
    __syncthreads();

    // ---- 32 -> 64: lower-left 32x32 block = -Ai_BB L_BA Ai_AA; wave w builds tile (2 + w/2, w%2)
    {
        const int I = 2 + (wave >> 1), J = wave & 1;
        auto Lt = [&](int a, int b) { return sL + 16 * a * LP + 16 * b; };
        auto Xt = [&](int a, int b) { return sX + 16 * a * LP + 16 * b; };
        // T[Ip][J] = L[Ip][0] AiAA[0][J] + L[Ip][1] AiAA[1][J]   (AiAA[0][1] = 0)
        auto tcalc = [&](int Ip) {
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
            if (J == 0) {
                mm16_f32_lds(t, Lt(Ip, 0), LP, Xt(0, 0), LP);
                mm16_f32_lds(t, Lt(Ip, 1), LP, Xt(1, 0), LP);
            } else {
                mm16_f32_lds(t, Lt(Ip, 1), LP, Xt(1, 1), LP);
            }
            return t;
        };
        const f32x4 T2 = tcalc(2);
        f32x4 oo = {0.f, 0.f, 0.f, 0.f};
        if (I == 2) {
            mm16_f32_regB(oo, Xt(2, 2), LP, T2);
        } else {
            const f32x4 T3 = tcalc(3);
            mm16_f32_regB(oo, Xt(3, 2), LP, T2);
            mm16_f32_regB(oo, Xt(3, 3), LP, T3);
        }
        __syncthreads();  // every wave has read L's lower-left blocks (X may overwrite them)
#pragma unroll
        for (int r = 0; r < 4; ++r) sX[(16 * I + 4 * grp + r) * LP + 16 * J + l16] = -oo[r];
    }
    __syncthreads();
}

// Store the inverse as the unit lower triangular A (zero above the diagonal) in the input dtype,
// [64][64] row-major at A.  X's 16x16 tiles on and below the diagonal are the inverse itself (the
// diagonal tiles come out of the substitution with exact ones on the diagonal and exact zeros above
// it); the tiles above the diagonal hold stale data and are written as zeros.
template <typename T>
__device__ __forceinline__ void store_unit_lower(const float *sX, T *A) {
    constexpr int VEC = Vec16<T>::N, LP = 64 + 4;
#pragma unroll
    for (int it = 0; it < 64 * 64 / VEC / 256; ++it) {
        const int idx = threadIdx.x + 256 * it;
        const int row = idx / (64 / VEC), c0 = (idx - row * (64 / VEC)) * VEC;
        u32x4 out = {0u, 0u, 0u, 0u};
        if ((c0 >> 4) <= (row >> 4)) {             // a tile on or below the diagonal
            T vals[VEC];
#pragma unroll
            for (int e = 0; e < VEC; e += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(sX + row * LP + c0 + e);
                vals[e] = from_f32<T>(v.x); vals[e + 1] = from_f32<T>(v.y);
                vals[e + 2] = from_f32<T>(v.z); vals[e + 3] = from_f32<T>(v.w);
            }
            out = *reinterpret_cast<const u32x4 *>(vals);
        }
        *reinterpret_cast<u32x4 *>(A + row * 64 + c0) = out;
    }
}

// Scalar gate: A and the gate block.  Only K (and later the inverse) and A_raw use LDS.
template <typename T, int DK>
__global__ __launch_bounds__(256) void intra_kernel(IntraParams p) {
    constexpr int VEC = Vec16<T>::N;
    constexpr int KP = DK + VEC;   // row stride of the K tile (padded against bank conflicts)
    constexpr int LP = 64 + 4;     // row stride of the fp32 64x64 tiles
    constexpr int K_BYTES = 64 * KP * (int)sizeof(T);
    constexpr int X_BYTES = 64 * LP * 4;
    constexpr int R0 = K_BYTES > X_BYTES ? K_BYTES : X_BYTES;
    constexpr int NKB = DK / 32;
    // one region: the K tile, then A_raw, then its inverse X in place (a small footprint keeps
    // eight workgroups on a CU to hide each one's serial latency)
    __shared__ __attribute__((aligned(16))) unsigned char smem[R0];
    __shared__ float sGl[64], sB[64], sRk[64], sRq[64];
    T *sK = reinterpret_cast<T *>(smem);
    float *sX = reinterpret_cast<float *>(smem);
    float *sL = sX;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, grp = lane >> 4;
    const int cg = blockIdx.x / p.H_v, h = blockIdx.x - cg * p.H_v;
    const int ci = piece_chunk(cg, p.T, p.piece_lo, p.piece_cnt);
    const int hq = h / (p.H_v / p.H_qk);
    const ChunkInfo cinfo = chunk_info(p.chunks, ci, p.T);
    const int t0 = cinfo.tok0, nv = cinfo.nv;
    const T *k = static_cast<const T *>(p.k);
    const float *g = static_cast<const float *>(p.g);
    const T *beta = static_cast<const T *>(p.beta);

    // this wave's lower tiles t = wave, wave + 4, wave + 8 (< 10): (ti, tj) with tj <= ti
    constexpr int NT = 3;
    int TI[NT], TJ[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int t = wave + 4 * n;
        TI[n] = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
        TJ[n] = t - TI[n] * (TI[n] + 1) / 2;
    }
    const int ntiles = wave < 2 ? 3 : 2;

    // ---- loads: K rows into LDS (clamped into the chunk, masked at staging).  All loads are
    //      unconditional.
    const int last = max(nv - 1, 0);
    constexpr int VPR = DK / VEC;
    constexpr int NV = 64 * VPR / 256;
    // wave 0: this lane's token's log-gate and beta, in flight together with the K rows
    const int64_t gidx = (int64_t)(t0 + min(lane, last)) * p.H_v + h;
    float gx = 0.f, bx = 0.f;
    if (wave == 0) {
        gx = g[gidx];
        bx = to_f32(beta[gidx]);
    }
    u32x4 kv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int idx = tid + 256 * i, row = min(idx / VPR, last), cv = idx % VPR;
        kv[i] = *reinterpret_cast<const u32x4 *>(k + ((int64_t)(t0 + row) * p.H_qk + hq) * DK + cv * VEC);
    }
    // prologue: the L2-norm factors r = (sum x^2 + eps)^-1/2 of every K and Q row (the VPR threads
    // holding a row reduce their partial sums), else r = 1.  Q is read only for these factors.
    if (p.pro.qk_l2norm) {
        const T *q = static_cast<const T *>(p.q);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = tid + 256 * i, row = min(idx / VPR, last), cv = idx % VPR;
            u32x4 qv = *reinterpret_cast<const u32x4 *>(q + ((int64_t)(t0 + row) * p.H_qk + hq) * DK + cv * VEC);
            const T *xk = reinterpret_cast<const T *>(&kv[i]);
            const T *xq = reinterpret_cast<const T *>(&qv);
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                sk += to_f32(xk[e]) * to_f32(xk[e]);
                sq += to_f32(xq[e]) * to_f32(xq[e]);
            }
#pragma unroll
            for (int off = 1; off < VPR; off <<= 1) {
                sk += __shfl_xor(sk, off, 64);
                sq += __shfl_xor(sq, off, 64);
            }
            if (cv == 0) {
                sRk[idx / VPR] = 1.f / sqrtf(sk + kL2Eps);
                sRq[idx / VPR] = 1.f / sqrtf(sq + kL2Eps);
            }
        }
    } else if (tid < 64) {
        sRk[tid] = sRq[tid] = 1.f;
    }
    if (nv == kChunk) {                  // a full chunk (the common case): no row masking
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = tid + 256 * i, row = idx / VPR, cv = idx % VPR;
            *reinterpret_cast<u32x4 *>(sK + row * KP + cv * VEC) = kv[i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = tid + 256 * i, row = idx / VPR, cv = idx % VPR;
            *reinterpret_cast<u32x4 *>(sK + row * KP + cv * VEC) = row < nv ? kv[i] : u32x4{0u, 0u, 0u, 0u};
        }
    }
    __syncthreads();
    if (wave == 0) {
        const float gv = lane < nv ? (p.pro.A_log ? gate_activation(p.pro, gx, p.pro.A_log[h], p.pro.dt_bias ? p.pro.dt_bias[h] : 0.f) : gx) : 0.f;
        const float bv = lane < nv ? beta_value(p.pro, bx) : 0.f;
        const float gl = wave_inclusive_scan(gv) * kLog2e;     // log2 gamma_t
        const float glC = __shfl(gl, 63, 64);                  // at the last valid token
        const float rk = sRk[lane], rq = sRq[lane];
        sGl[lane] = gl;
        sB[lane] = bv * rk;                                    // the row factor of A_raw
        // gate block of the recurrence
        float *gbk = p.gates + ((int64_t)ci * p.H_v + h) * GB_FLOATS;
        const float gam = fast_exp2(gl);
        gbk[GB_BETA + lane] = bv;
        gbk[GB_SC + lane] = fast_exp2(glC - gl) * rk;
        gbk[GB_GAK + lane] = gam * rk;
        gbk[GB_GAQ + lane] = gam * rq;
        gbk[GB_GLQ + lane] = gl + __log2f(rq);
        gbk[GB_GLK + lane] = gl - __log2f(rk);
        if (lane == 0) gbk[GB_GC] = fast_exp2(glC);
    }

    // ---- this wave's tiles of A_raw = strictLower(diag(beta) (Gamma (.) K K^T)), all accumulators
    //      in flight together
    f32x4 aa[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) aa[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        Frag<T> ki[NT], kj[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            if (n >= ntiles) break;
            ki[n] = ld8(sK + (16 * TI[n] + l16) * KP + 32 * kb + 8 * grp);
            kj[n] = ld8(sK + (16 * TJ[n] + l16) * KP + 32 * kb + 8 * grp);
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            if (n >= ntiles) break;
            mma(aa[n], ki[n], kj[n]);
        }
    }
    __syncthreads();  // every wave has read the K tile: A_raw takes its region
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        if (n >= ntiles) break;
        const int j = 16 * TJ[n] + l16;
        const float glj = sGl[j], rj = sRk[j];
        const bool diag = TI[n] == TJ[n];            // only diagonal tiles have entries j >= i
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * TI[n] + 4 * grp + r;
            const float x = sB[i] * fast_exp2(sGl[i] - glj) * rj * aa[n][r];
            sL[i * LP + j] = (!diag || j < i) ? x : 0.f;
        }
    }
    __syncthreads();  // A_raw is complete

    invert_unit_lower(sL, sX);
    store_unit_lower<T>(sX, static_cast<T *>(p.A) + ((int64_t)ci * p.H_v + h) * 4096);
}

// ------------------------------------------------------------------------------------------
// Kernel (a), per-channel gates (KDA source walk-through, sections 3-5): per (chunk, value head),
// with G the chunk-local inclusive cumsum of the [D_k] log-gates (log2 units here),
//   A_raw[i][j] = beta_i sum_d k_id k_jd 2^(G_id - G_jd)          (j < i)
//   P[i][j]     = scale sum_d q_id k_jd 2^(G_id - G_jd)            (j <= i)
//   A = (I + A_raw)^{-1},  Kg = K (.) 2^G,  Qg = Q (.) 2^G,  Kd = K (.) 2^(G_C - G),  decay = 2^G_C
// (G_C: G at the last valid token; tail rows are zero in every output).  The recurrence kernel
// then runs the scalar-gate schedule on these operands, with P read instead of formed.  The
// decay factors make Kg, Kd, Qg inexact (unlike K and Q themselves), and bf16 rounding of Kd or Qg
// would move the state or the output by about 1e-2 RMS; so for bf16 inputs every stored operand
// (Kg, Kd, Qg, P, A) is fp16, rounded to nearest once (11 significant bits), and the recurrence
// multiplies them on the fp16 matrix cores.  This needs each stored value below 65504 in
// magnitude, which holds for L2-normalised q and k rows (the method's convention): decayed
// entries of unit rows, P of at most scale in size, and the inverse of I plus a strictly lower
// Gram-like matrix.
//
// The pairwise factor 2^(G_i - G_j) is split per 16x16 tile at a reference row r between j and i
// (r = last row of the column block for tiles below the diagonal, the first row of the block on
// it), so both operand factors are decays over at most 15 tokens or at most 1:
//   left_i = x_i (.) 2^(G_i - G_r) <= |x_i|,   right_j = k_j (.) 2^(G_r - G_j).
// A diagonal tile whose gates decay by more than 2^-64 across its 16 rows in some channel (where
// right_j could overflow and left_i underflow) forms each pair's factor 2^(G_i - G_j) <= 1 whole, in
// fp32 on the vector ALU, so no gate value can produce inf or NaN.
// Inside this kernel P's operands are hi/lo bf16 pairs (three MFMAs per block), A_raw's rounded once.
// ------------------------------------------------------------------------------------------
// PRO: some part of the prologue is on (q/k L2 norm, gate activation, sigma(beta)); the template
// flag keeps all of it out of the plain build, whose timing it would otherwise change
// Largest decay (in log2 units) across a diagonal 16-row block for which the split factors of that
// block are used: the key factor is then at most 2^64 and the query/key factor at least 2^-64
// (fp32 operands), or at most 2^12 and at least 2^-12 (fp16 operands: inside their normal range).
constexpr float kMaxRange = 64.f, kMaxRangeF16 = 12.f;

template <typename T, int DK, bool PRO>
__global__ __launch_bounds__(256) void intra_kda_kernel(IntraKdaParams p) {
    using OT = typename KdaOperand<T>::type;
    static_assert(sizeof(OT) == sizeof(T), "stored operands keep the input's element size");
    constexpr int VEC = Vec16<T>::N;
    constexpr int KP = DK + VEC;   // row stride of the K and Q tiles
    constexpr int LP = 64 + 4;     // row stride of the fp32 64x64 tiles
    constexpr int GP = DK + 4;     // row stride of the fp32 G tile
    constexpr int K_BYTES = 64 * KP * (int)sizeof(T);
    constexpr int X_BYTES = 64 * LP * 4;
    constexpr int R0 = K_BYTES > X_BYTES ? K_BYTES : X_BYTES;
    constexpr int NKB = DK / 32;
    // region 0: K tile, then the odd waves' P partials, then the inverse X; the G tile, then A_raw
    // (written only after every wave is done with G).  Q stays in registers: each thread's share for
    // the gated output, and each lane's operand rows for P.  51 KiB in all at D_k = 128 (bf16), so
    // three workgroups share a CU.
    __shared__ __attribute__((aligned(16))) unsigned char smem[R0];
    __shared__ __attribute__((aligned(16))) float sG[64 * GP];
    __shared__ float sB[64], sRq[64], sRk[64], sWarm[4];
    static_assert(64 * LP <= 64 * GP, "A_raw fits where the G tile was");
    T *sK = reinterpret_cast<T *>(smem);
    float *sX = reinterpret_cast<float *>(smem);
    float *sL = sG;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, grp = lane >> 4;
    const int cg = blockIdx.x / p.H_v, h = blockIdx.x - cg * p.H_v;
    const int ci = piece_chunk(cg, p.T, p.piece_lo, p.piece_cnt);
    const int hq = h / (p.H_v / p.H_qk);
    const ChunkInfo cinfo = chunk_info(p.chunks, ci, p.T);
    const int t0 = cinfo.tok0, nv = cinfo.nv, last = max(nv - 1, 0);
    const T *k = static_cast<const T *>(p.k);
    const T *q = static_cast<const T *>(p.q);
    const T *g = static_cast<const T *>(p.g);
    const T *beta = static_cast<const T *>(p.beta);

    // the row blocks of this wave's tiles (waves 0, 1: 3 and 0; waves 2, 3: 2 and 1) and its half of
    // the channel blocks (the even wave of each pair the first half)
    constexpr int HKB = NKB / 2;
    const int half = wave & 1, kb0 = HKB * half;
    const int RB0 = wave < 2 ? 3 : 2, RB1 = wave < 2 ? 0 : 1;
    // ---- K tile (clamped rows, tail masked at staging), Q in registers, gate columns, beta
    constexpr int VPR = DK / VEC;
    constexpr int NV = 64 * VPR / 256;
    u32x4 kv[NV], qv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int idx = tid + 256 * i, row = min(idx / VPR, last), cv = idx % VPR;
        const int64_t off = ((int64_t)(t0 + row) * p.H_qk + hq) * DK + cv * VEC;
        kv[i] = *reinterpret_cast<const u32x4 *>(k + off);
        qv[i] = *reinterpret_cast<const u32x4 *>(q + off);
    }
    // Q operand rows of this lane's P tiles (row 16 I + l16 of both row blocks, 8 columns per block)
    Frag<T> qt[2][HKB];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int row = min(16 * (b ? RB1 : RB0) + l16, last);
#pragma unroll
        for (int kk = 0; kk < HKB; ++kk)
            qt[b][kk] = ld8(q + ((int64_t)(t0 + row) * p.H_qk + hq) * DK + 32 * (kb0 + kk) + 8 * grp);
    }
    // thread (d, part) scans NT consecutive tokens of channel d.  The gate rows load through a
    // buffer resource over the chunk's valid rows: the row offset is a scalar, the channel a fixed
    // lane offset, and rows past the end read as zero (a clamped 64-bit address per element and a
    // tail mask had cost about a fifth of the kernel's vector instructions)
    constexpr int NPART = 256 / DK, NT = 64 / NPART;
    const int d = tid % DK, part = tid / DK;
    const int grow = p.H_v * DK * (int)sizeof(T);   // bytes from one token's gate row to the next
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(g + ((int64_t)t0 * p.H_v + h) * DK,
                                                nv > 0 ? (nv - 1) * grow + DK * (int)sizeof(T) : 0);
    float gs[NT];
#pragma unroll
    for (int e = 0; e < NT; ++e) {
        const int soff = (part * NT + e) * grow;
        if constexpr (sizeof(T) == 2)
            gs[e] = __uint_as_float((unsigned)__builtin_amdgcn_raw_buffer_load_b16(rg, d * 2, soff, 0) << 16);
        else
            gs[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, d * 4, soff, 0));
    }
    if (PRO && p.pro.A_log) {
        // prologue: raw gate inputs through the gate activation, one rolled loop over this thread's
        // own cells of the G tile (an unrolled one would double the kernel's code)
        const float al = p.pro.A_log[h], bias = p.pro.dt_bias ? p.pro.dt_bias[h * DK + d] : 0.f;
#pragma unroll
        for (int e = 0; e < NT; ++e) sG[(part * NT + e) * GP + d] = gs[e];
#pragma unroll 1
        for (int e = 0; e < NT; ++e) {
            float *c = sG + (part * NT + e) * GP + d;
            *c = gate_activation(p.pro, *c, al, bias);
        }
#pragma unroll
        for (int e = 0; e < NT; ++e) gs[e] = sG[(part * NT + e) * GP + d];
    }
    {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < NT; ++e) {
            // rows past the end read zero; with the prologue they went through the activation
            acc += !PRO || part * NT + e < nv ? gs[e] : 0.f;
            gs[e] = acc;
        }
    }
    if (wave == 0) {
        const float bv = to_f32(beta[(int64_t)(t0 + min(lane, last)) * p.H_v + h]);
        sB[lane] = lane < nv ? (PRO ? beta_value(p.pro, bv) : bv) : 0.f;
    }
    if (PRO && p.pro.qk_l2norm) {
        // prologue: the q and k rows' L2-norm factors (the VPR threads holding a row reduce their
        // partial sums); they stay fp32 and scale the rows wherever an operand is formed, since
        // rounding the normalised rows to the input dtype perturbs the inputs themselves
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const T *xk = reinterpret_cast<const T *>(&kv[i]);
            const T *xq = reinterpret_cast<const T *>(&qv[i]);
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                sk += to_f32(xk[e]) * to_f32(xk[e]);
                sq += to_f32(xq[e]) * to_f32(xq[e]);
            }
#pragma unroll
            for (int off = 1; off < VPR; off <<= 1) {
                sk += __shfl_xor(sk, off, 64);
                sq += __shfl_xor(sq, off, 64);
            }
            const int idx = tid + 256 * i;
            if (idx % VPR == 0) {
                sRk[idx / VPR] = 1.f / sqrtf(sk + kL2Eps);
                sRq[idx / VPR] = 1.f / sqrtf(sq + kL2Eps);
            }
        }
    } else if (PRO && tid < 64) {
        sRk[tid] = sRq[tid] = 1.f;
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int idx = tid + 256 * i, row = idx / VPR, cv = idx % VPR;
        const u32x4 z = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4 *>(sK + row * KP + cv * VEC) = row < nv ? kv[i] : z;
        if (row >= nv) qv[i] = z;
    }
#pragma unroll
    for (int e = 0; e < NT; ++e) sG[(part * NT + e) * GP + d] = gs[e];
    __syncthreads();
    float base = 0.f;  // totals of the earlier parts of this channel
    for (int pp = 0; pp < part; ++pp) base += sG[(pp * NT + NT - 1) * GP + d];
    __syncthreads();
#pragma unroll
    for (int e = 0; e < NT; ++e) sG[(part * NT + e) * GP + d] = (gs[e] + base) * kLog2e;
    __syncthreads();

    // ---- gated operands of the recurrence and the per-channel chunk decay
    const int64_t tile = ((int64_t)ci * p.H_v + h) * 64 * DK;
    OT *kg = static_cast<OT *>(p.kg) + tile, *kd = static_cast<OT *>(p.kd) + tile, *qg = static_cast<OT *>(p.qg) + tile;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int idx = tid + 256 * i, row = idx / VPR, c0 = (idx % VPR) * VEC;
        T qs[VEC];
        OT vk[VEC], vq[VEC], vd[VEC];
        *reinterpret_cast<u32x4 *>(qs) = qv[i];
        const float rk = PRO ? sRk[row] : 1.f, rq = PRO ? sRq[row] : 1.f;   // L2-norm factors (else 1)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float G = sG[row * GP + c0 + e], GC = sG[last * GP + c0 + e];
            const float kk = to_f32(sK[row * KP + c0 + e]) * rk, qq = to_f32(qs[e]) * rq;
            const float eg = fast_exp2(G);
            vk[e] = from_f32<OT>(kk * eg);
            vq[e] = from_f32<OT>(qq * eg);
            vd[e] = from_f32<OT>(kk * fast_exp2(GC - G));
        }
        *reinterpret_cast<u32x4 *>(kg + row * DK + c0) = *reinterpret_cast<const u32x4 *>(vk);
        *reinterpret_cast<u32x4 *>(qg + row * DK + c0) = *reinterpret_cast<const u32x4 *>(vq);
        *reinterpret_cast<u32x4 *>(kd + row * DK + c0) = *reinterpret_cast<const u32x4 *>(vd);
    }
    float *gbk = p.gates + ((int64_t)ci * p.H_v + h) * GB_FLOATS;
    if (tid < DK) gbk[GB_DEC + tid] = fast_exp2(sG[last * GP + tid]);
    if (tid < 64) gbk[GB_BETA + tid] = sB[tid];
    // the chunk's decay bound for warmup CP: the sum over tokens of each token's largest channel
    // log-decay (G_t - G_{t-1}, zero past the end); four threads per token, one partial per wave
    {
        const int t = tid >> 2, d0 = (tid & 3) * (DK / 4);
        float m = -INFINITY;
#pragma unroll 8
        for (int e = 0; e < DK / 4; ++e)
            m = fmaxf(m, sG[t * GP + d0 + e] - (t > 0 ? sG[(t - 1) * GP + d0 + e] : 0.f));
        m = fmaxf(m, __shfl_xor(m, 1, 64));
        m = fmaxf(m, __shfl_xor(m, 2, 64));
        float x = (tid & 3) == 0 ? m : 0.f;
#pragma unroll
        for (int off = 4; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
        if (lane == 0) sWarm[wave] = x;
    }

    // ---- A_raw (strict lower) and P (lower with diagonal): the 10 lower 16x16 tiles.  The operands
    //      are rounded once to the stored type (fp16 or fp32).  Every tile (I, J) of row block I splits
    //      its pairwise factor at the row r = 16 I - 1 (G_r = 0 for I = 0), so the left operands
    //      k_i 2^(G_i - G_r) and q_i 2^(G_i - G_r) (at most |x_i|) are formed once per row block and
    //      channel block, and only the key operand k_j 2^(G_r - G_j) per tile: at most 1 below the
    //      diagonal, at most the decay across the 17 rows r .. 16 I + 15 on it.  P is formed
    //      transposed (keys as the rows of the product), so each lane holds four consecutive key
    //      columns of one query row and stores them straight from its registers.  Each pair of waves
    //      shares five tiles and splits their channel blocks; the odd wave hands its partial sums to
    //      the even one through LDS.
    OT *P = static_cast<OT *>(p.P) + ((int64_t)ci * p.H_v + h) * 4096;
    constexpr float range_max = is_f16<OT> ? kMaxRangeF16 : kMaxRange;
    auto store_p4 = [&](int row, int col, const f32x4 &x) __attribute__((always_inline)) {
        if constexpr (is_f16<OT>) {
            const f16x4 v = {(f16)x[0], (f16)x[1], (f16)x[2], (f16)x[3]};
            *reinterpret_cast<f16x4 *>(P + row * 64 + col) = v;
        } else {
            *reinterpret_cast<float4 *>(P + row * 64 + col) = make_float4(x[0], x[1], x[2], x[3]);
        }
    };
    // accumulator slots: 0 .. 3 tiles (RB0, J), 4 .. 5 tiles (RB1, J)
    f32x4 aa[6], pa[6];
#pragma unroll
    for (int s = 0; s < 6; ++s) aa[s] = pa[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int I = b ? RB1 : RB0, r = 16 * I - 1;
        const int i = 16 * I + l16;                  // this lane's left operand row
        // the diagonal tile has no reference row between every pair's two tokens: its key factor
        // 2^(G_r - G_j) grows across the block.  If some channel decays by more than 2^-range_max
        // across rows r .. 16 I + 15, the split factors could leave the operand type's range, so every
        // pair's factor 2^(G_i - G_j) <= 1 is then formed whole instead.
        float range = 0.f;
#pragma unroll
        for (int d = lane; d < DK; d += 64) range = fmaxf(range, (I ? sG[r * GP + d] : 0.f) - sG[(16 * I + 15) * GP + d]);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) range = fmaxf(range, __shfl_xor(range, off, 64));
        const bool whole = range > range_max;
        const float qmask = i < nv ? (PRO ? sRq[i] : 1.f) : 0.f;   // with the prologue: Q row i's L2-norm factor
        const float rki = PRO ? sRk[i] : 1.f;
#pragma unroll
        for (int kk = 0; kk < HKB; ++kk) {
            const int d0 = 32 * (kb0 + kk) + 8 * grp;
            float gr[8], kl[8], ql[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                gr[e] = I ? sG[r * GP + d0 + e] : 0.f;
                const float el = fast_exp2(sG[i * GP + d0 + e] - gr[e]);
                kl[e] = to_f32(sK[i * KP + d0 + e]) * (rki * el);
                ql[e] = to_f32(qt[b][kk].v[e]) * (qmask * el);
            }
            Frag<OT> fkl, fql;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                set_elem(fkl, e, from_f32<OT>(kl[e]));
                set_elem(fql, e, from_f32<OT>(ql[e]));
            }
#pragma unroll
            for (int J = 0; J < (b ? 2 : 4); ++J) {
                if (J > I || (J == I && whole)) continue;
                const int j = 16 * J + l16, s = b ? 4 + J : J;
                const float rkj = PRO ? sRk[j] : 1.f;
                Frag<OT> fkr;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    set_elem(fkr, e, from_f32<OT>(to_f32(sK[j * KP + d0 + e]) * (rkj * fast_exp2(gr[e] - sG[j * GP + d0 + e]))));
                mma(aa[s], fkl, fkr);
                mma(pa[s], fkr, fql);   // P^T: row 4 grp + rr of key block J, column l16 of query block I
            }
        }
        if (whole) {
            // this wave's channels of the diagonal tile.  A_raw: rows ii = 16 I + 4 grp + rr, column
            // j = 16 I + l16 (the accumulator layout); P: query row i, key columns ii (transposed)
            const int j = i;
            const float rkj = PRO ? sRk[j] : 1.f;
            f32x4 wa, wp;
            const T *qi = q + ((int64_t)(t0 + min(i, last)) * p.H_qk + hq) * DK;
#pragma unroll 1
            for (int rr = 0; rr < 4; ++rr) {
                const int ii = 16 * I + 4 * grp + rr;
                float sa = 0.f, sp = 0.f;
                if (j < ii) {
#pragma unroll 4
                    for (int d = 32 * kb0; d < 32 * (kb0 + HKB); ++d) {
                        const float e = fast_exp2(sG[ii * GP + d] - sG[j * GP + d]);   // <= 1
                        sa += to_f32(sK[ii * KP + d]) * to_f32(sK[j * KP + d]) * e;
                    }
                }
                if (ii <= i) {
#pragma unroll 4
                    for (int d = 32 * kb0; d < 32 * (kb0 + HKB); ++d) {
                        const float e = fast_exp2(sG[i * GP + d] - sG[ii * GP + d]);   // <= 1
                        sp += to_f32(qi[d]) * to_f32(sK[ii * KP + d]) * e;
                    }
                }
                const float rkii = PRO ? sRk[ii] : 1.f;
                wa[rr] = sa * rkii * rkj;
                wp[rr] = sp * qmask * rkii;
            }
#pragma unroll
            for (int J = 0; J < (b ? 2 : 4); ++J)   // the diagonal tile's slot, kept a compile-time index
                if (J == I) {
                    aa[b ? 4 + J : J] = wa;
                    pa[b ? 4 + J : J] = wp;
                }
        }
    }
    __syncthreads();   // every wave has read the K and G tiles: P partials and A_raw take their places
    float *sPart = reinterpret_cast<float *>(smem) + (wave >> 1) * (6 * 64 * 4);
    static_assert(2 * 6 * 64 * 4 * 4 <= R0, "the P partials of both wave pairs fit where the K tile was");
    auto each_tile = [&](auto &&f) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < 6; ++s) {
            const int I = s < 4 ? RB0 : RB1, J = s < 4 ? s : s - 4;
            if (J > I) continue;
            f(s, I, J);
        }
    };
    if (half) {
        // A partials straight into their A_raw cells, P partials lane-private; the two tiles above
        // the diagonal that the recurrence reads, (0, 1) and (2, 3), are written as zeros
        each_tile([&](int s, int I, int J) __attribute__((always_inline)) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sL[(16 * I + 4 * grp + rr) * LP + 16 * J + l16] = aa[s][rr];
            *reinterpret_cast<f32x4 *>(sPart + (s * 64 + lane) * 4) = pa[s];
        });
        store_p4(16 * (wave == 1 ? 0 : 2) + l16, 16 * (wave == 1 ? 1 : 3) + 4 * grp, f32x4{0.f, 0.f, 0.f, 0.f});
    }
    __syncthreads();
    if (!half) {
        each_tile([&](int s, int I, int J) __attribute__((always_inline)) {
            const int i = 16 * I + l16, jj = 16 * J + l16;
            const f32x4 pp = *reinterpret_cast<const f32x4 *>(sPart + (s * 64 + lane) * 4);
            f32x4 pv;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int ii = 16 * I + 4 * grp + rr;
                float *c = sL + ii * LP + jj;
                *c = jj < ii ? sB[ii] * (aa[s][rr] + *c) : 0.f;
                pv[rr] = 16 * J + 4 * grp + rr <= i ? p.scale * (pa[s][rr] + pp[rr]) : 0.f;
            }
            store_p4(i, 16 * J + 4 * grp, pv);
        });
    }
    __syncthreads();   // A_raw is complete in sL, the partial decay bounds in sWarm; the K tile is free
    if (tid == 0) gbk[GB_GC] = fast_exp2(sWarm[0] + sWarm[1] + sWarm[2] + sWarm[3]);
    invert_unit_lower(sL, sX);
    store_unit_lower<OT>(sX, static_cast<OT *>(p.A) + ((int64_t)ci * p.H_v + h) * 4096);
}

}  // namespace

hipError_t launch_intra(int dtype, int D_k, const IntraParams &p, hipStream_t s) {
    const int items = p.piece_cnt ? p.N * p.piece_cnt : p.n_chunks;
    const dim3 grid((unsigned)items * (unsigned)p.H_v), block(256);
    if (items == 0) return hipSuccess;
    if (dtype == 1 && D_k == 128) launch_k(intra_kernel<bf16, 128>, grid, block, s, p);
    else if (dtype == 1 && D_k == 64) launch_k(intra_kernel<bf16, 64>, grid, block, s, p);
    else if (dtype == 0 && D_k == 128) launch_k(intra_kernel<float, 128>, grid, block, s, p);
    else if (dtype == 0 && D_k == 64) launch_k(intra_kernel<float, 64>, grid, block, s, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_intra_kda(int dtype, int D_k, const IntraKdaParams &p, hipStream_t s) {
    const int items = p.piece_cnt ? p.N * p.piece_cnt : p.n_chunks;
    const dim3 grid((unsigned)items * (unsigned)p.H_v), block(256);
    if (items == 0) return hipSuccess;
    const bool pro = p.pro.qk_l2norm || p.pro.beta_sigmoid || p.pro.A_log;
#define GDN_INTRA_KDA_CASE(T, DK)                                                                   \
    if (pro) launch_k(intra_kda_kernel<T, DK, true>, grid, block, s, p);             \
    else launch_k(intra_kda_kernel<T, DK, false>, grid, block, s, p);
    if (dtype == 1 && D_k == 128) { GDN_INTRA_KDA_CASE(bf16, 128) }
    else if (dtype == 1 && D_k == 64) { GDN_INTRA_KDA_CASE(bf16, 64) }
    else if (dtype == 0 && D_k == 128) { GDN_INTRA_KDA_CASE(float, 128) }
    else if (dtype == 0 && D_k == 64) { GDN_INTRA_KDA_CASE(float, 64) }
    else return hipErrorInvalidValue;
#undef GDN_INTRA_KDA_CASE
    return hipGetLastError();
}

}  // namespace gdn
