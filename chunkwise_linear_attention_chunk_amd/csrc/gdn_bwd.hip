// Backward of the chunked gated delta rule (scalar gate): GDN-in-FLA notes, backward Steps 1-7,
// and the Flash Linear Attention page, section 7 (reverse-time state-gradient scan, recomputed
// chunk states, the gate gradient as a reverse cumsum).  A first, plain form: fp32 arithmetic on
// LDS tiles, no matrix cores, correctness before speed.
//
// Per chunk (tokens i < nv, gl_i the chunk-local cumsum of the log-gates, gamma_i = e^{gl_i},
// D_i = e^{gl_C - gl_i}, S the state entering the chunk, A the stored (I + L)^-1):
//   forward:  X = diag(beta)(V - diag(gamma) K S),  V' = A X,
//             O = scale (diag(gamma) Q S + Pt V'),  Pt_ij = e^{gl_i - gl_j} q_i.k_j  (j <= i),
//             S_next = gamma_C S + K^T diag(D) V'
//   backward, given dO and dS_next (the gradient of the state leaving the chunk):
//     dV' = diag(D) K dS_next + scale Pt^T dO,      dX = A^T dV',     dA = dV' X^T,
//     dL  = -A^T dA A^T (strictly lower),           dPt = scale dO V'^T (lower with diagonal),
//     dS  = gamma_C dS_next + scale Q^T diag(gamma) dO - K^T diag(beta gamma) dX,
//     dQ  = scale diag(gamma) dO S^T + (dPt (.) Gam) K,
//     dK  = diag(D) V' dS_next^T - diag(beta gamma) dX S^T + (dPt (.) Gam)^T Q + E K + E^T K,
//           E_ij = dL_ij beta_i e^{gl_i - gl_j}  (j < i),
//     dV  = diag(beta) dX,   dbeta_i = dX_i.(v_i - gamma_i (K S)_i) + sum_j dL_ij G_ij,
//           G_ij = e^{gl_i - gl_j} k_i.k_j  (j < i),
//     d gl_i from every e^{gl} factor (the X, O, Pt, L, D and gamma_C terms), then
//     dg_t = sum_{i >= t} d gl_i within the chunk (the reverse cumsum of the notes' Step 7).
#include "gdn_internal.h"
#include "gdn_device.h"

namespace gdn {
namespace {

constexpr int kBw = 16;     // value columns per workgroup of the per-channel reverse scan
constexpr int kBwR = 32;    // value columns per workgroup of the forward replays
constexpr int kBwD = 32;    // value columns per workgroup of the reverse scan (measured: 16 columns
                            // 5.8 ms, 32 columns 5.4 ms on the Qwen3-Next shape; the replay is
                            // faster at 16: 2.1 against 3.1 ms)
constexpr int kBw3 = 8;     // value columns per block of the per-chunk gradient kernel
constexpr int kBwT = 1024;  // threads of the backward kernels (P, replay, scan, gradients): waves per
                            // SIMD hide their LDS latency (256 and 512 threads measured slower)

// chunk-local gates of chunk (tok0, nv) and head h into sgl (cumsum, natural log) and sb (beta);
// rows past the end carry beta = 0 and the last valid cumsum.  Wave 0 only.
template <typename T>
__device__ __forceinline__ void load_gates(const BwdParams &p, int64_t tok0, int nv, int h, float *sgl, float *sb) {
    const int lane = threadIdx.x & 63;
    const int64_t t = tok0 + min(lane, max(nv - 1, 0));
    const float gv = lane < nv ? static_cast<const float *>(p.g)[t * p.H_v + h] : 0.f;
    sgl[lane] = wave_inclusive_scan(gv);
    sb[lane] = lane < nv ? to_f32(static_cast<const T *>(p.beta)[t * p.H_v + h]) : 0.f;
}

// rows [0, nv) of a [64][cols] tile of x (row stride ld, column offset c0) into fp32 LDS, zero
// past the end
// (NT threads; the element loads of a thread are independent and issued together, rows past
// the end are clamped to the last valid row and zeroed at the store)
template <int COLS, typename T, int NT>
__device__ __forceinline__ void load_rows(float *dst, int dst_ld, const T *x, int64_t tok0, int nv, int64_t ld,
                                          int c0) {
    constexpr int N = (64 * COLS + NT - 1) / NT;   // threads past 64 COLS elements idle
    float v[N];
#pragma unroll
    for (int it = 0; it < N; ++it) {
        const int idx = threadIdx.x + NT * it, i = idx / COLS, j = idx - i * COLS;
        v[it] = idx < 64 * COLS ? to_f32(x[(tok0 + min(i, nv - 1)) * ld + c0 + j]) : 0.f;
    }
#pragma unroll
    for (int it = 0; it < N; ++it) {
        const int idx = threadIdx.x + NT * it, i = idx / COLS, j = idx - i * COLS;
        if (idx < 64 * COLS) dst[i * dst_ld + j] = i < nv ? v[it] : 0.f;
    }
}

// a [64][64] tile of the input dtype (or fp32) into fp32 LDS rows of stride 65 (NT threads)
template <typename T, int NT>
__device__ __forceinline__ void load_tile64(float (*dst)[65], const T *x) {
    constexpr int N = 4096 / NT;
    float v[N];
#pragma unroll
    for (int it = 0; it < N; ++it) v[it] = to_f32(x[threadIdx.x + NT * it]);
#pragma unroll
    for (int it = 0; it < N; ++it) {
        const int idx = threadIdx.x + NT * it;
        dst[idx / 64][idx % 64] = v[it];
    }
}

// ---- recomputed chunk states: S entering every chunk, per (sequence, value head, kBwR columns)
template <typename T, int DK>
__global__ __launch_bounds__(kBwT) void bwd_states_kernel(BwdParams p) {
    constexpr int NT = kBwT;
    // odd row strides (+1) keep the column walks of these tiles free of LDS bank conflicts
    __shared__ float sK[64][DK + 1], sA[64][65], sS[DK][kBwR + 1], sV[64][kBwR + 1], sX[64][kBwR + 1], sVp[64][kBwR + 1];
    __shared__ float sgl[64], sb[64], sD[64];
    const int tid = threadIdx.x;
    const int ncb = p.D_v / kBwR;
    const int cb = blockIdx.x % ncb, nh = blockIdx.x / ncb, h = nh % p.H_v, n = nh / p.H_v;
    const int hq = h / (p.H_v / p.H_qk);
    const SeqInfo si = seq_info(p.seq, n, p.T);
    const int64_t DV = p.D_v;
    for (int idx = tid; idx < DK * kBwR; idx += NT) {
        const int d = idx / kBwR, j = idx % kBwR;
        sS[d][j] = p.h0 ? p.h0[(((int64_t)n * p.H_v + h) * DK + d) * DV + cb * kBwR + j] : 0.f;
    }
    for (int c = 0; c < si.nchunks; ++c) {
        const int64_t gci = si.chunk0 + c, tok0 = si.tok0 + (int64_t)c * kChunk;
        const int nv = min(kChunk, si.len - c * kChunk);
        __syncthreads();   // the previous chunk is done with every tile
        float *st = p.states + ((gci * p.H_v + h) * DK) * DV + cb * kBwR;
        for (int idx = tid; idx < DK * kBwR; idx += NT) st[(idx / kBwR) * DV + idx % kBwR] = sS[idx / kBwR][idx % kBwR];
        load_rows<DK, T, NT>(&sK[0][0], DK + 1, static_cast<const T *>(p.k) + (int64_t)hq * DK, tok0, nv, (int64_t)p.H_qk * DK, 0);
        load_rows<kBwR, T, NT>(&sV[0][0], kBwR + 1, static_cast<const T *>(p.v) + (int64_t)h * DV, tok0, nv, (int64_t)p.H_v * DV, cb * kBwR);
        load_tile64<T, NT>(sA, static_cast<const T *>(p.A) + (gci * p.H_v + h) * 4096);
        if (tid < 64) {
            load_gates<T>(p, tok0, nv, h, sgl, sb);
            sD[tid] = __expf(__shfl(sgl[tid], 63, 64) - sgl[tid]);   // D_i = gamma_C / gamma_i
        }
        __syncthreads();
        for (int idx = tid; idx < 64 * kBwR; idx += NT) {   // X = beta (V - gamma K S)
            const int i = idx / kBwR, j = idx % kBwR;
            float s = 0.f;
            for (int d = 0; d < DK; ++d) s += sK[i][d] * sS[d][j];
            sX[i][j] = sb[i] * (sV[i][j] - __expf(sgl[i]) * s);
        }
        __syncthreads();
        for (int idx = tid; idx < 64 * kBwR; idx += NT) {   // V' = A X (A lower)
            const int i = idx / kBwR, j = idx % kBwR;
            float s = 0.f;
            for (int t = 0; t <= i; ++t) s += sA[i][t] * sX[t][j];
            sVp[i][j] = s;
        }
        __syncthreads();
        const float gC = __expf(sgl[63]);
        for (int idx = tid; idx < DK * kBwR; idx += NT) {   // S = gamma_C S + K^T diag(D) V'
            const int d = idx / kBwR, j = idx % kBwR;
            float s = 0.f;
            for (int i = 0; i < 64; ++i) s += sK[i][d] * sD[i] * sVp[i][j];
            sS[d][j] = gC * sS[d][j] + s;
        }
    }
}

// ---- scale Pt of every (chunk, value head), for the reverse scan (which would otherwise form it
//      once per value-column group): fp32 [64][64], or for bf16 inputs a bf16 pair [2][64][64]
template <typename T, int DK>
__global__ __launch_bounds__(kBwT) void bwd_p_kernel(BwdParams p) {
    constexpr int NT = kBwT;
    __shared__ float sK[64][DK + 1], sQ[64][DK + 1];
    __shared__ float sgl[64], sb[64];
    const int tid = threadIdx.x;
    const int ci = blockIdx.x / p.H_v, h = blockIdx.x - ci * p.H_v;
    const int hq = h / (p.H_v / p.H_qk);
    const ChunkInfo cinfo = chunk_info(p.chunks, ci, p.T);
    const int64_t qks = (int64_t)p.H_qk * DK;
    load_rows<DK, T, NT>(&sK[0][0], DK + 1, static_cast<const T *>(p.k) + (int64_t)hq * DK, cinfo.tok0, cinfo.nv, qks, 0);
    load_rows<DK, T, NT>(&sQ[0][0], DK + 1, static_cast<const T *>(p.q) + (int64_t)hq * DK, cinfo.tok0, cinfo.nv, qks, 0);
    if (tid < 64) load_gates<T>(p, cinfo.tok0, cinfo.nv, h, sgl, sb);
    __syncthreads();
    float *P = p.pmat + ((int64_t)ci * p.H_v + h) * 4096;
    for (int idx = tid; idx < 4096; idx += NT) {
        const int i = idx / 64, j = idx % 64;
        float s = 0.f;
        if (j <= i)
            for (int d = 0; d < DK; ++d) s += sQ[i][d] * sK[j][d];
        const float x = j <= i ? p.scale * __expf(sgl[i] - sgl[j]) * s : 0.f;
        if constexpr (sizeof(T) == 2) {
            // bf16 inputs: as the operand pair of the matrix-core reverse scan, hi [64][64] then lo
            bf16 *Pb = reinterpret_cast<bf16 *>(P);
            const bf16 hi = (bf16)x;
            Pb[idx] = hi;
            Pb[4096 + idx] = (bf16)(x - (float)hi);
        } else {
            P[idx] = x;
        }
    }
}

// ---- the same scale Pt for bf16 inputs on the matrix cores (the bf16 pair [2][64][64]): 256
//      threads, wave w forms the lower 16x16 tiles w, w + 4, w + 8 (< 10) of
//      P_ij = scale e^{gl_i - gl_j} (Q K^T)_ij (j <= i, zero past the chunk's end) from Q and K
//      fragments read straight from memory (exact bf16 products, fp32 sums), transposed -- keys as
//      the rows of the product, so a lane holds four consecutive key columns of one query row and
//      stores them with one 8-byte store per part -- and writes the upper tiles w, w + 4 (< 6) as
//      zeros.  (bwd_p_kernel's LDS dot products took 237 us per step on the Qwen3-Next shape.)
//      Used when the states were not replayed: the replay (chunk_kernel's state-storing build)
//      forms the same pair from the tiles it holds (71 us less per step on the Qwen3-Next shape,
//      the replay ~50 us more).
template <int DK>
__global__ __launch_bounds__(256) void bwd_p_mma_kernel(BwdParams p) {
    constexpr int NKB = DK / 32;
    __shared__ float sgl[64], sb[64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, grp = lane >> 4;
    const int ci = blockIdx.x / p.H_v, h = blockIdx.x - ci * p.H_v;
    const int hq = h / (p.H_v / p.H_qk);
    const ChunkInfo cinfo = chunk_info(p.chunks, ci, p.T);
    const int nv = cinfo.nv, last = max(nv - 1, 0);
    const int64_t qks = (int64_t)p.H_qk * DK;
    const bf16 *qb = static_cast<const bf16 *>(p.q) + cinfo.tok0 * qks + (int64_t)hq * DK;
    const bf16 *kb_ = static_cast<const bf16 *>(p.k) + cinfo.tok0 * qks + (int64_t)hq * DK;
    if (wave == 0) load_gates<bf16>(p, cinfo.tok0, nv, h, sgl, sb);
    int TI[3], TJ[3];
#pragma unroll
    for (int n = 0; n < 3; ++n) {
        const int t = wave + 4 * n;
        TI[n] = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
        TJ[n] = t - TI[n] * (TI[n] + 1) / 2;
    }
    const int ntiles = wave < 2 ? 3 : 2;
    f32x4 acc[3];
#pragma unroll
    for (int n = 0; n < 3; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int n = 0; n < 3; ++n) {
            if (n >= ntiles) break;
            const Frag<bf16> kf = ld8(kb_ + min(16 * TJ[n] + l16, last) * qks + 32 * kb + 8 * grp);
            const Frag<bf16> qf = ld8(qb + min(16 * TI[n] + l16, last) * qks + 32 * kb + 8 * grp);
            mma(acc[n], kf, qf);   // [key 16 TJ + 4 grp + r][query 16 TI + l16]
        }
    __syncthreads();   // the gate cumsum
    bf16 *Pb = reinterpret_cast<bf16 *>(p.pmat + ((int64_t)ci * p.H_v + h) * 4096);
    auto put = [&](int i, int j0, const float *x) __attribute__((always_inline)) {
        bf16x4 hi, lo;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            hi[r] = (bf16)x[r];
            lo[r] = (bf16)(x[r] - (float)hi[r]);
        }
        *reinterpret_cast<bf16x4 *>(Pb + i * 64 + j0) = hi;
        *reinterpret_cast<bf16x4 *>(Pb + 4096 + i * 64 + j0) = lo;
    };
#pragma unroll
    for (int n = 0; n < 3; ++n) {
        if (n >= ntiles) break;
        const int i = 16 * TI[n] + l16, j0 = 16 * TJ[n] + 4 * grp;
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = j0 + r;
            x[r] = j <= i && i < nv ? p.scale * __expf(sgl[i] - sgl[j]) * acc[n][r] : 0.f;
        }
        put(i, j0, x);
    }
    const float zero[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int u = wave + 4 * m;                       // upper tiles (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
        if (u >= 6) break;
        const int I = u < 3 ? 0 : u < 5 ? 1 : 2, J = u < 3 ? u + 1 : u < 5 ? u - 1 : 3;
        put(16 * I + l16, 16 * J + 4 * grp, zero);
    }
}

// ---- reverse scan of the state gradient: dS_next of every chunk, and dh0 (kBwT threads: two
//      waves per SIMD hide the LDS latency of the products)
template <typename T, int DK>
__global__ __launch_bounds__(kBwT) void bwd_dstate_kernel(BwdParams p) {
    constexpr int NT = kBwT;
    __shared__ float sK[64][DK + 1], sQ[64][DK + 1];
    __shared__ float sA[64][65], sP[64][65];
    __shared__ float sdS[DK][kBwD + 1], sdO[64][kBwD + 1], sKdS[64][kBwD + 1], sdVp[64][kBwD + 1], sdX[64][kBwD + 1];
    __shared__ float sgl[64], sb[64], sfq[64], sfk[64], sD[64];
    const int tid = threadIdx.x;
    const int ncb = p.D_v / kBwD;
    const int cb = blockIdx.x % ncb, nh = blockIdx.x / ncb, h = nh % p.H_v, n = nh / p.H_v;
    const int hq = h / (p.H_v / p.H_qk);
    const SeqInfo si = seq_info(p.seq, n, p.T);
    const int64_t DV = p.D_v;
    for (int idx = tid; idx < DK * kBwD; idx += NT) {
        const int d = idx / kBwD, j = idx % kBwD;
        sdS[d][j] = p.dht ? p.dht[(((int64_t)n * p.H_v + h) * DK + d) * DV + cb * kBwD + j] : 0.f;
    }
    for (int c = si.nchunks - 1; c >= 0; --c) {
        const int64_t gci = si.chunk0 + c, tok0 = si.tok0 + (int64_t)c * kChunk;
        const int nv = min(kChunk, si.len - c * kChunk);
        __syncthreads();
        float *dsn = p.dsnext + ((gci * p.H_v + h) * DK) * DV + cb * kBwD;
        for (int idx = tid; idx < DK * kBwD; idx += NT) dsn[(idx / kBwD) * DV + idx % kBwD] = sdS[idx / kBwD][idx % kBwD];
        const int64_t qks = (int64_t)p.H_qk * DK;
        load_rows<DK, T, NT>(&sK[0][0], DK + 1, static_cast<const T *>(p.k) + (int64_t)hq * DK, tok0, nv, qks, 0);
        load_rows<DK, T, NT>(&sQ[0][0], DK + 1, static_cast<const T *>(p.q) + (int64_t)hq * DK, tok0, nv, qks, 0);
        load_rows<kBwD, T, NT>(&sdO[0][0], kBwD + 1, static_cast<const T *>(p.dout) + (int64_t)h * DV, tok0, nv, (int64_t)p.H_v * DV,
                     cb * kBwD);
        load_tile64<T, NT>(sA, static_cast<const T *>(p.A) + (gci * p.H_v + h) * 4096);
        load_tile64<float, NT>(sP, p.pmat + (gci * p.H_v + h) * 4096);  // scale Pt (lower with diagonal)
        if (tid < 64) {
            load_gates<T>(p, tok0, nv, h, sgl, sb);
            // row factors: scale gamma_i (output), beta_i gamma_i (erase), D_i = gamma_C / gamma_i
            const float gi = __expf(sgl[tid]);
            sfq[tid] = p.scale * gi;
            sfk[tid] = sb[tid] * gi;
            sD[tid] = __expf(__shfl(sgl[tid], 63, 64) - sgl[tid]);
        }
        __syncthreads();
        for (int idx = tid; idx < 64 * kBwD; idx += NT) {   // K dS_next
            const int i = idx / kBwD, j = idx % kBwD;
            float s = 0.f;
            for (int d = 0; d < DK; ++d) s += sK[i][d] * sdS[d][j];
            sKdS[i][j] = s;
        }
        __syncthreads();
        const float gC = __expf(sgl[63]);
        for (int idx = tid; idx < 64 * kBwD; idx += NT) {   // dV' = D K dS_next + scale Pt^T dO
            const int i = idx / kBwD, j = idx % kBwD;
            float s = sD[i] * sKdS[i][j];
            for (int t = i; t < 64; ++t) s += sP[t][i] * sdO[t][j];
            sdVp[i][j] = s;
        }
        __syncthreads();
        for (int idx = tid; idx < 64 * kBwD; idx += NT) {   // dX = A^T dV'
            const int i = idx / kBwD, j = idx % kBwD;
            float s = 0.f;
            for (int t = i; t < 64; ++t) s += sA[t][i] * sdVp[t][j];
            sdX[i][j] = s;
        }
        __syncthreads();
        for (int idx = tid; idx < DK * kBwD; idx += NT) {   // dS = gamma_C dS_next + Q^T(...) - K^T(...)
            const int d = idx / kBwD, j = idx % kBwD;
            float s = 0.f;
            for (int i = 0; i < 64; ++i) s += sfq[i] * sQ[i][d] * sdO[i][j] - sfk[i] * sK[i][d] * sdX[i][j];
            sdS[d][j] = gC * sdS[d][j] + s;
        }
    }
    __syncthreads();
    if (p.dh0) {
        for (int idx = tid; idx < DK * kBwD; idx += NT) {
            const int d = idx / kBwD, j = idx % kBwD;
            p.dh0[(((int64_t)n * p.H_v + h) * DK + d) * DV + cb * kBwD + j] = sdS[d][j];
        }
    }
}

// ---- reverse scan of the state gradient on the matrix cores (bf16 inputs, scalar gate): the same
//      quantities as bwd_dstate_kernel.  One workgroup per (sequence, value head, 32 value columns),
//      four waves: two groups of 16 columns times two halves of the D_k rows.  Each wave holds dS for
//      its columns and rows in registers, so K dS and the update take the state-side operand straight
//      from its accumulators (pi order); the two halves' partial K dS are summed through LDS, and
//      both waves of a column group then form the same dV' and dX.  Per chunk, newest first:
//        store dS (= dS_next of the chunk);  Y = K dS;  dV' = D (.) Y + Pt^T dO;  dX = A^T dV';
//        dS <- gamma_C dS + Q^T (scale gamma (.) dO) - K^T (beta gamma (.) dX)
//      K, Q, A, the Pt pair, the dO columns and the gate block of the next-older chunk stream into
//      the other of two padded LDS stages meanwhile.  Operands that are not inputs are bf16 pairs.
template <int DK>
struct DsLayout {
    static constexpr int NW = 4, WC = 32;             // waves, value columns per workgroup
    using K = Pad<DK * 2 / 16>;                       // K and Q tiles
    using A = Pad<8>;                                 // A, and each part of the Pt pair (64 x 64)
    using O = Pad<WC * 2 / 16>;                       // dO columns of the workgroup
    static constexpr int GT = GB_FLOATS * 4;
    static constexpr int K0 = 0, Q0 = K::BYTES, A0 = 2 * K::BYTES, P0 = A0 + A::BYTES, O0 = P0 + 2 * A::BYTES;
    static constexpr int G0 = O0 + O::BYTES, STAGE = G0 + GT;
    static constexpr int NLG = GT / 1024;
    static constexpr int XCH = NW * 4 * 64 * 16;      // each wave's partial K dS (four f32x4 per lane)
    static constexpr int MD = DK / 16, NKB = DK / 32;   // over all D_k rows
    static constexpr int MH = MD / 2, KH = NKB / 2;     // over one wave's half of them
    static_assert(2 * STAGE + XCH <= 160 * 1024, "LDS budget");
};

template <int DK>
__global__ __launch_bounds__(256, 1) void bwd_dstate_mma_kernel(BwdParams p) {
    using L = DsLayout<DK>;
    using KT = typename L::K;
    using AT = typename L::A;
    using OT = typename L::O;
    constexpr int MH = L::MH, KH = L::KH, NW = L::NW;
    __shared__ __attribute__((aligned(16))) unsigned char stg0[L::STAGE], stg1[L::STAGE];
    __shared__ f32x4 xch[NW][4][64];
    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ncb = p.D_v / L::WC;
    const int xcd = blockIdx.x & 7, rr = blockIdx.x >> 3;   // XCD-aware, see scan_grid
    const int cb = rr % ncb, nh = (rr / ncb) * 8 + xcd, h = nh % p.H_v, n = nh / p.H_v;
    if (n >= p.N) return;
    const int hq = h / (p.H_v / p.H_qk);
    const SeqInfo si = seq_info(p.seq, n, p.T);
    const int DV = p.D_v, qks = p.H_qk * DK, vs = p.H_v * DV;
    const int cg = wave & 1, rh = wave >> 1, RB = rh * (DK / 2);   // column group, first D_k row
    const int c0 = cb * L::WC, col = c0 + 16 * cg + l16;
    const bf16 *kb_ = static_cast<const bf16 *>(p.k) + (int64_t)hq * DK;
    const bf16 *qb = static_cast<const bf16 *>(p.q) + (int64_t)hq * DK;
    const bf16 *ob = static_cast<const bf16 *>(p.dout) + (int64_t)h * DV + c0;
    const bf16 *Ab = static_cast<const bf16 *>(p.A) + (int64_t)h * 4096;
    const bf16 *Pb = reinterpret_cast<const bf16 *>(p.pmat) + (int64_t)h * 2 * 4096;
    const float *Gb = p.gates + (int64_t)h * GB_FLOATS;

    // this wave's stage instructions: instruction i = wave + NW j of each tile (the K-shaped tiles
    // share their lane offsets, as do the 64 x 64 ones); pad granules read zeros
    constexpr int kOut = 1 << 30;
    constexpr int JK = (KT::NI + NW - 1) / NW, JA = (AT::NI + NW - 1) / NW, JO = (OT::NI + NW - 1) / NW;
    int offK[JK], offA[JA], offO[JO];
#pragma unroll
    for (int j = 0; j < JK; ++j) {
        const int pos = 64 * (wave + NW * j) + lane, row = pos / KT::P, g = pos % KT::P;
        offK[j] = g < KT::P - 1 ? row * qks * 2 + 16 * g : kOut;
    }
#pragma unroll
    for (int j = 0; j < JA; ++j) {
        const int pos = 64 * (wave + NW * j) + lane, row = pos / AT::P, g = pos % AT::P;
        offA[j] = g < AT::P - 1 ? row * 128 + 16 * g : kOut;
    }
#pragma unroll
    for (int j = 0; j < JO; ++j) {
        const int pos = 64 * (wave + NW * j) + lane, row = pos / OT::P, g = pos % OT::P;
        offO[j] = g < OT::P - 1 ? row * vs * 2 + 16 * g : kOut;
    }
    auto load_stage = [&](int c, unsigned char *tb) __attribute__((always_inline)) {
        const int64_t tok = si.tok0 + (int64_t)c * kChunk, gci = si.chunk0 + c;
        const int nv = min(kChunk, si.len - c * kChunk);
        const u32x4 rK = rsrc_words(kb_ + tok * qks, ((nv - 1) * qks + DK) * 2);
        const u32x4 rQ = rsrc_words(qb + tok * qks, ((nv - 1) * qks + DK) * 2);
        const u32x4 rA = rsrc_words(Ab + gci * p.H_v * 4096, 4096 * 2);
        const u32x4 rPh = rsrc_words(Pb + gci * p.H_v * 2 * 4096, 4096 * 2);
        const u32x4 rPl = rsrc_words(Pb + gci * p.H_v * 2 * 4096 + 4096, 4096 * 2);
        const u32x4 rO = rsrc_words(ob + tok * vs, ((nv - 1) * vs + L::WC) * 2);
        const u32x4 rG = rsrc_words(Gb + gci * p.H_v * GB_FLOATS, GB_FLOATS * 4);
#pragma unroll
        for (int j = 0; j < JK; ++j) {
            const int i = wave + NW * j;
            if (i < KT::NI) {
                dma_granules(rK, tb + L::K0 + 1024 * i, offK[j]);
                dma_granules(rQ, tb + L::Q0 + 1024 * i, offK[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < JA; ++j) {
            const int i = wave + NW * j;
            if (i < AT::NI) {
                dma_granules(rA, tb + L::A0 + 1024 * i, offA[j]);
                dma_granules(rPh, tb + L::A0 + AT::BYTES + 1024 * i, offA[j]);
                dma_granules(rPl, tb + L::A0 + 2 * AT::BYTES + 1024 * i, offA[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < JO; ++j) {
            const int i = wave + NW * j;
            if (i < OT::NI) dma_granules(rO, tb + L::O0 + 1024 * i, offO[j]);
        }
        for (int i = wave; i < L::NLG; i += NW) dma_granules(rG, tb + L::G0 + 1024 * i, 1024 * i + 16 * lane);
    };

    f32x4 S[MH];   // dS: rows RB + 16 m + 4 grp + r of column col
#pragma unroll
    for (int m = 0; m < MH; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S[m][r] = p.dht ? p.dht[(((int64_t)n * p.H_v + h) * DK + RB + 16 * m + 4 * grp + r) * DV + col] : 0.f;

    auto step = [&](int c, const unsigned char *st) __attribute__((always_inline)) {
        const int64_t gci = si.chunk0 + c;
        const unsigned char *tK = st + L::K0, *tQ = st + L::Q0, *tA = st + L::A0, *tPh = st + L::P0;
        const unsigned char *tPl = tPh + AT::BYTES, *tO = st + L::O0;
        const float *g = reinterpret_cast<const float *>(st + L::G0);
        {   // dS_next of this chunk
            float *dsn = p.dsnext + (gci * p.H_v + h) * DK * DV;
#pragma unroll
            for (int m = 0; m < MH; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) dsn[(RB + 16 * m + 4 * grp + r) * DV + col] = S[m][r];
        }
        // Y = K dS (this wave's half of the D_k rows, then the other half's partial from LDS: both
        // waves of the column group add the same two partials), then dV' = D (.) Y + Pt^T dO
        f32x4 dv[4];
        {
            Frag<bf16> sh[KH], sl[KH];
#pragma unroll
            for (int kb = 0; kb < KH; ++kb) {
                float x[8];
                pack_pi(S[2 * kb], S[2 * kb + 1], x);
                split8_rne(x, sh[kb], sl[kb]);
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
                for (int kb = 0; kb < KH; ++kb) {
                    if (kb == 0) dv[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
                    mma_x(dv[tt], pi_row<KT>(tK, 16 * tt + l16, rh * KH + kb, grp), sh[kb], sl[kb]);
                }
                xch[wave][tt][lane] = dv[tt];
            }
        }
        lds_only_barrier();   // both halves' partials are in
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) dv[tt] += xch[wave ^ 2][tt][lane];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const float4 d4 = *reinterpret_cast<const float4 *>(g + GB_SC + 16 * tt + 4 * grp);
            dv[tt][0] *= d4.x; dv[tt][1] *= d4.y; dv[tt][2] *= d4.z; dv[tt][3] *= d4.w;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (32 * kb + 31 < 16 * tt) continue;        // Pt[s][t] = 0 for s < t
                mma_pair_x(dv[tt], pi_col<AT>(tPh, 16 * tt, kb, grp, l16), pi_col<AT>(tPl, 16 * tt, kb, grp, l16),
                           pi_col<OT>(tO, 16 * cg, kb, grp, l16));
            }
        }
        // dX = A^T dV'
        f32x4 dx[4];
        {
            Frag<bf16> vh[2], vl[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float x[8];
                pack_pi(dv[2 * kb], dv[2 * kb + 1], x);
                split8_rne(x, vh[kb], vl[kb]);
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                dx[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    if (32 * kb + 31 < 16 * tt) continue;    // A[s][t] = 0 for s < t
                    mma_x(dx[tt], pi_col<AT>(tA, 16 * tt, kb, grp, l16), vh[kb], vl[kb]);
                }
            }
        }
        // dS <- gamma_C dS + Q^T (scale gamma (.) dO) - K^T (beta gamma (.) dX)
        Frag<bf16> oh[2], ol[2], xh[2], xl[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int t0 = 32 * kb + 4 * grp;
            const float4 qa = *reinterpret_cast<const float4 *>(g + GB_GAQ + t0);
            const float4 qc = *reinterpret_cast<const float4 *>(g + GB_GAQ + t0 + 16);
            const float4 ba = *reinterpret_cast<const float4 *>(g + GB_BETA + t0);
            const float4 bc = *reinterpret_cast<const float4 *>(g + GB_BETA + t0 + 16);
            const float4 ka = *reinterpret_cast<const float4 *>(g + GB_GAK + t0);
            const float4 kc = *reinterpret_cast<const float4 *>(g + GB_GAK + t0 + 16);
            const float fq[8] = {qa.x, qa.y, qa.z, qa.w, qc.x, qc.y, qc.z, qc.w};
            const float fk[8] = {ba.x * ka.x, ba.y * ka.y, ba.z * ka.z, ba.w * ka.w,
                                 bc.x * kc.x, bc.y * kc.y, bc.z * kc.z, bc.w * kc.w};
            const Frag<bf16> o = pi_col<OT>(tO, 16 * cg, kb, grp, l16);   // dO[t][col], t in pi order
            float xo[8], xx[8];
            pack_pi(dx[2 * kb], dx[2 * kb + 1], xx);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                xo[e] = p.scale * fq[e] * (float)o.v[e];
                xx[e] = -fk[e] * xx[e];
            }
            split8_rne(xo, oh[kb], ol[kb]);
            split8_rne(xx, xh[kb], xl[kb]);
        }
        const float gC = g[GB_GC];
#pragma unroll
        for (int m = 0; m < MH; ++m) {
            S[m] *= gC;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                mma_x(S[m], pi_col<KT>(tQ, RB + 16 * m, kb, grp, l16), oh[kb], ol[kb]);
                mma_x(S[m], pi_col<KT>(tK, RB + 16 * m, kb, grp, l16), xh[kb], xl[kb]);
            }
            if (m & 1) reg_fence();
        }
    };

    const int nch = si.nchunks;
    if (nch > 0) {
        load_stage(nch - 1, stg0);
        wait_vm<0>();
        lds_only_barrier();
    }
    // chunks newest first; stage of chunk c: stg0 when (nch - 1 - c) is even
    for (int k = 0; k < nch; k += 2) {
        const int c = nch - 1 - k;
        if (c >= 1) load_stage(c - 1, stg1);
        step(c, stg0);
        wait_vm<0>();
        lds_only_barrier();    // chunk c - 1's stage; every wave is done with stg0
        if (c >= 1) {
            if (c >= 2) load_stage(c - 2, stg0);
            step(c - 1, stg1);
            wait_vm<0>();
            lds_only_barrier();
        }
    }
    if (p.dh0) {
#pragma unroll
        for (int m = 0; m < MH; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) p.dh0[(((int64_t)n * p.H_v + h) * DK + RB + 16 * m + 4 * grp + r) * DV + col] = S[m][r];
    }
}

// fp16 view of a 16-bit operand fragment read from an fp16 tile
__device__ __forceinline__ Frag<f16> as_f16(const Frag<bf16> &f) {
    Frag<f16> r;
    r.v = __builtin_bit_cast(f16x8, f.v);
    return r;
}
// fp16 pair of eight values: hi = fp16(x), lo = fp16(x - hi), both rounded to nearest
__device__ __forceinline__ void split8_h2(const float *x, Frag<f16> &h, Frag<f16> &l) {
    typedef float f32x8 __attribute__((ext_vector_type(8)));
    const f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
    h.v = __builtin_convertvector(v, f16x8);
    l.v = __builtin_convertvector(v - __builtin_convertvector(h.v, f32x8), f16x8);
}

// ---- reverse scan of the state gradient on the matrix cores (per-channel gates, bf16 inputs): the
//      quantities of bwd_dstate_kda_kernel, from the fp16 operands the per-chunk kernel stores for
//      every chunk (Kd = K (.) e^{G_C - G}, Kg = K (.) e^G, Qg = Q (.) e^G, scale P, A).  One
//      workgroup per (sequence, value head, 32 value columns), four waves: two groups of 16 columns
//      times two halves of the D_k rows, each holding dS for its columns and rows in registers; the
//      halves' partial Kd dS are summed through LDS (with D_k = 128 in the chunk's Kd tile, which
//      nothing reads after them), and both waves of a column group form the same dV' and dX.  Per
//      chunk, newest first:
//        store dS (= dS_next of the chunk);  dV' = Kd dS + (scale P)^T dO;  dX = A^T dV';
//        dS <- Diag(e^{G_C}) dS + Qg^T (scale dO) - Kg^T (beta (.) dX)
//      The next-older chunk's tiles stream into the other of two padded LDS stages meanwhile.  The
//      operands formed here (dS, dV', scale dO, dX) are fp16 hi/lo pairs (the steep-gate argument
//      of the per-chunk gradients: single terms of a chunk's first or last token can be far above
//      the RMS); dO itself is exact in fp16.
template <int DK>
struct DsKdaLayout {
    static constexpr int NW = 4, WC = 32;             // waves, value columns per workgroup
    using K = Pad<DK * 2 / 16>;                       // Kd, Kg, Qg tiles
    using A = Pad<8>;                                 // A and P (64 x 64)
    using O = Pad<WC * 2 / 16>;                       // dO columns of the workgroup
    static constexpr int GT = GB_FLOATS * 4;
    static constexpr int KD0 = 0, KG0 = K::BYTES, QG0 = 2 * K::BYTES, A0 = 3 * K::BYTES, P0 = A0 + A::BYTES;
    static constexpr int O0 = P0 + A::BYTES, G0 = O0 + O::BYTES, STAGE = G0 + GT;
    static constexpr int NLG = GT / 1024;
    static constexpr int MD = DK / 16, NKB = DK / 32;   // over all D_k rows
    static constexpr int MH = MD / 2, KH = NKB / 2;     // over one wave's half of them
    // the partial Kd dS of every wave: in a buffer of their own where it fits (D_k = 64), else in the
    // stage's Kd tile once every wave has read it
    static constexpr int XCH = NW * 4 * 64 * 16;
    static constexpr bool OWN_XCH = 2 * STAGE + XCH <= 160 * 1024;
    static_assert(OWN_XCH || XCH <= K::BYTES, "the partials fit in the Kd tile");
    static_assert(2 * STAGE <= 160 * 1024, "LDS budget");
};

template <int DK>
__global__ __launch_bounds__(256, 1) void bwd_dstate_kda_mma_kernel(BwdParams p) {
    using L = DsKdaLayout<DK>;
    using KT = typename L::K;
    using AT = typename L::A;
    using OT = typename L::O;
    constexpr int MH = L::MH, KH = L::KH, NW = L::NW;
    __shared__ __attribute__((aligned(16))) unsigned char stg0[L::STAGE], stg1[L::STAGE];
    __shared__ f32x4 xbuf[L::OWN_XCH ? L::XCH / 16 : 1];
    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ncb = p.D_v / L::WC;
    const int xcd = blockIdx.x & 7, rr = blockIdx.x >> 3;   // XCD-aware, see scan_grid
    const int cb = rr % ncb, nh = (rr / ncb) * 8 + xcd, h = nh % p.H_v, n = nh / p.H_v;
    if (n >= p.N) return;
    const SeqInfo si = seq_info(p.seq, n, p.T);
    const int DV = p.D_v, vs = p.H_v * DV;
    const int cg = wave & 1, rh = wave >> 1, RB = rh * (DK / 2);   // column group, first D_k row
    const int c0 = cb * L::WC, col = c0 + 16 * cg + l16;
    const f16 *kdb = static_cast<const f16 *>(p.kd) + (int64_t)h * 64 * DK;
    const f16 *kgb = static_cast<const f16 *>(p.kg) + (int64_t)h * 64 * DK;
    const f16 *qgb = static_cast<const f16 *>(p.qg) + (int64_t)h * 64 * DK;
    const f16 *Ab = static_cast<const f16 *>(p.A) + (int64_t)h * 4096;
    const f16 *Pb = static_cast<const f16 *>(p.P) + (int64_t)h * 4096;
    const bf16 *ob = static_cast<const bf16 *>(p.dout) + (int64_t)h * DV + c0;
    const float *Gb = p.gates + (int64_t)h * GB_FLOATS;

    // this wave's stage instructions: instruction i = wave + NW j of each tile (the K-shaped tiles
    // share their lane offsets, as do the 64 x 64 ones); pad granules read zeros
    constexpr int kOut = 1 << 30;
    constexpr int JK = (KT::NI + NW - 1) / NW, JA = (AT::NI + NW - 1) / NW, JO = (OT::NI + NW - 1) / NW;
    int offK[JK], offA[JA], offO[JO];
#pragma unroll
    for (int j = 0; j < JK; ++j) {
        const int pos = 64 * (wave + NW * j) + lane, row = pos / KT::P, g = pos % KT::P;
        offK[j] = g < KT::P - 1 ? row * DK * 2 + 16 * g : kOut;
    }
#pragma unroll
    for (int j = 0; j < JA; ++j) {
        const int pos = 64 * (wave + NW * j) + lane, row = pos / AT::P, g = pos % AT::P;
        offA[j] = g < AT::P - 1 ? row * 128 + 16 * g : kOut;
    }
#pragma unroll
    for (int j = 0; j < JO; ++j) {
        const int pos = 64 * (wave + NW * j) + lane, row = pos / OT::P, g = pos % OT::P;
        offO[j] = g < OT::P - 1 ? row * vs * 2 + 16 * g : kOut;
    }
    auto load_stage = [&](int c, unsigned char *tb) __attribute__((always_inline)) {
        const int64_t tok = si.tok0 + (int64_t)c * kChunk, gci = si.chunk0 + c;
        const int nv = min(kChunk, si.len - c * kChunk);
        const int64_t tile = gci * p.H_v * 64 * DK;
        const u32x4 rKd = rsrc_words(kdb + tile, 64 * DK * 2);
        const u32x4 rKg = rsrc_words(kgb + tile, 64 * DK * 2);
        const u32x4 rQg = rsrc_words(qgb + tile, 64 * DK * 2);
        const u32x4 rA = rsrc_words(Ab + gci * p.H_v * 4096, 4096 * 2);
        const u32x4 rP = rsrc_words(Pb + gci * p.H_v * 4096, 4096 * 2);
        const u32x4 rO = rsrc_words(ob + tok * vs, ((nv - 1) * vs + L::WC) * 2);
        const u32x4 rG = rsrc_words(Gb + gci * p.H_v * GB_FLOATS, GB_FLOATS * 4);
#pragma unroll
        for (int j = 0; j < JK; ++j) {
            const int i = wave + NW * j;
            if (i < KT::NI) {
                dma_granules(rKd, tb + L::KD0 + 1024 * i, offK[j]);
                dma_granules(rKg, tb + L::KG0 + 1024 * i, offK[j]);
                dma_granules(rQg, tb + L::QG0 + 1024 * i, offK[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < JA; ++j) {
            const int i = wave + NW * j;
            if (i < AT::NI) {
                dma_granules(rA, tb + L::A0 + 1024 * i, offA[j]);
                dma_granules(rP, tb + L::P0 + 1024 * i, offA[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < JO; ++j) {
            const int i = wave + NW * j;
            if (i < OT::NI) dma_granules(rO, tb + L::O0 + 1024 * i, offO[j]);
        }
        for (int i = wave; i < L::NLG; i += NW) dma_granules(rG, tb + L::G0 + 1024 * i, 1024 * i + 16 * lane);
    };

    f32x4 S[MH];   // dS: rows RB + 16 m + 4 grp + r of column col
#pragma unroll
    for (int m = 0; m < MH; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S[m][r] = p.dht ? p.dht[(((int64_t)n * p.H_v + h) * DK + RB + 16 * m + 4 * grp + r) * DV + col] : 0.f;

    auto step = [&](int c, unsigned char *st) __attribute__((always_inline)) {
        const int64_t gci = si.chunk0 + c;
        const unsigned char *tKd = st + L::KD0, *tKg = st + L::KG0, *tQg = st + L::QG0;
        const unsigned char *tA = st + L::A0, *tP = st + L::P0, *tO = st + L::O0;
        const float *g = reinterpret_cast<const float *>(st + L::G0);
        {   // dS_next of this chunk
            float *dsn = p.dsnext + (gci * p.H_v + h) * DK * DV;
#pragma unroll
            for (int m = 0; m < MH; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) dsn[(RB + 16 * m + 4 * grp + r) * DV + col] = S[m][r];
        }
        // dV' = Kd dS (this wave's half of the D_k rows, then the other half's partial through the
        // Kd tile: both waves of the column group add the same two partials) + (scale P)^T dO
        f32x4 dv[4];
        {
            Frag<f16> sh[KH], sl[KH];
#pragma unroll
            for (int kb = 0; kb < KH; ++kb) {
                float x[8];
                pack_pi(S[2 * kb], S[2 * kb + 1], x);
                split8_h2(x, sh[kb], sl[kb]);
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                dv[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < KH; ++kb) {
                    const Frag<f16> kf = as_f16(pi_row<KT>(tKd, 16 * tt + l16, rh * KH + kb, grp));
                    mma(dv[tt], kf, sh[kb]);
                    mma(dv[tt], kf, sl[kb]);
                }
            }
        }
        f32x4 *xch = L::OWN_XCH ? xbuf : reinterpret_cast<f32x4 *>(st + L::KD0);
        if constexpr (!L::OWN_XCH) lds_only_barrier();   // every wave is done with the Kd tile
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) xch[(wave * 4 + tt) * 64 + lane] = dv[tt];
        lds_only_barrier();   // both halves' partials are in
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) dv[tt] += xch[((wave ^ 2) * 4 + tt) * 64 + lane];
        Frag<f16> of[2], osh[2], osl[2];   // dO[t][col] and the pair of scale dO[t][col], t in pi order
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const Frag<bf16> o = pi_col<OT>(tO, 16 * cg, kb, grp, l16);
            float x[8], y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                x[e] = (float)o.v[e];
                y[e] = p.scale * x[e];
            }
            Frag<f16> unused;
            split8(x, of[kb], unused);
            split8_h2(y, osh[kb], osl[kb]);
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (32 * kb + 31 < 16 * tt) continue;        // P[s][t] = 0 for s < t
                mma(dv[tt], as_f16(pi_col<AT>(tP, 16 * tt, kb, grp, l16)), of[kb]);
            }
        // dX = A^T dV'
        f32x4 dx[4];
        {
            Frag<f16> vh[2], vl[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float x[8];
                pack_pi(dv[2 * kb], dv[2 * kb + 1], x);
                split8_h2(x, vh[kb], vl[kb]);
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                dx[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    if (32 * kb + 31 < 16 * tt) continue;    // A[s][t] = 0 for s < t
                    const Frag<f16> af = as_f16(pi_col<AT>(tA, 16 * tt, kb, grp, l16));
                    mma(dx[tt], af, vh[kb]);
                    mma(dx[tt], af, vl[kb]);
                }
            }
        }
        // dS <- Diag(e^{G_C}) dS + Qg^T (scale dO) - Kg^T (beta (.) dX)
        Frag<f16> xh[2], xl[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int t0 = 32 * kb + 4 * grp;
            const float4 ba = *reinterpret_cast<const float4 *>(g + GB_BETA + t0);
            const float4 bc = *reinterpret_cast<const float4 *>(g + GB_BETA + t0 + 16);
            const float fb[8] = {ba.x, ba.y, ba.z, ba.w, bc.x, bc.y, bc.z, bc.w};
            float xx[8];
            pack_pi(dx[2 * kb], dx[2 * kb + 1], xx);
#pragma unroll
            for (int e = 0; e < 8; ++e) xx[e] = -fb[e] * xx[e];
            split8_h2(xx, xh[kb], xl[kb]);
        }
#pragma unroll
        for (int m = 0; m < MH; ++m) {
            const float4 dec = *reinterpret_cast<const float4 *>(g + GB_DEC + RB + 16 * m + 4 * grp);
            S[m][0] *= dec.x; S[m][1] *= dec.y; S[m][2] *= dec.z; S[m][3] *= dec.w;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const Frag<f16> qf = as_f16(pi_col<KT>(tQg, RB + 16 * m, kb, grp, l16));
                const Frag<f16> kf = as_f16(pi_col<KT>(tKg, RB + 16 * m, kb, grp, l16));
                mma(S[m], qf, osh[kb]);
                mma(S[m], qf, osl[kb]);
                mma(S[m], kf, xh[kb]);
                mma(S[m], kf, xl[kb]);
            }
        }
    };

    const int nch = si.nchunks;
    if (nch > 0) {
        load_stage(nch - 1, stg0);
        wait_vm<0>();
        lds_only_barrier();
    }
    // chunks newest first; stage of chunk c: stg0 when (nch - 1 - c) is even
    for (int k = 0; k < nch; k += 2) {
        const int c = nch - 1 - k;
        if (c >= 1) load_stage(c - 1, stg1);
        step(c, stg0);
        wait_vm<0>();
        lds_only_barrier();    // chunk c - 1's stage; every wave is done with stg0
        if (c >= 1) {
            if (c >= 2) load_stage(c - 2, stg0);
            step(c - 1, stg1);
            wait_vm<0>();
            lds_only_barrier();
        }
    }
    if (p.dh0) {
#pragma unroll
        for (int m = 0; m < MH; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) p.dh0[(((int64_t)n * p.H_v + h) * DK + RB + 16 * m + 4 * grp + r) * DV + col] = S[m][r];
    }
}

// ---- per (chunk, value head): every gradient of the chunk's inputs
template <typename T, int DK>
__global__ __launch_bounds__(kBwT) void bwd_chunk_kernel(BwdParams p) {
    constexpr int NT = kBwT;
    constexpr int EPT = 64 * DK / NT;           // dq / dk elements per thread (rows e * NT / DK + tid / DK)
    constexpr int RS = NT / DK;
    constexpr int W3 = kBw3 + 1;                // odd row strides against LDS bank conflicts
    __shared__ float sK[64][DK + 1], sQ[64][DK + 1];
    __shared__ float sA[64][65], sdA[64][65], sPt[64][65], sdP[64][65];
    // per value-column block; after the blocks the same space holds A^T dA, then G
    constexpr int BLK = 2 * DK * W3 + 8 * 64 * W3;
    __shared__ float sBlk[BLK > 64 * 65 ? BLK : 64 * 65];
    __shared__ float sgl[64], sb[64], sdgl[64], sdb[64], sc[64];
    __shared__ float sdglC;
    float (*sS)[W3] = reinterpret_cast<float (*)[W3]>(sBlk);
    float (*sdS)[W3] = reinterpret_cast<float (*)[W3]>(sBlk + DK * W3);
    float (*sV)[W3] = reinterpret_cast<float (*)[W3]>(sBlk + 2 * DK * W3);
    float (*sdO)[W3] = sV + 64;
    float (*sKS)[W3] = sV + 2 * 64;
    float (*sX)[W3] = sV + 3 * 64;
    float (*sVp)[W3] = sV + 4 * 64;
    float (*sKdS)[W3] = sV + 5 * 64;
    float (*sdVp)[W3] = sV + 6 * 64;
    float (*sdX)[W3] = sV + 7 * 64;
    float (*sT)[65] = reinterpret_cast<float (*)[65]>(sBlk);

    const int tid = threadIdx.x, lane = tid & 63;
    const int ci = blockIdx.x / p.H_v, h = blockIdx.x - ci * p.H_v;
    const int hq = h / (p.H_v / p.H_qk);
    const ChunkInfo cinfo = chunk_info(p.chunks, ci, p.T);
    const int64_t tok0 = cinfo.tok0;
    const int nv = cinfo.nv;
    const int64_t DV = p.D_v, qks = (int64_t)p.H_qk * DK, vs = (int64_t)p.H_v * DV;
    load_rows<DK, T, NT>(&sK[0][0], DK + 1, static_cast<const T *>(p.k) + (int64_t)hq * DK, tok0, nv, qks, 0);
    load_rows<DK, T, NT>(&sQ[0][0], DK + 1, static_cast<const T *>(p.q) + (int64_t)hq * DK, tok0, nv, qks, 0);
    load_tile64<T, NT>(sA, static_cast<const T *>(p.A) + ((int64_t)ci * p.H_v + h) * 4096);
    for (int idx = tid; idx < 4096; idx += NT) {
        sdA[idx / 64][idx % 64] = 0.f;
        sdP[idx / 64][idx % 64] = 0.f;
    }
    if (tid < 64) {
        load_gates<T>(p, tok0, nv, h, sgl, sb);
        sdgl[tid] = sdb[tid] = sc[tid] = 0.f;
    }
    if (tid == 0) sdglC = 0.f;
    __syncthreads();
    for (int idx = tid; idx < 4096; idx += NT) {           // Pt (lower with diagonal, no scale)
        const int i = idx / 64, j = idx % 64;
        float s = 0.f;
        if (j <= i)
            for (int d = 0; d < DK; ++d) s += sQ[i][d] * sK[j][d];
        sPt[i][j] = j <= i ? __expf(sgl[i] - sgl[j]) * s : 0.f;
    }
    const float glC = sgl[63], gC = __expf(glC);
    float dq[EPT], dk[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) dq[e] = dk[e] = 0.f;
    const int col = tid % DK;

    const float *St = p.states + (((int64_t)ci * p.H_v + h) * DK) * DV;
    const float *dSt = p.dsnext + (((int64_t)ci * p.H_v + h) * DK) * DV;
    for (int c0 = 0; c0 < p.D_v; c0 += kBw3) {
        __syncthreads();   // Pt is complete; the previous block is done with its tiles
        {
            constexpr int NE = (DK * kBw3 + NT - 1) / NT;   // threads past DK kBw3 elements idle
            float a[NE], b[NE];
#pragma unroll
            for (int it = 0; it < NE; ++it) {
                const int idx = min(tid + NT * it, DK * kBw3 - 1), d = idx / kBw3, j = idx % kBw3;
                a[it] = St[d * DV + c0 + j];
                b[it] = dSt[d * DV + c0 + j];
            }
#pragma unroll
            for (int it = 0; it < NE; ++it) {
                const int idx = tid + NT * it, d = idx / kBw3, j = idx % kBw3;
                if (idx < DK * kBw3) {
                    sS[d][j] = a[it];
                    sdS[d][j] = b[it];
                }
            }
        }
        load_rows<kBw3, T, NT>(&sV[0][0], W3, static_cast<const T *>(p.v) + (int64_t)h * DV, tok0, nv, vs, c0);
        load_rows<kBw3, T, NT>(&sdO[0][0], W3, static_cast<const T *>(p.dout) + (int64_t)h * DV, tok0, nv, vs, c0);
        __syncthreads();
        for (int idx = tid; idx < 64 * kBw3; idx += NT) {  // K S, K dS_next
            const int i = idx / kBw3, j = idx % kBw3;
            float a = 0.f, e = 0.f;
            for (int d = 0; d < DK; ++d) {
                a += sK[i][d] * sS[d][j];
                e += sK[i][d] * sdS[d][j];
            }
            sKS[i][j] = a;
            sKdS[i][j] = e;
            sX[i][j] = sb[i] * (sV[i][j] - __expf(sgl[i]) * a);
        }
        {   // gamma_C <S, dS_next> over this block
            float s = 0.f;
            for (int idx = tid; idx < DK * kBw3; idx += NT) s += sS[idx / kBw3][idx % kBw3] * sdS[idx / kBw3][idx % kBw3];
            for (int off = 1; off < 64; off <<= 1) s += __shfl_xor(s, off, 64);
            if (lane == 0) atomicAdd(&sdglC, gC * s);
        }
        __syncthreads();
        for (int idx = tid; idx < 64 * kBw3; idx += NT) {  // V' = A X
            const int i = idx / kBw3, j = idx % kBw3;
            float s = 0.f;
            for (int t = 0; t <= i; ++t) s += sA[i][t] * sX[t][j];
            sVp[i][j] = s;
        }
        __syncthreads();
        for (int idx = tid; idx < 64 * kBw3; idx += NT) {  // dV' = D K dS_next + scale Pt^T dO
            const int i = idx / kBw3, j = idx % kBw3;
            float s = __expf(glC - sgl[i]) * sKdS[i][j];
            float u = 0.f;
            for (int t = i; t < 64; ++t) u += sPt[t][i] * sdO[t][j];
            sdVp[i][j] = s + p.scale * u;
        }
        if (tid < 64) {    // d gl from D; the D terms' sum goes to gl_C
            const int i = tid;
            const float Di = __expf(glC - sgl[i]);
            float cd = 0.f;
            for (int j = 0; j < kBw3; ++j) cd += sKdS[i][j] * sVp[i][j];
            sdgl[i] -= Di * cd;
            sc[i] += Di * cd;
        }
        __syncthreads();
        for (int idx = tid; idx < 64 * kBw3; idx += NT) {  // dX = A^T dV'
            const int i = idx / kBw3, j = idx % kBw3;
            float s = 0.f;
            for (int t = i; t < 64; ++t) s += sA[t][i] * sdVp[t][j];
            sdX[i][j] = s;
        }
        __syncthreads();
        if (tid < 64) {    // dbeta and d gl from X; dV = diag(beta) dX
            const int i = tid;
            const float gi = __expf(sgl[i]);
            float db = 0.f, dg = 0.f;
            for (int j = 0; j < kBw3; ++j) {
                db += sdX[i][j] * (sV[i][j] - gi * sKS[i][j]);
                dg += sdX[i][j] * sKS[i][j];
            }
            sdb[i] += db;
            sdgl[i] -= sb[i] * gi * dg;
        }
        for (int idx = tid; idx < 64 * kBw3; idx += NT) {
            const int i = idx / kBw3, j = idx % kBw3;
            if (i < nv) p.dv[(tok0 + i) * vs + (int64_t)h * DV + c0 + j] = sb[i] * sdX[i][j];
        }
        for (int idx = tid; idx < 4096; idx += NT) {       // dA += dV' X^T, dPt += scale dO V'^T
            const int i = idx / 64, t = idx % 64;
            float a = 0.f, b = 0.f;
            for (int j = 0; j < kBw3; ++j) {
                a += sdVp[i][j] * sX[t][j];
                b += sdO[i][j] * sVp[t][j];
            }
            sdA[i][t] += a;
            sdP[i][t] += p.scale * b;
        }
#pragma unroll
        for (int e = 0; e < EPT; ++e) {                      // dq, dk terms through S and dS_next
            const int row = e * RS + tid / DK;
            const float gi = __expf(sgl[row]), Di = __expf(glC - sgl[row]);
            float a = 0.f, b = 0.f, x = 0.f;
            for (int j = 0; j < kBw3; ++j) {
                a += sdO[row][j] * sS[col][j];
                b += sVp[row][j] * sdS[col][j];
                x += sdX[row][j] * sS[col][j];
            }
            dq[e] += p.scale * gi * a;
            dk[e] += Di * b - sb[row] * gi * x;
        }
    }
    // d gl from the output's gamma: q_i . (scale gamma_i S dO_i), the inter-chunk dq accumulated so
    // far; the DK / 64 waves holding a row add their sums
    __syncthreads();   // the row-owner updates of sdgl above are done
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int row = e * RS + tid / DK;
        float x = sQ[row][col] * dq[e];
        for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
        if (lane == 0) atomicAdd(&sdgl[row], x);
    }
    __syncthreads();
    // dL = -A^T dA A^T (strictly lower), via T = A^T dA in the block space
    for (int idx = tid; idx < 4096; idx += NT) {
        const int i = idx / 64, j = idx % 64;
        float s = 0.f;
        for (int t = i; t < 64; ++t) s += sA[t][i] * sdA[t][j];
        sT[i][j] = s;
    }
    __syncthreads();
    for (int idx = tid; idx < 4096; idx += NT) {
        const int i = idx / 64, j = idx % 64;
        float s = 0.f;
        if (j < i)
            for (int t = 0; t <= j; ++t) s += sT[i][t] * sA[j][t];   // A lower: A[j][t] = 0 past t = j
        sdA[i][j] = j < i ? -s : 0.f;                        // sdA now holds dL
    }
    __syncthreads();
    for (int idx = tid; idx < 4096; idx += NT) {           // G (gated K K^T, strictly lower) over T
        const int i = idx / 64, j = idx % 64;
        float s = 0.f;
        if (j < i)
            for (int d = 0; d < DK; ++d) s += sK[i][d] * sK[j][d];
        sT[i][j] = j < i ? __expf(sgl[i] - sgl[j]) * s : 0.f;
    }
    __syncthreads();
    if (tid < 64) {        // dbeta and d gl from L = diag(beta) G, d gl from Pt
        const int i = tid;
        float db = 0.f, dg = 0.f;
        for (int j = 0; j < 64; ++j) {
            const float dpij = j <= i ? sdP[i][j] : 0.f, dpji = i <= j ? sdP[j][i] : 0.f;
            db += sdA[i][j] * sT[i][j];
            dg += sb[i] * sdA[i][j] * sT[i][j] - sb[j] * sdA[j][i] * sT[j][i];
            dg += dpij * sPt[i][j] - dpji * sPt[j][i];
        }
        sdb[i] += db;
        sdgl[i] += dg;
    }
    __syncthreads();
    for (int idx = tid; idx < 4096; idx += NT) {           // M1 = dPt (.) Gam over dP, E over dL
        const int i = idx / 64, j = idx % 64;
        const float f = __expf(sgl[i] - sgl[j]);
        sdP[i][j] = j <= i ? sdP[i][j] * f : 0.f;
        sdA[i][j] = j < i ? sdA[i][j] * sb[i] * f : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int row = e * RS + tid / DK;
        float a = 0.f, b = 0.f;
        for (int j = 0; j < 64; ++j) {
            a += sdP[row][j] * sK[j][col];
            b += sdP[j][row] * sQ[j][col] + (sdA[row][j] + sdA[j][row]) * sK[j][col];
        }
        dq[e] += a;
        dk[e] += b;
    }
    // gl_C: the last valid token; then dg = reverse cumsum of d gl within the chunk
    if (tid < 64) {
        float s = tid == 0 ? sdglC : 0.f;
        for (int j = 0; j < 64; ++j) s += tid == 0 ? sc[j] : 0.f;
        if (tid == 0) sdgl[max(nv - 1, 0)] += s;
    }
    __syncthreads();
    if (tid < 64) {
        const float x = tid < nv ? sdgl[tid] : 0.f;
        const float incl = wave_inclusive_scan(x);
        const float tot = __shfl(incl, 63, 64);
        if (tid < nv) {
            p.dg[(tok0 + tid) * p.H_v + h] = tot - incl + x;
            p.dbeta[(tok0 + tid) * p.H_v + h] = sdb[tid];
        }
    }
    float *dqo = p.dq_v, *dko = p.dk_v;      // per value head (fp32), reduced over groups later, or final
    const int hs = p.dq_v == p.dq ? hq : h, hn = p.dq_v == p.dq ? p.H_qk : p.H_v;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int row = e * RS + tid / DK;
        if (row < nv) {
            const int64_t o = ((tok0 + row) * hn + hs) * DK + col;
            dqo[o] = dq[e];
            dko[o] = dk[e];
        }
    }
}

// ==========================================================================================
// Per-channel gates (KDA walk-through, sections 3-5): the decay Diag(e^{G_t}) acts on the rows of
// S, G the chunk-local cumsum of the [D_k] log-gates.  Per chunk, with Kg = K (.) e^G,
// Kd = K (.) e^{G_C - G}, Qg = Q (.) e^G and the per-channel factors inside P and L,
//   forward:  X = diag(beta)(V - Kg S),  V' = A X,  O = scale (Qg S + P V'),
//             P_ij = sum_d q_id k_jd e^{G_id - G_jd} (j <= i),  S_next = Diag(e^{G_C}) S + Kd^T V'
//   backward: dV' = Kd dS_next + scale P^T dO,  dX = A^T dV',  dA = dV' X^T,  dL = -A^T dA A^T,
//             dS = Diag(e^{G_C}) dS_next + scale Qg^T dO - Kg^T diag(beta) dX,
//             dq = scale e^G (.) (dO S^T) + dq_P,  dq_P[i][d] = sum_{j<=i} dP_ij k_jd e^{G_id - G_jd},
//             dk = -diag(beta) e^G (.) (dX S^T) + e^{G_C - G} (.) (V' dS_next^T) + dk_P + dk_Lrow + dk_Lcol,
//             dG = q (.) dq + k (.) (dk_X + dk_Lrow) - k (.) (dk_D + dk_P + dk_Lcol), the e^{G_C} terms
//             on the last valid row, and dgk its reverse cumsum within the chunk per channel.
// Two kernels per chunk: (a) the products with S and dS_next over value-column blocks, dL; (b) the
// P and L terms with their per-channel factors.  The inverse A is read as the per-chunk kernel
// stores it for per-channel gates (fp16 for bf16 inputs).

// chunk-local cumsum of per-channel log-gates: G (fp32 LDS rows of stride ld) holds the raw gates
// of the chunk (zero past the end) on entry; the first DK threads scan one channel each
template <int DK>
__device__ __forceinline__ void cumsum_rows(float *G, int ld) {
    __syncthreads();
    if (threadIdx.x < DK) {
        float acc = 0.f;
        for (int i = 0; i < 64; ++i) {
            acc += G[i * ld + threadIdx.x];
            G[i * ld + threadIdx.x] = acc;
        }
    }
    __syncthreads();
}

template <typename T>
__device__ __forceinline__ void load_beta(const BwdParams &p, int64_t tok0, int nv, int h, float *sb) {
    const int lane = threadIdx.x & 63;
    sb[lane] = lane < nv ? to_f32(static_cast<const T *>(p.beta)[(tok0 + lane) * p.H_v + h]) : 0.f;
}

// ---- recomputed chunk states (per-channel gates)
template <typename T, int DK>
__global__ __launch_bounds__(kBwT) void bwd_states_kda_kernel(BwdParams p) {
    constexpr int NT = kBwT;
    __shared__ float sKg[64][DK + 1], sKd[64][DK + 1], sA[64][65];
    __shared__ float sS[DK][kBwR + 1], sV[64][kBwR + 1], sX[64][kBwR + 1], sVp[64][kBwR + 1];
    __shared__ float sb[64], sgc[DK];
    const int tid = threadIdx.x;
    const int ncb = p.D_v / kBwR;
    const int cb = blockIdx.x % ncb, nh = blockIdx.x / ncb, h = nh % p.H_v, n = nh / p.H_v;
    const int hq = h / (p.H_v / p.H_qk);
    const SeqInfo si = seq_info(p.seq, n, p.T);
    const int64_t DV = p.D_v, gks = (int64_t)p.H_v * DK;
    for (int idx = tid; idx < DK * kBwR; idx += NT) {
        const int d = idx / kBwR, j = idx % kBwR;
        sS[d][j] = p.h0 ? p.h0[(((int64_t)n * p.H_v + h) * DK + d) * DV + cb * kBwR + j] : 0.f;
    }
    for (int c = 0; c < si.nchunks; ++c) {
        const int64_t gci = si.chunk0 + c, tok0 = si.tok0 + (int64_t)c * kChunk;
        const int nv = min(kChunk, si.len - c * kChunk);
        __syncthreads();
        float *st = p.states + ((gci * p.H_v + h) * DK) * DV + cb * kBwR;
        for (int idx = tid; idx < DK * kBwR; idx += NT) st[(idx / kBwR) * DV + idx % kBwR] = sS[idx / kBwR][idx % kBwR];
        load_rows<DK, T, NT>(&sKg[0][0], DK + 1, static_cast<const T *>(p.k) + (int64_t)hq * DK, tok0, nv, (int64_t)p.H_qk * DK, 0);
        load_rows<DK, T, NT>(&sKd[0][0], DK + 1, static_cast<const T *>(p.g) + (int64_t)h * DK, tok0, nv, gks, 0);
        load_rows<kBwR, T, NT>(&sV[0][0], kBwR + 1, static_cast<const T *>(p.v) + (int64_t)h * DV, tok0, nv, (int64_t)p.H_v * DV, cb * kBwR);
        load_tile64<typename KdaOperand<T>::type, NT>(sA, static_cast<const typename KdaOperand<T>::type *>(p.A) + (gci * p.H_v + h) * 4096);
        if (tid < 64) load_beta<T>(p, tok0, nv, h, sb);
        cumsum_rows<DK>(&sKd[0][0], DK + 1);                 // sKd holds G
        if (tid < DK) sgc[tid] = sKd[63][tid];
        __syncthreads();
        for (int idx = tid; idx < 64 * DK; idx += NT) {    // Kg = K e^G, Kd = K e^{G_C - G}
            const int i = idx / DK, d = idx % DK;
            const float k = sKg[i][d], G = sKd[i][d];
            sKg[i][d] = k * __expf(G);
            sKd[i][d] = k * __expf(sgc[d] - G);
        }
        __syncthreads();
        for (int idx = tid; idx < 64 * kBwR; idx += NT) {   // X = beta (V - Kg S)
            const int i = idx / kBwR, j = idx % kBwR;
            float s = 0.f;
            for (int d = 0; d < DK; ++d) s += sKg[i][d] * sS[d][j];
            sX[i][j] = sb[i] * (sV[i][j] - s);
        }
        __syncthreads();
        for (int idx = tid; idx < 64 * kBwR; idx += NT) {   // V' = A X
            const int i = idx / kBwR, j = idx % kBwR;
            float s = 0.f;
            for (int t = 0; t <= i; ++t) s += sA[i][t] * sX[t][j];
            sVp[i][j] = s;
        }
        __syncthreads();
        for (int idx = tid; idx < DK * kBwR; idx += NT) {   // S = Diag(e^{G_C}) S + Kd^T V'
            const int d = idx / kBwR, j = idx % kBwR;
            float s = 0.f;
            for (int i = 0; i < 64; ++i) s += sKd[i][d] * sVp[i][j];
            sS[d][j] = __expf(sgc[d]) * sS[d][j] + s;
        }
    }
}

// ---- scale P of every (chunk, value head), per-channel factors inside the sum.  For a query below
//      key j's 16-row block the factor e^{G_id - G_jd} is split at the block's last row r
//      (j <= r < i), both parts at most 1, so one exponential per operand element replaces one per
//      term of the sum; pairs inside one block take the whole factor per term.  No factor exceeds 1,
//      whatever the gates.
template <typename T, int DK>
__global__ __launch_bounds__(kBwT) void bwd_p_kda_kernel(BwdParams p) {
    constexpr int NT = kBwT;
    __shared__ float sK[64][DK + 1], sQ[64][DK + 1], sG[64][DK + 1], sQx[64][DK + 1], sKx[16][DK + 1];
    const int tid = threadIdx.x;
    const int ci = blockIdx.x / p.H_v, h = blockIdx.x - ci * p.H_v;
    const int hq = h / (p.H_v / p.H_qk);
    const ChunkInfo cinfo = chunk_info(p.chunks, ci, p.T);
    const int64_t qks = (int64_t)p.H_qk * DK;
    load_rows<DK, T, NT>(&sK[0][0], DK + 1, static_cast<const T *>(p.k) + (int64_t)hq * DK, cinfo.tok0, cinfo.nv, qks, 0);
    load_rows<DK, T, NT>(&sQ[0][0], DK + 1, static_cast<const T *>(p.q) + (int64_t)hq * DK, cinfo.tok0, cinfo.nv, qks, 0);
    load_rows<DK, T, NT>(&sG[0][0], DK + 1, static_cast<const T *>(p.g) + (int64_t)h * DK, cinfo.tok0, cinfo.nv,
                         (int64_t)p.H_v * DK, 0);
    cumsum_rows<DK>(&sG[0][0], DK + 1);
    float *P = p.pmat + ((int64_t)ci * p.H_v + h) * 4096;
    for (int J = 0; J < 4; ++J) {                         // keys of block J: rows i >= 16 J
        // Queries below the block and the block's keys are split at its last row r, which lies
        // between every such pair: q_i e^{G_i - G_r} and k_j e^{G_r - G_j}, both at most their row.
        // Pairs inside the block have no such row and take their factor e^{G_i - G_j} <= 1 whole.
        const int r = 16 * J + 15;
        __syncthreads();                                  // sG ready; sQx, sKx free
        for (int idx = tid; idx < (48 - 16 * J) * DK; idx += NT) {
            const int i = 16 * J + 16 + idx / DK, d = idx % DK;
            sQx[i][d] = sQ[i][d] * __expf(sG[i][d] - sG[r][d]);
        }
        for (int idx = tid; idx < 16 * DK; idx += NT) {
            const int jj = idx / DK, d = idx % DK;
            sKx[jj][d] = sK[16 * J + jj][d] * __expf(sG[r][d] - sG[16 * J + jj][d]);
        }
        __syncthreads();
        for (int idx = tid; idx < 64 * 16; idx += NT) {
            const int i = idx / 16, jj = idx % 16, j = 16 * J + jj;
            if (i < 16 * J) continue;                     // above the diagonal: written below
            float s = 0.f;
            if (i > r) {
                for (int d = 0; d < DK; ++d) s += sQx[i][d] * sKx[jj][d];
            } else if (j <= i) {
                for (int d = 0; d < DK; ++d) s += sQ[i][d] * sK[j][d] * __expf(sG[i][d] - sG[j][d]);
            }
            P[i * 64 + j] = j <= i ? p.scale * s : 0.f;
        }
    }
    for (int idx = tid; idx < 4096; idx += NT) {          // the blocks above the diagonal
        const int i = idx / 64, j = idx % 64;
        if ((j >> 4) > (i >> 4)) P[idx] = 0.f;
    }
}

// ---- reverse scan of the state gradient (per-channel gates; kBwT threads)
template <typename T, int DK>
__global__ __launch_bounds__(kBwT) void bwd_dstate_kda_kernel(BwdParams p) {
    constexpr int NT = kBwT;
    __shared__ float sKd[64][DK + 1], sKg[64][DK + 1], sQg[64][DK + 1];
    __shared__ float sA[64][65], sP[64][65];
    __shared__ float sdS[DK][kBw + 1], sdO[64][kBw + 1], sKdS[64][kBw + 1], sdVp[64][kBw + 1], sdX[64][kBw + 1];
    __shared__ float sb[64], sgc[DK];
    const int tid = threadIdx.x;
    const int ncb = p.D_v / kBw;
    const int cb = blockIdx.x % ncb, nh = blockIdx.x / ncb, h = nh % p.H_v, n = nh / p.H_v;
    const int hq = h / (p.H_v / p.H_qk);
    const SeqInfo si = seq_info(p.seq, n, p.T);
    const int64_t DV = p.D_v;
    for (int idx = tid; idx < DK * kBw; idx += NT) {
        const int d = idx / kBw, j = idx % kBw;
        sdS[d][j] = p.dht ? p.dht[(((int64_t)n * p.H_v + h) * DK + d) * DV + cb * kBw + j] : 0.f;
    }
    for (int c = si.nchunks - 1; c >= 0; --c) {
        const int64_t gci = si.chunk0 + c, tok0 = si.tok0 + (int64_t)c * kChunk;
        const int nv = min(kChunk, si.len - c * kChunk);
        __syncthreads();
        float *dsn = p.dsnext + ((gci * p.H_v + h) * DK) * DV + cb * kBw;
        for (int idx = tid; idx < DK * kBw; idx += NT) dsn[(idx / kBw) * DV + idx % kBw] = sdS[idx / kBw][idx % kBw];
        const int64_t qks = (int64_t)p.H_qk * DK;
        load_rows<DK, T, NT>(&sKg[0][0], DK + 1, static_cast<const T *>(p.k) + (int64_t)hq * DK, tok0, nv, qks, 0);
        load_rows<DK, T, NT>(&sQg[0][0], DK + 1, static_cast<const T *>(p.q) + (int64_t)hq * DK, tok0, nv, qks, 0);
        load_rows<DK, T, NT>(&sKd[0][0], DK + 1, static_cast<const T *>(p.g) + (int64_t)h * DK, tok0, nv, (int64_t)p.H_v * DK, 0);
        load_rows<kBw, T, NT>(&sdO[0][0], kBw + 1, static_cast<const T *>(p.dout) + (int64_t)h * DV, tok0, nv, (int64_t)p.H_v * DV,
                       cb * kBw);
        load_tile64<typename KdaOperand<T>::type, NT>(sA, static_cast<const typename KdaOperand<T>::type *>(p.A) + (gci * p.H_v + h) * 4096);
        load_tile64<float, NT>(sP, p.pmat + (gci * p.H_v + h) * 4096);
        if (tid < 64) load_beta<T>(p, tok0, nv, h, sb);
        cumsum_rows<DK>(&sKd[0][0], DK + 1);                 // sKd holds G
        if (tid < DK) sgc[tid] = sKd[63][tid];
        __syncthreads();
        for (int idx = tid; idx < 64 * DK; idx += NT) {    // Kd, Kg, Qg
            const int i = idx / DK, d = idx % DK;
            const float G = sKd[i][d], e = __expf(G), k = sKg[i][d];
            sKd[i][d] = k * __expf(sgc[d] - G);
            sKg[i][d] = k * e;
            sQg[i][d] *= e;
        }
        __syncthreads();
        for (int idx = tid; idx < 64 * kBw; idx += NT) {   // Kd dS_next
            const int i = idx / kBw, j = idx % kBw;
            float s = 0.f;
            for (int d = 0; d < DK; ++d) s += sKd[i][d] * sdS[d][j];
            sKdS[i][j] = s;
        }
        __syncthreads();
        for (int idx = tid; idx < 64 * kBw; idx += NT) {   // dV' = Kd dS_next + scale P^T dO
            const int i = idx / kBw, j = idx % kBw;
            float s = sKdS[i][j];
            for (int t = i; t < 64; ++t) s += sP[t][i] * sdO[t][j];
            sdVp[i][j] = s;
        }
        __syncthreads();
        for (int idx = tid; idx < 64 * kBw; idx += NT) {   // dX = A^T dV'
            const int i = idx / kBw, j = idx % kBw;
            float s = 0.f;
            for (int t = i; t < 64; ++t) s += sA[t][i] * sdVp[t][j];
            sdX[i][j] = s;
        }
        __syncthreads();
        for (int idx = tid; idx < DK * kBw; idx += NT) {   // dS = Diag(e^{G_C}) dS_next + Qg^T(...) - Kg^T(...)
            const int d = idx / kBw, j = idx % kBw;
            float s = 0.f;
            for (int i = 0; i < 64; ++i) s += p.scale * sQg[i][d] * sdO[i][j] - sb[i] * sKg[i][d] * sdX[i][j];
            sdS[d][j] = __expf(sgc[d]) * sdS[d][j] + s;
        }
    }
    __syncthreads();
    if (p.dh0) {
        for (int idx = tid; idx < DK * kBw; idx += NT) {
            const int d = idx / kBw, j = idx % kBw;
            p.dh0[(((int64_t)n * p.H_v + h) * DK + d) * DV + cb * kBw + j] = sdS[d][j];
        }
    }
}

// the thread's G values down its column: rows e * RS + tid / DK of the chunk (G_C in *gc)
template <typename T, int DK, int EPT, int NT>
__device__ __forceinline__ void column_cumsum(const BwdParams &p, int64_t tok0, int nv, int h, float *Gr, float *gc) {
    constexpr int RS = NT / DK;
    const int col = threadIdx.x % DK, r0 = threadIdx.x / DK;
    const T *g = static_cast<const T *>(p.g) + (int64_t)h * DK + col;
    float acc = 0.f;
    int e = 0;
    for (int t = 0; t < 64; ++t) {
        if (t < nv) acc += to_f32(g[(tok0 + t) * p.H_v * DK]);
        if (e < EPT && t == e * RS + r0) Gr[e++] = acc;
    }
    *gc = acc;
}

// ---- (a) per (chunk, value head): the products with S and dS_next, dV, dbeta from X, dL
template <typename T, int DK>
__global__ __launch_bounds__(kBwT) void bwd_chunk_kda_a_kernel(BwdParams p) {
    constexpr int NT = kBwT;
    constexpr int EPT = 64 * DK / NT;
    constexpr int RS = NT / DK;
    constexpr int W3 = kBw3 + 1;
    __shared__ float sKg[64][DK + 1], sKd[64][DK + 1];
    __shared__ float sA[64][65], sP[64][65], sdA[64][65];
    constexpr int BLK = 2 * DK * W3 + 8 * 64 * W3;
    __shared__ float sBlk[BLK > 64 * 65 ? BLK : 64 * 65];
    __shared__ float sb[64], sdb[64], sgc[DK], sdgc[DK];
    float (*sS)[W3] = reinterpret_cast<float (*)[W3]>(sBlk);
    float (*sdS)[W3] = reinterpret_cast<float (*)[W3]>(sBlk + DK * W3);
    float (*sV)[W3] = reinterpret_cast<float (*)[W3]>(sBlk + 2 * DK * W3);
    float (*sdO)[W3] = sV + 64;
    float (*sKS)[W3] = sV + 2 * 64;
    float (*sX)[W3] = sV + 3 * 64;
    float (*sVp)[W3] = sV + 4 * 64;
    float (*sKdS)[W3] = sV + 5 * 64;
    float (*sdVp)[W3] = sV + 6 * 64;
    float (*sdX)[W3] = sV + 7 * 64;
    float (*sT)[65] = reinterpret_cast<float (*)[65]>(sBlk);

    const int tid = threadIdx.x;
    const int ci = blockIdx.x / p.H_v, h = blockIdx.x - ci * p.H_v;
    const int hq = h / (p.H_v / p.H_qk);
    const ChunkInfo cinfo = chunk_info(p.chunks, ci, p.T);
    const int64_t tok0 = cinfo.tok0;
    const int nv = cinfo.nv;
    const int64_t DV = p.D_v, qks = (int64_t)p.H_qk * DK, vs = (int64_t)p.H_v * DV;
    load_rows<DK, T, NT>(&sKg[0][0], DK + 1, static_cast<const T *>(p.k) + (int64_t)hq * DK, tok0, nv, qks, 0);
    load_rows<DK, T, NT>(&sKd[0][0], DK + 1, static_cast<const T *>(p.g) + (int64_t)h * DK, tok0, nv, (int64_t)p.H_v * DK, 0);
    load_tile64<typename KdaOperand<T>::type, NT>(sA, static_cast<const typename KdaOperand<T>::type *>(p.A) + ((int64_t)ci * p.H_v + h) * 4096);
    load_tile64<float, NT>(sP, p.pmat + ((int64_t)ci * p.H_v + h) * 4096);
    for (int idx = tid; idx < 4096; idx += NT) sdA[idx / 64][idx % 64] = 0.f;
    if (tid < 64) {
        load_beta<T>(p, tok0, nv, h, sb);
        sdb[tid] = 0.f;
    }
    cumsum_rows<DK>(&sKd[0][0], DK + 1);
    if (tid < DK) {
        sgc[tid] = sKd[63][tid];
        sdgc[tid] = 0.f;
    }
    __syncthreads();
    for (int idx = tid; idx < 64 * DK; idx += NT) {
        const int i = idx / DK, d = idx % DK;
        const float G = sKd[i][d], k = sKg[i][d];
        sKd[i][d] = k * __expf(sgc[d] - G);
        sKg[i][d] = k * __expf(G);
    }
    float accQ[EPT], accX[EPT], accD[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) accQ[e] = accX[e] = accD[e] = 0.f;
    const int col = tid % DK;
    const float *St = p.states + (((int64_t)ci * p.H_v + h) * DK) * DV;
    const float *dSt = p.dsnext + (((int64_t)ci * p.H_v + h) * DK) * DV;
    float *vpw = p.vp + ((int64_t)ci * p.H_v + h) * 64 * DV;
    for (int c0 = 0; c0 < p.D_v; c0 += kBw3) {
        __syncthreads();
        {
            constexpr int NE = (DK * kBw3 + NT - 1) / NT;   // threads past DK kBw3 elements idle
            float a[NE], b[NE];
#pragma unroll
            for (int it = 0; it < NE; ++it) {
                const int idx = min(tid + NT * it, DK * kBw3 - 1), d = idx / kBw3, j = idx % kBw3;
                a[it] = St[d * DV + c0 + j];
                b[it] = dSt[d * DV + c0 + j];
            }
#pragma unroll
            for (int it = 0; it < NE; ++it) {
                const int idx = tid + NT * it, d = idx / kBw3, j = idx % kBw3;
                if (idx < DK * kBw3) {
                    sS[d][j] = a[it];
                    sdS[d][j] = b[it];
                }
            }
        }
        load_rows<kBw3, T, NT>(&sV[0][0], W3, static_cast<const T *>(p.v) + (int64_t)h * DV, tok0, nv, vs, c0);
        load_rows<kBw3, T, NT>(&sdO[0][0], W3, static_cast<const T *>(p.dout) + (int64_t)h * DV, tok0, nv, vs, c0);
        __syncthreads();
        for (int idx = tid; idx < 64 * kBw3; idx += NT) {  // Kg S, Kd dS_next, X
            const int i = idx / kBw3, j = idx % kBw3;
            float a = 0.f, e = 0.f;
            for (int d = 0; d < DK; ++d) {
                a += sKg[i][d] * sS[d][j];
                e += sKd[i][d] * sdS[d][j];
            }
            sKS[i][j] = a;
            sKdS[i][j] = e;
            sX[i][j] = sb[i] * (sV[i][j] - a);
        }
        if (tid < DK) {    // e^{G_C} <S, dS_next> per channel (row d of both)
            float s = 0.f;
            for (int j = 0; j < kBw3; ++j) s += sS[tid][j] * sdS[tid][j];
            sdgc[tid] += __expf(sgc[tid]) * s;
        }
        __syncthreads();
        for (int idx = tid; idx < 64 * kBw3; idx += NT) {  // V' = A X
            const int i = idx / kBw3, j = idx % kBw3;
            float s = 0.f;
            for (int t = 0; t <= i; ++t) s += sA[i][t] * sX[t][j];
            sVp[i][j] = s;
            vpw[i * DV + c0 + j] = s;
        }
        __syncthreads();
        for (int idx = tid; idx < 64 * kBw3; idx += NT) {  // dV' = Kd dS_next + scale P^T dO
            const int i = idx / kBw3, j = idx % kBw3;
            float s = sKdS[i][j];
            for (int t = i; t < 64; ++t) s += sP[t][i] * sdO[t][j];
            sdVp[i][j] = s;
        }
        __syncthreads();
        for (int idx = tid; idx < 64 * kBw3; idx += NT) {  // dX = A^T dV'
            const int i = idx / kBw3, j = idx % kBw3;
            float s = 0.f;
            for (int t = i; t < 64; ++t) s += sA[t][i] * sdVp[t][j];
            sdX[i][j] = s;
        }
        __syncthreads();
        if (tid < 64) {    // dbeta from X
            float db = 0.f;
            for (int j = 0; j < kBw3; ++j) db += sdX[tid][j] * (sV[tid][j] - sKS[tid][j]);
            sdb[tid] += db;
        }
        for (int idx = tid; idx < 64 * kBw3; idx += NT) {
            const int i = idx / kBw3, j = idx % kBw3;
            if (i < nv) p.dv[(tok0 + i) * vs + (int64_t)h * DV + c0 + j] = sb[i] * sdX[i][j];
        }
        for (int idx = tid; idx < 4096; idx += NT) {       // dA += dV' X^T
            const int i = idx / 64, t = idx % 64;
            float a = 0.f;
            for (int j = 0; j < kBw3; ++j) a += sdVp[i][j] * sX[t][j];
            sdA[i][t] += a;
        }
#pragma unroll
        for (int e = 0; e < EPT; ++e) {                      // the raw products with S and dS_next
            const int row = e * RS + tid / DK;
            float a = 0.f, b = 0.f, x = 0.f;
            for (int j = 0; j < kBw3; ++j) {
                a += sdO[row][j] * sS[col][j];
                x += sdX[row][j] * sS[col][j];
                b += sVp[row][j] * sdS[col][j];
            }
            accQ[e] += a;
            accX[e] += x;
            accD[e] += b;
        }
    }
    __syncthreads();
    // dL = -A^T dA A^T (strictly lower), to the workspace
    for (int idx = tid; idx < 4096; idx += NT) {
        const int i = idx / 64, j = idx % 64;
        float s = 0.f;
        for (int t = i; t < 64; ++t) s += sA[t][i] * sdA[t][j];
        sT[i][j] = s;
    }
    __syncthreads();
    float *dLw = p.dlmat + ((int64_t)ci * p.H_v + h) * 4096;
    for (int idx = tid; idx < 4096; idx += NT) {
        const int i = idx / 64, j = idx % 64;
        float s = 0.f;
        if (j < i)
            for (int t = 0; t <= j; ++t) s += sT[i][t] * sA[j][t];
        dLw[idx] = j < i ? -s : 0.f;
    }
    // the gate factors of this thread's elements, then dq, dk and dG of these terms
    float Gr[EPT], gC;
    column_cumsum<T, DK, EPT, NT>(p, tok0, nv, h, Gr, &gC);
    const T *q = static_cast<const T *>(p.q) + (int64_t)hq * DK + col;
    const T *k = static_cast<const T *>(p.k) + (int64_t)hq * DK + col;
    float dgcs = 0.f;
    float dqo[EPT], dko[EPT], dGo[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int row = e * RS + tid / DK;
        const float qv = row < nv ? to_f32(q[(tok0 + row) * qks]) : 0.f;
        const float kv = row < nv ? to_f32(k[(tok0 + row) * qks]) : 0.f;
        const float eg = __expf(Gr[e]);
        const float dq_o = p.scale * eg * accQ[e];
        const float dk_x = -sb[row] * eg * accX[e];
        const float dk_d = __expf(gC - Gr[e]) * accD[e];
        dqo[e] = dq_o;
        dko[e] = dk_x + dk_d;
        // the last valid row's factor e^{G_C - G_C} = 1 has no gate gradient: its - (own row) and
        // + (G_C) terms would cancel exactly, so neither is added (see the diagonal pairs of (b))
        const float dgd = row == nv - 1 ? 0.f : kv * dk_d;
        dGo[e] = qv * dq_o + kv * dk_x - dgd;
        dgcs += dgd;
    }
    atomicAdd(&sdgc[col], dgcs);
    __syncthreads();
    const int hs = p.dq_v == p.dq ? hq : h, hn = p.dq_v == p.dq ? p.H_qk : p.H_v;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int row = e * RS + tid / DK;
        if (row < nv) {
            const int64_t o = ((tok0 + row) * hn + hs) * DK + col;
            p.dq_v[o] = dqo[e];
            p.dk_v[o] = dko[e];
            p.dg[((tok0 + row) * p.H_v + h) * DK + col] = dGo[e] + (row == nv - 1 ? sdgc[col] : 0.f);
        }
    }
    if (tid < nv) p.dbeta[(tok0 + tid) * p.H_v + h] = sdb[tid];
}

// ---- (b) per (chunk, value head): the P and L terms with their per-channel factors, then the
//      per-channel reverse cumsum of dG
template <typename T, int DK>
__global__ __launch_bounds__(kBwT) void bwd_chunk_kda_b_kernel(BwdParams p) {
    constexpr int NT = kBwT;
    constexpr int EPT = 64 * DK / NT;
    constexpr int RS = NT / DK;
    constexpr int W3 = kBw3 + 1;
    __shared__ float sK[64][DK + 1], sQ[64][DK + 1], sG[64][DK + 1];
    __shared__ float sdL[64][65], sdP[64][65];
    __shared__ float sdO[64][W3], sVp[64][W3];
    __shared__ float sb[64], sdb[64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int ci = blockIdx.x / p.H_v, h = blockIdx.x - ci * p.H_v;
    const int hq = h / (p.H_v / p.H_qk);
    const ChunkInfo cinfo = chunk_info(p.chunks, ci, p.T);
    const int64_t tok0 = cinfo.tok0;
    const int nv = cinfo.nv;
    const int64_t DV = p.D_v, qks = (int64_t)p.H_qk * DK, vs = (int64_t)p.H_v * DV;
    load_rows<DK, T, NT>(&sK[0][0], DK + 1, static_cast<const T *>(p.k) + (int64_t)hq * DK, tok0, nv, qks, 0);
    load_rows<DK, T, NT>(&sQ[0][0], DK + 1, static_cast<const T *>(p.q) + (int64_t)hq * DK, tok0, nv, qks, 0);
    load_rows<DK, T, NT>(&sG[0][0], DK + 1, static_cast<const T *>(p.g) + (int64_t)h * DK, tok0, nv, (int64_t)p.H_v * DK, 0);
    load_tile64<float, NT>(sdL, p.dlmat + ((int64_t)ci * p.H_v + h) * 4096);
    for (int idx = tid; idx < 4096; idx += NT) sdP[idx / 64][idx % 64] = 0.f;
    if (tid < 64) {
        load_beta<T>(p, tok0, nv, h, sb);
        sdb[tid] = 0.f;
    }
    cumsum_rows<DK>(&sG[0][0], DK + 1);
    // dP = scale dO V'^T (lower with diagonal), over value-column blocks
    const float *vpw = p.vp + ((int64_t)ci * p.H_v + h) * 64 * DV;
    for (int c0 = 0; c0 < p.D_v; c0 += kBw3) {
        __syncthreads();
        load_rows<kBw3, T, NT>(&sdO[0][0], W3, static_cast<const T *>(p.dout) + (int64_t)h * DV, tok0, nv, vs, c0);
        for (int idx = tid; idx < 64 * kBw3; idx += NT) sVp[idx / kBw3][idx % kBw3] = vpw[(idx / kBw3) * DV + c0 + idx % kBw3];
        __syncthreads();
        for (int idx = tid; idx < 4096; idx += NT) {
            const int i = idx / 64, t = idx % 64;
            float a = 0.f;
            for (int j = 0; j < kBw3; ++j) a += sdO[i][j] * sVp[t][j];
            sdP[i][t] += t <= i ? p.scale * a : 0.f;
        }
    }
    __syncthreads();
    const int col = tid % DK;
    float dqp[EPT], dkb[EPT], dGb[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int r = e * RS + tid / DK;
        const float Gr = sG[r][col], qr = sQ[r][col], kr = sK[r][col];
        float aq = 0.f, ar = 0.f, ap = 0.f, al = 0.f;
        for (int t = 0; t < 64; ++t) {
            if (t < r) {                                   // r as the row: e^{G_r - G_t}
                const float f = __expf(Gr - sG[t][col]);
                aq += sdP[r][t] * sK[t][col] * f;
                ar += sdL[r][t] * sK[t][col] * f;
            }
            if (t > r) {                                   // r as the column: e^{G_t - G_r}
                const float f = __expf(sG[t][col] - Gr);
                ap += sdP[t][r] * sQ[t][col] * f;
                al += sdL[t][r] * sb[t] * sK[t][col] * f;
            }
        }
        // the diagonal pair (t = r) has the factor e^0 = 1: it enters dq and dk, but its two gate
        // terms (+ as the row, - as the column) cancel exactly, so it is left out of dG rather than
        // added twice with opposite signs (which loses the small dG of steep gates to rounding)
        const float dpd = sdP[r][r];
        const float dk_lrow = sb[r] * ar;
        dqp[e] = aq + dpd * kr;
        dkb[e] = ap + dpd * qr + dk_lrow + al;
        dGb[e] = qr * aq + kr * dk_lrow - kr * (ap + al);
        float x = kr * ar;                                  // dbeta from L: sum_d k_rd R_rd
        for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
        if (lane == 0) atomicAdd(&sdb[r], x);
    }
    __syncthreads();
    // finish dq, dk, dG; dG into the Q tile (every thread is done with Q) for the reverse cumsum
    const int hs = p.dq_v == p.dq ? hq : h, hn = p.dq_v == p.dq ? p.H_qk : p.H_v;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int r = e * RS + tid / DK;
        float dG = 0.f;
        if (r < nv) {
            const int64_t o = ((tok0 + r) * hn + hs) * DK + col;
            p.dq_v[o] += dqp[e];
            p.dk_v[o] += dkb[e];
            dG = p.dg[((tok0 + r) * p.H_v + h) * DK + col] + dGb[e];
        }
        sQ[r][col] = dG;
    }
    __syncthreads();
    if (tid < DK) {
        float acc = 0.f;
        for (int t = nv - 1; t >= 0; --t) {
            acc += sQ[t][tid];
            p.dg[((tok0 + t) * p.H_v + h) * DK + tid] = acc;
        }
    }
    if (tid < nv) p.dbeta[(tok0 + tid) * p.H_v + h] += sdb[tid];
}

// dq, dk of a query/key head: the sum over the value heads of its group
__global__ __launch_bounds__(256) void bwd_group_sum_kernel(BwdParams p, int DK, int64_t n) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= n) return;
    const int G = p.H_v / p.H_qk;
    const int64_t d = idx % DK, th = idx / DK, hq = th % p.H_qk, t = th / p.H_qk;
    float a = 0.f, b = 0.f;
    for (int g = 0; g < G; ++g) {
        const int64_t o = (t * p.H_v + hq * G + g) * DK + d;
        a += p.dq_v[o];
        b += p.dk_v[o];
    }
    p.dq[idx] = a;
    p.dk[idx] = b;
}

}  // namespace

// Grid of the matrix-core dS scans, one workgroup per (sequence, head, 32 value columns), mapped so
// that the column blocks of one (sequence, head) share blockIdx % 8, i.e. one XCD and its L2: the
// K, A, P and gate tiles one block fetches are then L2 hits for the others (with consecutive
// blocks on different XCDs the per-channel scan read 4.97 GB per step on the KDA shape, four
// copies of its tiles).
static int64_t scan_grid(const BwdParams &p) {
    return ((int64_t)p.N * p.H_v + 7) / 8 * 8 * (p.D_v / 32);
}

hipError_t launch_bwd(int dtype, int D_k, const BwdParams &p, hipStream_t s) {
    if (p.channel) {
        const int64_t scans = (int64_t)p.N * p.H_v * (p.D_v / kBw), chunks = (int64_t)p.n_chunks * p.H_v;
        const int64_t replays = (int64_t)p.N * p.H_v * (p.D_v / kBwR), mscans = scan_grid(p);
        if (scans == 0) return hipSuccess;
// every kernel of the backward runs kBwT threads per workgroup
#define GDN_BWDK(K, T, DK, grid) hipLaunchKernelGGL((K<T, DK>), dim3((unsigned)(grid)), dim3(kBwT), 0, s, p)
#define GDN_BWDK_ALL(T, DK)                                  \
    if (!p.replayed) GDN_BWDK(bwd_states_kda_kernel, T, DK, replays); \
    /* bf16 inputs read the per-chunk kernel's scale P instead */ \
    if (chunks && sizeof(T) != 2) GDN_BWDK(bwd_p_kda_kernel, T, DK, chunks); \
    if (sizeof(T) == 2)                                      \
        hipLaunchKernelGGL((bwd_dstate_kda_mma_kernel<DK>), dim3((unsigned)mscans), dim3(256), 0, s, p); \
    else                                                     \
        GDN_BWDK(bwd_dstate_kda_kernel, T, DK, scans);       \
    if (chunks) {                                            \
        if (sizeof(T) == 2) {                                \
            const hipError_t em = launch_bwd_chunk_kda_mma(DK, p, s); \
            if (em != hipSuccess) return em;                 \
        } else {                                             \
            GDN_BWDK(bwd_chunk_kda_a_kernel, T, DK, chunks); \
            GDN_BWDK(bwd_chunk_kda_b_kernel, T, DK, chunks); \
        }                                                    \
    }
        if (dtype == 1 && D_k == 128) { GDN_BWDK_ALL(bf16, 128) }
        else if (dtype == 1 && D_k == 64) { GDN_BWDK_ALL(bf16, 64) }
        else if (dtype == 0 && D_k == 128) { GDN_BWDK_ALL(float, 128) }
        else if (dtype == 0 && D_k == 64) { GDN_BWDK_ALL(float, 64) }
        else return hipErrorInvalidValue;
#undef GDN_BWDK_ALL
#undef GDN_BWDK
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || p.dq_v == p.dq) return e;
        const int64_t n = (int64_t)p.T_total * p.H_qk * D_k;
        if (n) hipLaunchKernelGGL(bwd_group_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, D_k, n);
        return hipGetLastError();
    }
    const int64_t scans = (int64_t)p.N * p.H_v * (p.D_v / kBwR), rscans = (int64_t)p.N * p.H_v * (p.D_v / kBwD);
    const int64_t mscans = scan_grid(p);
    const int64_t chunks = (int64_t)p.n_chunks * p.H_v;
    if (scans == 0) return hipSuccess;
#define GDN_BWD(K, T, DK, grid) hipLaunchKernelGGL((K<T, DK>), dim3((unsigned)(grid)), dim3(kBwT), 0, s, p)
#define GDN_BWD_ALL(T, DK)                                                                                 \
    if (!p.replayed) GDN_BWD(bwd_states_kernel, T, DK, scans);                                             \
    if (chunks) {                                                                                          \
        /* bf16: the replay (chunk_kernel's state-storing build) has formed scale P already */           \
        if (sizeof(T) == 2) { if (!p.replayed) hipLaunchKernelGGL((bwd_p_mma_kernel<DK>), dim3((unsigned)chunks), dim3(256), 0, s, p); } \
        else GDN_BWD(bwd_p_kernel, T, DK, chunks);                                                         \
    }                                                                                                      \
    if (sizeof(T) == 2)                                                                                    \
        hipLaunchKernelGGL((bwd_dstate_mma_kernel<DK>), dim3((unsigned)mscans), dim3(256), 0, s, p);      \
    else                                                                                                   \
        GDN_BWD(bwd_dstate_kernel, T, DK, rscans);                                                         \
    if (chunks) {                                                                                          \
        if (sizeof(T) == 2) {                                                                              \
            const hipError_t em = launch_bwd_chunk_mma(DK, p, s);                                          \
            if (em != hipSuccess) return em;                                                               \
        } else {                                                                                           \
            GDN_BWD(bwd_chunk_kernel, T, DK, chunks);                                                      \
        }                                                                                                  \
    }
    if (dtype == 1 && D_k == 128) { GDN_BWD_ALL(bf16, 128) }
    else if (dtype == 1 && D_k == 64) { GDN_BWD_ALL(bf16, 64) }
    else if (dtype == 0 && D_k == 128) { GDN_BWD_ALL(float, 128) }
    else if (dtype == 0 && D_k == 64) { GDN_BWD_ALL(float, 64) }
    else return hipErrorInvalidValue;
#undef GDN_BWD_ALL
#undef GDN_BWD
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.dq_v != p.dq) {
        const int64_t n = (int64_t)p.T_total * p.H_qk * D_k;
        if (n) hipLaunchKernelGGL(bwd_group_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, D_k, n);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace gdn
