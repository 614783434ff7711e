// Kernels (b)+(d): the serial inter-chunk state recurrence fused with the chunk output, and the
// device-side plan kernel (sequence and chunk tables for packed variable-length input).
//
// Per chunk (FlashQLA announcement (Qwen), the four-step forward for chunk i, in its rewritten
// form V^Delta = V - diag(gamma) K S, V' = A diag(beta) V^Delta -- equal to U - W S with the
// WY factors W = A diag(beta) diag(gamma) K, U = A diag(beta) V, which are applied here and
// never written to memory):
//   X   = diag(beta) (V - diag(gamma) K S)
//   V'  = A X
//   O   = scale (diag(gamma) Q S + (Lower(Gamma) (.) Q K^T) V')          (mask includes diagonal)
//   S  <- gamma_C S + K^T diag(gamma_C / gamma) V'                       (stored state is the
//                                                                         entering one: 06 . Flash
//                                                                         Linear Attention sec. 2, 6)
// One workgroup owns one (sequence, value head, slice of BV value columns): the columns of the
// state evolve independently (06 . Flash Linear Attention, section 6: the delta rule cannot split
// D_k, it can split D_v).  The fp32 state [D_k, BV] stays in VGPRs for the whole sequence; each
// wave owns D_k/4 of its rows.  A bf16 (or fp32) copy of it goes to LDS once per chunk as the
// matrix-core operand of K S and Q S.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

// ------------------------------------------------------------------------------------------
// Plan: sequence table, chunk table and a longest-first order of the sequences.
// One workgroup of 256 threads.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void plan_kernel(PlanParams p) {
    __shared__ int sScan[256];
    const int tid = threadIdx.x;
    // every chunk entry starts empty (nv = 0: the intra kernel then reads nothing)
    for (int i = tid; i < p.total_chunks; i += 256) p.chunks[i] = ChunkInfo{0, 0};
    int carry = 0;
    for (int base = 0; base < p.N; base += 256) {
        const int n = base + tid;
        int tok0 = 0, len = 0;
        if (n < p.N) {
            tok0 = p.cu ? p.cu[n] : n * p.T;
            len = p.cu ? p.cu[n + 1] - p.cu[n] : p.T;
            // the host validated its copy of cu_seqlens; clamp so that a device copy that
            // disagrees can never index past the token axis
            tok0 = min(max(tok0, 0), p.total_tokens);
            len = min(max(len, 0), p.total_tokens - tok0);
        }
        const int nc = (len + kChunk - 1) / kChunk;
        sScan[tid] = nc;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int y = tid >= off ? sScan[tid - off] : 0;
            __syncthreads();
            sScan[tid] += y;
            __syncthreads();
        }
        if (n < p.N) {
            // never more chunks than the host sized the workspace and the intra grid for
            const int chunk0 = min(carry + sScan[tid] - nc, p.total_chunks);
            const int ncc = min(nc, p.total_chunks - chunk0);
            p.seq[n] = SeqInfo{tok0, min(len, ncc * kChunk), chunk0, ncc};
        }
        carry += sScan[255];
        __syncthreads();
    }
    __syncthreads();
    for (int n = tid; n < p.N; n += 256) {
        const SeqInfo si = p.seq[n];
        for (int c = 0; c < si.nchunks; ++c) {
            const int rem = si.len - c * kChunk;
            p.chunks[si.chunk0 + c] = ChunkInfo{si.tok0 + c * kChunk, rem < kChunk ? rem : kChunk};
        }
    }
    // rank sort (longest first, ties by index); identity for the batched form and very many sequences
    const bool sort = p.cu != nullptr && p.N <= 4096;
    for (int n = tid; n < p.N; n += 256) {
        int rank = n;
        if (sort) {
            const int len = p.seq[n].len;
            rank = 0;
            for (int m = 0; m < p.N; ++m) {
                const int lm = p.seq[m].len;
                rank += (lm > len) || (lm == len && m < n);
            }
        }
        p.order[rank] = n;
    }
}

// ------------------------------------------------------------------------------------------
// Register staging of one chunk's global tiles (loaded one chunk ahead): vectors per thread.
// ------------------------------------------------------------------------------------------
template <typename T, int DK, int BV>
struct Stage {
    static constexpr int VEC = Vec16<T>::N;
    static constexpr int QV = 64 * DK / VEC / 256;                 // 16-byte vectors per thread (Q, K)
    static constexpr int AV = 64 * 64 / VEC / 256;                 // (A)
    static constexpr int VV = (64 * BV / VEC + 255) / 256;         // (V slice)
};

// LDS carve-up of the recurrence kernel (element offsets in T).
template <typename T, int DK, int BV>
struct ChunkLds {
    static constexpr int VEC = Vec16<T>::N;
    static constexpr int KP = DK + VEC;   // row stride of [*, DK] tiles (padded against bank conflicts)
    static constexpr int TP = 64 + VEC;   // row stride of [*, 64] tiles
    static constexpr int NS = Split<T>::parts;
    static constexpr int Q = 0, K = Q + 64 * KP, A = K + 64 * KP;
    static constexpr int P = A + 64 * TP;                 // NS x [64][TP]   scale * Lower(Gamma) (.) Q K^T
    static constexpr int St = P + NS * 64 * TP;           // NS x [BV][KP]   S^T
    static constexpr int Xt = St + NS * BV * KP;          // NS x [BV][TP]   X^T
    static constexpr int V = Xt + NS * BV * TP;           // [64][BV]        V slice
    static constexpr int VP_BYTES = 2 * NS * BV * TP;     // V'^T and V''^T = (diag(gamma_C/gamma) V')^T
    static constexpr bool VP_IN_Q = VP_BYTES <= 64 * KP;  // alias them onto Q once Q is consumed
    static constexpr int Vp = VP_IN_Q ? Q : V + 64 * BV;
    static constexpr int END = VP_IN_Q ? V + 64 * BV : Vp + VP_BYTES;
    static constexpr int BYTES = END * (int)sizeof(T);
};

template <typename T, int DK, int BV>
__global__ __launch_bounds__(256) void chunk_kernel(ChunkParams p) {
    using St = Stage<T, DK, BV>;
    using L = ChunkLds<T, DK, BV>;
    constexpr int VEC = St::VEC, KP = L::KP, TP = L::TP;
    constexpr bool SPLIT = Split<T>::parts == 2;
    constexpr int NT = BV / 16;    // value-column tiles
    constexpr int MT = DK / 64;    // 16-row state tiles per wave
    constexpr int VPR = DK / VEC;  // vectors per Q/K row
    constexpr int VPV = BV / VEC;  // vectors per V-slice row

    __shared__ __attribute__((aligned(16))) T smem[L::END];
    __shared__ float sGl[64], sB[64], sSc[64];
    T *sQ = smem + L::Q, *sK = smem + L::K, *sA = smem + L::A, *sV = smem + L::V;
    T *sPh = smem + L::P, *sPl = sPh + (SPLIT ? 64 * TP : 0);
    T *sSth = smem + L::St, *sStl = sSth + (SPLIT ? BV * KP : 0);
    T *sXth = smem + L::Xt, *sXtl = sXth + (SPLIT ? BV * TP : 0);
    T *sVph = smem + L::Vp, *sVpl = sVph + (SPLIT ? BV * TP : 0);          // V'^T
    T *sVqh = sVph + L::NS * BV * TP, *sVql = sVqh + (SPLIT ? BV * TP : 0);  // V''^T

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, grp = lane >> 4;

    // XCD-aware mapping: the slices of one (sequence, head) share blockIdx % 8, i.e. one XCD and
    // its L2, so Q/K/A tiles fetched by one slice are L2 hits for the others.
    const int bid = blockIdx.x, xcd = bid & 7, rr = bid >> 3;
    const int slice = rr % p.n_slices, unit = (rr / p.n_slices) * 8 + xcd;
    if (unit >= p.N * p.H_v) return;
    const int n = p.seq ? p.order[unit / p.H_v] : unit / p.H_v, h = unit % p.H_v;
    const int hq = h / (p.H_v / p.H_qk);
    const SeqInfo si = seq_info(p.seq, n, p.T);
    const int DV = p.D_v, c0 = slice * BV;

    const T *qb = static_cast<const T *>(p.q) + (int64_t)hq * DK;
    const T *kb_ = static_cast<const T *>(p.k) + (int64_t)hq * DK;
    const T *vb = static_cast<const T *>(p.v) + (int64_t)h * DV + c0;
    const float *gb = static_cast<const float *>(p.g) + h;
    const T *bb = static_cast<const T *>(p.beta) + h;
    const T *Ab = static_cast<const T *>(p.A) + (int64_t)h * 4096;
    const int64_t o_off = (int64_t)h * DV + c0;
    const int64_t qk_stride = (int64_t)p.H_qk * DK, v_stride = (int64_t)p.H_v * DV;

    // Loads are issued unconditionally from rows clamped into the chunk (every address stays in
    // bounds) and the tail is masked when the data is staged, so no load sits behind a branch that
    // would force a wait for it.
    u32x4 rq[St::QV], rk[St::QV], ra[St::AV], rv[St::VV];
    float rg, rb;
    auto load = [&](int c) __attribute__((always_inline)) {
        const int tok = si.tok0 + c * kChunk;
        const int last = min(kChunk, si.len - c * kChunk) - 1;
#pragma unroll
        for (int i = 0; i < St::QV; ++i) {
            const int idx = tid + 256 * i, row = min(idx / VPR, last), cv = idx % VPR;
            rq[i] = *reinterpret_cast<const u32x4 *>(qb + (tok + row) * qk_stride + cv * VEC);
            rk[i] = *reinterpret_cast<const u32x4 *>(kb_ + (tok + row) * qk_stride + cv * VEC);
        }
        const T *Ac = Ab + (int64_t)(si.chunk0 + c) * p.H_v * 4096;
#pragma unroll
        for (int i = 0; i < St::AV; ++i) ra[i] = reinterpret_cast<const u32x4 *>(Ac)[tid + 256 * i];
#pragma unroll
        for (int i = 0; i < St::VV; ++i) {
            const int idx = min(tid + 256 * i, 64 * VPV - 1), row = min(idx / VPV, last), cv = idx % VPV;
            rv[i] = *reinterpret_cast<const u32x4 *>(vb + (tok + row) * v_stride + cv * VEC);
        }
        const int tl = min(lane, last);
        rg = gb[(int64_t)(tok + tl) * p.H_v];
        rb = to_f32(bb[(int64_t)(tok + tl) * p.H_v]);
    };

    // ---- initial state (fp32 registers) and its matrix-core copy
    const int drow0 = wave * (DK / 4);
    f32x4 S[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = drow0 + 16 * mt + 4 * grp + r, col = c0 + 16 * nt + l16;
                S[mt][nt][r] = p.h0 ? p.h0[(((int64_t)n * p.H_v + h) * DK + d) * DV + col] : 0.f;
            }
            const int off = (16 * nt + l16) * KP + drow0 + 16 * mt + 4 * grp;
            st4_split(sSth + off, sStl + off, S[mt][nt]);
        }
    // P's upper tiles inside the contraction blocks that are used: (0,1) and (2,3); never rewritten
    for (int idx = tid; idx < 2 * 16 * 16; idx += 256) {
        const int tsel = idx >> 8, e = idx & 255, rrow = e >> 4, ccol = e & 15;
        const int off = (tsel ? 32 + rrow : rrow) * TP + (tsel ? 48 + ccol : 16 + ccol);
        sPh[off] = from_f32<T>(0.f);
        sPl[off] = from_f32<T>(0.f);
    }

    if (si.nchunks > 0) load(0);

    for (int c = 0; c < si.nchunks; ++c) {
        const int nv = min(kChunk, si.len - c * kChunk);
        const int tokc = si.tok0 + c * kChunk;
        __syncthreads();  // the previous chunk is done with every LDS tile

        // ---- stage chunk c (rows past the chunk end become zero)
        const u32x4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < St::QV; ++i) {
            const int idx = tid + 256 * i, row = idx / VPR, cv = idx - row * VPR;
            *reinterpret_cast<u32x4 *>(sQ + row * KP + cv * VEC) = row < nv ? rq[i] : z4;
            *reinterpret_cast<u32x4 *>(sK + row * KP + cv * VEC) = row < nv ? rk[i] : z4;
        }
#pragma unroll
        for (int i = 0; i < St::AV; ++i) {
            const int idx = tid + 256 * i, row = idx / (64 / VEC), cv = idx - row * (64 / VEC);
            *reinterpret_cast<u32x4 *>(sA + row * TP + cv * VEC) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < St::VV; ++i) {
            const int idx = tid + 256 * i;
            if (idx < 64 * VPV) reinterpret_cast<u32x4 *>(sV)[idx] = (idx / VPV) < nv ? rv[i] : z4;
        }
        const float gv = lane < nv ? rg : 0.f, bv = lane < nv ? rb : 0.f;
        const float gl = wave_inclusive_scan(gv) * kLog2e;    // lane t: log2 gamma_t
        const float glC = __shfl(gl, 63, 64);                  // tail tokens carry g = 0
        if (wave == 0) {
            sGl[lane] = gl;
            sB[lane] = bv;
            sSc[lane] = exp2f(glC - gl);                       // gamma_C / gamma_t
        }
        load(min(c + 1, si.nchunks - 1));                      // overlaps with the compute below
        __syncthreads();

        // ---- P = scale * Lower(Gamma) (.) Q K^T, built as P^T tiles (rows of P land contiguous)
        for (int t = wave; t < 10; t += 4) {
            const int ti = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
            const int tj = t - ti * (ti + 1) / 2;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb)
                mma(acc, ld8(sK + (16 * tj + l16) * KP + 32 * kb + 8 * grp),
                    ld8(sQ + (16 * ti + l16) * KP + 32 * kb + 8 * grp));
            const int i = 16 * ti + l16;  // acc[r] = (Q K^T)[i][16 tj + 4 grp + r]
            const float gli = sGl[i];
            f32x4 pv;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * tj + 4 * grp + r;
                pv[r] = (j <= i) ? p.scale * exp2f(gli - sGl[j]) * acc[r] : 0.f;
            }
            const int off = i * TP + 16 * tj + 4 * grp;
            st4_split(sPh + off, sPl + off, pv);
        }

        // ---- K S and Q S for rows 16w .. 16w+15 (S carried as hi + lo)
        f32x4 ks[NT], oacc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            ks[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            oacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
            const auto ak = ld8(sK + (16 * wave + l16) * KP + 32 * kb + 8 * grp);
            const auto aq = ld8(sQ + (16 * wave + l16) * KP + 32 * kb + 8 * grp);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int off = (16 * nt + l16) * KP + 32 * kb + 8 * grp;
                const auto bh = ld8(sSth + off);
                mma(ks[nt], ak, bh);
                mma(oacc[nt], aq, bh);
                if constexpr (SPLIT) {
                    const auto bl = ld8(sStl + off);
                    mma(ks[nt], ak, bl);
                    mma(oacc[nt], aq, bl);
                }
            }
        }
        // ---- X = diag(beta)(V - diag(gamma) K S) -> X^T; O_inter = scale diag(gamma) Q S
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 x;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * wave + 4 * grp + r;
                const float gam = exp2f(sGl[i]);
                x[r] = sB[i] * (to_f32(sV[i * BV + 16 * nt + l16]) - gam * ks[nt][r]);
                oacc[nt][r] *= p.scale * gam;
            }
            const int off = (16 * nt + l16) * TP + 16 * wave + 4 * grp;
            st4_split(sXth + off, sXtl + off, x);
        }
        __syncthreads();

        // ---- V' = A X for rows 16w.. (A lower triangular: blocks past the diagonal skipped);
        //      also V'' = diag(gamma_C / gamma) V' for the state update
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int kb = 0; kb <= (wave >> 1); ++kb) {
                const auto a = ld8(sA + (16 * wave + l16) * TP + 32 * kb + 8 * grp);
                const int off = (16 * nt + l16) * TP + 32 * kb + 8 * grp;
                mma(acc, a, ld8(sXth + off));
                if constexpr (SPLIT) mma(acc, a, ld8(sXtl + off));
            }
            const int off = (16 * nt + l16) * TP + 16 * wave + 4 * grp;
            st4_split(sVph + off, sVpl + off, acc);
            f32x4 accs;
#pragma unroll
            for (int r = 0; r < 4; ++r) accs[r] = acc[r] * sSc[16 * wave + 4 * grp + r];
            st4_split(sVqh + off, sVql + off, accs);
        }
        __syncthreads();

        // ---- O = O_inter + P V' (rows 16w..), both factors carried as hi + lo
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            for (int kb = 0; kb <= (wave >> 1); ++kb) {
                const int pa = (16 * wave + l16) * TP + 32 * kb + 8 * grp;
                const int vo = (16 * nt + l16) * TP + 32 * kb + 8 * grp;
                const auto ph = ld8(sPh + pa);
                const auto vh = ld8(sVph + vo);
                mma(oacc[nt], ph, vh);
                if constexpr (SPLIT) {
                    mma(oacc[nt], ph, ld8(sVpl + vo));
                    mma(oacc[nt], ld8(sPl + pa), vh);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * wave + 4 * grp + r;
                if (i < nv) {
                    const int64_t e = (int64_t)(tokc + i) * v_stride + o_off + 16 * nt + l16;
                    if (p.o_f32) static_cast<float *>(p.o)[e] = oacc[nt][r];
                    else static_cast<T *>(p.o)[e] = from_f32<T>(oacc[nt][r]);
                }
            }
        }

        // ---- S <- gamma_C S + K^T V''   (rows drow0 .. drow0 + DK/4; K columns read from the row tile)
        const float gC = exp2f(glC);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            Frag<T> a[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 8; ++e) set_elem(a[kb], e, sK[(32 * kb + 8 * grp + e) * KP + drow0 + 16 * mt + l16]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                S[mt][nt] *= gC;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int vo = (16 * nt + l16) * TP + 32 * kb + 8 * grp;
                    mma(S[mt][nt], a[kb], ld8(sVqh + vo));
                    if constexpr (SPLIT) mma(S[mt][nt], a[kb], ld8(sVql + vo));
                }
                const int off = (16 * nt + l16) * KP + drow0 + 16 * mt + 4 * grp;
                st4_split(sSth + off, sStl + off, S[mt][nt]);
            }
        }
    }

    if (p.final_state) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int d = drow0 + 16 * mt + 4 * grp + r, col = c0 + 16 * nt + l16;
                    p.final_state[(((int64_t)n * p.H_v + h) * DK + d) * DV + col] = S[mt][nt][r];
                }
    }
}

}  // namespace

hipError_t launch_plan(const PlanParams &p, hipStream_t s) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_chunk(int dtype, int D_k, int BV, const ChunkParams &p, hipStream_t s) {
    const int units = p.N * p.H_v;
    const unsigned groups = (unsigned)((units + 7) / 8);
    const dim3 grid(groups * 8u * (unsigned)p.n_slices), block(256);
    if (units == 0) return hipSuccess;
#define GDN_CHUNK_CASE(DT, T_, DK_, BV_)                                                        \
    if (dtype == DT && D_k == DK_ && BV == BV_) {                                               \
        hipLaunchKernelGGL((chunk_kernel<T_, DK_, BV_>), grid, block, 0, s, p);                 \
        return hipGetLastError();                                                               \
    }
    GDN_CHUNK_CASE(1, bf16, 128, 32)
    GDN_CHUNK_CASE(1, bf16, 128, 16)
    GDN_CHUNK_CASE(1, bf16, 64, 32)
    GDN_CHUNK_CASE(1, bf16, 64, 16)
    GDN_CHUNK_CASE(0, float, 128, 16)
    GDN_CHUNK_CASE(0, float, 64, 16)
#undef GDN_CHUNK_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdn
