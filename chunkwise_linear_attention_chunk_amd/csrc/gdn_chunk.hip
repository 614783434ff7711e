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
// Plan: sequence, chunk and segment tables, and a longest-first order of the segments.
// One workgroup of 256 threads.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void plan_kernel(PlanParams p) {
    __shared__ int sC[256], sS[256];
    const int tid = threadIdx.x;
    // every chunk entry starts empty (nv = 0: the intra kernel then reads nothing), every segment
    // entry empty and not last (it then writes no final state)
    for (int i = tid; i < p.total_chunks; i += 256) p.chunks[i] = ChunkInfo{0, 0};
    for (int i = tid; i < p.total_segs; i += 256) p.segs[i] = SegInfo{0, 0, 0, 0, 0};
    __syncthreads();
    int carry_c = 0, carry_s = 0;
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
        const int nc = n < p.N ? ceil_div(len, kChunk) : 0;
        const int ns = n < p.N ? max(1, ceil_div(nc, p.seg_chunks)) : 0;
        sC[tid] = nc;
        sS[tid] = ns;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int yc = tid >= off ? sC[tid - off] : 0, ys = tid >= off ? sS[tid - off] : 0;
            __syncthreads();
            sC[tid] += yc;
            sS[tid] += ys;
            __syncthreads();
        }
        if (n < p.N) {
            // never more chunks or segments than the host sized the workspace and grids for
            const int chunk0 = min(carry_c + sC[tid] - nc, p.total_chunks);
            const int ncc = min(nc, p.total_chunks - chunk0);
            const int seg0 = min(carry_s + sS[tid] - ns, p.total_segs);
            p.seq[n] = SeqInfo{tok0, min(len, ncc * kChunk), chunk0, ncc, seg0};
        }
        carry_c += sC[255];
        carry_s += sS[255];
        __syncthreads();
    }
    __syncthreads();
    for (int n = tid; n < p.N; n += 256) {
        const SeqInfo si = p.seq[n];
        for (int c = 0; c < si.nchunks; ++c) {
            const int rem = si.len - c * kChunk;
            p.chunks[si.chunk0 + c] = ChunkInfo{si.tok0 + c * kChunk, rem < kChunk ? rem : kChunk};
        }
        const int ns = max(1, ceil_div(si.nchunks, p.seg_chunks));
        for (int j = 0; j < ns && si.seg0 + j < p.total_segs; ++j) {
            const int c0 = j * p.seg_chunks;
            p.segs[si.seg0 + j] = SegInfo{n, j, c0, max(0, min(p.seg_chunks, si.nchunks - c0)), j == ns - 1 ? 1 : 0};
        }
    }
    __syncthreads();
    // rank sort of the segments (longest first, ties by index); identity past 1024 segments
    const bool sort = p.total_segs <= 1024;
    for (int g = tid; g < p.total_segs; g += 256) {
        int rank = g;
        if (sort) {
            const int len = p.segs[g].nchunks;
            rank = 0;
            for (int m = 0; m < p.total_segs; ++m) {
                const int lm = p.segs[m].nchunks;
                rank += (lm > len) || (lm == len && m < g);
            }
        }
        p.order[rank] = g;
    }
}

// ------------------------------------------------------------------------------------------
// Recurrence + output.  One workgroup per (sequence, value head, NSUB slices of 16 value columns);
// per slice a chain wave (waves 0 .. NSUB-1) and an output wave (waves NSUB .. 2 NSUB-1).
// Per chunk c, two phases separated by one workgroup barrier:
//   phase 1  chain: hand S_c to the output wave; KS = K S_c; X = diag(beta)(V - diag(gamma) KS);
//                   V' = A X; hand V' to the output wave; V'' = diag(gamma_C / gamma) V'
//            output: P = scale Lower(Gamma) (.) Q K^T (registers)
//   phase 2  chain: S_{c+1} = gamma_C S_c + K^T V''   (K^T read transposed from the K tile)
//            output: O = scale diag(gamma) Q S_c + P V', stored
// Accumulator tiles feed the next product directly (pi order, gdn_device.h).  Q, K, A and the V
// slice of chunk c + 1 stream into the other LDS buffer with direct-to-LDS loads while chunk c
// computes.  Rows past the end of a chunk are loaded from the last valid row (always in bounds);
// they meet beta = 0 and g = 0, so X and V' vanish there, and their outputs are not stored.
// ------------------------------------------------------------------------------------------
// Per-token gate rows of one chunk, staged once by wave 0.
// Scalar gate: log2 gamma, beta, gamma_C/gamma, gamma, scale*gamma.  Per-channel gate: beta and
// the [D_k] chunk decay 2^G_C.
enum { GL = 0, BETA = 64, SC = 128, GAM = 192, SGAM = 256, DEC = 320, GROWS = 448 };

template <typename T, int DK, int NSUB, int NBUF, int GATE>
struct RecLds {
    static constexpr int ESZ = (int)sizeof(T);
    static constexpr int BV = 16 * NSUB;
    static constexpr int KGPR = DK * ESZ / 16;     // 16-byte granules per Q/K row
    static constexpr int AGPR = 64 * ESZ / 16;     // per A row
    static constexpr int VGPR = BV * ESZ / 16;     // per V-slice row
    static constexpr int KT = 64 * KGPR * 16, AT = 64 * AGPR * 16, VT = 64 * VGPR * 16;  // tile bytes
    static constexpr int NKB = DK / 32;
    static constexpr int NS = Split<T>::parts;
    static constexpr bool CH = GATE == GDN_GATE_CHANNEL_K;
    // one tile buffer (byte offsets): K, Q, A, V slice of one chunk.  With per-channel gates K is
    // K 2^G and Q is Q 2^G (hi part), followed by K 2^(G_C - G) (hi, lo), Q 2^G's lo part and P (hi, lo)
    static constexpr int K0 = 0, Q0 = KT, A0 = 2 * KT, V0 = 2 * KT + AT, KD0 = V0 + VT;
    static constexpr int QL0 = KD0 + (CH ? NS * KT : 0), P0 = QL0 + (CH && NS == 2 ? KT : 0);
    static constexpr int TILES = P0 + (CH ? NS * AT : 0);
    static constexpr int SXN = NSUB * NKB * NS * 64;   // state fragments handed to the output waves
    static constexpr int VXN = NSUB * 2 * NS * 64;     // V' fragments handed to the output waves
    static constexpr int PXN = CH ? 1 : 6 * NS * 64;   // P fragments shared by the output waves
    static constexpr int BYTES = NBUF * TILES + (SXN + VXN + PXN) * (int)sizeof(Frag<T>) + 2 * GROWS * 4;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// 8 consecutive elements (col multiple of 8) of a swizzled tile row.
template <int GPR>
__device__ __forceinline__ Frag<bf16> ld8_t(const unsigned char *tile, int row, int col) {
    Frag<bf16> f;
    f.v = *reinterpret_cast<const bf16x8 *>(tile + tile_off<GPR, 2>(row, col));
    return f;
}
template <int GPR>
__device__ __forceinline__ Frag<float> ld8_t_f(const unsigned char *tile, int row, int col) {
    const float4 a = *reinterpret_cast<const float4 *>(tile + tile_off<GPR, 4>(row, col));
    const float4 b = *reinterpret_cast<const float4 *>(tile + tile_off<GPR, 4>(row, col + 4));
    Frag<float> f;
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
}
template <typename T, int GPR>
__device__ __forceinline__ Frag<T> ld8_tile(const unsigned char *tile, int row, int col) {
    if constexpr (sizeof(T) == 2) return ld8_t<GPR>(tile, row, col);
    else return ld8_t_f<GPR>(tile, row, col);
}
// pi-order operand of a swizzled tile row: elements [32kb + 4grp, +4) and [32kb + 16 + 4grp, +4).
template <typename T, int GPR>
__device__ __forceinline__ Frag<T> ldpi_tile(const unsigned char *tile, int row, int kb) {
    const int grp = (threadIdx.x & 63) >> 4;
    const int c0 = 32 * kb + 4 * grp, c1 = c0 + 16;
    Frag<T> f;
    if constexpr (sizeof(T) == 2) {
        const bf16x4 a = *reinterpret_cast<const bf16x4 *>(tile + tile_off<GPR, 2>(row, c0));
        const bf16x4 b = *reinterpret_cast<const bf16x4 *>(tile + tile_off<GPR, 2>(row, c1));
        f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else {
        const float4 a = *reinterpret_cast<const float4 *>(tile + tile_off<GPR, 4>(row, c0));
        const float4 b = *reinterpret_cast<const float4 *>(tile + tile_off<GPR, 4>(row, c1));
        f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
        f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    }
    return f;
}
// pi-order column operand of the K tile (the K^T operand of the state update): row d, tokens
// 32kb + 4grp + r and 32kb + 16 + 4grp + r.
template <typename T, int GPR>
__device__ __forceinline__ Frag<T> ldpi_col_tile(const unsigned char *tile, int d0, int kb) {
    const int lane = threadIdx.x & 63, grp = lane >> 4, j = lane & 15;
    Frag<T> f;
    if constexpr (sizeof(T) == 2) {
        // transposed reads: lane j = 4e + q of the group points at K[t_e][d0 + 4q .. + 3]
        const int e = j >> 2, q = j & 3;
        const int t0 = 32 * kb + 4 * grp + e;
        const bf16x4 a = lds_read_tr16(tile + tile_off<GPR, 2>(t0, d0 + 4 * q));
        const bf16x4 b = lds_read_tr16(tile + tile_off<GPR, 2>(t0 + 16, d0 + 4 * q));
        f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = 32 * kb + (e < 4 ? 4 * grp + e : 16 + 4 * grp + e - 4);
            f.v[e] = *reinterpret_cast<const float *>(tile + tile_off<GPR, 4>(t, d0 + j));
        }
    }
    return f;
}

// MODE 0: main pass (chain + output waves) over one segment of a sequence, from h0 or from the
//         segment's fixed-up start state; the last segment writes the final state.
// MODE 1: context-parallel pre-process (chain waves only) over "virtual" columns: value columns
//         (V as given, S = 0 at the segment start) give S*, identity columns (V = 0, S = I) give
//         the segment's transition matrix M; both are written to the workspace.
template <typename T, int DK, int NSUB, int NBUF, int MODE, int GATE>
__global__ __launch_bounds__(MODE == 0 ? 128 * NSUB : 64 * NSUB) void chunk_kernel(ChunkParams p) {
    using L = RecLds<T, DK, NSUB, NBUF, GATE>;
    constexpr bool OUT = MODE == 0;
    constexpr bool CH = L::CH;
    constexpr int NW = OUT ? 2 * NSUB : NSUB;      // waves
    constexpr int BV = L::BV, NKB = L::NKB, ESZ = L::ESZ;
    constexpr int EPG = 16 / ESZ;                  // elements per granule
    constexpr int MD = DK / 16;                    // 16-row state tiles

    // Separate LDS objects for the two tile buffers and for the exchange: the chunk loop is
    // unrolled by two, so every LDS access names its buffer at compile time and the compiler can
    // see that the direct-to-LDS loads into one buffer never alias the reads of the other (it
    // would otherwise wait for the loads before every LDS access).
    __shared__ __attribute__((aligned(16))) unsigned char tiles0[L::TILES];
    __shared__ __attribute__((aligned(16))) unsigned char tiles1[NBUF == 2 ? L::TILES : 16];
    __shared__ __attribute__((aligned(16))) Frag<T> sSx[OUT ? L::SXN : 1];
    __shared__ __attribute__((aligned(16))) Frag<T> sVx[OUT ? L::VXN : 1];
    __shared__ __attribute__((aligned(16))) Frag<T> sPx[OUT ? L::PXN : 1];
    __shared__ float sG[2 * GROWS];

    // the wave index is uniform across a wave: readfirstlane makes the role branches scalar
    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool chain = wave < NSUB;
    const int sub = chain ? wave : wave - NSUB;

    // XCD-aware mapping: the slices of one (segment, head) share blockIdx % 8, i.e. one XCD and
    // its L2, so Q/K/A fetched by one workgroup are L2 hits for the others.
    const int bid = blockIdx.x, xcd = bid & 7, rr = bid >> 3;
    const int slice = rr % p.n_slices, unit = (rr / p.n_slices) * 8 + xcd;
    if (unit >= p.total_segs * p.H_v) return;
    const int gsi = unit / p.H_v, h = unit % p.H_v;
    const int gs = p.segs ? p.order[gsi] : gsi;
    const SegInfo sg = seg_info(p.segs, gs, p.T, p.seg_chunks);
    const int n = sg.n;
    const int hq = h / (p.H_v / p.H_qk);
    const SeqInfo si = seq_info(p.seq, n, p.T);
    const int DV = p.D_v;
    // pre-process: slices past the value columns are identity (M) columns
    const bool mcols = !OUT && slice * BV >= DV;
    if constexpr (!OUT) {
        if (sg.last) return;                        // the last segment's maps are never needed
        if (mcols && sg.j == 0 && !p.h0) return;    // M of the first segment multiplies h0 = 0
    }
    const int c0 = mcols ? slice * BV - DV : slice * BV;           // first column of this slice
    const int col = c0 + 16 * sub + l16;                           // this lane's column
    const int ccols = mcols ? DK : DV;                             // columns of the state matrix

    const T *qb = static_cast<const T *>(p.q) + (int64_t)hq * DK;
    const T *kb_ = static_cast<const T *>(p.k) + (int64_t)hq * DK;
    const T *vb = static_cast<const T *>(p.v) + (int64_t)h * DV + (mcols ? 0 : c0);
    const float *gb = static_cast<const float *>(p.g) + h;
    const T *bb = static_cast<const T *>(p.beta) + h;
    const T *Ab = static_cast<const T *>(p.A) + (int64_t)h * 4096;
    // per-channel gates: gated tiles [chunk][H_v][64][DK] and P [chunk][H_v][NS][64][64]
    const T *kgb = static_cast<const T *>(p.kg) + (int64_t)h * 64 * DK;
    const T *kdb = static_cast<const T *>(p.kd) + (int64_t)h * L::NS * 64 * DK;
    const T *qgb = static_cast<const T *>(p.qg) + (int64_t)h * L::NS * 64 * DK;
    const T *Pb = static_cast<const T *>(p.P) + (int64_t)h * L::NS * 4096;
    const float *decb = p.decay + (int64_t)h * DK;
    const int64_t qk_stride = (int64_t)p.H_qk * DK, v_stride = (int64_t)p.H_v * DV;
    const int qks = (int)qk_stride, vs = (int)v_stride, hv = p.H_v;
    const int nch = sg.nchunks;
    // chunk c of the segment is chunk sg.c0 + c of the sequence
    auto nvalid = [&](int c) { return min(kChunk, si.len - (sg.c0 + c) * kChunk); };

    // ---- direct-to-LDS loads of chunk c into a tile buffer; instruction i of a tile goes to wave i % NW
    auto issue_loads = [&](int c, unsigned char *tb) __attribute__((always_inline)) {
        const int64_t tok = si.tok0 + (int64_t)(sg.c0 + c) * kChunk;
        const int last = nvalid(c) - 1;
        const int64_t gci = si.chunk0 + sg.c0 + c;   // global chunk index
        const T *vc = vb + tok * v_stride;
        const T *Ac = Ab + gci * p.H_v * 4096;
        // K and Q rows: the inputs (row stride H_qk DK, clamped into the chunk), or the gated tiles
        // (row stride DK, tail rows already zero)
        const T *kc = CH ? kgb + gci * p.H_v * 64 * DK : kb_ + tok * qk_stride;
        const T *qc = CH ? qgb + gci * p.H_v * L::NS * 64 * DK : qb + tok * qk_stride;
        const T *kdc = kdb + gci * p.H_v * L::NS * 64 * DK;
        const int kst = CH ? DK : qks;
#pragma unroll
        for (int i = wave; i < L::KGPR; i += NW) {         // 64 * KGPR granules = KGPR instructions
            const int pos = 64 * i + lane, row = pos / L::KGPR, g = pos % L::KGPR;
            const int cv = g ^ tile_swz<L::KGPR>(row), rowc = CH ? row : min(row, last);
            load_granule_to_lds(kc + rowc * kst + cv * EPG, tb + L::K0 + 1024 * i);
            if constexpr (OUT) load_granule_to_lds(qc + rowc * kst + cv * EPG, tb + L::Q0 + 1024 * i);
            if constexpr (CH) {
                load_granule_to_lds(kdc + row * DK + cv * EPG, tb + L::KD0 + 1024 * i);
                if constexpr (L::NS == 2) {
                    load_granule_to_lds(kdc + 64 * DK + row * DK + cv * EPG, tb + L::KD0 + L::KT + 1024 * i);
                    if constexpr (OUT) load_granule_to_lds(qc + 64 * DK + row * DK + cv * EPG, tb + L::QL0 + 1024 * i);
                }
            }
        }
        if constexpr (CH && OUT) {
            const T *Pc = Pb + gci * p.H_v * L::NS * 4096;
#pragma unroll
            for (int i = wave; i < L::NS * L::AGPR; i += NW) {
                const int part = i / L::AGPR, ii = i % L::AGPR;
                const int pos = 64 * ii + lane, row = pos / L::AGPR, g = pos % L::AGPR;
                const int cv = g ^ tile_swz<L::AGPR>(row);
                load_granule_to_lds(Pc + part * 4096 + row * 64 + cv * EPG, tb + L::P0 + part * L::AT + 1024 * ii);
            }
        }
#pragma unroll
        for (int i = wave; i < L::AGPR; i += NW) {
            const int pos = 64 * i + lane, row = pos / L::AGPR, g = pos % L::AGPR;
            const int cv = g ^ tile_swz<L::AGPR>(row);
            load_granule_to_lds(Ac + row * 64 + cv * EPG, tb + L::A0 + 1024 * i);
        }
        if (!mcols) {
#pragma unroll
            for (int i = wave; i < L::VGPR; i += NW) {
                const int pos = 64 * i + lane, row = pos / L::VGPR, g = pos % L::VGPR;
                const int cv = g ^ tile_swz<L::VGPR>(row), rowc = min(row, last);
                load_granule_to_lds(vc + rowc * vs + cv * EPG, tb + L::V0 + 1024 * i);
            }
        }
    };
    float rg = 0.f;   // wave 0: gate and (raw) beta of token `lane` of the next chunk; converted
    T rb = T(0.f);    // only when used, so the loads are not waited for here
    float rdec[DK / 64];  // per-channel gates: the chunk decay of channels lane, lane + 64
    auto load_gates = [&](int c) __attribute__((always_inline)) {
        const int64_t tok = si.tok0 + (int64_t)(sg.c0 + c) * kChunk;
        const int tl = min(lane, nvalid(c) - 1);
        if constexpr (CH) {
            const float *dc = decb + (si.chunk0 + sg.c0 + c) * (int64_t)p.H_v * DK;
#pragma unroll
            for (int u = 0; u < DK / 64; ++u) rdec[u] = dc[lane + 64 * u];
        } else {
            rg = (gb + tok * hv)[tl * hv];
        }
        rb = (bb + tok * hv)[tl * hv];
    };

    // ---- chain state: S [DK][16] of this slice in fp32 accumulator tiles (rows 16m + 4grp + r)
    //      main pass: h0 (first segment) or the fixed-up start state; pre-process: 0 or identity
    f32x4 S[MD];
    const float *s_init = nullptr;
    if constexpr (OUT) {
        s_init = sg.j == 0 ? (p.h0 ? p.h0 + ((int64_t)n * p.H_v + h) * DK * DV : nullptr)
                           : p.seg_start + ((int64_t)gs * p.H_v + h) * DK * DV;
    }
#pragma unroll
    for (int m = 0; m < MD; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d = 16 * m + 4 * grp + r;
            S[m][r] = (chain && s_init) ? s_init[d * DV + col] : (mcols && d == col) ? 1.f : 0.f;
        }

    // ---- one chunk; B = tile buffer holding it (compile time)
    auto step = [&]<int B>(int c) __attribute__((always_inline)) {
        unsigned char *tcur = B == 0 ? tiles0 : tiles1;
        unsigned char *tnext = B == 0 ? tiles1 : tiles0;
        if constexpr (NBUF == 1) {
            if (c > 0) {
                __syncthreads();  // every wave is done with the single buffer
                issue_loads(c, tiles0);
            }
        }
        const int nv = nvalid(c);
        float *g3 = sG + B * GROWS;
        if (wave == 0) {
            g3[BETA + lane] = lane < nv ? to_f32(rb) : 0.f;
            if constexpr (CH) {
#pragma unroll
                for (int u = 0; u < DK / 64; ++u) g3[DEC + lane + 64 * u] = rdec[u];
            } else {
                const float gv = lane < nv ? rg : 0.f;                   // tail tokens carry g = 0
                const float gl = wave_inclusive_scan(gv) * kLog2e;       // log2 gamma_t
                const float glC = __shfl(gl, 63, 64);
                const float gam = fast_exp2(gl);
                g3[GL + lane] = gl;
                g3[SC + lane] = fast_exp2(glC - gl);                     // gamma_C / gamma_t
                g3[GAM + lane] = gam;
                g3[SGAM + lane] = p.scale * gam;
            }
        }
        // vmcnt(0) (gfx9 encoding: vmcnt bits [3:0],[15:14] = 0; expcnt [6:4] and lgkmcnt [11:8]
        // left at their maxima): this wave's direct-to-LDS loads of chunk c have landed
        __builtin_amdgcn_s_waitcnt(0x0f70);
        __syncthreads();  // tiles and gates of chunk c are visible
        if constexpr (NBUF == 2) {
            if (c + 1 < nch) issue_loads(c + 1, tnext);               // stream chunk c + 1 meanwhile
        }
        if (wave == 0) load_gates(min(c + 1, nch - 1));
        const unsigned char *tK = tcur + L::K0, *tQ = tcur + L::Q0, *tA = tcur + L::A0, *tV = tcur + L::V0;
        const unsigned char *tKd = CH ? tcur + L::KD0 : tK, *tP = tcur + L::P0, *tQl = tcur + L::QL0;
        // =========================== phase 1 ===========================
        Frag<T> Wh[2], Wl[2];          // chain: V'' (pi order over tokens)
        if (chain) {
            Frag<T> Sh[NKB], Sl[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                float x[8];
                pack_pi(S[2 * kb], S[2 * kb + 1], x);
                split8(x, Sh[kb], Sl[kb]);
                if constexpr (OUT) {
                    Frag<T> *dst = sSx + ((sub * NKB + kb) * L::NS) * 64 + lane;
                    dst[0] = Sh[kb];
                    if constexpr (L::NS == 2) dst[64] = Sl[kb];
                }
            }
            f32x4 ks[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                ks[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) mma_x(ks[m], ldpi_tile<T, L::KGPR>(tK, 16 * m + l16, kb), Sh[kb], Sl[kb]);
            }
            f32x4 xx[4];
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * m + 4 * grp + r;
                    const float v = mcols ? 0.f : to_f32(*reinterpret_cast<const T *>(tV + tile_off<L::VGPR, ESZ>(i, 16 * sub + l16)));
                    xx[m][r] = CH ? g3[BETA + i] * (v - ks[m][r]) : g3[BETA + i] * (v - g3[GAM + i] * ks[m][r]);
                }
            Frag<T> Xh[2], Xl[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float x[8];
                pack_pi(xx[2 * kb], xx[2 * kb + 1], x);
                split8(x, Xh[kb], Xl[kb]);
            }
            f32x4 vp[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                vp[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb <= m / 2; ++kb) mma_x(vp[m], ldpi_tile<T, L::AGPR>(tA, 16 * m + l16, kb), Xh[kb], Xl[kb]);
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float x[8];
                pack_pi(vp[2 * kb], vp[2 * kb + 1], x);
                Frag<T> vh, vl;
                split8(x, vh, vl);
                if constexpr (OUT) {
                    Frag<T> *dst = sVx + ((sub * 2 + kb) * L::NS) * 64 + lane;
                    dst[0] = vh;
                    if constexpr (L::NS == 2) dst[64] = vl;
                }
                if constexpr (!CH) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int t = 32 * kb + (e < 4 ? 4 * grp + e : 16 + 4 * grp + e - 4);
                        x[e] *= g3[SC + t];
                    }
                }
                split8(x, Wh[kb], Wl[kb]);
            }
        } else if constexpr (OUT && !CH) {
            // P^T tiles: acc[r] = (Q K^T)[i = 16 ti + l16][j = 16 tj + 4 grp + r], grouped into the six
            // pi-order fragments (ti, kb); the output waves share the work and the result through LDS.
#pragma unroll
            for (int f = 0; f < 6; ++f) {
                constexpr int FTI[6] = {0, 1, 2, 2, 3, 3}, FKB[6] = {0, 0, 0, 1, 0, 1};
                // balanced split of the ten tiles: owner of fragment f
                constexpr int OWN2[6] = {1, 0, 0, 0, 1, 1};
                const int owner = NSUB == 1 ? 0 : (NSUB == 2 ? OWN2[f] : f % NSUB);
                if (sub != owner) continue;
                const int ti = FTI[f], kb = FKB[f];
                const float gli = g3[GL + 16 * ti + l16];
                float x[8];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int tj = 2 * kb + half;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    if (tj <= ti) {
#pragma unroll
                        for (int kd = 0; kd < NKB; ++kd)
                            mma(acc, ld8_tile<T, L::KGPR>(tK, 16 * tj + l16, 32 * kd + 8 * grp),
                                ld8_tile<T, L::KGPR>(tQ, 16 * ti + l16, 32 * kd + 8 * grp));
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * tj + 4 * grp + r;
                        const float v = p.scale * fast_exp2(gli - g3[GL + j]) * acc[r];
                        x[4 * half + r] = tj < ti ? v : (tj == ti && 4 * grp + r <= l16) ? v : 0.f;
                    }
                }
                Frag<T> ph, pl;
                split8(x, ph, pl);
                sPx[(f * L::NS) * 64 + lane] = ph;
                if constexpr (L::NS == 2) sPx[(f * L::NS + 1) * 64 + lane] = pl;
            }
        }
        if constexpr (OUT) lds_only_barrier();  // S_c and V' of chunk c are visible to the output waves

        // =========================== phase 2 ===========================
        if (chain) {
            const float gC = g3[GAM + 63];
#pragma unroll
            for (int m = 0; m < MD; ++m) {
                if constexpr (CH) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) S[m][r] *= g3[DEC + 16 * m + 4 * grp + r];
                } else {
                    S[m] *= gC;
                }
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const Frag<T> kdh = ldpi_col_tile<T, L::KGPR>(tKd, 16 * m, kb);
                    if constexpr (CH && L::NS == 2)
                        mma_xx(S[m], kdh, ldpi_col_tile<T, L::KGPR>(tKd + L::KT, 16 * m, kb), Wh[kb], Wl[kb]);
                    else
                        mma_x(S[m], kdh, Wh[kb], Wl[kb]);
                }
            }
        } else if constexpr (OUT) {
            const Frag<T> *sxs = sSx + (sub * NKB * L::NS) * 64 + lane;
            const Frag<T> *vxs = sVx + (sub * 2 * L::NS) * 64 + lane;
            f32x4 o[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) o[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                Frag<T> sh = sxs[kb * L::NS * 64], sl;
                if constexpr (L::NS == 2) sl = sxs[kb * L::NS * 64 + 64];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const Frag<T> qh = ldpi_tile<T, L::KGPR>(tQ, 16 * m + l16, kb);
                    if constexpr (CH && L::NS == 2)
                        mma_xx(o[m], qh, ldpi_tile<T, L::KGPR>(tQl, 16 * m + l16, kb), sh, sl);
                    else
                        mma_x(o[m], qh, sh, sl);
                }
            }
            Frag<T> Vh[2], Vl[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                Vh[kb] = vxs[kb * L::NS * 64];
                if constexpr (L::NS == 2) Vl[kb] = vxs[kb * L::NS * 64 + 64];
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
#pragma unroll
                for (int r = 0; r < 4; ++r) o[m][r] *= CH ? p.scale : g3[SGAM + 16 * m + 4 * grp + r];
#pragma unroll
                for (int kb = 0; kb <= m / 2; ++kb) {
                    Frag<T> ph, pl;
                    if constexpr (CH) {
                        ph = ldpi_tile<T, L::AGPR>(tP, 16 * m + l16, kb);
                        if constexpr (L::NS == 2) pl = ldpi_tile<T, L::AGPR>(tP + L::AT, 16 * m + l16, kb);
                    } else {
                        const int f = m == 0 ? 0 : m == 1 ? 1 : m == 2 ? 2 + kb : 4 + kb;
                        ph = sPx[(f * L::NS) * 64 + lane];
                        if constexpr (L::NS == 2) pl = sPx[(f * L::NS + 1) * 64 + lane];
                    }
                    mma_xx(o[m], ph, pl, Vh[kb], Vl[kb]);
                }
            }
            // buffer stores: the resource covers the chunk's valid rows only (rows past the end are
            // dropped by the bounds check); row offsets are scalar, the lane offset is computed once
            const int64_t ebase = (int64_t)(si.tok0 + (sg.c0 + c) * kChunk) * v_stride + (int64_t)h * DV + c0;
            const int oes = p.o_f32 ? 4 : ESZ;
            const __amdgpu_buffer_rsrc_t ors = make_rsrc(static_cast<char *>(p.o) + ebase * oes,
                                                         ((nv - 1) * vs + BV) * oes);
            const int vlane = ((4 * grp) * vs + 16 * sub + l16) * oes;
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int soff = (16 * m + r) * vs * oes;
                    if (p.o_f32) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[m][r]), ors, vlane, soff, 0);
                    else if constexpr (ESZ == 2)
                        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (bf16)o[m][r]), ors, vlane, soff, 0);
                    else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[m][r]), ors, vlane, soff, 0);
                }
        }
    };

    if (nch > 0) {
        issue_loads(0, tiles0);
        if (wave == 0) load_gates(0);
    }
    for (int c = 0; c < nch; c += 2) {
        step.template operator()<0>(c);
        if (c + 1 < nch) step.template operator()<NBUF == 2 ? 1 : 0>(c + 1);
    }

    // ---- end of the segment: final state (main pass, last segment) or the segment's maps
    float *s_end = nullptr;
    if constexpr (OUT) {
        if (sg.last && p.final_state) s_end = p.final_state + ((int64_t)n * p.H_v + h) * DK * DV;
    } else {
        s_end = (mcols ? p.seg_m : p.seg_sstar) + ((int64_t)gs * p.H_v + h) * DK * ccols;
    }
    if (chain && s_end) {
#pragma unroll
        for (int m = 0; m < MD; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) s_end[(16 * m + 4 * grp + r) * ccols + col] = S[m][r];
    }
}

// ------------------------------------------------------------------------------------------
// Context-parallel fix-up (FlashQLA page, the S_{j,0} update of the CP pre-process): per
// (sequence, value head, 16 value columns), serially over the sequence's segments,
//   S_start(0) = h0 (or 0),   S_start(j + 1) = S*_j + M_j S_start(j),
// writing S_start(j) for j >= 1.  Four waves each produce DK/64 16-row tiles of the product; the
// new state goes through LDS to become the next step's operand.  M is prefetched one segment
// ahead into registers and staged in LDS (hi + lo bf16 pairs, or fp32).
// ------------------------------------------------------------------------------------------
template <typename T, int DK>
__global__ __launch_bounds__(256) void cp_fix_kernel(FixParams p) {
    constexpr int NS = Split<T>::parts, MP = DK + 16 / (int)sizeof(T);  // padded row of M
    constexpr int MT = DK / 64;                    // 16-row output tiles per wave
    constexpr int NV = DK * DK / 4 / 256;          // float4 of M per thread
    __shared__ __attribute__((aligned(16))) T sM[NS][DK * MP];
    __shared__ __attribute__((aligned(16))) float sS[DK * 17];  // S_start [DK][16], padded
    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nsl = p.D_v / 16;
    const int unit = blockIdx.x / nsl, slice = blockIdx.x - unit * nsl;
    if (unit >= p.N * p.H_v) return;
    const int n = unit / p.H_v, h = unit - n * p.H_v;
    const SeqInfo si = seq_info(p.seq, n, p.T);
    const int gs0 = p.seq ? si.seg0 : n * max(1, ceil_div(si.nchunks, p.seg_chunks));
    // segments of this sequence (bounded by the planned count, so every index below is in range)
    const int ns = min(max(1, ceil_div(si.nchunks, p.seg_chunks)), p.total_segs - gs0);
    if (ns < 2) return;
    const int c0 = slice * 16, DV = p.D_v;
    const int64_t hstride = (int64_t)DK * DV;

    // S_start(0): h0 or zero
    for (int i = tid; i < DK * 16; i += 256) {
        const int d = i >> 4, c = i & 15;
        sS[d * 17 + c] = p.h0 ? p.h0[((int64_t)n * p.H_v + h) * hstride + d * DV + c0 + c] : 0.f;
    }
    float4 mreg[NV];
    auto load_m = [&](int j) __attribute__((always_inline)) {
        const float4 *src = reinterpret_cast<const float4 *>(p.seg_m + ((int64_t)(gs0 + j) * p.H_v + h) * DK * DK);
#pragma unroll
        for (int i = 0; i < NV; ++i) mreg[i] = src[tid + 256 * i];
    };
    load_m(0);
    for (int j = 0; j + 1 < ns; ++j) {
        __syncthreads();  // the previous step is done with sM and sS
        // stage M_j
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = 4 * (tid + 256 * i), row = e / DK, cc = e - row * DK;
            const float x[4] = {mreg[i].x, mreg[i].y, mreg[i].z, mreg[i].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (NS == 2) {
                    const bf16 hi = (bf16)x[q];
                    sM[0][row * MP + cc + q] = hi;
                    sM[1][row * MP + cc + q] = (bf16)(x[q] - (float)hi);
                } else {
                    sM[0][row * MP + cc + q] = from_f32<T>(x[q]);
                }
            }
        }
        if (j + 2 < ns) load_m(j + 1);
        __syncthreads();
        // B operand: S_start(j) in pi order over d, as hi/lo fragments
        Frag<T> Bh[DK / 32], Bl[DK / 32];
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = 32 * kb + (e < 4 ? 4 * grp + e : 16 + 4 * grp + e - 4);
                x[e] = sS[d * 17 + l16];
            }
            split8(x, Bh[kb], Bl[kb]);
        }
        // this wave's output tiles: rows 16 (wave * MT + t) ..
        f32x4 acc[MT];
        const float *sst = p.seg_sstar + ((int64_t)(gs0 + j) * p.H_v + h) * hstride;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int m = wave * MT + t;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[t][r] = sst[(16 * m + 4 * grp + r) * DV + c0 + l16];
            if (j == 0 && !p.h0) continue;  // S_start(0) = 0 (M_0 was not computed)
#pragma unroll
            for (int kb = 0; kb < DK / 32; ++kb) {
                const Frag<T> ah = ld_pi(&sM[0][(16 * m + l16) * MP], kb);
                if constexpr (NS == 2) {
                    const Frag<T> al = ld_pi(&sM[1][(16 * m + l16) * MP], kb);
                    mma_xx(acc[t], ah, al, Bh[kb], Bl[kb]);
                } else {
                    mma(acc[t], ah, Bh[kb]);
                }
            }
        }
        __syncthreads();  // every wave has read S_start(j)
        float *dst = const_cast<float *>(p.seg_start) + ((int64_t)(gs0 + j + 1) * p.H_v + h) * hstride;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int m = wave * MT + t;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = 16 * m + 4 * grp + r;
                sS[d * 17 + l16] = acc[t][r];
                dst[d * DV + c0 + l16] = acc[t][r];
            }
        }
    }
}

}  // namespace

hipError_t launch_plan(const PlanParams &p, hipStream_t s) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int MODE, int GATE>
static hipError_t launch_rec(int dtype, int D_k, int BV, const ChunkParams &p, hipStream_t s) {
    const int units = p.total_segs * p.H_v;
    const unsigned groups = (unsigned)((units + 7) / 8);
    const dim3 grid(groups * 8u * (unsigned)p.n_slices);
    if (units == 0) return hipSuccess;
#define GDN_CHUNK_CASE(DT, T_, DK_, NSUB_, NBUF_)                                                         \
    if (dtype == DT && D_k == DK_ && BV == 16 * NSUB_) {                                                  \
        hipLaunchKernelGGL((chunk_kernel<T_, DK_, NSUB_, NBUF_, MODE, GATE>), grid, dim3((MODE == 0 ? 128 : 64) * NSUB_), \
                           0, s, p);                                                                      \
        return hipGetLastError();                                                                         \
    }
    if constexpr (GATE == GDN_GATE_CHANNEL_K) {
        // the gated and decayed K tiles and P take LDS: one tile buffer for D_k = 128
        GDN_CHUNK_CASE(1, bf16, 128, 2, 1)
        GDN_CHUNK_CASE(1, bf16, 64, 2, 2)
        GDN_CHUNK_CASE(0, float, 128, 1, 1)
        GDN_CHUNK_CASE(0, float, 64, 1, 1)
    } else {
        GDN_CHUNK_CASE(1, bf16, 128, 2, 2)
        GDN_CHUNK_CASE(1, bf16, 128, 1, 2)
        GDN_CHUNK_CASE(1, bf16, 64, 2, 2)
        GDN_CHUNK_CASE(1, bf16, 64, 1, 2)
        GDN_CHUNK_CASE(0, float, 128, 1, 1)
        GDN_CHUNK_CASE(0, float, 64, 2, 2)
        GDN_CHUNK_CASE(0, float, 64, 1, 2)
    }
#undef GDN_CHUNK_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_chunk(int dtype, int D_k, int BV, int gate, const ChunkParams &p, hipStream_t s) {
    return gate == GDN_GATE_CHANNEL_K ? launch_rec<0, GDN_GATE_CHANNEL_K>(dtype, D_k, BV, p, s)
                                      : launch_rec<0, 0>(dtype, D_k, BV, p, s);
}
hipError_t launch_cp_pre(int dtype, int D_k, int BV, int gate, const ChunkParams &p, hipStream_t s) {
    return gate == GDN_GATE_CHANNEL_K ? launch_rec<1, GDN_GATE_CHANNEL_K>(dtype, D_k, BV, p, s)
                                      : launch_rec<1, 0>(dtype, D_k, BV, p, s);
}
hipError_t launch_cp_fix(int dtype, int D_k, const FixParams &p, hipStream_t s) {
    const dim3 grid((unsigned)(p.N * p.H_v * (p.D_v / 16))), block(256);
    if (p.N * p.H_v == 0) return hipSuccess;
    if (dtype == 1 && D_k == 128) hipLaunchKernelGGL((cp_fix_kernel<bf16, 128>), grid, block, 0, s, p);
    else if (dtype == 1 && D_k == 64) hipLaunchKernelGGL((cp_fix_kernel<bf16, 64>), grid, block, 0, s, p);
    else if (dtype == 0 && D_k == 128) hipLaunchKernelGGL((cp_fix_kernel<float, 128>), grid, block, 0, s, p);
    else if (dtype == 0 && D_k == 64) hipLaunchKernelGGL((cp_fix_kernel<float, 64>), grid, block, 0, s, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gdn
