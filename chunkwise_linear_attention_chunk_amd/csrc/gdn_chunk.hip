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
    constexpr int kSortMax = 1024;   // segments ranked longest first (identity order beyond)
    constexpr int kSeqMax = 4096;    // sequences whose chunk tables all threads fill together
    __shared__ int sC[256], sS[256];
    __shared__ int sLen[kSortMax];
    __shared__ int sChunk0[kSeqMax + 1], sTok0[kSeqMax], sSeqLen[kSeqMax];
    const int tid = threadIdx.x;
    const bool sort = p.total_segs <= kSortMax;
    const bool shared_fill = p.N <= kSeqMax;
    // every chunk entry starts empty (nv = 0: the intra kernel then reads nothing), every segment
    // entry empty and not last (it then writes no final state)
    for (int i = tid; i < p.total_chunks; i += 256) p.chunks[i] = ChunkInfo{0, 0};
    for (int i = tid; i < p.total_segs; i += 256) {
        p.segs[i] = SegInfo{0, 0, 0, 0, 0};
        if (sort) sLen[i] = 0;
    }
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
            const SeqInfo si{tok0, min(len, ncc * kChunk), chunk0, ncc, seg0};
            p.seq[n] = si;
            if (shared_fill) {
                sChunk0[n] = chunk0;
                sTok0[n] = si.tok0;
                sSeqLen[n] = si.len;
                if (n == p.N - 1) sChunk0[p.N] = chunk0 + ncc;
            } else {
                for (int c = 0; c < si.nchunks; ++c) {
                    const int rem = si.len - c * kChunk;
                    p.chunks[si.chunk0 + c] = ChunkInfo{si.tok0 + c * kChunk, rem < kChunk ? rem : kChunk};
                }
            }
            const int nseg = max(1, ceil_div(si.nchunks, p.seg_chunks));
            for (int j = 0; j < nseg && si.seg0 + j < p.total_segs; ++j) {
                const int c0 = j * p.seg_chunks, segn = max(0, min(p.seg_chunks, si.nchunks - c0));
                p.segs[si.seg0 + j] = SegInfo{n, j, c0, segn, j == nseg - 1 ? 1 : 0};
                if (sort) sLen[si.seg0 + j] = segn;
            }
        }
        carry_c += sC[255];
        carry_s += sS[255];
        __syncthreads();
    }
    // chunk table, all threads: chunk i belongs to the last sequence whose first chunk is <= i
    // (empty sequences share their first chunk index with the next one and are skipped)
    if (shared_fill) {
        const int nchunks = sChunk0[p.N];
        for (int i = tid; i < nchunks; i += 256) {
            int lo = 0, hi = p.N - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (sChunk0[mid] <= i) lo = mid; else hi = mid - 1;
            }
            const int c = i - sChunk0[lo];
            const int rem = sSeqLen[lo] - c * kChunk;
            p.chunks[i] = ChunkInfo{sTok0[lo] + c * kChunk, rem < kChunk ? rem : kChunk};
        }
    }
    // rank sort of the segments (longest first, ties by index) on the lengths held in LDS
    for (int g = tid; g < p.total_segs; g += 256) {
        int rank = g;
        if (sort) {
            const int len = sLen[g];
            rank = 0;
            for (int m = 0; m < p.total_segs; ++m) {
                const int lm = sLen[m];
                rank += (lm > len) || (lm == len && m < g);
            }
        }
        p.order[rank] = g;
    }
}

// tile selections of the recurrence kernel's loads
// (LD_KD: with per-channel gates, the decayed K tile K 2^(G_C - G) of the state update)
enum { LD_A = 1, LD_P = 2, LD_V = 4, LD_G = 8, LD_K = 16, LD_Q = 32, LD_KD = 64, LD_ALL = 127 };

// ------------------------------------------------------------------------------------------
// Recurrence + output.  One workgroup per (sequence segment, value head, NSUB slices of 16 value
// columns); per slice a chain wave (waves 0 .. NSUB-1) and an output wave (waves NSUB .. 2 NSUB-1).
// Per chunk c, two phases separated by one workgroup barrier:
//   phase 1  chain: KS = K S_c; X = diag(beta)(V - diag(gamma) KS); V' = A X; hand V' to the
//                   output wave; V'' = diag(gamma_C / gamma) V'
//            output: O = scale diag(gamma) Q S_c
//   phase 2  chain: S_{c+1} = gamma_C S_c + K^T V''   (K^T read transposed from the K tile), then
//                   hand S_{c+1} to the output waves for the next chunk
//            output: O += P V' (P = scale Lower(Gamma) (.) Q K^T from the per-chunk kernel), stored
// The tiles of chunk c + 1 (K, Q, A, P, the V slice and the gate block of per-token gate rows, also
// from the per-chunk kernel) stream into the other LDS buffer with direct-to-LDS loads meanwhile,
// issued by the output waves between their Q S products, so the chain waves only compute (loads
// issued by the chain waves measured slower: they delay its first products).  Accumulator tiles
// feed the next product directly (pi order, gdn_device.h).  Rows past the end of a chunk read as
// zero (buffer bounds) and carry beta = 0, g = 0, so X and V' vanish there; their outputs are not
// stored.
// ------------------------------------------------------------------------------------------

template <typename T, int DK, int NSUB, int NBUF, int MODE, int GATE>
struct RecLds {
    static constexpr int ESZ = (int)sizeof(T);
    static constexpr int BV = 16 * NSUB;
    static constexpr int KGPR = DK * ESZ / 16;     // 16-byte granules per Q/K row
    static constexpr int AGPR = 64 * ESZ / 16;     // per A (and P) row
    static constexpr int VGPR = BV * ESZ / 16;     // per V-slice row
    static constexpr int KT = 64 * KGPR * 16, AT = 64 * AGPR * 16, VT = 64 * VGPR * 16;  // tile bytes
    static constexpr int NKB = DK / 32;
    static constexpr int NS = Split<T>::parts;
    static constexpr bool CH = GATE == GDN_GATE_CHANNEL_K, OUT = MODE == 0;
    static constexpr bool PL = OUT && CH;          // P loaded with the tiles (else formed in LDS)
    // one tile buffer (byte offsets): K, Q, A, V slice (and P, NS parts, with per-channel gates) of
    // one chunk.  With per-channel gates K is K 2^G and Q is Q 2^G (hi part), followed by
    // K 2^(G_C - G) (NS parts) and the lo part of Q 2^G.  The pre-process (no output) holds no Q.
    static constexpr int K0 = 0, Q0 = KT, A0 = Q0 + (OUT ? KT : 0), V0 = A0 + AT, P0 = V0 + VT;
    static constexpr int KD0 = P0 + (PL ? NS * AT : 0), QL0 = KD0 + (CH ? NS * KT : 0);
    static constexpr int G0 = QL0 + (CH && OUT && NS == 2 ? KT : 0);   // the chunk's gate block
    static constexpr int TILES = G0 + GB_FLOATS * 4;
    static constexpr int SXN = NSUB * NKB * NS * 64;   // state fragments handed to the output waves
    static constexpr int VXN = NSUB * 2 * NS * 64;     // V' fragments handed to the output waves
    static constexpr int BYTES = NBUF * TILES + (OUT ? (SXN + VXN) * (int)sizeof(Frag<T>) : 0);
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// V[16m + 4grp + r][col], r = 0..3, from the swizzled V-slice tile (col = this lane's column).
template <typename T, int GPR>
__device__ __forceinline__ void ld_vcol4(const unsigned char *tile, int m, int col0, float *v) {
    const int lane = threadIdx.x & 63, grp = lane >> 4, j = lane & 15;
    if constexpr (sizeof(T) == 2) {
        // transposed read: lane j = 4e + q points at V[16m + 4grp + e][col0 + 4q .. + 3]
        const bf16x4 a = lds_read_tr16(tile + tile_off<GPR, 2>(16 * m + 4 * grp + (j >> 2), col0 + 4 * (j & 3)));
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (float)a[r];
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            v[r] = *reinterpret_cast<const float *>(tile + tile_off<GPR, 4>(16 * m + 4 * grp + r, col0 + j));
    }
}

// MODE 0: main pass (chain + output waves) over one segment of a sequence, from h0 or from the
//         segment's fixed-up start state; the last segment writes the final state.
// MODE 1: context-parallel pre-process (chain waves only) over "virtual" columns: value columns
//         (V as given, S = 0 at the segment start) give S*, identity columns (V = 0, S = I) give
//         the segment's transition matrix M; both are written to the workspace.
// ST (main pass only): also store the state entering every chunk (the backward's recomputed
//         states); a separate build, so the forward carries none of it.
template <typename T, int DK, int NSUB, int NBUF, int MODE, int GATE, bool ST = false>
__global__ __launch_bounds__(MODE == 0 ? 128 * NSUB : 64 * NSUB,
                             NBUF == 1 && MODE == 0 && GATE == 0 && sizeof(T) == 2 ? 2 : 1)
void chunk_kernel(ChunkParams p) {
    using L = RecLds<T, DK, NSUB, NBUF, MODE, GATE>;
    constexpr bool OUT = L::OUT, CH = L::CH;
    constexpr int BV = L::BV, NKB = L::NKB, ESZ = L::ESZ;
    constexpr int EPG = 16 / ESZ;                  // elements per granule
    constexpr int MD = DK / 16;                    // 16-row state tiles
    constexpr int NL = NSUB;                       // waves sharing each group of tile loads
    // main pass with two tile buffers: the chain waves stream the next chunk's K and A tiles, the
    // output waves the rest
    constexpr bool CHAIN_LD = MODE == 0 && NBUF == 2;
    constexpr int OUT_LD = CHAIN_LD ? LD_ALL & ~(LD_K | LD_KD | LD_A) : LD_ALL;
    // main pass with one tile buffer and per-channel gates: the tiles that only phase 1 reads
    // (everything but the gate block and the decayed K tile) are refilled with the next chunk's
    // right after the mid-chunk barrier, so their loads overlap phase 2; the rest at the chunk top.
    // (With a scalar gate the one-buffer build runs two workgroups per CU, which already cover
    // each other's loads; refilling early measured slower there.)
    constexpr bool EARLY_LD = MODE == 0 && NBUF == 1 && CH;
    constexpr int LATE_LD = CH ? (LD_KD | LD_G) : LD_G;
    // L2 prefetch (per-channel main pass with two tile buffers, whose chunk step is otherwise bound
    // by the latency of its tile loads): the chain waves of a head's column slices together touch
    // every 128-byte line of chunk c + PF_DIST's tiles right after issuing chunk c + 1's loads, so
    // the tile loads of that chunk hit L2.  Each chain wave issues exactly NPF such loads per chunk
    // (and NPF in the prologue): its chunk-top wait then leaves the NPF newest loads in flight,
    // which, loads returning in order, still covers every tile load issued before them.  The lines
    // land in a sink that nothing reads.  In the state-storing replay the chain waves' state stores
    // come before their loads of a chunk; the wait still covers every tile load (stores only add to
    // the count it waits through).
    constexpr bool PF = CH && MODE == 0 && NBUF == 2;
    constexpr int NPF = 2;
#ifndef GDN_PF_DIST
#define GDN_PF_DIST 2
#endif
    constexpr int PF_DIST = GDN_PF_DIST;
    // the same build stores each chunk's output one step late, after the next step's tile loads are
    // issued, so the output waves' chunk-top wait does not wait for those stores to land (with a
    // scalar gate this measured slower: 133 -> 136 us on the Qwen3-Next shape, 523 -> 572 us varlen)
    constexpr bool DEFER_O = PF && !ST;
    // the scalar-gate main pass with two tile buffers: the output waves store each chunk's output
    // in the next chunk, right after its mid-chunk barrier, where they would otherwise wait for the
    // chain's state update (phase 2 is the chain's).  Stored at the end of its own chunk, the output
    // made the output waves' chunk-top wait (a vmcnt wait, which counts stores too) wait for the
    // stores to land: 133.8 us on the Qwen3-Next shape; handed through LDS to the chain waves, which
    // stored it before their mid-chunk barrier, 128.0 us; stored this way, 124.2 us (the same as
    // the hand-over with the chain waves' stores removed).
    constexpr bool MIDOUT = MODE == 0 && NBUF == 2 && !ST && !CH;
    // the state-storing build with a scalar gate and bf16 inputs also forms the backward scan's scale P
    constexpr bool PSTORE = ST && !CH && sizeof(T) == 2;
    constexpr int NRT = 4 / NSUB;                  // token tiles of each output wave

    // Separate LDS objects for the two tile buffers and for the exchange: the chunk loop is
    // unrolled by two, so every LDS access names its buffer at compile time and the compiler can
    // see that the direct-to-LDS loads into one buffer never alias the reads of the other (it
    // would otherwise wait for the loads before every LDS access).
    __shared__ __attribute__((aligned(16))) unsigned char tiles0[L::TILES];
    __shared__ __attribute__((aligned(16))) unsigned char tiles1[NBUF == 2 ? L::TILES : 16];
    __shared__ __attribute__((aligned(16))) Frag<T> sSx[OUT ? L::SXN : 1];
    __shared__ __attribute__((aligned(16))) Frag<T> sVx[OUT ? L::VXN : 1];
    __shared__ __attribute__((aligned(16))) unsigned char pf_sink[PF ? 1024 : 16];

    // the wave index is uniform across a wave: readfirstlane makes the role branches scalar
    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool chain = wave < NSUB;
    const int sub = chain ? wave : wave - NSUB;

    // XCD-aware mapping: the slices of one (segment, head) share blockIdx % 8, i.e. one XCD and
    // its L2, so Q/K/A fetched by one workgroup are L2 hits for the others.
    const int bid = blockIdx.x, xcd = bid & 7, rr = bid >> 3;
    const int slice = rr % p.n_slices, unit = (rr / p.n_slices) * 8 + xcd;
    if (unit >= (p.seg_only ? p.N : p.total_segs) * p.H_v) return;
    const int gsi = unit / p.H_v, h = unit % p.H_v;
    // one piece of a batched input: segment seg_only - 1 of sequence gsi
    const int gs = p.seg_only ? gsi * max(1, ceil_div(ceil_div(p.T, kChunk), p.seg_chunks)) + p.seg_only - 1
                              : p.segs ? p.order[gsi] : gsi;
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
    const T *Ab = static_cast<const T *>(p.A) + (int64_t)h * 4096;
    const T *Pb = static_cast<const T *>(p.P) + (int64_t)h * L::NS * 4096;
    // per-channel gates: gated tiles [chunk][H_v][parts][64][DK]
    const T *kgb = static_cast<const T *>(p.kg) + (int64_t)h * 64 * DK;
    const T *kdb = static_cast<const T *>(p.kd) + (int64_t)h * L::NS * 64 * DK;
    const T *qgb = static_cast<const T *>(p.qg) + (int64_t)h * L::NS * 64 * DK;
    const float *Gb = p.gates + (int64_t)h * GB_FLOATS;
    const int64_t qk_stride = (int64_t)p.H_qk * DK, v_stride = (int64_t)p.H_v * DV;
    const int qks = (int)qk_stride, vs = (int)v_stride;
    // warmup CP: the segment starts wup chunks early (from S = 0, or from h0 at the sequence start),
    // and those chunks write no output
    const int wup = OUT && p.warm ? p.warm[(int64_t)gs * p.H_v + h] : 0;
    const int cs = sg.c0 - wup;                  // chunk c of this workgroup is chunk cs + c of the sequence
    const int nch = sg.nchunks + wup;
    auto nvalid = [&](int c) { return min(kChunk, si.len - (cs + c) * kChunk); };

    // ---- direct-to-LDS loads of chunk c into a tile buffer.  Instruction i of a tile goes to
    //      loader wave i % NL; each lane's byte offset within the tile source is fixed, only the
    //      buffer base moves with the chunk.  The buffer range ends after the chunk's last valid
    //      row, so rows past the end read as zero.
    constexpr int NKI = (L::KGPR + NL - 1) / NL, NAI = (L::AGPR + NL - 1) / NL, NVI = (L::VGPR + NL - 1) / NL;
    const int kst = CH ? DK : qks;   // K and Q row stride (elements): inputs, or the gated tiles
    int offK[NKI], offA[NAI], offV[NVI];
#pragma unroll
    for (int j = 0; j < NKI; ++j) {
        const int pos = 64 * (sub + NL * j) + lane, row = pos / L::KGPR, g = pos % L::KGPR;
        offK[j] = (row * kst + (g ^ tile_swz<L::KGPR>(row)) * EPG) * ESZ;
    }
#pragma unroll
    for (int j = 0; j < NAI; ++j) {
        const int pos = 64 * (sub + NL * j) + lane, row = pos / L::AGPR, g = pos % L::AGPR;
        offA[j] = (row * 64 + (g ^ tile_swz<L::AGPR>(row)) * EPG) * ESZ;
    }
#pragma unroll
    for (int j = 0; j < NVI; ++j) {
        const int pos = 64 * (sub + NL * j) + lane, row = pos / L::VGPR, g = pos % L::VGPR;
        offV[j] = (row * vs + (g ^ tile_swz<L::VGPR>(row)) * EPG) * ESZ;
    }
    // Part q of np issues the instructions j with j % np == q of each tile (a caller can spread its
    // loads over other work; issuing them together measured fastest here).
    // K and Q as selected by `what` (LD_K | LD_Q; with per-channel gates K brings K 2^(G_C - G) and
    // Q brings Q 2^G's lo part):
    auto issue_kq = [&](int c, unsigned char *tb, int part_q, int np, int what) __attribute__((always_inline)) {
        const int64_t tok = si.tok0 + (int64_t)(cs + c) * kChunk;
        const int nvc = nvalid(c);
        const int64_t gci = si.chunk0 + cs + c;      // global chunk index
        const T *kc = CH ? kgb + gci * p.H_v * 64 * DK : kb_ + tok * qk_stride;
        const T *qc = CH ? qgb + gci * p.H_v * L::NS * 64 * DK : qb + tok * qk_stride;
        const int kbytes = CH ? 64 * DK * ESZ : ((nvc - 1) * qks + DK) * ESZ;
        const auto rK = make_rsrc(kc, kbytes);
        const auto rQ = make_rsrc(qc, CH ? L::NS * 64 * DK * ESZ : kbytes);
        const auto rKd = make_rsrc(kdb + gci * p.H_v * L::NS * 64 * DK, L::NS * 64 * DK * ESZ);
#pragma unroll
        for (int j = 0; j < NKI; ++j) {
            const int i = sub + NL * j;
            if (j % np != part_q) continue;
            if (NKI * NL != L::KGPR && i >= L::KGPR) break;
            if (what & LD_K) buffer_granule_to_lds(rK, tb + L::K0 + 1024 * i, offK[j], 0);
            if constexpr (CH) {
                if (what & LD_KD) {
#pragma unroll
                    for (int part = 0; part < L::NS; ++part)
                        buffer_granule_to_lds(rKd, tb + L::KD0 + part * L::KT + 1024 * i, offK[j], part * 64 * DK * ESZ);
                }
            }
            if constexpr (OUT) {
                if (what & LD_Q) {
                    buffer_granule_to_lds(rQ, tb + L::Q0 + 1024 * i, offK[j], 0);
                    if constexpr (CH && L::NS == 2) buffer_granule_to_lds(rQ, tb + L::QL0 + 1024 * i, offK[j], 64 * DK * ESZ);
                }
            }
        }
    };
    // A, P, the V slice and the gate block, as selected by `what` (LD_A | LD_P | LD_V | LD_G):
    auto issue_apvg = [&](int c, unsigned char *tb, int part_q, int np, int what) __attribute__((always_inline)) {
        const int64_t tok = si.tok0 + (int64_t)(cs + c) * kChunk;
        const int nvc = nvalid(c);
        const int64_t gci = si.chunk0 + cs + c;      // global chunk index
        const auto rA = make_rsrc(Ab + gci * p.H_v * 4096, 4096 * ESZ);
        const auto rP = make_rsrc(Pb + gci * p.H_v * L::NS * 4096, L::NS * 4096 * ESZ);
#pragma unroll
        for (int j = 0; j < NAI; ++j) {
            const int i = sub + NL * j;
            if (j % np != part_q) continue;
            if (NAI * NL != L::AGPR && i >= L::AGPR) break;
            if (what & LD_A) buffer_granule_to_lds(rA, tb + L::A0 + 1024 * i, offA[j], 0);
            if constexpr (L::PL) {
                if (what & LD_P) {
#pragma unroll
                    for (int part = 0; part < L::NS; ++part)
                        buffer_granule_to_lds(rP, tb + L::P0 + part * L::AT + 1024 * i, offA[j], part * 4096 * ESZ);
                }
            }
        }
        if (!mcols && (what & LD_V)) {
            const auto rV = make_rsrc(vb + tok * v_stride, ((nvc - 1) * vs + BV) * ESZ);
#pragma unroll
            for (int j = 0; j < NVI; ++j) {
                const int i = sub + NL * j;
                if (j % np != part_q) continue;
                if (NVI * NL != L::VGPR && i >= L::VGPR) break;
                buffer_granule_to_lds(rV, tb + L::V0 + 1024 * i, offV[j], 0);
            }
        }
        if ((what & LD_G) && sub == 0 && part_q == 0) {   // the gate block: 64 granules per instruction
            const auto rG = make_rsrc(Gb + gci * p.H_v * GB_FLOATS, GB_FLOATS * 4);
#pragma unroll
            for (int gi = 0; gi < GB_FLOATS / 256; ++gi) buffer_granule_to_lds(rG, tb + L::G0 + 1024 * gi, lane * 16, 1024 * gi);
        }
    };

    // The prefetch units of a chunk: 8 KiB pieces of its Kg, Kd, Qg, P, A tiles and gate block
    // (one 128-byte line per lane), then this slice's V rows (one row per lane).  Unit u goes to
    // prefetch slot u of the head's n_slices * NSUB chain waves * NPF slots.
    auto issue_pf = [&](int c2) __attribute__((always_inline)) {
        constexpr int UB = 8192;
        constexpr int UK = (L::KT + UB - 1) / UB, UKN = (L::NS * L::KT + UB - 1) / UB;
        constexpr int UP = (L::NS * L::AT + UB - 1) / UB, UA = (L::AT + UB - 1) / UB;
        const bool ok = c2 < nch;
        const int64_t gci = si.chunk0 + cs + c2;
        const int pid = slice * NSUB + sub, npf = p.n_slices * NSUB;
#pragma unroll
        for (int q = 0; q < NPF; ++q) {
            const int u = pid + npf * q;
            const void *base;
            int bytes, soff, voff = lane * 128;
            if (u < UK) {
                base = kgb + gci * p.H_v * 64 * DK; bytes = L::KT; soff = u * UB;
            } else if (u < UK + UKN) {
                base = kdb + gci * p.H_v * L::NS * 64 * DK; bytes = L::NS * L::KT; soff = (u - UK) * UB;
            } else if (u < UK + 2 * UKN) {
                base = qgb + gci * p.H_v * L::NS * 64 * DK; bytes = L::NS * L::KT; soff = (u - UK - UKN) * UB;
            } else if (u < UK + 2 * UKN + UP) {
                base = Pb + gci * p.H_v * L::NS * 4096; bytes = L::NS * L::AT; soff = (u - UK - 2 * UKN) * UB;
            } else if (u < UK + 2 * UKN + UP + UA) {
                base = Ab + gci * p.H_v * 4096; bytes = L::AT; soff = (u - UK - 2 * UKN - UP) * UB;
            } else if (u == UK + 2 * UKN + UP + UA) {
                base = Gb + gci * p.H_v * GB_FLOATS; bytes = GB_FLOATS * 4; soff = 0;
            } else {
                const int64_t tok = si.tok0 + (int64_t)(cs + c2) * kChunk;
                base = vb + tok * v_stride; soff = 0; voff = lane * vs * ESZ;
                bytes = ok ? ((nvalid(c2) - 1) * vs + BV) * ESZ : 0;
            }
            buffer_granule_to_lds(make_rsrc(base, ok ? bytes : 0), pf_sink, voff, soff);
        }
    };

    // ---- chain state: S [DK][16] of this slice in fp32 accumulator tiles (rows 16m + 4grp + r)
    //      main pass: h0 (first segment) or the fixed-up start state; pre-process: 0 or identity.
    //      Set up by the chain waves only (below).
    f32x4 S[MD];

    // ---- the entering state of the next chunk as matrix-core operand pairs (pi order over rows),
    //      handed to the output waves through LDS.  Formed at the end of each chunk, in the time the
    //      chain waves would otherwise wait for the output waves.
    Frag<T> Sh[NKB], Sl[NKB];
    auto split_state = [&]() __attribute__((always_inline)) {
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
    };

    // ---- the start of chunk c: with one tile buffer, every wave is done with it before the loader
    //      waves refill it; the loaders wait for their direct-to-LDS loads of chunk c (vmcnt(0), gfx9
    //      encoding: vmcnt bits [3:0],[15:14] = 0, expcnt [6:4] and lgkmcnt [11:8] at their maxima),
    //      and the barrier makes the tiles, the gate block and S_c visible to every wave.  Both roles
    //      below pass the same barriers in the same order.  (Waiting for the loads only, with the
    //      output stores issued after them left in flight, measured no faster.)
    auto chunk_top = [&]<bool LD, int VM = 0>(int c) __attribute__((always_inline)) {
        if constexpr (NBUF == 1) {
            if (c > 0) {
                __syncthreads();
                if constexpr (LD) {
                    constexpr int what = EARLY_LD ? LATE_LD : LD_ALL;
                    issue_kq(c, tiles0, 0, 1, what);
                    issue_apvg(c, tiles0, 0, 1, what);
                }
            }
        }
        static_assert(VM >= 0 && VM < 16, "vmcnt immediate");
        if constexpr (LD) __builtin_amdgcn_s_waitcnt(0x0f70 | VM);
        // (a workgroup barrier with its fence would wait for every memory operation in flight,
        // vmcnt(0), the prefetches included; each wave's tile loads are covered by its own wait
        // above, and no wave reads global memory another wave writes here)
        lds_only_barrier();
    };

    // ---- output role (main pass): streams the tiles of the next chunk into LDS and forms
    //      O = scale diag(gamma) Q S_c + P V' for its token tiles and all BV columns of the slice:
    //      with two output waves, wave 0 owns tiles 0 and 3 and wave 1 tiles 1 and 2 (which balances
    //      the causal P work); a single output wave owns all four.  Its own loop, so that none of
    //      the chain's registers (the state, its operand pairs) are live here and vice versa.
    //      It accumulates O^T = scale (S_c^T Q^T diag(gamma) + V'^T P^T): the operand fragments are
    //      the same with their roles swapped, and a lane then holds four consecutive value columns
    //      of one token, which it stores straight from registers (one 8-byte bf16 or 16-byte fp32
    //      store per 16 x 16 tile).
    // the output tile i of output wave s: token tile; wave 0 owns tiles 0 and 3, wave 1 tiles 1 and
    // 2 (which balances the causal P work); a single output wave owns all four
    auto out_tile = [](int s, int i) { return NSUB == 1 ? i : (i == 0 ? (s ? 1 : 0) : (s ? 2 : 3)); };
    // chunk c's output from the output wave s's registers: lane (grp, l16) of tile (i, g) holds
    // O[16 out_tile(s, i) + l16][16 g + 4 grp + r], r = 0..3.  The resource covers the chunk's valid
    // rows only (rows past the end are dropped by the bounds check).
    auto store_tiles = [&](int c, int s, auto &&tile) __attribute__((always_inline)) {
        const int nv = nvalid(c);
        const int64_t ebase = (int64_t)(si.tok0 + (cs + c) * kChunk) * v_stride + (int64_t)h * DV + c0;
        const int oes = p.o_f32 ? 4 : ESZ;
        const __amdgpu_buffer_rsrc_t ors = make_rsrc(static_cast<char *>(p.o) + ebase * oes,
                                                     p.o ? ((nv - 1) * vs + BV) * oes : 0);
#pragma unroll
        for (int i = 0; i < NRT; ++i)
#pragma unroll
            for (int g = 0; g < NSUB; ++g) {
                const int off = (16 * out_tile(s, i) + l16) * vs + 16 * g + 4 * grp;   // elements
                const f32x4 x = tile(i, g);
                if (ESZ == 2 && !p.o_f32) {
                    const bf16x4 b = {(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, b), ors, off * 2, 0, 0);
                } else {
                    const u32x4 w = {__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                                     __float_as_uint(x[3])};
                    __builtin_amdgcn_raw_buffer_store_b128(w, ors, off * 4, 0, 0);
                }
            }
    };
    if constexpr (OUT) {
        if (!chain) {
            constexpr int NR = NRT;                       // token tiles of this wave
            int mt[NR];
#pragma unroll
            for (int i = 0; i < NR; ++i) mt[i] = out_tile(sub, i);
            // the causal blocks of P V': (token tile i, contraction block kb <= m / 2)
            constexpr int NPB = NSUB == 1 ? 6 : 3;
            auto pb_tile = [&](int b) { return NSUB == 1 ? (b < 4 ? b : b - 2) : (b == 0 ? 0 : 1); };
            auto pb_kb = [&](int b) { return NSUB == 1 ? (b < 4 ? 0 : 1) : (b == 2 ? 1 : 0); };
            // (NSUB == 2: blocks (tile 0, kb 0), (tile 1, kb 0), (tile 1, kb 1); tile 1 is m = 3 or 2)
            // the output of a chunk straight from the accumulators (copied to o_prev, register renames,
            // where it is stored one step late)
            f32x4 o_prev[NR][NSUB];
            auto store_o = [&](int c) __attribute__((always_inline)) {
                if (c < wup) return;                       // warmup chunk: no output
                store_tiles(c, sub, [&](int i, int g) { return o_prev[i][g]; });
            };
            auto out_step = [&]<int B>(int c) __attribute__((always_inline)) {
                unsigned char *tcur = B == 0 ? tiles0 : tiles1;
                unsigned char *tnext = B == 0 ? tiles1 : tiles0;
                chunk_top.template operator()<true>(c);
                const float *g3 = reinterpret_cast<const float *>(tcur + L::G0);
                const bool more = NBUF == 2 && c + 1 < nch;               // stream chunk c + 1 meanwhile
                const unsigned char *tQ = tcur + L::Q0, *tK = tcur + L::K0, *tQl = tcur + L::QL0;
                // inter-chunk part: scale diag(gamma) Q S_c (S_c was handed over before this chunk);
                // the state and Q fragments first (the Q lo parts of per-channel gates as they are used)
                if (more) {                                       // the output waves' share, at once
                    issue_kq(c + 1, tnext, 0, 1, ST && !PSTORE ? OUT_LD & ~LD_Q : OUT_LD);
                    issue_apvg(c + 1, tnext, 0, 1, OUT_LD);
                }
                if constexpr (DEFER_O) {
                    if (c > 0) store_o(c - 1);
                }
                if constexpr (ST) {   // states only: the loads and the chain's barriers, no output
                    if constexpr (PSTORE) {
                        // scale P of the chunk for the backward's scan, once per head (the first
                        // column slice): the blocks of P V' below, stored as a bf16 pair per row
                        if (slice == 0 && p.pmat) {
                            Frag<T> qf[NKB][NR];
#pragma unroll
                            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                                for (int i = 0; i < NR; ++i) qf[kb][i] = ldpi_tile<T, L::KGPR>(tQ, 16 * mt[i] + l16, kb);
                            bf16 *Pb = static_cast<bf16 *>(p.pmat) + ((int64_t)(si.chunk0 + cs + c) * p.H_v + h) * 2 * 4096;
                            const float lsc = __log2f(p.scale);
#pragma unroll
                            for (int b = 0; b < NPB; ++b) {
                                const int i = pb_tile(b), kb = pb_kb(b), m = mt[i], t = 16 * m + l16;
                                const float glt = g3[GB_GLQ + t] + lsc;
#pragma unroll
                                for (int u = 0; u < 2; ++u) {
                                    const int nn = 2 * kb + u, s0 = 16 * nn + 4 * grp;   // key tile, first key
                                    f32x4 pt = {0.f, 0.f, 0.f, 0.f};                      // P[t][s0 .. s0 + 3]
                                    if (nn <= m) {
#pragma unroll
                                        for (int kk = 0; kk < NKB; ++kk)
                                            mma(pt, ldpi_tile<T, L::KGPR>(tK, 16 * nn + l16, kk), qf[kk][i]);
                                        const float4 gs = *reinterpret_cast<const float4 *>(g3 + GB_GLK + s0);
                                        const float gsv[4] = {gs.x, gs.y, gs.z, gs.w};
#pragma unroll
                                        for (int r = 0; r < 4; ++r) pt[r] = s0 + r <= t ? fast_exp2(glt - gsv[r]) * pt[r] : 0.f;
                                    }
                                    bf16x4 hi, lo;
#pragma unroll
                                    for (int r = 0; r < 4; ++r) {
                                        hi[r] = (bf16)pt[r];
                                        lo[r] = (bf16)(pt[r] - (float)hi[r]);
                                    }
                                    *reinterpret_cast<bf16x4 *>(Pb + t * 64 + s0) = hi;
                                    *reinterpret_cast<bf16x4 *>(Pb + 4096 + t * 64 + s0) = lo;
                                }
                            }
                        }
                    }
                    lds_only_barrier();
                    if constexpr (EARLY_LD) {
                        if (c + 1 < nch) {
                            issue_kq(c + 1, tiles0, 0, 1, LD_ALL & ~LATE_LD & ~LD_Q);
                            issue_apvg(c + 1, tiles0, 0, 1, LD_ALL & ~LATE_LD);
                        }
                    }
                    return;
                }
                Frag<T> sh[NSUB][NKB], sl[NSUB][NKB], qf[NKB][NR];
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                    for (int g = 0; g < NSUB; ++g) {
                        const Frag<T> *sxs = sSx + ((g * NKB + kb) * L::NS) * 64 + lane;
                        sh[g][kb] = sxs[0];
                        if constexpr (L::NS == 2) sl[g][kb] = sxs[64];
                    }
#pragma unroll
                    for (int i = 0; i < NR; ++i) qf[kb][i] = ldpi_tile<T, L::KGPR>(tQ, 16 * mt[i] + l16, kb);
                }
                f32x4 o[NR][NSUB];
#pragma unroll
                for (int i = 0; i < NR; ++i)
#pragma unroll
                    for (int g = 0; g < NSUB; ++g) o[i][g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                    for (int i = 0; i < NR; ++i) {
                        Frag<T> ql;
                        if constexpr (CH && L::NS == 2) ql = ldpi_tile<T, L::KGPR>(tQl, 16 * mt[i] + l16, kb);
#pragma unroll
                        for (int g = 0; g < NSUB; ++g) {
                            if constexpr (CH && L::NS == 2) mma_xx(o[i][g], sh[g][kb], sl[g][kb], qf[kb][i], ql);
                            else mma_pair_x(o[i][g], sh[g][kb], sl[g][kb], qf[kb][i]);
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < NR; ++i) {
                    // this lane's token is 16 mt[i] + l16
                    const float f = CH ? p.scale : p.scale * g3[GB_GAQ + 16 * mt[i] + l16];
#pragma unroll
                    for (int g = 0; g < NSUB; ++g) o[i][g] *= f;
                }
                // P operand pairs of the causal blocks.  Per-channel gates: read from the tile the
                // per-chunk kernel formed.  Scalar gate: P = scale Lower(Gamma) (.) Q K^T formed here
                // (06 . Flash Linear Attention, section 3) from the Q fragments above and the K tile,
                // transposed (C = K Q^T: a lane holds four consecutive key tokens s of one query token
                // t), which is lane for lane the pi-order row operand of P V' once the two 16-token
                // halves of a block are packed.
                Frag<T> ph[NPB], pl[NPB];
                if constexpr (CH) {
                    const unsigned char *tP = tcur + L::P0;
#pragma unroll
                    for (int b = 0; b < NPB; ++b) {
                        const int row = 16 * mt[pb_tile(b)] + l16;
                        ph[b] = ldpi_tile<T, L::AGPR>(tP, row, pb_kb(b));
                        if constexpr (L::NS == 2) pl[b] = ldpi_tile<T, L::AGPR>(tP + L::AT, row, pb_kb(b));
                    }
                }
                // scalar gate: block b of P (query rows' log-gates from GLQ, key rows' from GLK)
                const float *glq = g3 + GB_GLQ, *glk = g3 + GB_GLK;
                const float lsc = __log2f(p.scale);
                auto form_p = [&](int b) __attribute__((always_inline)) {
                    const int i = pb_tile(b), kb = pb_kb(b), m = mt[i];
                    const int t = 16 * m + l16;
                    const float glt = glq[t] + lsc;
                    f32x4 pt[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int nn = 2 * kb + u;             // key tile
                        pt[u] = f32x4{0.f, 0.f, 0.f, 0.f};
                        if (nn > m) continue;                  // above the diagonal: zero
#pragma unroll
                        for (int kk = 0; kk < NKB; ++kk) mma(pt[u], ldpi_tile<T, L::KGPR>(tK, 16 * nn + l16, kk), qf[kk][i]);
                        const int s0 = 16 * nn + 4 * grp;
                        const float4 gs = *reinterpret_cast<const float4 *>(glk + s0);
                        const float gsv[4] = {gs.x, gs.y, gs.z, gs.w};
#pragma unroll
                        for (int r = 0; r < 4; ++r) pt[u][r] = (s0 + r <= t) ? fast_exp2(glt - gsv[r]) * pt[u][r] : 0.f;
                    }
                    float x[8];
                    pack_pi(pt[0], pt[1], x);
                    split8(x, ph[b], pl[b]);
                };
                if constexpr (!CH) {
#pragma unroll
                    for (int b = 0; b < NPB; ++b) form_p(b);
                }
                lds_only_barrier();  // V' of chunk c is visible; every wave is done with phase 1
                if constexpr (MIDOUT) {
                    if (c > 0) store_o(c - 1);
                }
                if constexpr (EARLY_LD) {
                    if (c + 1 < nch) {
                        issue_kq(c + 1, tiles0, 0, 1, LD_ALL & ~LATE_LD);
                        issue_apvg(c + 1, tiles0, 0, 1, LD_ALL & ~LATE_LD);
                    }
                }
                // intra-chunk part: P V'
#pragma unroll
                for (int g = 0; g < NSUB; ++g) {
                    const Frag<T> *vxs = sVx + (g * 2 * L::NS) * 64 + lane;
                    Frag<T> Vh[2], Vl[2];
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        Vh[kb] = vxs[kb * L::NS * 64];
                        if constexpr (L::NS == 2) Vl[kb] = vxs[kb * L::NS * 64 + 64];
                    }
#pragma unroll
                    for (int b = 0; b < NPB; ++b) mma_xx(o[pb_tile(b)][g], Vh[pb_kb(b)], Vl[pb_kb(b)], ph[b], pl[b]);
                }
#pragma unroll
                for (int i = 0; i < NR; ++i)
#pragma unroll
                    for (int g = 0; g < NSUB; ++g) o_prev[i][g] = o[i][g];
                if constexpr (!DEFER_O && !MIDOUT) store_o(c);
            };
            if (nch > 0) {
                issue_kq(0, tiles0, 0, 1, LD_ALL);
                issue_apvg(0, tiles0, 0, 1, LD_ALL);
            }
            for (int c = 0; c < nch; c += 2) {
                out_step.template operator()<0>(c);
                if (c + 1 < nch) out_step.template operator()<NBUF == 2 ? 1 : 0>(c + 1);
            }
            if constexpr (DEFER_O || MIDOUT) {
                if (nch > 0) store_o(nch - 1);
            }
            return;
        }
    }

    // ---- chain role: the state recurrence (in the pre-process the chain waves also load the tiles)
    {
        const float *s_init = nullptr;
        if constexpr (OUT) {
            if (cs == 0) s_init = p.h0 ? p.h0 + ((int64_t)n * p.H_v + h) * DK * DV : nullptr;  // sequence start
            else if (!p.warm) s_init = p.seg_start + ((int64_t)gs * p.H_v + h) * DK * DV;       // fixed-up start
            // (warmup CP from a later chunk: S = 0)
        }
#pragma unroll
        for (int m = 0; m < MD; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = 16 * m + 4 * grp + r;
                S[m][r] = s_init ? s_init[d * DV + col] : (mcols && d == col) ? 1.f : 0.f;
            }
    }
    auto chain_step = [&]<int B>(int c) __attribute__((always_inline)) {
        unsigned char *tcur = B == 0 ? tiles0 : tiles1;
        unsigned char *tnext = B == 0 ? tiles1 : tiles0;
        chunk_top.template operator()<!OUT || CHAIN_LD, PF ? NPF : 0>(c);
        if constexpr (OUT && ST) {
            {   // the state entering this chunk (no CP: segment = sequence); non-temporal: another
                // kernel reads it, well after this one has moved on
                float *st = p.chunk_states + ((int64_t)(si.chunk0 + cs + c) * p.H_v + h) * DK * DV;
#pragma unroll
                for (int m = 0; m < MD; ++m)
#pragma unroll
                    for (int r = 0; r < 4; ++r) __builtin_nontemporal_store(S[m][r], &st[(16 * m + 4 * grp + r) * DV + col]);
            }
        }
        const float *g3 = reinterpret_cast<const float *>(tcur + L::G0);
        const bool more = NBUF == 2 && c + 1 < nch;
        if constexpr (!OUT) {
            if (more) {
                issue_kq(c + 1, tnext, 0, 1, LD_ALL);
                issue_apvg(c + 1, tnext, 0, 1, LD_ALL);
            }
        }
        const unsigned char *tK = tcur + L::K0, *tA = tcur + L::A0, *tV = tcur + L::V0;
        const unsigned char *tKd = CH ? tcur + L::KD0 : tK;
        // =========================== phase 1 ===========================
        Frag<T> Wh[2], Wl[2];          // V'' (pi order over tokens)
        Frag<T> kt[2][MD];             // the K^T fragments of the state update, read early

        // this lane's V values and gate rows first, so their LDS latency hides behind K S
        float v[4][4], b4[4][4], ga[4][4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
            for (int r = 0; r < 4; ++r) { v[m][r] = 0.f; ga[m][r] = 1.f; }
            if (!mcols) ld_vcol4<T, L::VGPR>(tV, m, 16 * sub, v[m]);
            const float4 be = *reinterpret_cast<const float4 *>(g3 + GB_BETA + 16 * m + 4 * grp);
            b4[m][0] = be.x; b4[m][1] = be.y; b4[m][2] = be.z; b4[m][3] = be.w;
            if constexpr (!CH) {
                const float4 gg = *reinterpret_cast<const float4 *>(g3 + GB_GAK + 16 * m + 4 * grp);
                ga[m][0] = gg.x; ga[m][1] = gg.y; ga[m][2] = gg.z; ga[m][3] = gg.w;
            }
        }
        // every K and A fragment of the chunk's products is read up front, so the reads overlap
        // each other and the first products instead of each waiting in turn
        Frag<T> kf[NKB][4], af[6];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int m = 0; m < 4; ++m) kf[kb][m] = ldpi_tile<T, L::KGPR>(tK, 16 * m + l16, kb);
#pragma unroll
        for (int f = 0; f < 6; ++f) {
            const int m = f < 4 ? f : f - 2, kb = f < 4 ? 0 : 1;   // (m, kb): (0..3, 0), (2, 1), (3, 1)
            af[f] = ldpi_tile<T, L::AGPR>(tA, 16 * m + l16, kb);
        }
        // K S: contraction block outer, the four row tiles inner (independent accumulators)
        f32x4 ks[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) ks[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int m = 0; m < 4; ++m) mma_x(ks[m], kf[kb][m], Sh[kb], Sl[kb]);
        f32x4 xx[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) xx[m][r] = b4[m][r] * (v[m][r] - ga[m][r] * ks[m][r]);
        Frag<T> Xh[2], Xl[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            float x[8];
            pack_pi(xx[2 * kb], xx[2 * kb + 1], x);
            split8(x, Xh[kb], Xl[kb]);
        }
        // V' = A X (A lower triangular: row tile m needs contraction blocks kb <= m / 2)
        f32x4 vp[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) vp[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < 6; ++f) {
            const int m = f < 4 ? f : f - 2, kb = f < 4 ? 0 : 1;
            mma_x(vp[m], af[f], Xh[kb], Xl[kb]);
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
                const float4 s0 = *reinterpret_cast<const float4 *>(g3 + GB_SC + 32 * kb + 4 * grp);
                const float4 s1 = *reinterpret_cast<const float4 *>(g3 + GB_SC + 32 * kb + 16 + 4 * grp);
                x[0] *= s0.x; x[1] *= s0.y; x[2] *= s0.z; x[3] *= s0.w;
                x[4] *= s1.x; x[5] *= s1.y; x[6] *= s1.z; x[7] *= s1.w;
            }
            split8(x, Wh[kb], Wl[kb]);
        }
        // the state update's K^T fragments, read while the output waves finish phase 1
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int m = 0; m < MD; ++m) kt[kb][m] = ldpi_col_tile<T, L::KGPR>(tKd, 16 * m, kb);
        if constexpr (CHAIN_LD) {
            // the K and A tiles of chunk c + 1 (the chain waves reach this barrier first)
            if (more) {
                issue_kq(c + 1, tnext, 0, 1, LD_K | LD_KD);
                issue_apvg(c + 1, tnext, 0, 1, LD_A);
            }
            if constexpr (PF) issue_pf(c + PF_DIST);
        }
        if constexpr (OUT) lds_only_barrier();  // V' of chunk c is visible to the output waves
        // =========================== phase 2 ===========================

        float4 dec[MD];
#pragma unroll
        for (int m = 0; m < MD; ++m) {
            if constexpr (CH) dec[m] = *reinterpret_cast<const float4 *>(g3 + GB_DEC + 16 * m + 4 * grp);
            else dec[m] = make_float4(g3[GB_GC], g3[GB_GC], g3[GB_GC], g3[GB_GC]);
        }
#pragma unroll
        for (int m = 0; m < MD; ++m) {
            S[m][0] *= dec[m].x; S[m][1] *= dec[m].y; S[m][2] *= dec[m].z; S[m][3] *= dec[m].w;
        }
        // S += K^T V'': contraction block outer, the row tiles inner
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int m0 = 0; m0 < MD; m0 += 4) {
                Frag<T> kl[4];
                if constexpr (CH && L::NS == 2) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) kl[u] = ldpi_col_tile<T, L::KGPR>(tKd + L::KT, 16 * (m0 + u), kb);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if constexpr (CH && L::NS == 2) mma_xx(S[m0 + u], kt[kb][m0 + u], kl[u], Wh[kb], Wl[kb]);
                    else mma_x(S[m0 + u], kt[kb][m0 + u], Wh[kb], Wl[kb]);
                }
            }
        split_state();  // S_{c+1} for the next chunk (the output waves read S_c before the barrier)
    };
    if (nch > 0) {
        if constexpr (!OUT) {
            issue_kq(0, tiles0, 0, 1, LD_ALL);
            issue_apvg(0, tiles0, 0, 1, LD_ALL);
        }
        if constexpr (PF) {
#pragma unroll
            for (int c2 = 1; c2 < PF_DIST; ++c2) issue_pf(c2);
        }
        split_state();
    }
    for (int c = 0; c < nch; c += 2) {
        chain_step.template operator()<0>(c);
        if (c + 1 < nch) chain_step.template operator()<NBUF == 2 ? 1 : 0>(c + 1);
    }
    if constexpr (PF) __builtin_amdgcn_s_waitcnt(0x0f70);   // no prefetch into the sink outlives the workgroup

    // ---- end of the segment: final state (main pass, last segment) or the segment's maps
    float *s_end = nullptr;
    if constexpr (OUT) {
        if (sg.last && p.final_state) s_end = p.final_state + ((int64_t)n * p.H_v + h) * DK * DV;
        else if (!sg.last && p.seg_next) s_end = p.seg_next + ((int64_t)(gs + 1) * p.H_v + h) * DK * DV;
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
// writing S_start(j) for j >= 1.  One wave per 16-row tile of the product.  Each wave's rows of
// M_j and its S*_j values come straight from memory into registers, two segments ahead (three
// register sets), and M_j is split into operand pairs off the serial path; only the new state
// goes through LDS (two buffers, one barrier per segment).  The column slices of one (sequence,
// head) share an XCD, so M and S* are L2 hits after the first slice reads them.
// ------------------------------------------------------------------------------------------
template <typename T, int DK>
__global__ __launch_bounds__(DK * 4) void cp_fix_kernel(FixParams p) {
    constexpr int NKB = DK / 32;                   // contraction blocks
    constexpr int SP = 17;                         // padded row of the LDS state [DK][16]
    __shared__ __attribute__((aligned(16))) float sS[2][DK * SP];
    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
    const int m = __builtin_amdgcn_readfirstlane(tid >> 6);   // this wave's row tile
    const int nsl = p.D_v / 16;
    const int bid = blockIdx.x, xcd = bid & 7, rr = bid >> 3;
    const int slice = rr % nsl, unit = (rr / nsl) * 8 + xcd;
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
    for (int i = tid; i < DK * 16; i += DK * 4) {
        const int d = i >> 4, c = i & 15;
        sS[0][d * SP + c] = p.h0 ? p.h0[((int64_t)n * p.H_v + h) * hstride + d * DV + c0 + c] : 0.f;
    }
    // raw (fp32) M row 16 m + l16 at the pi-order columns of each block, and the S* values of this
    // lane's accumulator positions, for one segment
    struct Raw {
        float4 m[NKB][2];
        float sst[4];
    };
    auto load_raw = [&](int j, Raw &rw) __attribute__((always_inline)) {
        const float *row = p.seg_m + ((int64_t)(gs0 + j) * p.H_v + h) * DK * DK + (16 * m + l16) * DK;
        const float *Sj = p.seg_sstar + ((int64_t)(gs0 + j) * p.H_v + h) * hstride;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            rw.m[kb][0] = *reinterpret_cast<const float4 *>(row + 32 * kb + 4 * grp);
            rw.m[kb][1] = *reinterpret_cast<const float4 *>(row + 32 * kb + 16 + 4 * grp);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) rw.sst[r] = Sj[(16 * m + 4 * grp + r) * DV + c0 + l16];
    };
    Raw raw[3];
    load_raw(0, raw[0]);
    if (ns > 2) load_raw(1, raw[1]);

    // one segment step; B2 = state buffer (j % 2), B3 = raw register set (j % 3), both compile time
    auto step = [&]<int B2, int B3>(int j) __attribute__((always_inline)) {
        // segment j + 2's M and S* (needed only while j + 2 < ns - 1)
        if (j + 3 < ns) load_raw(j + 2, raw[(B3 + 2) % 3]);
        // M_j as operand pairs (off the serial path: independent of the state)
        Frag<T> mh[NKB], ml[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const float4 a = raw[B3].m[kb][0], b = raw[B3].m[kb][1];
            const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            split8(x, mh[kb], ml[kb]);
        }
        lds_only_barrier();  // S_start(j) is complete in sS[B2] (the loads of later segments stay in flight)
        const float *cur = sS[B2];
        // S_start(j) in pi order over d, as operand pairs
        Frag<T> bh[NKB], bl[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = 32 * kb + (e < 4 ? 4 * grp + e : 16 + 4 * grp + e - 4);
                x[e] = cur[d * SP + l16];
            }
            split8(x, bh[kb], bl[kb]);
        }
        f32x4 acc = {raw[B3].sst[0], raw[B3].sst[1], raw[B3].sst[2], raw[B3].sst[3]};
        if (!(j == 0 && !p.h0)) {   // S_start(0) = 0: M_0 was not computed
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) mma_xx(acc, mh[kb], ml[kb], bh[kb], bl[kb]);
        }
        float *nxt = sS[B2 ^ 1];
        float *dst = p.seg_start + ((int64_t)(gs0 + j + 1) * p.H_v + h) * hstride;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d = 16 * m + 4 * grp + r;
            nxt[d * SP + l16] = acc[r];
            dst[d * DV + c0 + l16] = acc[r];
        }
    };
    // steps j = 0 .. ns - 2, unrolled by six so both parities are compile-time constants
    for (int j = 0; j + 1 < ns; j += 6) {
        step.template operator()<0, 0>(j);
        if (j + 2 < ns) step.template operator()<1, 1>(j + 1);
        if (j + 3 < ns) step.template operator()<0, 2>(j + 2);
        if (j + 4 < ns) step.template operator()<1, 0>(j + 3);
        if (j + 5 < ns) step.template operator()<0, 1>(j + 4);
        if (j + 6 < ns) step.template operator()<1, 2>(j + 5);
    }
}

// ------------------------------------------------------------------------------------------
// Warmup CP gate statistics (FlashQLA announcement, section "further optimisation through gate
// decay": a separate kernel collects the gate statistics that fix each rank's warmup length).
// One wave per (segment, value head): W = the fewest chunks right before the segment whose decay
// bounds (gate block GC: the chunk decay, or for per-channel gates the product of each token's
// largest channel decay) multiply to <= tol, summed in log2 units; the whole prefix (W = c0,
// which starts from h0 and is exact) when none do.  The wave walks back 64 chunks per step, one
// chunk per lane, with a running sum across steps.
__global__ __launch_bounds__(256) void warm_stats_kernel(WarmParams p) {
    const int lane = threadIdx.x & 63;
    const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (unit >= p.total_segs * p.H_v) return;
    const int gs = unit / p.H_v, h = unit - gs * p.H_v;
    const SegInfo sg = seg_info(p.segs, gs, p.T, p.seg_chunks);
    const SeqInfo si = seq_info(p.seq, sg.n, p.T);
    int W = 0;
    if (sg.j > 0) {
        W = sg.c0;
        float carry = 0.f;
        for (int base = 0; base < sg.c0; base += 64) {
            const int w = base + lane + 1;           // the warmup length whose oldest chunk this lane adds
            const bool in = w <= sg.c0;
            const float lg = in ? __log2f(p.gates[((int64_t)(si.chunk0 + sg.c0 - w) * p.H_v + h) * GB_FLOATS + GB_GC])
                                : 0.f;               // log2 0 = -inf: a decay that underflowed ends the warmup
            const float cum = carry + wave_inclusive_scan(lg);
            const unsigned long long hit = __ballot(in && cum <= p.log2_tol);
            if (hit) {
                W = base + __ffsll(hit);             // lowest lane that reaches the bound, plus one
                break;
            }
            carry = __shfl(cum, 63, 64);
        }
    }
    if (lane == 0) p.warm[unit] = W;
}

}  // namespace

hipError_t launch_plan(const PlanParams &p, hipStream_t s) {
    launch_k(plan_kernel, dim3(1), dim3(256), s, p);
    return hipGetLastError();
}

template <int MODE, int GATE, bool ST = false>
static hipError_t launch_rec(int dtype, int D_k, int BV, const ChunkParams &p, hipStream_t s) {
    const int units = (p.seg_only ? p.N : p.total_segs) * p.H_v;
    const unsigned groups = (unsigned)((units + 7) / 8);
    const dim3 grid(groups * 8u * (unsigned)p.n_slices);
    if (units == 0) return hipSuccess;
#define GDN_CHUNK_CASE(DT, T_, DK_, NSUB_, NBUF_)                                                         \
    if (dtype == DT && D_k == DK_ && BV == 16 * NSUB_) {                                                  \
        launch_k((chunk_kernel<T_, DK_, NSUB_, NBUF_, MODE, GATE, ST>), grid, dim3((MODE == 0 ? 128 : 64) * NSUB_), s, p);                                                                      \
        return hipGetLastError();                                                                         \
    }
    if constexpr (GATE == GDN_GATE_CHANNEL_K) {
        // bf16 inputs: the per-chunk kernel's gated tiles, P and A are fp16 operands (one part each),
        // so two tile buffers fit
        GDN_CHUNK_CASE(1, f16, 128, 2, 2)
        GDN_CHUNK_CASE(1, f16, 64, 2, 2)
        GDN_CHUNK_CASE(0, float, 128, 1, 1)
        GDN_CHUNK_CASE(0, float, 64, 1, 1)
    } else {
        if constexpr (MODE == 0) {
            // enough workgroups for two per CU (large batches, many packed sequences): the one-buffer
            // build, whose 75 KiB of LDS and 256 registers per wave let two workgroups share a CU and
            // fill each other's waits (its own loads then do not overlap its work)
            if (grid.x >= 2u * (unsigned)p.n_cus) { GDN_CHUNK_CASE(1, bf16, 128, 2, 1) }
        }
        GDN_CHUNK_CASE(1, bf16, 128, 2, 2)
        GDN_CHUNK_CASE(1, bf16, 128, 1, 2)
        GDN_CHUNK_CASE(1, bf16, 64, 2, 2)
        GDN_CHUNK_CASE(1, bf16, 64, 1, 2)
        GDN_CHUNK_CASE(0, float, 128, 1, 1)
        GDN_CHUNK_CASE(0, float, 64, 2, 1)
        GDN_CHUNK_CASE(0, float, 64, 1, 2)
    }
#undef GDN_CHUNK_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_chunk(int dtype, int D_k, int BV, int gate, const ChunkParams &p, hipStream_t s) {
    if (p.chunk_states)
        return gate == GDN_GATE_CHANNEL_K ? launch_rec<0, GDN_GATE_CHANNEL_K, true>(dtype, D_k, BV, p, s)
                                          : launch_rec<0, 0, true>(dtype, D_k, BV, p, s);
    return gate == GDN_GATE_CHANNEL_K ? launch_rec<0, GDN_GATE_CHANNEL_K>(dtype, D_k, BV, p, s)
                                      : launch_rec<0, 0>(dtype, D_k, BV, p, s);
}
hipError_t launch_cp_pre(int dtype, int D_k, int BV, int gate, const ChunkParams &p, hipStream_t s) {
    return gate == GDN_GATE_CHANNEL_K ? launch_rec<1, GDN_GATE_CHANNEL_K>(dtype, D_k, BV, p, s)
                                      : launch_rec<1, 0>(dtype, D_k, BV, p, s);
}
hipError_t launch_warm_stats(const WarmParams &p, hipStream_t s) {
    const int64_t units = (int64_t)p.total_segs * p.H_v;
    if (units == 0) return hipSuccess;
    launch_k(warm_stats_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), s, p);
    return hipGetLastError();
}
hipError_t launch_cp_fix(int dtype, int D_k, const FixParams &p, hipStream_t s) {
    // XCD-aware: blockIdx = ((unit / 8) * slices + slice) * 8 + unit % 8
    const unsigned groups = (unsigned)((p.N * p.H_v + 7) / 8);
    const dim3 grid(groups * 8u * (unsigned)(p.D_v / 16)), block((unsigned)(D_k * 4));
    if (p.N * p.H_v == 0) return hipSuccess;
    if (dtype == 1 && D_k == 128) launch_k(cp_fix_kernel<bf16, 128>, grid, block, s, p);
    else if (dtype == 1 && D_k == 64) launch_k(cp_fix_kernel<bf16, 64>, grid, block, s, p);
    else if (dtype == 0 && D_k == 128) launch_k(cp_fix_kernel<float, 128>, grid, block, s, p);
    else if (dtype == 0 && D_k == 64) launch_k(cp_fix_kernel<float, 64>, grid, block, s, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gdn
