// Context-parallel pre-process in the X/Y/Z form (FlashQLA page, "a balanced solution: in-GPU CP
// alongside the fused kernels", step 2.1, and its CP pre-process kernel table), scalar gate, bf16
// inputs.
//
// A segment that starts from an unknown state H maps it chunk by chunk through S -> T_c S + b_c, so
// it ends in M H + S*: S* is its end state from H = 0, M the product of its chunks' transitions
// (from M = I).  With the per-chunk kernel's gated inverse A = (I + StrictLower(diag(beta)(Gamma (.)
// K K^T)))^-1, gamma_t = 2^(G_t) and the chunk decay gamma_C, one chunk is
//   X^T = -K^T diag(gamma_C / gamma) A diag(beta)          [D_k x 64], shared by S* and M
//   S*  <- gamma_C S* + X^T (diag(gamma) K S* - V)          (the pages' S* and Y)
//   M   <- gamma_C M  + X^T  diag(gamma) K M                (the pages' M and Z)
// which is the pages' recurrence with its factors placed differently: they build X from the
// ungated inverse A' and put gamma_C, gamma_C / gamma into Y; since A = Gamma (.) A' the products
// are the same, and here every factor is a decay of at most 1 and the stored gated inverse is used
// as it is.  Two products per column and chunk (K S, then X^T Y) instead of the main pass's three.
//
// Workgroup = (segment, value head, WC columns of the virtual [S* | M] column space: all of them
// when D_k = D_v), NW waves.
// Every wave owns CT 16-column tiles of all D_k rows in registers, so K S (over d) and X^T Y (over
// tokens) take their state-side operand straight from its own accumulators (pi order): the waves
// share only X^T, which they form together, and the tiles.  Per chunk c:
//   1  stage loads of chunk c + 1 (K, A, the gate block and, for S* columns, the V tile; direct to
//      LDS, two stages)
//   2  Y = diag(gamma) K S - V, S <- gamma_C S + X^T Y     (X^T, K, V of chunk c)
//   3  wait for chunk c + 1's stage; barrier
//   4  X^T of chunk c + 1 -> LDS; barrier
// Operands that are not inputs are bf16 hi/lo pairs (the state, Y, X^T, diag(gamma_C / gamma) A),
// as everywhere else in the forward.
//
// LDS tiles have a padded row pitch (one 16-byte granule more than the row): rows then start on
// distinct bank groups, so the 16-row operand reads are conflict free, and every address is a
// per-lane part fixed for the kernel plus a compile-time offset (no per-read address arithmetic).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

template <int DK, int NW, int CT, int VW>
struct CpLayout {
    static constexpr int WC = 16 * CT * NW;           // columns per workgroup
    using K = Pad<DK * 2 / 16>;                       // K tile
    using A = Pad<8>;                                 // A tile (64 x 64)
    using V = Pad<VW * 2 / 16>;                       // V tile of the workgroup's S* columns
    using X = Pad<8, DK>;                             // one part (hi or lo) of X^T: D_k rows of 64 tokens
    static constexpr int GT = GB_FLOATS * 4;          // gate block (unpadded)
    static constexpr int K0 = 0, A0 = K::BYTES, G0 = A0 + A::BYTES, V0 = G0 + GT, STAGE = V0 + V::BYTES;
    // stage instructions, in the order K, A, gate block, V (identity columns skip V); instruction i
    // is issued by wave i % NW
    static constexpr int NLG = GT / 1024;
    static constexpr int NLOAD_M = K::NI + A::NI + NLG, NLOAD = NLOAD_M + V::NI;
    static constexpr int NLW = (NLOAD + NW - 1) / NW;
    static constexpr int MD = DK / 16, NKB = DK / 32;
    static constexpr int TPW = MD * 4 / NW;           // X d-tiles per wave (16 tokens each)
    static_assert(NW == 4 || NW == 8, "four token tiles of X over the waves");
    static_assert(2 * STAGE + 2 * X::BYTES <= 160 * 1024, "LDS budget");
};

template <int DK, int NW, int CT, int VW>
__global__ __launch_bounds__(64 * NW, 1) void cp_pre_xyz_kernel(ChunkParams p, int n_blocks) {
    using L = CpLayout<DK, NW, CT, VW>;
    using KT = typename L::K;
    using AT = typename L::A;
    using VT = typename L::V;
    using XT = typename L::X;
    constexpr int MD = L::MD, NKB = L::NKB, NLW = L::NLW, TPW = L::TPW;
    // the two stages and the two X^T parts are separate objects, each named at compile time
    __shared__ __attribute__((aligned(16))) unsigned char sXh[XT::BYTES], sXl[XT::BYTES];
    __shared__ __attribute__((aligned(16))) unsigned char stg0[L::STAGE], stg1[L::STAGE];

    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // XCD-aware mapping: the column blocks of one (segment, head) share blockIdx % 8 (one XCD and
    // its L2), so the K and A tiles one of them fetches are L2 hits for the others
    const int bid = blockIdx.x, xcd = bid & 7, rr = bid >> 3;
    const int blk = rr % n_blocks, unit = (rr / n_blocks) * 8 + xcd;
    if (unit >= p.total_segs * p.H_v) return;
    const int gsi = unit / p.H_v, h = unit % p.H_v;
    const int gs = p.segs ? p.order[gsi] : gsi;
    const SegInfo sg = seg_info(p.segs, gs, p.T, p.seg_chunks);
    if (sg.last) return;                             // the last segment's maps are never needed
    const int DV = p.D_v;
    const int cb = blk * L::WC;                      // first virtual column of this workgroup
    const bool wblk = cb >= DV;                      // the workgroup holds identity columns only
    if (wblk && sg.j == 0 && !p.h0) return;          // M of a first segment multiplies h0 = 0
    const int wc0 = cb + 16 * CT * wave;             // this wave's first virtual column
    const bool mblk = wc0 >= DV;                     // identity columns: M
    const bool skip = mblk && sg.j == 0 && !p.h0;    // (formed with the S* columns, not stored)
    const int col0 = (mblk ? wc0 - DV : wc0) + l16;
    const int n = sg.n, hq = h / (p.H_v / p.H_qk);
    const SeqInfo si = seq_info(p.seq, n, p.T);
    const int cs = sg.c0, nch = sg.nchunks;
    const int qks = p.H_qk * DK, vs = p.H_v * DV;
    auto nvalid = [&](int c) { return min(kChunk, si.len - (cs + c) * kChunk); };

    const bf16 *kbase = static_cast<const bf16 *>(p.k) + (int64_t)hq * DK;
    const bf16 *vb = static_cast<const bf16 *>(p.v) + (int64_t)h * DV + cb;   // S* columns
    const bf16 *Ab = static_cast<const bf16 *>(p.A) + (int64_t)h * 4096;
    const float *Gb = p.gates + (int64_t)h * GB_FLOATS;

    // this wave's stage instructions: source byte offset (pad granules: out of range, zeros), LDS
    // position within the stage, source tile
    constexpr int kOut = 1 << 30;
    int soff[NLW], dst[NLW], kind[NLW];
#pragma unroll
    for (int j = 0; j < NLW; ++j) {
        const int i = wave + NW * j;
        int ii = i, pos, row, g;
        if (ii < KT::NI) {
            pos = 64 * ii + lane, row = pos / KT::P, g = pos % KT::P;
            kind[j] = 0;
            soff[j] = g < KT::P - 1 ? row * qks * 2 + 16 * g : kOut;
            dst[j] = L::K0 + 1024 * ii;
        } else if ((ii -= KT::NI) < AT::NI) {
            pos = 64 * ii + lane, row = pos / AT::P, g = pos % AT::P;
            kind[j] = 1;
            soff[j] = g < AT::P - 1 ? row * 128 + 16 * g : kOut;
            dst[j] = L::A0 + 1024 * ii;
        } else if ((ii -= AT::NI) < L::NLG) {
            kind[j] = 2;
            soff[j] = 1024 * ii + 16 * lane;
            dst[j] = L::G0 + 1024 * ii;
        } else {
            ii -= L::NLG;
            pos = 64 * ii + lane, row = pos / VT::P, g = pos % VT::P;
            kind[j] = i < L::NLOAD && !wblk ? 3 : 4;
            soff[j] = g < VT::P - 1 ? row * vs * 2 + 16 * g : kOut;
            dst[j] = L::V0 + 1024 * ii;
        }
    }
    // chunk c's tiles (past the segment: empty ranges, nothing is read; such stages are never used)
    auto load_stage = [&](int c, unsigned char *tb) __attribute__((always_inline)) {
        const bool live = c < nch;
        const int cc = live ? c : 0;
        const int64_t tok = si.tok0 + (int64_t)(cs + cc) * kChunk;
        const int64_t gci = si.chunk0 + cs + cc;
        const u32x4 rK = rsrc_words(kbase + tok * qks, live ? ((nvalid(cc) - 1) * qks + DK) * 2 : 0);
        const u32x4 rA = rsrc_words(Ab + gci * p.H_v * 4096, live ? 4096 * 2 : 0);
        const u32x4 rG = rsrc_words(Gb + gci * p.H_v * GB_FLOATS, live ? GB_FLOATS * 4 : 0);
        const u32x4 rV = rsrc_words(vb + tok * vs, live && !wblk ? ((nvalid(cc) - 1) * vs + VW) * 2 : 0);
#pragma unroll
        for (int j = 0; j < NLW; ++j) {
            if (kind[j] == 4) continue;
            const u32x4 r = kind[j] == 0 ? rK : kind[j] == 1 ? rA : kind[j] == 2 ? rG : rV;
            dma_granules(r, tb + dst[j], soff[j]);
        }
    };

    // state rows 16 m + 4 grp + r: S* from 0, M from the identity
    f32x4 S[MD][CT];
#pragma unroll
    for (int m = 0; m < MD; ++m)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) S[m][ct][r] = mblk && 16 * m + 4 * grp + r == col0 + 16 * ct ? 1.f : 0.f;

    // X^T of the chunk whose stage is st.  Wave w forms the transpose X[t][d] = -beta_t sum_s
    // (gamma_C / gamma_s) A[s][t] K[s][d] for the 16 tokens t of tile w % 4 and TPW tiles of d,
    // so each element of the scaled A is formed by NW / 4 waves; its accumulator runs (four
    // consecutive tokens of one d) are 8-byte runs of X^T rows.  (Token tiles 2 and 3 meet only
    // zeros of A in the first contraction block; those products are formed anyway, by waves that
    // would otherwise wait for the others at the barrier.)
    const int tw = wave & 3, dt0 = (wave >> 2) * TPW;
    auto form_x = [&](const unsigned char *st) __attribute__((always_inline)) {
        const unsigned char *tK = st + L::K0, *tA = st + L::A0;
        const float *g = reinterpret_cast<const float *>(st + L::G0);
        f32x4 acc[TPW];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const float4 sa = *reinterpret_cast<const float4 *>(g + GB_SC + 32 * kb + 4 * grp);
            const float4 sb = *reinterpret_cast<const float4 *>(g + GB_SC + 32 * kb + 16 + 4 * grp);
            const float sc[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
            const Frag<bf16> a = pi_col<AT>(tA, 16 * tw, kb, grp, l16);   // A[s][16 tw + l16]
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = sc[e] * (float)a.v[e];
            Frag<bf16> wh, wl;
            split8_rne(x, wh, wl);
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const Frag<bf16> kf = pi_col<KT>(tK, 16 * (dt0 + i), kb, grp, l16);
                if (kb == 0) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
                mma_pair_x(acc[i], wh, wl, kf);
            }
        }
        const float4 b4 = *reinterpret_cast<const float4 *>(g + GB_BETA + 16 * tw + 4 * grp);
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const f32x4 x = {-b4.x * acc[i][0], -b4.y * acc[i][1], -b4.z * acc[i][2], -b4.w * acc[i][3]};
            u32x2 hi, lo;
            split4(x, hi, lo);
            const int off = XT::off(16 * (dt0 + i) + l16, (16 * tw + 4 * grp) * 2);
            *reinterpret_cast<u32x2 *>(sXh + off) = hi;
            *reinterpret_cast<u32x2 *>(sXl + off) = lo;
        }
    };

    // Y = diag(gamma) K S - V, then S <- gamma_C S + X^T Y (chunk whose stage is st).  Every K and
    // X^T fragment read from LDS serves the wave's CT column tiles.
    auto advance = [&](const unsigned char *st) __attribute__((always_inline)) {
        const unsigned char *tK = st + L::K0;
        const float *g = reinterpret_cast<const float *>(st + L::G0);
        f32x4 y[4][CT];
        {
            Frag<bf16> sh[NKB][CT], sl[NKB][CT];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    float x[8];
                    pack_pi(S[2 * kb][ct], S[2 * kb + 1][ct], x);
                    split8_rne(x, sh[kb][ct], sl[kb][ct]);
                }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const Frag<bf16> kf = pi_row<KT>(tK, 16 * tt + l16, kb, grp);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) {
                        if (kb == 0) y[tt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
                        mma_x(y[tt][ct], kf, sh[kb][ct], sl[kb][ct]);
                    }
                }
                if (tt & 1) reg_fence();
            }
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const float4 ga = *reinterpret_cast<const float4 *>(g + GB_GAK + 16 * tt + 4 * grp);
            const float gav[4] = {ga.x, ga.y, ga.z, ga.w};
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                // V[16 tt + 4 grp + r][col]: transposed read, lane 4e + q of the group pointing at row
                // 16 tt + 4 grp + e, columns 16 (CT wave + ct) + 4 q .. + 3 of the workgroup's tile
                bf16x4 vv = {};
                if (!mblk)
                    vv = lds_read_tr16(st + L::V0 + VT::off(16 * tt + 4 * grp + (l16 >> 2),
                                                            (wc0 - cb + 16 * ct + 4 * (l16 & 3)) * 2));
#pragma unroll
                for (int r = 0; r < 4; ++r) y[tt][ct][r] = gav[r] * y[tt][ct][r] - (float)vv[r];
            }
        }
        Frag<bf16> yh[2][CT], yl[2][CT];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                float x[8];
                pack_pi(y[2 * kb][ct], y[2 * kb + 1][ct], x);
                split8_rne(x, yh[kb][ct], yl[kb][ct]);
            }
        const float gC = g[GB_GC];
#pragma unroll
        for (int m = 0; m < MD; ++m) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) S[m][ct] *= gC;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const Frag<bf16> xh = pi_row<XT>(sXh, 16 * m + l16, kb, grp);
                const Frag<bf16> xl = pi_row<XT>(sXl, 16 * m + l16, kb, grp);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) mma_xx(S[m][ct], xh, xl, yh[kb][ct], yl[kb][ct]);
            }
            if (m & 1) reg_fence();
        }
    };

    // prologue: the stage of chunk 0 and its X^T
    load_stage(0, stg0);
    wait_vm<0>();
    lds_only_barrier();
    form_x(stg0);
    lds_only_barrier();

    auto step = [&]<int SB>(int c) __attribute__((always_inline)) {
        const unsigned char *cur = SB == 0 ? stg0 : stg1;     // chunk c
        unsigned char *nxt = SB == 0 ? stg1 : stg0;           // chunk c + 1 (held chunk c - 1)
        if (c + 1 < nch) load_stage(c + 1, nxt);
        advance(cur);
        if (c + 1 < nch) {
            wait_vm<0>();          // this wave's share of chunk c + 1's stage
            lds_only_barrier();    // every wave's share; every wave is done with X^T of chunk c
            form_x(nxt);
            lds_only_barrier();    // X^T of chunk c + 1
        }
    };
    for (int c = 0; c < nch; c += 2) {
        step.template operator()<0>(c);
        if (c + 1 < nch) step.template operator()<1>(c + 1);
    }

    if (skip) return;
    if (!mblk) {
        float *dst = p.seg_sstar + ((int64_t)gs * p.H_v + h) * DK * DV;
#pragma unroll
        for (int m = 0; m < MD; ++m)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(16 * m + 4 * grp + r) * DV + col0 + 16 * ct] = S[m][ct][r];
    } else {
        // M as the fix-up's operand: bf16 hi and lo parts [2][D_k][D_k], each row's columns k in pi
        // order within every 32-block, so that one 16-byte load gives a lane its 8 values
        bf16 *dst = reinterpret_cast<bf16 *>(p.seg_m) + ((int64_t)gs * p.H_v + h) * 2 * DK * DK;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int k = col0 + 16 * ct;
            const int pos = (k & ~31) + 8 * ((k & 15) >> 2) + (k & 3) + 4 * ((k & 31) >> 4);
#pragma unroll
            for (int m = 0; m < MD; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float x = S[m][ct][r];
                    const bf16 hi = (bf16)x;
                    const int d = 16 * m + 4 * grp + r;
                    dst[d * DK + pos] = hi;
                    dst[(DK + d) * DK + pos] = (bf16)(x - (float)hi);
                }
        }
    }
}

// Context-parallel fix-up over the maps of the pre-process above (FlashQLA page, step 2.2):
// per (sequence, value head, 16 value columns), serially over the sequence's segments,
//   S_start(0) = h0 (or 0),   S_start(j + 1) = S*_j + M_j S_start(j),
// writing S_start(j) for j >= 1.  One wave per 16-row tile of the product.  M_j comes as bf16 pairs
// whose rows hold the operand order (one 16-byte load per lane, contraction block and part), three
// segments ahead, straight into registers; the new state goes through LDS as pairs, transposed, so
// the next step reads its operand with two 8-byte reads per block and part (one barrier per
// segment, two buffers).
// The steps run in rounds of eight with no branch inside a round: a round's loads are all consumed
// within it (so the compiler's wait counting needs no guess across the loop's back edge, where it
// would wait for every load in flight), steps past the last segment redo the last one's loads and
// drop their stores (empty buffer range), and the first step's product with M_0, which the
// pre-process does not form when h0 = 0, is computed and then dropped.
template <int DK>
__global__ __launch_bounds__(DK * 4) void cp_fix_xyz_kernel(FixParams p) {
    constexpr int NKB = DK / 32, PF = 3, NB = PF + 1, ROUND = 8;
    constexpr int TP = DK * 2 + 16;                // LDS row pitch (bytes) of the transposed state
    __shared__ __attribute__((aligned(16))) unsigned char sT[2][2][16 * TP];   // [buffer][part][col][row]
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

    // state as pairs into buffer buf: lane (wave m) writes rows 16 m + 4 grp .. + 3 of column l16
    auto put = [&](int buf, const f32x4 &x) __attribute__((always_inline)) {
        u32x2 hi, lo;
        split4(x, hi, lo);
        const int off = l16 * TP + (16 * m + 4 * grp) * 2;
        *reinterpret_cast<u32x2 *>(&sT[buf][0][off]) = hi;
        *reinterpret_cast<u32x2 *>(&sT[buf][1][off]) = lo;
    };
    {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (p.h0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = p.h0[((int64_t)n * p.H_v + h) * hstride + (16 * m + 4 * grp + r) * DV + c0 + l16];
        }
        put(0, x);
    }
    // segment j's operands (j clamped to the last step's): M_j row 16 m + l16 (pi order, both
    // parts) and this lane's S*_j values
    struct Raw {
        u32x4 mh[NKB], ml[NKB];
        float sst[4];
    };
    auto load_raw = [&](int j, Raw &rw) __attribute__((always_inline)) {
        j = min(j, ns - 2);
        const bf16 *Mj = reinterpret_cast<const bf16 *>(p.seg_m) + ((int64_t)(gs0 + j) * p.H_v + h) * 2 * DK * DK;
        const bf16 *rowh = Mj + (16 * m + l16) * DK + 8 * grp, *rowl = rowh + DK * DK;
        const float *Sj = p.seg_sstar + ((int64_t)(gs0 + j) * p.H_v + h) * hstride;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            rw.mh[kb] = *reinterpret_cast<const u32x4 *>(rowh + 32 * kb);
            rw.ml[kb] = *reinterpret_cast<const u32x4 *>(rowl + 32 * kb);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) rw.sst[r] = Sj[(16 * m + 4 * grp + r) * DV + c0 + l16];
    };
    Raw raw[NB];

    // step j of a round (k = j - j0); B2 = state buffer (k % 2), BR = register set (k % NB)
    auto step = [&]<int K, int B2, int BR>(int j) __attribute__((always_inline)) {
        if constexpr (K + PF < ROUND) load_raw(j + PF, raw[(BR + PF) % NB]);
        reg_fence();       // the loads stay here, PF steps ahead of their use
        lds_only_barrier();   // S_start(j) is complete in buffer B2
        f32x4 acc0 = {raw[BR].sst[0], raw[BR].sst[1], raw[BR].sst[2], raw[BR].sst[3]};
        f32x4 acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const unsigned char *bh = &sT[B2][0][l16 * TP + (32 * kb + 4 * grp) * 2];
            const unsigned char *bl = &sT[B2][1][l16 * TP + (32 * kb + 4 * grp) * 2];
            const bf16x4 h0 = *reinterpret_cast<const bf16x4 *>(bh), h1 = *reinterpret_cast<const bf16x4 *>(bh + 32);
            const bf16x4 l0 = *reinterpret_cast<const bf16x4 *>(bl), l1 = *reinterpret_cast<const bf16x4 *>(bl + 32);
            Frag<bf16> fbh, fbl, fmh, fml;
            fbh.v = bf16x8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
            fbl.v = bf16x8{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
            fmh.v = __builtin_bit_cast(bf16x8, raw[BR].mh[kb]);
            fml.v = __builtin_bit_cast(bf16x8, raw[BR].ml[kb]);
            mma_xx(kb & 1 ? acc1 : acc0, fmh, fml, fbh, fbl);
        }
        f32x4 acc = acc0 + acc1;
        if (j == 0 && !p.h0) acc = f32x4{raw[BR].sst[0], raw[BR].sst[1], raw[BR].sst[2], raw[BR].sst[3]};
        put(B2 ^ 1, acc);
        // S_start(j + 1), dropped past the last segment
        const bool live = j + 1 < ns;
        const float *dst = p.seg_start + ((int64_t)(gs0 + (live ? j + 1 : 1)) * p.H_v + h) * hstride;
        const auto rs = make_rsrc(dst, live ? (int)(hstride * 4) : 0);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[r]), rs, ((16 * m + 4 * grp + r) * DV + c0 + l16) * 4, 0, 0);
    };
    for (int j0 = 0; j0 + 1 < ns; j0 += ROUND) {
#pragma unroll
        for (int q = 0; q < PF; ++q) load_raw(j0 + q, raw[q]);
        step.template operator()<0, 0, 0>(j0);
        step.template operator()<1, 1, 1>(j0 + 1);
        step.template operator()<2, 0, 2>(j0 + 2);
        step.template operator()<3, 1, 3>(j0 + 3);
        step.template operator()<4, 0, 0>(j0 + 4);
        step.template operator()<5, 1, 1>(j0 + 5);
        step.template operator()<6, 0, 2>(j0 + 6);
        step.template operator()<7, 1, 3>(j0 + 7);
    }
}

}  // namespace

hipError_t launch_cp_pre_xyz(int D_k, const ChunkParams &p, hipStream_t s) {
    const int DV = p.D_v;
    const int64_t units = (int64_t)p.total_segs * p.H_v;
    if (units == 0) return hipSuccess;
    // equal key and value widths: one workgroup per (segment, head) holds S* and M together (eight
    // waves, X^T formed once); otherwise workgroups of 64 columns of either
    const bool one = DV == D_k;
    const int n_blocks = one ? 1 : (DV + D_k) / 64;
    const dim3 grid((unsigned)(((units + 7) / 8) * 8 * n_blocks));
    if (one && D_k == 128) launch_k(cp_pre_xyz_kernel<128, 8, 2, 128>, grid, dim3(512), s, p, n_blocks);
    else if (one && D_k == 64) launch_k(cp_pre_xyz_kernel<64, 8, 1, 64>, grid, dim3(512), s, p, n_blocks);
    else if (D_k == 128 && DV == 64) launch_k(cp_pre_xyz_kernel<128, 4, 1, 64>, grid, dim3(256), s, p, n_blocks);
    else if (D_k == 64 && DV == 128) launch_k(cp_pre_xyz_kernel<64, 4, 1, 64>, grid, dim3(256), s, p, n_blocks);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_cp_fix_xyz(int D_k, const FixParams &p, hipStream_t s) {
    // XCD-aware: blockIdx = ((unit / 8) * slices + slice) * 8 + unit % 8
    const unsigned groups = (unsigned)((p.N * p.H_v + 7) / 8);
    const dim3 grid(groups * 8u * (unsigned)(p.D_v / 16)), block((unsigned)(D_k * 4));
    if (p.N * p.H_v == 0) return hipSuccess;
    if (D_k == 128) launch_k(cp_fix_xyz_kernel<128>, grid, block, s, p);
    else if (D_k == 64) launch_k(cp_fix_xyz_kernel<64>, grid, block, s, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gdn
