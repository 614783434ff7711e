// Per-chunk gradients of the backward on the matrix cores (bf16 inputs, scalar gate): the same
// quantities as the plain bwd_chunk_kernel (GDN-in-FLA notes, backward Steps 3-7; the formulas are
// in gdn_bwd.hip's header), per (chunk, value head) workgroup of eight waves:
//   value columns in halves of 64:  K S, K dS_next;  X = diag(beta)(V - diag(gamma) K S);
//     V' = A X;  dV' = diag(D) K dS_next + Pt^T dO;  dX = A^T dV';  dv = diag(beta) dX;
//     dA += dV' X^T;  dPt += dO V'^T;  dq_S += dO S^T;  dk_D += V' dS_next^T;  dk_X += dX S^T
//   then:  dq = scale diag(gamma) dq_S,  dk = diag(D) dk_D - diag(beta gamma) dk_X;
//     T = A^T dA,  dL = -T A^T (strictly lower),  G = Gamma (.) K K^T (strictly lower);
//     M1 = scale dPt (.) Gamma (lower with the diagonal),  E = diag(beta) dL (.) Gamma;
//     dq += M1 K,  dk += M1^T Q + E K + E^T K;  dbeta and d gl from every term, dg their reverse
//     cumsum within the chunk.
// Operands that are not inputs (the recomputed states, every intermediate) are bf16 hi/lo pairs, as
// in the forward.  Token-by-column intermediates are kept in LDS transposed ([column][token]), so
// that both the products over tokens and those over columns read them with 8-byte or transposed
// reads; the tiles are padded (one granule per row) and filled with direct-to-LDS loads.
// The phase barriers wait for LDS traffic only (explicit waits cover the tile loads): the gradient
// stores and the state values read ahead for the next phase stay in flight across them.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

template <int DK>
struct BcLayout {
    static constexpr int NW = 8;
    using K = Pad<DK * 2 / 16>;               // K and Q tiles
    using S = Pad<8>;                         // every 64 x 64 bf16 tile
    static constexpr int K0 = 0, Q0 = K::BYTES, A0 = 2 * K::BYTES;
    static constexpr int PH = A0 + S::BYTES, PL = PH + S::BYTES;     // Pt pair [i][j]
    static constexpr int V0 = PL + S::BYTES, O0 = V0 + S::BYTES;     // V, dO halves [t][c]
    static constexpr int X0 = O0 + S::BYTES;                         // X, V', dV', dX pairs [c][t]
    static constexpr int G0 = X0 + 8 * S::BYTES, BYTES = G0 + GB_FLOATS * 4;
    static constexpr int MD = DK / 16, NKB = DK / 32, NQT = MD / 2;  // dq/dk tiles per wave
    static_assert(BYTES <= 160 * 1024 - 1024, "LDS budget");
};

// rows [row0, row0 + 4) of column col of a tile (transposed read; the row0 / col of lane l16 of
// group grp must be 16 a + 4 grp and 16 b + l16)
template <typename PT>
__device__ __forceinline__ bf16x4 col4(const unsigned char *tile, int r16, int c16, int grp, int l16) {
    return lds_read_tr16(tile + PT::off(16 * r16 + 4 * grp + (l16 >> 2), (16 * c16 + 4 * (l16 & 3)) * 2));
}
// the pair of four accumulator values (rows a .. a + 3 of column b) stored transposed: row b,
// columns a .. a + 3
template <typename PT>
__device__ __forceinline__ void put_t(unsigned char *th, unsigned char *tl, int b, int a, const f32x4 &x) {
    u32x2 hi, lo;
    split4(x, hi, lo);
    *reinterpret_cast<u32x2 *>(th + PT::off(b, a * 2)) = hi;
    *reinterpret_cast<u32x2 *>(tl + PT::off(b, a * 2)) = lo;
}
// x from the lane the DPP control picks within this lane's row of 16 (all lanes active)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}
// over the 16 lanes of a group, on the DPP crossbar instead of LDS permutes: quad_perm [1,0,3,2]
// and [2,3,0,1] (lane xor 1, xor 2), then row_half_mirror and row_mirror, which pair the quads and
// the halves of the row as xor 4 and xor 8 would; every lane ends with the same total, added in the
// same order as the xor butterfly.  Call with the whole wave active.
__device__ __forceinline__ float sum16(float x) {
    x += dpp_f32<0xb1>(x);
    x += dpp_f32<0x4e>(x);
    x += dpp_f32<0x141>(x);
    x += dpp_f32<0x140>(x);
    return x;
}
__device__ __forceinline__ float sum_groups(float x) {   // over the 4 groups (same l16)
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}

template <int DK>
__global__ __launch_bounds__(512, 1) void bwd_chunk_mma_kernel(BwdParams p) {
    using L = BcLayout<DK>;
    using KT = typename L::K;
    using ST = typename L::S;
    constexpr int NKB = L::NKB, MD = L::MD, NQT = L::NQT, NW = L::NW;
    __shared__ __attribute__((aligned(16))) unsigned char lds[L::BYTES];
    __shared__ float rdgl[64], rdb[64], rsc[64], rglc[1];
    unsigned char *tK = lds + L::K0, *tQ = lds + L::Q0, *tA = lds + L::A0, *tPh = lds + L::PH, *tPl = lds + L::PL;
    unsigned char *tV = lds + L::V0, *tO = lds + L::O0;
    unsigned char *tXh = lds + L::X0, *tXl = tXh + ST::BYTES, *tVh = tXl + ST::BYTES, *tVl = tVh + ST::BYTES;
    unsigned char *tDh = tVl + ST::BYTES, *tDl = tDh + ST::BYTES, *tEh = tDl + ST::BYTES, *tEl = tEh + ST::BYTES;
    const float *g = reinterpret_cast<const float *>(lds + L::G0);

    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ci = blockIdx.x / p.H_v, h = blockIdx.x - ci * p.H_v;
    const int hq = h / (p.H_v / p.H_qk);
    const ChunkInfo cinfo = chunk_info(p.chunks, ci, p.T);
    const int64_t tok0 = cinfo.tok0;
    const int nv = cinfo.nv;
    const int DV = p.D_v, qks = p.H_qk * DK, vs = p.H_v * DV;
    const float *St = p.states + ((int64_t)ci * p.H_v + h) * DK * DV;
    const float *dSt = p.dsnext + ((int64_t)ci * p.H_v + h) * DK * DV;

    // ---- tiles: padded rows through direct-to-LDS loads (pad granules read zeros)
    auto load = [&]<typename PT>(unsigned char *tile, u32x4 r, int stride) __attribute__((always_inline)) {
        for (int i = w; i < PT::NI; i += NW) {
            const int pos = 64 * i + lane, row = pos / PT::P, gg = pos % PT::P;
            dma_granules(r, tile + 1024 * i, gg < PT::P - 1 ? row * stride + 16 * gg : (1 << 30));
        }
    };
    auto load_half = [&](int hv) __attribute__((always_inline)) {
        const bf16 *vb = static_cast<const bf16 *>(p.v) + tok0 * vs + (int64_t)h * DV + 64 * hv;
        const bf16 *ob = static_cast<const bf16 *>(p.dout) + tok0 * vs + (int64_t)h * DV + 64 * hv;
        load.template operator()<ST>(tV, rsrc_words(vb, ((nv - 1) * vs + 64) * 2), vs * 2);
        load.template operator()<ST>(tO, rsrc_words(ob, ((nv - 1) * vs + 64) * 2), vs * 2);
    };
    {
        const bf16 *kb_ = static_cast<const bf16 *>(p.k) + tok0 * qks + (int64_t)hq * DK;
        const bf16 *qb = static_cast<const bf16 *>(p.q) + tok0 * qks + (int64_t)hq * DK;
        load.template operator()<KT>(tK, rsrc_words(kb_, ((nv - 1) * qks + DK) * 2), qks * 2);
        load.template operator()<KT>(tQ, rsrc_words(qb, ((nv - 1) * qks + DK) * 2), qks * 2);
        load.template operator()<ST>(tA, rsrc_words(static_cast<const bf16 *>(p.A) + ((int64_t)ci * p.H_v + h) * 4096, 8192), 128);
        if (w < GB_FLOATS * 4 / 1024)
            dma_granules(rsrc_words(p.gates + ((int64_t)ci * p.H_v + h) * GB_FLOATS, GB_FLOATS * 4),
                         lds + L::G0 + 1024 * w, 1024 * w + 16 * lane);
        load_half(0);
    }
    // S and dS_next values of P1 (this lane's value column, D_k rows in pi order), read from memory
    // ahead of the barrier that precedes their use, together with the tile loads
    const int ct = w & 3, tt0 = 2 * (w >> 2);             // token x column tiles of the half
    float ps[NKB][8], pd[NKB][8];
    auto ld_p1 = [&](int hv) __attribute__((always_inline)) {
        const int cg = 64 * hv + 16 * ct + l16;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = 32 * kb + (e < 4 ? 4 * grp + e : 16 + 4 * grp + e - 4);
                ps[kb][e] = St[d * DV + cg];
                pd[kb][e] = dSt[d * DV + cg];
            }
    };
    // S and dS_next values of P4 (rows 16 m + l16, this half's columns in pi order), read at the
    // start of P3
    const int m = w % MD;
    float qs[2][8], qd[2][8];
    auto ld_p4 = [&](int hv) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = 64 * hv + 32 * kb + (e < 4 ? 4 * grp + e : 16 + 4 * grp + e - 4);
                qs[kb][e] = St[(16 * m + l16) * DV + c];
                qd[kb][e] = dSt[(16 * m + l16) * DV + c];
            }
    };
    ld_p1(0);
    if (tid < 64) rdgl[tid] = rdb[tid] = rsc[tid] = 0.f;
    if (tid == 0) rglc[0] = 0.f;
    wait_vm<0>();
    lds_only_barrier();

    // gate rows of this lane's accumulator rows 16 a + 4 grp + r
    auto rows4 = [&](int off, int a) __attribute__((always_inline)) {
        return *reinterpret_cast<const float4 *>(g + off + 16 * a + 4 * grp);
    };

    // ---- Pt = scale Gamma (.) Q K^T (lower with the diagonal), a pair [i][j]; tiles w, w + 8
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int tix = w + 8 * q, ti = tix >> 2, tj = tix & 3;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (tj <= ti) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) mma(acc, pi_row<KT>(tQ, 16 * ti + l16, kb, grp), pi_row<KT>(tK, 16 * tj + l16, kb, grp));
        }
        const float4 gq = rows4(GB_GLQ, ti);
        const float glk = g[GB_GLK + 16 * tj + l16];
        const float gqv[4] = {gq.x, gq.y, gq.z, gq.w};
        const int j = 16 * tj + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * ti + 4 * grp + r;
            const float x = j <= i ? p.scale * fast_exp2(gqv[r] - glk) * acc[r] : 0.f;
            const bf16 hi = (bf16)x;
            *reinterpret_cast<bf16 *>(tPh + ST::off(i, j * 2)) = hi;
            *reinterpret_cast<bf16 *>(tPl + ST::off(i, j * 2)) = (bf16)(x - (float)hi);
        }
    }

    // accumulators over both halves
    f32x4 dA[2], dP[2];                                   // 64 x 64 tiles w, w + 8
    f32x4 dqS[NQT], dkD[NQT], dkX[NQT];                   // dq / dk tiles (tt, m)
#pragma unroll
    for (int q = 0; q < 2; ++q) dA[q] = dP[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < NQT; ++q) dqS[q] = dkD[q] = dkX[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int qt0 = (w / MD) * NQT;                       // dq / dk tiles: rows 16 m of D_k, tokens
    const float gC = g[GB_GC];

    const int NH = DV / 64;                               // halves of the value columns
    // one half of the value columns; the second half is a separate inlined copy, so that the state
    // values read ahead for its P1 are not carried around a loop
    auto half = [&](int hv) __attribute__((always_inline)) {
        lds_only_barrier();   // the half's V and dO tiles have landed; Pt (first half) is complete
        const int colg = 64 * hv + 16 * ct + l16;          // this lane's value column (P1 - P3)
        // ---- P1: K S, K dS_next, X
        f32x4 ks[2], kd[2];
        {
            Frag<bf16> sh[NKB], sl[NKB], dh[NKB], dl[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                split8_rne(ps[kb], sh[kb], sl[kb]);
                split8_rne(pd[kb], dh[kb], dl[kb]);
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int tt = tt0 + q;
                ks[q] = kd[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const Frag<bf16> kf = pi_row<KT>(tK, 16 * tt + l16, kb, grp);
                    mma_x(ks[q], kf, sh[kb], sl[kb]);
                    mma_x(kd[q], kf, dh[kb], dl[kb]);
                }
            }
        }
        float vv[2][4];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int tt = tt0 + q;
            const bf16x4 v4 = col4<ST>(tV, tt, ct, grp, l16);
            const float4 be = rows4(GB_BETA, tt), ga = rows4(GB_GAK, tt);
            const float bev[4] = {be.x, be.y, be.z, be.w}, gav[4] = {ga.x, ga.y, ga.z, ga.w};
            f32x4 x;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                vv[q][r] = (float)v4[r];
                x[r] = bev[r] * (vv[q][r] - gav[r] * ks[q][r]);
            }
            put_t<ST>(tXh, tXl, 16 * ct + l16, 16 * tt + 4 * grp, x);
        }
        lds_only_barrier();
        // ---- P2: V' = A X, dV' = diag(D) K dS_next + Pt^T dO; the D terms of d gl
        f32x4 vp[2], dvp[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int tt = tt0 + q;
            vp[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (32 * kb > 16 * tt + 15) continue;         // A[t][s] = 0 for s > t
                mma_x(vp[q], pi_row<ST>(tA, 16 * tt + l16, kb, grp), pi_row<ST>(tXh, 16 * ct + l16, kb, grp),
                      pi_row<ST>(tXl, 16 * ct + l16, kb, grp));
            }
            const float4 d4 = rows4(GB_SC, tt);
            const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) dvp[q][r] = dv4[r] * kd[q][r];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (32 * kb + 31 < 16 * tt) continue;         // Pt[s][t] = 0 for s < t
                mma_pair_x(dvp[q], pi_col<ST>(tPh, 16 * tt, kb, grp, l16), pi_col<ST>(tPl, 16 * tt, kb, grp, l16),
                           pi_col<ST>(tO, 16 * ct, kb, grp, l16));
            }
            put_t<ST>(tVh, tVl, 16 * ct + l16, 16 * tt + 4 * grp, vp[q]);
            put_t<ST>(tDh, tDl, 16 * ct + l16, 16 * tt + 4 * grp, dvp[q]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float cd = sum16(kd[q][r] * vp[q][r]) * dv4[r];
                if (l16 == 0) {
                    atomicAdd(&rdgl[16 * tt + 4 * grp + r], -cd);
                    atomicAdd(&rsc[16 * tt + 4 * grp + r], cd);
                }
            }
        }
        lds_only_barrier();
        // ---- P3: dX = A^T dV', dv, the X terms of dbeta and d gl
        ld_p4(hv);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int tt = tt0 + q;
            f32x4 dx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (32 * kb + 31 < 16 * tt) continue;         // A[s][t] = 0 for s < t
                mma_x(dx, pi_col<ST>(tA, 16 * tt, kb, grp, l16), pi_row<ST>(tDh, 16 * ct + l16, kb, grp),
                      pi_row<ST>(tDl, 16 * ct + l16, kb, grp));
            }
            const float4 be = rows4(GB_BETA, tt), ga = rows4(GB_GAK, tt);
            const float bev[4] = {be.x, be.y, be.z, be.w}, gav[4] = {ga.x, ga.y, ga.z, ga.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * tt + 4 * grp + r;
                if (t < nv) p.dv[(tok0 + t) * vs + (int64_t)h * DV + colg] = bev[r] * dx[r];
                const float db = sum16(dx[r] * (vv[q][r] - gav[r] * ks[q][r]));
                const float dg = sum16(dx[r] * ks[q][r]);
                if (l16 == 0) {
                    atomicAdd(&rdb[t], db);
                    atomicAdd(&rdgl[t], -bev[r] * gav[r] * dg);
                }
            }
            put_t<ST>(tEh, tEl, 16 * ct + l16, 16 * tt + 4 * grp, dx);
        }
        lds_only_barrier();
        // ---- P4: the products over this half's columns
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int tix = w + 8 * q, ti = tix >> 2, tj = tix & 3;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                mma_xx(dA[q], pi_col<ST>(tDh, 16 * ti, kb, grp, l16), pi_col<ST>(tDl, 16 * ti, kb, grp, l16),
                       pi_col<ST>(tXh, 16 * tj, kb, grp, l16), pi_col<ST>(tXl, 16 * tj, kb, grp, l16));
                if (tj <= ti)
                    mma_x(dP[q], pi_row<ST>(tO, 16 * ti + l16, kb, grp), pi_col<ST>(tVh, 16 * tj, kb, grp, l16),
                          pi_col<ST>(tVl, 16 * tj, kb, grp, l16));
            }
        }
        {
            // S and dS_next rows 16 m + l16 over this half's columns, in pi order
            Frag<bf16> sh[2], sl[2], dh[2], dl[2];
            float fro = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int e = 0; e < 8; ++e) fro += qs[kb][e] * qd[kb][e];
                split8_rne(qs[kb], sh[kb], sl[kb]);
                split8_rne(qd[kb], dh[kb], dl[kb]);
            }
            // gamma_C <S, dS_next> (each element once: the waves past the D_k rows' owners skip it)
            if (w < MD) {
                fro = sum_groups(sum16(fro));
                if (lane == 0) atomicAdd(&rglc[0], gC * fro);
            }
#pragma unroll
            for (int q = 0; q < NQT; ++q) {
                const int tt = qt0 + q;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    mma_x(dqS[q], pi_row<ST>(tO, 16 * tt + l16, kb, grp), sh[kb], sl[kb]);
                    mma_xx(dkD[q], pi_col<ST>(tVh, 16 * tt, kb, grp, l16), pi_col<ST>(tVl, 16 * tt, kb, grp, l16), dh[kb], dl[kb]);
                    mma_xx(dkX[q], pi_col<ST>(tEh, 16 * tt, kb, grp, l16), pi_col<ST>(tEl, 16 * tt, kb, grp, l16), sh[kb], sl[kb]);
                }
            }
        }
    };
    half(0);
    if (NH > 1) {
        lds_only_barrier();   // every wave is done with the first half's tiles
        load_half(1);
        ld_p1(1);
        wait_vm<0>();
        half(1);
    }

    // ---- dq, dk through the states; the q . dq term of d gl
    f32x4 dq[NQT], dk[NQT];
#pragma unroll
    for (int q = 0; q < NQT; ++q) {
        const int tt = qt0 + q;
        const float4 gq = rows4(GB_GAQ, tt), d4 = rows4(GB_SC, tt), be = rows4(GB_BETA, tt), ga = rows4(GB_GAK, tt);
        const float gqv[4] = {gq.x, gq.y, gq.z, gq.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
        const float bev[4] = {be.x, be.y, be.z, be.w}, gav[4] = {ga.x, ga.y, ga.z, ga.w};
        const bf16x4 q4 = col4<KT>(tQ, tt, m, grp, l16);   // q[t][16 m + l16]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            dq[q][r] = p.scale * gqv[r] * dqS[q][r];
            dk[q][r] = dv4[r] * dkD[q][r] - bev[r] * gav[r] * dkX[q][r];
            const float e = sum16((float)q4[r] * dq[q][r]);
            if (l16 == 0) atomicAdd(&rdgl[16 * tt + 4 * grp + r], e);
        }
    }
    lds_only_barrier();   // every wave is done with the pair buffers
    // ---- dA transposed ([s][t]) into the X buffers
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int tix = w + 8 * q, ti = tix >> 2, tj = tix & 3;
        put_t<ST>(tXh, tXl, 16 * tj + l16, 16 * ti + 4 * grp, dA[q]);
    }
    lds_only_barrier();
    // ---- T = A^T dA, transposed ([t][i]) into the V' buffers
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int tix = w + 8 * q, ti = tix >> 2, tj = tix & 3;
        f32x4 T = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (32 * kb + 31 < 16 * ti) continue;             // A[t][i] = 0 for t < i
            mma_x(T, pi_col<ST>(tA, 16 * ti, kb, grp, l16), pi_row<ST>(tXh, 16 * tj + l16, kb, grp),
                  pi_row<ST>(tXl, 16 * tj + l16, kb, grp));
        }
        put_t<ST>(tVh, tVl, 16 * tj + l16, 16 * ti + 4 * grp, T);
    }
    lds_only_barrier();
    // ---- dL, G, the L and Pt terms of dbeta and d gl; M1 and E transposed into the dV' and dX buffers
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int tix = w + 8 * q, ti = tix >> 2, tj = tix & 3;
        f32x4 dl = {0.f, 0.f, 0.f, 0.f}, gm = {0.f, 0.f, 0.f, 0.f};
        if (tj <= ti) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (32 * kb > 16 * tj + 15) continue;         // A[j][t] = 0 for t > j
                mma_pair_x(dl, pi_col<ST>(tVh, 16 * ti, kb, grp, l16), pi_col<ST>(tVl, 16 * ti, kb, grp, l16),
                           pi_row<ST>(tA, 16 * tj + l16, kb, grp));
            }
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) mma(gm, pi_row<KT>(tK, 16 * ti + l16, kb, grp), pi_row<KT>(tK, 16 * tj + l16, kb, grp));
        }
        const bf16x4 ph = col4<ST>(tPh, ti, tj, grp, l16), pl = col4<ST>(tPl, ti, tj, grp, l16);
        const float4 gq = rows4(GB_GLQ, ti), gk = rows4(GB_GLK, ti), be = rows4(GB_BETA, ti);
        const float gqv[4] = {gq.x, gq.y, gq.z, gq.w}, gkv[4] = {gk.x, gk.y, gk.z, gk.w}, bev[4] = {be.x, be.y, be.z, be.w};
        const int j = 16 * tj + l16;
        const float glkj = g[GB_GLK + j];
        f32x4 m1, e1;
        float colsum = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * ti + 4 * grp + r;
            const bool lo = j < i, le = j <= i;
            const float dL = lo ? -dl[r] : 0.f;
            const float G = lo ? fast_exp2(gkv[r] - glkj) * gm[r] : 0.f;
            const float a = dL * G;
            const float f = le ? dP[q][r] * ((float)ph[r] + (float)pl[r]) : 0.f;
            const float u = bev[r] * a + f;                   // + to d gl_i, - to d gl_j
            colsum += u;
            const float db = sum16(a), du = sum16(u);
            if (l16 == 0) {
                atomicAdd(&rdb[i], db);
                atomicAdd(&rdgl[i], du);
            }
            const float gam = fast_exp2(gqv[r] - glkj);
            m1[r] = le ? p.scale * dP[q][r] * gam : 0.f;
            e1[r] = lo ? dL * bev[r] * fast_exp2(gkv[r] - glkj) : 0.f;
        }
        colsum = sum_groups(colsum);
        if (grp == 0) atomicAdd(&rdgl[j], -colsum);
        put_t<ST>(tDh, tDl, j, 16 * ti + 4 * grp, m1);
        put_t<ST>(tEh, tEl, j, 16 * ti + 4 * grp, e1);
    }
    lds_only_barrier();
    // ---- dq += M1 K, dk += M1^T Q + E K + E^T K; stores
    const int hs = p.dq_v == p.dq ? hq : h, hn = p.dq_v == p.dq ? p.H_qk : p.H_v;
#pragma unroll
    for (int q = 0; q < NQT; ++q) {
        const int tt = qt0 + q;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const Frag<bf16> kc = pi_col<KT>(tK, 16 * m, kb, grp, l16);     // K[j][16 m + l16]
            if (32 * kb <= 16 * tt + 15) {                    // M1[t][j], E[t][j]: j <= t
                mma_pair_x(dq[q], pi_col<ST>(tDh, 16 * tt, kb, grp, l16), pi_col<ST>(tDl, 16 * tt, kb, grp, l16), kc);
                mma_pair_x(dk[q], pi_col<ST>(tEh, 16 * tt, kb, grp, l16), pi_col<ST>(tEl, 16 * tt, kb, grp, l16), kc);
            }
            if (32 * kb + 31 >= 16 * tt) {                    // M1[j][t], E[j][t]: j >= t
                mma_pair_x(dk[q], pi_row<ST>(tDh, 16 * tt + l16, kb, grp), pi_row<ST>(tDl, 16 * tt + l16, kb, grp),
                           pi_col<KT>(tQ, 16 * m, kb, grp, l16));
                mma_pair_x(dk[q], pi_row<ST>(tEh, 16 * tt + l16, kb, grp), pi_row<ST>(tEl, 16 * tt + l16, kb, grp), kc);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * tt + 4 * grp + r;
            if (t < nv) {
                const int64_t o = ((tok0 + t) * hn + hs) * DK + 16 * m + l16;
                p.dq_v[o] = dq[q][r];
                p.dk_v[o] = dk[q][r];
            }
        }
    }
    lds_only_barrier();   // every row term of d gl and dbeta is in
    if (tid < 64) {
        float x = tid < nv ? rdgl[tid] : 0.f;
        if (tid == max(nv - 1, 0)) {
            float s = rglc[0];
            for (int j = 0; j < 64; ++j) s += rsc[j];
            x += s;
        }
        const float incl = wave_inclusive_scan(x);
        const float tot = __shfl(incl, 63, 64);
        if (tid < nv) {
            p.dg[(tok0 + tid) * p.H_v + h] = tot - incl + x;
            p.dbeta[(tok0 + tid) * p.H_v + h] = rdb[tid];
        }
    }
}

// ==========================================================================================
// Per-channel gates, bf16 inputs: every gradient of a chunk's inputs (the quantities of the plain
// kernels (a) and (b) together), per (chunk, value head) workgroup of eight waves, from the
// per-chunk kernel's fp16 operands (Kg = K e^G, Kd = K e^{G_C - G}, A, scale P):
//   value columns in halves of 64:  Kg S, Kd dS_next;  X = diag(beta)(V - Kg S);  V' = A X;
//     dV' = Kd dS_next + (scale P)^T dO;  dX = A^T dV';  dv = diag(beta) dX;  dA += dV' X^T;
//     dP += dO V'^T;  dq_S += dO S^T;  dk_D += V' dS_next^T;  dk_X += dX S^T;
//     e^{G_C} <S, dS_next> per channel
//   then:  dq = scale e^G (.) dq_S,  dk = e^{G_C - G} (.) dk_D - diag(beta) e^G (.) dk_X,
//     dL = -A^T dA A^T (strictly lower), dP scaled (lower with the diagonal);
//     the P and L terms with their per-channel factors e^{G_r - G_t}, for the rows r of block R:
//       aq = sum_{t<r} dP[r][t] k_t e^{G_r - G_t},   ar = sum_{t<r} dL[r][t] k_t e^{G_r - G_t},
//       ap = sum_{t>r} dP[t][r] q_t e^{G_t - G_r},   al = sum_{t>r} dL[t][r] beta_t k_t e^{G_t - G_r},
//     each one contraction on the matrix cores with the factor split at one reference row, 16 R - 1
//     (left sums) or 16 R + 15 (right sums): e^{G_r - G_t} = e^{G_r - G_a} e^{G_a - G_t}, the first
//     at most 1, the second at most 1 outside block R and at most the block's own decay inside it;
//     a column whose decay across block R exceeds e^kMaxLn takes that block's pairs whole on the
//     vector ALU instead;
//     dq += aq + dP[r][r] k_r,  dk += ap + dP[r][r] q_r + beta_r ar + al,
//     dG = q (.) dq_S-part + k (.) (dk_X part) - k (.) (dk_D part) + q aq + k beta ar - k (ap + al),
//     with the e^{G_C} terms on the chunk's last valid row, and dg its reverse cumsum per channel;
//     dbeta from X and from L (sum_d k_rd ar_rd).
// The operands formed here (S, dS_next, X, V', dV', dX, dA, dP, dL and the factored K and Q) are
// fp16 hi/lo pairs, hi = fp16(x), lo = fp16(x - hi): with steep gates single terms of a chunk's
// first or last token are far above the gradients' RMS, and one fp16 rounding of them would not
// keep those within the bound.
// Largest decay (natural log) across a 16-row block for which a column's split factors are used:
// the factors inside the block then stay below e^kMaxLn (fp16 holds them with room to spare).
constexpr float kMaxLn = 9.5f;

template <int DK>
struct KaLayout {
    static constexpr int NW = 8;
    using K = Pad<DK * 2 / 16>;               // Kg and Kd tiles
    using S = Pad<8>;                         // every 64 x 64 16-bit tile
    static constexpr int KG0 = 0, KD0 = K::BYTES, A0 = 2 * K::BYTES, P0 = A0 + S::BYTES;
    static constexpr int V0 = P0 + S::BYTES, O0 = V0 + S::BYTES;     // V, dO halves [t][c] (bf16)
    static constexpr int X0 = O0 + S::BYTES;                         // X, V', dV', dX pairs [c][t] (fp16)
    static constexpr int G0 = X0 + 8 * S::BYTES, BYTES = G0 + GB_FLOATS * 4;
    static constexpr int MD = DK / 16, NKB = DK / 32, NQT = MD / 2;  // dq/dk tiles per wave
    static_assert(BYTES <= 160 * 1024 - 1024, "LDS budget");
};

// fp16 operand of eight bf16 values (exact inside fp16's normal range)
__device__ __forceinline__ Frag<f16> bf_to_f16(const Frag<bf16> &f) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)f.v[e];
    Frag<f16> r, unused;
    split8(x, r, unused);
    return r;
}
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
// the fp16 pair of four accumulator values (rows a .. a + 3 of column b) stored transposed: row b,
// columns a .. a + 3 of the hi and lo tiles
template <typename PT>
__device__ __forceinline__ void put_t16(unsigned char *th, unsigned char *tl, int b, int a, const f32x4 &x) {
    f16x4 hv, lv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        hv[r] = (f16)x[r];
        lv[r] = (f16)(x[r] - (float)hv[r]);
    }
    *reinterpret_cast<f16x4 *>(th + PT::off(b, a * 2)) = hv;
    *reinterpret_cast<f16x4 *>(tl + PT::off(b, a * 2)) = lv;
}
// acc += a (bh + bl);  acc += (ah + al)(bh + bl) without lo * lo
__device__ __forceinline__ void mma_h1(f32x4 &acc, const Frag<f16> &a, const Frag<f16> &bh, const Frag<f16> &bl) {
    mma(acc, a, bh);
    mma(acc, a, bl);
}
__device__ __forceinline__ void mma_h2(f32x4 &acc, const Frag<f16> &ah, const Frag<f16> &al, const Frag<f16> &bh,
                                       const Frag<f16> &bl) {
    mma(acc, ah, bh);
    mma(acc, ah, bl);
    mma(acc, al, bh);
}

template <int DK>
__global__ __launch_bounds__(512, 1) void bwd_chunk_kda_mma_kernel(BwdParams p) {
    using L = KaLayout<DK>;
    using KT = typename L::K;
    using ST = typename L::S;
    constexpr int NKB = L::NKB, MD = L::MD, NQT = L::NQT, NW = L::NW;
    __shared__ __attribute__((aligned(16))) unsigned char lds[L::BYTES];
    __shared__ float rdb[64], rdgc[DK], rdpd[64], rtot[512];
    unsigned char *tKg = lds + L::KG0, *tKd = lds + L::KD0, *tA = lds + L::A0, *tP = lds + L::P0;
    unsigned char *tV = lds + L::V0, *tO = lds + L::O0;
    unsigned char *tXh = lds + L::X0, *tXl = tXh + ST::BYTES, *tVh = tXl + ST::BYTES, *tVl = tVh + ST::BYTES;
    unsigned char *tDh = tVl + ST::BYTES, *tDl = tDh + ST::BYTES, *tEh = tDl + ST::BYTES, *tEl = tEh + ST::BYTES;
    const float *g = reinterpret_cast<const float *>(lds + L::G0);

    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ci = blockIdx.x / p.H_v, h = blockIdx.x - ci * p.H_v;
    const int hq = h / (p.H_v / p.H_qk);
    const ChunkInfo cinfo = chunk_info(p.chunks, ci, p.T);
    const int64_t tok0 = cinfo.tok0;
    const int nv = cinfo.nv;
    const int DV = p.D_v, qks = p.H_qk * DK, vs = p.H_v * DV;
    const int64_t unit = (int64_t)ci * p.H_v + h;
    const float *St = p.states + unit * DK * DV;
    const float *dSt = p.dsnext + unit * DK * DV;

    // ---- tiles: padded rows through direct-to-LDS loads (pad granules read zeros)
    auto load = [&]<typename PT>(unsigned char *tile, u32x4 r, int stride) __attribute__((always_inline)) {
        for (int i = w; i < PT::NI; i += NW) {
            const int pos = 64 * i + lane, row = pos / PT::P, gg = pos % PT::P;
            dma_granules(r, tile + 1024 * i, gg < PT::P - 1 ? row * stride + 16 * gg : (1 << 30));
        }
    };
    auto load_half = [&](int hv) __attribute__((always_inline)) {
        const bf16 *vb = static_cast<const bf16 *>(p.v) + tok0 * vs + (int64_t)h * DV + 64 * hv;
        const bf16 *ob = static_cast<const bf16 *>(p.dout) + tok0 * vs + (int64_t)h * DV + 64 * hv;
        load.template operator()<ST>(tV, rsrc_words(vb, ((nv - 1) * vs + 64) * 2), vs * 2);
        load.template operator()<ST>(tO, rsrc_words(ob, ((nv - 1) * vs + 64) * 2), vs * 2);
    };
    {
        load.template operator()<KT>(tKg, rsrc_words(static_cast<const f16 *>(p.kg) + unit * 64 * DK, 64 * DK * 2), DK * 2);
        load.template operator()<KT>(tKd, rsrc_words(static_cast<const f16 *>(p.kd) + unit * 64 * DK, 64 * DK * 2), DK * 2);
        load.template operator()<ST>(tA, rsrc_words(static_cast<const f16 *>(p.A) + unit * 4096, 8192), 128);
        load.template operator()<ST>(tP, rsrc_words(static_cast<const f16 *>(p.P) + unit * 4096, 8192), 128);
        if (w < GB_FLOATS * 4 / 1024)
            dma_granules(rsrc_words(p.gates + unit * GB_FLOATS, GB_FLOATS * 4), lds + L::G0 + 1024 * w, 1024 * w + 16 * lane);
        load_half(0);
    }
    // S and dS_next values of P1 (this lane's value column, D_k rows in pi order), read from memory
    // ahead of the barrier that precedes their use, together with the tile loads
    const int ct = w & 3, tt0 = 2 * (w >> 2);             // token x column tiles of the half
    float ps[NKB][8], pd[NKB][8];
    auto ld_p1 = [&](int hv) __attribute__((always_inline)) {
        const int cg = 64 * hv + 16 * ct + l16;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = 32 * kb + (e < 4 ? 4 * grp + e : 16 + 4 * grp + e - 4);
                ps[kb][e] = St[d * DV + cg];
                pd[kb][e] = dSt[d * DV + cg];
            }
    };
    // S and dS_next values of P4 (rows 16 m + l16, this half's columns in pi order), read at the
    // start of P3
    const int m = w % MD;
    float qs[2][8], qd[2][8];
    auto ld_p4 = [&](int hv) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = 64 * hv + 32 * kb + (e < 4 ? 4 * grp + e : 16 + 4 * grp + e - 4);
                qs[kb][e] = St[(16 * m + l16) * DV + c];
                qd[kb][e] = dSt[(16 * m + l16) * DV + c];
            }
    };
    ld_p1(0);
    if (tid < 64) rdb[tid] = 0.f;
    if (tid < DK) rdgc[tid] = 0.f;
    wait_vm<0>();
    lds_only_barrier();

    auto rows4 = [&](int off, int a) __attribute__((always_inline)) {
        return *reinterpret_cast<const float4 *>(g + off + 16 * a + 4 * grp);
    };

    f32x4 dA[2], dP[2];                                   // 64 x 64 tiles w, w + 8
    f32x4 dqS[NQT], dkD[NQT], dkX[NQT];                   // dq / dk tiles (tt, m)
    dA[0] = dA[1] = dP[0] = dP[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < NQT; ++q) dqS[q] = dkD[q] = dkX[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int qt0 = (w / MD) * NQT;                       // dq / dk tiles: rows 16 m of D_k, tokens

    const int NH = DV / 64;                               // halves of the value columns
    // one half of the value columns; the second half is a separate inlined copy, so that the state
    // values read ahead for its P1 are not carried around a loop
    auto half = [&](int hv) __attribute__((always_inline)) {
        lds_only_barrier();   // the half's V and dO tiles have landed
        const int colg = 64 * hv + 16 * ct + l16;          // this lane's value column
        // ---- P1: Kg S, Kd dS_next, X
        f32x4 ks[2], kd[2];
        {
            Frag<f16> sh[NKB], sl[NKB], dh[NKB], dl[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                split8_h2(ps[kb], sh[kb], sl[kb]);
                split8_h2(pd[kb], dh[kb], dl[kb]);
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int tt = tt0 + q;
                ks[q] = kd[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    mma_h1(ks[q], as_f16(pi_row<KT>(tKg, 16 * tt + l16, kb, grp)), sh[kb], sl[kb]);
                    mma_h1(kd[q], as_f16(pi_row<KT>(tKd, 16 * tt + l16, kb, grp)), dh[kb], dl[kb]);
                }
            }
        }
        float vk[2][4];                                   // V - Kg S
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int tt = tt0 + q;
            const bf16x4 v4 = col4<ST>(tV, tt, ct, grp, l16);
            const float4 be = rows4(GB_BETA, tt);
            const float bev[4] = {be.x, be.y, be.z, be.w};
            f32x4 x;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                vk[q][r] = (float)v4[r] - ks[q][r];
                x[r] = bev[r] * vk[q][r];
            }
            put_t16<ST>(tXh, tXl, 16 * ct + l16, 16 * tt + 4 * grp, x);
        }
        lds_only_barrier();
        // ---- P2: V' = A X, dV' = Kd dS_next + (scale P)^T dO
        {
            Frag<f16> of[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) of[kb] = bf_to_f16(pi_col<ST>(tO, 16 * ct, kb, grp, l16));
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int tt = tt0 + q;
                f32x4 vp = {0.f, 0.f, 0.f, 0.f}, dvp = kd[q];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    if (32 * kb > 16 * tt + 15) continue;         // A[t][s] = 0 for s > t
                    mma_h1(vp, as_f16(pi_row<ST>(tA, 16 * tt + l16, kb, grp)), as_f16(pi_row<ST>(tXh, 16 * ct + l16, kb, grp)),
                           as_f16(pi_row<ST>(tXl, 16 * ct + l16, kb, grp)));
                }
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    if (32 * kb + 31 < 16 * tt) continue;         // P[s][t] = 0 for s < t
                    mma(dvp, as_f16(pi_col<ST>(tP, 16 * tt, kb, grp, l16)), of[kb]);
                }
                put_t16<ST>(tVh, tVl, 16 * ct + l16, 16 * tt + 4 * grp, vp);
                put_t16<ST>(tDh, tDl, 16 * ct + l16, 16 * tt + 4 * grp, dvp);
            }
        }
        lds_only_barrier();
        // ---- P3: dX = A^T dV', dv, the X term of dbeta
        ld_p4(hv);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int tt = tt0 + q;
            f32x4 dx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (32 * kb + 31 < 16 * tt) continue;         // A[s][t] = 0 for s < t
                mma_h1(dx, as_f16(pi_col<ST>(tA, 16 * tt, kb, grp, l16)), as_f16(pi_row<ST>(tDh, 16 * ct + l16, kb, grp)),
                       as_f16(pi_row<ST>(tDl, 16 * ct + l16, kb, grp)));
            }
            const float4 be = rows4(GB_BETA, tt);
            const float bev[4] = {be.x, be.y, be.z, be.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * tt + 4 * grp + r;
                if (t < nv) p.dv[(tok0 + t) * vs + (int64_t)h * DV + colg] = bev[r] * dx[r];
                const float db = sum16(dx[r] * vk[q][r]);
                if (l16 == 0) atomicAdd(&rdb[t], db);
            }
            put_t16<ST>(tEh, tEl, 16 * ct + l16, 16 * tt + 4 * grp, dx);
        }
        lds_only_barrier();
        // ---- P4: the products over this half's columns
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int tix = w + 8 * q, ti = tix >> 2, tj = tix & 3;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                mma_h2(dA[q], as_f16(pi_col<ST>(tDh, 16 * ti, kb, grp, l16)), as_f16(pi_col<ST>(tDl, 16 * ti, kb, grp, l16)),
                       as_f16(pi_col<ST>(tXh, 16 * tj, kb, grp, l16)), as_f16(pi_col<ST>(tXl, 16 * tj, kb, grp, l16)));
                if (tj <= ti)
                    mma_h1(dP[q], bf_to_f16(pi_row<ST>(tO, 16 * ti + l16, kb, grp)), as_f16(pi_col<ST>(tVh, 16 * tj, kb, grp, l16)),
                           as_f16(pi_col<ST>(tVl, 16 * tj, kb, grp, l16)));
            }
        }
        {
            // S and dS_next rows 16 m + l16 over this half's columns, in pi order
            Frag<f16> sh[2], sl[2], dh[2], dl[2];
            float fro = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                split8_h2(qs[kb], sh[kb], sl[kb]);
                split8_h2(qd[kb], dh[kb], dl[kb]);
#pragma unroll
                for (int e = 0; e < 8; ++e) fro += qs[kb][e] * qd[kb][e];
            }
            // e^{G_C} <S, dS_next> of channel 16 m + l16 (each row once: the waves past the D_k
            // rows' owners skip it)
            if (w < MD) {
                fro = sum_groups(fro);
                if (grp == 0) atomicAdd(&rdgc[16 * m + l16], g[GB_DEC + 16 * m + l16] * fro);
            }
#pragma unroll
            for (int q = 0; q < NQT; ++q) {
                const int tt = qt0 + q;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    mma_h1(dqS[q], bf_to_f16(pi_row<ST>(tO, 16 * tt + l16, kb, grp)), sh[kb], sl[kb]);
                    mma_h2(dkD[q], as_f16(pi_col<ST>(tVh, 16 * tt, kb, grp, l16)), as_f16(pi_col<ST>(tVl, 16 * tt, kb, grp, l16)),
                           dh[kb], dl[kb]);
                    mma_h2(dkX[q], as_f16(pi_col<ST>(tEh, 16 * tt, kb, grp, l16)), as_f16(pi_col<ST>(tEl, 16 * tt, kb, grp, l16)),
                           sh[kb], sl[kb]);
                }
            }
        }
    };
    half(0);
    if (NH > 1) {
        lds_only_barrier();   // every wave is done with the first half's tiles
        load_half(1);
        ld_p1(1);
        wait_vm<0>();
        half(1);
    }

    // ---- the tail.  G (every channel's inclusive cumsum down the chunk; rows past the end repeat
    //      the last) goes where the Kg and Kd tiles were, the raw K tile where the V and dO halves
    //      were, the raw Q tile where the dX pair was; dA^T, then dL, use the X pair's place.
    static_assert(64 * (DK + 4) * 4 <= 2 * KT::BYTES, "G fits where the Kg and Kd tiles were");
    static_assert(KT::BYTES <= 2 * ST::BYTES, "K and Q each fit where two 64 x 64 tiles were");
    float *sG = reinterpret_cast<float *>(lds + L::KG0);
    unsigned char *tK = tV, *tQ = tEh;
    constexpr int GP = DK + 4, NPART = 512 / DK, NR = 64 / NPART;
    lds_only_barrier();   // every wave is done with the Kg, Kd, V, dO and dX tiles
    const bf16 *kin = static_cast<const bf16 *>(p.k) + tok0 * qks + (int64_t)hq * DK;
    const bf16 *qin = static_cast<const bf16 *>(p.q) + tok0 * qks + (int64_t)hq * DK;
    load.template operator()<KT>(tK, rsrc_words(kin, ((nv - 1) * qks + DK) * 2), qks * 2);
    load.template operator()<KT>(tQ, rsrc_words(qin, ((nv - 1) * qks + DK) * 2), qks * 2);
    {   // thread (dd, part) scans NR rows of channel dd; every load issued before any is used
        const int dd = tid % DK, part = tid / DK;
        const bf16 *gp = static_cast<const bf16 *>(p.g) + tok0 * p.H_v * DK + (int64_t)h * DK + dd;
        float v[NR];
#pragma unroll
        for (int e = 0; e < NR; ++e) v[e] = (float)gp[(int64_t)min(part * NR + e, nv - 1) * p.H_v * DK];
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < NR; ++e) {
            acc += part * NR + e < nv ? v[e] : 0.f;
            v[e] = acc;
        }
        rtot[part * DK + dd] = acc;
        lds_only_barrier();
        float base = 0.f;
        for (int pp = 0; pp < part; ++pp) base += rtot[pp * DK + dd];
#pragma unroll
        for (int e = 0; e < NR; ++e) sG[(part * NR + e) * GP + dd] = v[e] + base;
        lds_only_barrier();
    }
    wait_vm<0>();      // this wave's K and Q tile loads
    lds_only_barrier();   // both tiles are complete
    const int d = 16 * m + l16;
    const float gC = sG[63 * GP + d];
    auto kq_at = [&](const unsigned char *t, int row) __attribute__((always_inline)) {
        return (float)*reinterpret_cast<const bf16 *>(t + KT::off(row, d * 2));
    };
    // ---- dA transposed and scale dP transposed (strictly lower; its diagonal kept apart)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int tix = w + 8 * q, ti = tix >> 2, tj = tix & 3, j = 16 * tj + l16;
        f32x4 x;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * ti + 4 * grp + r;
            x[r] = j < i ? p.scale * dP[q][r] : 0.f;
            if (j == i) rdpd[i] = p.scale * dP[q][r];
        }
        put_t16<ST>(tXh, tXl, j, 16 * ti + 4 * grp, dA[q]);
        put_t16<ST>(tDh, tDl, j, 16 * ti + 4 * grp, x);
    }
    lds_only_barrier();
    // ---- T = A^T dA, transposed ([t][i]) into the V' buffers
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int tix = w + 8 * q, ti = tix >> 2, tj = tix & 3;
        f32x4 T = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (32 * kb + 31 < 16 * ti) continue;             // A[t][i] = 0 for t < i
            mma_h1(T, as_f16(pi_col<ST>(tA, 16 * ti, kb, grp, l16)), as_f16(pi_row<ST>(tXh, 16 * tj + l16, kb, grp)),
                   as_f16(pi_row<ST>(tXl, 16 * tj + l16, kb, grp)));
        }
        put_t16<ST>(tVh, tVl, 16 * tj + l16, 16 * ti + 4 * grp, T);
    }
    lds_only_barrier();   // every wave is done with dA^T: dL takes its place
    // ---- dL = -T A^T (strictly lower), transposed into the X buffers
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int tix = w + 8 * q, ti = tix >> 2, tj = tix & 3;
        f32x4 dl = {0.f, 0.f, 0.f, 0.f};
        if (tj <= ti) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (32 * kb > 16 * tj + 15) continue;         // A[j][t] = 0 for t > j
                const Frag<f16> af = as_f16(pi_row<ST>(tA, 16 * tj + l16, kb, grp));
                mma(dl, as_f16(pi_col<ST>(tVh, 16 * ti, kb, grp, l16)), af);
                mma(dl, as_f16(pi_col<ST>(tVl, 16 * ti, kb, grp, l16)), af);
            }
        }
        const int j = 16 * tj + l16;
        f32x4 x;
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = j < 16 * ti + 4 * grp + r ? -dl[r] : 0.f;
        put_t16<ST>(tXh, tXl, j, 16 * ti + 4 * grp, x);
    }
    lds_only_barrier();   // dP and dL are complete
    // ---- the P and L terms, block R of rows at a time (the dq / dk tiles of this wave)
    auto dpair = [&](const unsigned char *th, const unsigned char *tl, int row, int col) __attribute__((always_inline)) {
        return (float)*reinterpret_cast<const f16 *>(th + ST::off(row, col * 2)) +
               (float)*reinterpret_cast<const f16 *>(tl + ST::off(row, col * 2));
    };
    unsigned char *tLh = tXh, *tLl = tXl;
    // dG of the chunk, fp32 [64][DK]: columns 0..63 where A and P were, 64..127 where T was (both
    // free now), rows of 68 floats
    static_assert(64 * 68 * 4 <= 2 * ST::BYTES, "a 64-column half of dG fits in two 64 x 64 tiles");
    auto dG_at = [&](int row, int col) __attribute__((always_inline)) {
        return reinterpret_cast<float *>(col < 64 ? tA : tVh) + row * 68 + (col & 63);
    };
    const int hs = p.dq_v == p.dq ? hq : h, hn = p.dq_v == p.dq ? p.H_qk : p.H_v;
    float dgd_sum = 0.f;
#pragma unroll
    for (int q = 0; q < NQT; ++q) {
        const int R = qt0 + q;
        const float4 be = rows4(GB_BETA, R);
        const float bev[4] = {be.x, be.y, be.z, be.w};
        // dq, dk through the states and their terms of dG (rows past the end read zero q and k)
        f32x4 dq, dk, dG;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * R + 4 * grp + r;
            const float G = sG[t * GP + d], eg = __expf(G);
            const float qv = kq_at(tQ, t), kv = kq_at(tK, t);
            const float dq_o = p.scale * eg * dqS[q][r];
            const float dk_x = -bev[r] * eg * dkX[q][r];
            const float dk_d = __expf(gC - G) * dkD[q][r];
            dq[r] = dq_o;
            dk[r] = dk_x + dk_d;
            // the last valid row's factor e^{G_C - G_C} = 1 has no gate gradient: its - (own row) and
            // + (G_C) terms would cancel exactly, so neither is added
            const float dgd = t >= nv - 1 ? 0.f : kv * dk_d;
            dG[r] = qv * dq_o + kv * dk_x - dgd;
            dgd_sum += dgd;
        }
        // the P and L terms of block R of rows
        const float Ga = R > 0 ? sG[(16 * R - 1) * GP + d] : 0.f;    // reference rows 16 R - 1, 16 R + 15
        const float Gb = sG[(16 * R + 15) * GP + d];
        const bool whole = Ga - Gb > kMaxLn;   // the block's decay in this column: split factors would overflow fp16
        f32x4 aq = {0.f, 0.f, 0.f, 0.f}, ar = aq, ap = aq, al = aq;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (32 * kb > 16 * R + 15) continue;              // left sums: t <= 16 R + 15
            const Frag<bf16> kc = pi_col<KT>(tK, 16 * m, kb, grp, l16);
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = 32 * kb + (e < 4 ? 4 * grp + e : 16 + 4 * grp + e - 4);
                const bool in = t <= 16 * R + 15 && !(whole && t >= 16 * R);
                x[e] = in ? (float)kc.v[e] * __expf(Ga - sG[t * GP + d]) : 0.f;
            }
            Frag<f16> bh, bl;
            split8_h2(x, bh, bl);
            mma_h2(aq, as_f16(pi_col<ST>(tDh, 16 * R, kb, grp, l16)), as_f16(pi_col<ST>(tDl, 16 * R, kb, grp, l16)), bh, bl);
            mma_h2(ar, as_f16(pi_col<ST>(tLh, 16 * R, kb, grp, l16)), as_f16(pi_col<ST>(tLl, 16 * R, kb, grp, l16)), bh, bl);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (32 * kb + 31 < 16 * R) continue;              // right sums: t >= 16 R
            const Frag<bf16> qc = pi_col<KT>(tQ, 16 * m, kb, grp, l16), kc = pi_col<KT>(tK, 16 * m, kb, grp, l16);
            const int t0 = 32 * kb + 4 * grp;
            const float4 ba = *reinterpret_cast<const float4 *>(g + GB_BETA + t0);
            const float4 bc = *reinterpret_cast<const float4 *>(g + GB_BETA + t0 + 16);
            const float fb[8] = {ba.x, ba.y, ba.z, ba.w, bc.x, bc.y, bc.z, bc.w};
            float xq[8], xk[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = 32 * kb + (e < 4 ? 4 * grp + e : 16 + 4 * grp + e - 4);
                const bool in = t >= 16 * R && !(whole && t <= 16 * R + 15);
                const float f = in ? __expf(sG[t * GP + d] - Gb) : 0.f;
                xq[e] = (float)qc.v[e] * f;
                xk[e] = fb[e] * (float)kc.v[e] * f;
            }
            Frag<f16> qh, ql, kh, kl;
            split8_h2(xq, qh, ql);
            split8_h2(xk, kh, kl);
            mma_h2(ap, as_f16(pi_row<ST>(tDh, 16 * R + l16, kb, grp)), as_f16(pi_row<ST>(tDl, 16 * R + l16, kb, grp)), qh, ql);
            mma_h2(al, as_f16(pi_row<ST>(tLh, 16 * R + l16, kb, grp)), as_f16(pi_row<ST>(tLl, 16 * R + l16, kb, grp)), kh, kl);
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int r = 16 * R + 4 * grp + rr;
            const float Gr = sG[r * GP + d];
            float vq = aq[rr] * __expf(Gr - Ga), vr = ar[rr] * __expf(Gr - Ga);
            float vp = ap[rr] * __expf(Gb - Gr), vl = al[rr] * __expf(Gb - Gr);
            if (whole) {   // block R's pairs of this column with their whole factors (each at most 1)
                for (int t = 16 * R; t < r; ++t) {
                    const float f = __expf(Gr - sG[t * GP + d]), kt = kq_at(tK, t) * f;
                    vq += dpair(tDh, tDl, t, r) * kt;             // dP[r][t] (tile [t][r])
                    vr += dpair(tLh, tLl, t, r) * kt;
                }
                for (int t = r + 1; t <= 16 * R + 15; ++t) {
                    const float f = __expf(sG[t * GP + d] - Gr);
                    vp += dpair(tDh, tDl, r, t) * kq_at(tQ, t) * f;   // dP[t][r] (tile [r][t])
                    vl += dpair(tLh, tLl, r, t) * g[GB_BETA + t] * kq_at(tK, t) * f;
                }
            }
            const float kr = kq_at(tK, r), qr = kq_at(tQ, r), dpd = rdpd[r];
            dq[rr] += vq + dpd * kr;
            dk[rr] += vp + dpd * qr + bev[rr] * vr + vl;
            dG[rr] += qr * vq + kr * bev[rr] * vr - kr * (vp + vl);
            const float db = sum16(kr * vr);
            if (l16 == 0) atomicAdd(&rdb[r], db);
            if (r < nv) {
                const int64_t o = ((tok0 + r) * hn + hs) * DK + d;
                p.dq_v[o] = dq[rr];
                p.dk_v[o] = dk[rr];
            }
            *dG_at(r, d) = r < nv ? dG[rr] : 0.f;
        }
        reg_fence();
    }
    dgd_sum = sum_groups(dgd_sum);
    if (grp == 0) atomicAdd(&rdgc[d], dgd_sum);
    lds_only_barrier();   // dG, rdb and rdgc are complete
    // ---- the last valid row's e^{G_C} terms, then dG's reverse cumsum per channel (the notes'
    //      Step 7) and dbeta
    if (tid < DK && nv > 0) *dG_at(nv - 1, tid) += rdgc[tid];
    if (tid < nv) p.dbeta[(tok0 + tid) * p.H_v + h] = rdb[tid];
    lds_only_barrier();
    {
        const int dd = tid % DK, part = tid / DK;
        float v[NR];
        float acc = 0.f;
#pragma unroll
        for (int e = NR - 1; e >= 0; --e) {
            acc += *dG_at(part * NR + e, dd);
            v[e] = acc;
        }
        rtot[part * DK + dd] = acc;
        lds_only_barrier();
        float later = 0.f;
        for (int pp = part + 1; pp < NPART; ++pp) later += rtot[pp * DK + dd];
#pragma unroll
        for (int e = 0; e < NR; ++e) {
            const int t = part * NR + e;
            if (t < nv) p.dg[((tok0 + t) * p.H_v + h) * DK + dd] = v[e] + later;
        }
    }
}

}  // namespace

hipError_t launch_bwd_chunk_kda_mma(int D_k, const BwdParams &p, hipStream_t s) {
    const int64_t chunks = (int64_t)p.n_chunks * p.H_v;
    if (chunks == 0) return hipSuccess;
    if (p.D_v != 64 && p.D_v != 128) return hipErrorInvalidValue;
    if (D_k == 128) hipLaunchKernelGGL((bwd_chunk_kda_mma_kernel<128>), dim3((unsigned)chunks), dim3(512), 0, s, p);
    else if (D_k == 64) hipLaunchKernelGGL((bwd_chunk_kda_mma_kernel<64>), dim3((unsigned)chunks), dim3(512), 0, s, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_bwd_chunk_mma(int D_k, const BwdParams &p, hipStream_t s) {
    const int64_t chunks = (int64_t)p.n_chunks * p.H_v;
    if (chunks == 0) return hipSuccess;
    if (p.D_v != 64 && p.D_v != 128) return hipErrorInvalidValue;
    if (D_k == 128) hipLaunchKernelGGL((bwd_chunk_mma_kernel<128>), dim3((unsigned)chunks), dim3(512), 0, s, p);
    else if (D_k == 64) hipLaunchKernelGGL((bwd_chunk_mma_kernel<64>), dim3((unsigned)chunks), dim3(512), 0, s, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gdn
