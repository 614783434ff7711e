// Kernel (a): per (chunk, value head) -- chunk-local gate cumsum, gated beta*K K^T on the
// matrix cores, and the exact inverse A = (I + strictLower(diag(beta)(Gamma (.) K K^T)))^{-1}.
//
// Sources: 06 . Flash Linear Attention, section 3 (chunk-local cumsum of log-gates, exp2 of
// pre-scaled differences) and section 4 (solve_tril: forward substitution inside 16x16
// diagonal blocks, row i absorbing the rows above it, then the exact block-triangular merge
// inv([[I+A00, 0], [A10, I+A11]]) = [[A00i, 0], [-A11i A10 A00i, A11i]] from 16 to 32 to 64);
// FlashQLA announcement (Qwen), the first step of the chunk-i forward.
//
// The inverse is computed in fp32 throughout (the pages use tf32 dots for the merges; gfx950
// has no tf32 path, so the merges run on fp32 MFMA).  A is stored in the input dtype.
//
// One workgroup of 256 threads (4 waves) per (chunk, head); many workgroups per CU hide the
// latency of the serial 16-step substitutions.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

template <typename T, int DK>
__global__ __launch_bounds__(256) void intra_kernel(IntraParams p) {
    constexpr int VEC = Vec16<T>::N;
    constexpr int KP = DK + VEC;   // row stride of the K tile (padded against bank conflicts)
    constexpr int LP = 64 + 4;     // row stride of the fp32 64x64 tiles
    constexpr int K_BYTES = 64 * KP * (int)sizeof(T);
    constexpr int X_BYTES = 64 * LP * 4;
    constexpr int R0 = K_BYTES > X_BYTES ? K_BYTES : X_BYTES;
    // region 0 holds the K tile, later (after K K^T) the inverse; region 1 holds A_raw.
    __shared__ __attribute__((aligned(16))) unsigned char smem[R0 + X_BYTES];
    __shared__ float sGl[64], sB[64];
    T *sK = reinterpret_cast<T *>(smem);
    float *sX = reinterpret_cast<float *>(smem);
    float *sL = reinterpret_cast<float *>(smem + R0);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, grp = lane >> 4;
    const int ci = blockIdx.x / p.H_v, h = blockIdx.x - ci * p.H_v;
    const int hq = h / (p.H_v / p.H_qk);
    const ChunkInfo cinfo = chunk_info(p.chunks, ci, p.T);
    const int t0 = cinfo.tok0, nv = cinfo.nv;
    const T *k = static_cast<const T *>(p.k);
    const float *g = static_cast<const float *>(p.g);
    const T *beta = static_cast<const T *>(p.beta);

    // ---- chunk-local inclusive cumsum of the log-gate (log2 units) and beta; tail rows are 0
    // Loads are unconditional from rows clamped into the chunk (always in bounds); the tail is
    // masked afterwards, so the loads are not serialised behind branches.
    const int last = max(nv - 1, 0);
    constexpr int VPR = DK / VEC;
    constexpr int NV = 64 * VPR / 256;
    u32x4 kv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int idx = tid + 256 * i, row = min(idx / VPR, last), cv = idx % VPR;
        kv[i] = *reinterpret_cast<const u32x4 *>(k + ((int64_t)(t0 + row) * p.H_qk + hq) * DK + cv * VEC);
    }
    if (wave == 0) {
        const int64_t idx = (int64_t)(t0 + min(lane, last)) * p.H_v + h;
        const float gv = lane < nv ? g[idx] : 0.f;
        const float bv = lane < nv ? to_f32(beta[idx]) : 0.f;
        sGl[lane] = wave_inclusive_scan(gv) * kLog2e;
        sB[lane] = bv;
    }
    // ---- K tile [64][DK] (rows past the chunk end are zero)
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int idx = tid + 256 * i, row = idx / VPR, cv = idx % VPR;
        *reinterpret_cast<u32x4 *>(sK + row * KP + cv * VEC) = row < nv ? kv[i] : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();

    // ---- A_raw = strictLower(diag(beta) (Gamma (.) K K^T)): the 10 lower 16x16 tiles
    for (int t = wave; t < 10; t += 4) {
        const int ti = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
        const int tj = t - ti * (ti + 1) / 2;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb)
            mma(acc, ld8(sK + (16 * ti + l16) * KP + 32 * kb + 8 * grp), ld8(sK + (16 * tj + l16) * KP + 32 * kb + 8 * grp));
        const int j = 16 * tj + l16;
        const float glj = sGl[j];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * ti + 4 * grp + r;
            sL[i * LP + j] = (j < i) ? sB[i] * exp2f(sGl[i] - glj) * acc[r] : 0.f;
        }
    }
    __syncthreads();

    // ---- inverses of the four 16x16 diagonal blocks: lane c owns column c, row i absorbs rows < i
    {
        const float *L = sL + (16 * wave) * LP + 16 * wave;
        const int c = l16;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s = (i == c) ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < i; ++j) s -= L[i * LP + j] * x[j];
            x[i] = s;
        }
        if (grp == 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sX[(16 * wave + i) * LP + 16 * wave + c] = x[i];
        }
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
        // the tiles written here (rows 32..63, cols 0..31) are read by no wave in this step
#pragma unroll
        for (int r = 0; r < 4; ++r) sX[(16 * I + 4 * grp + r) * LP + 16 * J + l16] = -oo[r];
    }
    __syncthreads();

    // ---- store A (unit lower triangular, zero above the diagonal) in the input dtype
    T *A = static_cast<T *>(p.A) + ((int64_t)ci * p.H_v + h) * 4096;
    for (int idx = tid; idx < 64 * 64 / VEC; idx += 256) {
        const int row = idx / (64 / VEC), c0 = (idx - row * (64 / VEC)) * VEC;
        T vals[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const int col = c0 + e;
            vals[e] = from_f32<T>(col < row ? sX[row * LP + col] : (col == row ? 1.f : 0.f));
        }
        *reinterpret_cast<u32x4 *>(A + row * 64 + c0) = *reinterpret_cast<const u32x4 *>(vals);
    }
}

}  // namespace

hipError_t launch_intra(int dtype, int D_k, const IntraParams &p, hipStream_t s) {
    const dim3 grid((unsigned)p.n_chunks * (unsigned)p.H_v), block(256);
    if (p.n_chunks == 0) return hipSuccess;
    if (dtype == 1 && D_k == 128) hipLaunchKernelGGL((intra_kernel<bf16, 128>), grid, block, 0, s, p);
    else if (dtype == 1 && D_k == 64) hipLaunchKernelGGL((intra_kernel<bf16, 64>), grid, block, 0, s, p);
    else if (dtype == 0 && D_k == 128) hipLaunchKernelGGL((intra_kernel<float, 128>), grid, block, 0, s, p);
    else if (dtype == 0 && D_k == 64) hipLaunchKernelGGL((intra_kernel<float, 64>), grid, block, 0, s, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gdn
