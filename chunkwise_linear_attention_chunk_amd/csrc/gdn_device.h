// Device-side building blocks for the gfx950 gated-delta-rule kernels.
//
// Matrix-core tiles are 16x16 with fp32 accumulators.  One "contraction block"
// covers 32 values of the contracted index:
//   bf16: one v_mfma_f32_16x16x32_bf16,
//   fp32: eight v_mfma_f32_16x16x4_f32 (MFMA s takes element s of each lane's 8).
// Operand lanes (lane = 0..63, l16 = lane % 16, grp = lane / 16):
//   A operand: row l16, contraction indices 8*grp .. 8*grp+7 of the block
//   B operand: col l16, contraction indices 8*grp .. 8*grp+7 of the block
// Accumulator: lane holds C[4*grp + r][l16], r = 0..3.
// (Layouts checked on gfx950 with an in-bounds probe.)  Any permutation of the
// contraction index that both operands share gives the same sum; helpers that
// take an operand straight from accumulator registers rely on that.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // raw 16 bytes (a native vector, so
                                                              // selects and copies stay in registers)

constexpr float kLog2e = 1.4426950408889634f;

template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { float v[8]; };

__device__ __forceinline__ void mma(f32x4 &c, const Frag<bf16> &a, const Frag<bf16> &b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4 &c, const Frag<float> &a, const Frag<float> &b) {
#pragma unroll
    for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], c, 0, 0, 0);
}

// 8 consecutive elements at p (16-byte aligned for bf16, 32-byte for fp32).
__device__ __forceinline__ Frag<bf16> ld8(const bf16 *p) {
    Frag<bf16> f;
    f.v = *reinterpret_cast<const bf16x8 *>(p);
    return f;
}
__device__ __forceinline__ Frag<float> ld8(const float *p) {
    Frag<float> f;
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

// Store 4 consecutive values (one accumulator column run) at p.
__device__ __forceinline__ void st4(bf16 *p, float a, float b, float c, float d) {
    bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
    *reinterpret_cast<bf16x4 *>(p) = v;
}
__device__ __forceinline__ void st4(float *p, float a, float b, float c, float d) {
    *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
}

// Precision policy of matrix-core operands that are not exact inputs.  bf16 operands are carried
// as a pair x = hi + lo (hi = bf16(x), lo = bf16(x - hi)): a product with an exact bf16 operand
// takes two MFMAs, a product of two such pairs three (lo * lo dropped), for ~16 mantissa bits.
// fp32 operands need no split.
template <typename T> struct Split { static constexpr int parts = 1; };
template <> struct Split<bf16> { static constexpr int parts = 2; };

__device__ __forceinline__ void st4_split(bf16 *hi, bf16 *lo, const f32x4 &x) {
    const bf16x4 h = {(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
    const bf16x4 l = {(bf16)(x[0] - (float)h[0]), (bf16)(x[1] - (float)h[1]), (bf16)(x[2] - (float)h[2]),
                      (bf16)(x[3] - (float)h[3])};
    *reinterpret_cast<bf16x4 *>(hi) = h;
    *reinterpret_cast<bf16x4 *>(lo) = l;
}
__device__ __forceinline__ void st4_split(float *hi, float *, const f32x4 &x) {
    *reinterpret_cast<float4 *>(hi) = make_float4(x[0], x[1], x[2], x[3]);
}

__device__ __forceinline__ void set_elem(Frag<bf16> &f, int e, bf16 x) { f.v[e] = x; }
__device__ __forceinline__ void set_elem(Frag<float> &f, int e, float x) { f.v[e] = x; }

// 16-byte vector of T: 8 bf16 or 4 fp32.
template <typename T> struct Vec16 { static constexpr int N = 16 / sizeof(T); };

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_inclusive_scan(float x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

// fp32 16x16x16 product on the matrix cores, both operands read from LDS with
// natural contraction order: C += A[16 x 16] * B[16 x 16] (MFMA s takes k = 4s + grp).
__device__ __forceinline__ void mm16_f32_lds(f32x4 &c, const float *A, int lda, const float *B, int ldb) {
    const int lane = threadIdx.x & 63, l16 = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(A[l16 * lda + 4 * s + grp], B[(4 * s + grp) * ldb + l16], c, 0, 0,
                                                 0);
}
// Same product with B taken from accumulator registers Bc (B[4*grp + r][l16] in lane):
// MFMA r takes contraction index k = 4*grp + r from both operands.
__device__ __forceinline__ void mm16_f32_regB(f32x4 &c, const float *A, int lda, const f32x4 &Bc) {
    const int lane = threadIdx.x & 63, l16 = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(A[l16 * lda + 4 * grp + r], Bc[r], c, 0, 0, 0);
}

}  // namespace gdn
