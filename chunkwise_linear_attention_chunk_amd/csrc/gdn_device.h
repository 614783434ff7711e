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
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // raw 16 bytes (a native vector, so
                                                              // selects and copies stay in registers)
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));  // raw 8 bytes

constexpr float kLog2e = 1.4426950408889634f;

template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<f16> { f16x8 v; };
template <> struct Frag<float> { float v[8]; };

__device__ __forceinline__ void mma(f32x4 &c, const Frag<bf16> &a, const Frag<bf16> &b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4 &c, const Frag<f16> &a, const Frag<f16> &b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, c, 0, 0, 0);
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
template <> __device__ __forceinline__ f16 from_f32<f16>(float x) { return (f16)x; }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(f16 x) { return (float)x; }

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
// fp16 operands (11 significant bits, rounded to nearest) and fp32 operands need no split.
template <typename T> struct Split { static constexpr int parts = 1; };
template <typename T> inline constexpr bool is_f16 = false;
template <> inline constexpr bool is_f16<f16> = true;
// Element type of the per-channel-gate operands the per-chunk kernel stores (gated K and Q tiles,
// P, the inverse A): fp16 for bf16 inputs, fp32 for fp32 inputs.
template <typename T> struct KdaOperand { using type = T; };
template <> struct KdaOperand<bf16> { using type = f16; };
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
__device__ __forceinline__ void set_elem(Frag<f16> &f, int e, f16 x) { f.v[e] = x; }
__device__ __forceinline__ void set_elem(Frag<float> &f, int e, float x) { f.v[e] = x; }

// ---- operands taken from accumulator registers ----------------------------------------------
// A 32-wide contraction block made of two 16-row accumulator tiles C0 (rows 0..15) and C1
// (rows 16..31) is, lane for lane, an operand fragment whose lane group grp holds contraction
// indices {4grp..4grp+3} from C0 and {16+4grp..16+4grp+3} from C1 ("pi order").  The partner
// operand is read from memory in the same pi order with ld_pi.

// 2^x on the hardware transcendental unit (results below 2^-126 flush to zero, which the
// decays here tolerate: such a factor multiplies a contribution that is already negligible).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x -> hi (+ lo) fragments; fp32 keeps the value whole.  hi is x truncated to bf16 (its upper 16
// bits), lo = bf16(x - hi) carries the next 8+ bits; together ~16 significant bits.
__device__ __forceinline__ void split8(const float *x, Frag<bf16> &h, Frag<bf16> &l) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t bits = __float_as_uint(x[e]) & 0xffff0000u;
        h.v[e] = __builtin_bit_cast(bf16, (unsigned short)(bits >> 16));
        l.v[e] = (bf16)(x[e] - __uint_as_float(bits));
    }
}
// fp16: one rounding to nearest (v_cvt_pk_f16_f32 per two values), no lo part
__device__ __forceinline__ void split8(const float *x, Frag<f16> &h, Frag<f16> &) {
    typedef float f32x8 __attribute__((ext_vector_type(8)));
    h.v = __builtin_convertvector(f32x8{x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]}, f16x8);
}
__device__ __forceinline__ void split8(const float *x, Frag<float> &h, Frag<float> &) {
#pragma unroll
    for (int e = 0; e < 8; ++e) h.v[e] = x[e];
}
// Pack two accumulator tiles into the 8 pi-order values of this lane.
__device__ __forceinline__ void pack_pi(const f32x4 &c0, const f32x4 &c1, float *x) {
    x[0] = c0[0]; x[1] = c0[1]; x[2] = c0[2]; x[3] = c0[3];
    x[4] = c1[0]; x[5] = c1[1]; x[6] = c1[2]; x[7] = c1[3];
}

// Row operand in pi order: elements [32kb + 4grp, +4) and [32kb + 16 + 4grp, +4) of `row`.
__device__ __forceinline__ Frag<bf16> ld_pi(const bf16 *row, int kb) {
    const int grp = (threadIdx.x & 63) >> 4;
    const bf16x4 a = *reinterpret_cast<const bf16x4 *>(row + 32 * kb + 4 * grp);
    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(row + 32 * kb + 16 + 4 * grp);
    Frag<bf16> f;
    f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return f;
}
__device__ __forceinline__ Frag<float> ld_pi(const float *row, int kb) {
    const int grp = (threadIdx.x & 63) >> 4;
    const float4 a = *reinterpret_cast<const float4 *>(row + 32 * kb + 4 * grp);
    const float4 b = *reinterpret_cast<const float4 *>(row + 32 * kb + 16 + 4 * grp);
    Frag<float> f;
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
}
// Column operand in pi order from a row-major tile: M[32kb + 4grp + r][col] and M[32kb+16+4grp+r][col].
template <typename T>
__device__ __forceinline__ Frag<T> ld_pi_col(const T *m, int ld, int col, int kb) {
    const int grp = (threadIdx.x & 63) >> 4;
    Frag<T> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int t = 32 * kb + (e < 4 ? 4 * grp + e : 16 + 4 * grp + e - 4);
        set_elem(f, e, m[t * ld + col]);
    }
    return f;
}

// acc += a * (bh + bl)            (one exact operand, one hi/lo pair)
template <typename T>
__device__ __forceinline__ void mma_x(f32x4 &acc, const Frag<T> &a, const Frag<T> &bh, const Frag<T> &bl) {
    mma(acc, a, bh);
    if constexpr (Split<T>::parts == 2) mma(acc, a, bl);
}
// acc += (ah + al) * b            (a hi/lo pair, then an exact operand)
template <typename T>
__device__ __forceinline__ void mma_pair_x(f32x4 &acc, const Frag<T> &ah, const Frag<T> &al, const Frag<T> &b) {
    mma(acc, ah, b);
    if constexpr (Split<T>::parts == 2) mma(acc, al, b);
}
// acc += (ah + al) * (bh + bl)    (lo * lo dropped)
template <typename T>
__device__ __forceinline__ void mma_xx(f32x4 &acc, const Frag<T> &ah, const Frag<T> &al, const Frag<T> &bh,
                                       const Frag<T> &bl) {
    mma(acc, ah, bh);
    if constexpr (Split<T>::parts == 2) {
        mma(acc, ah, bl);
        mma(acc, al, bh);
    }
}

// ---- tiles loaded straight into LDS ----------------------------------------------------------
// A tile of R rows of RB bytes is stored as 16-byte granules.  Granule (row, cv) sits at position
// row * GPR + (cv ^ swz(row)) (GPR = RB / 16 granules per row).  The XOR spreads the 16 rows an
// MFMA operand read touches over all 16 four-bank groups, so 16-byte row reads are conflict free.
template <int GPR>
__device__ __forceinline__ int tile_swz(int row) {
    constexpr int DIV = GPR >= 16 ? 1 : 16 / GPR;
    constexpr int MOD = GPR >= 16 ? 16 : GPR;
    return (row / DIV) % MOD;
}
// Byte offset of element `col` of row `row` (elements of ESZ bytes).
template <int GPR, int ESZ>
__device__ __forceinline__ int tile_off(int row, int col) {
    const int g = (col * ESZ) >> 4, within = (col * ESZ) & 15;
    return (row * GPR + (g ^ tile_swz<GPR>(row))) * 16 + within;
}
typedef __attribute__((address_space(3))) void lds_void;
// One wave instruction moves 64 granules of global memory into LDS positions lds + 16 * lane.
__device__ __forceinline__ void load_granule_to_lds(const void *src, void *lds_base) {
    __builtin_amdgcn_global_load_lds(src, (lds_void *)lds_base, 16, 0, 0);
}
// One wave instruction moves 64 granules into LDS positions lds + 16 * lane, lane l reading the
// buffer at byte voff + soff; lanes out of the resource's range write zeros.  (Layout and zero
// fill checked on gfx950 with an in-bounds probe.)
__device__ __forceinline__ void buffer_granule_to_lds(__amdgpu_buffer_rsrc_t r, void *lds_base, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_base, 16, voff, soff, 0, 0);
}
// Raw buffer resource over [base, base + bytes): out-of-range accesses are dropped (stores) or
// read as zero (loads).  Word 3 is the gfx9 default descriptor format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// Workgroup barrier that waits only for this wave's LDS operations (lgkmcnt), not for its
// direct-to-LDS loads in flight into the other tile buffer: a fence would have to wait for those,
// since they are LDS writes too.  The memory clobber keeps the compiler from moving memory
// accesses across it.  Only for LDS data produced by ds_* instructions.
__device__ __forceinline__ void lds_only_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Transposed LDS read (ds_read_b64_tr_b16): within each group of 16 lanes, lane j = 4e + q points at
// 4 consecutive 16-bit elements M[t_e][d_q .. d_q + 3]; lane i = 4q + s then receives
// M[t_0 .. t_3][d_q + s].  (Checked on gfx950 with an in-bounds probe.)
__device__ __forceinline__ bf16x4 lds_read_tr16(const void *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4 *)(p));
}

// pi-order operand of a swizzled tile row: elements [32kb + 4grp, +4) and [32kb + 16 + 4grp, +4).
template <typename T, int GPR>
__device__ __forceinline__ Frag<T> ldpi_tile(const unsigned char *tile, int row, int kb) {
    const int grp = (threadIdx.x & 63) >> 4;
    const int c0 = 32 * kb + 4 * grp, c1 = c0 + 16;
    Frag<T> f;
    if constexpr (sizeof(T) == 2 && !is_f16<T>) {
        const bf16x4 a = *reinterpret_cast<const bf16x4 *>(tile + tile_off<GPR, 2>(row, c0));
        const bf16x4 b = *reinterpret_cast<const bf16x4 *>(tile + tile_off<GPR, 2>(row, c1));
        f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else if constexpr (is_f16<T>) {
        const f16x4 a = *reinterpret_cast<const f16x4 *>(tile + tile_off<GPR, 2>(row, c0));
        const f16x4 b = *reinterpret_cast<const f16x4 *>(tile + tile_off<GPR, 2>(row, c1));
        f.v = f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else {
        const float4 a = *reinterpret_cast<const float4 *>(tile + tile_off<GPR, 4>(row, c0));
        const float4 b = *reinterpret_cast<const float4 *>(tile + tile_off<GPR, 4>(row, c1));
        f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
        f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    }
    return f;
}
// pi-order column operand of a K-shaped tile (the K^T operand of the state update): row d, tokens
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
        // (the transpose moves 16-bit lanes: fp16 tiles come back bit for bit)
        f.v = __builtin_bit_cast(decltype(f.v), bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]});
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = 32 * kb + (e < 4 ? 4 * grp + e : 16 + 4 * grp + e - 4);
            f.v[e] = *reinterpret_cast<const float *>(tile + tile_off<GPR, 4>(t, d0 + j));
        }
    }
    return f;
}
// ---- packed operand pairs ---------------------------------------------------------------------
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// two values rounded to nearest-even bf16, packed in one dword (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// hi = bf16(x), lo = bf16(x - hi) for two values, each part packed in one dword
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = pk_bf16(a, b);
    lo = pk_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}
// the pair of four values (one accumulator run), two per dword
__device__ __forceinline__ void split4(const f32x4 &x, u32x2 &hi, u32x2 &lo) {
    uint32_t h0, l0, h1, l1;
    split2(x[0], x[1], h0, l0);
    split2(x[2], x[3], h1, l1);
    hi = u32x2{h0, h1};
    lo = u32x2{l0, l1};
}
// the pair of eight values as operand fragments
__device__ __forceinline__ void split8_rne(const float *x, Frag<bf16> &h, Frag<bf16> &l) {
    uint32_t hh[4], ll[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split2(x[2 * e], x[2 * e + 1], hh[e], ll[e]);
    h.v = __builtin_bit_cast(bf16x8, u32x4{hh[0], hh[1], hh[2], hh[3]});
    l.v = __builtin_bit_cast(bf16x8, u32x4{ll[0], ll[1], ll[2], ll[3]});
}

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt in bits [3:0] and [15:14], expcnt and lgkmcnt left at
// their maxima).  A wave's vector memory loads complete in issue order, so this waits for all but
// its N most recently issued.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

// ---- padded LDS tiles and their direct-to-LDS loads --------------------------------------------
// 64 (or ROWS) rows of G granules, row pitch G + 1 granules; loaded with G + 1 instructions of 64
// granules each (the pad granules read zeros)
template <int G, int ROWS = 64>
struct Pad {
    static constexpr int P = G + 1, PB = 16 * P, BYTES = ROWS * PB, NI = ROWS * P / 64;
    __device__ static constexpr int off(int row, int col_bytes) { return row * PB + col_bytes; }
};

// Buffer resource words over [base, base + bytes) (as make_rsrc builds them), for asm operands.
__device__ __forceinline__ u32x4 rsrc_words(const void *base, int bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, (uint32_t)bytes, 0x00020000u};
}
// One wave instruction moving 64 granules into LDS at lds + 16 * lane, lane l reading the buffer at
// byte voff (out of range: zeros), written in asm.  The compiler's wait insertion does not see this
// load, so reads of other LDS buffers are not made to wait for it (with the builtin, the compiler
// cannot tell tile buffers apart and waits for every load in flight before such reads); the kernel
// waits for it itself (wait_vm) before the barrier that publishes the buffer.  M0 carries the LDS
// base; one wait state separates its write from the load that reads it.
__device__ __forceinline__ void dma_granules(u32x4 rsrc, const void *lds, int voff) {
    const uint32_t m0 = (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void *)lds);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(m0), "v"(voff), "s"(rsrc) : "memory", "m0");
}

// pi-order operand of a padded tile row: elements [32kb + 4grp, +4) and [32kb + 16 + 4grp, +4)
template <typename PT>
__device__ __forceinline__ Frag<bf16> pi_row(const unsigned char *tile, int row, int kb, int grp) {
    const unsigned char *p = tile + PT::off(row, (32 * kb + 4 * grp) * 2);
    const bf16x4 a = *reinterpret_cast<const bf16x4 *>(p);
    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(p + 32);
    Frag<bf16> f;
    f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return f;
}
// pi-order column operand of a padded tile: column c0 + l16, rows 32kb + 4grp + r and
// 32kb + 16 + 4grp + r (transposed reads: lane 4e + q of the group points at row 32kb + 4grp + e,
// columns c0 + 4q .. + 3)
template <typename PT>
__device__ __forceinline__ Frag<bf16> pi_col(const unsigned char *tile, int c0, int kb, int grp, int l16) {
    const unsigned char *p = tile + PT::off(32 * kb + 4 * grp + (l16 >> 2), (c0 + 4 * (l16 & 3)) * 2);
    const bf16x4 a = lds_read_tr16(p);
    const bf16x4 b = lds_read_tr16(p + 16 * PT::PB);
    Frag<bf16> f;
    f.v = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return f;
}

// Keeps the compiler from hoisting LDS operand reads of later iterations above this point: hoisted
// all at once they would need more registers than a wave has.
__device__ __forceinline__ void reg_fence() { asm volatile("" ::: "memory"); }

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
