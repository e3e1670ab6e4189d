// Matrix-core helpers shared by the prompt-form kernels: operand types, the
// gfx950 fp16 products, conversions, the LDS transpose load and DPP prefix
// sums.  Internal to libgdn; every function is inlined into its kernel.
#pragma once

#include "gdn_internal.hpp"

namespace gdn {
namespace {

typedef _Float16 f16;
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16;
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// The same product on bf16 operands (fp32's exponent range).
__device__ __forceinline__ f32x4 mfma_bf(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ f16x4 zh4() {
    const f16 z = static_cast<f16>(0.f);
    return f16x4{z, z, z, z};
}
__device__ __forceinline__ f16x8 cat(f16x4 a, f16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f16x4 h4(f32x4 x) { return __builtin_convertvector(x, f16x4); }
__device__ __forceinline__ f32x4 f4(f16x4 x) { return __builtin_convertvector(x, f32x4); }
__device__ __forceinline__ bf16x8 catb(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Split operands.  A product whose operand x is rounded once to fp16 carries
// x's relative rounding error 2^-11; written as hi + lo, with hi = fp16(x) and
// lo = fp16(x - hi), the pair holds x to about 2^-22 (relative to x, for hi
// normal).  A product with one split operand is one K = 32 product of
// [hi lo] with [b; b]; with both split, either (hi + lo) b_hi and hi b_lo
// (the lo * lo term dropped) or, where the [hi lo] operand serves both,
// (hi + lo) b_hi and (hi + lo) b_lo (prod_split).
struct h4x2 {
    f16x4 hi, lo;
};
// -1 in a scalar register that the compiler cannot see through: x + hi * (-1)
// then stays one mixed-precision fused multiply-add per value (v_fma_mixlo_f16
// and v_fma_mixhi_f16 read hi as fp16 straight from its packed register and
// round to fp16 into either half of the lo register), where a visible -1 lets
// the compiler fold it into a convert, a subtract and a second convert.
__device__ __forceinline__ float opaque_minus_one() {
    float m = -1.f;
    asm volatile("" : "+s"(m));
    return m;
}
// x - hi is exact in fp32 (hi is x rounded to the nearest fp16, or x's
// residual is below fp16's subnormal step), so lo is x - hi rounded once.
__device__ __forceinline__ h4x2 split_h4(f32x4 x) {
    const f16x4 hi = h4(x);
    const float m1 = opaque_minus_one();
    f16x4 lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) lo[i] = static_cast<f16>(__builtin_fmaf(static_cast<float>(hi[i]), m1, x[i]));
    return h4x2{hi, lo};
}
// The same split in bf16 (8 significant bits each, about 2^-17 together, with
// fp32's exponent range).
struct b4x2 {
    bf16x4 hi, lo;
};
__device__ __forceinline__ b4x2 split_b4(f32x4 x) {
    const bf16x4 hi = __builtin_convertvector(x, bf16x4);
    return b4x2{hi, __builtin_convertvector(x - __builtin_convertvector(hi, f32x4), bf16x4)};
}

// c + x y with both operands split: (x_hi + x_lo) y_hi and (x_hi + x_lo) y_lo,
// two K = 32 products sharing the [hi lo] operand (the lo * lo term, about
// 2^-22 of the product, comes with them).
__device__ __forceinline__ f32x4 prod_split(h4x2 x, h4x2 y, f32x4 c) {
    const f16x8 xa = cat(x.hi, x.lo);
    return mfma(xa, cat(y.lo, y.lo), mfma(xa, cat(y.hi, y.hi), c));
}

// Exact powers of two as floats, for exponents in [-126, 127].
__device__ __forceinline__ float pow2i(int e) { return __uint_as_float(static_cast<uint32_t>(e + 127) << 23); }
// floor(log2 |x|) of a normal float (its unbiased exponent field); -127 for 0
// and fp32 subnormals.
__device__ __forceinline__ int exponent_of(float x) {
    return static_cast<int>((__float_as_uint(x) >> 23) & 0xffu) - 127;
}
__device__ __forceinline__ f16x4 neg(f16x4 x) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(f16x4, __builtin_bit_cast(u32x2, x) ^ 0x80008000u);
}
__device__ __forceinline__ f16x4 rd4(const f16 *p) { return *reinterpret_cast<const f16x4 *>(p); }
__device__ __forceinline__ f16x8 rd8(const f16 *p) { return *reinterpret_cast<const f16x8 *>(p); }

// Hide a lane index from loop-invariant code motion: values derived from it
// are then recomputed in each period instead of being held in registers across
// the whole chunk loop.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// s_waitcnt operands (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8; a field at its maximum waits for nothing).  The
// vector-memory counter counts stores as well as loads.
constexpr int kVmcnt0 = 0x0f70;     // vmcnt(0)
constexpr int kLgkmcnt0 = 0xc07f;   // lgkmcnt(0)

// The lane's index in its wave, recomputed where it is called (two vector ALU
// instructions; volatile, so it is neither hoisted nor merged with another
// call): a kernel that needs lane-derived indices in every period then keeps
// no register for them across the loop, and never reloads one from scratch.
__device__ __forceinline__ int fresh_lane_id() {
    int x;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
    return x;
}

// Scheduling barrier: the compiler moves no instruction across it, so the
// reads issued above it overlap the products issued below it.
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// LDS transpose load: in each group of 16 lanes, lane L passes the address of
// halves 4(L%4)..+3 of row L/4 of a 4 x 16 block and receives column L of the
// block (its 4 rows in order).
__device__ __forceinline__ f16x4 rd_tr(const f16 *p) {
    typedef __fp16 v4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
    typedef __attribute__((address_space(3))) v4 lds_v4;
    return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_v4 *)(p)));
}

// Eight bf16 (one 16-byte load) to fp16; bf16 values inside the fp16 range are
// exact in fp16.
__device__ __forceinline__ f16x8 bf_to_h8(f32x4 raw) {
    const u32x4 w = __builtin_bit_cast(u32x4, raw);
    f16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[2 * i] = static_cast<f16>(__uint_as_float(w[i] << 16));
        r[2 * i + 1] = static_cast<f16>(__uint_as_float(w[i] & 0xffff0000u));
    }
    return r;
}

// A K = 16 product (one 16 x 16 tile, four k per lane group: lane l holds
// A[l % 16][4 (l / 16) ..+3] and B[4 (l / 16) ..+3][l % 16]; the result lane
// holds rows 4 (l / 16) ..+3 of column l % 16), issued as the K = 32 product
// with zero upper halves.  The gfx950 compiler does not keep VALU writes far
// enough behind the legacy 16x16x16 f16 instruction's read of its
// accumulator (a result came out with half of each lane's values taken from
// registers rewritten after the issue), so that instruction is not used.
__device__ __forceinline__ f32x4 mfma16(f16x4 a, f16x4 b, f32x4 c) {
    return mfma(cat(a, zh4()), cat(b, zh4()), c);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts
// within each row of 16 lanes, then the last lane of row 0 (of rows 0..1) is
// added to rows 1 and 3 (rows 2 and 3).  Lanes a shift leaves without a source
// add zero.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
    const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, true);
    return v + __builtin_bit_cast(float, t);
}
__device__ __forceinline__ float wave_prefix_sum(float x) {
    x = dpp_add<0x111, 0xf>(x);   // row_shr:1
    x = dpp_add<0x112, 0xf>(x);   // row_shr:2
    x = dpp_add<0x114, 0xf>(x);   // row_shr:4
    x = dpp_add<0x118, 0xf>(x);   // row_shr:8
    x = dpp_add<0x142, 0xa>(x);   // row_bcast:15 into rows 1, 3
    x = dpp_add<0x143, 0xc>(x);   // row_bcast:31 into rows 2, 3
    return x;
}
// The maxima below take IEEE maximum (a NaN operand gives NaN) rather than
// maxNum: maxNum must first quiet each operand that a product may have left
// signalling, one extra instruction per value, where maximum maps to gfx950's
// three-operand v_maximum3_f32 with |.| folded into its operand modifiers.
__device__ __forceinline__ float fmax_ieee(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Maximum of a non-negative value over the 64 lanes of a wave (DPP moves as in
// wave_prefix_sum, lanes without a source contributing 0), returned to every
// lane.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max(float v) {
    const int t = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, true);
    return fmax_ieee(v, __builtin_bit_cast(float, t));
}
__device__ __forceinline__ float wave_max_nonneg(float x) {
    x = dpp_max<0x111, 0xf>(x);   // row_shr:1
    x = dpp_max<0x112, 0xf>(x);   // row_shr:2
    x = dpp_max<0x114, 0xf>(x);   // row_shr:4
    x = dpp_max<0x118, 0xf>(x);   // row_shr:8
    x = dpp_max<0x142, 0xa>(x);   // row_bcast:15 into rows 1, 3
    x = dpp_max<0x143, 0xc>(x);   // row_bcast:31 into rows 2, 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
// Largest |x| of a lane's tile values.
__device__ __forceinline__ float absmax4(f32x4 x, float m) {
    return fmax_ieee(fmax_ieee(fmax_ieee(__builtin_fabsf(x[0]), __builtin_fabsf(x[1])), m),
                     fmax_ieee(__builtin_fabsf(x[2]), __builtin_fabsf(x[3])));
}

// Bound on the scale exponents, so that a change of scale is one exact
// multiplication by a normal power of two.
constexpr int kMaxScaleExp = 62;

// Power-of-two scale of a wave's value-side quantities (the state columns it
// owns and everything linear in them), chosen so that the largest of them
// lands in [8, 16): fp16 operands then keep their full relative precision
// (11 bits for a single rounding, 22 for a split pair) relative to that
// largest value, whatever the magnitude of the values and states the caller
// passes.  `mscaled` is the largest |x| already held at the current scale
// 2^cur, `mtrue` the largest |x| of unscaled ones; returns the new exponent
// (unchanged when both are zero).
__device__ __forceinline__ int choose_scale(float mscaled, int cur, float mtrue) {
    int e = -1000;
    if (mscaled > 0.f) e = exponent_of(mscaled) - cur;
    if (mtrue > 0.f) e = max(e, exponent_of(mtrue));
    if (e == -1000) return cur;
    return min(max(3 - e, -kMaxScaleExp), kMaxScaleExp);
}

// Lower bound on each token's log-decay g before the in-chunk prefix sums.
// exp(-64) ~ 1.6e-28 is below anything an fp32 result resolves, so the bound
// changes no result, while it keeps the prefix sums of a chunk small (|G| <=
// 64 per token): the decay factor between two tokens is exp of a difference
// of prefix sums, and after a token that clears the state (g of -1e4, say)
// unbounded sums would carry that difference with an error of ~1e-3.
constexpr float kMinLogDecay = -64.f;
__device__ __forceinline__ float bounded_log_decay(float g) { return __builtin_fmaxf(g, kMinLogDecay); }
// log2(e) x, rounded once and kept out of any later fused multiply-add, so
// that exp2(G_last - G_t) is exactly 1 for the last row.
__device__ __forceinline__ float log2e_times(float x) { return __fmul_rn(x, 1.4426950408889634f); }

// Inclusive prefix sum within each row of 16 lanes.
__device__ __forceinline__ float row16_prefix_sum(float x) {
    x = dpp_add<0x111, 0xf>(x);   // row_shr:1
    x = dpp_add<0x112, 0xf>(x);   // row_shr:2
    x = dpp_add<0x114, 0xf>(x);   // row_shr:4
    x = dpp_add<0x118, 0xf>(x);   // row_shr:8
    return x;
}

}  // namespace
}  // namespace gdn
