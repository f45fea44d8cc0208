// Device helpers for the gfx950 kernels: 16-byte vector element access,
// wavefront reductions and the FP8 / FP4 / 16-bit conversions built on the
// CDNA4 conversion instructions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rmsq {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

struct BF16 {};
struct F16 {};

// ---- streaming global memory access -----------------------------------------
// Activations are read once and outputs written once, so their accesses carry
// the non-temporal hint (they should not displace gamma and other reused lines
// in L2 / Infinity Cache).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_stream(const void* base, int64_t i16) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + i16);
    return make_uint4(v.x, v.y, v.z, v.w);
}
// The same load from base + byte_off where base is the same in every active
// lane of the wavefront: base goes to scalar registers and the lanes add one
// 32-bit offset, so several rows can share a lane's offset register.
__device__ __forceinline__ uint4 load_stream_uniform(const void* base, uint32_t byte_off) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint64_t u = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                       (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(u) + byte_off));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(void* base, int64_t i16, const uint4& v) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(base) + i16);
}
__device__ __forceinline__ void store_stream(void* base, int64_t i8, const uint2& v) {
    const u32x2 w = {v.x, v.y};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(base) + i8);
}
__device__ __forceinline__ void store_stream(void* base, int64_t i4, uint32_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(base) + i4);
}
__device__ __forceinline__ void store_stream(void* base, int64_t i2, uint16_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<uint16_t*>(base) + i2);
}

// ---- one 16-byte vector of input elements --------------------------------
template <typename T>
struct Vec;

template <>
struct Vec<float> {
    static constexpr int EPV = 4;  // elements per 16-byte vector
    static constexpr int BYTES = 4;
    __device__ __forceinline__ static void unpack(const uint4& v, float* f) {
        f[0] = __uint_as_float(v.x);
        f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z);
        f[3] = __uint_as_float(v.w);
    }
    // Round fp32 values to the element type (identity for fp32).
    __device__ __forceinline__ static uint4 pack(const float* f) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                          __float_as_uint(f[3]));
    }
    // Sum of squares of the vector's elements (fp32 fused multiply-adds).
    __device__ __forceinline__ static float sumsq(const uint4& v) {
        float f[4];
        unpack(v, f);
        return fmaf(f[3], f[3], fmaf(f[2], f[2], fmaf(f[1], f[1], f[0] * f[0])));
    }
};

template <>
struct Vec<BF16> {
    static constexpr int EPV = 8;
    static constexpr int BYTES = 2;
    __device__ __forceinline__ static void unpack2(uint32_t w, float* f) {
        f[0] = __uint_as_float(w << 16);
        f[1] = __uint_as_float(w & 0xFFFF0000u);
    }
    __device__ __forceinline__ static void unpack(const uint4& v, float* f) {
        unpack2(v.x, f + 0);
        unpack2(v.y, f + 2);
        unpack2(v.z, f + 4);
        unpack2(v.w, f + 6);
    }
    // v_cvt_pk_bf16_f32: two fp32 -> two bf16, round to nearest even.
    __device__ __forceinline__ static uint32_t pack2(float a, float b) {
        f32x2 p = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
    }
    __device__ __forceinline__ static uint4 pack(const float* f) {
        return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]));
    }
    // Sum of squares straight from the packed pairs: v_dot2c_f32_bf16 (each
    // bf16 square is exact in fp32; accumulation in fp32).
    __device__ __forceinline__ static float sumsq(const uint4& v) {
        float acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.x), __builtin_bit_cast(bf16x2, v.x),
                                                    0.0f, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.y), __builtin_bit_cast(bf16x2, v.y), acc,
                                              false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.z), __builtin_bit_cast(bf16x2, v.z), acc,
                                              false);
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.w), __builtin_bit_cast(bf16x2, v.w), acc,
                                               false);
    }
};

template <>
struct Vec<F16> {
    static constexpr int EPV = 8;
    static constexpr int BYTES = 2;
    __device__ __forceinline__ static void unpack2(uint32_t w, float* f) {
        f32x2 p = __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
        f[0] = p.x;
        f[1] = p.y;
    }
    __device__ __forceinline__ static void unpack(const uint4& v, float* f) {
        unpack2(v.x, f + 0);
        unpack2(v.y, f + 2);
        unpack2(v.z, f + 4);
        unpack2(v.w, f + 6);
    }
    // v_cvt_pk_f16_f32: two fp32 -> two binary16, round to nearest even.
    __device__ __forceinline__ static uint32_t pack2(float a, float b) {
        f32x2 p = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(p, f16x2));
    }
    __device__ __forceinline__ static uint4 pack(const float* f) {
        return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]));
    }
    // Sum of squares from the packed pairs: v_dot2c_f32_f16 (each fp16 square
    // is exact in fp32; accumulation in fp32).
    __device__ __forceinline__ static float sumsq(const uint4& v) {
        float acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, v.x), __builtin_bit_cast(f16x2, v.x), 0.0f, false);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, v.y), __builtin_bit_cast(f16x2, v.y), acc, false);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, v.z), __builtin_bit_cast(f16x2, v.z), acc, false);
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, v.w), __builtin_bit_cast(f16x2, v.w), acc, false);
    }
};

// Largest |t_e| of a vector of fp32 values, folded into m (v_max3_f32 with
// absolute-value source modifiers, two elements per instruction).
template <int N>
__device__ __forceinline__ float abs_max(float m, const float* t) {
#pragma unroll
    for (int e = 0; e < N; ++e) m = fmaxf(m, fabsf(t[e]));
    return m;
}

// ---- per-row scalars in fp64 --------------------------------------------------
// 1/sqrt(m) and 1/d: the hardware estimate (v_rsq_f64 / v_rcp_f64) refined by
// two Newton steps, each of which squares the relative error, so the result
// is within a few fp64 units of the exact value whatever the estimate's
// accuracy.  Computed once per row or block, so fp64 costs nothing measurable.
__device__ __forceinline__ double rsqrt_refined(double m) {
    double r = __builtin_amdgcn_rsq(m);
    r = r * (1.5 - 0.5 * m * r * r);
    return r * (1.5 - 0.5 * m * r * r);
}
__device__ __forceinline__ double rcp_refined(double d) {
    double r = __builtin_amdgcn_rcp(d);
    r = r * (2.0 - d * r);
    return r * (2.0 - d * r);
}

// ---- wavefront (64-lane) reductions ----------------------------------------
// DPP permutations inside each 16-lane row (every lane has a source, so no
// bound control is involved), then the four row results are read out of
// lanes 0, 16, 32 and 48.  Each step combines the same pair of operands in
// every lane it reaches (addition and max are commutative), so all lanes end
// with bit-identical results.
enum : int {
    DPP_SWAP1 = 0xB1,         // quad_perm [1,0,3,2]: lane ^ 1
    DPP_SWAP2 = 0x4E,         // quad_perm [2,3,0,1]: lane ^ 2
    DPP_HALF_MIRROR = 0x141,  // lane i <-> 7 - i within 8 lanes
    DPP_MIRROR = 0x140        // lane i <-> 15 - i within 16 lanes
};

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)dpp_i32<CTRL>((int)(uint32_t)b);
    const uint32_t hi = (uint32_t)dpp_i32<CTRL>((int)(uint32_t)(b >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double wave_sum(double v) {
    v += dpp_f64<DPP_SWAP1>(v);
    v += dpp_f64<DPP_SWAP2>(v);
    v += dpp_f64<DPP_HALF_MIRROR>(v);
    v += dpp_f64<DPP_MIRROR>(v);
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// Max of non-negative floats, taken on their bit patterns: for values >= 0
// the integer order is the floating-point order, and integer max needs no
// NaN canonicalization.
__device__ __forceinline__ int max_bits(int a, int b) { return a > b ? a : b; }

__device__ __forceinline__ float wave_max_nonneg(float v) {
    int b = __float_as_int(v);
    b = max_bits(b, dpp_i32<DPP_SWAP1>(b));
    b = max_bits(b, dpp_i32<DPP_SWAP2>(b));
    b = max_bits(b, dpp_i32<DPP_HALF_MIRROR>(b));
    b = max_bits(b, dpp_i32<DPP_MIRROR>(b));
    const int r = max_bits(max_bits(__builtin_amdgcn_readlane(b, 0), __builtin_amdgcn_readlane(b, 16)),
                           max_bits(__builtin_amdgcn_readlane(b, 32), __builtin_amdgcn_readlane(b, 48)));
    return __int_as_float(r);
}

// max(v, v of lane ^ 1) for non-negative v (the two halves of a 16-element
// FP4 block).
__device__ __forceinline__ float pair_max_nonneg(float v) {
    const int b = __float_as_int(v);
    return __int_as_float(max_bits(b, dpp_i32<DPP_SWAP1>(b)));
}

// max over the lanes 4j .. 4j+3 for non-negative v (the four quarters of a
// 32-element FP4 block of 16-bit inputs).
__device__ __forceinline__ float quad_max_nonneg(float v) {
    int b = __float_as_int(v);
    b = max_bits(b, dpp_i32<DPP_SWAP1>(b));
    b = max_bits(b, dpp_i32<DPP_SWAP2>(b));
    return __int_as_float(b);
}

// max over the lanes 8j .. 8j+7 for non-negative v (a 32-element FP4 block
// of fp32 inputs): the two quads' maxima meet through the 8-lane mirror.
__device__ __forceinline__ float oct_max_nonneg(float v) {
    int b = __float_as_int(quad_max_nonneg(v));
    b = max_bits(b, dpp_i32<DPP_HALF_MIRROR>(b));
    return __int_as_float(b);
}

// max over the LPB lanes that hold one FP4 block.
template <int LPB>
__device__ __forceinline__ float block_max_nonneg(float v) {
    static_assert(LPB == 2 || LPB == 4 || LPB == 8, "a block spans 2, 4 or 8 lanes");
    if constexpr (LPB == 2) return pair_max_nonneg(v);
    else if constexpr (LPB == 4) return quad_max_nonneg(v);
    else return oct_max_nonneg(v);
}

// max over the wave of non-negative doubles, on their bit patterns (the
// integer order of non-negative IEEE doubles is their numeric order).
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)dpp_i32<CTRL>((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)dpp_i32<CTRL>((int)(uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ double wave_max_nonneg(double v) {
    uint64_t b = __builtin_bit_cast(uint64_t, v);
    b = max_u64(b, dpp_u64<DPP_SWAP1>(b));
    b = max_u64(b, dpp_u64<DPP_SWAP2>(b));
    b = max_u64(b, dpp_u64<DPP_HALF_MIRROR>(b));
    b = max_u64(b, dpp_u64<DPP_MIRROR>(b));
    b = max_u64(max_u64(readlane_u64(b, 0), readlane_u64(b, 16)), max_u64(readlane_u64(b, 32), readlane_u64(b, 48)));
    return __builtin_bit_cast(double, b);
}

// ---- conversions ------------------------------------------------------------
// OCP E4M3 (e4m3fn): saturating round-to-nearest-even.  The input is clamped
// to +-448 first so that saturation never depends on the instruction's own
// overflow behaviour; v_cvt_pk_fp8_f32 then rounds to nearest even.
// Byte i of the result holds value i.
__device__ __forceinline__ uint32_t e4m3fn_x4(float a, float b, float c, float d) {
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
    d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
    // the first conversion writes the low half, the second the high half; the
    // initial high half is never used, so a's dead register serves as it
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// E4M3FNUZ (bias 8, max 240, no -0).  Same bit layout as e4m3fn with the
// exponent bias one higher, so for |v| <= 224 its code is the e4m3fn code of
// 2v.  Above that: (224, 232] rounds to 224 (0x7E, even mantissa) and
// (232, ...) to 240 (0x7F), which e4m3fn cannot express (0x7F is its NaN).
// Zero magnitudes lose their sign (0x80 is the fnuz NaN).
__device__ __forceinline__ uint32_t e4m3fnuz_x4(float a, float b, float c, float d) {
    uint32_t w = e4m3fn_x4(2.0f * a, 2.0f * b, 2.0f * c, 2.0f * d);
    uint32_t big = (fabsf(a) > 232.0f ? 0x000000FFu : 0u) | (fabsf(b) > 232.0f ? 0x0000FF00u : 0u) |
                   (fabsf(c) > 232.0f ? 0x00FF0000u : 0u) | (fabsf(d) > 232.0f ? 0xFF000000u : 0u);
    w = (w & ~big) | (big & (0x7F7F7F7Fu | (w & 0x80808080u)));
    uint32_t mag = w & 0x7F7F7F7Fu;
    uint32_t nonzero = (mag + 0x7F7F7F7Fu) & 0x80808080u;  // bit 7 set where mag != 0 (no carries)
    return mag | (w & nonzero);
}

template <bool FNUZ>
__device__ __forceinline__ uint32_t fp8_x4(float a, float b, float c, float d) {
    if constexpr (FNUZ)
        return e4m3fnuz_x4(a, b, c, d);
    else
        return e4m3fn_x4(a, b, c, d);
}

// E4M3 code of one non-negative scale value (clamped to 448, RNE), in the
// low byte of the result; the other bytes are unspecified.
__device__ __forceinline__ uint32_t e4m3fn_scale_code(float v) {
    v = fminf(v, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, __float_as_int(v), false);
}

// UE8M0 block-scale code of a non-negative fp32 value v: the exponent of the
// smallest power of two >= v, plus 127, clamped to [0, 255] (0 for v = 0).
// For a normal v that is the exponent field, plus one when any mantissa bit
// is set: adding 0x7FFFFF to the bits carries into the exponent exactly then
// (and the largest finite value gives 255).  A subnormal v (< 2^-126) has
// code 1 above 2^-127 and 0 at or below it.
__device__ __forceinline__ uint32_t ue8m0_code(float v) {
    const uint32_t b = __float_as_uint(v);
    return b >= 0x00800000u ? (b + 0x007FFFFFu) >> 23 : (b > 0x00400000u ? 1u : 0u);
}

// c * 2^(127 - code), and 0 for code 0: the element factor of a UE8M0 block
// (v_ldexp_f32 scales exactly unless the result leaves the fp32 range).
__device__ __forceinline__ float ue8m0_factor(float c, uint32_t code) {
    return code == 0 ? 0.0f : __builtin_amdgcn_ldexpf(c, 127 - (int)code);
}

// Exact value of the e4m3fn code in the low byte of `code` (v_cvt_f32_fp8).
__device__ __forceinline__ float e4m3fn_decode(uint32_t code) {
    return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

// FP4 E2M1: eight values -> eight nibbles, value 2k in the low nibble of byte
// k.  v_cvt_scalef32_pk_fp4_f32 with scale 1.0 rounds to nearest even and
// saturates to +-6 by itself (checked over the whole fp32 range, infinities
// included, against the reference encoder), so no clamp is needed.
__device__ __forceinline__ uint32_t e2m1_x8(const float* q) {
    // each conversion writes one byte and all four are written, so the
    // initial value is irrelevant: q[0]'s dead register serves as it
    uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(__float_as_uint(q[0]), q[0], q[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[2], q[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[4], q[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[6], q[7], 1.0f, 3);
    return w;
}

// Four values -> four nibbles in the low 16 bits (value 2k in the low nibble
// of byte k); the upper 16 bits are unspecified.
__device__ __forceinline__ uint32_t e2m1_x4(const float* q) {
    uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(__float_as_uint(q[0]), q[0], q[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[2], q[3], 1.0f, 1);
    return w;
}

// Round an fp32 scale to the scales dtype; returns the stored bits in *bits
// and the stored value.
__device__ __forceinline__ float round_scale(float v, int scales_dtype, uint32_t* bits) {
    if (scales_dtype == 2 /* RMSQ_BF16 */) {
        uint32_t w = Vec<BF16>::pack2(v, 0.0f) & 0xFFFFu;
        *bits = w;
        return __uint_as_float(w << 16);
    }
    if (scales_dtype == 1 /* RMSQ_F16 */) {
        uint32_t w = Vec<F16>::pack2(v, 0.0f) & 0xFFFFu;
        *bits = w;
        float f[2];
        Vec<F16>::unpack2(w, f);
        return f[0];
    }
    *bits = __float_as_uint(v);
    return v;
}

__device__ __forceinline__ void store_scale(void* scales, int64_t i, int scales_dtype, uint32_t bits) {
    if (scales_dtype == 0 /* RMSQ_F32 */)
        reinterpret_cast<uint32_t*>(scales)[i] = bits;
    else
        reinterpret_cast<uint16_t*>(scales)[i] = (uint16_t)bits;
}

// ---- FP8 per-row numerics -------------------------------------------------
// The codes follow q = s * (gamma + weight_offset) * rstd / stored_scale
// rounded ONCE to fp32 (the precision the conversion instruction takes), so
// they agree with the exact definition except where q lies within a few
// units of 2^-46 of an fp32 rounding midpoint:
//  * sum of squares: every s^2 is exact in fp64 and accumulated there (the
//    row's rstd then carries ~2^-50 relative error instead of the ~2^-29 of
//    fp32 partial sums, which decided near-ties of the codes);
//  * the factor k = rstd / stored_scale is formed in fp64 and split into two
//    fp32 terms hi + lo (k to ~2^-48);
//  * the product s * g' and its row maximum are exact, formed one of three
//    ways (compile time, chosen by the input type and whether a weight offset
//    is added):
//      kProdF32  16-bit inputs, no offset: s * g has at most 22 significant
//                bits, so t = s * g is exact in fp32; q = t * hi + t * lo
//                (one multiply, one FMA);
//      kProdTwo  fp32 inputs, no offset: s * g = th + tl exactly (th the fp32
//                product, tl its error from an FMA); the row maximum in fp64;
//                q = th * hi + (th * lo + tl * hi) (three FMAs);
//      kProdF64  a weight offset (g + offset is not exact in fp32): s * g'
//                in fp64, q = fp32(s * g' * k).
//    A row whose |q| could exceed 2^100 (a binding scale_ub far below the
//    row's scale, or a row maximum below ~2^-92) takes fp64 for every
//    element: the fp32 terms could overflow.
enum : int { kProdF32 = 0, kProdTwo = 1, kProdF64 = 2 };

template <typename InT>
inline constexpr int prod_mode(float weight_offset) {
    return weight_offset != 0.0f ? kProdF64 : (Vec<InT>::BYTES == 4 ? kProdTwo : kProdF32);
}

// acc + s^2 in fp64 for each of N fp32 values (their squares are exact in
// fp64); two interleaved chains keep the FMAs independent.
template <int N>
__device__ __forceinline__ void sumsq64(double& a0, double& a1, const float* s) {
#pragma unroll
    for (int e = 0; e < N; e += 2) {
        const double d0 = s[e];
        a0 = fma(d0, d0, a0);
        if (e + 1 < N) {
            const double d1 = s[e + 1];
            a1 = fma(d1, d1, a1);
        }
    }
}

// |s * (g + off)| exact in fp64 (off = 0 for kProdTwo)
__device__ __forceinline__ double abs_prod64(float s, float g, double off) {
    return fabs((double)s * ((double)g + off));
}

struct Fp8Row {
    double k;        // rstd / stored scale (0 for a zero scale)
    float hi, lo;    // k = hi + lo to ~2^-48 relative
    bool split;      // the fp32-term forms cannot overflow (else fp64)
    uint32_t sbits;  // the stored scale's bits in the scales dtype
};

// The row's scale min(amax * rstd / FMAX, scale_ub) (fp64), rounded to fp32
// and then to the scales dtype, and the quantization factor for it.  amax is
// max |s * g'| over the row, exact.
__device__ __forceinline__ Fp8Row fp8_row(double amax, double rstd, double inv_fmax, float scale_ub,
                                          int scales_dtype) {
    Fp8Row r;
    double sc = amax * rstd * inv_fmax;
    if (sc > (double)scale_ub) sc = (double)scale_ub;
    const float sc_st = round_scale((float)sc, scales_dtype, &r.sbits);
    r.k = sc_st > 0.0f ? rstd * rcp_refined((double)sc_st) : 0.0;
    // hi = k rounded toward zero, so lo = k - hi >= 0: then every term of
    // the split forms carries the sign of a zero product (an fp32 sum of
    // zeros of opposite signs would be +0, and the code's sign bit -0)
    float hi = (float)r.k;
    if ((double)hi > r.k) hi = __uint_as_float(__float_as_uint(hi) - 1u);
    r.hi = hi;
    r.lo = (float)(r.k - (double)hi);
    // |q| <= amax * k: below 2^100 no fp32 term can overflow; a zero scale
    // (k = 0) takes fp64, where y * 0 keeps the sign of y
    r.split = r.k > 0.0 && r.k < 0x1p100 && amax * r.k < 0x1p100;
    return r;
}

// kProdF32: q = fp32(t * k) for t exact in fp32 (split rows).
__device__ __forceinline__ float fp8_q1(float t, const Fp8Row& r) { return fmaf(t, r.hi, t * r.lo); }

// kProdTwo: q = fp32(s * g * k) for fp32 s and raw gamma g (split rows).  The product's
// error tl = s * g - th (exact) is formed as -(th - s * g) so that it is a
// zero of th's sign when the product is zero.
__device__ __forceinline__ float fp8_q2(float s, float g, const Fp8Row& r) {
    g += 0.0f;  // the definition's g + offset (offset 0 here): a -0 gamma becomes +0
    const float th = s * g;
    const float tl = -fmaf(-s, g, th);
    return fmaf(th, r.hi, fmaf(th, r.lo, tl * r.hi));
}

// kProdF64 (and every row that is not split): q = fp32(s * (g + off) * k).
__device__ __forceinline__ float fp8_q64(float s, float g, double off, const Fp8Row& r) {
    return (float)((double)s * ((double)g + off) * r.k);
}

}  // namespace rmsq
