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
};

// ---- wavefront (64-lane) reductions ----------------------------------------
// Butterfly exchanges: every lane ends with the same value because each step
// combines the same pair of operands (addition and max are commutative).
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float max_nonneg(float a, float b) { return a > b ? a : b; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max_nonneg(v, __shfl_xor(v, o, 64));
    return v;
}

// Lane l exchanges with lane l^1 (DPP quad_perm [1,0,3,2]).
__device__ __forceinline__ float swap_adjacent_lanes(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
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
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
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

// E4M3 code of one non-negative scale value (clamped to 448, RNE).
__device__ __forceinline__ uint32_t e4m3fn_scale_code(float v) {
    v = fminf(v, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xFFu;
}

// Exact value of an e4m3fn code (v_cvt_f32_fp8).
__device__ __forceinline__ float e4m3fn_decode(uint32_t code) {
    return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

// FP4 E2M1: eight values -> eight nibbles, value 2k in the low nibble of byte
// k.  Clamped to +-6, then v_cvt_scalef32_pk_fp4_f32 with scale 1.0 rounds to
// nearest even.
__device__ __forceinline__ uint32_t e2m1_x8(const float* q) {
    float c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = __builtin_amdgcn_fmed3f(q[i], -6.0f, 6.0f);
    uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, c[0], c[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, c[2], c[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, c[4], c[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, c[6], c[7], 1.0f, 3);
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

}  // namespace rmsq
