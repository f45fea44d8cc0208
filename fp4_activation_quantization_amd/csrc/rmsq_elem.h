// Single-element access for the FP8 kernels that work off the 16-byte
// vector grid (rmsq_fp8_elem_kernel.h, rmsq_fp8_phased_kernel.h).
#pragma once

#include "rmsq_device.h"

namespace rmsq {

// One element of the input type: its storage bits, widened to fp32, and an
// fp32 value rounded (to nearest even) back to the type.
template <typename T>
struct Elem;

template <>
struct Elem<float> {
    using Bits = uint32_t;
    __device__ __forceinline__ static float widen(uint32_t b) { return __uint_as_float(b); }
    __device__ __forceinline__ static uint32_t round(float f) { return __float_as_uint(f); }
};

template <>
struct Elem<BF16> {
    using Bits = uint16_t;
    __device__ __forceinline__ static float widen(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
    __device__ __forceinline__ static uint16_t round(float f) { return (uint16_t)Vec<BF16>::pack2(f, 0.0f); }
};

template <>
struct Elem<F16> {
    using Bits = uint16_t;
    __device__ __forceinline__ static float widen(uint16_t b) {
        float f[2];
        Vec<F16>::unpack2(b, f);
        return f[0];
    }
    __device__ __forceinline__ static uint16_t round(float f) { return (uint16_t)Vec<F16>::pack2(f, 0.0f); }
};

template <typename B>
__device__ __forceinline__ B load_elem(const B* p) {
    return __builtin_nontemporal_load(p);
}
template <typename B>
__device__ __forceinline__ void store_elem(B* p, B v) {
    __builtin_nontemporal_store(v, p);
}

}  // namespace rmsq
