// rmsq_fused.hpp -- C++ (HIP) interface of librmsq: RMSNorm + per-row FP8
// quantization of rows that a caller-defined source produces element by
// element as the kernel loads them, the analogue of the input_fn parameter
// of Mojo docs "rms_norm_fused_fp8" (Parameters: input_fn, the function that
// loads input values; epsilon, weight_offset, scale_ub and the per-row scale
// output as in include/rmsq.h's rmsnorm_fp8).
//
// Build: hipcc --offload-arch=gfx950 -std=c++17 with -I <repo>/include and
// -I <repo>/fp4_activation_quantization_amd/csrc (the kernel template is
// compiled into the caller's translation unit); link librmsq.so for
// rmsq_query_shape.  Compile with -Xclang -target-feature -Xclang
// -packed-fp32-ops as the library is.
//
// A source is a copyable struct, passed to the kernel by value, with
//   __device__ uint4 operator()(int64_t row, int v) const;
// returning the 16-byte vector v of row `row` -- elements 8v..8v+7 of a
// 16-bit row, 4v..4v+3 of an fp32 row -- packed as InT (rmsq::BF16,
// rmsq::F16 or float).  The kernel asks for each vector of a row exactly
// once, from the lane that normalizes it, and then treats it exactly as
// rmsnorm_fp8 treats a loaded vector of x: the produced values are the s of
// the operation.  A source must not write anything the same call reads.
#pragma once

#include <cmath>
#include <cstdint>

#include "rmsq.h"
#include "rmsq_fp8_kernel.h"

namespace rmsq {

template <typename InT>
struct InTypeCode;
template <>
struct InTypeCode<float> {
    static constexpr int value = RMSQ_F32;
};
template <>
struct InTypeCode<F16> {
    static constexpr int value = RMSQ_F16;
};
template <>
struct InTypeCode<BF16> {
    static constexpr int value = RMSQ_BF16;
};

// The source behind gated_rmsnorm_fp8 (include/rmsq.h): x = a * b element by
// element (the gate and up projections of a gated MLP, the activation
// applied upstream), computed in fp32 and rounded once to InT (RNE).  The
// fp32 product of two 16-bit values is exact unless it falls below 2^-126 in
// magnitude (bf16 operands only), so the result is the exact product rounded
// once; fp32 operands are rounded once by the multiply itself.
template <typename InT>
struct GatedProduct {
    const char* a;
    const char* b;
    int64_t stride;  // bytes between consecutive rows of a and of b
    __device__ __forceinline__ uint4 operator()(int64_t row, int v) const {
        using V = Vec<InT>;
        float fa[V::EPV], fb[V::EPV];
        V::unpack(load_stream(a + row * stride, v), fa);
        V::unpack(load_stream(b + row * stride, v), fb);
#pragma unroll
        for (int e = 0; e < V::EPV; ++e) fa[e] *= fb[e];
        return V::pack(fa);
    }
};

// RMSNorm + per-row FP8 quantization of `rows` rows of `hidden` elements of
// type InT produced by `src`; outputs as rmsnorm_fp8: out [rows, hidden]
// codes (16-byte aligned, rows adjacent), scales [rows] of scales_dtype.
// hidden must be a multiple of 8 (16-bit) or 4 (fp32) and at most 4096
// vectors; gamma [hidden] of InT, 16-byte aligned; out, scales and gamma
// must not overlap (RMSQ_ERR_ALIAS), nor may what the source reads overlap
// out or scales (not checked).  Returns an RMSQ_* status;
// every check happens before the launch (RMSQ_ERR_LAUNCH after a failed one).
// Enqueues one kernel on `stream`; the launch shape is rmsq_query_shape's
// (path 0), so rmsq_set_tuning applies.
template <typename InT, class Src>
int rmsnorm_fp8_from(const Src& src, int64_t rows, int64_t hidden, const void* gamma, float eps, float weight_offset,
                     float scale_ub, int out_fp8, void* out, int scales_dtype, void* scales, hipStream_t stream) {
    constexpr int epv = Vec<InT>::EPV;
    constexpr int esz = Vec<InT>::BYTES;
    if (out_fp8 != RMSQ_E4M3FN && out_fp8 != RMSQ_E4M3FNUZ) return RMSQ_ERR_DTYPE;
    if (scales_dtype != RMSQ_F32 && scales_dtype != RMSQ_F16 && scales_dtype != RMSQ_BF16) return RMSQ_ERR_DTYPE;
    if (rows < 0 || hidden <= 0 || hidden % epv != 0 || rows > (INT64_MAX / 4) / (hidden * esz))
        return RMSQ_ERR_SHAPE;
    if (!(eps >= 0.0f) || !std::isfinite(eps) || !std::isfinite(weight_offset) || !(scale_ub > 0.0f))
        return RMSQ_ERR_VALUE;
    if (hidden / epv > kMaxVec) return RMSQ_ERR_UNSUPPORTED;
    if (rows == 0) return RMSQ_OK;
    if (!gamma || !out || !scales) return RMSQ_ERR_NULL;
    const int ssz = scales_dtype == RMSQ_F32 ? 4 : 2;
    const uintptr_t o = reinterpret_cast<uintptr_t>(out), sc = reinterpret_cast<uintptr_t>(scales),
                    g = reinterpret_cast<uintptr_t>(gamma);
    if (g % 16 || o % 16 || sc % ssz) return RMSQ_ERR_ALIGN;
    // the outputs overlap neither each other nor gamma (what the source reads
    // is the caller's to keep apart from them)
    const auto overlap = [](uintptr_t a, uintptr_t an, uintptr_t b, uintptr_t bn) { return a < b + bn && b < a + an; };
    const uintptr_t on = (uintptr_t)(rows * hidden), sn = (uintptr_t)(rows * ssz), gn = (uintptr_t)(hidden * esz);
    if (overlap(o, on, sc, sn) || overlap(o, on, g, gn) || overlap(sc, sn, g, gn)) return RMSQ_ERR_ALIAS;
    Shape s{};
    if (int rc = rmsq_query_shape(rows, hidden, InTypeCode<InT>::value, 0, &s.waves, &s.vpt, &s.rpb)) return rc;
    s.grid = 0;
    FusedArgs a{};
    a.gamma = gamma;
    a.out = out;
    a.scales = scales;
    a.rows = rows;
    a.hidden = (int32_t)hidden;
    a.inv_hidden = 1.0 / (double)hidden;
    a.nvec = (int32_t)(hidden / epv);
    a.eps = eps;
    a.weight_offset = weight_offset;
    a.scale_ub = scale_ub;
    a.scales_dtype = scales_dtype;
    a.x_stride = hidden * esz;
    a.out_stride = hidden;
    return launch_fp8_from<InT>(a, src, out_fp8 == RMSQ_E4M3FNUZ, s, stream) == hipSuccess ? RMSQ_OK
                                                                                          : RMSQ_ERR_LAUNCH;
}

}  // namespace rmsq
