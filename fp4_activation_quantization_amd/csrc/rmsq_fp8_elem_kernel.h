// Fused (residual +) RMSNorm + per-row dynamic FP8 quantization for rows the
// 16-byte vector kernel (rmsq_fp8_kernel.h) cannot take: a hidden size that
// is not a multiple of the vector width (8 16-bit or 4 fp32 elements), or
// row starts and strides aligned only to the element size; rows of up to
// 16384 elements.  gfx950.
//
// Operation: the same as the vector kernel (Mojo docs "rms_norm_fused_fp8":
// epsilon, weight_offset, scale_ub, per-row scales; the local share of
// "allreduce_residual_rmsnorm_fp8": residual, residual_output = the pre-norm
// sum).  Those functions take any shape: their input_fn is generic in its
// SIMD width, so a row need not be a whole number of vectors.
//
// Work mapping: `waves` wavefronts own a row (1..16; a block holds 4/waves
// rows for 1-2 waves) and lane l of a row group owns the elements l, l + T,
// l + 2T, ... (T = 64 * waves, EPL elements per lane, compile time).  Every
// wave instruction therefore touches 64 consecutive elements: 128 bytes of a
// 16-bit input, 64 bytes of codes.  Each element is loaded and stored on its
// own (2- or 4-byte loads, 1-byte code stores), so any element-aligned row
// start works; the price is 8x (16-bit) or 4x (fp32) more memory
// instructions than the vector kernel, paid only off its fast path.
//
// Precision: s^2 summed in fp64 (exact products), rstd, the scale and the
// quantization factor in fp64 once per row; per element t = s * g' and
// q = t * k in fp32, as in the vector kernel.
#pragma once

#include "rmsq_device.h"
#include "rmsq_elem.h"
#include "rmsq_internal.h"

namespace rmsq {

template <typename InT, bool RESID, bool FNUZ, int EPL>
__global__ void __launch_bounds__(1024) fp8_elem_kernel(const FusedArgs a) {
    using E = Elem<InT>;
    using Bits = typename E::Bits;
    constexpr double INV_FMAX = FNUZ ? 1.0 / 240.0 : 1.0 / 448.0;
    constexpr int EPL4 = (EPL + 3) / 4 * 4;  // codes are converted four at a time

    const int waves = a.waves;
    const int T = waves * 64;
    const int rpb = blockDim.x / T;
    const int tid = threadIdx.x;
    const int slot = tid / T;
    const int lt = tid - slot * T;
    const int red = slot * waves + (lt >> 6);
    const int hidden = a.hidden;
    auto live = [&](int j) { return lt + j * T < hidden; };
    const Bits* gamma = static_cast<const Bits*>(a.gamma);

    __shared__ double red_sum[2][16];
    __shared__ int red_max[2][16];

    int parity = 0;
    for (int64_t row0 = (int64_t)blockIdx.x * rpb; row0 < a.rows; row0 += (int64_t)gridDim.x * rpb) {
        const int64_t row = row0 + slot;
        const bool active = row < a.rows;

        float t[EPL4];  // s * g' (zero past the row)
#pragma unroll
        for (int j = 0; j < EPL4; ++j) t[j] = 0.0f;
        double ssq = 0.0;
        float amax = 0.0f;
        if (active) {
            const Bits* xr = reinterpret_cast<const Bits*>(static_cast<const char*>(a.x) + row * a.x_stride);
            Bits xv[EPL], rv[RESID ? EPL : 1], gv[EPL];
            // all of the row's loads are issued before any store (residual_out
            // may be x or residual itself)
#pragma unroll
            for (int j = 0; j < EPL; ++j) xv[j] = live(j) ? load_elem(xr + lt + j * T) : (Bits)0;
            if constexpr (RESID) {
                const Bits* rr =
                    reinterpret_cast<const Bits*>(static_cast<const char*>(a.residual) + row * a.residual_stride);
#pragma unroll
                for (int j = 0; j < EPL; ++j) rv[j] = live(j) ? load_elem(rr + lt + j * T) : (Bits)0;
            }
#pragma unroll
            for (int j = 0; j < EPL; ++j) gv[j] = live(j) ? gamma[lt + j * T] : (Bits)0;
            Bits* ro = RESID ? reinterpret_cast<Bits*>(static_cast<char*>(a.residual_out) + row * a.residual_out_stride)
                             : nullptr;
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                float s = E::widen(xv[j]);
                if constexpr (RESID) {
                    // one rounding of the fp32 sum to the element type; the lane
                    // that read the element writes it
                    const Bits sb = E::round(s + E::widen(rv[j]));
                    s = E::widen(sb);
                    if (live(j)) store_elem(ro + lt + j * T, sb);
                }
                ssq += (double)s * (double)s;
                t[j] = s * (E::widen(gv[j]) + a.weight_offset);
                amax = fmaxf(amax, fabsf(t[j]));
            }
        }

        ssq = wave_sum(ssq);
        amax = wave_max_nonneg(amax);
        if (waves > 1) {  // uniform over the block
            if ((lt & 63) == 0) {
                red_sum[parity][red] = ssq;
                red_max[parity][red] = __float_as_int(amax);
            }
            __syncthreads();
            ssq = 0.0;
            int m = 0;
            for (int w = 0; w < waves; ++w) {
                ssq += red_sum[parity][slot * waves + w];
                m = max_bits(m, red_max[parity][slot * waves + w]);
            }
            amax = __int_as_float(m);
            // the other parity's slots are rewritten only after the next
            // barrier, which every wave reaches after finishing these reads
            parity ^= 1;
        }

        if (active) {
            const double rstd = rsqrt_refined(ssq * a.inv_hidden + (double)a.eps);
            double sc = (double)amax * rstd * INV_FMAX;
            if (sc > (double)a.scale_ub) sc = (double)a.scale_ub;
            uint32_t sbits;
            const float sc_st = round_scale((float)sc, a.scales_dtype, &sbits);
            const float kq = sc_st > 0.0f ? (float)(rstd * rcp_refined((double)sc_st)) : 0.0f;

            uint8_t* orow = static_cast<uint8_t*>(a.out) + row * a.out_stride;
#pragma unroll
            for (int j = 0; j < EPL4; j += 4) {
                const uint32_t c = fp8_x4<FNUZ>(t[j] * kq, t[j + 1] * kq, t[j + 2] * kq, t[j + 3] * kq);
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (j + k < EPL && live(j + k)) store_elem(orow + lt + (j + k) * T, (uint8_t)(c >> (8 * k)));
            }
            if (lt == 0) store_scale(a.scales, row, a.scales_dtype, sbits);
        }
    }
}

namespace fp8_elem_launch {

template <typename InT, bool RESID, bool FNUZ, int EPL>
hipError_t launch(FusedArgs a, Shape s, hipStream_t stream) {
    a.waves = s.waves;
    const int64_t groups = (a.rows + s.rpb - 1) / s.rpb;
    // default: one block per row group
    int64_t grid = s.grid > 0 ? s.grid : groups;
    if (grid > groups) grid = groups;
    if (grid > INT32_MAX) grid = INT32_MAX;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL((fp8_elem_kernel<InT, RESID, FNUZ, EPL>), dim3((unsigned)grid), dim3(s.waves * s.rpb * 64),
                       0, stream, a);
    return hipGetLastError();
}

// s.vpt carries the elements per lane: one of kElemPerLane (rmsq_internal.h)
template <typename InT, bool RESID, bool FNUZ>
hipError_t by_epl(const FusedArgs& a, Shape s, hipStream_t st) {
    switch (s.vpt) {
    case 1: return launch<InT, RESID, FNUZ, 1>(a, s, st);
    case 2: return launch<InT, RESID, FNUZ, 2>(a, s, st);
    case 4: return launch<InT, RESID, FNUZ, 4>(a, s, st);
    case 8: return launch<InT, RESID, FNUZ, 8>(a, s, st);
    case 12: return launch<InT, RESID, FNUZ, 12>(a, s, st);
    default: return launch<InT, RESID, FNUZ, 16>(a, s, st);
    }
}

}  // namespace fp8_elem_launch

// All element-path variants for one input type (one translation unit each).
template <typename InT>
hipError_t launch_fp8_elem_typed(const FusedArgs& a, bool residual, bool fnuz, Shape s, hipStream_t stream) {
    using namespace fp8_elem_launch;
    if (residual) return fnuz ? by_epl<InT, true, true>(a, s, stream) : by_epl<InT, true, false>(a, s, stream);
    return fnuz ? by_epl<InT, false, true>(a, s, stream) : by_epl<InT, false, false>(a, s, stream);
}

}  // namespace rmsq
