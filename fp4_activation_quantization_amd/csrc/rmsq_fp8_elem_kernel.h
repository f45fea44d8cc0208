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
// Precision: as the vector kernel (the PROD forms of rmsq_device.h): s^2
// summed in fp64, rstd, the scale and the factor k in fp64 once per row,
// s * g' and its row maximum exact, and q = s * g' * k rounded once to fp32.
// Held across the barrier: t = s * g' (kProdF32), or s and gamma's bits.
#pragma once

#include "rmsq_device.h"
#include "rmsq_elem.h"
#include "rmsq_internal.h"

namespace rmsq {

template <typename InT, bool RESID, bool FNUZ, int EPL, int PROD>
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
    const double offd = PROD == kProdF64 ? (double)a.weight_offset : 0.0;
    constexpr bool T32 = PROD == kProdF32;  // t = s * g' (exact in fp32) held

    __shared__ double red_sum[2][16];
    __shared__ uint64_t red_max[2][16];  // bits of each wave's (non-negative fp64) max |s * g'|

    int parity = 0;
    for (int64_t row0 = (int64_t)blockIdx.x * rpb; row0 < a.rows; row0 += (int64_t)gridDim.x * rpb) {
        const int64_t row = row0 + slot;
        const bool active = row < a.rows;

        float sv[EPL4];  // s (zero past the row), or t = s * g' (T32)
        Bits gv[EPL];    // gamma's bits
#pragma unroll
        for (int j = 0; j < EPL4; ++j) sv[j] = 0.0f;
        double ssq0 = 0.0, ssq1 = 0.0;
        double amax = 0.0;
        if (active) {
            const Bits* xr = reinterpret_cast<const Bits*>(static_cast<const char*>(a.x) + row * a.x_stride);
            Bits xv[EPL], rv[RESID ? EPL : 1];
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
                const double d = s;
                if (j & 1)
                    ssq1 = fma(d, d, ssq1);
                else
                    ssq0 = fma(d, d, ssq0);
                if constexpr (T32) {
                    // + weight_offset (0.0f here) as the definition's g + offset: a -0 gamma becomes +0
                    sv[j] = s * (E::widen(gv[j]) + a.weight_offset);
                    amax = fmax(amax, (double)fabsf(sv[j]));
                } else {
                    sv[j] = s;
                    amax = fmax(amax, abs_prod64(s, E::widen(gv[j]), offd));
                }
            }
        }

        double ssq = wave_sum(ssq0 + ssq1);
        amax = wave_max_nonneg(amax);
        if (waves > 1) {  // uniform over the block
            if ((lt & 63) == 0) {
                red_sum[parity][red] = ssq;
                red_max[parity][red] = __builtin_bit_cast(uint64_t, amax);
            }
            __syncthreads();
            ssq = 0.0;
            uint64_t m = 0;
            for (int w = 0; w < waves; ++w) {
                ssq += red_sum[parity][slot * waves + w];
                m = max_u64(m, red_max[parity][slot * waves + w]);
            }
            amax = __builtin_bit_cast(double, m);
            // the other parity's slots are rewritten only after the next
            // barrier, which every wave reaches after finishing these reads
            parity ^= 1;
        }

        if (active) {
            const double rstd = rsqrt_refined(ssq * a.inv_hidden + (double)a.eps);
            const Fp8Row fr = fp8_row(amax, rstd, INV_FMAX, a.scale_ub, a.scales_dtype);
            const bool split = PROD != kProdF64 && __builtin_amdgcn_readfirstlane((int)fr.split);  // uniform
            float q[EPL4];
            if (split) {
#pragma unroll
                for (int j = 0; j < EPL4; ++j)
                    q[j] = j >= EPL ? 0.0f : T32 ? fp8_q1(sv[j], fr) : fp8_q2(sv[j], E::widen(gv[j]), fr);
            } else {
#pragma unroll
                for (int j = 0; j < EPL4; ++j)
                    q[j] = j >= EPL ? 0.0f
                           : T32    ? (float)((double)sv[j] * fr.k)
                                    : fp8_q64(sv[j], E::widen(gv[j]), offd, fr);
            }
            uint8_t* orow = static_cast<uint8_t*>(a.out) + row * a.out_stride;
#pragma unroll
            for (int j = 0; j < EPL4; j += 4) {
                const uint32_t c = fp8_x4<FNUZ>(q[j], q[j + 1], q[j + 2], q[j + 3]);
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (j + k < EPL && live(j + k)) store_elem(orow + lt + (j + k) * T, (uint8_t)(c >> (8 * k)));
            }
            if (lt == 0) store_scale(a.scales, row, a.scales_dtype, fr.sbits);
        }
    }
}

namespace fp8_elem_launch {

template <typename InT, bool RESID, bool FNUZ, int EPL, int PROD>
hipError_t launch_prod(FusedArgs a, Shape s, hipStream_t stream) {
    a.waves = s.waves;
    const int64_t groups = (a.rows + s.rpb - 1) / s.rpb;
    // default: one block per row group
    int64_t grid = s.grid > 0 ? s.grid : groups;
    if (grid > groups) grid = groups;
    if (grid > INT32_MAX) grid = INT32_MAX;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL((fp8_elem_kernel<InT, RESID, FNUZ, EPL, PROD>), dim3((unsigned)grid),
                       dim3(s.waves * s.rpb * 64), 0, stream, a);
    return hipGetLastError();
}

// the product form: kProdF32 / kProdTwo without a weight offset, else kProdF64
template <typename InT, bool RESID, bool FNUZ, int EPL>
hipError_t launch(const FusedArgs& a, Shape s, hipStream_t stream) {
    if (prod_mode<InT>(a.weight_offset) == kProdF64) return launch_prod<InT, RESID, FNUZ, EPL, kProdF64>(a, s, stream);
    return launch_prod<InT, RESID, FNUZ, EPL, prod_mode<InT>(0.0f)>(a, s, stream);
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
