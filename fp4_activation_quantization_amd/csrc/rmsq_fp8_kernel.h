// Fused (residual +) RMSNorm + per-row dynamic FP8 quantization, gfx950.
//
// Operation: Mojo docs "rms_norm_fused_fp8" (epsilon, weight_offset, scale_ub,
// per-row scale output) and the local share of
// "allreduce_residual_rmsnorm_fp8" (residual, residual_output = pre-norm sum).
//
// One pass over HBM: every input element is read once into VGPRs, the row
// stays in registers between the reduction and the quantization, and every
// output byte is written once, all with non-temporal hints.
//
// Work mapping: `waves` wavefronts (1..16, a launch parameter) cooperate on
// one row; a block holds one row, or 4/waves rows for 1-2 waves.  Lane l of a
// row group owns the 16-byte vectors l, l + T, l + 2T, ... (T = 64 * waves,
// VPT vectors per lane, a compile-time constant), so each wave instruction
// moves 1 KiB of contiguous input.  EXACT (compile time) means the lanes hold
// the row exactly (nvec == VPT * T): no lane is idle and no access needs a
// guard.  Blocks stride over row groups; by default the grid has one block per
// row group (large batches stream best that way on MI355X, and
// gamma + weight_offset comes from L2).  STRIDED (compile time) reads each
// row tensor's row stride from the arguments; otherwise rows are adjacent.
//
// Precision: q = s * g' * rstd / stored_scale is rounded once to fp32 (the
// helpers and the PROD forms in rmsq_device.h, "FP8 per-row numerics"): s^2
// is accumulated in fp64, the factor k = rstd / stored_scale is formed in
// fp64, and s * g' and its row maximum are exact.  What is held across the
// barrier: t = s * g' in fp32 (kProdF32); the packed row s and packed 16-bit
// gamma (the other forms), with fp32 gamma staged in LDS instead of held
// (its 4 VGPRs per vector would leave room for only one 1024-thread block
// per CU; taken from L2 again after the barrier instead it measured 8% slower
// on 32768 x 8192 fp32 rows, the load's latency exposed on every row).
//
// The row to normalize comes from a source policy Src (the analogue of the
// input_fn parameter of Mojo docs "rms_norm_fused_fp8"): either InputRows
// (the x tensor of the arguments), or a copyable struct with
//   __device__ uint4 operator()(int64_t row, int v) const
// returning the 16-byte vector v of that row as packed InT elements, which a
// producer computes from its own operands (each vector is requested once per
// row, by the lane that owns it, before any of the row's stores).
#pragma once

#include <type_traits>

#include "rmsq_device.h"
#include "rmsq_internal.h"

namespace rmsq {

// The default source: the rows of FusedArgs::x (x_stride bytes apart).
struct InputRows {};

template <class Src, typename InT, bool RESID, bool FNUZ, int VPT, bool EXACT, bool ONE_ROW, bool STRIDED,
          bool GAMMA_FIRST, int PROD>
__global__ void __launch_bounds__(1024) fp8_kernel(const FusedArgs a, const Src src) {
    using V = Vec<InT>;
    constexpr int EPV = V::EPV;
    constexpr double INV_FMAX = FNUZ ? 1.0 / 240.0 : 1.0 / 448.0;
    static_assert(PROD != kProdF32 || V::BYTES == 2, "fp32 products are not exact in fp32");
    static_assert(PROD != kProdTwo || V::BYTES == 4, "the two-term form is for fp32 inputs");
    constexpr bool T32 = PROD == kProdF32;  // t = s * g' held in fp32
    // gamma held across the barrier (else taken from L2 again after it)
    constexpr bool HOLD_G = GAMMA_FIRST || V::BYTES == 2;

    const int waves = a.waves;       // wavefronts per row
    const int T = waves * 64;        // lanes per row
    // ONE_ROW: the block is one row group, so the row index is uniform
    const int rpb = ONE_ROW ? 1 : blockDim.x / T;  // rows per block
    const int tid = threadIdx.x;
    const int slot = ONE_ROW ? 0 : tid / T;        // row slot within the block
    const int lt = tid - slot * T;  // lane within the row group
    const int red = slot * waves + (lt >> 6);  // this wave's reduction slot
    const int nvec = a.nvec;
    auto live = [&](int k) { return EXACT || lt + k * T < nvec; };
    // bytes between rows: one value for the adjacent-row case
    const int64_t row_bytes = (int64_t)a.hidden * V::BYTES;
    const int64_t x_stride = STRIDED ? a.x_stride : row_bytes;
    const int64_t r_stride = STRIDED ? a.residual_stride : row_bytes;
    const int64_t ro_stride = STRIDED ? a.residual_out_stride : row_bytes;
    const int64_t out_stride = STRIDED ? a.out_stride : (int64_t)a.hidden;
    const double offd = PROD == kProdF64 ? (double)a.weight_offset : 0.0;

    __shared__ double red_sum[2][16];
    __shared__ uint64_t red_max[2][16];  // bits of each wave's (non-negative fp64) max |s * g'|
    // fp32 gamma, VPT vectors per thread (dynamic LDS of blockDim * VPT * 16
    // bytes; HOLD_G false only): each lane writes its own vectors with the
    // row's loads and reads them back to quantize, so no barrier is involved
    extern __shared__ uint4 g_stash[];

    // Gamma for this lane's columns (zero past the row): g + weight_offset in
    // fp32 (kProdF32, where the offset is 0), or packed gamma (the other
    // forms; the offset added in fp64).  GAMMA_FIRST (small batches without a
    // residual): loaded once, before the rows; otherwise loaded with each
    // row, after the row's own loads and in flight together with them.
    // Measured on MI355X: a one-row call has ~6% lower latency the first way;
    // large batches stream 3.5-7% faster the second way without a residual,
    // ~1% with one.
    float g[T32 ? VPT : 1][EPV];
    uint4 gp[T32 ? 1 : VPT];  // packed gamma (the forms other than kProdF32)
    auto load_gamma = [&]() {
        uint4 gv[VPT];
#pragma unroll
        for (int k = 0; k < VPT; ++k)
            gv[k] = live(k) ? reinterpret_cast<const uint4*>(a.gamma)[lt + k * T] : make_uint4(0, 0, 0, 0);
        if constexpr (!T32) {
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                gp[k] = gv[k];
                if constexpr (!HOLD_G) g_stash[k * blockDim.x + tid] = gv[k];
            }
        } else {
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                V::unpack(gv[k], g[k]);
                // + 0.0f as the definition's g + offset (a -0 gamma becomes +0)
#pragma unroll
                for (int e = 0; e < EPV; ++e) g[k][e] = live(k) ? g[k][e] + a.weight_offset : 0.0f;
            }
        }
    };
    if constexpr (GAMMA_FIRST) load_gamma();

    int parity = 0;
    for (int64_t row0 = (int64_t)blockIdx.x * rpb; row0 < a.rows; row0 += (int64_t)gridDim.x * rpb) {
        const int64_t row = row0 + slot;
        const bool active = row < a.rows;

        float t[T32 ? VPT : 1][EPV];  // s * g' (exact in fp32)
        uint4 xv[VPT];                // the row s (packed); held across the barrier by the other forms
        double ssq0 = 0.0, ssq1 = 0.0;
        float amax32 = 0.0f;
        double amax64 = 0.0;
        if (active) {
            // vectors past the end of the row are zero: they add nothing
            if constexpr (std::is_same_v<Src, InputRows>) {
                const char* xr = static_cast<const char*>(a.x) + row * x_stride;
#pragma unroll
                for (int k = 0; k < VPT; ++k) xv[k] = live(k) ? load_stream(xr, lt + k * T) : make_uint4(0, 0, 0, 0);
            } else {
#pragma unroll
                for (int k = 0; k < VPT; ++k) xv[k] = live(k) ? src(row, lt + k * T) : make_uint4(0, 0, 0, 0);
            }
            // every load of the row is issued before any store: residual_out
            // may alias residual, so a load placed after a store could not be
            // moved ahead of it and each vector would cost a round trip
            uint4 rv[RESID ? VPT : 1];
            if constexpr (RESID) {
                const char* rr = static_cast<const char*>(a.residual) + row * r_stride;
#pragma unroll
                for (int k = 0; k < VPT; ++k) rv[k] = live(k) ? load_stream(rr, lt + k * T) : make_uint4(0, 0, 0, 0);
            }
            if constexpr (!GAMMA_FIRST) load_gamma();  // an L2 hit after the first block
            if constexpr (RESID) {
                // residual_out may be x or residual itself: each vector is read
                // (above) and then written by the one lane that owns it
                char* ro = static_cast<char*>(a.residual_out) + row * ro_stride;
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    float xf[EPV], rf[EPV];
                    V::unpack(xv[k], xf);
                    V::unpack(rv[k], rf);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) xf[e] += rf[e];
                    // one rounding of the fp32 sum to the element type; fp32 keeps
                    // at least 2p+2 bits of a 16-bit sum, so this equals rounding
                    // the exact sum once
                    xv[k] = V::pack(xf);
                    if (live(k)) store_stream(ro, lt + k * T, xv[k]);
                }
            }
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                float s[EPV];
                V::unpack(xv[k], s);
                sumsq64<EPV>(ssq0, ssq1, s);
                if constexpr (T32) {
#pragma unroll
                    for (int e = 0; e < EPV; ++e) t[k][e] = s[e] * g[k][e];
                    amax32 = abs_max<EPV>(amax32, t[k]);
                } else {
                    float gf[EPV];
                    V::unpack(gp[k], gf);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) amax64 = fmax(amax64, abs_prod64(s[e], gf[e], offd));
                }
            }
        }

        double ssq = wave_sum(ssq0 + ssq1);
        double amax = T32 ? (double)wave_max_nonneg(amax32) : wave_max_nonneg(amax64);
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
            uint8_t* orow = static_cast<uint8_t*>(a.out) + row * out_stride;
            // vector k's codes stored (8 or 4 bytes per lane)
            auto emit = [&](int k, const float (&q)[EPV]) {
                if constexpr (EPV == 8) {
                    uint2 w;
                    w.x = fp8_x4<FNUZ>(q[0], q[1], q[2], q[3]);
                    w.y = fp8_x4<FNUZ>(q[4], q[5], q[6], q[7]);
                    store_stream(orow, lt + k * T, w);
                } else {
                    store_stream(orow, lt + k * T, fp8_x4<FNUZ>(q[0], q[1], q[2], q[3]));
                }
            };
            // the forms that recompute s * g' from the packed row and gamma
            auto gamma_at = [&](int k, float (&gf)[EPV]) {
                V::unpack(HOLD_G ? gp[T32 ? 0 : k] : g_stash[k * blockDim.x + tid], gf);
            };
            if (split) {
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    if (!live(k)) continue;
                    float q[EPV];
                    if constexpr (T32) {
#pragma unroll
                        for (int e = 0; e < EPV; ++e) q[e] = fp8_q1(t[k][e], fr);
                    } else {
                        float s[EPV], gf[EPV];
                        V::unpack(xv[k], s);
                        gamma_at(k, gf);
#pragma unroll
                        for (int e = 0; e < EPV; ++e) q[e] = fp8_q2(s[e], gf[e], fr);
                    }
                    emit(k, q);
                }
            } else {
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    if (!live(k)) continue;
                    float q[EPV];
                    if constexpr (T32) {
#pragma unroll
                        for (int e = 0; e < EPV; ++e) q[e] = (float)((double)t[k][e] * fr.k);
                    } else {
                        float s[EPV], gf[EPV];
                        V::unpack(xv[k], s);
                        gamma_at(k, gf);
#pragma unroll
                        for (int e = 0; e < EPV; ++e) q[e] = fp8_q64(s[e], gf[e], offd, fr);
                    }
                    emit(k, q);
                }
            }
            if (lt == 0) store_scale(a.scales, row, a.scales_dtype, fr.sbits);
        }
    }
}

namespace fp8_launch {

template <class Src, typename InT, bool RESID, bool FNUZ, int VPT, bool STRIDED, bool GAMMA_FIRST, int PROD>
void launch_shape(const FusedArgs& a, const Src& src, Shape s, dim3 gd, dim3 bd, hipStream_t stream) {
    const bool exact = a.nvec == VPT * s.waves * 64;
    // the LDS gamma stash of fp32 rows (the forms other than kProdF32)
    const size_t lds = PROD != kProdF32 && Vec<InT>::BYTES == 4 && !GAMMA_FIRST ? (size_t)bd.x * VPT * 16 : 0;
    if (s.rpb == 1) {
        if (exact)
            hipLaunchKernelGGL((fp8_kernel<Src, InT, RESID, FNUZ, VPT, true, true, STRIDED, GAMMA_FIRST, PROD>), gd, bd,
                               lds, stream, a, src);
        else
            hipLaunchKernelGGL((fp8_kernel<Src, InT, RESID, FNUZ, VPT, false, true, STRIDED, GAMMA_FIRST, PROD>), gd, bd,
                               lds, stream, a, src);
    } else {
        if (exact)
            hipLaunchKernelGGL((fp8_kernel<Src, InT, RESID, FNUZ, VPT, true, false, STRIDED, GAMMA_FIRST, PROD>), gd,
                               bd, lds, stream, a, src);
        else
            hipLaunchKernelGGL((fp8_kernel<Src, InT, RESID, FNUZ, VPT, false, false, STRIDED, GAMMA_FIRST, PROD>), gd,
                               bd, lds, stream, a, src);
    }
}

// the product form: kProdF32 / kProdTwo without a weight offset, else kProdF64
template <class Src, typename InT, bool RESID, bool FNUZ, int VPT, bool STRIDED, bool GAMMA_FIRST>
void launch_numerics(const FusedArgs& a, const Src& src, Shape s, dim3 gd, dim3 bd, hipStream_t stream) {
    if (prod_mode<InT>(a.weight_offset) == kProdF64)
        launch_shape<Src, InT, RESID, FNUZ, VPT, STRIDED, GAMMA_FIRST, kProdF64>(a, src, s, gd, bd, stream);
    else
        launch_shape<Src, InT, RESID, FNUZ, VPT, STRIDED, GAMMA_FIRST, prod_mode<InT>(0.0f)>(a, src, s, gd, bd,
                                                                                             stream);
}

template <class Src, typename InT, bool RESID, bool FNUZ, int VPT, bool STRIDED>
hipError_t launch_vpt(FusedArgs a, const Src& src, Shape s, hipStream_t stream) {
    a.waves = s.waves;
    const int64_t groups = (a.rows + s.rpb - 1) / s.rpb;
    // default: one block per row group
    int64_t grid = s.grid > 0 ? s.grid : groups;
    if (grid > groups) grid = groups;
    if (grid > INT32_MAX) grid = INT32_MAX;
    if (grid < 1) grid = 1;
    const dim3 gd((unsigned)grid), bd(s.waves * s.rpb * 64);
    // gamma before the rows only for small batches without a residual
    if (!RESID && a.rows <= kLatencyRows)
        launch_numerics<Src, InT, RESID, FNUZ, VPT, STRIDED, !RESID>(a, src, s, gd, bd, stream);
    else
        launch_numerics<Src, InT, RESID, FNUZ, VPT, STRIDED, false>(a, src, s, gd, bd, stream);
    return hipGetLastError();
}

template <class Src, typename InT, bool RESID, bool FNUZ, bool STRIDED>
hipError_t by_vpt(const FusedArgs& a, const Src& src, Shape s, hipStream_t st) {
    switch (s.vpt) {
    case 1: return launch_vpt<Src, InT, RESID, FNUZ, 1, STRIDED>(a, src, s, st);
    case 2: return launch_vpt<Src, InT, RESID, FNUZ, 2, STRIDED>(a, src, s, st);
    default: return launch_vpt<Src, InT, RESID, FNUZ, 4, STRIDED>(a, src, s, st);
    }
}

template <typename InT, bool STRIDED>
hipError_t by_variant(const FusedArgs& a, bool resid, bool fnuz, Shape s, hipStream_t st) {
    const InputRows src;
    if (resid)
        return fnuz ? by_vpt<InputRows, InT, true, true, STRIDED>(a, src, s, st)
                    : by_vpt<InputRows, InT, true, false, STRIDED>(a, src, s, st);
    return fnuz ? by_vpt<InputRows, InT, false, true, STRIDED>(a, src, s, st)
                : by_vpt<InputRows, InT, false, false, STRIDED>(a, src, s, st);
}

}  // namespace fp8_launch

// All FP8 variants for one input type (instantiated once per type, each in
// its own translation unit so they compile in parallel).
template <typename InT>
hipError_t launch_fp8_typed(const FusedArgs& a, bool residual, bool fnuz, Shape s, hipStream_t stream) {
    const int64_t rb = (int64_t)a.hidden * Vec<InT>::BYTES;
    const bool adjacent = a.x_stride == rb && a.out_stride == a.hidden &&
                          (!residual || (a.residual_stride == rb && a.residual_out_stride == rb));
    return adjacent ? fp8_launch::by_variant<InT, false>(a, residual, fnuz, s, stream)
                    : fp8_launch::by_variant<InT, true>(a, residual, fnuz, s, stream);
}

// The FP8 kernel without a residual over rows from a source policy (adjacent
// output rows; `a.x` and `a.x_stride` unused).
template <typename InT, class Src>
hipError_t launch_fp8_from(const FusedArgs& a, const Src& src, bool fnuz, Shape s, hipStream_t stream) {
    return fnuz ? fp8_launch::by_vpt<Src, InT, false, true, false>(a, src, s, stream)
                : fp8_launch::by_vpt<Src, InT, false, false, false>(a, src, s, stream);
}

}  // namespace rmsq
