// Fused (residual +) RMSNorm + per-row dynamic FP8 quantization, gfx950.
//
// Operation: Mojo docs "rms_norm_fused_fp8" (epsilon, weight_offset, scale_ub,
// per-row scale output) and the local share of
// "allreduce_residual_rmsnorm_fp8" (residual, residual_output = pre-norm sum).
//
// One pass over HBM: every input element is read once into VGPRs, the row
// stays in registers between the reduction and the quantization, and every
// output byte is written once.
//
// Work mapping: `WAVES` wavefronts cooperate on one row; a block holds
// WPB/WAVES rows.  Lane l of a row group owns the 16-byte vectors
// l, l + T, l + 2T, ... (T = 64 * WAVES), so each wave instruction moves
// 1 KiB of contiguous input.  The grid is persistent: blocks stride over row
// groups, so gamma (+ weight_offset) is unpacked into fp32 registers once per
// block.
//
// Precision: s^2 is accumulated in fp32 within a 16-byte vector, then in
// fp64 per lane and across lanes; rstd, the scale and the quantization
// factor are formed in fp64 once per row.  Per element the kernel computes
// t = s * g' (fp32) and q = t * k with k = rstd / stored_scale (fp32), so the
// codes see at most a few fp32 roundings of relative error.
#include "rmsq_device.h"
#include "rmsq_internal.h"

namespace rmsq {

template <typename InT, bool RESID, bool FNUZ, int WAVES, int WPB, int VPT>
__global__ void __launch_bounds__(WPB * 64) fp8_kernel(const FusedArgs a) {
    using V = Vec<InT>;
    constexpr int EPV = V::EPV;
    constexpr int T = WAVES * 64;   // lanes per row
    constexpr int RPB = WPB / WAVES;  // rows per block
    constexpr double FMAX = FNUZ ? 240.0 : 448.0;

    const int tid = threadIdx.x;
    const int slot = tid / T;       // row slot within the block
    const int lt = tid - slot * T;  // lane within the row group
    const int wv = lt >> 6;         // wave within the row group
    const int nvec = a.nvec;
    const int64_t row_bytes = (int64_t)a.hidden * V::BYTES;

    __shared__ double red_sum[2][RPB][WAVES];
    __shared__ float red_max[2][RPB][WAVES];

    // gamma + weight_offset for this lane's columns, fp32, once per block
    float g[VPT][EPV];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int v = lt + k * T;
        if (v < nvec) {
            const uint4 gv = reinterpret_cast<const uint4*>(a.gamma)[v];
            V::unpack(gv, g[k]);
#pragma unroll
            for (int e = 0; e < EPV; ++e) g[k][e] += a.weight_offset;
        } else {
#pragma unroll
            for (int e = 0; e < EPV; ++e) g[k][e] = 0.0f;
        }
    }

    int parity = 0;
    for (int64_t row0 = (int64_t)blockIdx.x * RPB; row0 < a.rows; row0 += (int64_t)gridDim.x * RPB) {
        const int64_t row = row0 + slot;
        const bool active = row < a.rows;

        float t[VPT][EPV];  // s * g'
        double ssq = 0.0;
        float amax = 0.0f;
        if (active) {
            const uint4* xr = reinterpret_cast<const uint4*>(static_cast<const char*>(a.x) + row * row_bytes);
            uint4 xv[VPT];
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int v = lt + k * T;
                xv[k] = v < nvec ? xr[v] : make_uint4(0, 0, 0, 0);
            }
            if constexpr (RESID) {
                const uint4* rr =
                    reinterpret_cast<const uint4*>(static_cast<const char*>(a.residual) + row * row_bytes);
                uint4* ro = reinterpret_cast<uint4*>(static_cast<char*>(a.residual_out) + row * row_bytes);
                uint4 rv[VPT];
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int v = lt + k * T;
                    rv[k] = v < nvec ? rr[v] : make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int v = lt + k * T;
                    float xf[EPV], rf[EPV];
                    V::unpack(xv[k], xf);
                    V::unpack(rv[k], rf);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) xf[e] += rf[e];
                    // one rounding of the fp32 sum to the element type; fp32 keeps
                    // at least 2p+2 bits of a 16-bit sum, so this equals rounding
                    // the exact sum once
                    xv[k] = V::pack(xf);
                    if (v < nvec) ro[v] = xv[k];
                }
            }
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                float s[EPV];
                V::unpack(xv[k], s);
                float part = 0.0f;
#pragma unroll
                for (int e = 0; e < EPV; ++e) part = fmaf(s[e], s[e], part);
                ssq += (double)part;
#pragma unroll
                for (int e = 0; e < EPV; ++e) {
                    t[k][e] = s[e] * g[k][e];
                    amax = max_nonneg(amax, fabsf(t[k][e]));
                }
            }
        }

        ssq = wave_sum(ssq);
        amax = wave_max(amax);
        if constexpr (WAVES > 1) {
            if ((lt & 63) == 0) {
                red_sum[parity][slot][wv] = ssq;
                red_max[parity][slot][wv] = amax;
            }
            __syncthreads();
            ssq = 0.0;
            amax = 0.0f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) {
                ssq += red_sum[parity][slot][w];
                amax = max_nonneg(amax, red_max[parity][slot][w]);
            }
            // the other parity's slots are rewritten only after the next
            // barrier, which every wave reaches after finishing these reads
            parity ^= 1;
        }

        if (active) {
            const double rstd = 1.0 / sqrt(ssq / (double)a.hidden + (double)a.eps);
            double sc = (double)amax * rstd / FMAX;
            if (sc > (double)a.scale_ub) sc = (double)a.scale_ub;
            uint32_t sbits;
            const float sc_st = round_scale((float)sc, a.scales_dtype, &sbits);
            const float kq = sc_st > 0.0f ? (float)(rstd / (double)sc_st) : 0.0f;

            uint8_t* orow = static_cast<uint8_t*>(a.out) + row * (int64_t)a.hidden;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int v = lt + k * T;
                if (v < nvec) {
                    if constexpr (EPV == 8) {
                        uint2 w;
                        w.x = fp8_x4<FNUZ>(t[k][0] * kq, t[k][1] * kq, t[k][2] * kq, t[k][3] * kq);
                        w.y = fp8_x4<FNUZ>(t[k][4] * kq, t[k][5] * kq, t[k][6] * kq, t[k][7] * kq);
                        reinterpret_cast<uint2*>(orow)[v] = w;
                    } else {
                        reinterpret_cast<uint32_t*>(orow)[v] =
                            fp8_x4<FNUZ>(t[k][0] * kq, t[k][1] * kq, t[k][2] * kq, t[k][3] * kq);
                    }
                }
            }
            if (lt == 0) store_scale(a.scales, row, a.scales_dtype, sbits);
        }
    }
}

namespace {

template <typename InT, bool RESID, bool FNUZ, int WAVES, int VPT>
hipError_t launch_shape(const FusedArgs& a, Shape s, hipStream_t stream) {
    constexpr int WPB = WAVES >= 4 ? WAVES : 4;
    constexpr int RPB = WPB / WAVES;
    auto kern = fp8_kernel<InT, RESID, FNUZ, WAVES, WPB, VPT>;
    const int64_t groups = (a.rows + RPB - 1) / RPB;
    int64_t grid = persistent_blocks(reinterpret_cast<const void*>(kern), WPB * 64);
    if (s.grid > 0 && s.grid < grid) grid = s.grid;
    if (grid > groups) grid = groups;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WPB * 64), 0, stream, a);
    return hipGetLastError();
}

template <typename InT, bool RESID, bool FNUZ, int WAVES>
hipError_t by_vpt(const FusedArgs& a, Shape s, hipStream_t st) {
    switch (s.vpt) {
    case 1: return launch_shape<InT, RESID, FNUZ, WAVES, 1>(a, s, st);
    case 2: return launch_shape<InT, RESID, FNUZ, WAVES, 2>(a, s, st);
    default: return launch_shape<InT, RESID, FNUZ, WAVES, 4>(a, s, st);
    }
}

template <typename InT, bool RESID, bool FNUZ>
hipError_t by_waves(const FusedArgs& a, Shape s, hipStream_t st) {
    switch (s.waves) {
    case 1: return by_vpt<InT, RESID, FNUZ, 1>(a, s, st);
    case 2: return by_vpt<InT, RESID, FNUZ, 2>(a, s, st);
    case 4: return by_vpt<InT, RESID, FNUZ, 4>(a, s, st);
    case 8: return by_vpt<InT, RESID, FNUZ, 8>(a, s, st);
    default: return by_vpt<InT, RESID, FNUZ, 16>(a, s, st);
    }
}

template <typename InT>
hipError_t by_variant(const FusedArgs& a, bool resid, bool fnuz, Shape s, hipStream_t st) {
    if (resid) return fnuz ? by_waves<InT, true, true>(a, s, st) : by_waves<InT, true, false>(a, s, st);
    return fnuz ? by_waves<InT, false, true>(a, s, st) : by_waves<InT, false, false>(a, s, st);
}

}  // namespace

hipError_t launch_fp8(const FusedArgs& a, int in_dtype, bool residual, int out_fp8, Shape s,
                      hipStream_t stream) {
    const bool fnuz = out_fp8 == 1;
    if (in_dtype == 0) return by_variant<float>(a, residual, fnuz, s, stream);
    if (in_dtype == 1) return by_variant<F16>(a, residual, fnuz, s, stream);
    return by_variant<BF16>(a, residual, fnuz, s, stream);
}

}  // namespace rmsq
