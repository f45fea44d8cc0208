// Fused (residual +) RMSNorm + FP8 / FP4 quantization for rows wider than
// the register-resident kernels hold (more than 16 waves x 64 lanes x 4
// vectors = 4096 16-byte vectors: 32768 16-bit or 16384 fp32 elements),
// gfx950: the row is staged in LDS (160 KB per CU) between the reduction and
// the quantization.
//
// Operation: that of rmsq_fp8_kernel.h (Mojo docs "rms_norm_fused_fp8",
// per-row scale; the residual form of "allreduce_residual_rmsnorm_fp8") and
// of rmsq_fp4_kernel.h (FlashInfer "rmsnorm_fp4quant.py": E4M3 or UE8M0
// block scales over 16 or 32 elements, row-major or swizzled, optionally the
// page's 16-bit x * w product), with or without the residual, computed with
// the same fp32 / fp64 steps as those kernels.
//
// Work mapping: one 1024-thread block per row (blocks stride over rows).
// Pass 1: lane l takes the 16-byte vectors l, l + 1024, ..., U of them in
// flight at a time; it forms s (x, or x + residual rounded once to the input
// type and stored to residual_out), keeps s in LDS and accumulates sum(s^2)
// and, for FP8, max |s * g'| (g' = gamma + weight_offset, read from L2).
// The block reduces both through LDS.  Pass 2: every lane takes its vectors
// back from LDS, forms t = s * g' again (the same fp32 products) and
// quantizes: FP8 with the row's scale, FP4 per block, whose lanes are
// adjacent as in the FP4 kernel.  HBM traffic is that of the register
// kernels: every input element read once, every output written once.
#pragma once

#include "rmsq_device.h"
#include "rmsq_internal.h"

namespace rmsq {

constexpr int kWideThreads = 1024;

template <typename InT, bool RESID, int OUT, int BLOCK, bool UE8M0>
__global__ void __launch_bounds__(1024) wide_kernel(const FusedArgs a) {
    using V = Vec<InT>;
    constexpr int EPV = V::EPV;
    // vectors per lane loaded together in pass 1: 8 with a residual, 4
    // without (measured: 8 is 9-13% faster with a residual; without one the
    // extra registers cost a second resident block on rows that leave LDS
    // room for it, 14% at 40000 elements)
    constexpr int T = kWideThreads, U = RESID ? 8 : 4;
    constexpr bool FP4 = OUT == kWideFp4;
    constexpr bool FNUZ = OUT == kWideFp8Fnuz;
    constexpr int LPB = BLOCK / EPV;  // FP4: lanes (vectors) per block
    constexpr double INV_FMAX = FNUZ ? 1.0 / 240.0 : 1.0 / 448.0;

    extern __shared__ uint4 row_s[];  // s of the current row: nvec vectors
    __shared__ double red_sum[16];
    __shared__ int red_max[16];

    const int tid = threadIdx.x;
    const int nvec = a.nvec;
    const int steps = (nvec + U * T - 1) / (U * T);  // uniform over the block
    const uint4* gv = static_cast<const uint4*>(a.gamma);
    auto gamma_of = [&](int d, float (&g)[EPV]) {
        V::unpack(gv[d], g);
#pragma unroll
        for (int e = 0; e < EPV; ++e) g[e] += a.weight_offset;
    };

    // chunk i of a row: this lane's vectors tid + (i * U + u) * T, u < U.
    // Every load of a chunk comes before any of its stores (residual_out may
    // be x or residual itself; the lane that reads a vector writes it).
    auto fetch = [&](int64_t row, int i, uint4 (&xv)[U], uint4 (&rv)[U]) {
        const char* xr = static_cast<const char*>(a.x) + row * a.x_stride;
        const char* rr = RESID ? static_cast<const char*>(a.residual) + row * a.residual_stride : nullptr;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int d = tid + (i * U + u) * T;
            if (d < nvec) {
                xv[u] = load_stream(xr, d);
                if constexpr (RESID) rv[u] = load_stream(rr, d);
            }
        }
    };

    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        // ---- pass 1: s into LDS, sum of squares (and FP8's amax) ----
        char* ro = RESID ? static_cast<char*>(a.residual_out) + row * a.residual_out_stride : nullptr;
        double ssq = 0.0;
        float amax = 0.0f;
        for (int i = 0; i < steps; ++i) {
            uint4 xv[U], rv[U];
            fetch(row, i, xv, rv);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int d = tid + (i * U + u) * T;
                if (d >= nvec) continue;
                uint4 s = xv[u];
                if constexpr (RESID) {
                    float xf[EPV], rf[EPV];
                    V::unpack(xv[u], xf);
                    V::unpack(rv[u], rf);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) xf[e] += rf[e];
                    s = V::pack(xf);  // one rounding of the fp32 sum
                    store_stream(ro, d, s);
                }
                row_s[d] = s;
                ssq += (double)V::sumsq(s);
                if constexpr (!FP4) {
                    float sf[EPV], g[EPV], t[EPV];
                    V::unpack(s, sf);
                    gamma_of(d, g);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) t[e] = sf[e] * g[e];
                    amax = abs_max<EPV>(amax, t);
                }
            }
        }

        // ---- the row's sums over the block (the barrier also orders the
        // row's LDS writes before pass 2 reads them) ----
        ssq = wave_sum(ssq);
        if constexpr (!FP4) amax = wave_max_nonneg(amax);
        if ((tid & 63) == 0) {
            red_sum[tid >> 6] = ssq;
            red_max[tid >> 6] = __float_as_int(amax);
        }
        __syncthreads();
        ssq = 0.0;
        int m = 0;
        for (int w = 0; w < T / 64; ++w) {
            ssq += red_sum[w];
            m = max_bits(m, red_max[w]);
        }
        amax = __int_as_float(m);
        const double rstd = rsqrt_refined(ssq * a.inv_hidden + (double)a.eps);

        // ---- pass 2: quantize from LDS ----
        if constexpr (!FP4) {
            double sc = (double)amax * rstd * INV_FMAX;
            if (sc > (double)a.scale_ub) sc = (double)a.scale_ub;
            uint32_t sbits;
            const float sc_st = round_scale((float)sc, a.scales_dtype, &sbits);
            const float kq = sc_st > 0.0f ? (float)(rstd * rcp_refined((double)sc_st)) : 0.0f;
            uint8_t* orow = static_cast<uint8_t*>(a.out) + row * a.out_stride;
            for (int i = 0; i < steps; ++i) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int d = tid + (i * U + u) * T;
                    if (d >= nvec) continue;
                    float sf[EPV], g[EPV], t[EPV];
                    V::unpack(row_s[d], sf);
                    gamma_of(d, g);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) t[e] = sf[e] * g[e];
                    if constexpr (EPV == 8) {
                        uint2 w;
                        w.x = fp8_x4<FNUZ>(t[0] * kq, t[1] * kq, t[2] * kq, t[3] * kq);
                        w.y = fp8_x4<FNUZ>(t[4] * kq, t[5] * kq, t[6] * kq, t[7] * kq);
                        store_stream(orow, d, w);
                    } else {
                        store_stream(orow, d, fp8_x4<FNUZ>(t[0] * kq, t[1] * kq, t[2] * kq, t[3] * kq));
                    }
                }
            }
            if (tid == 0) store_scale(a.scales, row, a.scales_dtype, sbits);
        } else {
            // E4M3: block scale gs * (amax_t * rstd) / 6, element factor
            // gs * rstd / d; UE8M0 (gs = 1): code from amax_t * rstd / 6,
            // element factor rstd * 2^(127 - code)
            const double gs = a.global_scale ? (double)*a.global_scale : 1.0;
            const float c_scale = (float)(gs * rstd * (1.0 / 6.0));
            const float c_elem = (float)(gs * rstd);
            const bool swz = a.sf_swizzled != 0;
            const int nblk = a.hidden / BLOCK;
            uint8_t* orow = static_cast<uint8_t*>(a.out) + row * a.out_stride;
            // this row's scale bytes: row-major, or the row's place in its
            // 128 x 4 tiles ((row/128) * K * 512 + (row%32) * 16 + ((row%128)/32) * 4)
            uint8_t* srow = static_cast<uint8_t*>(a.scales) +
                            (swz ? (row >> 7) * ((int64_t)a.sf_k_tiles * 512) + (row & 31) * 16 +
                                       ((row & 127) >> 5) * 4
                                 : row * (int64_t)nblk);
            for (int i = 0; i < steps; ++i) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    // every lane takes part in the block's lane swaps: a
                    // block's lanes are all inside the row or all past it
                    // (nvec and T are multiples of LPB), and past it t = 0
                    const int d = tid + (i * U + u) * T;
                    const bool live = d < nvec;
                    float t[EPV];
                    if (live) {
                        float g[EPV];
                        V::unpack(row_s[d], t);
                        gamma_of(d, g);
#pragma unroll
                        for (int e = 0; e < EPV; ++e) t[e] *= g[e];
                        if (a.round_product) V::unpack(V::pack(t), t);
                    } else {
#pragma unroll
                        for (int e = 0; e < EPV; ++e) t[e] = 0.0f;
                    }
                    const float bmax = block_max_nonneg<LPB>(abs_max<EPV>(0.0f, t));
                    uint32_t code;
                    float kq;
                    if constexpr (UE8M0) {
                        code = ue8m0_code(bmax * c_scale);
                        kq = ue8m0_factor(c_elem, code);
                    } else {
                        code = e4m3fn_scale_code(bmax * c_scale);
                        const float dv = e4m3fn_decode(code);
                        kq = dv > 0.0f ? c_elem * __builtin_amdgcn_rcpf(dv) : 0.0f;
                    }
                    if (live) {
                        float q[EPV];
#pragma unroll
                        for (int e = 0; e < EPV; ++e) q[e] = t[e] * kq;
                        if constexpr (EPV == 8)
                            store_stream(orow, d, e2m1_x8(q));            // 4 bytes per lane
                        else
                            store_stream(orow, d, (uint16_t)e2m1_x4(q));  // 2 bytes per lane
                        if ((d & (LPB - 1)) == 0) {
                            const int j = d / LPB;  // block index in the row
                            srow[swz ? (j >> 2) * 512 + (j & 3) : j] = (uint8_t)code;
                        }
                    }
                }
            }
        }
        // the LDS row and the reduction slots are rewritten by the next row
        __syncthreads();
    }
}

namespace wide_launch {

// The row's LDS exceeds the default dynamic-LDS limit of a launch: the
// kernel's limit is raised to it first (on the current device, every call).
template <typename InT, bool RESID, int OUT, int BLOCK, bool UE8M0>
hipError_t launch(const FusedArgs& a, int grid_blocks, hipStream_t stream) {
    auto kern = wide_kernel<InT, RESID, OUT, BLOCK, UE8M0>;
    const size_t lds = (size_t)a.nvec * 16;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    int64_t grid = grid_blocks;
    if (grid <= 0) grid = persistent_blocks(reinterpret_cast<const void*>(kern), kWideThreads, lds);
    if (grid > a.rows) grid = a.rows;
    if (grid > INT32_MAX) grid = INT32_MAX;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kWideThreads), lds, stream, a);
    return hipGetLastError();
}

template <typename InT, bool RESID>
hipError_t by_output(const FusedArgs& a, int out, Fp4Format f, int grid, hipStream_t st) {
    if (out == kWideFp8) return launch<InT, RESID, kWideFp8, 16, false>(a, grid, st);
    if (out == kWideFp8Fnuz) return launch<InT, RESID, kWideFp8Fnuz, 16, false>(a, grid, st);
    if (f.block == 32)
        return f.ue8m0 ? launch<InT, RESID, kWideFp4, 32, true>(a, grid, st)
                       : launch<InT, RESID, kWideFp4, 32, false>(a, grid, st);
    return f.ue8m0 ? launch<InT, RESID, kWideFp4, 16, true>(a, grid, st)
                   : launch<InT, RESID, kWideFp4, 16, false>(a, grid, st);
}

}  // namespace wide_launch

// All wide-row variants for one input type (one translation unit each).
template <typename InT>
hipError_t launch_wide_typed(const FusedArgs& a, bool residual, int out, Fp4Format fmt, int grid,
                             hipStream_t stream) {
    return residual ? wide_launch::by_output<InT, true>(a, out, fmt, grid, stream)
                    : wide_launch::by_output<InT, false>(a, out, fmt, grid, stream);
}

}  // namespace rmsq
