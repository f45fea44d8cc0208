// Fused RMSNorm + block-scaled FP4 quantization (E2M1 codes, one E4M3 scale
// per 16 contiguous elements), gfx950.
//
// Operation: FlashInfer "rmsnorm_fp4quant.py" (block_size 16, E4M3 scale
// factors, row-major scale layout): per block, scale = min(gs * amax / 6, 448)
// rounded to E4M3, then elements are quantized as y * gs / decoded_scale with
// saturating round-to-nearest-even E2M1.  The page's kernel reads the row
// twice (an async copy for the sum of squares, then again from global memory
// for quantization) and multiplies x * w in 16-bit; here the row is read once
// into VGPRs and every product is fp32.
//
// Work mapping: as the FP8 kernel (WAVES wavefronts per row, lane l owns the
// 16-byte vectors l, l+T, ...).  A vector holds 8 elements, so a 16-element
// block spans the adjacent lanes (2j, 2j+1); they combine their partial amax
// through one DPP lane swap, both compute the block scale, the even lane
// stores the scale byte and each lane stores its own 4 bytes of codes.
#include "rmsq_device.h"
#include "rmsq_internal.h"

namespace rmsq {

template <typename InT, int WAVES, int WPB, int VPT>
__global__ void __launch_bounds__(WPB * 64) fp4_kernel(const FusedArgs a) {
    using V = Vec<InT>;
    constexpr int EPV = 8;
    static_assert(V::EPV == EPV, "FP4 path takes 16-bit inputs");
    constexpr int T = WAVES * 64;
    constexpr int RPB = WPB / WAVES;

    const int tid = threadIdx.x;
    const int slot = tid / T;
    const int lt = tid - slot * T;
    const int wv = lt >> 6;
    const int nvec = a.nvec;  // even: hidden is a multiple of 16
    const int64_t row_bytes = (int64_t)a.hidden * 2;
    const int nblk = a.hidden >> 4;

    __shared__ double red_sum[2][RPB][WAVES];

    const float gs = a.global_scale ? *a.global_scale : 1.0f;

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

        float t[VPT][EPV];
        double ssq = 0.0;
        if (active) {
            const uint4* xr = reinterpret_cast<const uint4*>(static_cast<const char*>(a.x) + row * row_bytes);
            uint4 xv[VPT];
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int v = lt + k * T;
                xv[k] = v < nvec ? xr[v] : make_uint4(0, 0, 0, 0);
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
                for (int e = 0; e < EPV; ++e) t[k][e] = s[e] * g[k][e];
            }
        } else {
#pragma unroll
            for (int k = 0; k < VPT; ++k)
#pragma unroll
                for (int e = 0; e < EPV; ++e) t[k][e] = 0.0f;
        }

        ssq = wave_sum(ssq);
        if constexpr (WAVES > 1) {
            if ((lt & 63) == 0) red_sum[parity][slot][wv] = ssq;
            __syncthreads();
            ssq = 0.0;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) ssq += red_sum[parity][slot][w];
            parity ^= 1;
        }

        const double rstd = 1.0 / sqrt(ssq / (double)a.hidden + (double)a.eps);
        // block scale = gs * (amax_t * rstd) / 6; element factor = gs * rstd / d
        const float c_scale = (float)((double)gs * rstd / 6.0);
        const float c_elem = (float)((double)gs * rstd);

        uint32_t* orow = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(a.out) + row * (int64_t)(a.hidden >> 1));
        uint8_t* srow = static_cast<uint8_t*>(a.scales) + row * (int64_t)nblk;
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int v = lt + k * T;
            float amax = 0.0f;
#pragma unroll
            for (int e = 0; e < EPV; ++e) amax = max_nonneg(amax, fabsf(t[k][e]));
            // all lanes take part in the swap (inactive vectors carry zeros)
            amax = max_nonneg(amax, swap_adjacent_lanes(amax));
            const uint32_t code = e4m3fn_scale_code(amax * c_scale);
            const float d = e4m3fn_decode(code);
            const float kq = d > 0.0f ? c_elem * __builtin_amdgcn_rcpf(d) : 0.0f;
            if (active && v < nvec) {
                float q[EPV];
#pragma unroll
                for (int e = 0; e < EPV; ++e) q[e] = t[k][e] * kq;
                orow[v] = e2m1_x8(q);
                if ((v & 1) == 0) srow[v >> 1] = (uint8_t)code;
            }
        }
    }
}

namespace {

template <typename InT, int WAVES, int VPT>
hipError_t launch_shape(const FusedArgs& a, Shape s, hipStream_t stream) {
    constexpr int WPB = WAVES >= 4 ? WAVES : 4;
    constexpr int RPB = WPB / WAVES;
    auto kern = fp4_kernel<InT, WAVES, WPB, VPT>;
    const int64_t groups = (a.rows + RPB - 1) / RPB;
    int64_t grid = persistent_blocks(reinterpret_cast<const void*>(kern), WPB * 64);
    if (s.grid > 0 && s.grid < grid) grid = s.grid;
    if (grid > groups) grid = groups;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WPB * 64), 0, stream, a);
    return hipGetLastError();
}

template <typename InT, int WAVES>
hipError_t by_vpt(const FusedArgs& a, Shape s, hipStream_t st) {
    switch (s.vpt) {
    case 1: return launch_shape<InT, WAVES, 1>(a, s, st);
    case 2: return launch_shape<InT, WAVES, 2>(a, s, st);
    default: return launch_shape<InT, WAVES, 4>(a, s, st);
    }
}

template <typename InT>
hipError_t by_waves(const FusedArgs& a, Shape s, hipStream_t st) {
    switch (s.waves) {
    case 1: return by_vpt<InT, 1>(a, s, st);
    case 2: return by_vpt<InT, 2>(a, s, st);
    case 4: return by_vpt<InT, 4>(a, s, st);
    case 8: return by_vpt<InT, 8>(a, s, st);
    default: return by_vpt<InT, 16>(a, s, st);
    }
}

}  // namespace

hipError_t launch_fp4(const FusedArgs& a, int in_dtype, Shape s, hipStream_t stream) {
    if (in_dtype == 1) return by_waves<F16>(a, s, stream);
    return by_waves<BF16>(a, s, stream);
}

}  // namespace rmsq
