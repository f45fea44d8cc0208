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
// Work mapping: as the FP8 kernel (`waves` wavefronts per row, lane l owns
// the 16-byte vectors l, l+T, ...; EXACT when the lanes hold the row
// exactly).  A vector holds 8 elements, so a 16-element block spans the
// adjacent lanes (2j, 2j+1); they combine their partial amax through one DPP
// lane swap, both compute the block scale, the even lane stores the scale
// byte and each lane stores its own 4 bytes of codes.  The grid is persistent
// (one block per resident slot), so gamma + weight_offset is unpacked into
// registers once per block: this path is close to the VALU limit at HBM rate.
#include "rmsq_device.h"
#include "rmsq_internal.h"

namespace rmsq {

template <typename InT, int VPT, bool EXACT>
__global__ void __launch_bounds__(1024) fp4_kernel(const FusedArgs a) {
    using V = Vec<InT>;
    constexpr int EPV = 8;
    static_assert(V::EPV == EPV, "FP4 path takes 16-bit inputs");

    const int waves = a.waves;
    const int T = waves * 64;
    const int rpb = blockDim.x / T;
    const int tid = threadIdx.x;
    const int slot = tid / T;
    const int lt = tid - slot * T;
    const int red = slot * waves + (lt >> 6);
    const int nvec = a.nvec;  // even: hidden is a multiple of 16
    const int64_t row_bytes = (int64_t)a.hidden * 2;
    const int nblk = a.hidden >> 4;
    auto live = [&](int k) { return EXACT || lt + k * T < nvec; };

    __shared__ double red_sum[2][16];

    const double gs = a.global_scale ? (double)*a.global_scale : 1.0;

    float g[VPT][EPV];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        if (live(k)) {
            V::unpack(reinterpret_cast<const uint4*>(a.gamma)[lt + k * T], g[k]);
#pragma unroll
            for (int e = 0; e < EPV; ++e) g[k][e] += a.weight_offset;
        } else {
#pragma unroll
            for (int e = 0; e < EPV; ++e) g[k][e] = 0.0f;
        }
    }

    // Software pipeline over the rows this block owns: the next row's loads are
    // issued before the current row is reduced and quantized, so every block
    // keeps a row's worth of reads in flight while it computes.
    const int64_t stride = (int64_t)gridDim.x * rpb;
    uint4 xn[VPT];  // the next row (zero past the end of the row)
    auto fetch = [&](int64_t r) {
        const char* xr = static_cast<const char*>(a.x) + r * row_bytes;
#pragma unroll
        for (int k = 0; k < VPT; ++k) xn[k] = live(k) ? load_stream(xr, lt + k * T) : make_uint4(0, 0, 0, 0);
    };
    if ((int64_t)blockIdx.x * rpb + slot < a.rows) fetch((int64_t)blockIdx.x * rpb + slot);

    int parity = 0;
    for (int64_t row0 = (int64_t)blockIdx.x * rpb; row0 < a.rows; row0 += stride) {
        const int64_t row = row0 + slot;
        const bool active = row < a.rows;

        float t[VPT][EPV];
        double ssq = 0.0;
        if (active) {
            uint4 xv[VPT];
#pragma unroll
            for (int k = 0; k < VPT; ++k) xv[k] = xn[k];
            if (row + stride < a.rows) fetch(row + stride);
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                ssq += (double)V::sumsq(xv[k]);
                float s[EPV];
                V::unpack(xv[k], s);
#pragma unroll
                for (int e = 0; e < EPV; ++e) t[k][e] = s[e] * g[k][e];
            }
        }

        ssq = wave_sum(ssq);
        if (waves > 1) {  // uniform over the block
            if ((lt & 63) == 0) red_sum[parity][red] = ssq;
            __syncthreads();
            ssq = 0.0;
            for (int w = 0; w < waves; ++w) ssq += red_sum[parity][slot * waves + w];
            parity ^= 1;
        }

        // A row's lanes are whole wavefronts, so `active` is uniform within a
        // wave: every lane of a wave that reaches the lane swap below is live.
        if (active) {
            const double rstd = rsqrt_refined(ssq * a.inv_hidden + (double)a.eps);
            // block scale = gs * (amax_t * rstd) / 6; element factor = gs * rstd / d
            const float c_scale = (float)(gs * rstd * (1.0 / 6.0));
            const float c_elem = (float)(gs * rstd);

            uint8_t* orow = static_cast<uint8_t*>(a.out) + row * (int64_t)(a.hidden >> 1);
            uint8_t* srow = static_cast<uint8_t*>(a.scales) + row * (int64_t)nblk;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int v = lt + k * T;
                // all lanes take part in the swap (vectors past the row are zero)
                const float amax = pair_max_nonneg(abs_max<EPV>(0.0f, t[k]));
                const uint32_t code = e4m3fn_scale_code(amax * c_scale);
                const float d = e4m3fn_decode(code);
                const float kq = d > 0.0f ? c_elem * __builtin_amdgcn_rcpf(d) : 0.0f;
                if (live(k)) {
                    float q[EPV];
#pragma unroll
                    for (int e = 0; e < EPV; ++e) q[e] = t[k][e] * kq;
                    store_stream(orow, v, e2m1_x8(q));
                    if ((v & 1) == 0) srow[v >> 1] = (uint8_t)code;
                }
            }
        }
    }
}

namespace {

template <typename InT, int VPT, bool EXACT>
hipError_t launch_kernel(const FusedArgs& a, Shape s, hipStream_t stream) {
    auto kern = fp4_kernel<InT, VPT, EXACT>;
    const int threads = s.waves * s.rpb * 64;
    const int64_t groups = (a.rows + s.rpb - 1) / s.rpb;
    // default: persistent, one block per resident slot
    int64_t grid = s.grid > 0 ? s.grid : (int64_t)persistent_blocks(reinterpret_cast<const void*>(kern), threads);
    if (grid > groups) grid = groups;
    if (grid > INT32_MAX) grid = INT32_MAX;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), 0, stream, a);
    return hipGetLastError();
}

template <typename InT, int VPT>
hipError_t launch_vpt(FusedArgs a, Shape s, hipStream_t stream) {
    a.waves = s.waves;
    if (a.nvec == VPT * s.waves * 64) return launch_kernel<InT, VPT, true>(a, s, stream);
    return launch_kernel<InT, VPT, false>(a, s, stream);
}

template <typename InT>
hipError_t by_vpt(const FusedArgs& a, Shape s, hipStream_t st) {
    switch (s.vpt) {
    case 1: return launch_vpt<InT, 1>(a, s, st);
    case 2: return launch_vpt<InT, 2>(a, s, st);
    default: return launch_vpt<InT, 4>(a, s, st);
    }
}

}  // namespace

hipError_t launch_fp4(const FusedArgs& a, int in_dtype, Shape s, hipStream_t stream) {
    if (in_dtype == 1) return by_vpt<F16>(a, s, stream);
    return by_vpt<BF16>(a, s, stream);
}

}  // namespace rmsq
