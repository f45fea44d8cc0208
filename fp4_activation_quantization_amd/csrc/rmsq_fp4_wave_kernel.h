// FP4 (E2M1 codes + block scales) for 16-bit rows without a residual on large
// batches: one wavefront per row, gfx950.
//
// Operation: that of rmsq_fp4_kernel.h (FlashInfer "rmsnorm_fp4quant.py"),
// with the same per-vector steps (fp4_codes_vector) and the same row
// reduction (v_dot2c within a vector, fp64 across vectors and lanes).
//
// Work mapping: each wavefront of a 4-wavefront block owns whole rows; lane l
// holds the row's 16-byte vectors l, l + 64, ..., l + 64 * (VPT - 1) (VPT 8 or
// 12: rows of up to 768 vectors, 6144 elements).  Every load of the row is in
// flight at once, the row's sum of squares is reduced inside the wavefront
// (DPP and readlane, no barrier and no LDS round trip per row), and the
// wavefronts of a block run their rows independently.  gamma + weight_offset
// is unpacked to fp32 once per block into LDS (the row's registers leave no
// room for it) and read back per row, 16 bytes per lane, conflict-free.  The
// grid is persistent: logical row i = k * (grid * 4) + wave * grid + block, so
// the rows in flight form one compact window and, with a grid that is a
// multiple of 8, the blocks of one XCD take the indices i with i % 8 equal to
// that XCD (the swizzled layout's row map relies on it, fp4_row_of).
//
// Measured on MI355X (A/B in one process against the block kernel): see the
// launch shape note in rmsq_api.cpp (choose_shape).
#pragma once

#include "rmsq_fp4_kernel.h"

namespace rmsq {

constexpr int kWaveRowThreads = 256;  // 4 wavefronts, each with rows of its own

template <typename InT, int VPT, bool EXACT, int BLOCK, bool UE8M0>
__global__ void __launch_bounds__(kWaveRowThreads) fp4_wave_kernel(const FusedArgs a) {
    using V = Vec<InT>;
    constexpr int EPV = V::EPV;
    static_assert(EPV == 8, "16-bit inputs");
    const int lane = threadIdx.x & 63;
    // the wavefront index is uniform over the wave: made so for the compiler,
    // the row index and every row pointer are scalar (SGPR bases, one lane
    // offset in a VGPR)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    const int nvec = a.nvec;  // a multiple of the lanes per block: hidden is a multiple of BLOCK
    const int nblk = a.hidden / BLOCK;
    const bool swz = a.sf_swizzled != 0;
    const bool round_prod = a.round_product != 0;
    constexpr int LPB = BLOCK / EPV;
    const int sstep = fp4_scale_step(64, LPB, swz);
    auto live = [&](int k) { return EXACT || lane + 64 * k < nvec; };

    // gamma + weight_offset in fp32: elements 0-3 of vector v at g_lds[v],
    // 4-7 at g_lds[nvec + v] (2 * nvec * 16 bytes of dynamic LDS)
    extern __shared__ float4 g_lds[];
    for (int v = threadIdx.x; v < nvec; v += blockDim.x) {
        float g[EPV];
        V::unpack(reinterpret_cast<const uint4*>(a.gamma)[v], g);
#pragma unroll
        for (int e = 0; e < EPV; ++e) g[e] += a.weight_offset;
        g_lds[v] = make_float4(g[0], g[1], g[2], g[3]);
        g_lds[nvec + v] = make_float4(g[4], g[5], g[6], g[7]);
    }
    __syncthreads();  // the only barrier: gamma is read-only from here on

    // E4M3 scales only (the API passes no global scale with UE8M0 scales)
    const double gs = a.global_scale ? (double)*a.global_scale : 1.0;
    const int64_t perm_rows = swz ? (a.rows & ~(int64_t)255) : 0;
    const int64_t step = (int64_t)gridDim.x * nw;
    for (int64_t i = (int64_t)wave * gridDim.x + blockIdx.x; i < a.rows; i += step) {  // uniform per wave
        const int64_t row = fp4_row_of(i, perm_rows);
        const char* xr = static_cast<const char*>(a.x) + row * a.x_stride;
        uint4 xv[VPT];  // vectors past the row are zero
#pragma unroll
        for (int k = 0; k < VPT; ++k) xv[k] = live(k) ? load_stream(xr, lane + 64 * k) : make_uint4(0, 0, 0, 0);
        double ssq = 0.0;
#pragma unroll
        for (int k = 0; k < VPT; ++k) ssq += (double)V::sumsq(xv[k]);
        ssq = wave_sum(ssq);
        const double rstd = rsqrt_refined(ssq * a.inv_hidden + (double)a.eps);
        const float c_scale = (float)(gs * rstd * (1.0 / 6.0));
        const float c_elem = (float)(gs * rstd);
        uint8_t* orow = static_cast<uint8_t*>(a.out) + row * a.out_stride;
        uint8_t* sbase = fp4_scale_row(a, row, nblk) + fp4_scale_base(lane / LPB, swz);
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int v = lane + 64 * k;
            float g[EPV];
            if (live(k)) {
                const float4 lo = g_lds[v], hi = g_lds[nvec + v];
                g[0] = lo.x, g[1] = lo.y, g[2] = lo.z, g[3] = lo.w;
                g[4] = hi.x, g[5] = hi.y, g[6] = hi.z, g[7] = hi.w;
            } else {
#pragma unroll
                for (int e = 0; e < EPV; ++e) g[e] = 0.0f;
            }
            const uint32_t cw =
                fp4_codes_vector<InT, BLOCK, UE8M0>(xv[k], g, live(k), v, c_scale, c_elem, round_prod, sbase + k * sstep);
            if (live(k)) fp4_store_codes<EPV>(orow, v, cw);
            // one vector at a time: without this fence the compiler hoists
            // every vector's gamma reads and products ahead of the first
            // stores (211 VGPRs instead of 100 at 14 vectors per lane)
            asm volatile("" ::: "memory");
        }
    }
}

namespace fp4_wave_launch {

template <typename InT, int VPT, int BLOCK, bool UE8M0>
hipError_t launch_vpt(FusedArgs a, Shape s, hipStream_t stream) {
    a.waves = 1;
    const bool exact = a.nvec == VPT * 64;
    const void* kern = exact ? reinterpret_cast<const void*>(fp4_wave_kernel<InT, VPT, true, BLOCK, UE8M0>)
                             : reinterpret_cast<const void*>(fp4_wave_kernel<InT, VPT, false, BLOCK, UE8M0>);
    const size_t lds = (size_t)a.nvec * 32;
    const int64_t groups = (a.rows + kWaveRowThreads / 64 - 1) / (kWaveRowThreads / 64);
    int64_t grid = s.grid > 0 ? s.grid : persistent_blocks(kern, kWaveRowThreads, lds);
    if (grid > groups) grid = groups;
    if (grid > INT32_MAX) grid = INT32_MAX;
    if (grid >= 8) grid &= ~(int64_t)7;  // each XCD's blocks take the indices of its residue (swizzled rows)
    if (grid < 1) grid = 1;
    void* args[] = {&a};
    return hipLaunchKernel(kern, dim3((unsigned)grid), dim3(kWaveRowThreads), args, lds, stream);
}

// s.vpt: vectors per lane, one of kWaveRowVpt (rmsq_internal.h)
template <typename InT, int BLOCK, bool UE8M0>
hipError_t by_vpt(const FusedArgs& a, Shape s, hipStream_t st) {
    switch (s.vpt) {
    case 8: return launch_vpt<InT, 8, BLOCK, UE8M0>(a, s, st);
    default: return launch_vpt<InT, 12, BLOCK, UE8M0>(a, s, st);
    }
}

}  // namespace fp4_wave_launch

// The wave-per-row FP4 kernel for one 16-bit input type, every block size and
// scale format.
template <typename InT>
hipError_t launch_fp4_wave_typed(const FusedArgs& a, Fp4Format f, Shape s, hipStream_t stream) {
    using namespace fp4_wave_launch;
    if (f.block == 32) return f.ue8m0 ? by_vpt<InT, 32, true>(a, s, stream) : by_vpt<InT, 32, false>(a, s, stream);
    return f.ue8m0 ? by_vpt<InT, 16, true>(a, s, stream) : by_vpt<InT, 16, false>(a, s, stream);
}

}  // namespace rmsq
