// Fused RMSNorm + block-scaled FP4 quantization (E2M1 codes, one scale per
// block of 16 or 32 contiguous elements), gfx950.
//
// Operation: FlashInfer "rmsnorm_fp4quant.py".  E4M3 scales (kernel Phase 3):
// scale = min(gs * amax / 6, 448) rounded to E4M3, elements quantized as
// y * gs / decoded_scale.  UE8M0 scales (section "UE8M0 Intrinsics (for
// MXFP4)"): code = exponent of the smallest power of two >= amax / 6, plus
// 127, clamped to [0, 255]; elements quantized as y * 2^(127 - code), zero
// for code 0; no global scale.  E2M1 rounding is RNE with saturation.  Scales
// are stored row-major or in the page's swizzled 128 x 4 tiles.  The page's
// kernel reads the row twice (an async copy for the sum of squares, then
// again from global memory for quantization) and multiplies x * w in 16-bit;
// here the row is read once into VGPRs and every product is fp32.
//
// Inputs: bf16, fp16 or fp32 rows; the residual variant first forms
// s = round_to_input_type(x + r) and writes it to residual_out (the pre-norm
// sum of Mojo "allreduce_residual_rmsnorm_fp8", Args: residual,
// residual_output), then quantizes s.
//
// Work mapping: as the FP8 kernel (`waves` wavefronts per row, lane l owns
// the 16-byte vectors l, l+T, ...; EXACT when the lanes hold the row
// exactly).  A vector holds EPV = 8 (16-bit) or 4 (fp32) elements, so a block
// spans LPB = BLOCK / EPV adjacent lanes (2, 4 or 8); they combine their
// partial amax through DPP lane swaps, all compute the block scale, the
// first lane stores the scale byte and each lane stores its own EPV / 2
// bytes of codes (16-byte stores after an exchange through LDS within the
// wave measured 1-6% slower on MI355X).
// The grid strides over rows, so gamma + weight_offset is unpacked into
// registers once per block, and the row loop is software-pipelined.
#pragma once

#include <algorithm>

#include "rmsq_device.h"
#include "rmsq_internal.h"

namespace rmsq {

// One 16-byte vector of a row quantized to E2M1 with its block's scale:
// t = s * g' (g' = gamma + weight_offset, fp32), optionally rounded once to
// the input type (the page's 16-bit x * w), the block's amax from the
// LPB = BLOCK / EPV lanes holding it (DPP swaps; every lane of the wave takes
// part, vectors past the row being zero), the scale code, the element factor,
// and the codes (EPV / 2 bytes at vector v of the row) and, from the block's
// first lane, its scale byte at sbyte (the caller's place for it: row-major,
// or the 128 x 4 tile slot, fp4_scale_step).
//   E4M3: scale = E4M3(min(gs * amax_t * rstd / 6, 448)) with c_scale =
//   gs * rstd / 6; factor c_elem / decoded scale (c_elem = gs * rstd), 0 for
//   a zero code.  UE8M0 (gs = 1): code from amax_t * rstd / 6, factor
//   rstd * 2^(127 - code).
template <typename InT, int BLOCK, bool UE8M0>
__device__ __forceinline__ uint32_t fp4_codes_vector(const uint4& sv, const float (&g)[Vec<InT>::EPV], bool live, int v,
                                                     float c_scale, float c_elem, bool round_prod, uint8_t* sbyte) {
    using V = Vec<InT>;
    constexpr int EPV = V::EPV;
    constexpr int LPB = BLOCK / EPV;  // lanes (vectors) per block: 2, 4 or 8
    float t[EPV];  // s * g'
    V::unpack(sv, t);
#pragma unroll
    for (int e = 0; e < EPV; ++e) t[e] *= g[e];
    // the page's numerics (optional, uniform): its kernel forms x * w as a
    // 16-bit product, i.e. s * g' rounded once
    if (round_prod) V::unpack(V::pack(t), t);
    const float amax = block_max_nonneg<LPB>(abs_max<EPV>(0.0f, t));
    uint32_t code;
    float kq;
    if constexpr (UE8M0) {
        code = ue8m0_code(amax * c_scale);
        kq = ue8m0_factor(c_elem, code);
    } else {
        code = e4m3fn_scale_code(amax * c_scale);
        const float d = e4m3fn_decode(code);
        kq = d > 0.0f ? c_elem * __builtin_amdgcn_rcpf(d) : 0.0f;
    }
    float q[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) q[e] = t[e] * kq;
    if (live && (v & (LPB - 1)) == 0) *sbyte = (uint8_t)code;
    return EPV == 8 ? e2m1_x8(q) : e2m1_x4(q);  // 4 bytes (2 for fp32 inputs: the low half)
}

// The codes of vector v (the word fp4_codes_vector returned) stored on their
// own: 4 bytes per lane (2 for fp32 inputs).
template <int EPV>
__device__ __forceinline__ void fp4_store_codes(uint8_t* orow, int v, uint32_t cw) {
    if constexpr (EPV == 8)
        store_stream(orow, v, cw);
    else
        store_stream(orow, v, (uint16_t)cw);
}

// Swizzled scales: a 128-byte line of the scale buffer holds the scales of 32
// rows (same row / 128, same (row % 32) / 8).  Blocks go to the 8 XCDs round
// robin and each XCD has its own L2, so in row order a line would be
// assembled from pieces written back by up to 8 L2s.  Logical row index i is
// therefore mapped to a row so that the indices with i % 8 == x (those the
// blocks of XCD x take when the grid is a multiple of 8) are whole 32-row
// groups; indices from perm_rows on (past the last multiple of 256) are not
// remapped.  The map permutes each run of 256 rows.
__device__ __forceinline__ int64_t fp4_row_of(int64_t i, int64_t perm_rows) {
    if (i >= perm_rows) return i;
    const int64_t grp = (i >> 8) * 8 + (i & 7);  // 32-row group
    const int m = (int)((i >> 3) & 31);          // member of the group
    return (grp >> 2) * 128 + (m >> 3) * 32 + (grp & 3) * 8 + (m & 7);
}

// The scale byte of block j of a row: row-major, srow[j]; swizzled,
// srow[(j / 4) * 512 + j % 4].  A lane holds the vectors v0 + k * T (T a
// multiple of 64), whose blocks j0 + k * (T / LPB) advance by a multiple of 4,
// so its scale bytes are sbase + k * step with fp4_scale_base and this step.
__device__ __forceinline__ int fp4_scale_base(int j0, bool swz) { return swz ? (j0 >> 2) * 512 + (j0 & 3) : j0; }
__device__ __forceinline__ int fp4_scale_step(int T, int lpb, bool swz) { return swz ? 128 * (T / lpb) : T / lpb; }

// This row's first scale byte: row-major, or the row's place in its 128 x 4
// tiles ((row/128) * K * 512 + (row%32) * 16 + ((row%128)/32) * 4).
__device__ __forceinline__ uint8_t* fp4_scale_row(const FusedArgs& a, int64_t row, int nblk) {
    return static_cast<uint8_t*>(a.scales) +
           (a.sf_swizzled ? (row >> 7) * ((int64_t)a.sf_k_tiles * 512) + (row & 31) * 16 + ((row & 127) >> 5) * 4
                          : row * (int64_t)nblk);
}

template <typename InT, bool RESID, int VPT, bool EXACT, bool ONE_ROW, int DEPTH, int BLOCK, bool UE8M0>
__global__ void __launch_bounds__(1024) fp4_kernel(const FusedArgs a) {
    using V = Vec<InT>;
    constexpr int EPV = V::EPV;  // elements per 16-byte vector: 8 or 4
    static_assert(BLOCK == 16 || BLOCK == 32, "16- or 32-element blocks");
    constexpr int LPB = BLOCK / EPV;  // lanes (vectors) per block: 2, 4 or 8
    constexpr int RV = RESID ? VPT : 1;

    const int waves = a.waves;
    const int T = waves * 64;
    // ONE_ROW: the block is one row group, so the row index is uniform
    const int rpb = ONE_ROW ? 1 : blockDim.x / T;
    const int tid = threadIdx.x;
    const int slot = ONE_ROW ? 0 : tid / T;
    const int lt = tid - slot * T;
    const int red = slot * waves + (lt >> 6);
    const int nvec = a.nvec;  // a multiple of LPB: hidden is a multiple of BLOCK
    const int nblk = a.hidden / BLOCK;
    const bool swz = a.sf_swizzled != 0;
    const bool round_prod = a.round_product != 0;
    auto live = [&](int k) { return EXACT || lt + k * T < nvec; };

    __shared__ double red_sum[2][16];
    // E4M3 scales only (the API passes no global scale with UE8M0 scales)
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

    // Software pipeline over the rows this block owns: the loads of the next
    // DEPTH - 1 rows are in flight while the current row is reduced and
    // quantized.  DEPTH register buffers rotate (the loop body is unrolled
    // DEPTH times, so buffer indices are compile-time and no row is ever
    // copied between registers).  A lane's vectors past the end of the row are
    // the same on every row: they are zeroed once and never loaded.
    const int64_t stride = (int64_t)gridDim.x * rpb;
    uint4 xb[DEPTH][VPT], rb[DEPTH][RV];
#pragma unroll
    for (int b = 0; b < DEPTH; ++b) {
#pragma unroll
        for (int k = 0; k < VPT; ++k) xb[b][k] = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int k = 0; k < RV; ++k) rb[b][k] = make_uint4(0, 0, 0, 0);
    }
    // swizzled scales: rows remapped so that each XCD writes whole 128-byte
    // scale lines (fp4_row_of)
    const int64_t perm_rows = swz ? (a.rows & ~(int64_t)255) : 0;
    auto row_of = [&](int64_t i) -> int64_t { return fp4_row_of(i, perm_rows); };

    auto fetch = [&](uint4 (&xn)[VPT], uint4 (&rn)[RV], int64_t i) {
        if (i < a.rows) {
            const int64_t row = row_of(i);
            const char* xr = static_cast<const char*>(a.x) + row * a.x_stride;
#pragma unroll
            for (int k = 0; k < VPT; ++k)
                if (live(k)) xn[k] = load_stream(xr, lt + k * T);
            if constexpr (RESID) {
                const char* rr = static_cast<const char*>(a.residual) + row * a.residual_stride;
#pragma unroll
                for (int k = 0; k < VPT; ++k)
                    if (live(k)) rn[k] = load_stream(rr, lt + k * T);
            }
        }
    };

    int parity = 0;
    // One row group: (residual add,) reduce, then quantize.  Every wave of the
    // block calls this for the same row0 (the barrier inside is uniform).
    auto process = [&](const uint4 (&xv)[VPT], const uint4 (&rv)[RV], int64_t row0) {
        const bool active = row0 + slot < a.rows;
        const int64_t row = row_of(row0 + slot);

        uint4 sv[VPT];  // the row that is normalized
        double ssq = 0.0;
        if (active) {
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                if constexpr (RESID) {
                    // one rounding of the fp32 sum to the element type (fp32
                    // holds a 16-bit sum exactly; fp32 inputs round once);
                    // residual_out may be x or residual itself: the lane that
                    // read a vector is the one that writes it
                    float xf[EPV], rf[EPV];
                    V::unpack(xv[k], xf);
                    V::unpack(rv[k], rf);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) xf[e] += rf[e];
                    sv[k] = V::pack(xf);
                    if (live(k))
                        store_stream(static_cast<char*>(a.residual_out) + row * a.residual_out_stride, lt + k * T, sv[k]);
                } else {
                    sv[k] = xv[k];
                }
                ssq += (double)V::sumsq(sv[k]);
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
        // wave: every lane of a wave that reaches the lane swaps below is live.
        if (active) {
            const double rstd = rsqrt_refined(ssq * a.inv_hidden + (double)a.eps);
            // E4M3: block scale = gs * (amax_t * rstd) / 6, element factor
            // gs * rstd / d.  UE8M0 (gs = 1): code from amax_t * rstd / 6,
            // element factor rstd * 2^(127 - code).
            const float c_scale = (float)(gs * rstd * (1.0 / 6.0));
            const float c_elem = (float)(gs * rstd);

            uint8_t* orow = static_cast<uint8_t*>(a.out) + row * a.out_stride;
            uint8_t* sbase = fp4_scale_row(a, row, nblk) + fp4_scale_base(lt / LPB, swz);
            const int sstep = fp4_scale_step(T, LPB, swz);
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const uint32_t cw = fp4_codes_vector<InT, BLOCK, UE8M0>(sv[k], g[k], live(k), lt + k * T, c_scale,
                                                                        c_elem, round_prod, sbase + k * sstep);
                if (live(k)) fp4_store_codes<EPV>(orow, lt + k * T, cw);
            }
        }
    };

    int64_t row0 = (int64_t)blockIdx.x * rpb;
#pragma unroll
    for (int b = 0; b + 1 < DEPTH; ++b) fetch(xb[b], rb[b], row0 + b * stride + slot);
    while (row0 < a.rows) {
#pragma unroll
        for (int b = 0; b < DEPTH; ++b) {
            fetch(xb[(b + DEPTH - 1) % DEPTH], rb[(b + DEPTH - 1) % DEPTH], row0 + (DEPTH - 1) * stride + slot);
            process(xb[b], rb[b], row0);
            row0 += stride;
            if (row0 >= a.rows) break;
        }
    }
}

namespace fp4_launch {

// Rows in flight per block: the current one and the next (three measured no
// faster on MI355X and costs 16 more VGPRs at four vectors per lane).  The
// residual variant holds two inputs per row, and two rows of both exceed the
// 128 VGPRs a 1024-thread block allows at four vectors per lane, so it keeps
// one row (as the FP8 kernel, which streams at the same rate without it).
template <bool RESID>
constexpr int kDepth = RESID ? 1 : 2;

template <typename InT, bool RESID, int VPT, bool EXACT, bool ONE_ROW, int BLOCK, bool UE8M0>
hipError_t launch_kernel(const FusedArgs& a, Shape s, hipStream_t stream) {
    auto kern = fp4_kernel<InT, RESID, VPT, EXACT, ONE_ROW, kDepth<RESID>, BLOCK, UE8M0>;
    const int threads = s.waves * s.rpb * 64;
    const int64_t groups = (a.rows + s.rpb - 1) / s.rpb;
    // default: at most 4 row groups per block (MI355X streams this kernel best
    // that way), and at least one block per resident slot while rows last
    int64_t grid = s.grid;
    if (grid <= 0) {
        const int64_t resident = persistent_blocks(reinterpret_cast<const void*>(kern), threads);
        grid = std::max(std::min(groups, resident), (groups + 3) / 4);
    }
    if (grid > groups) grid = groups;
    if (grid > INT32_MAX) grid = INT32_MAX;
    // swizzled scales: a multiple of 8 blocks keeps each XCD on its own rows
    if (a.sf_swizzled && grid >= 8) grid &= ~(int64_t)7;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), 0, stream, a);
    return hipGetLastError();
}

template <typename InT, bool RESID, int VPT, int BLOCK, bool UE8M0>
hipError_t launch_vpt(FusedArgs a, Shape s, hipStream_t stream) {
    a.waves = s.waves;
    const bool exact = a.nvec == VPT * s.waves * 64;
    if (s.rpb == 1)
        return exact ? launch_kernel<InT, RESID, VPT, true, true, BLOCK, UE8M0>(a, s, stream)
                     : launch_kernel<InT, RESID, VPT, false, true, BLOCK, UE8M0>(a, s, stream);
    return exact ? launch_kernel<InT, RESID, VPT, true, false, BLOCK, UE8M0>(a, s, stream)
                 : launch_kernel<InT, RESID, VPT, false, false, BLOCK, UE8M0>(a, s, stream);
}

template <typename InT, bool RESID, int BLOCK, bool UE8M0>
hipError_t by_vpt(const FusedArgs& a, Shape s, hipStream_t st) {
    switch (s.vpt) {
    case 1: return launch_vpt<InT, RESID, 1, BLOCK, UE8M0>(a, s, st);
    case 2: return launch_vpt<InT, RESID, 2, BLOCK, UE8M0>(a, s, st);
    default: return launch_vpt<InT, RESID, 4, BLOCK, UE8M0>(a, s, st);
    }
}

template <typename InT, bool RESID>
hipError_t by_format(const FusedArgs& a, Fp4Format f, Shape s, hipStream_t st) {
    if (f.block == 32)
        return f.ue8m0 ? by_vpt<InT, RESID, 32, true>(a, s, st) : by_vpt<InT, RESID, 32, false>(a, s, st);
    return f.ue8m0 ? by_vpt<InT, RESID, 16, true>(a, s, st) : by_vpt<InT, RESID, 16, false>(a, s, st);
}

}  // namespace fp4_launch

// All FP4 variants for one input type (instantiated once per type, each in
// its own translation unit so they compile in parallel).
template <typename InT>
hipError_t launch_fp4_typed(const FusedArgs& a, bool residual, Fp4Format fmt, Shape s, hipStream_t stream) {
    return residual ? fp4_launch::by_format<InT, true>(a, fmt, s, stream)
                    : fp4_launch::by_format<InT, false>(a, fmt, s, stream);
}

}  // namespace rmsq
