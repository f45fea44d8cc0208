// Fused (residual +) RMSNorm + FP8 / FP4 quantization for rows wider than
// the register-resident kernels hold (more than 16 waves x 64 lanes x 4
// vectors = 4096 16-byte vectors: 32768 16-bit or 16384 fp32 elements),
// gfx950.
//
// Operation: that of rmsq_fp8_kernel.h (Mojo docs "rms_norm_fused_fp8",
// per-row scale; the residual form of "allreduce_residual_rmsnorm_fp8") and
// of rmsq_fp4_kernel.h (FlashInfer "rmsnorm_fp4quant.py": E4M3 or UE8M0
// block scales over 16 or 32 elements, row-major or swizzled, optionally the
// page's 16-bit x * w product), with or without the residual.  The sum of
// squares and the steps after it are those of the register kernels: FP8
// accumulates the squares in fp64 and rounds q = s * g' * k once to fp32
// (t = s * g' exact in fp32 for 16-bit inputs without a weight offset, else
// s * g' and its row maximum in fp64); FP4 takes the FP4 kernel's fp32
// element steps.
//
// Work mapping: one 1024-thread block per row (blocks stride over rows);
// lane l owns the 16-byte vectors l, l + 1024, ...  Pass 1 forms s (x, or
// x + residual rounded once to the input type and stored to residual_out)
// and accumulates sum(s^2) and, for FP8, max |s * g'| (g' = gamma +
// weight_offset, read from L2 by the LDS form and from an LDS copy by the
// register form); the block reduces both.  Pass 2 forms
// s * g' again (the same products) and quantizes: FP8 with the
// row's scale, FP4 per block, whose lanes are adjacent as in the FP4 kernel.
// HBM traffic is that of the register kernels: every input element read
// once, every output written once.
//
// Between the passes s is kept in one of two places:
//  - LDS (wide_kernel): the row's vectors in dynamic shared memory, up to
//    158 KiB, read in chunks of U vectors per lane;
//  - registers (wide_reg_kernel): NV packed vectors per lane, the raw
//    16-byte words at 4 VGPRs each (NV = 10, 40 VGPRs, at the widest row),
//    every load of the row in flight at once; the LDS left free holds
//    gamma, copied once per block, so the two passes' gamma reads (twice
//    the row's bytes for 16-bit rows) stay off the L1/L2 path that carries
//    the row (measured: 6-20% faster than reading gamma from L2 on rows of
//    40000-65536 elements, outputs identical).
// Measured on MI355X (A/B in one process, outputs identical): without a
// residual the register form is 10-28% faster whenever the LDS form leaves
// room for only one block per CU (rows above ~80 KiB), and 8% slower on
// rows that let two LDS blocks share a CU; with a residual, whose second
// input doubles the registers in flight, it is faster only up to 6 or 7
// vectors per lane (kResidRegMaxNv).  The launch takes the register form
// where the occupancy API reports one resident LDS block per CU, for rows
// with a residual only up to kResidRegMaxNv vectors per lane.
#pragma once

#include "rmsq_device.h"
#include "rmsq_internal.h"

namespace rmsq {

constexpr int kWideThreads = 1024;

namespace wide_detail {

// g' = gamma + weight_offset for vector d
template <typename InT>
__device__ __forceinline__ void gamma_of(const FusedArgs& a, const uint4* gam, int d, float (&g)[Vec<InT>::EPV]) {
    Vec<InT>::unpack(gam[d], g);
#pragma unroll
    for (int e = 0; e < Vec<InT>::EPV; ++e) g[e] += a.weight_offset;
}

// t = s * g' for vector d of a row
template <typename InT>
__device__ __forceinline__ void product(const FusedArgs& a, const uint4* gam, int d, const uint4& s,
                                        float (&t)[Vec<InT>::EPV]) {
    float g[Vec<InT>::EPV];
    Vec<InT>::unpack(s, t);
    gamma_of<InT>(a, gam, d, g);
#pragma unroll
    for (int e = 0; e < Vec<InT>::EPV; ++e) t[e] *= g[e];
}

// The FP8 product form (rmsq_device.h) for these arguments: uniform, so the
// branches on it are scalar
template <typename InT>
__device__ __forceinline__ int prod_of(const FusedArgs& a) {
    return prod_mode<InT>(a.weight_offset);
}

// Sum of squares and amax over the block (16 waves).  The slots are read
// after the barrier; the caller keeps a later row from rewriting them before
// every wave has read them.
__device__ __forceinline__ void block_reduce(double& ssq, double& amax, bool with_max, double* red_sum,
                                             uint64_t* red_max) {
    const int tid = threadIdx.x;
    ssq = wave_sum(ssq);
    if (with_max) amax = wave_max_nonneg(amax);
    if ((tid & 63) == 0) {
        red_sum[tid >> 6] = ssq;
        red_max[tid >> 6] = __builtin_bit_cast(uint64_t, amax);
    }
    __syncthreads();
    ssq = 0.0;
    uint64_t m = 0;
    for (int w = 0; w < kWideThreads / 64; ++w) {
        ssq += red_sum[w];
        m = max_u64(m, red_max[w]);
    }
    amax = __builtin_bit_cast(double, m);
}

// FP8 codes of vector d (s packed) into the row's output
template <typename InT, bool FNUZ>
__device__ __forceinline__ void fp8_store(const FusedArgs& a, const uint4* gam, uint8_t* orow, int d, const uint4& s,
                                          const Fp8Row& r, bool split) {
    using V = Vec<InT>;
    constexpr int EPV = V::EPV;
    float q[EPV];
    const int prod = prod_of<InT>(a);
    if (prod == kProdF32) {
        float t[EPV];
        product<InT>(a, gam, d, s, t);
        if (split) {
#pragma unroll
            for (int e = 0; e < EPV; ++e) q[e] = fp8_q1(t[e], r);
        } else {
#pragma unroll
            for (int e = 0; e < EPV; ++e) q[e] = (float)((double)t[e] * r.k);
        }
    } else {
        float sf[EPV], g[EPV];
        V::unpack(s, sf);
        V::unpack(gam[d], g);
        if (prod == kProdTwo && split) {
#pragma unroll
            for (int e = 0; e < EPV; ++e) q[e] = fp8_q2(sf[e], g[e], r);
        } else {
            const double offd = (double)a.weight_offset;
#pragma unroll
            for (int e = 0; e < EPV; ++e) q[e] = fp8_q64(sf[e], g[e], offd, r);
        }
    }
    if constexpr (EPV == 8) {
        uint2 w;
        w.x = fp8_x4<FNUZ>(q[0], q[1], q[2], q[3]);
        w.y = fp8_x4<FNUZ>(q[4], q[5], q[6], q[7]);
        store_stream(orow, d, w);
    } else {
        store_stream(orow, d, fp8_x4<FNUZ>(q[0], q[1], q[2], q[3]));
    }
}

// FP4: the row's constants and output places
struct Fp4Row {
    float c_scale;  // E4M3: block scale = bmax * c_scale (gs * rstd / 6)
    float c_elem;   // element factor numerator (gs * rstd)
    uint8_t* orow;  // E2M1 codes
    uint8_t* srow;  // the row's first scale byte
    bool swz;
};

template <int BLOCK>
__device__ __forceinline__ Fp4Row fp4_row(const FusedArgs& a, int64_t row, double rstd) {
    // E4M3: block scale gs * (amax_t * rstd) / 6, element factor
    // gs * rstd / d; UE8M0 (gs = 1): code from amax_t * rstd / 6,
    // element factor rstd * 2^(127 - code)
    const double gs = a.global_scale ? (double)*a.global_scale : 1.0;
    Fp4Row r;
    r.c_scale = (float)(gs * rstd * (1.0 / 6.0));
    r.c_elem = (float)(gs * rstd);
    r.swz = a.sf_swizzled != 0;
    r.orow = static_cast<uint8_t*>(a.out) + row * a.out_stride;
    // this row's scale bytes: row-major, or the row's place in its 128 x 4
    // tiles ((row/128) * K * 512 + (row%32) * 16 + ((row%128)/32) * 4)
    r.srow = static_cast<uint8_t*>(a.scales) +
             (r.swz ? (row >> 7) * ((int64_t)a.sf_k_tiles * 512) + (row & 31) * 16 + ((row & 127) >> 5) * 4
                    : row * (int64_t)(a.hidden / BLOCK));
    return r;
}

// FP4 codes of vector d and, from the block's first lane, its scale byte.
// Every lane of the block calls it (the block maximum is a lane swap): a
// block's lanes are all inside the row or all past it (nvec and the lane
// count are multiples of the lanes per block), and past it (live false)
// t = 0 and nothing is stored.
template <typename InT, int BLOCK, bool UE8M0>
__device__ __forceinline__ void fp4_store(const FusedArgs& a, const uint4* gam, const Fp4Row& r, int d, bool live,
                                          const uint4& s) {
    using V = Vec<InT>;
    constexpr int EPV = V::EPV;
    constexpr int LPB = BLOCK / EPV;  // lanes (vectors) per block
    float t[EPV];
    if (live) {
        product<InT>(a, gam, d, s, t);
        if (a.round_product) V::unpack(V::pack(t), t);
    } else {
#pragma unroll
        for (int e = 0; e < EPV; ++e) t[e] = 0.0f;
    }
    const float bmax = block_max_nonneg<LPB>(abs_max<EPV>(0.0f, t));
    uint32_t code;
    float kq;
    if constexpr (UE8M0) {
        code = ue8m0_code(bmax * r.c_scale);
        kq = ue8m0_factor(r.c_elem, code);
    } else {
        code = e4m3fn_scale_code(bmax * r.c_scale);
        const float dv = e4m3fn_decode(code);
        kq = dv > 0.0f ? r.c_elem * __builtin_amdgcn_rcpf(dv) : 0.0f;
    }
    if (live) {
        float q[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) q[e] = t[e] * kq;
        if constexpr (EPV == 8)
            store_stream(r.orow, d, e2m1_x8(q));            // 4 bytes per lane
        else
            store_stream(r.orow, d, (uint16_t)e2m1_x4(q));  // 2 bytes per lane
        if ((d & (LPB - 1)) == 0) {
            const int j = d / LPB;  // block index in the row
            r.srow[r.swz ? (j >> 2) * 512 + (j & 3) : j] = (uint8_t)code;
        }
    }
}

// Pass 1's per-vector step: s of vector d (x, or x + residual rounded once
// and stored to residual_out), its sum of squares (fp64) and, for FP8, its
// max |s * g'| (exact)
template <typename InT, bool RESID, bool FP8>
__device__ __forceinline__ uint4 form_s(const FusedArgs& a, const uint4* gam, char* ro, int d, const uint4& xv,
                                        const uint4& rv, double& ssq, double& amax) {
    using V = Vec<InT>;
    constexpr int EPV = V::EPV;
    uint4 s = xv;
    if constexpr (RESID) {
        float xf[EPV], rf[EPV];
        V::unpack(xv, xf);
        V::unpack(rv, rf);
#pragma unroll
        for (int e = 0; e < EPV; ++e) xf[e] += rf[e];
        s = V::pack(xf);  // one rounding of the fp32 sum
        store_stream(ro, d, s);
    }
    if constexpr (!FP8) {
        // FP4: fp32 within the vector (v_dot2c on packed 16-bit pairs), as
        // the FP4 register kernel; unpacked floats here would be carried into
        // pass 2 by the compiler and spill the register form
        ssq += (double)V::sumsq(s);
    } else {
        float sf[EPV];
        V::unpack(s, sf);
        double s1 = 0.0;
        sumsq64<EPV>(ssq, s1, sf);
        ssq += s1;
        if (prod_of<InT>(a) != kProdF32) {
            float g[EPV];
            V::unpack(gam[d], g);
            const double offd = (double)a.weight_offset;
#pragma unroll
            for (int e = 0; e < EPV; ++e) amax = fmax(amax, abs_prod64(sf[e], g[e], offd));
        } else {
            float t[EPV];
            product<InT>(a, gam, d, s, t);
            amax = fmax(amax, (double)abs_max<EPV>(0.0f, t));
        }
    }
    return s;
}

}  // namespace wide_detail

// s staged in LDS between the passes (any row up to kMaxWideVec vectors).
template <typename InT, bool RESID, int OUT, int BLOCK, bool UE8M0>
__global__ void __launch_bounds__(1024) wide_kernel(const FusedArgs a) {
    using namespace wide_detail;
    // vectors per lane loaded together in pass 1: 8 with a residual, 4
    // without (measured: 8 is 9-13% faster with a residual; without one the
    // extra registers cost a second resident block on rows that leave LDS
    // room for it, 14% at 40000 elements)
    constexpr int T = kWideThreads, U = RESID ? 8 : 4;
    constexpr bool FP4 = OUT == kWideFp4;
    constexpr bool FNUZ = OUT == kWideFp8Fnuz;

    extern __shared__ uint4 row_s[];  // s of the current row: nvec vectors
    __shared__ double red_sum[16];
    __shared__ uint64_t red_max[16];
    const uint4* gam = static_cast<const uint4*>(a.gamma);  // from L2

    const int tid = threadIdx.x;
    const int nvec = a.nvec;
    const int steps = (nvec + U * T - 1) / (U * T);  // uniform over the block

    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        // ---- pass 1: s into LDS, sum of squares (and FP8's amax) ----
        const char* xr = static_cast<const char*>(a.x) + row * a.x_stride;
        const char* rr = RESID ? static_cast<const char*>(a.residual) + row * a.residual_stride : nullptr;
        char* ro = RESID ? static_cast<char*>(a.residual_out) + row * a.residual_out_stride : nullptr;
        double ssq = 0.0, amax = 0.0;
        for (int i = 0; i < steps; ++i) {
            // chunk i: this lane's vectors tid + (i * U + u) * T.  Every load
            // of a chunk comes before any of its stores (residual_out may be
            // x or residual itself; the lane that reads a vector writes it).
            uint4 xv[U], rv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int d = tid + (i * U + u) * T;
                if (d < nvec) {
                    xv[u] = load_stream(xr, d);
                    if constexpr (RESID) rv[u] = load_stream(rr, d);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int d = tid + (i * U + u) * T;
                if (d < nvec) row_s[d] = form_s<InT, RESID, !FP4>(a, gam, ro, d, xv[u], rv[u], ssq, amax);
            }
        }

        // ---- the row's sums (the barrier also orders the row's LDS writes
        // before pass 2 reads them) ----
        block_reduce(ssq, amax, !FP4, red_sum, red_max);
        const double rstd = rsqrt_refined(ssq * a.inv_hidden + (double)a.eps);

        // ---- pass 2: quantize from LDS ----
        if constexpr (!FP4) {
            const Fp8Row fr = fp8_row(amax, rstd, FNUZ ? 1.0 / 240.0 : 1.0 / 448.0, a.scale_ub, a.scales_dtype);
            const bool split = __builtin_amdgcn_readfirstlane((int)fr.split);  // uniform over the block
            uint8_t* orow = static_cast<uint8_t*>(a.out) + row * a.out_stride;
            for (int i = 0; i < steps; ++i) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int d = tid + (i * U + u) * T;
                    if (d < nvec) fp8_store<InT, FNUZ>(a, gam, orow, d, row_s[d], fr, split);
                }
            }
            if (tid == 0) store_scale(a.scales, row, a.scales_dtype, fr.sbits);
        } else {
            const Fp4Row r = fp4_row<BLOCK>(a, row, rstd);
            for (int i = 0; i < steps; ++i) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int d = tid + (i * U + u) * T;
                    const bool live = d < nvec;
                    fp4_store<InT, BLOCK, UE8M0>(a, gam, r, d, live, live ? row_s[d] : make_uint4(0, 0, 0, 0));
                }
            }
        }
        // the LDS row and the reduction slots are rewritten by the next row
        __syncthreads();
    }
}

// s held in registers between the passes: NV vectors per lane (nvec <=
// NV * 1024).
template <typename InT, bool RESID, int OUT, int BLOCK, bool UE8M0, int NV>
__global__ void __launch_bounds__(1024) wide_reg_kernel(const FusedArgs a) {
    using namespace wide_detail;
    constexpr int T = kWideThreads;
    constexpr bool FP4 = OUT == kWideFp4;
    constexpr bool FNUZ = OUT == kWideFp8Fnuz;

    // two sets of reduction slots, alternating by row: a wave that reaches
    // the next row's barrier has passed this row's, so no wave can still be
    // reading the set it writes; one barrier per row
    __shared__ double red_sum[2][16];
    __shared__ uint64_t red_max[2][16];
    // gamma, copied into LDS once per block (nvec vectors): both passes read
    // it from there instead of from L2
    extern __shared__ uint4 gam[];

    const int tid = threadIdx.x;
    const int nvec = a.nvec;
    for (int d = tid; d < nvec; d += T) gam[d] = static_cast<const uint4*>(a.gamma)[d];
    __syncthreads();
    int set = 0;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x, set ^= 1) {
        // ---- pass 1: the whole row's loads, then s's sums ----
        // every load of the row comes before any store (residual_out may be
        // x or residual itself; the lane that reads a vector writes it)
        const char* xr = static_cast<const char*>(a.x) + row * a.x_stride;
        const char* rr = RESID ? static_cast<const char*>(a.residual) + row * a.residual_stride : nullptr;
        char* ro = RESID ? static_cast<char*>(a.residual_out) + row * a.residual_out_stride : nullptr;
        uint4 sv[NV], rv[RESID ? NV : 1];
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int d = tid + k * T;
            sv[k] = d < nvec ? load_stream(xr, d) : make_uint4(0, 0, 0, 0);
            if constexpr (RESID) rv[k] = d < nvec ? load_stream(rr, d) : make_uint4(0, 0, 0, 0);
        }
        double ssq = 0.0, amax = 0.0;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int d = tid + k * T;
            if (d < nvec) sv[k] = form_s<InT, RESID, !FP4>(a, gam, ro, d, sv[k], rv[RESID ? k : 0], ssq, amax);
        }
        block_reduce(ssq, amax, !FP4, red_sum[set], red_max[set]);
        const double rstd = rsqrt_refined(ssq * a.inv_hidden + (double)a.eps);

        // ---- pass 2: quantize from registers ----
        if constexpr (!FP4) {
            const Fp8Row fr = fp8_row(amax, rstd, FNUZ ? 1.0 / 240.0 : 1.0 / 448.0, a.scale_ub, a.scales_dtype);
            const bool split = __builtin_amdgcn_readfirstlane((int)fr.split);  // uniform over the block
            uint8_t* orow = static_cast<uint8_t*>(a.out) + row * a.out_stride;
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const int d = tid + k * T;
                if (d < nvec) fp8_store<InT, FNUZ>(a, gam, orow, d, sv[k], fr, split);
            }
            if (tid == 0) store_scale(a.scales, row, a.scales_dtype, fr.sbits);
        } else {
            const Fp4Row r = fp4_row<BLOCK>(a, row, rstd);
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const int d = tid + k * T;
                fp4_store<InT, BLOCK, UE8M0>(a, gam, r, d, d < nvec, sv[k]);
            }
        }
    }
}

namespace wide_launch {

inline hipError_t launch_grid(const void* kern, const FusedArgs& a, int grid_blocks, size_t lds,
                              hipStream_t stream) {
    int64_t grid = grid_blocks;
    if (grid <= 0) grid = persistent_blocks(kern, kWideThreads, lds);
    if (grid > a.rows) grid = a.rows;
    if (grid > INT32_MAX) grid = INT32_MAX;
    if (grid < 1) grid = 1;
    void* args[] = {const_cast<FusedArgs*>(&a)};
    return hipLaunchKernel(kern, dim3((unsigned)grid), dim3(kWideThreads), args, lds, stream);
}

// The vectors per lane up to which the register form takes rows with a
// residual (it loads two inputs per vector): measured against the LDS form
// (A/B in one process), 16-bit FP8 rows were 5-9% faster at 5-7 vectors per
// lane and 5% slower at 10, FP4 rows 2-4% faster at 5-6 and 3% slower at 8,
// fp32 FP8 rows 3% faster at 5, even at 6 and 2-6% slower at 7-10.
template <typename InT, int OUT>
constexpr int kResidRegMaxNv = (Vec<InT>::BYTES == 2 && OUT != kWideFp4) ? 7 : 6;

template <typename InT, bool RESID, int OUT, int BLOCK, bool UE8M0>
hipError_t launch_reg(const FusedArgs& a, int grid_blocks, hipStream_t stream) {
    // NV = the vectors per lane the row needs (rows here exceed 4096
    // vectors, so 5 or more), each compiled: rounding NV up costs the
    // registers of the idle slots (measured: 9000-vector rows 13% slower at
    // NV = 10 than at 9); with a residual, NV <= kResidRegMaxNv
    const int nv = (a.nvec + kWideThreads - 1) / kWideThreads;
    const void* kern;
    if constexpr (RESID) {
        kern = nv <= 5   ? reinterpret_cast<const void*>(wide_reg_kernel<InT, true, OUT, BLOCK, UE8M0, 5>)
               : nv <= 6 ? reinterpret_cast<const void*>(wide_reg_kernel<InT, true, OUT, BLOCK, UE8M0, 6>)
                         : reinterpret_cast<const void*>(wide_reg_kernel<InT, true, OUT, BLOCK, UE8M0, 7>);
    } else {
        kern = nv <= 5   ? reinterpret_cast<const void*>(wide_reg_kernel<InT, false, OUT, BLOCK, UE8M0, 5>)
               : nv <= 6 ? reinterpret_cast<const void*>(wide_reg_kernel<InT, false, OUT, BLOCK, UE8M0, 6>)
               : nv <= 7 ? reinterpret_cast<const void*>(wide_reg_kernel<InT, false, OUT, BLOCK, UE8M0, 7>)
               : nv <= 8 ? reinterpret_cast<const void*>(wide_reg_kernel<InT, false, OUT, BLOCK, UE8M0, 8>)
               : nv <= 9 ? reinterpret_cast<const void*>(wide_reg_kernel<InT, false, OUT, BLOCK, UE8M0, 9>)
                         : reinterpret_cast<const void*>(wide_reg_kernel<InT, false, OUT, BLOCK, UE8M0, 10>);
    }
    const size_t lds = (size_t)a.nvec * 16;
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    return launch_grid(kern, a, grid_blocks, lds, stream);
}

// The LDS row exceeds the default dynamic-LDS limit of a launch: the LDS
// kernel's limit is raised to it first (on the current device, every call).
template <typename InT, bool RESID, int OUT, int BLOCK, bool UE8M0>
hipError_t launch(const FusedArgs& a, int grid_blocks, hipStream_t stream) {
    const void* kern = reinterpret_cast<const void*>(wide_kernel<InT, RESID, OUT, BLOCK, UE8M0>);
    const size_t lds = (size_t)a.nvec * 16;
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (blocks_per_cu(kern, kWideThreads, lds) < 2) {
        const int nv = (a.nvec + kWideThreads - 1) / kWideThreads;
        if (!RESID || nv <= kResidRegMaxNv<InT, OUT>)
            return launch_reg<InT, RESID, OUT, BLOCK, UE8M0>(a, grid_blocks, stream);
    }
    return launch_grid(kern, a, grid_blocks, lds, stream);
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
