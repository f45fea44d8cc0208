// Sum of several input buffers + residual, RMSNorm and per-row dynamic FP8
// quantization, gfx950: the computation Mojo "allreduce_residual_rmsnorm_fp8"
// performs on each GPU once the input buffers are visible to it (Args:
// input_buffers, one per GPU; residual; residual_output = the pre-norm sum;
// output and scale_output as "rms_norm_fused_fp8").  The buffers are plain
// device pointers: local tensors, or peer memory the caller has mapped and
// made ready; this kernel does no communication or signalling.
//
// s = round_to_in_dtype(residual + sum of inputs), the exact sum rounded once:
// the terms are accumulated in fp64 (exact for realistic activations: the
// terms' exponents would have to span more than 53 - p bits to round), and
// the fp64 sum goes to the input type without double rounding (fp32: one
// conversion; 16-bit types: rounded to odd at fp32 precision, then to nearest
// even at 8 / 11 bits, which is exact because fp32 keeps more than two
// extra bits).  s is stored to residual_out and normalized and quantized as
// in the residual FP8 kernel (rmsq_fp8_kernel.h), with the same mapping and
// numerics (the PROD forms of rmsq_device.h): `waves` wavefronts per row, lane l owns the
// 16-byte vectors l, l + T, ...  Rows are adjacent and whole vectors.
#pragma once

#include "rmsq_device.h"
#include "rmsq_internal.h"

namespace rmsq {

// fp64 sum -> the 16-bit type's bits, one rounding: round to odd at fp32
// precision (truncate toward zero, set the last bit if anything was cut),
// then the hardware's round to nearest even to 8 / 11 significant bits.
__device__ __forceinline__ float to_odd_f32(double d) {
    float f = (float)d;
    if ((double)f != d) {
        uint32_t b = __float_as_uint(f);
        if (fabs((double)f) > fabs(d)) b -= 1;  // rounded away from zero: one step back
        f = __uint_as_float(b | 1u);
    }
    return f;
}

template <typename InT>
__device__ __forceinline__ uint4 round_sum(const double (&acc)[Vec<InT>::EPV]) {
    using V = Vec<InT>;
    float f[V::EPV];
#pragma unroll
    for (int e = 0; e < V::EPV; ++e) {
        if constexpr (V::BYTES == 4)
            f[e] = (float)acc[e];
        else
            f[e] = to_odd_f32(acc[e]);
    }
    return V::pack(f);
}

// Waves per SIMD the compiler must leave room for: six for the forms that
// fit 80 VGPRs without spilling (one vector per lane, one row per block, no
// fp64 product, e4m3fn), so that three 8-wave blocks share a CU instead of
// two (8 inputs of 8192 x 4096 bf16: 118.5 -> 115.7 us, A/B in one process,
// outputs identical); the other forms would spill at that budget.
template <int VPT, bool ONE_ROW, int PROD, bool FNUZ>
constexpr int kSumMinWaves = (VPT == 1 && ONE_ROW && PROD != kProdF64 && !FNUZ) ? 6 : 1;

template <typename InT, bool FNUZ, int VPT, bool EXACT, bool ONE_ROW, int PROD>
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(kSumMinWaves<VPT, ONE_ROW, PROD, FNUZ>)))
fp8_sum_kernel(const SumArgs sa) {
    const FusedArgs& a = sa.a;
    using V = Vec<InT>;
    constexpr int EPV = V::EPV;
    constexpr double INV_FMAX = FNUZ ? 1.0 / 240.0 : 1.0 / 448.0;

    const int waves = a.waves;
    const int T = waves * 64;
    const int rpb = ONE_ROW ? 1 : blockDim.x / T;
    const int tid = threadIdx.x;
    const int slot = ONE_ROW ? 0 : tid / T;
    const int lt = tid - slot * T;
    const int red = slot * waves + (lt >> 6);
    const int nvec = a.nvec;
    const int nin = sa.ninputs;
    constexpr int GRP = VPT > 2 ? 4 : 8;  // input vectors loaded together (measured: 8 is 4% faster at 2)
    auto live = [&](int k) { return EXACT || lt + k * T < nvec; };
    const int64_t row_bytes = (int64_t)a.hidden * V::BYTES;
    const double offd = PROD == kProdF64 ? (double)a.weight_offset : 0.0;
    static_assert(PROD != kProdF32 || V::BYTES == 2, "fp32 products are not exact in fp32");
    static_assert(PROD != kProdTwo || V::BYTES == 4, "the two-term form is for fp32 inputs");
    constexpr bool T32 = PROD == kProdF32;  // t = s * g' held in fp32
    constexpr bool HOLD_G = V::BYTES == 2;  // packed gamma held; fp32 gamma from L2 again

    __shared__ double red_sum[2][16];
    __shared__ uint64_t red_max[2][16];

    // one vector per lane: the input buffers' bases, read from the kernel
    // arguments once (the other forms read them per row, which keeps fewer
    // registers live)
    const char* in_base[VPT == 1 ? kMaxSumInputs : 1];
    if constexpr (VPT == 1) {
#pragma unroll
        for (int j = 0; j < kMaxSumInputs; ++j) in_base[j] = static_cast<const char*>(sa.inputs[j < nin ? j : 0]);
    }

    int parity = 0;
    for (int64_t row0 = (int64_t)blockIdx.x * rpb; row0 < a.rows; row0 += (int64_t)gridDim.x * rpb) {
        const int64_t row = row0 + slot;
        const bool active = row < a.rows;

        float t[T32 ? VPT : 1][EPV];   // s * g' (exact in fp32)
        uint4 sv[VPT];                 // the row s (packed); held across the barrier by the other forms
        uint4 gp[T32 ? 1 : VPT];       // packed gamma (the other forms)
        uint4 g1 = make_uint4(0, 0, 0, 0);  // gamma, loaded with the row at one vector per lane
        double ssq0 = 0.0, ssq1 = 0.0;
        float amax32 = 0.0f;
        double amax64 = 0.0;
        if (active) {
            const int64_t off = row * row_bytes;
            // s, vector by vector: the residual's vector, then the inputs'
            // GRP at a time (8 up to 2 vectors per lane, 4 at 4, which keeps
            // the registers bounded), summed in fp64 and rounded once; every
            // load of the row comes before any store (residual_out may be
            // residual).  At one vector per lane every load of the vector --
            // residual, inputs, gamma -- is issued before the first is used
            // (1.3% faster on 8 inputs of 4096 bf16 elements than waiting for
            // the residual first; at 2 and 4 vectors per lane the same order
            // spills registers).
            if constexpr (VPT == 1) {
                sv[0] = make_uint4(0, 0, 0, 0);
                if (live(0)) {
                    const uint32_t voff = (uint32_t)lt * 16u;
                    uint4 iv[kMaxSumInputs];
                    const uint4 rk = load_stream_uniform(static_cast<const char*>(a.residual) + off, voff);
#pragma unroll
                    for (int j = 0; j < kMaxSumInputs; ++j)
                        if (j < nin) iv[j] = load_stream_uniform(in_base[j] + off, voff);
                    g1 = reinterpret_cast<const uint4*>(a.gamma)[lt];
                    float f[EPV];
                    double acc[EPV];
                    V::unpack(rk, f);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) acc[e] = (double)f[e];
#pragma unroll
                    for (int j = 0; j < kMaxSumInputs; ++j) {
                        if (j < nin) {
                            V::unpack(iv[j], f);
#pragma unroll
                            for (int e = 0; e < EPV; ++e) acc[e] += (double)f[e];
                        }
                    }
                    sv[0] = round_sum<InT>(acc);
                }
            }
#pragma unroll
            for (int k = 0; k < (VPT == 1 ? 0 : VPT); ++k) {
                sv[k] = make_uint4(0, 0, 0, 0);
                if (!live(k)) continue;
                const int d = lt + k * T;
                float f[EPV];
                double acc[EPV];
                V::unpack(load_stream(static_cast<const char*>(a.residual) + off, d), f);
#pragma unroll
                for (int e = 0; e < EPV; ++e) acc[e] = (double)f[e];
                for (int g0 = 0; g0 < nin; g0 += GRP) {
                    uint4 iv[GRP];
#pragma unroll
                    for (int j = 0; j < GRP; ++j)
                        if (g0 + j < nin) iv[j] = load_stream(static_cast<const char*>(sa.inputs[g0 + j]) + off, d);
#pragma unroll
                    for (int j = 0; j < GRP; ++j) {
                        if (g0 + j < nin) {
                            V::unpack(iv[j], f);
#pragma unroll
                            for (int e = 0; e < EPV; ++e) acc[e] += (double)f[e];
                        }
                    }
                }
                sv[k] = round_sum<InT>(acc);
            }
            char* ro = static_cast<char*>(a.residual_out) + off;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                if (live(k)) store_stream(ro, lt + k * T, sv[k]);
                // gamma with the row (L2 hits)
                float s[EPV], g[EPV];
                const uint4 gv = VPT == 1 ? g1
                                 : live(k) ? reinterpret_cast<const uint4*>(a.gamma)[lt + k * T]
                                           : make_uint4(0, 0, 0, 0);
                V::unpack(gv, g);
                V::unpack(sv[k], s);
                sumsq64<EPV>(ssq0, ssq1, s);
                if constexpr (!T32) {
                    gp[k] = gv;
#pragma unroll
                    for (int e = 0; e < EPV; ++e) amax64 = fmax(amax64, abs_prod64(s[e], g[e], offd));
                } else {
                    // + weight_offset (0.0f here) as the definition's g + offset: a -0 gamma becomes +0
#pragma unroll
                    for (int e = 0; e < EPV; ++e) t[k][e] = live(k) ? s[e] * (g[e] + a.weight_offset) : 0.0f;
                    amax32 = abs_max<EPV>(amax32, t[k]);
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
            uint8_t* orow = static_cast<uint8_t*>(a.out) + row * (int64_t)a.hidden;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                if (!live(k)) continue;
                float q[EPV];
                if constexpr (T32) {
                    if (split) {
#pragma unroll
                        for (int e = 0; e < EPV; ++e) q[e] = fp8_q1(t[k][e], fr);
                    } else {
#pragma unroll
                        for (int e = 0; e < EPV; ++e) q[e] = (float)((double)t[k][e] * fr.k);
                    }
                } else {
                    float s[EPV], g[EPV];
                    V::unpack(sv[k], s);
                    V::unpack(HOLD_G ? gp[k] : reinterpret_cast<const uint4*>(a.gamma)[lt + k * T], g);
                    if (split) {
#pragma unroll
                        for (int e = 0; e < EPV; ++e) q[e] = fp8_q2(s[e], g[e], fr);
                    } else {
#pragma unroll
                        for (int e = 0; e < EPV; ++e) q[e] = fp8_q64(s[e], g[e], offd, fr);
                    }
                }
                if constexpr (EPV == 8) {
                    uint2 w;
                    w.x = fp8_x4<FNUZ>(q[0], q[1], q[2], q[3]);
                    w.y = fp8_x4<FNUZ>(q[4], q[5], q[6], q[7]);
                    store_stream(orow, lt + k * T, w);
                } else {
                    store_stream(orow, lt + k * T, fp8_x4<FNUZ>(q[0], q[1], q[2], q[3]));
                }
            }
            if (lt == 0) store_scale(a.scales, row, a.scales_dtype, fr.sbits);
        }
    }
}

namespace fp8_sum_launch {

template <typename InT, bool FNUZ, int VPT, int PROD>
hipError_t launch_prod(SumArgs sa, Shape s, hipStream_t stream) {
    FusedArgs& a = sa.a;
    a.waves = s.waves;
    const int64_t groups = (a.rows + s.rpb - 1) / s.rpb;
    // default: one block per row group
    int64_t grid = s.grid > 0 ? s.grid : groups;
    if (grid > groups) grid = groups;
    if (grid > INT32_MAX) grid = INT32_MAX;
    if (grid < 1) grid = 1;
    const dim3 gd((unsigned)grid), bd(s.waves * s.rpb * 64);
    const bool exact = a.nvec == VPT * s.waves * 64;
    if (s.rpb == 1) {
        if (exact)
            hipLaunchKernelGGL((fp8_sum_kernel<InT, FNUZ, VPT, true, true, PROD>), gd, bd, 0, stream, sa);
        else
            hipLaunchKernelGGL((fp8_sum_kernel<InT, FNUZ, VPT, false, true, PROD>), gd, bd, 0, stream, sa);
    } else {
        if (exact)
            hipLaunchKernelGGL((fp8_sum_kernel<InT, FNUZ, VPT, true, false, PROD>), gd, bd, 0, stream, sa);
        else
            hipLaunchKernelGGL((fp8_sum_kernel<InT, FNUZ, VPT, false, false, PROD>), gd, bd, 0, stream, sa);
    }
    return hipGetLastError();
}

// the product form: kProdF32 / kProdTwo without a weight offset, else kProdF64
template <typename InT, bool FNUZ, int VPT>
hipError_t launch_vpt(const SumArgs& sa, Shape s, hipStream_t stream) {
    if (prod_mode<InT>(sa.a.weight_offset) == kProdF64) return launch_prod<InT, FNUZ, VPT, kProdF64>(sa, s, stream);
    return launch_prod<InT, FNUZ, VPT, prod_mode<InT>(0.0f)>(sa, s, stream);
}

template <typename InT, bool FNUZ>
hipError_t by_vpt(const SumArgs& sa, Shape s, hipStream_t st) {
    switch (s.vpt) {
    case 1: return launch_vpt<InT, FNUZ, 1>(sa, s, st);
    case 2: return launch_vpt<InT, FNUZ, 2>(sa, s, st);
    default: return launch_vpt<InT, FNUZ, 4>(sa, s, st);
    }
}

}  // namespace fp8_sum_launch

// All variants for one input type (one translation unit each).
template <typename InT>
hipError_t launch_fp8_sum_typed(const SumArgs& sa, bool fnuz, Shape s, hipStream_t stream) {
    return fnuz ? fp8_sum_launch::by_vpt<InT, true>(sa, s, stream) : fp8_sum_launch::by_vpt<InT, false>(sa, s, stream);
}

}  // namespace rmsq
