// Fused (residual +) RMSNorm + per-row dynamic FP8 quantization for rows that
// are not whole 16-byte vectors but all sit at a common offset ("phase") from
// the 16-byte grid: a hidden size that is not a multiple of the vector width
// (8 16-bit or 4 fp32 elements) in contiguous tensors, or tensors that all
// start the same number of elements past a 16-byte boundary.  gfx950.
//
// Operation: as the vector kernel (rmsq_fp8_kernel.h): Mojo docs
// "rms_norm_fused_fp8" and the local share of
// "allreduce_residual_rmsnorm_fp8".  Their input_fn is generic in its SIMD
// width, so a row need not be a whole number of vectors.
//
// Work mapping: a row whose first element lies h elements past a 16-byte
// boundary has a head of EPV - h elements (none for h = 0) before the next
// boundary; the first lanes of the row group take one head element each
// (element loads and stores).  From the boundary on, the row is the vector
// kernel's: lane l owns the aligned vectors l, l + T, ..., all whole but the
// last, whose bytes past the row are zeroed after the load (the aligned 16
// bytes around an element of the row never leave its page, so the load
// cannot fault) and whose own elements are stored one by one, so rows that
// share a vector never write each other's elements.  A row thus needs the
// lanes of a ceil(hidden / EPV)-vector row, like an aligned one.  Codes and
// residual_out are stored 8 / 16 bytes at a time: the host takes this kernel
// only when every tensor has x's phase (codes: the same offset modulo the
// code bytes of a vector).  gamma' for a vector starts `head` elements into
// gamma's aligned vector d and runs into d + 1 (both L2 hits; taking d + 1
// from the next lane through ds_bpermute instead measured 2-4% slower); the
// window is cut with byte funnel shifts (v_alignbyte_b32) chosen by a switch
// on the head, which is uniform over the wavefronts of a row.
//
// Precision: as the vector kernel (the PROD forms of rmsq_device.h): s^2
// accumulated in fp64, s * g' and its row maximum exact, and q = s * g' * k
// rounded once to fp32.  Held across the barrier: t = s * g' (kProdF32), or
// the row and its gamma window, packed.
#pragma once

#include "rmsq_device.h"
#include "rmsq_elem.h"
#include "rmsq_internal.h"

namespace rmsq {

// The low `hi` bytes of a 16-byte vector kept, the others zeroed.
__device__ __forceinline__ uint32_t dword_keep_low(int hi, int w) {
    const int b = min(max(hi - 4 * w, 0), 4);
    return b == 4 ? 0xFFFFFFFFu : (1u << (8 * b)) - 1u;
}
__device__ __forceinline__ uint4 keep_low_bytes(uint4 v, int hi) {
    v.x &= dword_keep_low(hi, 0);
    v.y &= dword_keep_low(hi, 1);
    v.z &= dword_keep_low(hi, 2);
    v.w &= dword_keep_low(hi, 3);
    return v;
}

// The 16 bytes starting OFF bytes into the 32-byte concatenation p | c.
template <int OFF>
__device__ __forceinline__ uint4 window_at(const uint4& p, const uint4& c) {
    const uint32_t w[8] = {p.x, p.y, p.z, p.w, c.x, c.y, c.z, c.w};
    constexpr int q = OFF / 4, r = OFF % 4;
    if constexpr (r == 0) {
        return make_uint4(w[q], w[q + 1], w[q + 2], w[q + 3]);
    } else {
        return make_uint4(__builtin_amdgcn_alignbyte(w[q + 1], w[q], r), __builtin_amdgcn_alignbyte(w[q + 2], w[q + 1], r),
                          __builtin_amdgcn_alignbyte(w[q + 3], w[q + 2], r), __builtin_amdgcn_alignbyte(w[q + 4], w[q + 3], r));
    }
}

// Elements s .. s + EPV - 1 of p | c (elements of ESZ bytes), 0 <= s < EPV.
template <int ESZ>
__device__ __forceinline__ uint4 window_from(const uint4& p, const uint4& c, int s) {
    if constexpr (ESZ == 2) {
        switch (s) {
        case 0: return p;
        case 1: return window_at<2>(p, c);
        case 2: return window_at<4>(p, c);
        case 3: return window_at<6>(p, c);
        case 4: return window_at<8>(p, c);
        case 5: return window_at<10>(p, c);
        case 6: return window_at<12>(p, c);
        default: return window_at<14>(p, c);
        }
    } else {
        switch (s) {
        case 0: return p;
        case 1: return window_at<4>(p, c);
        case 2: return window_at<8>(p, c);
        default: return window_at<12>(p, c);
        }
    }
}

template <typename InT, bool RESID, bool FNUZ, int VPT, bool ONE_ROW, int PROD>
__global__ void __launch_bounds__(1024) fp8_phased_kernel(const FusedArgs a) {
    using V = Vec<InT>;
    using E = Elem<InT>;
    using Bits = typename E::Bits;
    constexpr int EPV = V::EPV;    // elements per 16-byte vector
    constexpr int ESZ = V::BYTES;  // bytes per element
    constexpr double INV_FMAX = FNUZ ? 1.0 / 240.0 : 1.0 / 448.0;

    const int waves = a.waves;
    const int T = waves * 64;
    const int rpb = ONE_ROW ? 1 : blockDim.x / T;
    const int tid = threadIdx.x;
    const int slot = ONE_ROW ? 0 : tid / T;
    const int lt = tid - slot * T;
    const int red = slot * waves + (lt >> 6);
    const int hidden = a.hidden;
    const int ngv = (hidden + EPV - 1) / EPV;  // gamma's vectors (gamma is 16-byte aligned)

    const uint4* gv = static_cast<const uint4*>(a.gamma);
    const double offd = PROD == kProdF64 ? (double)a.weight_offset : 0.0;
    constexpr bool T32 = PROD == kProdF32;  // t = s * g' (exact in fp32) held

    __shared__ double red_sum[2][16];
    __shared__ uint64_t red_max[2][16];  // bits of each wave's (non-negative fp64) max |s * g'|

    int parity = 0;
    // Adjacent rows share the 16-byte block at their boundary (one's last
    // vector, the other's head).  Blocks go to the 8 XCDs round robin, each
    // with its own L2, so the logical index i = row0 + slot is mapped to a
    // row such that every XCD takes runs of 8 adjacent rows of each 64-row
    // window (i % 8 picks the run, i / 8 % 8 the row in it; rows past the
    // last whole window keep their index).  Measured 1-2.5% faster.
    const int64_t full = a.rows & ~(int64_t)63;
    for (int64_t row0 = (int64_t)blockIdx.x * rpb; row0 < a.rows; row0 += (int64_t)gridDim.x * rpb) {
        const int64_t li = row0 + slot;
        const int64_t row = li >= full ? li : ((li >> 6) * 8 + (li & 7)) * 8 + ((li >> 3) & 7);
        const bool active = li < a.rows;

        // the row's head (elements before its first 16-byte boundary) and
        // the aligned vectors from there on: all whole but the last, which
        // holds `tail` of the row's elements
        const char* xr = static_cast<const char*>(a.x) + row * a.x_stride;
        const int h = (int)((reinterpret_cast<uintptr_t>(xr) & 15) / ESZ);
        const int head = min(h != 0 ? EPV - h : 0, hidden);
        const int nv = (hidden - head + EPV - 1) / EPV;
        const int tail = hidden - head - (nv - 1) * EPV;
        auto whole = [&](int d) { return d != nv - 1 || tail == EPV; };

        uint4 xv[VPT];              // s (zero outside the row), packed
        uint4 gw[T32 ? 1 : VPT];    // gamma's window for each vector (zero outside the row)
        float t[T32 ? VPT : 1][EPV];  // s * g' (T32)
        float hs = 0.0f;    // the head element's s (lanes lt < head)
        Bits hg = 0;        // and its gamma
        double ssq0 = 0.0, ssq1 = 0.0;
        double amax = 0.0;
        if (active) {
            const char* xb = xr + head * ESZ;  // 16-byte aligned
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int d = lt + k * T;
                xv[k] = d < nv ? load_stream(xb, d) : make_uint4(0, 0, 0, 0);
            }
            Bits hx = 0, hr = 0;
            if (lt < head) {
                hx = load_elem(reinterpret_cast<const Bits*>(xr) + lt);
                hg = static_cast<const Bits*>(a.gamma)[lt];
            }
            // all of the row's loads before any store (residual_out may be
            // x or residual itself)
            uint4 rv[RESID ? VPT : 1];
            const char* rr = RESID ? static_cast<const char*>(a.residual) + row * a.residual_stride : nullptr;
            if constexpr (RESID) {
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int d = lt + k * T;
                    rv[k] = d < nv ? load_stream(rr + head * ESZ, d) : make_uint4(0, 0, 0, 0);
                }
                if (lt < head) hr = load_elem(reinterpret_cast<const Bits*>(rr) + lt);
            }
            // gamma's aligned vector d for each of this lane's vectors (zero
            // past gamma; L2 hits), loaded with the row so that its latency
            // overlaps the row's; a row with a head also needs vector d + 1.
            uint4 gc[VPT], gn[VPT];
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int d = lt + k * T;
                gc[k] = d < ngv ? gv[d] : make_uint4(0, 0, 0, 0);
                gn[k] = head != 0 && d + 1 < ngv ? gv[d + 1] : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int d = lt + k * T;
                if (d < nv && !whole(d)) {
                    xv[k] = keep_low_bytes(xv[k], tail * ESZ);
                    if constexpr (RESID) rv[k] = keep_low_bytes(rv[k], tail * ESZ);
                }
            }
            hs = E::widen(hx);
            if constexpr (RESID) {
                char* ro = static_cast<char*>(a.residual_out) + row * a.residual_out_stride;
                char* rob = ro + head * ESZ;
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int d = lt + k * T;
                    float xf[EPV], rf[EPV];
                    V::unpack(xv[k], xf);
                    V::unpack(rv[k], rf);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) xf[e] += rf[e];
                    // one rounding of the fp32 sum to the element type
                    // (bytes past the row are zero and stay zero)
                    xv[k] = V::pack(xf);
                    if (d < nv) {
                        if (whole(d)) {
                            store_stream(rob, d, xv[k]);
                        } else {
                            const uint32_t wd[4] = {xv[k].x, xv[k].y, xv[k].z, xv[k].w};
#pragma unroll
                            for (int e = 0; e < EPV; ++e) {
                                if (e >= tail) continue;
                                if constexpr (ESZ == 2)
                                    reinterpret_cast<uint16_t*>(rob)[d * EPV + e] =
                                        (uint16_t)(wd[e >> 1] >> (16 * (e & 1)));
                                else
                                    reinterpret_cast<uint32_t*>(rob)[d * EPV + e] = wd[e];
                            }
                        }
                    }
                }
                if (lt < head) {
                    const Bits sb = E::round(hs + E::widen(hr));
                    store_elem(reinterpret_cast<Bits*>(ro) + lt, sb);
                    hs = E::widen(sb);
                }
            }
            float amax32 = 0.0f;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int d = lt + k * T;
                if constexpr (T32) {
#pragma unroll
                    for (int e = 0; e < EPV; ++e) t[k][e] = 0.0f;
                } else {
                    gw[k] = make_uint4(0, 0, 0, 0);
                }
                if (d < nv) {
                    uint4 w = head != 0 ? window_from<ESZ>(gc[k], gn[k], head) : gc[k];
                    // gamma' past the row is not gamma (or not a number):
                    // zero, so that s * g' = 0 there
                    if (!whole(d)) w = keep_low_bytes(w, tail * ESZ);
                    float s[EPV], gf[EPV];
                    V::unpack(xv[k], s);
                    V::unpack(w, gf);
                    sumsq64<EPV>(ssq0, ssq1, s);
                    if constexpr (T32) {
                        // + weight_offset (0.0f here) as the definition's g + offset
#pragma unroll
                        for (int e = 0; e < EPV; ++e) t[k][e] = s[e] * (gf[e] + a.weight_offset);
                        amax32 = abs_max<EPV>(amax32, t[k]);
                    } else {
                        gw[k] = w;
#pragma unroll
                        for (int e = 0; e < EPV; ++e) amax = fmax(amax, abs_prod64(s[e], gf[e], offd));
                    }
                }
            }
            amax = fmax(amax, (double)amax32);
            if (lt < head) {
                const double d = hs;
                ssq0 = fma(d, d, ssq0);
                amax = fmax(amax, abs_prod64(hs, E::widen(hg), T32 ? (double)a.weight_offset : offd));
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

            uint8_t* orow = static_cast<uint8_t*>(a.out) + row * a.out_stride;
            // codes of vector d start at ob + d * EPV (the host checked that
            // this is EPV-byte aligned on every row)
            uint8_t* ob = orow + head;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int d = lt + k * T;
                if (d >= nv) continue;
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
                    float s[EPV], gf[EPV];
                    V::unpack(xv[k], s);
                    V::unpack(gw[k], gf);
                    if (split) {
#pragma unroll
                        for (int e = 0; e < EPV; ++e) q[e] = fp8_q2(s[e], gf[e], fr);
                    } else {
#pragma unroll
                        for (int e = 0; e < EPV; ++e) q[e] = fp8_q64(s[e], gf[e], offd, fr);
                    }
                }
                uint32_t wd[EPV / 4];
                wd[0] = fp8_x4<FNUZ>(q[0], q[1], q[2], q[3]);
                if constexpr (EPV == 8) wd[1] = fp8_x4<FNUZ>(q[4], q[5], q[6], q[7]);
                if (whole(d)) {
                    if constexpr (EPV == 8)
                        store_stream(ob, d, make_uint2(wd[0], wd[1]));
                    else
                        store_stream(ob, d, wd[0]);
                } else {
#pragma unroll
                    for (int e = 0; e < EPV; ++e)
                        if (e < tail) ob[d * EPV + e] = (uint8_t)(wd[e >> 2] >> (8 * (e & 3)));
                }
            }
            if (lt < head)
                orow[lt] = (uint8_t)fp8_x4<FNUZ>(fp8_q64(hs, E::widen(hg), T32 ? (double)a.weight_offset : offd, fr),
                                                 0.0f, 0.0f, 0.0f);
            if (lt == 0) store_scale(a.scales, row, a.scales_dtype, fr.sbits);
        }
    }
}

namespace fp8_phased_launch {

template <typename InT, bool RESID, bool FNUZ, int VPT, int PROD>
hipError_t launch_prod(FusedArgs a, Shape s, hipStream_t stream) {
    a.waves = s.waves;
    const int64_t groups = (a.rows + s.rpb - 1) / s.rpb;
    // default: one block per row group
    int64_t grid = s.grid > 0 ? s.grid : groups;
    if (grid > groups) grid = groups;
    if (grid > INT32_MAX) grid = INT32_MAX;
    if (grid < 1) grid = 1;
    const dim3 gd((unsigned)grid), bd(s.waves * s.rpb * 64);
    if (s.rpb == 1)
        hipLaunchKernelGGL((fp8_phased_kernel<InT, RESID, FNUZ, VPT, true, PROD>), gd, bd, 0, stream, a);
    else
        hipLaunchKernelGGL((fp8_phased_kernel<InT, RESID, FNUZ, VPT, false, PROD>), gd, bd, 0, stream, a);
    return hipGetLastError();
}

// the product form: kProdF32 / kProdTwo without a weight offset, else kProdF64
template <typename InT, bool RESID, bool FNUZ, int VPT>
hipError_t launch_vpt(const FusedArgs& a, Shape s, hipStream_t stream) {
    if (prod_mode<InT>(a.weight_offset) == kProdF64) return launch_prod<InT, RESID, FNUZ, VPT, kProdF64>(a, s, stream);
    return launch_prod<InT, RESID, FNUZ, VPT, prod_mode<InT>(0.0f)>(a, s, stream);
}

template <typename InT, bool RESID, bool FNUZ>
hipError_t by_vpt(const FusedArgs& a, Shape s, hipStream_t st) {
    switch (s.vpt) {
    case 1: return launch_vpt<InT, RESID, FNUZ, 1>(a, s, st);
    case 2: return launch_vpt<InT, RESID, FNUZ, 2>(a, s, st);
    default: return launch_vpt<InT, RESID, FNUZ, 4>(a, s, st);
    }
}

}  // namespace fp8_phased_launch

// All phased variants for one input type (one translation unit each).
template <typename InT>
hipError_t launch_fp8_phased_typed(const FusedArgs& a, bool residual, bool fnuz, Shape s, hipStream_t stream) {
    using namespace fp8_phased_launch;
    if (residual) return fnuz ? by_vpt<InT, true, true>(a, s, stream) : by_vpt<InT, true, false>(a, s, stream);
    return fnuz ? by_vpt<InT, false, true>(a, s, stream) : by_vpt<InT, false, false>(a, s, stream);
}

}  // namespace rmsq
