// Streaming reference kernels for measurement (declared in rmsq_probe.h):
// they move a workload's bytes with 16-byte non-temporal accesses and no
// arithmetic beyond an XOR that keeps every load live, gfx950.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "rmsq_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxIn = 9, kMaxOut = 3;

__device__ __forceinline__ u32x4 ld(const void* base, int64_t i16) {
    return __builtin_nontemporal_load(static_cast<const u32x4*>(base) + i16);
}
__device__ __forceinline__ void st(void* base, int64_t i16, u32x4 v) {
    __builtin_nontemporal_store(v, static_cast<u32x4*>(base) + i16);
}

// One unit: rv chunks of B vectors read (NL loads per lane in flight), then wv
// chunks written (or, with interleave, written in step with the reads).
template <int NL>
__global__ void __launch_bounds__(1024) chunk_probe(const u32x4* __restrict__ src, int64_t nr, u32x4* __restrict__ dst,
                                                    int64_t nw, int rv, int wv, int64_t units, int interleave) {
    const int B = blockDim.x;
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
        u32x4 acc = {0u, 0u, 0u, 0u};
        const int64_t r0 = u * rv * (int64_t)B + threadIdx.x;
        const int64_t w0 = u * wv * (int64_t)B + threadIdx.x;
        int w = 0;
        for (int r = 0; r < rv; r += NL) {
            u32x4 v[NL];
#pragma unroll
            for (int j = 0; j < NL; ++j) {
                const int64_t i = r0 + (int64_t)(r + j) * B;
                v[j] = (r + j < rv && i < nr) ? ld(src, i) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int j = 0; j < NL; ++j) acc ^= v[j];
            if (interleave) {
                const int wend = (int)(((int64_t)(r + NL) * wv + rv - 1) / rv);
                for (; w < wend && w < wv; ++w) {
                    const int64_t i = w0 + (int64_t)w * B;
                    if (i < nw) st(dst, i, acc + (uint32_t)w);
                }
            }
        }
        for (; w < wv; ++w) {
            const int64_t i = w0 + (int64_t)w * B;
            if (i < nw) st(dst, i, acc + (uint32_t)w);
        }
    }
}

struct RowArgs {
    const char* in[kMaxIn];
    char* out[kMaxOut];
    int64_t out_bytes[kMaxOut];
    int64_t in_bytes;
    int64_t rows;
    int nout;
    int phased;  // first output stored, a block barrier, then the others
    int mapped;  // outputs in pieces matched to the input vectors (below)
};

// One block per row at a time: every input row's vectors of this lane loaded
// (NIN * VPT loads in flight), XORed, then stored to every output row.
template <int NIN, int VPT>
__global__ void __launch_bounds__(1024) row_probe(const RowArgs a) {
    const int T = blockDim.x, tid = threadIdx.x;
    const int nv = (int)(a.in_bytes / 16);
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        u32x4 v[NIN][VPT];
#pragma unroll
        for (int i = 0; i < NIN; ++i)
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int idx = tid + k * T;
                v[i][k] = idx < nv ? ld(a.in[i] + row * a.in_bytes, idx) : u32x4{0u, 0u, 0u, 0u};
            }
        u32x4 acc[VPT];
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            acc[k] = v[0][k];
#pragma unroll
            for (int i = 1; i < NIN; ++i) acc[k] ^= v[i][k];
        }
        for (int o = 0; o < a.nout; ++o) {
            if (a.phased && o == 1) __syncthreads();  // uniform over the block
            const int64_t ob = a.out_bytes[o];
            char* base = a.out[o] + row * ob;
            // mapped: the bytes of output o that belong to input vector idx
            // (ob / nv of them: 4, 8 or 16) stored by the lane holding it,
            // as a fused kernel stores a vector's codes
            const int64_t piece = a.mapped && ob % nv == 0 ? ob / nv : 0;
            if (piece == 4 || piece == 8) {
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int idx = tid + k * T;
                    if (idx < nv) {
                        const u32x4 v = acc[k] + (uint32_t)o;
                        if (piece == 4)
                            __builtin_nontemporal_store(v.x, reinterpret_cast<uint32_t*>(base) + idx);
                        else
                            __builtin_nontemporal_store(v.x | ((uint64_t)v.y << 32), reinterpret_cast<uint64_t*>(base) + idx);
                    }
                }
            } else if (ob % 16 == 0) {
                const int nvo = (int)(ob / 16);
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int idx = tid + k * T;
                    if (idx < nvo) st(base, idx, acc[k] + (uint32_t)o);
                }
            } else if (tid < ob / 4) {
                __builtin_nontemporal_store(acc[0].x + (uint32_t)o, reinterpret_cast<uint32_t*>(base) + tid);
            }
        }
    }
}

// at most 16 loads per lane in flight (nin * vpt <= 16, checked by the caller):
// every one held in VGPRs without spilling under the 1024-thread bound
template <int NIN, int VPT>
void launch_row_probe(const RowArgs& a, int block, int grid, size_t lds, hipStream_t stream) {
    if constexpr (NIN * VPT <= 16)
        hipLaunchKernelGGL((row_probe<NIN, VPT>), dim3(grid), dim3(block), lds, stream, a);
}

template <int NIN>
hipError_t launch_rows(const RowArgs& a, int vpt, int block, int grid, size_t lds, hipStream_t stream) {
    switch (vpt) {
    case 1: launch_row_probe<NIN, 1>(a, block, grid, lds, stream); break;
    case 2: launch_row_probe<NIN, 2>(a, block, grid, lds, stream); break;
    case 4: launch_row_probe<NIN, 4>(a, block, grid, lds, stream); break;
    default: launch_row_probe<NIN, 8>(a, block, grid, lds, stream); break;
    }
    return hipGetLastError();
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

}  // namespace

extern "C" int rmsq_probe_chunks(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes, int rv, int wv,
                                 int block, int loads_in_flight, int blocks_per_cu, int interleave,
                                 hipStream_t stream) {
    if (!src || !dst) return -1;
    if (read_bytes <= 0 || write_bytes <= 0 || read_bytes % 16 || write_bytes % 16 || rv < 1 || rv > 64 || wv < 1 ||
        wv > 64 || block < 64 || block > 1024 || block % 64 || blocks_per_cu < 0 || blocks_per_cu > 64)
        return -2;
    const int nl = loads_in_flight;
    if (nl != 1 && nl != 2 && nl != 4 && nl != 8 && nl != 16) return -2;
    if (!aligned16(src) || !aligned16(dst)) return -3;
    const char *s0 = static_cast<const char*>(src), *d0 = static_cast<const char*>(dst);
    if (s0 < d0 + write_bytes && d0 < s0 + read_bytes) return -2;
    const int64_t nr = read_bytes / 16, nw = write_bytes / 16;
    const int64_t units = std::max((nr + (int64_t)rv * block - 1) / ((int64_t)rv * block),
                                   (nw + (int64_t)wv * block - 1) / ((int64_t)wv * block));
    int64_t grid = blocks_per_cu > 0 ? std::min<int64_t>(units, (int64_t)blocks_per_cu * 256) : units;
    grid = std::min<int64_t>(grid, INT32_MAX);
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    const dim3 gd((unsigned)grid), bd(block);
    switch (nl) {
    case 1: hipLaunchKernelGGL(chunk_probe<1>, gd, bd, 0, stream, s, nr, d, nw, rv, wv, units, interleave); break;
    case 2: hipLaunchKernelGGL(chunk_probe<2>, gd, bd, 0, stream, s, nr, d, nw, rv, wv, units, interleave); break;
    case 4: hipLaunchKernelGGL(chunk_probe<4>, gd, bd, 0, stream, s, nr, d, nw, rv, wv, units, interleave); break;
    case 8: hipLaunchKernelGGL(chunk_probe<8>, gd, bd, 0, stream, s, nr, d, nw, rv, wv, units, interleave); break;
    default: hipLaunchKernelGGL(chunk_probe<16>, gd, bd, 0, stream, s, nr, d, nw, rv, wv, units, interleave); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int rmsq_probe_rows(int64_t rows, int nin, const void* const* inputs, int64_t in_row_bytes, int nout,
                               void* const* outputs, const int64_t* out_row_bytes, int block, int vpt, int grid,
                               int flags, int lds_bytes, hipStream_t stream) {
    if (!inputs || !outputs || !out_row_bytes) return -1;
    if (rows < 0 || nin < 1 || nin > kMaxIn || nout < 1 || nout > kMaxOut || in_row_bytes <= 0 ||
        in_row_bytes % 16 || block < 64 || block > 1024 || block % 64 || grid < 0 || lds_bytes < 0 ||
        lds_bytes > 64 * 1024)
        return -2;
    if ((vpt != 1 && vpt != 2 && vpt != 4 && vpt != 8) || nin * vpt > 16 || (flags & ~3)) return -2;
    if ((int64_t)block * vpt * 16 < in_row_bytes) return -2;
    RowArgs a{};
    for (int i = 0; i < nin; ++i) {
        if (!inputs[i]) return -1;
        if (!aligned16(inputs[i])) return -3;
        a.in[i] = static_cast<const char*>(inputs[i]);
    }
    for (int o = 0; o < nout; ++o) {
        const int64_t ob = out_row_bytes[o];
        if (!outputs[o]) return -1;
        if (!aligned16(outputs[o])) return -3;
        const bool vec = ob > 0 && ob % 16 == 0 && ob <= in_row_bytes;
        const bool tail = ob > 0 && ob % 4 == 0 && ob <= 4 * (int64_t)block;
        if (!vec && !tail) return -2;
        a.out[o] = static_cast<char*>(outputs[o]);
        a.out_bytes[o] = ob;
    }
    if (rows == 0) return 0;
    a.in_bytes = in_row_bytes;
    a.rows = rows;
    a.nout = nout;
    a.phased = flags & 1;
    a.mapped = (flags >> 1) & 1;
    const int g = (int)std::min<int64_t>(grid > 0 ? std::min<int64_t>(grid, rows) : rows, INT32_MAX);
    hipError_t e;
    switch (nin) {
    case 1: e = launch_rows<1>(a, vpt, block, g, (size_t)lds_bytes, stream); break;
    case 2: e = launch_rows<2>(a, vpt, block, g, (size_t)lds_bytes, stream); break;
    case 3: e = launch_rows<3>(a, vpt, block, g, (size_t)lds_bytes, stream); break;
    case 4: e = launch_rows<4>(a, vpt, block, g, (size_t)lds_bytes, stream); break;
    case 5: e = launch_rows<5>(a, vpt, block, g, (size_t)lds_bytes, stream); break;
    case 6: e = launch_rows<6>(a, vpt, block, g, (size_t)lds_bytes, stream); break;
    case 7: e = launch_rows<7>(a, vpt, block, g, (size_t)lds_bytes, stream); break;
    case 8: e = launch_rows<8>(a, vpt, block, g, (size_t)lds_bytes, stream); break;
    default: e = launch_rows<9>(a, vpt, block, g, (size_t)lds_bytes, stream); break;
    }
    return e == hipSuccess ? 0 : -4;
}
