// Streaming reference kernel for measurement: it moves a given number of
// bytes, read and written in the same proportion as a fused workload, with the
// same 16-byte non-temporal accesses, and computes nothing.  Its rate is the
// "achievable" HBM ceiling a fused kernel with that traffic mix is compared
// with (the 8 TB/s peak is never reached by mixed read/write streams).
//
// Work mapping: a unit is RV consecutive 256-vector chunks of the source and
// WV consecutive 256-vector chunks of the destination (RV : WV approximates
// the byte ratio); one 256-thread block handles a unit at a time, reading its
// chunks and then writing its chunks, as a fused kernel reads a row and then
// writes it.  Written values depend on the loaded ones, so no load is dead.
#include <algorithm>
#include <cmath>

#include "rmsq_device.h"
#include "rmsq_internal.h"

namespace rmsq {

namespace {

__global__ void __launch_bounds__(256) stream_kernel(const u32x4* __restrict__ src, int64_t nr,
                                                     u32x4* __restrict__ dst, int64_t nw, int rv, int wv,
                                                     int64_t units) {
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
        u32x4 acc = {0u, 0u, 0u, 0u};
        const int64_t r0 = u * rv * 256 + threadIdx.x;
#pragma unroll 4
        for (int r = 0; r < rv; ++r) {
            const int64_t i = r0 + (int64_t)r * 256;
            if (i < nr) acc ^= __builtin_nontemporal_load(src + i);
        }
        const int64_t w0 = u * wv * 256 + threadIdx.x;
#pragma unroll 4
        for (int w = 0; w < wv; ++w) {
            const int64_t i = w0 + (int64_t)w * 256;
            if (i < nw) __builtin_nontemporal_store(acc + (uint32_t)w, dst + i);
        }
    }
}

// Smallest RV, WV (RV + WV minimal, each <= 32) whose ratio is within 2% of
// reads : writes.
void unit_ratio(int64_t nr, int64_t nw, int* rv, int* wv) {
    const double want = (double)nr / (double)nw;
    for (int sum = 2; sum <= 64; ++sum)
        for (int r = 1; r < sum; ++r) {
            const int w = sum - r;
            if (r > 32 || w > 32) continue;
            if (std::fabs((double)r / w - want) <= 0.02 * want) {
                *rv = r;
                *wv = w;
                return;
            }
        }
    // far outside 1/32..32: the closest end
    *rv = want > 1.0 ? 32 : 1;
    *wv = want > 1.0 ? 1 : 32;
}

}  // namespace

hipError_t launch_stream(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes, hipStream_t stream) {
    const int64_t nr = read_bytes / 16, nw = write_bytes / 16;
    int rv = 1, wv = 1;
    unit_ratio(nr, nw, &rv, &wv);
    const int64_t units = std::max((nr + rv * 256 - 1) / (rv * 256), (nw + wv * 256 - 1) / (wv * 256));
    const int64_t grid = std::min<int64_t>(units, INT32_MAX);
    hipLaunchKernelGGL(stream_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       static_cast<const u32x4*>(src), nr, static_cast<u32x4*>(dst), nw, rv, wv, units);
    return hipGetLastError();
}

}  // namespace rmsq
