// C ABI of librmsq: argument validation, launch-shape choice and dispatch.
// Every check runs before the first HIP call, so each error path is testable
// on a machine without a GPU.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>

#include "../../include/rmsq.h"
#include "rmsq_internal.h"

namespace rmsq {

namespace {

thread_local int g_last_hip_error = 0;
std::atomic<int> g_tune_waves{0};
std::atomic<int> g_tune_vpt{0};
std::atomic<int> g_tune_blocks{0};

// Largest row the register-resident kernels hold: 16 waves x 64 lanes x 4
// vectors of 16 bytes.

bool valid_dtype(int dt) { return dt == RMSQ_F32 || dt == RMSQ_F16 || dt == RMSQ_BF16; }
int64_t elem_size(int dt) { return dt == RMSQ_F32 ? 4 : 2; }
int64_t elems_per_vec(int dt) { return 16 / elem_size(dt); }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
    Span(const void* p, int64_t bytes)
        : lo(reinterpret_cast<uintptr_t>(p)), hi(reinterpret_cast<uintptr_t>(p) + (uintptr_t)bytes) {}
};
bool overlap(const Span& a, const Span& b) { return a.lo < b.hi && b.lo < a.hi; }

// Bytes from the first element of a row tensor to past its last one.
int64_t extent(int64_t rows, int64_t row_bytes, int64_t stride_bytes) {
    return rows == 0 ? 0 : (rows - 1) * stride_bytes + row_bytes;
}

// A row stride (elements of esz bytes) is valid when it holds the row and
// keeps every row start on a `quantum`-byte boundary.
bool stride_ok(int64_t stride, int64_t row_elems, int64_t esz, int64_t quantum) {
    return stride >= row_elems && stride <= INT32_MAX && (stride * esz) % quantum == 0;
}

// rows * hidden * esz must fit comfortably in int64 (and hidden in int32)
bool size_ok(int64_t rows, int64_t hidden, int64_t esz) {
    if (hidden > INT32_MAX / 2) return false;
    return rows <= (INT64_MAX / 4) / (hidden * esz);
}

int check_scalars(float eps, float weight_offset, float scale_ub, bool check_ub) {
    if (!(eps >= 0.0f) || !isfinite(eps)) return RMSQ_ERR_VALUE;
    if (!isfinite(weight_offset)) return RMSQ_ERR_VALUE;
    if (check_ub && !(scale_ub > 0.0f)) return RMSQ_ERR_VALUE;  // NaN fails too
    return RMSQ_OK;
}

int launched(hipError_t e) {
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return RMSQ_ERR_LAUNCH;
    }
    return RMSQ_OK;
}

int fp8_common(int64_t rows, int64_t hidden, int in_dtype, const void* x, int64_t x_stride, const void* residual,
               int64_t r_stride, void* residual_out, int64_t ro_stride, bool resid, const void* gamma, float eps,
               float weight_offset, float scale_ub, int out_fp8, void* out, int64_t out_stride, int scales_dtype,
               void* scales, hipStream_t stream) {
    if (!valid_dtype(in_dtype) || !valid_dtype(scales_dtype)) return RMSQ_ERR_DTYPE;
    if (out_fp8 != RMSQ_E4M3FN && out_fp8 != RMSQ_E4M3FNUZ) return RMSQ_ERR_DTYPE;
    const int64_t esz = elem_size(in_dtype), epv = elems_per_vec(in_dtype);
    // any row width and any element-aligned rows (the kernel is chosen from
    // the layout below)
    if (rows < 0 || hidden <= 0) return RMSQ_ERR_SHAPE;
    if (!stride_ok(x_stride, hidden, esz, esz) || !stride_ok(out_stride, hidden, 1, 1)) return RMSQ_ERR_SHAPE;
    if (resid && (!stride_ok(r_stride, hidden, esz, esz) || !stride_ok(ro_stride, hidden, esz, esz)))
        return RMSQ_ERR_SHAPE;
    const int64_t widest = std::max({x_stride, out_stride / esz + 1, resid ? std::max(r_stride, ro_stride) : 0});
    if (!size_ok(rows, widest, esz)) return RMSQ_ERR_SHAPE;
    if (int rc = check_scalars(eps, weight_offset, scale_ub, true)) return rc;
    if (hidden > std::max(kMaxWideVec * epv, kMaxElemHidden)) return RMSQ_ERR_UNSUPPORTED;
    if (rows == 0) return RMSQ_OK;
    if (!x || !gamma || !out || !scales) return RMSQ_ERR_NULL;
    if (resid && (!residual || !residual_out)) return RMSQ_ERR_NULL;
    const int64_t ssz = elem_size(scales_dtype);
    if (!aligned(x, esz) || !aligned(gamma, esz) || !aligned(scales, (uintptr_t)ssz)) return RMSQ_ERR_ALIGN;
    if (resid && (!aligned(residual, esz) || !aligned(residual_out, esz))) return RMSQ_ERR_ALIGN;
    // Four kernels: rows of whole, 16-byte aligned vectors (the vector
    // kernel, or above 4096 vectors the wide-row kernel, the row staged in
    // LDS); rows at a common offset from the 16-byte grid (the phased
    // kernel: residual and residual_out at x's offset on every row, codes at
    // the same offset modulo epv, gamma aligned); anything else (the
    // element-wise kernel)
    const bool whole = hidden % epv == 0 && aligned(x, 16) && aligned(gamma, 16) && aligned(out, 16) &&
                       (x_stride * esz) % 16 == 0 && out_stride % epv == 0 &&
                       (!resid || (aligned(residual, 16) && aligned(residual_out, 16) &&
                                   (r_stride * esz) % 16 == 0 && (ro_stride * esz) % 16 == 0));
    const bool vec = whole && hidden / epv <= kMaxVec;
    const bool wide = whole && !vec && hidden / epv <= kMaxWideVec;
    const uintptr_t xph = reinterpret_cast<uintptr_t>(x) % 16;  // bytes past the 16-byte grid
    auto same_phase = [&](const void* p, int64_t stride) {
        return reinterpret_cast<uintptr_t>(p) % 16 == xph && ((stride - x_stride) * esz) % 16 == 0;
    };
    const int64_t phased_nvec = ceil_div(hidden, epv);  // lanes as for a whole-vector row
    const bool phased = !vec && phased_nvec <= kMaxVec && aligned(gamma, 16) &&
                        (int64_t)(reinterpret_cast<uintptr_t>(out) % epv) == (int64_t)(xph / esz) % epv &&
                        (out_stride - x_stride) % epv == 0 &&
                        (!resid || (same_phase(residual, r_stride) && same_phase(residual_out, ro_stride)));
    if (!vec && !wide && !phased && hidden > kMaxElemHidden) return RMSQ_ERR_UNSUPPORTED;
    const int nvec = (vec || wide) ? (int)(hidden / epv) : phased ? (int)phased_nvec : 0;

    // spans cover every row; strided tensors are compared by their extents
    const int64_t rb = hidden * esz;
    const Span sx(x, extent(rows, rb, x_stride * esz)), sg(gamma, rb), so(out, extent(rows, hidden, out_stride)),
        ss(scales, rows * ssz);
    // outputs never overlap inputs or each other ...
    if (overlap(so, ss) || overlap(so, sx) || overlap(so, sg) || overlap(ss, sx) || overlap(ss, sg))
        return RMSQ_ERR_ALIAS;
    if (resid) {
        const Span sr(residual, extent(rows, rb, r_stride * esz)), sro(residual_out, extent(rows, rb, ro_stride * esz));
        if (overlap(so, sr) || overlap(ss, sr) || overlap(sro, so) || overlap(sro, ss) || overlap(sro, sg))
            return RMSQ_ERR_ALIAS;
        // ... except an in-place residual update at exactly the same address
        // and row stride
        const bool on_x = residual_out == x && ro_stride == x_stride;
        const bool on_r = residual_out == residual && ro_stride == r_stride;
        if (!on_x && overlap(sro, sx)) return RMSQ_ERR_ALIAS;
        if (!on_r && overlap(sro, sr)) return RMSQ_ERR_ALIAS;
    }

    Shape shape;
    const int path = resid ? kPathFp8Residual : kPathFp8;
    if (wide ? !choose_wide_shape(nvec, &shape)
             : (vec || phased) ? !choose_shape(rows, nvec, path, (int)esz, &shape) : !choose_elem_shape(rows, hidden, &shape))
        return RMSQ_ERR_UNSUPPORTED;
    FusedArgs a{};
    a.x = x;
    a.residual = residual;
    a.residual_out = residual_out;
    a.gamma = gamma;
    a.out = out;
    a.scales = scales;
    a.global_scale = nullptr;
    a.rows = rows;
    a.hidden = (int32_t)hidden;
    a.inv_hidden = 1.0 / (double)hidden;
    a.nvec = nvec;
    a.eps = eps;
    a.weight_offset = weight_offset;
    a.scale_ub = scale_ub;
    a.scales_dtype = scales_dtype;
    a.x_stride = x_stride * esz;
    a.residual_stride = r_stride * esz;
    a.residual_out_stride = ro_stride * esz;
    a.out_stride = out_stride;
    if (wide)
        return launched(launch_wide(a, in_dtype, resid, out_fp8 == RMSQ_E4M3FNUZ ? kWideFp8Fnuz : kWideFp8,
                                    Fp4Format{16, false}, shape.grid, stream));
    return launched(vec      ? launch_fp8(a, in_dtype, resid, out_fp8, shape, stream)
                    : phased ? launch_fp8_phased(a, in_dtype, resid, out_fp8, shape, stream)
                             : launch_fp8_elem(a, in_dtype, resid, out_fp8, shape, stream));
}


// Several input buffers summed in front of the residual FP8 path: whole,
// 16-byte aligned vectors only (the vector mapping).
int sum_common(int64_t rows, int64_t hidden, int in_dtype, int ninputs, const void* const* inputs,
               const void* residual, void* residual_out, const void* gamma, float eps, float weight_offset,
               float scale_ub, int out_fp8, void* out, int scales_dtype, void* scales, hipStream_t stream) {
    if (!valid_dtype(in_dtype) || !valid_dtype(scales_dtype)) return RMSQ_ERR_DTYPE;
    if (out_fp8 != RMSQ_E4M3FN && out_fp8 != RMSQ_E4M3FNUZ) return RMSQ_ERR_DTYPE;
    if (ninputs < 1 || ninputs > kMaxSumInputs) return RMSQ_ERR_VALUE;
    const int64_t esz = elem_size(in_dtype), epv = elems_per_vec(in_dtype);
    if (rows < 0 || hidden <= 0 || hidden % epv != 0 || !size_ok(rows, hidden, esz)) return RMSQ_ERR_SHAPE;
    if (int rc = check_scalars(eps, weight_offset, scale_ub, true)) return rc;
    const int64_t nvec = hidden / epv;
    if (nvec > kMaxVec) return RMSQ_ERR_UNSUPPORTED;
    if (rows == 0) return RMSQ_OK;
    if (!inputs || !residual || !residual_out || !gamma || !out || !scales) return RMSQ_ERR_NULL;
    for (int g = 0; g < ninputs; ++g)
        if (!inputs[g]) return RMSQ_ERR_NULL;
    const int64_t ssz = elem_size(scales_dtype);
    if (!aligned(residual, 16) || !aligned(residual_out, 16) || !aligned(gamma, 16) || !aligned(out, 16) ||
        !aligned(scales, (uintptr_t)ssz))
        return RMSQ_ERR_ALIGN;
    for (int g = 0; g < ninputs; ++g)
        if (!aligned(inputs[g], 16)) return RMSQ_ERR_ALIGN;
    const int64_t rb = rows * hidden * esz;
    const Span sr(residual, rb), sro(residual_out, rb), sg(gamma, hidden * esz), so(out, rows * hidden),
        ss(scales, rows * ssz);
    // outputs never overlap an input, gamma or each other; residual_out may
    // be exactly residual (in-place update); inputs may share memory (they
    // are only read)
    if (overlap(so, ss) || overlap(so, sro) || overlap(ss, sro)) return RMSQ_ERR_ALIAS;
    for (const Span& o : {so, ss, sro}) {
        if (overlap(o, sg)) return RMSQ_ERR_ALIAS;
        for (int g = 0; g < ninputs; ++g)
            if (overlap(o, Span(inputs[g], rb))) return RMSQ_ERR_ALIAS;
    }
    if (overlap(so, sr) || overlap(ss, sr)) return RMSQ_ERR_ALIAS;
    if (residual_out != residual && overlap(sro, sr)) return RMSQ_ERR_ALIAS;

    Shape shape;
    if (!choose_shape(rows, (int)nvec, kPathFp8Sum, (int)esz, &shape)) return RMSQ_ERR_UNSUPPORTED;
    SumArgs sa{};
    FusedArgs& a = sa.a;
    a.residual = residual;
    a.residual_out = residual_out;
    a.gamma = gamma;
    a.out = out;
    a.scales = scales;
    a.rows = rows;
    a.hidden = (int32_t)hidden;
    a.inv_hidden = 1.0 / (double)hidden;
    a.nvec = (int32_t)nvec;
    a.eps = eps;
    a.weight_offset = weight_offset;
    a.scale_ub = scale_ub;
    a.scales_dtype = scales_dtype;
    for (int g = 0; g < ninputs; ++g) sa.inputs[g] = inputs[g];
    sa.ninputs = ninputs;
    return launched(launch_fp8_sum(sa, in_dtype, out_fp8, shape, stream));
}

}  // namespace

namespace {


// Vectors per lane for a given wave count: the smallest supported one that
// holds the row, or 0.
int vpt_for(int nvec, int waves) {
    const int64_t need = ceil_div(nvec, (int64_t)waves * 64);
    return need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 0;
}

int fp4_common(int64_t rows, int64_t hidden, int in_dtype, const void* x, int64_t x_stride, const void* residual,
               int64_t r_stride, void* residual_out, int64_t ro_stride, bool resid, const void* gamma, float eps,
               float weight_offset, const float* global_scale, int block_size, int scale_format, int scale_layout,
               int flags, void* out, int64_t out_stride, void* block_scales, hipStream_t stream) {
    if (!valid_dtype(in_dtype)) return RMSQ_ERR_DTYPE;
    if (scale_format != RMSQ_SF_E4M3 && scale_format != RMSQ_SF_UE8M0) return RMSQ_ERR_DTYPE;
    if (scale_layout != RMSQ_SF_ROW_MAJOR && scale_layout != RMSQ_SF_SWIZZLED) return RMSQ_ERR_DTYPE;
    if (block_size != 16 && block_size != 32) return RMSQ_ERR_VALUE;
    if (flags & ~RMSQ_FP4_ROUND_PRODUCT) return RMSQ_ERR_VALUE;
    const int64_t esz = elem_size(in_dtype);
    if (rows < 0 || hidden <= 0 || hidden % block_size != 0) return RMSQ_ERR_SHAPE;
    // code rows: hidden / 2 bytes, stored 2 or 4 bytes per lane -> 8-byte row starts
    if (!stride_ok(x_stride, hidden, esz, 16) || !stride_ok(out_stride, hidden / 2, 1, 8)) return RMSQ_ERR_SHAPE;
    if (resid && (!stride_ok(r_stride, hidden, esz, 16) || !stride_ok(ro_stride, hidden, esz, 16)))
        return RMSQ_ERR_SHAPE;
    const int64_t widest = std::max({x_stride, out_stride / esz + 1, resid ? std::max(r_stride, ro_stride) : 0});
    if (!size_ok(rows, widest, esz)) return RMSQ_ERR_SHAPE;
    if (int rc = check_scalars(eps, weight_offset, 1.0f, false)) return rc;
    const int64_t nvec64 = hidden / elems_per_vec(in_dtype);
    if (nvec64 > kMaxWideVec) return RMSQ_ERR_UNSUPPORTED;
    const int nvec = (int)nvec64;
    const bool wide = nvec > kMaxVec;  // the wide-row kernels
    if (rows == 0) return RMSQ_OK;
    if (!x || !gamma || !out || !block_scales) return RMSQ_ERR_NULL;
    if (resid && (!residual || !residual_out)) return RMSQ_ERR_NULL;
    if (!aligned(x, 16) || !aligned(gamma, 16) || !aligned(out, 16)) return RMSQ_ERR_ALIGN;
    if (resid && (!aligned(residual, 16) || !aligned(residual_out, 16))) return RMSQ_ERR_ALIGN;
    // the global scale is read only for E4M3 scales
    const float* gsp = scale_format == RMSQ_SF_E4M3 ? global_scale : nullptr;
    if (gsp && !aligned(gsp, 4)) return RMSQ_ERR_ALIGN;
    const int64_t rb = hidden * esz;
    const int64_t sbytes = rmsq_fp4_scale_bytes(rows, hidden, block_size, scale_layout);
    const Span sx(x, extent(rows, rb, x_stride * esz)), sg(gamma, rb), so(out, extent(rows, hidden / 2, out_stride)),
        ss(block_scales, sbytes);
    if (overlap(so, ss) || overlap(so, sx) || overlap(so, sg) || overlap(ss, sx) || overlap(ss, sg))
        return RMSQ_ERR_ALIAS;
    const Span sro(residual_out, resid ? extent(rows, rb, ro_stride * esz) : 0);
    if (gsp) {
        const Span sgs(gsp, 4);
        if (overlap(sgs, so) || overlap(sgs, ss)) return RMSQ_ERR_ALIAS;
        if (resid && overlap(sgs, sro)) return RMSQ_ERR_ALIAS;
    }
    if (resid) {
        const Span sr(residual, extent(rows, rb, r_stride * esz));
        if (overlap(so, sr) || overlap(ss, sr) || overlap(sro, so) || overlap(sro, ss) || overlap(sro, sg))
            return RMSQ_ERR_ALIAS;
        // an in-place residual update at exactly the same address and row
        // stride is allowed
        const bool on_x = residual_out == x && ro_stride == x_stride;
        const bool on_r = residual_out == residual && ro_stride == r_stride;
        if (!on_x && overlap(sro, sx)) return RMSQ_ERR_ALIAS;
        if (!on_r && overlap(sro, sr)) return RMSQ_ERR_ALIAS;
    }
    Shape shape;
    if (wide ? !choose_wide_shape(nvec, &shape) : !choose_shape(rows, nvec, resid ? kPathFp4Residual : kPathFp4, (int)esz, &shape))
        return RMSQ_ERR_UNSUPPORTED;
    FusedArgs a{};
    a.x = x;
    a.residual = residual;
    a.residual_out = residual_out;
    a.gamma = gamma;
    a.out = out;
    a.scales = block_scales;
    a.global_scale = gsp;
    a.rows = rows;
    a.hidden = (int32_t)hidden;
    a.inv_hidden = 1.0 / (double)hidden;
    a.nvec = nvec;
    a.eps = eps;
    a.weight_offset = weight_offset;
    a.sf_swizzled = scale_layout == RMSQ_SF_SWIZZLED ? 1 : 0;
    a.sf_k_tiles = (int32_t)ceil_div(hidden / block_size, 4);
    a.round_product = (flags & RMSQ_FP4_ROUND_PRODUCT) ? 1 : 0;
    a.x_stride = x_stride * esz;
    a.residual_stride = r_stride * esz;
    a.residual_out_stride = ro_stride * esz;
    a.out_stride = out_stride;
    const Fp4Format fmt{block_size, scale_format == RMSQ_SF_UE8M0};
    if (wide) return launched(launch_wide(a, in_dtype, resid, kWideFp4, fmt, shape.grid, stream));
    return launched(launch_fp4(a, in_dtype, resid, fmt, shape, stream));
}

}  // namespace

bool choose_shape(int64_t rows, int nvec, int path, int esz, Shape* s) {
    int waves = g_tune_waves.load(std::memory_order_relaxed);
    int vpt = g_tune_vpt.load(std::memory_order_relaxed);
    if (waves == 0 && vpt == 0) {
        if (rows <= kLatencyRows) {
            // small batches are latency bound: spread the row over up to 16
            // waves with 2 vectors per lane (a 16 KB row takes 2.4 us as
            // 8 x 2 on MI355X, 3.0 us as 16 x 1 and 2.8 us as 4 x 4)
            vpt = nvec <= 64 ? 1 : (nvec <= 16 * 64 * 2 ? 2 : 4);
            waves = (int)std::min<int64_t>(16, ceil_div(nvec, 64 * vpt));
        } else if (path == kPathFp4 && esz == 2 && nvec > 256 && nvec <= 64 * 12) {
            // FP4 of 16-bit rows of 257..768 vectors: one wavefront per row
            // with every load of the row in flight (the wave-per-row kernel).
            // A/B on MI355X against the block kernel's 4 x 4 / 4 x 2 shapes:
            // 16384 x 5120 bf16 0.93x the time, 8192 x 4096 0.97x; at 14 and
            // 16 vectors per lane it was slower (16384 x 7168 1.05x,
            // 8192 x 8192 1.08x: 100-112 VGPRs, four waves per SIMD)
            waves = 1;
            for (int v : kWaveRowVpt) {
                if ((int64_t)v * 64 >= nvec) {
                    vpt = v;
                    break;
                }
            }
            s->waves = waves;
            s->vpt = vpt;
            s->rpb = 4;
            s->grid = g_tune_blocks.load(std::memory_order_relaxed);
            return true;
        } else {
            // large batches: blocks of a multiple of 4 wavefronts, so the 4
            // SIMDs of a CU get equal work (odd counts measured 20-35% slower
            // on MI355X).  Among those shapes whose lanes hold the row, the one
            // with the fewest idle lanes; ties go to the vectors per lane
            // measured fastest on MI355X (bf16, 2048-16384 elements):
            //   rows of up to 256 vectors: 2, then 4, then 1 (FP4: 4, 2, 1);
            //   longer rows take at least 4 waves, and
            //     FP8 and FP4 without a residual: 4, 2, then 1 at 4 waves only
            //     (12 x 1 ran 640- and 768-vector rows 1.3-1.5x slower than
            //     4 x 4, 16 x 2 a 2048-vector row 1.3x slower than 8 x 4);
            //     FP8 with a residual: 2, 4, then 1 at 4 waves only (12 x 1
            //     ran 640- and 768-vector rows 1.13x slower than 8 x 2);
            //     FP4 with a residual: 1, 2, 4 (it holds two inputs per row:
            //     12 x 1 ran a 640-vector row 1.2x faster than 8 x 2, 16 x 1
            //     an 896-vector row 1.1x faster); the same for summed input
            //     buffers (8 x 1 ran 8 inputs of 512 vectors 3% faster than
            //     4 x 2).
            const int order_2[3] = {2, 4, 1}, order_4[3] = {4, 2, 1}, order_1[3] = {1, 2, 4};
            const bool wide = nvec > 256;
            const int* order = !wide ? (path == kPathFp4 ? order_4 : order_2)
                               : (path == kPathFp4Residual || path == kPathFp8Sum) ? order_1
                               : (path == kPathFp4 || path == kPathFp8) ? order_4
                                                                        : order_2;
            const bool one_at_4 = wide && path != kPathFp4Residual && path != kPathFp8Sum;  // 1 vector per lane only at 4 waves
            // fp32 rows with a residual hold more than 64 VGPRs per lane in
            // the FP8 kernel, so a 16-wave block leaves room for only one per
            // CU (12 waves: two): 16-wave shapes are taken only when no
            // other shape holds the row (32768 x 8192 fp32 rows: 562 us as
            // 8 x 4 against 649 us as 16 x 2, A/B in one process)
            const bool cap8 = esz == 4 && path == kPathFp8Residual;
            int64_t best_idle = INT64_MAX;
            waves = 0;
            for (int pass = 0; pass < (cap8 ? 2 : 1) && waves == 0; ++pass)
            for (int i = 0; i < 3; ++i) {
                const int v = order[i];
                for (int w : {1, 2, 4, 8, 12, 16}) {
                    if (cap8 && pass == 0 && w == 16) continue;
                    if (wide && (w < 4 || (one_at_4 && v == 1 && w > 4))) continue;
                    const int64_t idle = (int64_t)w * 64 * v - nvec;
                    if (idle >= 0 && idle < best_idle) {
                        best_idle = idle;
                        waves = w;
                        vpt = v;
                    }
                }
            }
            if (waves == 0) return false;
        }
    } else if (waves == 0) {
        waves = (int)std::min<int64_t>(16, ceil_div(nvec, 64 * (int64_t)vpt));
    }
    if (vpt == 0) vpt = vpt_for(nvec, waves);
    if (vpt == 0 || (int64_t)vpt * waves * 64 < nvec) return false;
    s->waves = waves;
    s->vpt = vpt;
    s->rpb = waves >= 4 ? 1 : 4 / waves;
    s->grid = g_tune_blocks.load(std::memory_order_relaxed);
    return true;
}

bool choose_wide_shape(int nvec, Shape* s) {
    // the wide-row kernels always run 16 waves (the row in LDS or in
    // registers); a forced wave count or vectors per lane cannot be honoured
    const int waves = g_tune_waves.load(std::memory_order_relaxed);
    const int vpt = g_tune_vpt.load(std::memory_order_relaxed);
    if ((waves != 0 && waves != 16) || vpt != 0 || nvec > kMaxWideVec) return false;
    s->waves = 16;
    s->vpt = (int)ceil_div(nvec, 16 * 64);
    s->rpb = 1;
    s->grid = g_tune_blocks.load(std::memory_order_relaxed);
    return true;
}

bool choose_elem_shape(int64_t rows, int64_t hidden, Shape* s) {
    (void)rows;
    // elements per lane for w waves: the smallest compiled count that holds
    // the row, or 0
    auto epl_for = [&](int w) {
        const int64_t need = ceil_div(hidden, (int64_t)w * 64);
        for (int e : kElemPerLane)
            if (e >= need) return e;
        return 0;
    };
    int waves = g_tune_waves.load(std::memory_order_relaxed), epl = 0;
    if (waves > 0) {
        epl = epl_for(waves);
    } else {
        // the fewest element slots that hold the row; ties to more waves
        // (shorter per-lane chains, more loads in flight)
        int64_t best = INT64_MAX;
        for (int w : {1, 2, 4, 8, 12, 16}) {
            const int e = epl_for(w);
            if (e == 0) continue;
            const int64_t slots = (int64_t)w * 64 * e;
            if (slots <= best) {
                best = slots;
                waves = w;
                epl = e;
            }
        }
    }
    if (epl == 0) return false;
    s->waves = waves;
    s->vpt = epl;
    s->rpb = waves >= 4 ? 1 : 4 / waves;
    s->grid = g_tune_blocks.load(std::memory_order_relaxed);
    return true;
}

namespace {

struct Occupancy {
    int cus;     // compute units of the device
    int per_cu;  // resident blocks per CU
};

Occupancy occupancy(const void* kernel, int block_threads, size_t dyn_lds) {
    static std::mutex mu;
    static std::map<std::tuple<int, int, size_t, const void*>, Occupancy> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_tuple(dev, block_threads, dyn_lds, kernel);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, block_threads, dyn_lds) != hipSuccess || per < 1)
        per = 1;
    const Occupancy o{cus, per};
    cache[key] = o;
    return o;
}

}  // namespace

int persistent_blocks(const void* kernel, int block_threads, size_t dyn_lds) {
    const Occupancy o = occupancy(kernel, block_threads, dyn_lds);
    return o.cus * o.per_cu;
}

int blocks_per_cu(const void* kernel, int block_threads, size_t dyn_lds) {
    return occupancy(kernel, block_threads, dyn_lds).per_cu;
}

}  // namespace rmsq

using namespace rmsq;

extern "C" {

int rmsnorm_fp8(int64_t rows, int64_t hidden, int in_dtype, const void* x, const void* gamma, float eps,
                float weight_offset, float scale_ub, int out_fp8, void* out, int scales_dtype, void* scales,
                hipStream_t stream) {
    return fp8_common(rows, hidden, in_dtype, x, hidden, nullptr, hidden, nullptr, hidden, false, gamma, eps,
                      weight_offset, scale_ub, out_fp8, out, hidden, scales_dtype, scales, stream);
}

int residual_rmsnorm_fp8(int64_t rows, int64_t hidden, int in_dtype, const void* x, const void* residual,
                         void* residual_out, const void* gamma, float eps, float weight_offset, float scale_ub,
                         int out_fp8, void* out, int scales_dtype, void* scales, hipStream_t stream) {
    return fp8_common(rows, hidden, in_dtype, x, hidden, residual, hidden, residual_out, hidden, true, gamma, eps,
                      weight_offset, scale_ub, out_fp8, out, hidden, scales_dtype, scales, stream);
}

int allreduce_residual_rmsnorm_fp8(int64_t rows, int64_t hidden, int in_dtype, int ninputs,
                                   const void* const* input_buffers, const void* residual, void* residual_out,
                                   const void* gamma, float eps, float weight_offset, float scale_ub, int out_fp8,
                                   void* out, int scales_dtype, void* scales, hipStream_t stream) {
    return sum_common(rows, hidden, in_dtype, ninputs, input_buffers, residual, residual_out, gamma, eps,
                      weight_offset, scale_ub, out_fp8, out, scales_dtype, scales, stream);
}

int gated_rmsnorm_fp8(int64_t rows, int64_t hidden, int in_dtype, const void* a, const void* b, const void* gamma,
                      float eps, float weight_offset, float scale_ub, int out_fp8, void* out, int scales_dtype,
                      void* scales, hipStream_t stream) {
    if (!valid_dtype(in_dtype) || !valid_dtype(scales_dtype)) return RMSQ_ERR_DTYPE;
    if (out_fp8 != RMSQ_E4M3FN && out_fp8 != RMSQ_E4M3FNUZ) return RMSQ_ERR_DTYPE;
    const int64_t esz = elem_size(in_dtype), epv = elems_per_vec(in_dtype);
    if (rows < 0 || hidden <= 0 || hidden % epv != 0 || !size_ok(rows, hidden, esz)) return RMSQ_ERR_SHAPE;
    if (int rc = check_scalars(eps, weight_offset, scale_ub, true)) return rc;
    const int64_t nvec = hidden / epv;
    if (nvec > kMaxVec) return RMSQ_ERR_UNSUPPORTED;
    if (rows == 0) return RMSQ_OK;
    if (!a || !b || !gamma || !out || !scales) return RMSQ_ERR_NULL;
    const int64_t ssz = elem_size(scales_dtype);
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(gamma, 16) || !aligned(out, 16) ||
        !aligned(scales, (uintptr_t)ssz))
        return RMSQ_ERR_ALIGN;
    const int64_t rb = rows * hidden * esz;
    const Span sa(a, rb), sb(b, rb), sg(gamma, hidden * esz), so(out, rows * hidden), ss(scales, rows * ssz);
    // the outputs overlap no input and not each other; a and b may share
    // memory (they are only read)
    for (const Span& o : {so, ss})
        if (overlap(o, sa) || overlap(o, sb) || overlap(o, sg)) return RMSQ_ERR_ALIAS;
    if (overlap(so, ss)) return RMSQ_ERR_ALIAS;
    Shape shape;
    if (!choose_shape(rows, (int)nvec, kPathFp8, (int)esz, &shape)) return RMSQ_ERR_UNSUPPORTED;
    FusedArgs fa{};
    fa.gamma = gamma;
    fa.out = out;
    fa.scales = scales;
    fa.rows = rows;
    fa.hidden = (int32_t)hidden;
    fa.inv_hidden = 1.0 / (double)hidden;
    fa.nvec = (int32_t)nvec;
    fa.eps = eps;
    fa.weight_offset = weight_offset;
    fa.scale_ub = scale_ub;
    fa.scales_dtype = scales_dtype;
    fa.x_stride = hidden * esz;
    fa.out_stride = hidden;
    return launched(launch_fp8_gated(fa, a, b, in_dtype, out_fp8 == RMSQ_E4M3FNUZ, shape, stream));
}

int rmsnorm_fp8_strided(int64_t rows, int64_t hidden, int in_dtype, const void* x, int64_t x_stride,
                        const void* residual, int64_t residual_stride, void* residual_out,
                        int64_t residual_out_stride, const void* gamma, float eps, float weight_offset,
                        float scale_ub, int out_fp8, void* out, int64_t out_stride, int scales_dtype, void* scales,
                        hipStream_t stream) {
    return fp8_common(rows, hidden, in_dtype, x, x_stride, residual, residual_stride, residual_out,
                      residual_out_stride, residual != nullptr, gamma, eps, weight_offset, scale_ub, out_fp8, out,
                      out_stride, scales_dtype, scales, stream);
}

int64_t rmsq_fp4_scale_bytes(int64_t rows, int64_t hidden, int block_size, int scale_layout) {
    if (block_size != 16 && block_size != 32) return RMSQ_ERR_VALUE;
    if (scale_layout != RMSQ_SF_ROW_MAJOR && scale_layout != RMSQ_SF_SWIZZLED) return RMSQ_ERR_DTYPE;
    if (rows < 0 || hidden <= 0 || hidden % block_size != 0 || !size_ok(rows, hidden, 2)) return RMSQ_ERR_SHAPE;
    const int64_t nsf = hidden / block_size;
    if (scale_layout == RMSQ_SF_ROW_MAJOR) return rows * nsf;
    return ceil_div(rows, 128) * ceil_div(nsf, 4) * 512;
}

int rmsnorm_fp4quant(int64_t rows, int64_t hidden, int in_dtype, const void* x, const void* gamma, float eps,
                     float weight_offset, const float* global_scale, int block_size, int scale_format,
                     int scale_layout, int flags, void* out, void* block_scales, hipStream_t stream) {
    return fp4_common(rows, hidden, in_dtype, x, hidden, nullptr, hidden, nullptr, hidden, false, gamma, eps,
                      weight_offset, global_scale, block_size, scale_format, scale_layout, flags, out, hidden / 2,
                      block_scales, stream);
}

int residual_rmsnorm_fp4quant(int64_t rows, int64_t hidden, int in_dtype, const void* x, const void* residual,
                              void* residual_out, const void* gamma, float eps, float weight_offset,
                              const float* global_scale, int block_size, int scale_format, int scale_layout,
                              int flags, void* out, void* block_scales, hipStream_t stream) {
    return fp4_common(rows, hidden, in_dtype, x, hidden, residual, hidden, residual_out, hidden, true, gamma, eps,
                      weight_offset, global_scale, block_size, scale_format, scale_layout, flags, out, hidden / 2,
                      block_scales, stream);
}

int rmsnorm_fp4quant_strided(int64_t rows, int64_t hidden, int in_dtype, const void* x, int64_t x_stride,
                             const void* residual, int64_t residual_stride, void* residual_out,
                             int64_t residual_out_stride, const void* gamma, float eps, float weight_offset,
                             const float* global_scale, int block_size, int scale_format, int scale_layout, int flags,
                             void* out, int64_t out_stride, void* block_scales, hipStream_t stream) {
    return fp4_common(rows, hidden, in_dtype, x, x_stride, residual, residual_stride, residual_out,
                      residual_out_stride, residual != nullptr, gamma, eps, weight_offset, global_scale, block_size,
                      scale_format, scale_layout, flags, out, out_stride, block_scales, stream);
}

int rmsnorm_fp4(int64_t rows, int64_t hidden, int in_dtype, const void* x, const void* gamma, float eps,
                float weight_offset, const float* global_scale, void* out, void* block_scales,
                hipStream_t stream) {
    return rmsnorm_fp4quant(rows, hidden, in_dtype, x, gamma, eps, weight_offset, global_scale, 16, RMSQ_SF_E4M3,
                            RMSQ_SF_ROW_MAJOR, 0, out, block_scales, stream);
}

int rmsq_convert(int kind, const void* in, void* out, int64_t n, hipStream_t stream) {
    if (kind < RMSQ_CVT_F32_TO_E4M3FN || kind > RMSQ_CVT_E4M3FN_TO_F32) return RMSQ_ERR_DTYPE;
    if (n < 0 || n > (INT64_MAX / 8)) return RMSQ_ERR_SHAPE;
    if (kind == RMSQ_CVT_F32_TO_E2M1 && (n % 2) != 0) return RMSQ_ERR_SHAPE;
    if (n == 0) return RMSQ_OK;
    if (!in || !out) return RMSQ_ERR_NULL;
    if (!aligned(in, 16) || !aligned(out, 16)) return RMSQ_ERR_ALIGN;
    const int64_t in_bytes = kind == RMSQ_CVT_E4M3FN_TO_F32 ? n : 4 * n;
    const int64_t out_bytes = kind == RMSQ_CVT_E4M3FN_TO_F32 ? 4 * n
                              : kind == RMSQ_CVT_F32_TO_E2M1 ? n / 2
                              : (kind == RMSQ_CVT_F32_TO_BF16 || kind == RMSQ_CVT_F32_TO_F16) ? 2 * n
                                                                                                : n;
    if (overlap(Span(in, in_bytes), Span(out, out_bytes))) return RMSQ_ERR_ALIAS;
    return launched(launch_convert(kind, in, out, n, stream));
}

int rmsq_set_tuning(int waves_per_row, int vectors_per_lane, int grid_blocks) {
    const bool w_ok = waves_per_row >= 0 && waves_per_row <= 16;
    const bool v_ok = vectors_per_lane == 0 || vectors_per_lane == 1 || vectors_per_lane == 2 ||
                      vectors_per_lane == 4;
    if (!w_ok || !v_ok || grid_blocks < 0) return RMSQ_ERR_VALUE;
    g_tune_waves.store(waves_per_row);
    g_tune_vpt.store(vectors_per_lane);
    g_tune_blocks.store(grid_blocks);
    return RMSQ_OK;
}

int rmsq_query_shape(int64_t rows, int64_t hidden, int in_dtype, int path, int* waves_per_row,
                     int* vectors_per_lane, int* rows_per_block) {
    if (!valid_dtype(in_dtype)) return RMSQ_ERR_DTYPE;
    if (path == kPathFp8Elem) {
        if (hidden <= 0) return RMSQ_ERR_SHAPE;
        if (hidden > kMaxElemHidden) return RMSQ_ERR_UNSUPPORTED;
        Shape s;
        if (!choose_elem_shape(rows, hidden, &s)) return RMSQ_ERR_UNSUPPORTED;
        if (waves_per_row) *waves_per_row = s.waves;
        if (vectors_per_lane) *vectors_per_lane = s.vpt;
        if (rows_per_block) *rows_per_block = s.rpb;
        return RMSQ_OK;
    }
    if (path != kPathFp8 && path != kPathFp4 && path != kPathFp4Residual && path != kPathFp8Residual &&
        path != kPathFp8Sum)
        return RMSQ_ERR_VALUE;
    // FP8 rows of any width (the vector and phased kernels hold a row in the
    // lanes of ceil(hidden / vector width) vectors); FP4 and summed-input rows
    // whole vectors.  Above 4096 vectors, rows of whole vectors (not summed
    // inputs) take the wide-row kernel.
    const bool fp8 = path == kPathFp8 || path == kPathFp8Residual;
    if (hidden <= 0 || (!fp8 && hidden % elems_per_vec(in_dtype) != 0)) return RMSQ_ERR_SHAPE;
    const int64_t nvec = ceil_div(hidden, elems_per_vec(in_dtype));
    Shape s;
    if (nvec > kMaxVec) {
        if (path == kPathFp8Sum || hidden % elems_per_vec(in_dtype) != 0 || nvec > kMaxWideVec ||
            !choose_wide_shape((int)nvec, &s))
            return RMSQ_ERR_UNSUPPORTED;
    } else if (!choose_shape(rows, (int)nvec, path, (int)elem_size(in_dtype), &s)) {
        return RMSQ_ERR_UNSUPPORTED;
    }
    if (waves_per_row) *waves_per_row = s.waves;
    if (vectors_per_lane) *vectors_per_lane = s.vpt;
    if (rows_per_block) *rows_per_block = s.rpb;
    return RMSQ_OK;
}

const char* rmsq_status_string(int status) {
    switch (status) {
    case RMSQ_OK: return "ok";
    case RMSQ_ERR_NULL: return "null pointer";
    case RMSQ_ERR_DTYPE: return "unsupported dtype or format";
    case RMSQ_ERR_SHAPE: return "invalid shape";
    case RMSQ_ERR_ALIGN: return "misaligned pointer";
    case RMSQ_ERR_VALUE: return "invalid scalar argument";
    case RMSQ_ERR_ALIAS: return "overlapping buffers";
    case RMSQ_ERR_UNSUPPORTED: return "hidden size not supported";
    case RMSQ_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

int rmsq_abi_version(void) { return RMSQ_ABI_VERSION; }

int rmsq_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
