// Internal interface between the C-ABI layer (rmsq_api.cpp) and the kernel
// translation units.  Not installed; the public interface is include/rmsq.h.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace rmsq {

// Argument block passed by value to the fused kernels.  All checks are done
// by the API layer before this is built.
struct FusedArgs {
    const void* x;
    const void* residual;      // residual variants only
    void* residual_out;        // residual variants only
    const void* gamma;
    void* out;                 // FP8: [rows, hidden]; FP4: [rows, hidden/2]
    void* scales;              // FP8: [rows]; FP4: [rows, hidden/block] or swizzled
    const float* global_scale; // FP4 E4M3 scales only; may be null (1.0)
    int64_t rows;
    double inv_hidden;         // 1.0 / hidden
    int32_t hidden;
    int32_t nvec;              // hidden / elements per 16-byte vector
    float eps;
    float weight_offset;
    float scale_ub;            // FP8 only
    int32_t scales_dtype;      // FP8 only (RMSQ_F32/F16/BF16)
    int32_t waves;             // wavefronts per row (set by the launcher)
    int32_t sf_swizzled;       // FP4: 1 for the 128x4-tile scale layout
    int32_t sf_k_tiles;        // FP4 swizzled: ceil((hidden / block) / 4)
    int32_t round_product;     // FP4: round s * g' to the input type (page numerics)
    // bytes between consecutive rows of each row tensor (16-byte multiples
    // for the vector kernels, element multiples for the FP8 element path;
    // the contiguous values unless a strided entry point set them)
    int64_t x_stride;
    int64_t residual_stride;
    int64_t residual_out_stride;
    int64_t out_stride;
};

// Several input buffers summed in front of the residual FP8 path (at most
// 8, the page's signal array size): `a` as for the residual FP8 kernel
// (a.x unused), inputs[0 .. ninputs-1] the buffers.
constexpr int kMaxSumInputs = 8;
struct SumArgs {
    FusedArgs a;
    const void* inputs[kMaxSumInputs];
    int32_t ninputs;
};

// FP4 variant: elements per block scale and the scale format.
struct Fp4Format {
    int block;   // 16 or 32
    bool ue8m0;  // UE8M0 power-of-two scales (else E4M3)
};

// Launch shape: one row is handled by `waves` wavefronts (64 lanes each, any
// count 1..16), each lane holding `vpt` 16-byte vectors of the row (on the
// FP8 element path: `vpt` single elements, one of kElemPerLane; on the FP4
// path, vpt above 4 selects the wave-per-row kernel with one wavefront per
// row and vpt one of kWaveRowVpt); a block holds `rpb` rows (waves * rpb
// wavefronts); `grid` blocks (0 = default).
struct Shape {
    int waves;
    int vpt;
    int rpb;
    int grid;
};

// Vectors per lane the wave-per-row FP4 kernel is compiled for (rows of 257
// to 768 vectors of 16-bit elements, without a residual, large batches).
constexpr int kWaveRowVpt[] = {8, 12};

// Which fused path a shape is chosen for (the rmsq_query_shape `path` values).
enum { kPathFp8 = 0, kPathFp4 = 1, kPathFp4Residual = 2, kPathFp8Elem = 3, kPathFp8Residual = 5, kPathFp8Sum = 6 };

// Batches of up to this many rows are latency bound (shapes and kernel
// variants are chosen for the time of one call); larger ones stream.
constexpr int64_t kLatencyRows = 256;

// Widest row of the vector kernels (16 waves x 4 vectors per lane); wider
// rows of whole vectors take the wide-row kernels.
constexpr int kMaxVec = 16 * 64 * 4;

// Pick the automatic shape for a row of nvec 16-byte vectors of esz-byte
// elements (or apply the process-wide override).  Returns false if no
// supported shape holds the row.
bool choose_shape(int64_t rows, int nvec, int path, int esz, Shape* s);

// Shape of the wide-row kernels (16 waves, the row in LDS or registers; vpt
// reports the vectors per lane they walk): false if a forced wave count other than 16 or
// a forced vectors per lane is set, or the row exceeds kMaxWideVec.
bool choose_wide_shape(int nvec, Shape* s);

// Elements per lane the FP8 element kernel is compiled for, and the widest
// row it holds (16 waves x 64 lanes x 16 elements; more per lane would spill
// the 128 VGPRs a 1024-thread block allows).
constexpr int kElemPerLane[] = {1, 2, 4, 8, 12, 16};
constexpr int64_t kMaxElemHidden = 16 * 64 * 16;

// Shape for the FP8 element path (honours the override's wave count and
// grid; its vectors per lane do not apply).  False if no shape holds the row.
bool choose_elem_shape(int64_t rows, int64_t hidden, Shape* s);

// Kernel launchers (no argument checks).  Return the hipError_t of the launch.
// gated_rmsnorm_fp8: the FP8 kernel without a residual over x = a * b
// (rmsq_fp8_gated.hip; `fa.x` unused).
hipError_t launch_fp8_gated(const FusedArgs& fa, const void* a, const void* b, int in_dtype, bool fnuz, Shape s,
                            hipStream_t stream);
hipError_t launch_fp8(const FusedArgs& a, int in_dtype, bool residual, int out_fp8,
                      Shape shape, hipStream_t stream);
hipError_t launch_fp8_phased(const FusedArgs& a, int in_dtype, bool residual, int out_fp8, Shape shape,
                             hipStream_t stream);
hipError_t launch_fp8_elem(const FusedArgs& a, int in_dtype, bool residual, int out_fp8, Shape shape,
                           hipStream_t stream);
hipError_t launch_fp8_sum(const SumArgs& sa, int in_dtype, int out_fp8, Shape shape, hipStream_t stream);
hipError_t launch_fp4(const FusedArgs& a, int in_dtype, bool residual, Fp4Format fmt, Shape shape,
                      hipStream_t stream);
hipError_t launch_convert(int kind, const void* in, void* out, int64_t n, hipStream_t stream);

// Rows wider than the register-resident kernels hold (more than 4096
// vectors) run the wide-row kernels (the row staged in LDS, or held in
// registers without a residual): up to this many 16-byte vectors per row
// (158 KiB of gfx950's 160 KiB of LDS per workgroup; 80896 16-bit or 40448
// fp32 elements), whole vectors and 16-byte aligned tensors only.
constexpr int kMaxWideVec = 158 * 1024 / 16;
// Output of the wide-row kernel: FP8 e4m3fn or e4m3fnuz codes with a per-row
// scale, or FP4 (the format from Fp4Format).
enum { kWideFp8 = 0, kWideFp8Fnuz = 1, kWideFp4 = 2 };
// grid_blocks: 0 = one block per resident slot (the row count at most).
hipError_t launch_wide(const FusedArgs& a, int in_dtype, bool residual, int out, Fp4Format fmt, int grid_blocks,
                       hipStream_t stream);

// Occupancy-based persistent grid size for a kernel with that block size and
// dynamic LDS per block (cached per device, kernel and launch parameters).
int persistent_blocks(const void* kernel, int block_threads, size_t dyn_lds = 0);
// Blocks of that kernel one CU holds at once (the occupancy API's figure,
// at least 1; same cache).
int blocks_per_cu(const void* kernel, int block_threads, size_t dyn_lds = 0);

}  // namespace rmsq
