/*
 * rmsq.h -- C ABI of librmsq: fused (residual +) RMSNorm + dynamic FP8 /
 * block-scaled FP4 quantization on AMD Instinct MI355X (gfx950).
 *
 * Operation (per row of a [rows, hidden] row-major tensor):
 *   s  = x                      or  s = round_to_in_dtype(x + residual)
 *   y  = s * rsqrt(mean(s^2) + eps) * (gamma + weight_offset)
 *   FP8: scale = min(max|y| / FMAX, scale_ub)  (FMAX 448 e4m3fn, 240 e4m3fnuz)
 *        out   = saturating round-to-nearest-even FP8 of y / scale
 *   FP4: per 16 contiguous elements, scale = min(gs * max|y| / 6, 448)
 *        rounded to E4M3; out = saturating RNE E2M1 of y * gs / scale.
 *
 * Sources: Mojo docs "rms_norm_fused_fp8" (parameters and arguments: dtype
 * lists, epsilon, weight_offset, scale_ub, per-row scale output); Mojo docs
 * "allreduce_residual_rmsnorm_fp8" (residual input, residual_output holding
 * the pre-norm sum; one GPU's local share); FlashInfer "rmsnorm_fp4quant.py"
 * (Constants; FP8 E4M3 / E2M1 conversion sections; kernel phases 2-3; the
 * rmsnorm_fp4quant API docstring for shapes, global_scale and layouts).
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or synchronizes.  Each call enqueues at most one
 *    kernel on `stream` (NULL = the null stream) and returns; results are
 *    valid once the caller has synchronized that stream.
 *  - Tensors are dense and row-major; leading dimensions are flattened into
 *    `rows` by the caller.  rows == 0 is a no-op returning RMSQ_OK.
 *  - Every argument check happens before any HIP call; on an error nothing is
 *    launched and outputs are untouched.  Input values are not checked:
 *    non-finite inputs, or eps == 0 on an all-zero row, give unspecified codes.
 *  - Calls are reentrant; concurrent calls on different streams are safe as
 *    long as their output buffers do not overlap.
 *  - Kernels run on the current HIP device, which must own the pointers and
 *    `stream`.  Host-side state: occupancy figures cached per device, kernel
 *    and launch size (mutex-guarded); before a wide-row launch the kernel's
 *    dynamic-LDS limit is raised on the current device (hipFuncSetAttribute,
 *    not a stream operation, so calls may be captured in a HIP graph); the
 *    launch-shape override of rmsq_set_tuning is process-wide.
 */
#ifndef RMSQ_H
#define RMSQ_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RMSQ_ABI_VERSION 1

/* Element types (in_dtype, scales_dtype). */
enum { RMSQ_F32 = 0, RMSQ_F16 = 1, RMSQ_BF16 = 2 };
/* FP8 output formats: OCP E4M3 (max 448, has -0) and E4M3FNUZ (bias 8,
 * max 240, no negative zero, 0x80 is NaN and never produced). */
enum { RMSQ_E4M3FN = 0, RMSQ_E4M3FNUZ = 1 };

/* Status codes. */
enum {
    RMSQ_OK = 0,
    RMSQ_ERR_NULL = -1,        /* a required pointer is NULL */
    RMSQ_ERR_DTYPE = -2,       /* unknown enum or unsupported combination */
    RMSQ_ERR_SHAPE = -3,       /* rows < 0, hidden <= 0, FP4 hidden not a multiple of
                                  the block (16 or 32), a row stride shorter than a row
                                  or off its granule, or size overflow */
    RMSQ_ERR_ALIGN = -4,       /* a tensor pointer is not aligned (FP4: 16 B for x,
                                  residual, residual_out, gamma, out; FP8: the element
                                  size for those; both: element size for scales) */
    RMSQ_ERR_VALUE = -5,       /* eps < 0 or non-finite; scale_ub <= 0 or NaN;
                                  weight_offset non-finite */
    RMSQ_ERR_ALIAS = -6,       /* an output overlaps an input or another output
                                  (other than residual_out == x or == residual) */
    RMSQ_ERR_UNSUPPORTED = -7, /* hidden above the largest row the kernels hold:
                                  80896 for 16-bit inputs, 40448 for fp32 (rows of
                                  whole, 16-byte aligned vectors; above 32768 / 16384
                                  the wide-row kernels); other FP8 layouts 32768 /
                                  16384 (phased) or 16384 (element-wise);
                                  allreduce_residual_rmsnorm_fp8 32768 / 16384; or a
                                  forced launch shape that cannot hold the row */
    RMSQ_ERR_LAUNCH = -8       /* the kernel launch failed; see rmsq_last_hip_error() */
};

/*
 * rmsnorm_fp8 -- RMSNorm + per-row dynamic FP8 quantization
 * (Mojo docs "rms_norm_fused_fp8", Args).
 *   rows, hidden : tensor shape; normalization runs over the last dimension.
 *                  Any hidden >= 1 (the page's input_fn is generic in its SIMD
 *                  width).  Four kernels compute the same results:
 *                  - rows of whole 16-byte vectors (hidden a multiple of 8
 *                    for 16-bit, 4 for fp32 input; x, gamma, out, residual,
 *                    residual_out 16-byte aligned): the vector kernel, the
 *                    row held in registers, up to 32768 16-bit / 16384 fp32
 *                    elements; wider rows up to 80896 / 40448 elements on the
 *                    wide-row kernels (one 1024-thread block per row, the
 *                    row staged in LDS, or held in registers with gamma
 *                    copied to LDS where LDS leaves room for only one
 *                    block per CU -- rows with a residual only up to 7
 *                    (16-bit FP8) or 6 vectors per lane; the same results);
 *                  - otherwise, rows that all sit at x's offset from the
 *                    16-byte grid (residual, residual_out: the same address
 *                    modulo 16 and row strides congruent modulo 16 bytes;
 *                    out: address and row stride congruent to x's element
 *                    offset and row stride modulo 8 for 16-bit, 4 for fp32
 *                    input; gamma 16-byte aligned), e.g. any hidden in
 *                    contiguous tensors: the phased kernel (0.75-0.9 of the
 *                    vector kernel's rate on the widths measured), up to the
 *                    same widths;
 *                  - anything else element-aligned: the element-wise kernel
 *                    (several times slower), hidden <= 16384.
 *   in_dtype     : RMSQ_F32 / RMSQ_F16 / RMSQ_BF16, the type of x and gamma.
 *   x            : [rows, hidden] input.
 *   gamma        : [hidden] weight; the multiplier is gamma + weight_offset,
 *                  formed in fp32 (not rounded to in_dtype).
 *   eps          : added to mean(s^2) before the reciprocal square root.
 *   scale_ub     : upper bound of the per-row scale (+inf: no bound).
 *   out_fp8      : RMSQ_E4M3FN or RMSQ_E4M3FNUZ.
 *   out          : [rows, hidden] bytes, the FP8 codes.
 *   scales_dtype : RMSQ_F32 / RMSQ_F16 / RMSQ_BF16 (RNE from the fp32 scale).
 *   scales       : [rows] dequantization scales: y ~= decode(out) * scale.  The
 *                  codes are computed with the stored (rounded) scale; a zero
 *                  scale (all-zero y) gives zero codes.
 */
int rmsnorm_fp8(int64_t rows, int64_t hidden, int in_dtype,
                const void* x, const void* gamma,
                float eps, float weight_offset, float scale_ub,
                int out_fp8, void* out, int scales_dtype, void* scales,
                hipStream_t stream);

/*
 * residual_rmsnorm_fp8 -- residual add + RMSNorm + per-row FP8 quantization:
 * one GPU's share of Mojo docs "allreduce_residual_rmsnorm_fp8" (Args:
 * residual, residual_output as the pre-norm sum).
 *   residual     : [rows, hidden] in in_dtype (the vector kernel also needs
 *                  residual and residual_out 16-byte aligned).
 *   residual_out : [rows, hidden] in in_dtype; receives s = x + residual
 *                  rounded once to in_dtype (RNE).  The normalization uses
 *                  exactly this stored s.  residual_out may be the same
 *                  pointer as x or as residual (in-place update); any other
 *                  overlap is RMSQ_ERR_ALIAS.
 *   other arguments as for rmsnorm_fp8.
 */
int residual_rmsnorm_fp8(int64_t rows, int64_t hidden, int in_dtype,
                         const void* x, const void* residual, void* residual_out,
                         const void* gamma,
                         float eps, float weight_offset, float scale_ub,
                         int out_fp8, void* out, int scales_dtype, void* scales,
                         hipStream_t stream);

/*
 * allreduce_residual_rmsnorm_fp8 -- the sum of several input buffers plus the
 * residual, then RMSNorm + per-row FP8 quantization: what Mojo docs
 * "allreduce_residual_rmsnorm_fp8" computes on each GPU (Args: input_buffers,
 * one per GPU; residual; residual_output = the pre-norm sum; output;
 * scale_output), for input buffers this GPU can already read.  It performs
 * no communication or synchronization: the buffers are device pointers to
 * local memory, or to peer memory the caller has mapped and made ready.
 *   ninputs       : 1..8 (the page's signal array holds 8 GPUs).
 *   input_buffers : HOST array of ninputs DEVICE pointers, each [rows, hidden]
 *                   in in_dtype, 16-byte aligned; they may share memory with
 *                   each other or with residual (they are only read).
 *   residual      : [rows, hidden] in in_dtype, 16-byte aligned.
 *   residual_out  : [rows, hidden]; receives s = round_to_in_dtype(residual +
 *                   sum of the inputs), the exact sum rounded once (RNE;
 *                   summed in fp64 on the GPU, exact unless the terms'
 *                   exponents span more than 53 - p bits).  May be exactly
 *                   residual (in-place update); any other overlap with an
 *                   input, gamma or an output is RMSQ_ERR_ALIAS.
 *   other arguments as for residual_rmsnorm_fp8; rows are contiguous whole
 *   16-byte vectors (hidden a multiple of 8 for 16-bit, 4 for fp32 input,
 *   else RMSQ_ERR_SHAPE).  ninputs outside 1..8 is RMSQ_ERR_VALUE.
 * With ninputs = 1 this equals residual_rmsnorm_fp8(x = input_buffers[0]).
 */
int allreduce_residual_rmsnorm_fp8(int64_t rows, int64_t hidden, int in_dtype, int ninputs,
                                   const void* const* input_buffers, const void* residual,
                                   void* residual_out, const void* gamma,
                                   float eps, float weight_offset, float scale_ub,
                                   int out_fp8, void* out, int scales_dtype, void* scales,
                                   hipStream_t stream);

/*
 * gated_rmsnorm_fp8 -- RMSNorm + per-row FP8 quantization of rows produced
 * while they are loaded: x = a * b element by element, rounded once to
 * in_dtype (RNE), never stored.  This is rms_norm_fused_fp8 with an input_fn
 * (Mojo docs "rms_norm_fused_fp8", Parameters: input_fn, the function that
 * loads input values) that multiplies the gate and up projections of a
 * gated MLP (the activation applied upstream); C++ callers can feed the same
 * kernel from a producer of their own (include/rmsq_fused.hpp).
 *   a, b    : [rows, hidden] in in_dtype, 16-byte aligned, rows adjacent;
 *             they may share memory (they are only read).  The product is
 *             formed in fp32: for 16-bit operands it is exact (unless below
 *             2^-126 in magnitude, bf16 only) and then rounded once; for
 *             fp32 operands the multiply rounds once.
 *   hidden  : a multiple of 8 (16-bit) or 4 (fp32), at most 4096 16-byte
 *             vectors (RMSQ_ERR_UNSUPPORTED above).
 *   out     : [rows, hidden], 16-byte aligned; out and scales overlap
 *             neither a, b, gamma nor each other (RMSQ_ERR_ALIAS).
 *   other arguments and the result as rmsnorm_fp8 of x.
 */
int gated_rmsnorm_fp8(int64_t rows, int64_t hidden, int in_dtype,
                      const void* a, const void* b, const void* gamma,
                      float eps, float weight_offset, float scale_ub,
                      int out_fp8, void* out, int scales_dtype, void* scales,
                      hipStream_t stream);

/*
 * rmsnorm_fp4 -- RMSNorm + block-scaled FP4 (NVFP4-style) quantization:
 * FlashInfer "rmsnorm_fp4quant.py" (rmsnorm_fp4quant, block_size 16, E4M3
 * scale factors, row-major scale layout).
 *   in_dtype     : RMSQ_BF16 or RMSQ_F16 (the page's inputs), or RMSQ_F32
 *                  (an extension; the same arithmetic on fp32 rows).
 *   hidden       : multiple of 16.
 *   weight_offset: added to gamma (0 gives the page's operation).
 *   global_scale : DEVICE pointer to one fp32 value gs (read by the kernel,
 *                  so it can change between graph replays), or NULL for 1.0.
 *                  Block scale = min(gs * max|y_block| / 6, 448) rounded to
 *                  E4M3; elements are quantized as y * gs / decoded_scale, so
 *                  y ~= decode(code) * decoded_scale / gs.  A zero block
 *                  scale gives zero codes.
 *   out          : [rows, hidden/2] bytes; element 2k in the low nibble of
 *                  byte k, E2M1 with the sign in bit 3.
 *   block_scales : [rows, hidden/16] E4M3FN codes, row-major.
 */
int rmsnorm_fp4(int64_t rows, int64_t hidden, int in_dtype,
                const void* x, const void* gamma,
                float eps, float weight_offset, const float* global_scale,
                void* out, void* block_scales, hipStream_t stream);

/* FP4 block-scale formats and layouts, and option flags (rmsnorm_fp4quant). */
enum { RMSQ_SF_E4M3 = 0, RMSQ_SF_UE8M0 = 1 };
enum { RMSQ_SF_ROW_MAJOR = 0, RMSQ_SF_SWIZZLED = 1 };
enum { RMSQ_FP4_ROUND_PRODUCT = 1 };

/*
 * rmsnorm_fp4quant -- the general form of rmsnorm_fp4, with the options of
 * FlashInfer "rmsnorm_fp4quant.py" (its API docstring: block_size,
 * scale_format, is_sf_swizzled_layout; section "UE8M0 Intrinsics (for
 * MXFP4)"; the kernel's swizzled scale store).
 *   block_size   : 16 or 32 elements per block scale (RMSQ_ERR_VALUE else);
 *                  hidden must be a multiple of it.
 *   scale_format : RMSQ_SF_E4M3 -- scale = min(gs * max|y_block| / 6, 448)
 *                  rounded to E4M3FN, elements quantized as y * gs / decoded
 *                  scale (the NVFP4 pairing is block 16);
 *                  RMSQ_SF_UE8M0 -- code = exponent of the smallest power of
 *                  two >= max|y_block| / 6, plus 127, clamped to [0, 255];
 *                  elements quantized as y * 2^(127 - code), and as zero for
 *                  code 0.  global_scale is not read (the MXFP4 pairing is
 *                  block 32).
 *   scale_layout : RMSQ_SF_ROW_MAJOR -- block_scales is [rows, hidden/block];
 *                  RMSQ_SF_SWIZZLED -- 128 x 4 tiles for FP4 GEMM operands:
 *                  the scale of (row, j) is at byte
 *                    (row/128) * K * 512 + (j/4) * 512 + (row%32) * 16
 *                    + ((row%128)/32) * 4 + j%4,   K = ceil((hidden/block)/4),
 *                  in a buffer of rmsq_fp4_scale_bytes() bytes; bytes of the
 *                  tiles' padding rows and columns are not written.
 *   flags        : 0, or RMSQ_FP4_ROUND_PRODUCT -- the page's numerics: its
 *                  kernel multiplies x and w as 16-bit pairs, so s * g' is
 *                  rounded once to in_dtype (RNE) before the rstd scaling.
 *                  Without it the product is exact.  Other bits:
 *                  RMSQ_ERR_VALUE.
 *   Other arguments, the code layout and the errors are as rmsnorm_fp4;
 *   RMSQ_ERR_DTYPE for an unknown scale_format or scale_layout.
 * rmsnorm_fp4(...) == rmsnorm_fp4quant(..., 16, RMSQ_SF_E4M3,
 * RMSQ_SF_ROW_MAJOR, 0, ...).
 */
int rmsnorm_fp4quant(int64_t rows, int64_t hidden, int in_dtype,
                     const void* x, const void* gamma,
                     float eps, float weight_offset, const float* global_scale,
                     int block_size, int scale_format, int scale_layout, int flags,
                     void* out, void* block_scales, hipStream_t stream);

/*
 * residual_rmsnorm_fp4quant -- rmsnorm_fp4quant of the pre-norm sum: the
 * residual input and residual_output of Mojo "allreduce_residual_rmsnorm_fp8"
 * (one GPU's share) in front of the FP4 quantizer.
 *   residual, residual_out : [rows, hidden] in in_dtype, 16-byte aligned;
 *                  residual_out = round_to_in_dtype(x + residual) (one
 *                  rounding), and that stored value is what is normalized and
 *                  quantized.  residual_out may be exactly x or exactly
 *                  residual (in-place update); any other overlap is
 *                  RMSQ_ERR_ALIAS.
 *   Everything else as rmsnorm_fp4quant.
 */
int residual_rmsnorm_fp4quant(int64_t rows, int64_t hidden, int in_dtype,
                              const void* x, const void* residual, void* residual_out,
                              const void* gamma, float eps, float weight_offset,
                              const float* global_scale, int block_size, int scale_format,
                              int scale_layout, int flags, void* out, void* block_scales,
                              hipStream_t stream);

/*
 * Strided forms -- the same operations on row tensors whose rows are not
 * adjacent (a slice of a wider buffer, rows of a larger tensor): Mojo
 * "rms_norm_fused_fp8" reads its input through an index function over a
 * rank-N shape; with the leading dims flattened to rows, a row stride per
 * tensor covers the layouts such a function describes with unit stride
 * along the row.
 *   *_stride     : distance between consecutive rows.  x, residual and
 *                  residual_out: in in_dtype elements, >= hidden; for FP4
 *                  stride * element size a multiple of 16 bytes.  out: in
 *                  bytes, >= the code bytes of a row (FP8: hidden; FP4:
 *                  hidden / 2); for FP4 a multiple of 8.  Else
 *                  RMSQ_ERR_SHAPE.  FP8 takes any such strides: rows that
 *                  start on 16-byte boundaries (element strides of 16 bytes'
 *                  multiples, out strides a multiple of 8 for 16-bit or 4 for
 *                  fp32 input) use the vector kernel, others the element-wise
 *                  kernel.
 *   residual     : NULL for no residual add (residual_out and the two
 *                  residual strides are then ignored).
 *   Aliasing is judged on each tensor's whole extent (first byte of row 0
 *   to last byte of the last row), so interleaved tensors that share an
 *   extent are rejected; residual_out may be exactly x or exactly residual
 *   only with the same row stride.  Scales stay contiguous (FP8 [rows]; FP4
 *   row-major or swizzled as rmsnorm_fp4quant).
 * With every stride at its contiguous value these equal rmsnorm_fp8 /
 * residual_rmsnorm_fp8 and rmsnorm_fp4quant / residual_rmsnorm_fp4quant.
 */
int rmsnorm_fp8_strided(int64_t rows, int64_t hidden, int in_dtype,
                        const void* x, int64_t x_stride,
                        const void* residual, int64_t residual_stride,
                        void* residual_out, int64_t residual_out_stride,
                        const void* gamma, float eps, float weight_offset, float scale_ub,
                        int out_fp8, void* out, int64_t out_stride,
                        int scales_dtype, void* scales, hipStream_t stream);
int rmsnorm_fp4quant_strided(int64_t rows, int64_t hidden, int in_dtype,
                             const void* x, int64_t x_stride,
                             const void* residual, int64_t residual_stride,
                             void* residual_out, int64_t residual_out_stride,
                             const void* gamma, float eps, float weight_offset,
                             const float* global_scale, int block_size, int scale_format,
                             int scale_layout, int flags, void* out, int64_t out_stride,
                             void* block_scales, hipStream_t stream);

/* Bytes of the block_scales buffer rmsnorm_fp4quant writes into for this
 * shape and layout (rows * hidden / block row-major; whole 128 x 4 tiles
 * swizzled), or a negative RMSQ_ERR_* for invalid arguments.  No HIP call. */
int64_t rmsq_fp4_scale_bytes(int64_t rows, int64_t hidden, int block_size, int scale_layout);

/*
 * rmsq_convert -- the device conversions the fused kernels use, applied
 * elementwise (standalone quantizers; also used to check the hardware
 * conversion semantics).  n elements of input, DEVICE pointers, 16-byte
 * aligned; n >= 0.
 *   RMSQ_CVT_F32_TO_E4M3FN   : float -> 1 byte, saturating RNE
 *   RMSQ_CVT_F32_TO_E4M3FNUZ : float -> 1 byte, saturating RNE, no -0
 *   RMSQ_CVT_F32_TO_E2M1     : float -> nibble, saturating RNE; n even,
 *                              out has n/2 bytes, element 2k in the low nibble
 *   RMSQ_CVT_F32_TO_BF16     : float -> bfloat16 bits (RNE)
 *   RMSQ_CVT_F32_TO_F16      : float -> binary16 bits (RNE)
 *   RMSQ_CVT_E4M3FN_TO_F32   : 1 byte -> float (exact decode)
 */
enum {
    RMSQ_CVT_F32_TO_E4M3FN = 0,
    RMSQ_CVT_F32_TO_E4M3FNUZ = 1,
    RMSQ_CVT_F32_TO_E2M1 = 2,
    RMSQ_CVT_F32_TO_BF16 = 3,
    RMSQ_CVT_F32_TO_F16 = 4,
    RMSQ_CVT_E4M3FN_TO_F32 = 5
};
int rmsq_convert(int kind, const void* in, void* out, int64_t n, hipStream_t stream);

/*
 * rmsq_set_tuning -- process-wide launch-shape override for subsequent calls
 * (tuning and shape cross-checks).  waves_per_row in 1..16 (wavefronts that
 * share one row; 1 and 2 put 4/waves rows in a block),
 * vectors_per_lane in {1,2,4} (each vector is 16 bytes of input),
 * grid_blocks sets the number of blocks of the row-strided grid (at most one
 * per row group).  By default the FP8 entry points launch one block per row
 * group and rmsnorm_fp4 launches max(min(groups, resident blocks),
 * ceil(groups / 4)) blocks.  0 for any field keeps the automatic choice.
 * Returns RMSQ_ERR_VALUE for an unsupported value.  A call whose hidden does
 * not fit the forced shape returns RMSQ_ERR_UNSUPPORTED.  Wide rows (above
 * 4096 vectors) always run 16 waves per row: a forced wave count other than 16,
 * or any forced vectors per lane, does not fit them; their grid defaults
 * to one block per resident slot and takes grid_blocks.
 */
int rmsq_set_tuning(int waves_per_row, int vectors_per_lane, int grid_blocks);

/* Launch shape the next call with these arguments would use (for logs).
 * path: 0 for the FP8 entry points without a residual and 5 for those with
 * one, on the vector or phased kernel (any hidden; see rmsnorm_fp8), 1 for
 * rmsnorm_fp4 / rmsnorm_fp4quant, 2 for residual_rmsnorm_fp4quant, 3 for
 * the FP8 entry points on the element-wise kernel (vectors_per_lane then
 * receives the elements per lane; rmsq_set_tuning's wave count and grid
 * apply to it, its vectors per lane do not), 6 for
 * allreduce_residual_rmsnorm_fp8.  For a wide row (whole vectors above 4096
 * of them) paths 0, 5, 1 and 2 report the wide-row kernel: 16 waves, the
 * vectors per lane it walks (ceil(vectors / 1024)), one row per block.
 * RMSQ_ERR_VALUE for another path. */
int rmsq_query_shape(int64_t rows, int64_t hidden, int in_dtype, int path,
                     int* waves_per_row, int* vectors_per_lane, int* rows_per_block);

/* Diagnostics. */
const char* rmsq_status_string(int status);
int rmsq_abi_version(void);
/* hipError_t of the last failed launch on the calling thread (0 if none). */
int rmsq_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RMSQ_H */
