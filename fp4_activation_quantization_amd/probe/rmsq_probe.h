/*
 * rmsq_probe.h -- streaming reference kernels for measurement (librmsq_probe.so).
 *
 * Not part of the method and not part of librmsq's ABI: these kernels move
 * bytes with the fused kernels' access widths (16-byte non-temporal loads and
 * stores) and compute nothing, so their rates bound what a fused kernel with
 * the same traffic can reach on this GPU.  The benchmark times them beside the
 * fused kernels and takes the best configuration as the streaming ceiling.
 *
 * All pointers are DEVICE pointers owned by the caller; nothing is allocated
 * or synchronized; each call enqueues one kernel on `stream` and returns 0, or
 * a negative code before any HIP call (-1 a NULL pointer, -2 a size or
 * launch parameter out of range or overlapping chunk buffers, -3 a
 * misaligned pointer) or -4 after a failed launch.  The bytes written are
 * unspecified.
 */
#ifndef RMSQ_PROBE_H
#define RMSQ_PROBE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * rmsq_probe_chunks -- one source and one destination stream.  A unit is
 * rv chunks of `block` 16-byte vectors read, then wv chunks written (each lane
 * writes values derived from its own loads only); one block handles a unit at
 * a time, with up to `loads_in_flight` (1, 2, 4, 8 or 16) loads per lane
 * issued before any is consumed.
 *   src, dst       : 16-byte aligned, not overlapping.
 *   read_bytes, write_bytes : > 0, multiples of 16.
 *   rv, wv         : 1..64 chunks per unit.
 *   block          : 64..1024 threads, a multiple of 64.
 *   blocks_per_cu  : 0 = one block per unit (one-shot grid); else a
 *                    persistent grid of blocks_per_cu * 256 blocks.
 *   interleave     : nonzero spreads the unit's writes between its read
 *                    batches instead of after them.
 */
int rmsq_probe_chunks(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes, int rv, int wv,
                      int block, int loads_in_flight, int blocks_per_cu, int interleave, hipStream_t stream);

/*
 * rmsq_probe_rows -- the tensor layout of a fused row kernel: `rows` rows,
 * every row of each of the nin inputs read (in_row_bytes each), then every
 * row of each of the nout outputs written (out_row_bytes[o] each).  One block
 * of `block` threads per row at a time (lane l holds vectors l, l + block,
 * ... of the row: vpt of them, all loads in flight before any store), so
 * block * vpt * 16 >= in_row_bytes.
 *   nin            : 1..9 inputs, 16-byte aligned, in_row_bytes a multiple
 *                    of 16 (rows adjacent).
 *   nout           : 1..3 outputs with rows adjacent; out_row_bytes[o] a
 *                    multiple of 16 and at most in_row_bytes (16-byte stores),
 *                    or a multiple of 4 up to 4 * block (4-byte stores by the
 *                    first lanes: per-row scales).
 *   block          : 64..1024 threads, a multiple of 64; vpt 1, 2, 4 or 8,
 *                    with nin * vpt <= 16 (the loads in flight per lane).
 *   grid           : 0 = one block per row; else that many blocks striding
 *                    over the rows.
 *   flags          : bit 0 (phased) stores the first output, then waits at
 *                    a block barrier, then stores the others (a fused
 *                    kernel's residual_out before its reduction, codes after
 *                    it); bit 1 (mapped) stores an output whose row is 4 or 8
 *                    bytes per input vector in those pieces, each by the lane
 *                    holding that input vector (a fused kernel's code
 *                    stores).  Other bits: -2.
 *   lds_bytes      : dynamic LDS reserved per block and left unused
 *                    (0..64 KiB, the default limit of a kernel's dynamic
 *                    LDS): caps the blocks per CU (160 KiB of LDS each) as a
 *                    fused kernel's own footprint does.
 */
int rmsq_probe_rows(int64_t rows, int nin, const void* const* inputs, int64_t in_row_bytes, int nout,
                    void* const* outputs, const int64_t* out_row_bytes, int block, int vpt, int grid,
                    int flags, int lds_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RMSQ_PROBE_H */
