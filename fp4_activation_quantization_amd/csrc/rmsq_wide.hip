// Wide-row launch dispatch by input type, and the bf16 instantiation of the
// wide-row kernel (rmsq_wide_kernel.h; fp16 and fp32 are instantiated in
// rmsq_wide_f16.hip and rmsq_wide_f32.hip).
#include "rmsq_wide_kernel.h"

namespace rmsq {

template hipError_t launch_wide_typed<BF16>(const FusedArgs&, bool, int, Fp4Format, int, hipStream_t);
extern template hipError_t launch_wide_typed<F16>(const FusedArgs&, bool, int, Fp4Format, int, hipStream_t);
extern template hipError_t launch_wide_typed<float>(const FusedArgs&, bool, int, Fp4Format, int, hipStream_t);

hipError_t launch_wide(const FusedArgs& a, int in_dtype, bool residual, int out, Fp4Format fmt, int grid_blocks,
                       hipStream_t stream) {
    if (in_dtype == 0) return launch_wide_typed<float>(a, residual, out, fmt, grid_blocks, stream);
    if (in_dtype == 1) return launch_wide_typed<F16>(a, residual, out, fmt, grid_blocks, stream);
    return launch_wide_typed<BF16>(a, residual, out, fmt, grid_blocks, stream);
}

}  // namespace rmsq
