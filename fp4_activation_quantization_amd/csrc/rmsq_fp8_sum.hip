// Summed-inputs FP8 launch dispatch by input type, and the bf16 instantiation
// of its kernel (rmsq_fp8_sum_kernel.h; fp16 and fp32 in rmsq_fp8_sum_f16.hip
// and rmsq_fp8_sum_f32.hip).
#include "rmsq_fp8_sum_kernel.h"

namespace rmsq {

template hipError_t launch_fp8_sum_typed<BF16>(const SumArgs&, bool, Shape, hipStream_t);
extern template hipError_t launch_fp8_sum_typed<F16>(const SumArgs&, bool, Shape, hipStream_t);
extern template hipError_t launch_fp8_sum_typed<float>(const SumArgs&, bool, Shape, hipStream_t);

hipError_t launch_fp8_sum(const SumArgs& sa, int in_dtype, int out_fp8, Shape s, hipStream_t stream) {
    const bool fnuz = out_fp8 == 1;
    if (in_dtype == 0) return launch_fp8_sum_typed<float>(sa, fnuz, s, stream);
    if (in_dtype == 1) return launch_fp8_sum_typed<F16>(sa, fnuz, s, stream);
    return launch_fp8_sum_typed<BF16>(sa, fnuz, s, stream);
}

}  // namespace rmsq
