// The f32 instantiation of the summed-inputs FP8 kernel (rmsq_fp8_sum_kernel.h).
#include "rmsq_fp8_sum_kernel.h"

namespace rmsq {

template hipError_t launch_fp8_sum_typed<float>(const SumArgs&, bool, Shape, hipStream_t);

}  // namespace rmsq
