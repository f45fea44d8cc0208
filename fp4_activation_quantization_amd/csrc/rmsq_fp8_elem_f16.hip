// The fp16 instantiation of the element-path FP8 kernel (rmsq_fp8_elem_kernel.h).
#include "rmsq_fp8_elem_kernel.h"

namespace rmsq {

template hipError_t launch_fp8_elem_typed<F16>(const FusedArgs&, bool, bool, Shape, hipStream_t);

}  // namespace rmsq
