// The fp32 instantiation of the FP8 kernel (rmsq_fp8_kernel.h).
#include "rmsq_fp8_kernel.h"

namespace rmsq {

template hipError_t launch_fp8_typed<float>(const FusedArgs&, bool, bool, Shape, hipStream_t);

}  // namespace rmsq
