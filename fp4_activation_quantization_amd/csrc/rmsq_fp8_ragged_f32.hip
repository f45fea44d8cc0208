// The f32 instantiations of the FP8 phased and element-wise kernels
// (rmsq_fp8_phased_kernel.h, rmsq_fp8_elem_kernel.h).
#include "rmsq_fp8_elem_kernel.h"
#include "rmsq_fp8_phased_kernel.h"

namespace rmsq {

template hipError_t launch_fp8_elem_typed<float>(const FusedArgs&, bool, bool, Shape, hipStream_t);
template hipError_t launch_fp8_phased_typed<float>(const FusedArgs&, bool, bool, Shape, hipStream_t);

}  // namespace rmsq
