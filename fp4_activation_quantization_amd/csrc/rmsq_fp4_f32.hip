// The fp32 instantiation of the FP4 kernel (rmsq_fp4_kernel.h).
#include "rmsq_fp4_kernel.h"

namespace rmsq {

template hipError_t launch_fp4_typed<float>(const FusedArgs&, bool, Fp4Format, Shape, hipStream_t);

}  // namespace rmsq
