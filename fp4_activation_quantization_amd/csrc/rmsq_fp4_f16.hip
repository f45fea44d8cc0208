// The fp16 instantiation of the FP4 kernel (rmsq_fp4_kernel.h).
#include "rmsq_fp4_kernel.h"

namespace rmsq {

template hipError_t launch_fp4_typed<F16>(const FusedArgs&, bool, Fp4Format, Shape, hipStream_t);

}  // namespace rmsq
