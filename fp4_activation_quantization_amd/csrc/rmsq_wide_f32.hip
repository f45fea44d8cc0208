// The fp32 instantiation of the wide-row kernel (rmsq_wide_kernel.h).
#include "rmsq_wide_kernel.h"

namespace rmsq {

template hipError_t launch_wide_typed<float>(const FusedArgs&, bool, int, Fp4Format, int, hipStream_t);

}  // namespace rmsq
