// The bf16 instantiation of the wave-per-row FP4 kernel (rmsq_fp4_wave_kernel.h).
#include "rmsq_fp4_wave_kernel.h"

namespace rmsq {

template hipError_t launch_fp4_wave_typed<BF16>(const FusedArgs&, Fp4Format, Shape, hipStream_t);

}  // namespace rmsq
