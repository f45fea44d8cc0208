// FP8 kernels off the vector fast path -- the phased kernel
// (rmsq_fp8_phased_kernel.h) and the element-wise kernel
// (rmsq_fp8_elem_kernel.h): launch dispatch by input type and the bf16
// instantiations (fp16 and fp32 are instantiated in rmsq_fp8_ragged_f16.hip
// and rmsq_fp8_ragged_f32.hip).
#include "rmsq_fp8_elem_kernel.h"
#include "rmsq_fp8_phased_kernel.h"

namespace rmsq {

template hipError_t launch_fp8_elem_typed<BF16>(const FusedArgs&, bool, bool, Shape, hipStream_t);
extern template hipError_t launch_fp8_elem_typed<F16>(const FusedArgs&, bool, bool, Shape, hipStream_t);
extern template hipError_t launch_fp8_elem_typed<float>(const FusedArgs&, bool, bool, Shape, hipStream_t);
template hipError_t launch_fp8_phased_typed<BF16>(const FusedArgs&, bool, bool, Shape, hipStream_t);
extern template hipError_t launch_fp8_phased_typed<F16>(const FusedArgs&, bool, bool, Shape, hipStream_t);
extern template hipError_t launch_fp8_phased_typed<float>(const FusedArgs&, bool, bool, Shape, hipStream_t);

hipError_t launch_fp8_elem(const FusedArgs& a, int in_dtype, bool residual, int out_fp8, Shape s,
                           hipStream_t stream) {
    const bool fnuz = out_fp8 == 1;
    if (in_dtype == 0) return launch_fp8_elem_typed<float>(a, residual, fnuz, s, stream);
    if (in_dtype == 1) return launch_fp8_elem_typed<F16>(a, residual, fnuz, s, stream);
    return launch_fp8_elem_typed<BF16>(a, residual, fnuz, s, stream);
}

hipError_t launch_fp8_phased(const FusedArgs& a, int in_dtype, bool residual, int out_fp8, Shape s,
                             hipStream_t stream) {
    const bool fnuz = out_fp8 == 1;
    if (in_dtype == 0) return launch_fp8_phased_typed<float>(a, residual, fnuz, s, stream);
    if (in_dtype == 1) return launch_fp8_phased_typed<F16>(a, residual, fnuz, s, stream);
    return launch_fp8_phased_typed<BF16>(a, residual, fnuz, s, stream);
}

}  // namespace rmsq
