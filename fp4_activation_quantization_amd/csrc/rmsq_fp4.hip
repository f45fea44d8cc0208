// FP4 launch dispatch by input type and kernel, and the bf16 instantiation of
// the FP4 block kernel (rmsq_fp4_kernel.h; fp16 and fp32 are instantiated in
// rmsq_fp4_f16.hip and rmsq_fp4_f32.hip, the wave-per-row kernel of
// rmsq_fp4_wave_kernel.h in rmsq_fp4_wave*.hip).
#include "rmsq_fp4_wave_kernel.h"

namespace rmsq {

template hipError_t launch_fp4_typed<BF16>(const FusedArgs&, bool, Fp4Format, Shape, hipStream_t);
extern template hipError_t launch_fp4_typed<F16>(const FusedArgs&, bool, Fp4Format, Shape, hipStream_t);
extern template hipError_t launch_fp4_typed<float>(const FusedArgs&, bool, Fp4Format, Shape, hipStream_t);
extern template hipError_t launch_fp4_wave_typed<BF16>(const FusedArgs&, Fp4Format, Shape, hipStream_t);
extern template hipError_t launch_fp4_wave_typed<F16>(const FusedArgs&, Fp4Format, Shape, hipStream_t);

hipError_t launch_fp4(const FusedArgs& a, int in_dtype, bool residual, Fp4Format fmt, Shape s, hipStream_t stream) {
    // more than 4 vectors per lane: the wave-per-row kernel (16-bit rows
    // without a residual; choose_shape picks it for nothing else)
    if (s.vpt > 4 && !residual && in_dtype != 0)
        return in_dtype == 1 ? launch_fp4_wave_typed<F16>(a, fmt, s, stream)
                             : launch_fp4_wave_typed<BF16>(a, fmt, s, stream);
    if (in_dtype == 0) return launch_fp4_typed<float>(a, residual, fmt, s, stream);
    if (in_dtype == 1) return launch_fp4_typed<F16>(a, residual, fmt, s, stream);
    return launch_fp4_typed<BF16>(a, residual, fmt, s, stream);
}

}  // namespace rmsq
