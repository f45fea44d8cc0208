// gated_rmsnorm_fp8: the FP8 kernel fed by the GatedProduct source
// (include/rmsq_fused.hpp), one instantiation per input type.
#include "rmsq_fused.hpp"

namespace rmsq {

hipError_t launch_fp8_gated(const FusedArgs& fa, const void* a, const void* b, int in_dtype, bool fnuz, Shape s,
                            hipStream_t stream) {
    const char *pa = static_cast<const char*>(a), *pb = static_cast<const char*>(b);
    if (in_dtype == 0) return launch_fp8_from<float>(fa, GatedProduct<float>{pa, pb, fa.x_stride}, fnuz, s, stream);
    if (in_dtype == 1) return launch_fp8_from<F16>(fa, GatedProduct<F16>{pa, pb, fa.x_stride}, fnuz, s, stream);
    return launch_fp8_from<BF16>(fa, GatedProduct<BF16>{pa, pb, fa.x_stride}, fnuz, s, stream);
}

}  // namespace rmsq
