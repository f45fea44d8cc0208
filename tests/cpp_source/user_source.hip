// A caller's own producer behind the library's FP8 kernel, through the public
// C++ template (include/rmsq_fused.hpp): x = |a| element by element, as a
// translation unit outside the library would write it.  Test infrastructure.
#include "rmsq_fused.hpp"

namespace {

// |a|: the sign bit of every element cleared (exact), rows adjacent
template <typename InT>
struct AbsRows {
    const char* a;
    int64_t stride;
    __device__ __forceinline__ uint4 operator()(int64_t row, int v) const {
        uint4 q = rmsq::load_stream(a + row * stride, v);
        const uint32_t m = rmsq::Vec<InT>::BYTES == 2 ? 0x7FFF7FFFu : 0x7FFFFFFFu;
        q.x &= m, q.y &= m, q.z &= m, q.w &= m;
        return q;
    }
};

template <typename InT>
int run(int64_t rows, int64_t hidden, const void* a, const void* gamma, float eps, float off, float ub, int fmt,
        void* out, int sdt, void* scales, hipStream_t s) {
    const AbsRows<InT> src{static_cast<const char*>(a), hidden * rmsq::Vec<InT>::BYTES};
    return rmsq::rmsnorm_fp8_from<InT>(src, rows, hidden, gamma, eps, off, ub, fmt, out, sdt, scales, s);
}

}  // namespace

// in_dtype as in rmsq.h (RMSQ_F32 / RMSQ_F16 / RMSQ_BF16); the rest as
// rmsnorm_fp8 with x = |a|
extern "C" int user_abs_rmsnorm_fp8(int64_t rows, int64_t hidden, int in_dtype, const void* a, const void* gamma,
                                    float eps, float off, float ub, int fmt, void* out, int sdt, void* scales,
                                    hipStream_t s) {
    if (in_dtype == RMSQ_F32) return run<float>(rows, hidden, a, gamma, eps, off, ub, fmt, out, sdt, scales, s);
    if (in_dtype == RMSQ_F16) return run<rmsq::F16>(rows, hidden, a, gamma, eps, off, ub, fmt, out, sdt, scales, s);
    if (in_dtype == RMSQ_BF16) return run<rmsq::BF16>(rows, hidden, a, gamma, eps, off, ub, fmt, out, sdt, scales, s);
    return RMSQ_ERR_DTYPE;
}
