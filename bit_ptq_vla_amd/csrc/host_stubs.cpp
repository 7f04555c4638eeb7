// Host-only stand-ins for the kernel launchers of the qlin library, for the
// sanitizer build of the C ABI's argument validation (qlin_api.cpp and
// plan.cpp compiled by the host compiler with AddressSanitizer and
// UndefinedBehaviorSanitizer, no device code).  Every launcher reports that
// no kernel is available; a validation test never reaches one.

#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "qlin_internal.h"

namespace qlin {

hipError_t launch_rotate_quant(const void*, int, int64_t, int64_t, int64_t, bool, const float*, int, int, void*,
                               float*, hipStream_t) {
    return hipErrorNoBinaryForGpu;
}

hipError_t launch_quant_groups_w4(const void*, int, int64_t, int64_t, void*, void*, hipStream_t) {
    return hipErrorNoBinaryForGpu;
}

hipError_t launch_rotate_quant_table(const void*, int, int64_t, int64_t, int64_t, const float*, int, int,
                                     const float*, bool, void*, float*, hipStream_t) {
    return hipErrorNoBinaryForGpu;
}

hipError_t launch_calibrate_step_scales(const void*, int, int64_t, int64_t, int64_t, const float*, int, int,
                                        float*, hipStream_t) {
    return hipErrorNoBinaryForGpu;
}

hipError_t launch_composite_quant(const void*, int, int64_t, int64_t, int64_t, const float*, const int32_t*,
                                  const float*, int, int, void*, float*, float*, hipStream_t) {
    return hipErrorNoBinaryForGpu;
}

hipError_t launch_calibrate_composite(const void*, int, int64_t, int64_t, const float*, int, int32_t*, float*,
                                      void*, hipStream_t) {
    return hipErrorNoBinaryForGpu;
}

hipError_t launch_calibrate_fold(const void*, int, int64_t, int64_t, int64_t, bool, const void*, int, int64_t,
                                 float*, float*, hipStream_t) {
    return hipErrorNoBinaryForGpu;
}

hipError_t launch_gemm(const GemmPlan&, const void*, const float*, const void*, const float*, int64_t, int64_t,
                       int64_t, bool, bool, void*, int, int32_t*, hipStream_t) {
    return hipErrorNoBinaryForGpu;
}

hipError_t static_scratch(int32_t**) {
    return hipErrorNoBinaryForGpu;
}

hipError_t launch_gemm_geglu(const void*, const float*, const void*, const float*, int64_t, int64_t, int64_t,
                             bool, void*, int, hipStream_t) {
    return hipErrorNoBinaryForGpu;
}

hipError_t launch_gemm_f6(const GemmPlan&, const void*, const float*, const void*, const float*, int64_t,
                          int64_t, int64_t, void*, int, bool, hipStream_t) {
    return hipErrorNoBinaryForGpu;
}

hipError_t launch_gemv_w4a16(const void*, const void*, const void*, int64_t, int64_t, int64_t, int, void*,
                             hipStream_t) {
    return hipErrorNoBinaryForGpu;
}

hipError_t launch_skinny_w4a16(const void*, const void*, const void*, int64_t, int64_t, int64_t, void*,
                               hipStream_t) {
    return hipErrorNoBinaryForGpu;
}

hipError_t launch_skinny_int(const void*, const float*, const void*, const float*, int64_t, int64_t, int64_t,
                             bool, bool, void*, int, hipStream_t) {
    return hipErrorNoBinaryForGpu;
}

hipError_t launch_stream_read(const void*, int64_t, uint32_t*, int64_t, hipStream_t) {
    return hipErrorNoBinaryForGpu;
}

}  // namespace qlin
