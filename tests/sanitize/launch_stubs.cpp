// Stand-ins for the kernel launchers, for the host sanitizer build of the C ABI (test
// infrastructure): the ABI's validation is what runs there, and any call that gets past
// it reaches one of these, which enqueue nothing and report a launch failure.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../mask_only_logits_amd/csrc/launch.h"

namespace mosaic {

hipError_t launch_idx_range_check(const int32_t *, int64_t, int64_t, int32_t *, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_mask_compact(const int32_t *, int64_t, int32_t, int32_t *, int32_t *, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_mask_compact_flags(const uint8_t *, int64_t, int32_t *, int32_t *, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_mask_compact_batched(const int32_t *, int64_t, const int32_t *, int32_t, int32_t, int32_t *,
                                       int32_t *, hipStream_t)
{
    return hipErrorInvalidValue;
}
bool gather_gemm_grid_fits(int, int64_t, int64_t) { return true; }
hipError_t launch_gather_gemm(int, const void *, const int32_t *, int64_t, const void *, int64_t, int64_t, void *,
                              int64_t, bool, int, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_gather_gemm_device_rows(const void *, const int32_t *, const int32_t *, int64_t, const void *,
                                          int64_t, int64_t, void *, int64_t, int, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_logits_argmax_lse(const void *, const int32_t *, int64_t, const void *, int64_t, int64_t, void *,
                                    int64_t, float *, int32_t *, float *, float *, int32_t *, float *, int, bool,
                                    hipStream_t, const int32_t *)
{
    return hipErrorInvalidValue;
}
hipError_t launch_quantize_rows_e4m3(const void *, bool, int64_t, const int32_t *, int64_t, uint8_t *, float *,
                                     hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_gemm_fp8(const uint8_t *, const float *, int64_t, const uint8_t *, const float *, int64_t, int64_t,
                           void *, int64_t, int, int, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_gemm_fp8_lowm(const uint8_t *, const float *, int64_t, const uint8_t *, const float *, int64_t,
                                int64_t, void *, int64_t, hipStream_t)
{
    return hipErrorInvalidValue;
}

}  // namespace mosaic
