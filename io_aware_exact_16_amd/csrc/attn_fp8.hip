// FP8 attention kernel: placeholder until the kernel lands; the entry point
// reports a launch failure instead of computing anything.
#include "fa_internal.h"
namespace fa {
hipError_t launch_attn_fp8(const uint8_t*, const uint8_t*, const uint8_t*, const float*, const float*, const float*,
                           void*, float*, int, int, int, float, bool, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace fa
