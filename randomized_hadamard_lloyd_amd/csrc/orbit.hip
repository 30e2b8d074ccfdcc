// placeholder, replaced below
#include "tq_kernels.h"
namespace tq {
hipError_t launch_orbit_quantize(const float*, int64_t, int64_t, int, const int32_t*,
                                 const int8_t*, const OrbitCodebook&, int, uint8_t*, float*,
                                 int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_orbit_dequantize(const uint8_t*, const float*, int64_t, int64_t, int,
                                   const int32_t*, const int8_t*, const OrbitCodebook&, int,
                                   int, void*, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace tq
