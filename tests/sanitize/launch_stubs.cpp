// Host stand-ins for the HIP side of libmxfp8partial.so, for the sanitizer build of the C-ABI
// layer (abi.cpp + paths.cpp, compiled by g++ with AddressSanitizer and UBSan; see
// tests/test_host_sanitizers.py).  The launchers enqueue nothing and report success, so every
// host-side path of the ABI (validation, direction selection, path queries, whole-call checks)
// runs under the sanitizers without a GPU.  Not part of the product.
#include <hip/hip_runtime_api.h>

#include "mxfp8_internal.h"

namespace mxfp8 {

hipError_t launch_partial_amax(const Piece*, int, hipStream_t) { return hipSuccess; }
hipError_t launch_partial_cast(const Piece*, int, hipStream_t) { return hipSuccess; }
hipError_t launch_scales_and_cast(const Piece*, int, hipStream_t) { return hipSuccess; }
hipError_t launch_quantize(const Piece*, int, hipStream_t) { return hipSuccess; }
hipError_t launch_compute_scales(const Piece*, int, hipStream_t) { return hipSuccess; }
hipError_t launch_combine(void*, const void* const*, int, int64_t, int, hipStream_t) {
  return hipSuccess;
}

}  // namespace mxfp8

extern "C" const char* hipGetErrorString(hipError_t) { return "host stub"; }
