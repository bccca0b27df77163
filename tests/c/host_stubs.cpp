// Stand-ins for the kernel launchers and for the five HIP runtime calls the host code makes,
// for building the library's host code alone (plan tables, codebook solver, Philox, argument
// checks) with the host compiler under the address and undefined-behaviour sanitizers,
// without the HIP runtime.  "Device" memory is host memory here, so plan creation runs to
// the end (every table built and copied); every kernel launcher reports that there is no
// device, so a call that would launch work returns an error instead.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>

#include "../../rotation_online_vector_amd/csrc/tq_internal.h"

extern "C" {
hipError_t hipGetDeviceCount(int* count) {
  *count = 1;
  return hipSuccess;
}
hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipMalloc(void** ptr, size_t size) {
  *ptr = std::aligned_alloc(256, (size + 255) / 256 * 256);
  return *ptr ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipMemcpy(void* dst, const void* src, size_t bytes, hipMemcpyKind) {
  std::memcpy(dst, src, bytes);
  return hipSuccess;
}
hipError_t hipFree(void* ptr) {
  std::free(ptr);
  return hipSuccess;
}
}

namespace tq {

static int no_device() { return (int)hipErrorNoDevice; }

int launch_encode(const PlanDev&, int, const void*, int, int64_t, int64_t, uint8_t*, void*,
                  int64_t) { return no_device(); }
int launch_qjl(const SubDev&, const float*, int64_t, uint32_t*, void*) { return no_device(); }
int launch_score(const PlanDev&, const void*, int, int64_t, int64_t, int64_t, const uint8_t*,
                 int64_t, float*, void*) { return no_device(); }
int launch_score_noalloc(const PlanDev&, const void*, int, int64_t, int64_t, int64_t,
                         const uint8_t*, int64_t, float*, void*) { return no_device(); }
int launch_topk(const float*, int64_t, int64_t, int, int64_t*, float*, void*) { return no_device(); }
int launch_dequantize(const PlanDev&, const uint8_t*, int64_t, void*, int, int64_t, void*) {
  return no_device();
}
int launch_attend(const PlanDev&, const float*, int64_t, int64_t, int64_t, float, const uint8_t*,
                  void*, int, int64_t, void*) { return no_device(); }
int launch_rerank(const void*, int, int64_t, int64_t, const void*, int, int64_t, int64_t, int,
                  const int64_t*, int, int, int64_t*, float*, void*) { return no_device(); }
int launch_calibrate_outliers(const void*, int, int64_t, int64_t, int, int, double*, uint8_t*,
                              void*) { return no_device(); }
int launch_encode_scatter(const PlanDev&, const void*, int, int64_t, int64_t, uint8_t*, int64_t,
                          const int64_t*, void*) { return no_device(); }
int launch_score_topk(const PlanDev&, const void*, int, int64_t, int64_t, int64_t,
                      const uint8_t*, int64_t, int, int64_t*, float*, void*) { return no_device(); }

}  // namespace tq
