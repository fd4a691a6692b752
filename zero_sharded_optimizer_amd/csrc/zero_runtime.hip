// Stream-ordering helpers of the launch layer (host code; no kernels): the
// HIP runtime calls the ABI layer needs besides kernel launches.
#include <hip/hip_runtime.h>

#include "zero_launch.h"

namespace zlaunch {

const char* stream_wait(void* stream, void* event) {
  const hipError_t e = hipStreamWaitEvent(static_cast<hipStream_t>(stream),
                                          static_cast<hipEvent_t>(event), 0);
  return e == hipSuccess ? nullptr : hipGetErrorString(e);
}

}  // namespace zlaunch
