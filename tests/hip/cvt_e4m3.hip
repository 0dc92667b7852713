// cvt_e4m3.hip -- test kernel: the library's binary32 -> OCP E4M3 conversion
// (ep::dev::e4m3_pack4, gfx950's packed FP8 convert) applied to an array of
// binary32 values, so a test can compare it code for code with the oracle's
// encoder.  TEST INFRASTRUCTURE: built beside the library, loaded only by
// tests/test_gpu_cvt.py.
//
// Page: [Perplexity blog] "Lower latency and higher throughput with multi-node
// DeepSeek deployment", "Magntölun" (activation blocks of 128 scaled by their
// amax and stored as FP8).
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "ep_device.h"

namespace {

// out[i] = the four codes of v[4i .. 4i+3] (byte j = code of v[4i+j])
__global__ __launch_bounds__(256) void cvt_e4m3_kernel(const float *__restrict__ v,
                                                       uint32_t *__restrict__ out, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) out[i] = ep::dev::e4m3_pack4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

}  // namespace

// n must be a multiple of 4; v holds n binary32 values, out n bytes (device
// pointers).  Returns the hipError_t of the launch.
extern "C" int cvt_e4m3(const float *v, uint8_t *out, int64_t n, hipStream_t s) {
  if (n <= 0 || n % 4 != 0 || !v || !out) return (int)hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  const int64_t grid = (n4 + 255) / 256;
  if (grid > 0x7FFFFFFF) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(cvt_e4m3_kernel, dim3((unsigned)grid), dim3(256), 0, s, v,
                     reinterpret_cast<uint32_t *>(out), n4);
  return (int)hipGetLastError();
}
