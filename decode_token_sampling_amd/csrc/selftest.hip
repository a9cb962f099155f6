// A test aid, built into its own library (libvs_selftest.so), never linked into
// libvs.so: it evaluates the sampling kernels' device exponential E on a range
// of fp32 bit patterns so that tests can compare it with the oracle on every
// input the method can produce.
#include <hip/hip_runtime.h>

#include "vs_device.h"

namespace {

__global__ __launch_bounds__(256) void k_exp_bits(uint32_t lo_bits, uint32_t n, float* __restrict__ out) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= n) return;
  out[i] = vsk::pinned_exp(__uint_as_float(lo_bits + i));
}

}  // namespace

// out[i] = E(the float with bits lo_bits + i), i < n; out: n floats of device
// memory. Returns a hipError_t code (0 on success).
extern "C" int vs_selftest_exp(uint32_t lo_bits, uint32_t n, float* out, hipStream_t stream) {
  if (!out || n == 0) return static_cast<int>(hipErrorInvalidValue);
  const uint32_t blocks = (n + 255u) / 256u;
  hipLaunchKernelGGL(k_exp_bits, dim3(blocks), dim3(256), 0, stream, lo_bits, n, out);
  return static_cast<int>(hipGetLastError());
}
