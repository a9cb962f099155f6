// Test and measurement aids, built into their own library (libvs_selftest.so),
// never linked into libvs.so: the sampling kernels' device exponential E on a
// range of fp32 bit patterns (so that tests can compare it with the oracle on
// every input the method can produce), and reference kernels for the
// benchmark (below).
#include <hip/hip_runtime.h>

#include "vs_device.h"

namespace {

// Each thread takes four consecutive inputs through the four-value form of E
// (as the histogram pass evaluates it) and each one alone through the
// one-value form; it writes the four-value result where both agree bit for
// bit and NaN where they do not (no E value is NaN), so that comparing the
// output with the oracle checks both forms.
__global__ __launch_bounds__(256) void k_exp_bits(uint32_t lo_bits, uint32_t n, float* __restrict__ out) {
  const uint32_t i0 = (blockIdx.x * 256u + threadIdx.x) * 4u;
  if (i0 >= n) return;
  float t[4], e4[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) t[u] = __uint_as_float(lo_bits + i0 + static_cast<uint32_t>(u));
  vsk::pinned_exp_n<4>(t, e4);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float e1 = vsk::pinned_exp(t[u]);
    if (i0 + u < n) out[i0 + u] = __float_as_uint(e1) == __float_as_uint(e4[u]) ? e4[u] : __builtin_nanf("");
  }
}

}  // namespace

// out[i] = E(the float with bits lo_bits + i), i < n; out: n floats of device
// memory. Returns a hipError_t code (0 on success).
extern "C" int vs_selftest_exp(uint32_t lo_bits, uint32_t n, float* out, hipStream_t stream) {
  if (!out || n == 0) return static_cast<int>(hipErrorInvalidValue);
  const uint32_t blocks = (n + 1023u) / 1024u;  // four inputs per thread
  hipLaunchKernelGGL(k_exp_bits, dim3(blocks), dim3(256), 0, stream, lo_bits, n, out);
  return static_cast<int>(hipGetLastError());
}

// ---------------------------------------------------------------------------
// Reference kernels for measurement (not part of the sampling step): a plain
// streaming read of a [B, ld] matrix, and a plain SplitMix64 stream. The
// benchmark times them on the same buffers and the same device as the
// sampling kernels, so that those can be stated as a fraction of what a pure
// read, or a pure run of the random stream's integer multiplies, achieves.

namespace {

constexpr int kReadThreads = 1024;  // 16 waves, as the streaming pass uses per row
constexpr int kReadUnroll = 8;      // 16-byte loads in flight per lane

template <bool NT>
__device__ __forceinline__ uint4 ld16(const uint4* p) {
  return NT ? vsk::load16_stream(p) : vsk::load16(p);
}

// One workgroup per row: the row's row_bytes / 16 vectors read by 1024
// threads, kReadUnroll loads issued before any is used; the bits are folded
// with max so that no load can be dropped.
template <bool NT>
__global__ __launch_bounds__(kReadThreads) void k_read_rows(const char* __restrict__ base,
                                                           int64_t ld_bytes, int64_t nvec,
                                                           uint32_t* __restrict__ out) {
  const uint4* p = reinterpret_cast<const uint4*>(base + static_cast<int64_t>(blockIdx.x) * ld_bytes);
  uint32_t acc = 0;
  int64_t i = threadIdx.x;
  for (; i + (kReadUnroll - 1) * kReadThreads < nvec; i += kReadUnroll * kReadThreads) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = ld16<NT>(p + i + u * kReadThreads);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc = max(acc, max(max(v[u].x, v[u].y), max(v[u].z, v[u].w)));
  }
  for (; i < nvec; i += kReadThreads) {
    const uint4 v = ld16<NT>(p + i);
    acc = max(acc, max(max(v.x, v.y), max(v.z, v.w)));
  }
  __shared__ uint32_t s[kReadThreads / 64];
  for (int o = 32; o > 0; o >>= 1) acc = max(acc, static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), o)));
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int w = 0; w < kReadThreads / 64; ++w) a = max(a, s[w]);
    out[blockIdx.x] = a;
  }
}

// SplitMix64 output mix (the same published finaliser the sampling kernels
// use), n rounds per thread chained through the state.
__device__ __forceinline__ uint64_t sm64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Each thread computes n words b = SM(a + j) for j = 0..n-1 (independent
// rounds, as the draw computes one word per id) and folds them with xor.
__global__ __launch_bounds__(256) void k_splitmix_stream(uint64_t a0, int n, uint64_t* __restrict__ out) {
  const uint64_t a = sm64(a0 ^ (static_cast<uint64_t>(blockIdx.x * 256u + threadIdx.x) << 20));
  uint64_t acc = 0;
  for (int j = 0; j < n; j += 4) {
    acc ^= sm64(a + j);
    acc ^= sm64(a + j + 1);
    acc ^= sm64(a + j + 2);
    acc ^= sm64(a + j + 3);
  }
  out[blockIdx.x * 256u + threadIdx.x] = acc;
}

}  // namespace

// Reads rows [0, B) of a matrix with row stride ld_bytes, row_bytes per row
// (both multiples of 16; base 16-byte aligned), one 1024-thread workgroup per
// row; nt != 0 uses non-temporal loads. out: B uint32 of device memory.
// Returns a hipError_t code (0 on success).
extern "C" int vs_selftest_read_rows(const void* base, int B, int64_t row_bytes, int64_t ld_bytes,
                                     int nt, uint32_t* out, hipStream_t stream) {
  if (!base || !out || B <= 0 || row_bytes <= 0 || row_bytes % 16 || ld_bytes % 16 ||
      ld_bytes < row_bytes || reinterpret_cast<uintptr_t>(base) % 16)
    return static_cast<int>(hipErrorInvalidValue);
  if (nt)
    hipLaunchKernelGGL(k_read_rows<true>, dim3(B), dim3(kReadThreads), 0, stream,
                       static_cast<const char*>(base), ld_bytes, row_bytes / 16, out);
  else
    hipLaunchKernelGGL(k_read_rows<false>, dim3(B), dim3(kReadThreads), 0, stream,
                       static_cast<const char*>(base), ld_bytes, row_bytes / 16, out);
  return static_cast<int>(hipGetLastError());
}

// blocks x 256 threads, each computing n (a multiple of 4) SplitMix64 words.
// out: blocks * 256 uint64 of device memory.
extern "C" int vs_selftest_splitmix(int blocks, int n, uint64_t* out, hipStream_t stream) {
  if (!out || blocks <= 0 || n <= 0 || n % 4) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(k_splitmix_stream, dim3(blocks), dim3(256), 0, stream, 0x1234ull, n, out);
  return static_cast<int>(hipGetLastError());
}
