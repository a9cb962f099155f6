// Per-row decode state updated after each sampled token, one thread per row.
//
// Top-p decay (TensorRT-LLM "Sampling", the Top-P decay bullets): the
// effective top_p is multiplied by the decay after every sampled token,
// bounded from below by top_p_min, and reset to the initial top_p when the
// reset id is sampled. Out-of-range parameters are rejected per row.
//
// Seed advance: one new seed per row per sampled token (the TT sampling
// README's seed contract; the Tunix sampler folds the decoding step into the
// key): the seed moves by the SplitMix64 increment, so successive seeds are
// the generator's successive states.
//
// Slot remap (the TT sampling README's decode update contract): new slot i
// takes the state of old slot slot_remap[i]; a gather from one array into
// another, 4- or 8-byte elements.
#include "vs_device.h"
#include "vs_kernels.h"

namespace vsk {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_topp_decay(int B, float* __restrict__ top_p,
                                                         const float* __restrict__ top_p_init,
                                                         const float* __restrict__ decay,
                                                         const float* __restrict__ top_p_min,
                                                         const int32_t* __restrict__ reset_ids,
                                                         const int32_t* __restrict__ sampled,
                                                         int32_t* __restrict__ out_status) {
  const int r = blockIdx.x * kThreads + static_cast<int>(threadIdx.x);
  if (r >= B) return;
  const float d = decay[r];
  const float lo = top_p_min ? top_p_min[r] : 1e-6f;
  const float p0 = top_p_init[r];
  const int32_t reset = reset_ids ? reset_ids[r] : -1;
  // a decay or floor outside (0, 1], an initial top_p outside [0, 1], or a
  // negative reset id other than -1 (no reset id) is rejected
  const bool bad = !(d > 0.0f && d <= 1.0f) || !(lo > 0.0f && lo <= 1.0f) ||
                   !(p0 >= 0.0f && p0 <= 1.0f) || reset < -1;
  if (out_status) out_status[r] = bad ? VS_ROW_BAD_PARAM : 0;
  const int32_t t = sampled[r];
  if (bad || t < 0) return;  // no token sampled: nothing decays
  if (reset >= 0 && t == reset) {
    top_p[r] = p0;
  } else {
    const float p = __fmul_rn(top_p[r], d);  // one rounded fp32 product
    top_p[r] = p > lo ? p : lo;
  }
}

__global__ __launch_bounds__(kThreads) void k_seed_advance(int B, uint64_t* __restrict__ seeds,
                                                           const int32_t* __restrict__ sampled) {
  const int r = blockIdx.x * kThreads + static_cast<int>(threadIdx.x);
  if (r >= B) return;
  if (!sampled || sampled[r] >= 0) seeds[r] += 0x9E3779B97F4A7C15ull;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_slot_remap(int B, int B_src,
                                                         const int32_t* __restrict__ remap,
                                                         const T* __restrict__ src,
                                                         T* __restrict__ dst,
                                                         int32_t* __restrict__ out_status) {
  const int r = blockIdx.x * kThreads + static_cast<int>(threadIdx.x);
  if (r >= B) return;
  const int32_t j = remap[r];
  if (out_status) out_status[r] = (j >= B_src) ? VS_ROW_BAD_PARAM : 0;
  if (j >= 0 && j < B_src) dst[r] = src[j];  // a negative entry: a new request, left as it is
}

}  // namespace

hipError_t launch_slot_remap(int B, int B_src, const int32_t* remap, const void* src, void* dst,
                             int elem_bytes, int32_t* out_status, hipStream_t st) {
  const dim3 grid((B + kThreads - 1) / kThreads);
  if (elem_bytes == 4)
    hipLaunchKernelGGL(k_slot_remap<uint32_t>, grid, dim3(kThreads), 0, st, B, B_src, remap,
                       static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), out_status);
  else
    hipLaunchKernelGGL(k_slot_remap<uint64_t>, grid, dim3(kThreads), 0, st, B, B_src, remap,
                       static_cast<const uint64_t*>(src), static_cast<uint64_t*>(dst), out_status);
  return hipGetLastError();
}

hipError_t launch_topp_decay(int B, float* top_p, const float* top_p_init, const float* decay,
                             const float* top_p_min, const int32_t* reset_ids,
                             const int32_t* sampled, int32_t* out_status, hipStream_t st) {
  hipLaunchKernelGGL(k_topp_decay, dim3((B + kThreads - 1) / kThreads), dim3(kThreads), 0, st, B,
                     top_p, top_p_init, decay, top_p_min, reset_ids, sampled, out_status);
  return hipGetLastError();
}

hipError_t launch_seed_advance(int B, uint64_t* seeds, const int32_t* sampled, hipStream_t st) {
  hipLaunchKernelGGL(k_seed_advance, dim3((B + kThreads - 1) / kThreads), dim3(kThreads), 0, st, B,
                     seeds, sampled);
  return hipGetLastError();
}

}  // namespace vsk
