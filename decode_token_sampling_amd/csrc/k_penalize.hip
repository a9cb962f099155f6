// vs_penalize: occurrence penalties in place, one 1024-thread workgroup per
// row: the shared routine of vs_penalty.h over the row's whole id range, with
// an LDS table of up to 2^14 slots; the segment's workgroup also reports ids
// outside [0, V).
#include "vs_device.h"
#include "vs_kernels.h"
#include "vs_penalty.h"

namespace vsk {
namespace {

constexpr int kThreads = 1024;
constexpr int kSlotsLog2 = 14;
constexpr int kSlots = 1 << kSlotsLog2;

template <typename E>
__global__ __launch_bounds__(kThreads) void k_penalize(
    E* __restrict__ logits, int B, int V, int64_t ld, const int32_t* __restrict__ pids,
    const int32_t* __restrict__ poff, const int32_t* __restrict__ oids,
    const int32_t* __restrict__ ooff, const float* __restrict__ presence,
    const float* __restrict__ frequency, const float* __restrict__ repetition,
    const int32_t* __restrict__ pignore, int32_t* __restrict__ out_status) {
  __shared__ uint32_t keys[kSlots];
  __shared__ uint32_t counts[kSlots];
  __shared__ PenSh ps;
  const int row = blockIdx.x;
  const PenRow pr = pen_row(row, pids, poff, oids, ooff, presence, frequency, repetition, pignore);
  const bool bad_id = penalize_range<E, kSlotsLog2>(logits + static_cast<int64_t>(row) * ld, pr, V,
                                                    0, V, true, keys, counts, ps, kThreads);
  if (threadIdx.x == 0 && out_status)
    out_status[row] = (pr.bad ? VS_ROW_BAD_PARAM : 0) | (bad_id ? VS_ROW_BAD_TOKEN_ID : 0);
}

}  // namespace

hipError_t launch_penalize(void* logits, int dt, int B, int V, int64_t ld,
                           const int32_t* prompt_ids, const int32_t* prompt_off,
                           const int32_t* output_ids, const int32_t* output_off,
                           const float* presence, const float* frequency,
                           const float* repetition, const int32_t* prompt_ignore,
                           int32_t* out_status, hipStream_t st) {
  if (dt == VS_F32)
    hipLaunchKernelGGL(k_penalize<float>, dim3(B), dim3(kThreads), 0, st,
                       static_cast<float*>(logits), B, V, ld, prompt_ids, prompt_off, output_ids,
                       output_off, presence, frequency, repetition, prompt_ignore, out_status);
  else
    hipLaunchKernelGGL(k_penalize<uint16_t>, dim3(B), dim3(kThreads), 0, st,
                       static_cast<uint16_t*>(logits), B, V, ld, prompt_ids, prompt_off, output_ids,
                       output_off, presence, frequency, repetition, prompt_ignore, out_status);
  return hipGetLastError();
}

}  // namespace vsk
