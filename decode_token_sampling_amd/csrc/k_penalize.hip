// vs_penalize: occurrence penalties in place, one 1024-thread workgroup per row.
//
// The history of a row is its prompt ids followed by its output ids (CSR). The
// workgroup counts occurrences in an LDS open-addressing hash table (of
// 2^10..2^14 slots of id and count, by the history's length) and then
// rewrites each distinct id's logit once:
// repetition (divide a non-negative logit, multiply a negative one), presence,
// frequency times the count, each a separately rounded fp32 operation
// (TensorRT-LLM "Sampling", occurrence-penalty bullets). With a prompt ignore
// length n (the prompt_ignore_length bullet), the first n prompt ids still put
// their id in the table, so that the repetition step applies, but add nothing
// to its count; presence and frequency apply to ids whose count is positive.
// Without one every id in the table has a positive count. A history with more
// distinct ids than the table holds is processed in hash classes: the ids
// whose hash falls in one class are counted and applied together, and a class
// that still overflows is split in two; no id is ever applied twice.
#include "vs_device.h"
#include "vs_kernels.h"

namespace vsk {
namespace {

constexpr int kThreads = 1024;
constexpr int kSlotsLog2 = 14;
constexpr int kSlots = 1 << kSlotsLog2;
constexpr uint32_t kEmpty = 0xffffffffu;

__device__ __forceinline__ uint32_t class_hash(uint32_t id) { return id * 0x9E3779B1u; }
// Slot of an id in a table of 2^lgs slots: the top lgs bits of its hash.
__device__ __forceinline__ uint32_t slot_hash(uint32_t id, int lgs) {
  return (id * 0x2545F491u) >> (32 - lgs);
}
// Class of an id among Q = 2^lq classes: the top lq bits of its hash.
__device__ __forceinline__ uint32_t id_class(uint32_t id, int lq) {
  return lq == 0 ? 0u : class_hash(id) >> (32 - lq);
}

template <typename E>
__device__ __forceinline__ void store_penalised(E* p, float y);
template <>
__device__ __forceinline__ void store_penalised<float>(float* p, float y) { *p = y; }
template <>
__device__ __forceinline__ void store_penalised<uint16_t>(uint16_t* p, float y) {
  *p = f32_to_bf16(y);
}

template <typename E>
__global__ __launch_bounds__(kThreads) void k_penalize(
    E* __restrict__ logits, int B, int V, int64_t ld, const int32_t* __restrict__ pids,
    const int32_t* __restrict__ poff, const int32_t* __restrict__ oids,
    const int32_t* __restrict__ ooff, const float* __restrict__ presence,
    const float* __restrict__ frequency, const float* __restrict__ repetition,
    const int32_t* __restrict__ pignore, int32_t* __restrict__ out_status) {
  __shared__ uint32_t keys[kSlots];
  __shared__ uint32_t counts[kSlots];
  __shared__ int s_overflow, s_badid;
  __shared__ int s_stack_lq[64];
  __shared__ uint32_t s_stack_q[64];
  __shared__ int s_top;

  const int row = blockIdx.x;
  const float pres = presence ? presence[row] : 0.0f;
  const float freq = frequency ? frequency[row] : 0.0f;
  const float rep = repetition ? repetition[row] : 1.0f;
  const bool bad = !(rep > 0.0f && rep <= 3.40282347e38f) || !(fabsf(pres) <= 3.40282347e38f) ||
                   !(fabsf(freq) <= 3.40282347e38f);
  const int p0 = (pids && poff) ? poff[row] : 0;
  const int lp = (pids && poff) ? poff[row + 1] - p0 : 0;
  const int o0 = (oids && ooff) ? ooff[row] : 0;
  const int lo = (oids && ooff) ? ooff[row + 1] - o0 : 0;
  const int L = lp + lo;
  // The table in use: the smallest power of two of at least twice the
  // history, between 2^10 and kSlots slots (clearing and scanning it is most
  // of the work for short histories).
  int lgs = 10;
  while ((1 << lgs) < 2 * L && lgs < kSlotsLog2) ++lgs;
  const int S = 1 << lgs;
  // the prompt ids [0, nign) count for repetition only (clamped to the prompt)
  const int nign = pignore ? min(max(pignore[row], 0), lp) : 0;
  E* rowp = logits + static_cast<int64_t>(row) * ld;

  auto hist_id = [&](int i) -> int32_t { return i < lp ? pids[p0 + i] : oids[o0 + (i - lp)]; };

  if (threadIdx.x == 0) {
    s_badid = 0;
    s_top = 0;
    if (!bad && L > 0) {
      // start with enough classes for about half a table of ids each
      int lq = 0;
      while ((static_cast<int64_t>(S / 2) << lq) < L && lq < 31) ++lq;
      // push every class of that level (in reverse so class 0 pops first);
      // at most 64 entries: lq <= 5 is enough for 2^19 history ids per row, and
      // longer histories are split further on overflow.
      const int nq = 1 << (lq < 5 ? lq : 5);
      const int lqe = lq < 5 ? lq : 5;
      for (int q = nq - 1; q >= 0; --q) {
        s_stack_lq[s_top] = lqe;
        s_stack_q[s_top] = static_cast<uint32_t>(q);
        ++s_top;
      }
    }
  }
  // the flag is cleared before any wave can set it
  __syncthreads();
  // ids outside [0, V) are skipped and reported
  for (int i = threadIdx.x; i < L; i += blockDim.x) {
    const int32_t id = hist_id(i);
    if (id < 0 || id >= V) s_badid = 1;
  }
  __syncthreads();

  while (true) {
    __syncthreads();
    const int top = s_top;
    if (top == 0) break;
    const int lq = s_stack_lq[top - 1];
    const uint32_t q = s_stack_q[top - 1];
    for (int i = threadIdx.x; i < S; i += blockDim.x) {
      keys[i] = kEmpty;
      counts[i] = 0u;
    }
    __syncthreads();  // every thread has read the stack top before it is popped
    if (threadIdx.x == 0) {
      s_overflow = 0;
      s_top = top - 1;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < L; i += blockDim.x) {
      const int32_t id = hist_id(i);
      if (id < 0 || id >= V) continue;
      const uint32_t u = static_cast<uint32_t>(id);
      if (id_class(u, lq) != q) continue;
      uint32_t slot = slot_hash(u, lgs);
      int probes = 0;
      while (true) {
        const uint32_t prev = atomicCAS(&keys[slot], kEmpty, u);
        if (prev == kEmpty || prev == u) {
          if (i >= nign) atomicAdd(&counts[slot], 1u);
          break;
        }
        slot = (slot + 1) & static_cast<uint32_t>(S - 1);
        if (++probes >= S) {
          s_overflow = 1;
          break;
        }
      }
    }
    __syncthreads();
    if (s_overflow) {
      // split the class in two (the next hash bit) and retry both halves
      if (threadIdx.x == 0) {
        const int t = s_top;
        s_stack_lq[t] = lq + 1;
        s_stack_q[t] = 2 * q + 1;
        s_stack_lq[t + 1] = lq + 1;
        s_stack_q[t + 1] = 2 * q;
        s_top = t + 2;
      }
      continue;
    }
    for (int i = threadIdx.x; i < S; i += blockDim.x) {
      const uint32_t id = keys[i];
      if (id == kEmpty) continue;
      const uint32_t n = counts[i];
      E* p = rowp + id;
      const float x = to_f32(*p);
      float y = (x >= 0.0f) ? x / rep : x * rep;
      if (n > 0u) {
        y = y - pres;
        const float fc = freq * static_cast<float>(n);
        y = y - fc;
      }
      store_penalised<E>(p, y);
    }
  }
  if (threadIdx.x == 0 && out_status)
    out_status[row] = (bad ? VS_ROW_BAD_PARAM : 0) | (s_badid ? VS_ROW_BAD_TOKEN_ID : 0);
}

}  // namespace

hipError_t launch_penalize(void* logits, vs_dtype dt, int B, int V, int64_t ld,
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
