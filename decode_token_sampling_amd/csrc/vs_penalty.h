// Occurrence penalties of one row over a range of ids, applied in place by one
// workgroup: shared by the penalty kernel (the whole row) and the streaming
// pass when it applies the penalties itself (the ids of its segment).
//
// The history of a row is its prompt ids followed by its output ids (CSR). The
// workgroup counts the occurrences of the ids in [lo, hi) in an LDS
// open-addressing hash table and then rewrites each distinct id's logit once:
// repetition (divide a non-negative logit, multiply a negative one), presence,
// frequency times the count, each a separately rounded fp32 operation
// (TensorRT-LLM "Sampling", occurrence-penalty bullets). With a prompt ignore
// length n (the prompt_ignore_length bullet), the first n prompt ids still put
// their id in the table, so that the repetition step applies, but add nothing
// to its count; presence and frequency apply to ids whose count is positive.
// Without one every id in the table has a positive count. More distinct ids
// than the table holds are processed in hash classes: the ids whose hash falls
// in one class are counted and applied together, and a class that still
// overflows is split in two; no id is ever applied twice.
#pragma once

#include "vs_device.h"

namespace vsk {

// One row's penalty inputs.
struct PenRow {
  const int32_t* pids;
  const int32_t* oids;
  int p0, lp;  // prompt ids [p0, p0 + lp)
  int o0, lo;  // output ids [o0, o0 + lo)
  float pres, freq, rep;
  bool bad;    // a bad parameter: the row is left unchanged
  int nign;    // prompt ids [0, nign) count for repetition only
  __device__ __forceinline__ int len() const { return lp + lo; }
  __device__ __forceinline__ int32_t id(int i) const {
    return i < lp ? pids[p0 + i] : oids[o0 + (i - lp)];
  }
};

__device__ __forceinline__ PenRow pen_row(int row, const int32_t* pids, const int32_t* poff,
                                          const int32_t* oids, const int32_t* ooff,
                                          const float* presence, const float* frequency,
                                          const float* repetition, const int32_t* pignore) {
  PenRow p;
  p.pids = pids;
  p.oids = oids;
  p.pres = presence ? presence[row] : 0.0f;
  p.freq = frequency ? frequency[row] : 0.0f;
  p.rep = repetition ? repetition[row] : 1.0f;
  p.bad = !(p.rep > 0.0f && p.rep <= 3.40282347e38f) || !(fabsf(p.pres) <= 3.40282347e38f) ||
          !(fabsf(p.freq) <= 3.40282347e38f);
  p.p0 = (pids && poff) ? poff[row] : 0;
  p.lp = (pids && poff) ? poff[row + 1] - p.p0 : 0;
  p.o0 = (oids && ooff) ? ooff[row] : 0;
  p.lo = (oids && ooff) ? ooff[row + 1] - p.o0 : 0;
  // the prompt ids [0, nign) count for repetition only (clamped to the prompt)
  p.nign = pignore ? min(max(pignore[row], 0), p.lp) : 0;
  return p;
}

// The workgroup's scalars for penalize_range (LDS).
struct PenSh {
  int overflow, badid, top;
  int stack_lq[64];
  uint32_t stack_q[64];
};

template <typename E>
__device__ __forceinline__ void store_penalised(E* p, float y);
template <>
__device__ __forceinline__ void store_penalised<float>(float* p, float y) { *p = y; }
template <>
__device__ __forceinline__ void store_penalised<uint16_t>(uint16_t* p, float y) {
  *p = f32_to_bf16(y);
}

// Applies the row's penalties to its ids in [lo, hi) in place (rowp: the row's
// logits). keys / counts: LDS tables of 2^kMaxLog2 slots. Returns, in every
// thread, whether the history holds an id outside [0, V) (when check_bad is
// set). Called by the whole workgroup (NT threads); barriers inside.
template <typename E, int kMaxLog2>
__device__ __forceinline__ bool penalize_range(E* rowp, const PenRow& pr, int V, int lo, int hi,
                                               bool check_bad, uint32_t* keys, uint32_t* counts,
                                               PenSh& ps, int NT) {
  constexpr uint32_t kEmpty = 0xffffffffu;
  const int L = pr.len();  // an upper bound on the range's distinct ids
  const int n = L;
  // The table in use: the smallest power of two of at least twice the
  // history, between 2^10 and 2^kMaxLog2 slots (clearing and scanning it is
  // most of the work for short histories).
  int lgs = 10 < kMaxLog2 ? 10 : kMaxLog2;
  while ((1 << lgs) < 2 * n && lgs < kMaxLog2) ++lgs;
  const int S = 1 << lgs;
  constexpr int kOwnMax = 4;  // history entries a thread holds at once
  if (2 * n <= S && L <= kOwnMax * NT) {  // uniform
    // One class, as below, with the history in registers: each thread's
    // entries are loaded before the table is cleared, and the thread whose
    // insert claims an id's slot (one per distinct id) loads that id's logit
    // at once, so that both loads overlap the table's work; after the barrier
    // that completes the counts, each owner applies its ids' penalties.
    int32_t hid[kOwnMax];
#pragma unroll
    for (int r = 0; r < kOwnMax; ++r) {
      const int i = static_cast<int>(threadIdx.x) + r * NT;
      hid[r] = i < L ? pr.id(i) : 0;
    }
    for (int i = threadIdx.x; i < S; i += NT) {
      keys[i] = kEmpty;
      counts[i] = 0u;
    }
    if (threadIdx.x == 0) ps.badid = 0;
    __syncthreads();  // the table and the flag are clear
    uint32_t own[kOwnMax];
    float ox[kOwnMax];
#pragma unroll
    for (int r = 0; r < kOwnMax; ++r) {
      own[r] = kEmpty;
      ox[r] = 0.0f;
      const int i = static_cast<int>(threadIdx.x) + r * NT;
      const int32_t id = hid[r];
      if (i >= L) continue;
      if (check_bad && (id < 0 || id >= V)) ps.badid = 1;
      if (pr.bad || id < lo || id >= hi) continue;
      const uint32_t u = static_cast<uint32_t>(id);
      uint32_t slot = (u * 0x2545F491u) >> (32 - lgs);
      while (true) {
        const uint32_t prev = atomicCAS(&keys[slot], kEmpty, u);
        if (prev == kEmpty || prev == u) {
          if (prev == kEmpty) {  // this thread owns the id
            own[r] = slot;
            ox[r] = to_f32(rowp[id]);
          }
          if (i >= pr.nign) atomicAdd(&counts[slot], 1u);
          break;
        }
        slot = (slot + 1) & static_cast<uint32_t>(S - 1);
      }
    }
    __syncthreads();  // every id is counted, the flag final
#pragma unroll
    for (int r = 0; r < kOwnMax; ++r) {
      if (own[r] == kEmpty) continue;
      const uint32_t c = counts[own[r]];
      const float x = ox[r];
      float y = (x >= 0.0f) ? x / pr.rep : x * pr.rep;
      if (c > 0u) {
        y = y - pr.pres;
        const float fc = pr.freq * static_cast<float>(c);
        y = y - fc;
      }
      store_penalised<E>(rowp + hid[r], y);
    }
    return ps.badid != 0;
  }
  if (2 * n <= S) {  // uniform
    // One class: the table holds every distinct id with half its slots to
    // spare, so no probe sequence can fail. Clear, count, apply, with two
    // barriers.
    for (int i = threadIdx.x; i < S; i += NT) {
      keys[i] = kEmpty;
      counts[i] = 0u;
    }
    if (threadIdx.x == 0) ps.badid = 0;
    __syncthreads();  // the table and the flag are clear
    for (int i = threadIdx.x; i < L; i += NT) {
      const int32_t id = pr.id(i);
      if (check_bad && (id < 0 || id >= V)) ps.badid = 1;
      if (pr.bad || id < lo || id >= hi) continue;
      const uint32_t u = static_cast<uint32_t>(id);
      uint32_t slot = (u * 0x2545F491u) >> (32 - lgs);
      while (true) {
        const uint32_t prev = atomicCAS(&keys[slot], kEmpty, u);
        if (prev == kEmpty || prev == u) {
          if (i >= pr.nign) atomicAdd(&counts[slot], 1u);
          break;
        }
        slot = (slot + 1) & static_cast<uint32_t>(S - 1);
      }
    }
    __syncthreads();  // every id is counted, the flag final
    for (int i = threadIdx.x; i < S; i += NT) {
      const uint32_t id = keys[i];
      if (id == kEmpty) continue;
      const uint32_t c = counts[i];
      E* p = rowp + id;
      const float x = to_f32(*p);
      float y = (x >= 0.0f) ? x / pr.rep : x * pr.rep;
      if (c > 0u) {
        y = y - pr.pres;
        const float fc = pr.freq * static_cast<float>(c);
        y = y - fc;
      }
      store_penalised<E>(p, y);
    }
    return ps.badid != 0;
  }
  if (threadIdx.x == 0) {
    ps.badid = 0;
    ps.top = 0;
  }
  __syncthreads();  // the flag is cleared before any thread can set it
  if (check_bad) {
    for (int i = threadIdx.x; i < L; i += NT) {
      const int32_t id = pr.id(i);
      if (id < 0 || id >= V) ps.badid = 1;
    }
  }
  if (threadIdx.x == 0 && !pr.bad && n > 0) {
    // start with enough classes for about half a table of ids each; push every
    // class of that level (in reverse so class 0 pops first); at most 32
    // entries, longer histories are split further on overflow
    int lq = 0;
    while ((static_cast<int64_t>(S / 2) << lq) < n && lq < 31) ++lq;
    const int lqe = lq < 5 ? lq : 5;
    for (int q = (1 << lqe) - 1; q >= 0; --q) {
      ps.stack_lq[ps.top] = lqe;
      ps.stack_q[ps.top] = static_cast<uint32_t>(q);
      ++ps.top;
    }
  }
  while (true) {
    __syncthreads();  // (the first time: the bad-id flag and the stack are complete)
    const int top = ps.top;
    if (top == 0) break;
    const int lq = ps.stack_lq[top - 1];
    const uint32_t q = ps.stack_q[top - 1];
    for (int i = threadIdx.x; i < S; i += NT) {
      keys[i] = kEmpty;
      counts[i] = 0u;
    }
    __syncthreads();  // every thread has read the stack top before it is popped
    if (threadIdx.x == 0) {
      ps.overflow = 0;
      ps.top = top - 1;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < L; i += NT) {
      const int32_t id = pr.id(i);
      if (id < lo || id >= hi) continue;
      const uint32_t u = static_cast<uint32_t>(id);
      // class: the top lq bits of one hash; slot: the top lgs bits of another
      if (lq != 0 && ((u * 0x9E3779B1u) >> (32 - lq)) != q) continue;
      uint32_t slot = (u * 0x2545F491u) >> (32 - lgs);
      int probes = 0;
      while (true) {
        const uint32_t prev = atomicCAS(&keys[slot], kEmpty, u);
        if (prev == kEmpty || prev == u) {
          if (i >= pr.nign) atomicAdd(&counts[slot], 1u);
          break;
        }
        slot = (slot + 1) & static_cast<uint32_t>(S - 1);
        if (++probes >= S) {
          ps.overflow = 1;
          break;
        }
      }
    }
    __syncthreads();
    if (ps.overflow) {
      // split the class in two (the next hash bit) and retry both halves
      if (threadIdx.x == 0) {
        const int t = ps.top;
        ps.stack_lq[t] = lq + 1;
        ps.stack_q[t] = 2 * q + 1;
        ps.stack_lq[t + 1] = lq + 1;
        ps.stack_q[t + 1] = 2 * q;
        ps.top = t + 2;
      }
      continue;
    }
    for (int i = threadIdx.x; i < S; i += NT) {
      const uint32_t id = keys[i];
      if (id == kEmpty) continue;
      const uint32_t c = counts[i];
      E* p = rowp + id;
      const float x = to_f32(*p);
      float y = (x >= 0.0f) ? x / pr.rep : x * pr.rep;
      if (c > 0u) {
        y = y - pr.pres;
        const float fc = pr.freq * static_cast<float>(c);
        y = y - fc;
      }
      store_penalised<E>(p, y);
    }
  }
  return ps.badid != 0;
}

}  // namespace vsk
