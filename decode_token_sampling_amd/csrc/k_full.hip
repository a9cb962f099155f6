// The parallel passes of the full-vocabulary top-p cut.
//
// A full-vocabulary row keeps the shortest prefix of its ids in the order
// (s desc, id asc) whose fixed-point mass reaches top_p of the total
// (TensorRT-LLM "Sampling", top-p; the mass and its rounding are the ones the
// oracle and the row kernels use). Both passes split each such row into
// segments read by many workgroups (all segments of a row on one XCD):
//  - the histogram pass adds every id's mass W = floor(E(s - m) 2^31) and a
//    count into 4096 buckets of t = s - m, first in LDS, then per nonempty
//    bucket into the row's histogram in the workspace (zeroed by the row
//    kernel);
//  - the gather pass finds, from that histogram, the bucket where the
//    cumulative mass (largest s first) reaches the target and the mass still
//    needed inside it, and appends the ids of that bucket (packed key and id)
//    to the row's list.
// The cut kernel then sorts the list and finds the exact cut; a bucket larger
// than the list goes to its one-workgroup path.
#include "vs_device.h"
#include "vs_kernels.h"

namespace vsk {
namespace {

constexpr int kThreads = 256;
constexpr int kPer = kFullBuckets / kThreads;  // buckets per thread (16)
constexpr int kGatherBuf = 2048;  // ids a gather workgroup collects in LDS before one global append

__device__ __forceinline__ float scaled_of(float x, float T) { return (T == 1.0f) ? x : x / T; }

// A full-vocabulary row whose top-p cut is still to be found.
__device__ __forceinline__ bool topp_row(const Job& j, int row, RowCfg* c, float* m) {
  const RowDesc d = j.desc[row];
  if (d.mode != kRowFull) return false;
  *c = load_cfg(row, j.V, j.T, j.k, j.p, j.mp, j.seeds);
  *m = d.m;
  return c->p < 1.0f;
}

// Visits the ids [lo, hi) of a row with the whole block: 16-byte loads (four
// in flight per thread) when the row is aligned (lo is a multiple of 8, so
// the segment starts on a 16-byte boundary), elements otherwise and at the
// end. f(id, x) is called by all lanes of a wave together in the vector loop.
template <typename E, typename F>
__device__ __forceinline__ void seg_visit(const E* __restrict__ rowp, int lo, int hi, bool aligned,
                                          F&& f) {
  constexpr int EPV = Epv<E>::n;
  constexpr int U = 4;
  int q0 = lo;
  if (aligned) {
    const int nvec = (hi - lo) / EPV;
    const E* base = rowp + lo;
    const int st = kThreads;
    int i = threadIdx.x;
    for (; i + (U - 1) * st < nvec; i += U * st) {
      uint4 raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) raw[u] = load16(base + (i + u * st) * EPV);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float x[EPV];
        unpack16(raw[u], x, rowp);
#pragma unroll
        for (int c = 0; c < EPV; ++c) f(lo + (i + u * st) * EPV + c, x[c]);
      }
    }
    for (; i < nvec; i += st) {
      float x[EPV];
      unpack16(load16(base + i * EPV), x, rowp);
#pragma unroll
      for (int c = 0; c < EPV; ++c) f(lo + i * EPV + c, x[c]);
    }
    q0 = lo + nvec * EPV;
  }
  for (int q = q0 + static_cast<int>(threadIdx.x); q < hi; q += kThreads) f(q, to_f32(rowp[q]));
}

template <typename E>
__global__ __launch_bounds__(kThreads) void k_full_hist(Job j) {
  __shared__ uint64_t hw[kFullBuckets];
  __shared__ uint32_t hc[kFullBuckets];
  int row, seg;
  if (!xcd_row_tile(blockIdx.x, j.B, j.fseg, &row, &seg)) return;  // uniform per block
  RowCfg c;
  float m;
  if (!topp_row(j, row, &c, &m)) return;  // uniform per block
  for (int i = threadIdx.x; i < kFullBuckets; i += kThreads) {
    hw[i] = 0ull;
    hc[i] = 0u;
  }
  __syncthreads();
  const FullTerms ft{m, c.mp};
  const E* rowp = static_cast<const E*>(j.logits) + static_cast<int64_t>(row) * j.ld;
  const int lo = seg * j.fseg_len;
  const int hi = min(j.V, lo + j.fseg_len);
  seg_visit(rowp, lo, hi, j.aligned != 0, [&](int, float x) {
    uint64_t w;
    int b;
    if (ft.mass(scaled_of(x, c.T), &w, &b)) {
      atomicAdd(reinterpret_cast<unsigned long long*>(&hw[b]), static_cast<unsigned long long>(w));
      atomicAdd(&hc[b], 1u);
    }
  });
  __syncthreads();
  uint64_t* ghw = j.fhw + static_cast<size_t>(row) * kFullBuckets;
  uint32_t* ghc = j.fhc + static_cast<size_t>(row) * kFullBuckets;
  for (int b = threadIdx.x; b < kFullBuckets; b += kThreads) {
    const uint32_t n = hc[b];
    if (n) {
      atomicAdd(reinterpret_cast<unsigned long long*>(&ghw[b]), static_cast<unsigned long long>(hw[b]));
      atomicAdd(&ghc[b], n);
    }
  }
}

template <typename E>
__global__ __launch_bounds__(kThreads) void k_full_gather(Job j) {
  __shared__ uint64_t sw[kThreads / kWave], sc[kThreads / kWave];
  __shared__ int s_bucket;
  __shared__ uint64_t s_above_w, s_above_c;
  __shared__ uint64_t sbuf[kGatherBuf];
  __shared__ uint32_t s_n, s_lim, s_base;
  int row, seg;
  if (!xcd_row_tile(blockIdx.x, j.B, j.fseg, &row, &seg)) return;  // uniform per block
  RowCfg c;
  float m;
  if (!topp_row(j, row, &c, &m)) return;  // uniform per block
  const uint64_t* ghw = j.fhw + static_cast<size_t>(row) * kFullBuckets;
  const uint32_t* ghc = j.fhc + static_cast<size_t>(row) * kFullBuckets;

  // The cut bucket: thread t holds buckets [16 t, 16 t + 16); an exclusive
  // scan over the threads gives the mass and count of the buckets before.
  uint64_t w[kPer];
  uint64_t lw = 0, lc = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    w[i] = ghw[threadIdx.x * kPer + i];
    lw += w[i];
    lc += ghc[threadIdx.x * kPer + i];
  }
  uint64_t total_w, total_c;
  uint64_t cw = block_scan_incl(lw, sw, &total_w) - lw;
  uint64_t cc = block_scan_incl(lc, sc, &total_c) - lc;
  // the kept prefix is the shortest whose mass reaches p * total; masses are
  // integers, so "cum >= thr" is "cum >= ceil(thr)" (at least one id)
  const double thr = static_cast<double>(c.p) * static_cast<double>(total_w);
  const uint64_t target = ceil(thr) >= 1.0 ? static_cast<uint64_t>(ceil(thr)) : 1ull;
  if (threadIdx.x == 0) {
    s_bucket = -1;
    s_n = 0u;
    s_lim = 0xffffffffu;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = threadIdx.x * kPer + i;
    if (cw < target && target <= cw + w[i]) {
      s_bucket = b;
      s_above_w = cw;
      s_above_c = cc;
    }
    cw += w[i];
    cc += ghc[b];
  }
  __syncthreads();
  const int bstar = s_bucket;
  if (bstar < 0) {  // uniform; unreachable (the row maximum has mass 2^31)
    // no stale record from an earlier call may stand: the cut kernel then
    // takes its one-workgroup path
    if (seg == 0 && threadIdx.x == 0) j.fcut[row].bucket = -1;
    return;
  }
  if (seg == 0 && threadIdx.x == 0)
    j.fcut[row] = FullCut{bstar, ghc[bstar], target - s_above_w, s_above_c, 0ull};

  // The ids of that bucket: collected in LDS (one LDS atomic add per wave),
  // then appended to the row's list with one global atomic add per workgroup;
  // ids beyond the LDS buffer go straight to the list, one atomic add per wave.
  const FullTerms ft{m, c.mp};
  const E* rowp = static_cast<const E*>(j.logits) + static_cast<int64_t>(row) * j.ld;
  uint64_t* lst = j.flist + static_cast<size_t>(row) * kFullListCap;
  uint32_t* cnt = j.fcnt + row;
  const int lo = seg * j.fseg_len;
  const int hi = min(j.V, lo + j.fseg_len);
  seg_visit(rowp, lo, hi, j.aligned != 0, [&](int id, float x) {
    const float s = scaled_of(x, c.T);
    bool hit = FullTerms::bucket_of(s - m) == bstar;  // the bucket alone, no exponential
    if (hit) {
      uint64_t wt;
      int b;
      hit = ft.mass(s, &wt, &b);  // the histogram's membership (e >= min_p, mass > 0)
    }
    const uint64_t bal = __ballot(hit);
    if (bal) {
      const int first = __ffsll(static_cast<unsigned long long>(bal)) - 1;
      const uint32_t nb = static_cast<uint32_t>(__popcll(bal));
      uint32_t at = 0;
      if (lane() == first) at = atomicAdd(&s_n, nb);
      at = __builtin_amdgcn_readlane(at, first);
      if (at + nb <= static_cast<uint32_t>(kGatherBuf)) {  // uniform
        if (hit) sbuf[at + lanes_below(bal)] = pack(f2key(s), id);
      } else {
        uint32_t base = 0;
        if (lane() == first) {
          atomicMin(&s_lim, at);
          base = atomicAdd(cnt, nb);
        }
        base = __builtin_amdgcn_readlane(base, first);
        const uint32_t pos = base + static_cast<uint32_t>(lanes_below(bal));
        if (hit && pos < static_cast<uint32_t>(kFullListCap)) lst[pos] = pack(f2key(s), id);
      }
    }
  });
  __syncthreads();
  // reservations are contiguous, so the buffer holds everything below the
  // first one that did not fit (s_lim), or all of s_n
  const uint32_t n = min(s_n, s_lim);
  if (threadIdx.x == 0) s_base = n ? atomicAdd(cnt, n) : 0u;
  __syncthreads();
  const uint32_t base = s_base;
  for (uint32_t i = threadIdx.x; i < n; i += kThreads)
    if (base + i < static_cast<uint32_t>(kFullListCap)) lst[base + i] = sbuf[i];
}

}  // namespace

hipError_t launch_full_prep(const Job& j, hipStream_t st) {
  const int grid = xcd_grid(j.B, j.fseg);
  if (j.dt == VS_F32)
    hipLaunchKernelGGL(k_full_hist<float>, dim3(grid), dim3(kThreads), 0, st, j);
  else
    hipLaunchKernelGGL(k_full_hist<uint16_t>, dim3(grid), dim3(kThreads), 0, st, j);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (j.dt == VS_F32)
    hipLaunchKernelGGL(k_full_gather<float>, dim3(grid), dim3(kThreads), 0, st, j);
  else
    hipLaunchKernelGGL(k_full_gather<uint16_t>, dim3(grid), dim3(kThreads), 0, st, j);
  return hipGetLastError();
}

}  // namespace vsk
