// The parallel passes of the full-vocabulary top-p cut.
//
// A full-vocabulary row keeps the shortest prefix of its ids in the order
// (s desc, id asc) whose fixed-point mass reaches top_p of the total
// (TensorRT-LLM "Sampling", top-p; the mass and its rounding are the ones the
// oracle and the row kernels use). Both passes split each such row into
// segments read by many workgroups (all segments of a row on one XCD):
//  - the histogram pass adds every id's mass W = floor(E(s - m) 2^31) into
//    4096 buckets of t = s - m, first in LDS, then per nonempty bucket into
//    the row's histogram in the workspace (zeroed by the row kernel);
//  - the gather pass finds, from that histogram, the bucket where the
//    cumulative mass (largest s first) reaches the target and the mass still
//    needed inside it, appends the ids of that bucket (packed key and id) to
//    the row's list, and counts them and the ids of the buckets above it.
//    E is nondecreasing in t, and the cut bucket holds an id of positive
//    mass that passes min-p, so every id in a bucket above it does too: the
//    ids above are counted from their bucket alone, with no exponential.
// The cut kernel then sorts the list and finds the exact cut; a bucket larger
// than the list goes to its one-workgroup path.
//
// The gather pass also draws over the ids above the cut bucket, which are
// all kept whatever the cut inside the bucket turns out to be: each
// workgroup's best Gumbel score e / -log u over them (e and u exactly as the
// Gumbel pass forms them, the same provable skips) goes to the row's
// per-segment records, and the cut kernel, which scores the kept ids of the
// list itself, takes the best of both as the draw. The row is then finished
// without the Gumbel pass over its kept set (unless kept masks are asked for,
// or the rejection draw is, or the list did not hold the whole bucket).
#include <type_traits>

#include "vs_device.h"
#include "vs_kernels.h"

namespace vsk {
namespace {

constexpr int kThreads = 1024;
constexpr int kPer = kFullBuckets / kThreads;  // buckets per thread (4)
constexpr int kGatherBuf = 2048;  // ids a gather workgroup collects in LDS before one global append

// The rows the passes take: kPassTopP, a full-vocabulary top-p row (the
// histogram, its cut bucket, the gather); kPassWhole, a full-vocabulary row
// without the cut (top_p >= 1), which only the drawing gather pass takes, to
// draw over all of its members; kPassNone, any other (route_row decides).
enum : int { kPassNone = 0, kPassTopP = 1, kPassWhole = 2 };
__device__ __forceinline__ int pass_row(const Job& j, int row, const RoutePre& rp, RowCfg* c,
                                        float* m) {
  const RowRoute r = route_row(j, row, rp);
  *c = r.c;
  *m = r.m;
  if (!r.full) return kPassNone;
  return c->p < 1.0f ? kPassTopP : kPassWhole;
}

// Reads the ids [lo, hi) of a row with the whole block: 16-byte loads when
// the row is aligned (lo is a multiple of 8, so the segment starts on a
// 16-byte boundary), elements otherwise and at the end. start() issues the
// loads of each thread's first U vectors, so that they are in flight while
// the workgroup does its set-up; visit() then calls f(id0, x, n) for every
// vector (x[c] the value of id id0 + c, c < n; the rest -inf), all lanes of
// a wave together in the vector loop, with the next U vectors' loads issued
// before the current ones are used. Two ways to hand out the vectors:
// statically (thread t takes t, t + kThreads, ...), or, for segments of at
// least kDynChunks chunks per wave when the caller asks for it, in chunks of
// U vectors per lane that each wave claims from an LDS counter as it starts
// the previous one (wave w starts with chunk w; a wave that runs ahead takes
// more chunks, so the waves end together). The counter is set by start() and
// published by a barrier of the caller's before visit().
template <typename E, int U>
struct SegReader {
  static constexpr int EPV = Epv<E>::n;
  static constexpr int kChunk = kWave * U;  // vectors per claimed chunk
  static constexpr int kDynChunks = 4;      // chunks per wave, at least, for the claimed hand-out
  const E* rowp;
  int lo, hi, nvec;
  bool dyn;   // claimed chunks (uniform over the block)
  int p;      // this thread's first vector of the current step
  int* next;  // the next unclaimed chunk (LDS)
  uint4 raw[U];

  __device__ __forceinline__ int stride() const { return dyn ? kWave : kThreads; }

  __device__ __forceinline__ void start(const E* __restrict__ r, int l, int h, bool aligned,
                                        int* counter = nullptr) {
    rowp = r;
    lo = l;
    hi = h;
    nvec = aligned ? (h - l) / EPV : 0;
    next = counter;
    dyn = counter && nvec >= kDynChunks * (kThreads / kWave) * kChunk;
    const int w = static_cast<int>(threadIdx.x) / kWave;
    p = dyn ? w * kChunk + lane() : static_cast<int>(threadIdx.x);
    if (dyn && threadIdx.x == 0) *counter = kThreads / kWave;
    const E* base = rowp + lo;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = p + u * stride();
      if (i < nvec) raw[u] = load16(base + i * EPV);
    }
  }

  template <typename F>
  __device__ __forceinline__ void visit(F&& f) {
    const E* base = rowp + lo;
    const int sd = stride();
    // (claimed: the condition is uniform per wave, p's chunk being the wave's)
    while (dyn ? (p - lane()) < nvec : p < nvec) {
      int pn;
      if (dyn) {
        int c2 = 0;
        if (lane() == 0) c2 = atomicAdd(next, 1);
        pn = __builtin_amdgcn_readfirstlane(c2) * kChunk + lane();
      } else {
        pn = p + U * kThreads;
      }
      uint4 nxt[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = pn + u * sd;
        if (i < nvec) nxt[u] = load16(base + i * EPV);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = p + u * sd;
        if (i < nvec) {
          float x[EPV];
          unpack16(raw[u], x, rowp);
          f(lo + i * EPV, x, EPV);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) raw[u] = nxt[u];
      p = pn;
    }
    for (int q = lo + nvec * EPV + static_cast<int>(threadIdx.x); q < hi; q += kThreads) {
      float x[EPV];
#pragma unroll
      for (int c = 0; c < EPV; ++c) x[c] = -kInf;
      x[0] = to_f32(rowp[q]);
      f(q, x, 1);
    }
  }
};

// s = x / T, with the division left out (x / 1 is x) for rows at T = 1: the
// callers branch once per workgroup on kDiv.
template <bool kDiv>
__device__ __forceinline__ float scaled_by(float x, float T) { return kDiv ? x / T : x; }

// A thread's kCandM best Gumbel candidates, best first in the order (score
// desc, id asc); empty slots score -1.
struct CandList {
  double s[kCandM];
  int32_t id[kCandM];
  uint32_t key[kCandM];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int i = 0; i < kCandM; ++i) {
      s[i] = -1.0;
      id[i] = 0x7fffffff;
      key[i] = 0u;
    }
  }
  __device__ __forceinline__ static bool before(double sa, int32_t ia, double sb, int32_t ib) {
    return sa > sb || (sa == sb && ia < ib);
  }
  // inserts (sc, i, k) in order when it beats the last entry
  __device__ __forceinline__ void insert(double sc, int32_t i, uint32_t k) {
    if (!before(sc, i, s[kCandM - 1], id[kCandM - 1])) return;
    s[kCandM - 1] = sc;
    id[kCandM - 1] = i;
    key[kCandM - 1] = k;
#pragma unroll
    for (int p = kCandM - 1; p > 0; --p) {
      if (before(s[p], id[p], s[p - 1], id[p - 1])) {
        const double ts = s[p];
        s[p] = s[p - 1];
        s[p - 1] = ts;
        const int32_t ti = id[p];
        id[p] = id[p - 1];
        id[p - 1] = ti;
        const uint32_t tk = key[p];
        key[p] = key[p - 1];
        key[p - 1] = tk;
      }
    }
  }
};

// kReject: the rejection draw's candidates are kept too (a separate instance,
// so that the histogram alone keeps its own code).
template <typename E, bool kReject>
__global__ __launch_bounds__(kThreads) void k_full_hist(Job j) {
  __shared__ uint64_t hw[kFullBuckets];
  __shared__ double sd[kThreads / kWave];
  __shared__ int si[kThreads / kWave];
  __shared__ uint64_t s_bound;  // bits of the best known lower bound on the segment's kCandM-th score
  int row, seg;
  if (!xcd_row_tile(blockIdx.x, j.B, j.fseg, &row, &seg)) return;  // uniform per block
  const E* rowp = static_cast<const E*>(j.logits) + static_cast<int64_t>(row) * j.ld;
  const int lo = seg * j.fseg_len;
  const int hi = min(j.V, lo + j.fseg_len);
  // the route's loads, then the segment's first ones, before the row's route
  // is known (wasted, and harmless, for a row this pass does not take)
  const RoutePre rp = route_preload(j, row);
  SegReader<E, 4> rd;
  rd.start(rowp, lo, hi, j.aligned != 0);
  RowCfg c;
  float m;
  if (pass_row(j, row, rp, &c, &m) != kPassTopP) return;  // uniform per block
  for (int i = threadIdx.x; i < kFullBuckets; i += kThreads) hw[i] = 0ull;
  if (threadIdx.x == 0) s_bound = 0ull;
  __syncthreads();
  constexpr bool reject = kReject;
  // The rejection draw's candidates: every member id's Gumbel score e / -log u
  // (e and u exactly as the Gumbel pass forms them) into this thread's best
  // kCandM. An id is skipped when it provably scores below a lower bound on
  // the segment's kCandM-th best score (the largest kCandM-th best any thread
  // has; shared through LDS, where a stale value is only a looser bound): 
  // -log u > 1 - u for u < 1, so 1 - u >= e / bound means e / -log u < bound;
  // e <= 1 gives a first test on the random word alone (an integer compare).
  const uint64_t rs = row_stream(c.seed, row);
  CandList cl;
  cl.clear();
  double lim = __builtin_inf();  // (1 + 2^-40) / bound
  uint64_t skip = 0ull;
  const auto refresh = [&]() {
    const uint64_t sb = __hip_atomic_load(&s_bound, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const double bd = __longlong_as_double(static_cast<long long>(sb));
    if (bd > 0.0 && (1.0 + 0x1p-40) / bd < lim) {
      lim = (1.0 + 0x1p-40) / bd;
      skip = skip_below(lim);
    }
  };
  const auto candidate = [&](int id, float e, uint32_t key) {
    const uint64_t b = random_bits(rs, id);
    if (b < skip) return;  // e <= 1: below the bound
    const double u = uniform_of_bits(b);
    const double one_u = (1.0 - u) * (1.0 - 0x1p-50);  // rounded down past any rounding error
    if (one_u >= lim * static_cast<double>(e)) return;  // below the bound
    const double sc = static_cast<double>(e) / -log(u);  // as the Gumbel pass scores it
    cl.insert(sc, id, key);
    if (cl.s[kCandM - 1] > 0.0) {  // this thread's own kCandM-th best bounds the segment's
      const uint64_t sb = static_cast<uint64_t>(__double_as_longlong(cl.s[kCandM - 1]));
      atomicMax(reinterpret_cast<unsigned long long*>(&s_bound), static_cast<unsigned long long>(sb));
      refresh();
    }
  };
  // one LDS atomic per member id (non-members, e.g. below min-p, skip it:
  // adding 0 at one shared address would serialize the wave's lanes)
  auto pass = [&](auto div) {
    rd.visit([&](int id0, const float* x, int n) {
      constexpr int EPV = SegReader<E, 4>::EPV;
      if constexpr (reject) {
        refresh();
        const FullTerms ft{m, c.mp};
#pragma unroll
        for (int q = 0; q < EPV; ++q) {
          uint64_t w;
          int b;
          float e;
          const float sv = scaled_by<decltype(div)::value>(x[q], c.T);
          if (ft.mass_e(sv, &w, &b, &e) && q < n) {
            atomicAdd(reinterpret_cast<unsigned long long*>(&hw[b]), static_cast<unsigned long long>(w));
            candidate(id0 + q, e, f2key(sv));
          }
        }
      } else {
        // the vector's exponentials first, evaluated together (their
        // dependent chains interleave), then its masses into the histogram:
        // the terms of FullTerms::mass_e
        float t[EPV], e[EPV];
#pragma unroll
        for (int q = 0; q < EPV; ++q) t[q] = scaled_by<decltype(div)::value>(x[q], c.T) - m;
        constexpr int G = EPV < 4 ? EPV : 4;
#pragma unroll
        for (int g0 = 0; g0 < EPV; g0 += G) pinned_exp_n<G>(t + g0, e + g0);
#pragma unroll
        for (int q = 0; q < EPV; ++q) {
          const uint64_t w = mass_of(e[q]);
          if (q < n && e[q] >= c.mp && w != 0)
            atomicAdd(reinterpret_cast<unsigned long long*>(&hw[FullTerms::bucket_of(t[q])]),
                      static_cast<unsigned long long>(w));
        }
      }
    });
  };
  if (c.T == 1.0f)  // uniform
    pass(std::false_type{});
  else
    pass(std::true_type{});
  __syncthreads();
  uint64_t* ghw = j.fhw + static_cast<size_t>(row) * kFullBuckets;
  for (int b = threadIdx.x; b < kFullBuckets; b += kThreads) {
    const uint64_t v = hw[b];
    if (v) atomicAdd(reinterpret_cast<unsigned long long*>(&ghw[b]), static_cast<unsigned long long>(v));
  }
  if constexpr (reject) {
    // the segment's kCandM best, one block argmax a round, the owner popping
    // its head
    GCand* out = j.fcand + (static_cast<size_t>(row) * j.ntile3 + seg) * kCandM;
    for (int r = 0; r < kCandM; ++r) {
      const double bs = block_max(cl.s[0], sd);
      const int bi = block_min(cl.s[0] == bs ? cl.id[0] : 0x7fffffff, si);
      const bool mine = cl.s[0] == bs && cl.id[0] == bi && bs >= 0.0;
      if (mine) {
        out[r] = GCand{bs, bi, cl.key[0]};
#pragma unroll
        for (int p = 0; p + 1 < kCandM; ++p) {
          cl.s[p] = cl.s[p + 1];
          cl.id[p] = cl.id[p + 1];
          cl.key[p] = cl.key[p + 1];
        }
        cl.s[kCandM - 1] = -1.0;
        cl.id[kCandM - 1] = 0x7fffffff;
      }
      if (threadIdx.x == 0 && bs < 0.0) out[r] = GCand{-1.0, 0x7fffffff, 0u};
    }
  }
}

template <typename E, bool kDraw>
__global__ __launch_bounds__(kThreads) void k_full_gather(Job j) {
  __shared__ uint64_t sw[kThreads / kWave];
  __shared__ double sd[kThreads / kWave];
  __shared__ int s_bucket;
  __shared__ uint64_t s_above_w;
  __shared__ uint64_t sbuf[kGatherBuf];
  __shared__ uint32_t s_n, s_lim, s_base;
  __shared__ uint64_t s_best;  // bits of the best score any thread has found
  __shared__ int s_chunk;      // the reader's next chunk, when claimed
  __shared__ int s_wi[kThreads / kWave];  // per-wave bests' ids, their s and counts
  __shared__ float s_ws[kThreads / kWave];
  __shared__ uint32_t s_wa[kThreads / kWave], s_wh[kThreads / kWave];
  int row, seg;
  if (!xcd_row_tile(blockIdx.x, j.B, j.fseg, &row, &seg)) return;  // uniform per block
  const E* rowp = static_cast<const E*>(j.logits) + static_cast<int64_t>(row) * j.ld;
  const int lo = seg * j.fseg_len;
  const int hi = min(j.V, lo + j.fseg_len);
  // vectors in flight per thread (fewer with the draw, whose random words
  // need the registers); the first before the row's route is known
  constexpr int kGU = kDraw ? 2 : 4;
  const RoutePre rp = route_preload(j, row);
  SegReader<E, kGU> rd;
  rd.start(rowp, lo, hi, j.aligned != 0, &s_chunk);
  RowCfg c;
  float m;
  const int kind = pass_row(j, row, rp, &c, &m);
  if (kind == kPassNone || (!kDraw && kind == kPassWhole)) return;  // uniform per block
  // a row without the cut: every member is drawn over (kDraw), nothing gathered
  const bool whole = kDraw && kind == kPassWhole;
  const uint64_t* ghw = j.fhw + static_cast<size_t>(row) * kFullBuckets;

  // The cut bucket: thread t holds buckets [4 t, 4 t + 4); an exclusive scan
  // over the threads gives the mass of the buckets before.
  // (an in-wave DPP scan, then the waves' totals through LDS: one barrier,
  // which also publishes the shared state cleared here)
  uint64_t w[kPer];
  uint64_t cw = 0, lw = 0, inc = 0;
  const int wv = static_cast<int>(threadIdx.x) / kWave;
  if (!whole) {  // uniform
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      w[i] = ghw[threadIdx.x * kPer + i];
      lw += w[i];
    }
    inc = wave_scan_incl_u64(lw);
    if (lane() == kWave - 1) sw[wv] = inc;
  }
  if (threadIdx.x == 0) {
    s_bucket = -1;
    s_n = 0u;
    s_lim = 0xffffffffu;
    s_best = 0ull;
  }
  __syncthreads();
  int bstar = kFullBuckets - 1;  // (whole rows: unused)
  if (!whole) {  // uniform
    uint64_t before = 0, total_w = 0;
    for (int q = 0; q < kThreads / kWave; ++q) {
      const uint64_t t = sw[q];
      before += q < wv ? t : 0ull;
      total_w += t;
    }
    cw = before + inc - lw;
    // the kept prefix is the shortest whose mass reaches p * total; masses
    // are integers, so "cum >= thr" is "cum >= ceil(thr)" (at least one id)
    const double thr = static_cast<double>(c.p) * static_cast<double>(total_w);
    const uint64_t target = ceil(thr) >= 1.0 ? static_cast<uint64_t>(ceil(thr)) : 1ull;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int b = threadIdx.x * kPer + i;
      if (cw < target && target <= cw + w[i]) {
        s_bucket = b;
        s_above_w = cw;
      }
      cw += w[i];
    }
    __syncthreads();
    bstar = s_bucket;
    if (bstar < 0) {  // uniform; unreachable (the row maximum has mass 2^31)
      // no stale record from an earlier call may stand: the cut kernel then
      // takes its one-workgroup path
      if (seg == 0 && threadIdx.x == 0) j.fcut[row].bucket = -1;
      return;
    }
    if (seg == 0 && threadIdx.x == 0) {
      j.fcut[row].bucket = bstar;
      j.fcut[row].rem = target - s_above_w;
    }
  }

  // The ids of that bucket: collected in LDS (one LDS atomic add per wave),
  // then appended to the row's list with one global atomic add per workgroup;
  // ids beyond the LDS buffer go straight to the list, one atomic add per wave.
  const FullTerms ft{m, c.mp};
  uint64_t* lst = j.flist + static_cast<size_t>(row) * kFullListCap;
  uint32_t* cnt = j.fcnt + row;
  uint32_t n_above = 0, n_hit = 0;
  // Every id of the cut bucket is a member (e >= min_p and a positive mass)
  // when the bucket's lowest t already is: t > -(b* + 1) / kFullPerUnit up to
  // the rounding of the bucket's product, and E is nondecreasing, so E at a t
  // just below that bound is a lower bound on each id's e. Then no id needs
  // its own exponential; else (a bucket at the min-p or zero-mass edge, or
  // the last bucket, which holds every smaller t) each id is tested.
  bool bucket_in = false;
  if (!whole && bstar < kFullBuckets - 1) {
    const float t_lo = -static_cast<float>(bstar + 1) / kFullPerUnit * (1.0f + 0x1p-20f);
    const float e_lo = pinned_exp(t_lo);
    bucket_in = e_lo >= c.mp && mass_of(e_lo) != 0ull;
  }
  constexpr int EPV = SegReader<E, kGU>::EPV;

  // The draw over the ids above the cut bucket (kDraw). A thread skips the
  // logarithm and the division for an id that provably scores below the best
  // score known in the workgroup (shared through LDS, where a stale value is
  // only a looser bound): -log u > 1 - u for u < 1, so 1 - u >= e / best
  // means e / -log u < best; an upper bound on e gives that test on the
  // random word alone (an integer compare).
  const uint64_t rs = row_stream(c.seed, row);
  double best = -1.0;
  int best_id = 0x7fffffff;
  float best_s = 0.0f;
  double lim = __builtin_inf();  // (1 + 2^-40) / (the best score known here)
  float lim_up = __builtin_inff();  // a float at or above lim
  const auto refresh = [&]() {
    const uint64_t sb = __hip_atomic_load(&s_best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const double bd = __longlong_as_double(static_cast<long long>(sb));
    if (bd > 0.0 && (1.0 + 0x1p-40) / bd < lim) {
      lim = (1.0 + 0x1p-40) / bd;
      lim_up = up_of(lim);
    }
  };
  // the score of an above id whose random word b passed the integer test,
  // unless a finer test shows it cannot beat the bound
  // (share: a new best of the thread is offered to the workgroup's bound)
  const auto score = [&](int id, float sv, uint64_t b, bool share) {
    const double u = uniform_of_bits(b);
    const double one_u = (1.0 - u) * (1.0 - 0x1p-50);  // rounded down past any rounding error
    if (one_u >= lim) return;                          // e <= 1: below the bound
    const float e = pinned_exp(sv - m);
    if (one_u >= lim * static_cast<double>(e)) return;  // below the bound
    const double g = static_cast<double>(e) / -log(u);  // as the Gumbel pass scores it
    if (g > best || (g == best && id < best_id)) {
      best = g;
      best_id = id;
      best_s = sv;
      if (share) {
        atomicMax(reinterpret_cast<unsigned long long*>(&s_best),
                  static_cast<unsigned long long>(__double_as_longlong(g)));
        refresh();
      }
    }
  };
  // The bucket of t is floor(-t kFullPerUnit) (a power of two: the product is
  // exact), capped at the last bucket, so bucket < b* is t > -b* / kFullPerUnit
  // and bucket == b* is -(b* + 1) / kFullPerUnit < t <= -b* / kFullPerUnit
  // (the lower end open for the last bucket; a NaN t fails both): two compares
  // against exact bounds instead of the bucket's arithmetic.
  const float t_above = -static_cast<float>(bstar) / kFullPerUnit;
  const float t_floor =
      bstar < kFullBuckets - 1 ? -static_cast<float>(bstar + 1) / kFullPerUnit : -kInf;
  const auto above = [&](float sv) { return sv - m > t_above; };
  // a member of a row without the cut: every id, or e >= min_p when it is set
  const bool minp = c.mp > 0.0f;
  const auto member = [&](float sv) { return !minp || pinned_exp(sv - m) >= c.mp; };
  if constexpr (kDraw) {
    // one id per thread first (the first of its first vector, when above),
    // so that the workgroup starts from the best of up to 1024 scores, taken
    // by a block maximum (not by 1024 atomics on one LDS word)
    if (rd.p < rd.nvec) {  // its first vector is in flight
      float x[EPV];
      unpack16(rd.raw[0], x, rowp);
      const int id = lo + rd.p * EPV;
      const float sv = c.T == 1.0f ? x[0] : x[0] / c.T;
      if (whole ? member(sv) : above(sv)) score(id, sv, random_bits(rs, id), false);
    }
    const double wb = wave_max(best);
    if (lane() == 0) sd[threadIdx.x / kWave] = wb;
    __syncthreads();
    if (threadIdx.x == 0) {
      double bb = sd[0];
      for (int i = 1; i < kThreads / kWave; ++i) bb = sd[i] > bb ? sd[i] : bb;
      if (bb > 0.0) s_best = static_cast<uint64_t>(__double_as_longlong(bb));
    }
    __syncthreads();
    refresh();
  }

  auto pass = [&](auto div) {
    rd.visit([&](int id0, const float* x, int n) {
      float sv[EPV];
      uint32_t hm = 0;  // ids in the cut bucket (the bucket alone, no exponential)
      uint32_t am = 0;  // ids above it (a whole row's members)
#pragma unroll
      for (int q = 0; q < EPV; ++q) sv[q] = scaled_by<decltype(div)::value>(x[q], c.T);
      if (whole) {  // uniform
#pragma unroll
        for (int q = 0; q < EPV; ++q) am |= (q < n && member(sv[q])) ? 1u << q : 0u;
      } else {
#pragma unroll
        for (int q = 0; q < EPV; ++q) {
          const float t = sv[q] - m;
          // (positions past n hold -inf: in no bucket by these bounds
          // either, except the last, whose ids the membership test below
          // drops)
          const bool in = q < n;
          am |= (in && t > t_above) ? 1u << q : 0u;
          hm |= (in && t <= t_above && t > t_floor) ? 1u << q : 0u;
        }
      }
      n_above += __popc(am);
      if constexpr (kDraw) {
        if (__ballot(am != 0u)) {  // uniform
          refresh();
          // the integer test for this vector, on the high halves of the
          // random words, from an upper bound on its ids' e (the hardware
          // exponential at the largest s, 2^-16 above any rounding of it;
          // at most 1: every id here is at or below the maximum)
          float vmax = sv[0];
#pragma unroll
          for (int q = 1; q < EPV; ++q) vmax = fmaxf(vmax, sv[q]);
          const float veub = fminf(__builtin_amdgcn_exp2f((vmax - m) * 1.44269504088896340736f) *
                                   (1.0f + 0x1p-16f), 1.0f);
          const uint32_t vskip = skip_hi(lim_up, veub);
          uint32_t need = 0;
#pragma unroll
          for (int q = 0; q < EPV; ++q)
            need |= ((am >> q) & 1u) && random_hi(rs, id0 + q) >= vskip ? 1u << q : 0u;
          // rare once a bound is known: each such id's value is read again
          // (a cache hit) and its word formed again, so that one copy of the
          // scoring code serves every position of the vector
          for (uint32_t nb = need; nb != 0u; nb &= nb - 1u) {
            const int id = id0 + __builtin_ctz(nb);
            score(id, scaled_by<decltype(div)::value>(to_f32(rowp[id]), c.T), random_bits(rs, id), true);
          }
        }
      }
      if (__ballot(hm != 0u)) {  // uniform; few vectors hold cut-bucket ids
        uint32_t hits = hm;
        if (!bucket_in) {  // uniform
#pragma unroll
          for (int q = 0; q < EPV; ++q) {
            if ((hits >> q) & 1u) {
              uint64_t wt;
              int bb;
              // the histogram's membership (e >= min_p, mass > 0)
              if (!ft.mass(sv[q], &wt, &bb)) hits &= ~(1u << q);
            }
          }
        }
        // one reservation for the wave's hits of this vector (lanes past the
        // segment's end may be inactive here: the counts go through ballots,
        // one per bit of a lane's count, and the first active lane reserves)
        const uint32_t nh = static_cast<uint32_t>(__popc(hits));
        n_hit += nh;
        uint32_t before = 0u, tot = 0u;
#pragma unroll
        for (int bit = 0; bit < 4; ++bit) {  // nh <= EPV <= 8
          const uint64_t bb = __ballot((nh >> bit) & 1u);
          before += static_cast<uint32_t>(lanes_below(bb)) << bit;
          tot += static_cast<uint32_t>(__popcll(bb)) << bit;
        }
        if (tot) {  // uniform
          const int lead = __ffsll(static_cast<unsigned long long>(__ballot(true))) - 1;
          uint32_t at = 0;
          if (lane() == lead) at = atomicAdd(&s_n, tot);
          at = __builtin_amdgcn_readlane(at, lead);
          uint32_t pos = before;
          if (at + tot <= static_cast<uint32_t>(kGatherBuf)) {  // uniform
            pos += at;
#pragma unroll
            for (int q = 0; q < EPV; ++q)
              if ((hits >> q) & 1u) sbuf[pos++] = pack(f2key(sv[q]), id0 + q);
          } else {
            uint32_t base = 0;
            if (lane() == lead) {
              atomicMin(&s_lim, at);
              base = atomicAdd(cnt, tot);
            }
            pos += __builtin_amdgcn_readlane(base, lead);
#pragma unroll
            for (int q = 0; q < EPV; ++q) {
              if ((hits >> q) & 1u) {
                if (pos < static_cast<uint32_t>(kFullListCap)) lst[pos] = pack(f2key(sv[q]), id0 + q);
                ++pos;
              }
            }
          }
        }
      }
    });
  };
  if (c.T == 1.0f)  // uniform
    pass(std::false_type{});
  else
    pass(std::true_type{});
  // The workgroup's draw record and counts with one barrier: each wave's
  // best (score desc, id asc, with its s) and counts through slots of its
  // own (the barrier also completes the LDS appends), combined by wave 0.
  {
    const int wv = static_cast<int>(threadIdx.x) / kWave;
    double wb = -1.0;
    int wi = 0x7fffffff;
    float ws = 0.0f;
    if constexpr (kDraw) {
      wb = wave_max(best);
      wi = wave_min(best == wb ? best_id : 0x7fffffff);
      const uint64_t own = __ballot(best == wb && best_id == wi);  // (ids are distinct)
      ws = own ? __shfl(best_s, __ffsll(static_cast<unsigned long long>(own)) - 1) : 0.0f;
    }
    const uint32_t wa = wave_sum(n_above), wh = wave_sum(n_hit);
    if (lane() == 0) {
      sd[wv] = wb;
      s_wi[wv] = wi;
      s_ws[wv] = ws;
      s_wa[wv] = wa;
      s_wh[wv] = wh;
    }
  }
  __syncthreads();
  // reservations are contiguous, so the buffer holds everything below the
  // first one that did not fit (s_lim), or all of s_n
  const uint32_t n = min(s_n, s_lim);
  if (threadIdx.x < kWave) {  // wave 0
    const int l = lane();
    const bool slot = l < kThreads / kWave;
    const double sb = slot ? sd[l] : -1.0;
    const int si = slot ? s_wi[l] : 0x7fffffff;
    const double bb = wave_max(sb);
    const int bid = wave_min(sb == bb ? si : 0x7fffffff);
    const uint64_t own = __ballot(slot && sb == bb && si == bid);
    const float bs = own ? __shfl(slot ? s_ws[l] : 0.0f, __ffsll(static_cast<unsigned long long>(own)) - 1)
                         : 0.0f;
    const uint32_t ta = wave_sum(slot ? s_wa[l] : 0u), th = wave_sum(slot ? s_wh[l] : 0u);
    if (l == 0) {
      // the segment's best over its above ids (a whole row's members), score
      // desc, id asc, into the row's per-segment record (score -1: none),
      // with a whole row's member count
      if constexpr (kDraw)
        j.gpart[static_cast<size_t>(row) * j.ntile3 + seg] =
            GPart{bb >= 0.0 ? bb : -1.0, bid, whole ? static_cast<int32_t>(ta) : 0,
                  bb >= 0.0 ? bs : 0.0f};
      s_base = n ? atomicAdd(cnt, n) : 0u;
      if (ta && !whole)
        atomicAdd(reinterpret_cast<unsigned long long*>(&j.fcut[row].above_c),
                  static_cast<unsigned long long>(ta));
      if (th) atomicAdd(&j.fcut[row].count, th);
    }
  }
  __syncthreads();
  const uint32_t base = s_base;
  for (uint32_t i = threadIdx.x; i < n; i += kThreads)
    if (base + i < static_cast<uint32_t>(kFullListCap)) lst[base + i] = sbuf[i];
}

}  // namespace

hipError_t launch_full_prep(const Job& j, hipStream_t st) {
  const int grid = xcd_grid(j.B, j.fseg);
  if (j.dt == VS_F32 && j.topp_reject)
    hipLaunchKernelGGL((k_full_hist<float, true>), dim3(grid), dim3(kThreads), 0, st, j);
  else if (j.dt == VS_F32)
    hipLaunchKernelGGL((k_full_hist<float, false>), dim3(grid), dim3(kThreads), 0, st, j);
  else if (j.topp_reject)
    hipLaunchKernelGGL((k_full_hist<uint16_t, true>), dim3(grid), dim3(kThreads), 0, st, j);
  else
    hipLaunchKernelGGL((k_full_hist<uint16_t, false>), dim3(grid), dim3(kThreads), 0, st, j);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (j.dt == VS_F32 && j.fdraw)
    hipLaunchKernelGGL((k_full_gather<float, true>), dim3(grid), dim3(kThreads), 0, st, j);
  else if (j.dt == VS_F32)
    hipLaunchKernelGGL((k_full_gather<float, false>), dim3(grid), dim3(kThreads), 0, st, j);
  else if (j.fdraw)
    hipLaunchKernelGGL((k_full_gather<uint16_t, true>), dim3(grid), dim3(kThreads), 0, st, j);
  else
    hipLaunchKernelGGL((k_full_gather<uint16_t, false>), dim3(grid), dim3(kThreads), 0, st, j);
  return hipGetLastError();
}

}  // namespace vsk
