// K1: the single streaming pass over the logits.
//
// A workgroup owns one segment of a row: a run of 2048-value tiles (the whole
// row when the batch alone fills the chip). Each of its W waves walks the
// segment's tiles W apart, the next tile's loads in flight while it works on
// the current one; a tile is 64 lanes x 32 values, loaded with 16-byte vector
// loads and held in registers. Per tile a wave updates:
//  - the flags (NaN or +inf seen, some value above -inf), from a
//    NaN-propagating maximum;
//  - in log-probability mode the log-sum-exp partial (max, sum of exp(x - max));
//  - for a list that wants the argmax of x: the tile argmax with its lowest id;
//  - for a list that wants the top k (2 <= k <= 64) of s = x / T: a pool of
//    candidates in LDS. Values are taken into the pool only if their key
//    reaches the best lower bound known for the segment's k-th largest key:
//    the k-th largest lane maximum of some tile, or the exact k-th largest key
//    of some wave's pool (each counts k real values at or above it). The bound
//    is shared by the waves of the workgroup through LDS and only grows, so
//    late tiles rarely contribute candidates (the selection is a streaming
//    top-k in the sense of "Top-k sampling", with the threshold pruning of
//    "Sampling: radix select and pivot search").
// At the end the waves' pools are merged: every value whose key reaches the
// segment's exact k-th largest key is written out (k of them unless keys tie),
// with that key; the row kernel merges the segments. A segment whose candidates
// do not fit sets an overflow flag and the row kernel selects exactly from the
// row itself.
#include "vs_device.h"
#include "vs_kernels.h"

namespace vsk {
namespace {

constexpr int kVals = kSelTile / kWave;  // values per lane and tile (32)
constexpr int kGroup = 8;         // values per group (a lane's maxima are kept per group)
constexpr int kGroups = kVals / kGroup;

constexpr int kPoolN = 3;         // pool slots per lane
constexpr int kPool = kWave * kPoolN;
constexpr int kCompactAt = 96;    // compact a pool once it holds more than this
constexpr int kMergeCap = 1024;   // merged candidates per segment and list
constexpr float kL2E = 1.44269504088896340736f;

template <typename E>
__device__ __forceinline__ int elem_index(int tile_base, int q) {
  constexpr int EPV = Epv<E>::n;
  return tile_base + ((q / EPV) * kWave + lane()) * EPV + (q % EPV);
}

template <typename E>
struct Raw {
  static constexpr int n = kVals / Epv<E>::n;  // 16-byte loads per lane and tile
  uint4 r[n];
};

// kStream: non-temporal loads (a compile-time choice, so that the hint cannot
// be merged away with the ordinary load of the same address).
// The 16-byte loads of the tile at base; stride 0 makes every load read the
// 16 bytes at base (a placeholder load that keeps the load count fixed).
template <typename E, bool kStream>
__device__ __forceinline__ void load_raw(const E* __restrict__ base, int stride, Raw<E>& raw) {
  constexpr int EPV = Epv<E>::n;
  const int l = lane();
#pragma unroll
  for (int i = 0; i < Raw<E>::n; ++i) {
    const E* p = base + (i * kWave + l) * EPV * stride;
    raw.r[i] = kStream ? load16_stream(p) : load16(p);
  }
}

template <typename E>
__device__ __forceinline__ void unpack_raw(const Raw<E>& raw, const E* rowp, float (&v)[kVals]) {
  constexpr int EPV = Epv<E>::n;
#pragma unroll
  for (int i = 0; i < Raw<E>::n; ++i) unpack16(raw.r[i], &v[i * EPV], rowp);
}

// A tile that ends past V: element loads, -inf beyond V.
template <typename E>
__device__ __forceinline__ void load_tail(const E* __restrict__ rowp, int tile_base, int V,
                                          float (&v)[kVals]) {
#pragma unroll
  for (int q = 0; q < kVals; ++q) {
    const int idx = elem_index<E>(tile_base, q);
    v[q] = (idx < V) ? to_f32(rowp[idx]) : -kInf;
  }
}

// Argmax of the tile with its lowest id: the wave max M, then a scan in id
// order (vector index ascending; within it lane, then component) that stops
// at the first value equal to M. Returns the packed candidate, 0 if none.
template <typename E>
__device__ __forceinline__ uint64_t tile_argmax(const float (&v)[kVals], float M, int tile_base,
                                                int V, bool vec) {
  constexpr int EPV = Epv<E>::n;
  constexpr int NV = kVals / EPV;
  if (!(M >= -kInf)) return 0ull;  // only NaN in this tile
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int cfirst = EPV;
#pragma unroll
    for (int c = EPV - 1; c >= 0; --c) {
      const int idx = tile_base + (i * kWave + lane()) * EPV + c;
      if (v[i * EPV + c] == M && (vec || idx < V)) cfirst = c;
    }
    const uint64_t bal = __ballot(cfirst < EPV);
    if (bal) {
      const int l0 = __ffsll(static_cast<unsigned long long>(bal)) - 1;
      const int c0 = __builtin_amdgcn_readlane(cfirst, l0);
      return pack(f2key(M), tile_base + (i * kWave + l0) * EPV + c0);
    }
  }
  return 0ull;
}

// Appends to the pool (keys sk, ids si, room free slots) every value of the
// tile that reaches the threshold: v >= pre, and for T != 1 also
// key(v / T) >= thr. g holds each lane's maxima of its 8 groups of 8 values;
// a group no lane's maximum of which reaches pre is skipped whole. Returns the
// count (only the first `room` are stored).
template <typename E, bool kVec, bool kT1>
__device__ __forceinline__ int extract(const float (&v)[kVals], const float (&g)[kGroups],
                                       int tile_base, int V, float pre, uint32_t thr, float T,
                                       uint32_t* __restrict__ sk, int32_t* __restrict__ si,
                                       int room) {
  int n = 0;
#pragma unroll
  for (int gi = 0; gi < kGroups; ++gi) {
    if (__builtin_amdgcn_ballot_w64(g[gi] >= pre) == 0ull) continue;  // uniform
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const int q = gi * kGroup + u;
      bool p = v[q] >= pre;
      if (!kVec) p = p && elem_index<E>(tile_base, q) < V;
      uint64_t bal = __builtin_amdgcn_ballot_w64(p);
      if (bal) {  // uniform: taken only when some lane has a candidate here
        uint32_t key = f2key(v[q]);
        if (!kT1) {
          if (p) {
            key = f2key(v[q] / T);
            p = key >= thr;
          }
          bal = __builtin_amdgcn_ballot_w64(p);
        }
        if (p) {
          const int pos = n + lanes_below(bal);
          if (pos < room) {
            sk[pos] = key;
            si[pos] = elem_index<E>(tile_base, q);
          }
        }
        n += __popcll(bal);
      }
    }
  }
  return n;
}

// The smallest float pre such that key(fl(x / T)) >= thr implies x >= pre:
// fl(x / T) >= s forces x / T >= pred(s), so x >= T * pred(s) (exact in
// double), rounded down to float.
__device__ __forceinline__ float prefilter(uint32_t thr, float T) {
  const float s = key2f(thr);
  if (T == 1.0f) return s;
  const double y = static_cast<double>(T) * static_cast<double>(nextafterf(s, -kInf));
  float pre = static_cast<float>(y);
  if (static_cast<double>(pre) > y) pre = nextafterf(pre, -kInf);
  return pre;
}

// The k-th largest lane maximum of the tile (of the lane top-two values when
// k > 32), as a key of s = x / T: at least k values of the tile reach it.
__device__ __forceinline__ uint32_t tile_bound(const float (&v)[kVals], float lmax, int k,
                                               float T) {
  uint32_t tk;
  if (k <= 32) {
    tk = wave_kth_largest(f2key(lmax), k);
  } else {
    // the lane's second largest value: the largest value below the lane
    // maximum, or the maximum itself when it occurs twice
    float b = -kInf;
    int nmax = 0;
#pragma unroll
    for (int q = 0; q < kVals; ++q) {
      b = fmaxf(b, v[q] < lmax ? v[q] : -kInf);
      nmax += (v[q] == lmax) ? 1 : 0;
    }
    if (nmax > 1) b = lmax;
    tk = wave_kth_largest2(f2key(lmax), f2key(b), k);
  }
  return (T == 1.0f) ? tk : f2key(key2f(tk) / T);
}

// One wave's candidate pool for one list.
struct Pool {
  uint32_t* key;  // kPool slots in LDS; slot i lives with lane i % 64
  int32_t* id;
  uint32_t* shared_thr;  // the workgroup's bound (LDS, only grows)
  int k;
  float T;
  int n;         // entries held
  uint32_t thr;  // this wave's bound: a lower bound on the segment's k-th key
  bool ovf;
};

__device__ __forceinline__ uint32_t lds_load_relaxed(uint32_t* p) {
  return __builtin_amdgcn_readfirstlane(
      __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
}

// Drops the pool entries below max(floor, exact k-th largest pool key).
__device__ __forceinline__ void pool_compact(Pool& P, uint32_t floor) {
  const int l = lane();
  uint32_t k3[kPoolN];
  int32_t i3[kPoolN];
#pragma unroll
  for (int s = 0; s < kPoolN; ++s) {
    const int slot = s * kWave + l;
    k3[s] = slot < P.n ? P.key[slot] : 0u;
    i3[s] = slot < P.n ? P.id[slot] : 0;
  }
  uint32_t cut = floor;
  if (P.n >= P.k) {
    const uint32_t kth = wave_kth_largest_n<kPoolN>(k3, P.k);
    cut = kth > cut ? kth : cut;
  }
  wave_lds_wait();
  int base = 0;
#pragma unroll
  for (int s = 0; s < kPoolN; ++s) {
    const bool keep = (s * kWave + l) < P.n && k3[s] >= cut;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
    if (keep) {
      const int pos = base + lanes_below(bal);
      P.key[pos] = k3[s];
      P.id[pos] = i3[s];
    }
    base += __popcll(bal);
  }
  P.n = base;
  P.thr = cut > P.thr ? cut : P.thr;
  wave_lds_wait();
}

template <typename E, bool kVec>
__device__ __forceinline__ int extract_any(const float (&v)[kVals], const float (&g)[kGroups],
                                           float lmax, int tile_base, int V, uint32_t thr,
                                           const Pool& P) {
  const float pre = prefilter(thr, P.T);
  if (__builtin_amdgcn_ballot_w64(lmax >= pre) == 0ull) return 0;  // nothing in the tile
  if (P.T == 1.0f)
    return extract<E, kVec, true>(v, g, tile_base, V, pre, thr, P.T, P.key + P.n, P.id + P.n,
                                  kPool - P.n);
  return extract<E, kVec, false>(v, g, tile_base, V, pre, thr, P.T, P.key + P.n, P.id + P.n,
                                 kPool - P.n);
}

// Adds one tile to the pool.
template <typename E>
__device__ __forceinline__ void pool_tile(const float (&v)[kVals], const float (&g)[kGroups],
                                          float lmax, int tile_base, int V, bool vec, Pool& P) {
  if (P.ovf) return;
  const uint32_t sh = lds_load_relaxed(P.shared_thr);
  uint32_t thr = P.thr > sh ? P.thr : sh;
  bool publish = false;
  if (thr == 0u) {  // no bound yet
    thr = tile_bound(v, lmax, P.k, P.T);
    publish = true;
  }
  int n = vec ? extract_any<E, true>(v, g, lmax, tile_base, V, thr, P)
              : extract_any<E, false>(v, g, lmax, tile_base, V, thr, P);
  if (P.n + n > kPool) {
    // Too many: raise the bound with this tile's own and the pool's k-th.
    uint32_t t2 = publish ? thr : tile_bound(v, lmax, P.k, P.T);
    t2 = t2 > thr ? t2 : thr;
    pool_compact(P, t2);
    t2 = P.thr > t2 ? P.thr : t2;
    n = vec ? extract_any<E, true>(v, g, lmax, tile_base, V, t2, P)
            : extract_any<E, false>(v, g, lmax, tile_base, V, t2, P);
    if (P.n + n > kPool) {
      P.ovf = true;
      return;
    }
    thr = t2;
    publish = true;
  }
  P.n += n;
  P.thr = thr > P.thr ? thr : P.thr;
  if (P.n > kCompactAt && P.n >= P.k) {
    pool_compact(P, P.thr);
    publish = true;
  }
  if (publish && lane() == 0) atomicMax(P.shared_thr, P.thr);
}

// Workgroup LDS, laid out at run time for W waves.
struct Layout {
  static constexpr int kPoolBytes = kPool * 8;  // keys and ids
  int W;
  __device__ __forceinline__ uint32_t* pool_key(char* base, int w, int list) const {
    return reinterpret_cast<uint32_t*>(base + (w * 2 + list) * kPoolBytes);
  }
  __device__ __forceinline__ int32_t* pool_id(char* base, int w, int list) const {
    return reinterpret_cast<int32_t*>(base + (w * 2 + list) * kPoolBytes + kPool * 4);
  }
  __device__ __forceinline__ uint64_t* merge(char* base) const {
    return reinterpret_cast<uint64_t*>(base + W * 2 * kPoolBytes);
  }
};

struct SegSh {
  uint32_t thr[2];
  int merge_n;
  int ovf[2];
  uint32_t flags;
  uint32_t hist[256];
  uint32_t prefix;
  int krem;
  int out_n;
  float wm[16];
  float ws[16];
  uint64_t best[2][16];
};

__host__ __device__ inline size_t dyn_lds_bytes(int W) {
  return static_cast<size_t>(W) * 2 * Layout::kPoolBytes + kMergeCap * sizeof(uint64_t);
}

// Exact k-th largest key of n (<= kMergeCap) packed entries, with the whole
// block: four 8-bit digit passes over LDS histograms.
__device__ uint32_t block_kth_key(const uint64_t* a, int n, int k, SegSh& sh) {
  uint32_t prefix = 0;
  for (int d = 3; d >= 0; --d) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) sh.hist[i] = 0u;
    __syncthreads();
    const uint32_t hmask = (d == 3) ? 0u : (0xffffffffu << (8 * (d + 1)));
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const uint32_t key = pkey(a[i]);
      if ((key & hmask) == prefix) atomicAdd(&sh.hist[(key >> (8 * d)) & 0xffu], 1u);
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      // bins scanned from the top: lane l owns bins 255-4l .. 252-4l
      uint32_t c[4];
      uint32_t lsum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = sh.hist[255 - 4 * threadIdx.x - i];
        lsum += c[i];
      }
      uint32_t incl = lsum;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t t = __shfl_up(incl, off);
        if (static_cast<int>(threadIdx.x) >= off) incl += t;
      }
      uint32_t above = incl - lsum;
      int found = -1;
      uint32_t above_found = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (found < 0 && above + c[i] >= static_cast<uint32_t>(k)) {
          found = 255 - 4 * static_cast<int>(threadIdx.x) - i;
          above_found = above;
        }
        above += c[i];
      }
      const uint64_t bal = __ballot(found >= 0);
      const int l0 = __ffsll(static_cast<unsigned long long>(bal)) - 1;
      if (static_cast<int>(threadIdx.x) == l0) {
        sh.prefix = prefix | (static_cast<uint32_t>(found) << (8 * d));
        sh.krem = k - static_cast<int>(above_found);
      }
    }
    __syncthreads();
    prefix = sh.prefix;
    k = sh.krem;
    __syncthreads();
  }
  return prefix;
}

// Merges list `li` of the W pools: writes the segment's candidates (every
// value whose key reaches the segment's exact k-th largest key) and that key.
// Returns the count, or -1 on overflow. Called by the whole block.
__device__ int merge_list(char* dyn, const Layout& lay, SegSh& sh, int li, int k,
                          const uint32_t* pkey_, const int32_t* pid_, int pn, bool povf,
                          uint64_t* __restrict__ out, uint32_t* kth_out) {
  const int w = threadIdx.x / kWave;
  const int l = lane();
  uint64_t* mb = lay.merge(dyn);
  __syncthreads();  // every thread is done with the previous merge's counters
  if (threadIdx.x == 0) {
    sh.merge_n = 0;
    sh.out_n = 0;
  }
  __syncthreads();
  const uint32_t thr = sh.thr[li];
  if (!povf) {
#pragma unroll
    for (int s = 0; s < kPoolN; ++s) {
      const int slot = s * kWave + l;
      const uint32_t key = slot < pn ? pkey_[slot] : 0u;
      const bool take = slot < pn && key >= thr;
      const uint64_t bal = __builtin_amdgcn_ballot_w64(take);
      int b0 = 0;
      if (l == 0 && bal) b0 = atomicAdd(&sh.merge_n, __popcll(bal));
      b0 = __shfl(b0, 0);
      if (take) {
        const int pos = b0 + lanes_below(bal);
        if (pos < kMergeCap) mb[pos] = pack(key, pid_[slot]);
      }
    }
  } else if (l == 0) {
    sh.ovf[li] = 1;
  }
  __syncthreads();
  const int n = sh.merge_n;
  if (sh.ovf[li] || n > kMergeCap) return -1;
  uint32_t kth = 0;
  if (n >= k) {
    if (n <= kPool) {
      if (w == 0) {
        uint32_t k3[kPoolN];
#pragma unroll
        for (int s = 0; s < kPoolN; ++s) {
          const int slot = s * kWave + l;
          k3[s] = slot < n ? pkey(mb[slot]) : 0u;
        }
        const uint32_t t = wave_kth_largest_n<kPoolN>(k3, k);
        if (l == 0) sh.prefix = t;
      }
      __syncthreads();
      kth = sh.prefix;
      __syncthreads();
    } else {
      kth = block_kth_key(mb, n, k, sh);
    }
  }
  // every entry reaching kth goes out (order is irrelevant to the reader)
  for (int i0 = 0; i0 < n; i0 += blockDim.x) {
    const int i = i0 + static_cast<int>(threadIdx.x);
    const uint64_t e = i < n ? mb[i] : 0ull;
    const bool take = i < n && pkey(e) >= kth;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(take);
    int b0 = 0;
    if (l == 0 && bal) b0 = atomicAdd(&sh.out_n, __popcll(bal));
    b0 = __shfl(b0, 0);
    if (take) {
      const int pos = b0 + lanes_below(bal);
      if (pos < kSelCap) out[pos] = e;
    }
  }
  __syncthreads();
  const int c = sh.out_n;
  if (threadIdx.x == 0) *kth_out = kth;
  return c > kSelCap ? -1 : c;
}

template <typename E, bool kStream>
__global__ __launch_bounds__(1024) void k_select(Job j) {
  extern __shared__ __align__(16) char dyn[];
  __shared__ SegSh sh;
  int row, seg;
  if (!xcd_row_tile(blockIdx.x, j.B, j.nseg, &row, &seg)) return;  // uniform per block
  const int W = blockDim.x / kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = lane();
  const Layout lay{W};
  const Plan pl = plan_row(j, row);
  const int t_begin = seg * j.tps;
  const int t_end = min(t_begin + j.tps, j.ntile);

  if (threadIdx.x == 0) {
    sh.thr[0] = sh.thr[1] = 0u;
    sh.ovf[0] = sh.ovf[1] = 0;
    sh.flags = 0u;
  }
  __syncthreads();

  Pool PA{lay.pool_key(dyn, w, 0), lay.pool_id(dyn, w, 0), &sh.thr[0], pl.kA, pl.TA, 0, 0u, false};
  Pool PB{lay.pool_key(dyn, w, 1), lay.pool_id(dyn, w, 1), &sh.thr[1], pl.kB, 1.0f, 0, 0u, false};
  const E* rowp = static_cast<const E*>(j.logits) + static_cast<int64_t>(row) * j.ld;

  float Mw = -kInf, Sw = 0.0f;  // this wave's log-sum-exp partial
  uint64_t bestA = 0ull, bestB = 0ull;
  bool bad = false, fin = false;
  // Each wave walks its tiles with the next tile's loads in flight while the
  // current one is processed: two register buffers used in turn, and a load
  // issued for every step (of the row's first 16 bytes when there is no next
  // full tile) so that the wait before a buffer's use covers only that buffer.
  auto full_tile = [&](int tt) __attribute__((always_inline)) {
    return j.aligned && (tt + 1) * kSelTile <= j.V;
  };
  auto issue = [&](Raw<E>& X, int tt) __attribute__((always_inline)) {
    const bool real = tt < t_end && full_tile(tt);  // else a placeholder load
    load_raw<E, kStream>(rowp + (real ? tt * kSelTile : 0), real ? 1 : 0, X);
  };
  auto step = [&](const float (&v)[kVals], int tt, bool vec) __attribute__((always_inline)) {
    const int tile_base = tt * kSelTile;
    // NaN-propagating maximum: a lane maximum is NaN or +inf exactly when the
    // lane holds a NaN or a +inf, which make the row invalid.
    float g[kGroups];
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) {
      float m = v[gi * kGroup];
#pragma unroll
      for (int u = 1; u < kGroup; ++u) m = __builtin_elementwise_maximum(m, v[gi * kGroup + u]);
      g[gi] = m;
    }
    float lmax = g[0];
#pragma unroll
    for (int gi = 1; gi < kGroups; ++gi) lmax = __builtin_elementwise_maximum(lmax, g[gi]);
    bad = bad || (__ballot(!(lmax < kInf)) != 0ull);
    const float M = wave_max_dpp(lmax);
    fin = fin || M > -kInf;

    if (j.lse && M > -kInf) {
      // sum of 2^(x log2 e - c) with c = fl(M log2 e) (one fma and one exp2 per
      // value), then times 2^-r with r = M log2 e - c exactly: the sum of
      // exp(x - M) up to the rounding of each term
      float sl = 0.0f;
      float corr;
      if (fabsf(M) < 0x1p100f) {
        const float c = M * kL2E;
        const float r = fmaf(M, kL2E, -c);
        float s2[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // independent partial sums
#pragma unroll
        for (int q = 0; q < kVals; ++q) s2[q & 3] += __builtin_amdgcn_exp2f(fmaf(v[q], kL2E, -c));
        sl = (s2[0] + s2[1]) + (s2[2] + s2[3]);
        corr = __builtin_amdgcn_exp2f(-r);
      } else {
#pragma unroll
        for (int q = 0; q < kVals; ++q) sl += __expf(v[q] - M);
        corr = 1.0f;
      }
      const float st = wave_sum_dpp(sl) * corr;
      if (M > Mw) {
        Sw = (Mw > -kInf ? Sw * __expf(Mw - M) : 0.0f) + st;
        Mw = M;
      } else {
        Sw += st * __expf(M - Mw);
      }
    }

    if (pl.kA == 1 || pl.kB == 1) {
      const uint64_t best = tile_argmax<E>(v, M, tile_base, j.V, vec);
      if (pl.kA == 1) bestA = best > bestA ? best : bestA;
      if (pl.kB == 1) bestB = best > bestB ? best : bestB;
    }
    if (pl.kA > 1) pool_tile<E>(v, g, lmax, tile_base, j.V, vec, PA);
    if (pl.kB > 1) pool_tile<E>(v, g, lmax, tile_base, j.V, vec, PB);
  };
  int t = t_begin + w;
  if (j.aligned && j.V >= kSelTile) {  // full tiles exist: row element 0 starts one
    const int tf_end = min(t_end, j.V / kSelTile);  // this segment's full tiles end here
    Raw<E> A, Bf;
    issue(A, t);
    while (t < tf_end) {
      issue(Bf, t + W);
      {
        float v[kVals];
        unpack_raw<E>(A, rowp, v);
        step(v, t, true);
      }
      t += W;
      if (t >= tf_end) break;
      issue(A, t + W);
      {
        float v[kVals];
        unpack_raw<E>(Bf, rowp, v);
        step(v, t, true);
      }
      t += W;
    }
  }
  // the tiles left: the row's last, partial tile, or all of them when the row
  // is not 16-byte aligned
  for (; t < t_end; t += W) {
    float v[kVals];
    load_tail<E>(rowp, t * kSelTile, j.V, v);
    step(v, t, false);
  }

  // Shrink each pool to its exact top k (and ties) and share the bound.
  if (pl.kA > 1 && !PA.ovf && PA.n > PA.k) {
    pool_compact(PA, PA.thr);
    if (l == 0) atomicMax(PA.shared_thr, PA.thr);
  }
  if (pl.kB > 1 && !PB.ovf && PB.n > PB.k) {
    pool_compact(PB, PB.thr);
    if (l == 0) atomicMax(PB.shared_thr, PB.thr);
  }
  if (l == 0) {
    sh.wm[w] = Mw;
    sh.ws[w] = Sw;
    sh.best[0][w] = bestA;
    sh.best[1][w] = bestB;
    uint32_t f = bad ? kMetaBadLogits : 0u;
    if (fin) f |= kMetaHasFinite;
    if (f) atomicOr(&sh.flags, f);
  }
  __syncthreads();

  const size_t slot = static_cast<size_t>(row) * j.nseg + seg;
  uint32_t meta = sh.flags;
  if (pl.kA > 1) {
    const int n = merge_list(dyn, lay, sh, 0, pl.kA, PA.key, PA.id, PA.n, PA.ovf,
                             j.candA + slot * kSelCap, &j.kthA[slot]);
    meta |= (n < 0) ? kMetaOverflowA : static_cast<uint32_t>(n);
  }
  if (pl.kB > 1) {
    const int n = merge_list(dyn, lay, sh, 1, pl.kB, PB.key, PB.id, PB.n, PB.ovf,
                             j.candB + slot * kSelCap, &j.kthB[slot]);
    meta |= (n < 0) ? kMetaOverflowB : (static_cast<uint32_t>(n) << kMetaCountBShift);
  }
  if (threadIdx.x == 0) {
    float M = -kInf;
    uint64_t bA = 0ull, bB = 0ull;
    for (int i = 0; i < W; ++i) {
      M = fmaxf(M, sh.wm[i]);
      bA = sh.best[0][i] > bA ? sh.best[0][i] : bA;
      bB = sh.best[1][i] > bB ? sh.best[1][i] : bB;
    }
    if (j.lse) {
      float S = 0.0f;
      if (M > -kInf) {
        for (int i = 0; i < W; ++i)
          if (sh.wm[i] > -kInf) S += sh.ws[i] * __expf(sh.wm[i] - M);
      }
      j.lpart[slot] = LsePart{M, S};
    }
    if (pl.kA == 1) {
      if (bA) {
        meta |= 1u;
        j.candA[slot * kSelCap] = bA;
      }
      j.kthA[slot] = pkey(bA);  // the segment maximum: its 1st-largest key
    }
    if (pl.kB == 1) {
      if (bB) {
        meta |= 1u << kMetaCountBShift;
        j.candB[slot * kSelCap] = bB;
      }
      j.kthB[slot] = pkey(bB);
    }
    j.meta[slot] = meta;
  }
}

}  // namespace

hipError_t launch_select(const Job& j, hipStream_t st) {
  const int grid = xcd_grid(j.B, j.nseg);
  const dim3 block(kWave * j.nwave);
  const size_t lds = dyn_lds_bytes(j.nwave);
  // Logits read once (no later kernel reads them again: no full log-softmax
  // output, and no full-vocabulary rows) stream past the caches.
  const bool stream = !j.out_full &&
                      (!j.sample || (j.hints & (VS_HINT_NO_FULLVOCAB | VS_HINT_ALL_GREEDY)));
  if (j.dt == VS_F32) {
    if (stream)
      hipLaunchKernelGGL((k_select<float, true>), dim3(grid), block, lds, st, j);
    else
      hipLaunchKernelGGL((k_select<float, false>), dim3(grid), block, lds, st, j);
  } else {
    if (stream)
      hipLaunchKernelGGL((k_select<uint16_t, true>), dim3(grid), block, lds, st, j);
    else
      hipLaunchKernelGGL((k_select<uint16_t, false>), dim3(grid), block, lds, st, j);
  }
  return hipGetLastError();
}

}  // namespace vsk
