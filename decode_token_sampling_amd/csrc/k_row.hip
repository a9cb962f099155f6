// Row kernels, after the streaming pass.
//
// k_row_light (256 threads per row) finishes every row that does not need the
// whole vocabulary:
//  - greedy rows: the lowest id of the row maximum, from the tiles' argmaxes;
//  - top-k rows (k <= 64): the exact top k of the union of the tiles' candidate
//    lists (a radix select over packed (key, id) values), sorted, then min-p,
//    top-p on fixed-point masses and the Gumbel-max draw in one wave;
//  - top-k rows with k > 64, or whose tiles overflowed: an exact radix select
//    of the k-th key over the row itself (three digit passes), the last kept
//    id inside a tie group, and a gather of exactly k ids;
//  - full-vocabulary rows: the row maximum m of s = x / T, handed on;
//  - log-probabilities: log-sum-exp from the tile partials, the top-k log-probs
//    from the candidate lists, and the log-prob of the sampled or given ids.
// k_row_full (1024 threads per row) finds the top-p cut of full-vocabulary rows:
// a histogram of fixed-point masses over 4096 buckets of (s - m) (128 per unit,
// monotone in s), the bucket where the cumulative mass reaches top_p * total,
// then the exact cut inside that bucket (gathered and sorted in LDS, or by a
// mass-weighted radix select when the bucket holds more than 8192 ids).
// When a call runs the full-vocabulary passes, the light kernel is not
// launched: k_row_full does its work at entry (same code, same results), the
// streaming pass clears the histogram counters, and every row is routed to the
// full-vocabulary path from its tiles' flags and maxima alone (route_row), so
// no row descriptor has to exist before the histogram pass.
#include "vs_device.h"
#include "vs_kernels.h"

namespace vsk {
namespace {

constexpr int kLightThreads = 256;
constexpr int kFullThreads = 1024;
constexpr int kSortCutMax = kFullThreads;  // longest gathered list cut by the sort (one entry per thread)
static_assert(kFullThreads <= kFullListCap, "every thread of the cut kernel has a list slot");
// Longest candidate union whose k best come from per-wave chunk sorts alone
// (four chunks per wave of the row kernel); longer ones are cut to the k-th
// largest first.
constexpr int kTopChunkMax = 1024;
constexpr int kBuckets = kFullBuckets;
constexpr int kMaxSegs = (VS_MAX_V + kSegMin - 1) / kSegMin;

template <int kBuf, int kBins>
struct RowSh {
  static constexpr int kBufCap = kBuf;
  static constexpr int kBinCap = kBins;
  uint64_t buf[kBuf];
  uint64_t hw[kBins];
  uint32_t hc[kBins];
  uint64_t r64[16];
  uint64_t r64b[16];
  double rd[16];
  int32_t ri[16];
  float rf[16];
  int n;
  uint32_t flags;
  uint64_t b64[4];
  int32_t b32[4];
  int32_t toff[kMaxSegs + 1];  // per-segment offsets of a candidate union
  int32_t rk[16];              // per-wave kept counts of a draw
  int32_t cr32[2][4];          // a long-list cut's round results (alternating)
  uint64_t cr64[2][4];
  uint64_t cut_v;              // a top-p cut as written to the descriptor:
  int32_t cut_kept;            //   pack(tau, id_cut) and the kept count
};
// A top-p cut into the row's descriptor, and into LDS for the workgroup's
// own draw (published by the caller's next barrier).
template <class Sh>
__device__ __forceinline__ void set_cut(RowDesc* d, Sh& sh, uint32_t mode, uint32_t tau,
                                        int32_t id_cut, int32_t kept) {
  d->mode = mode;
  d->tau = tau;
  d->id_cut = id_cut;
  d->kept = kept;
  sh.cut_v = pack(tau, id_cut);
  sh.cut_kept = kept;
}
// Candidate slots of rows short enough to be loaded whole at the row kernel's
// entry (segments x kSelCap), and the segments those rows may have.
constexpr int kStageMax = 1024;
constexpr int kStageSegs = kStageMax / kSelCap;
struct LightSh : RowSh<4096, 2048> {
  uint64_t stage[2][kStageMax];  // lists A and B, every slot of every segment
  uint32_t segm[kStageSegs];     // each segment's meta word
  uint32_t segk[2][kStageSegs];  // each segment's exact k-th key, per list
  LsePart segl[kStageSegs];      // each segment's log-sum-exp partial
};
using FullSh = RowSh<kFullListCap, kBuckets>;

__device__ __forceinline__ float scaled(float x, float T) { return (T == 1.0f) ? x : x / T; }

// Visit every element (j, x) of a row with the whole block; 16-byte loads,
// four in flight per thread.
template <typename E, typename F>
__device__ __forceinline__ void row_visit(const E* __restrict__ rowp, int V, bool aligned, F&& f) {
  constexpr int EPV = Epv<E>::n;
  constexpr int U = 4;
  int j0 = 0;
  if (aligned) {
    const int nvec = V / EPV;
    const int st = blockDim.x;
    int i = threadIdx.x;
    for (; i + (U - 1) * st < nvec; i += U * st) {
      uint4 raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) raw[u] = *reinterpret_cast<const uint4*>(rowp + (i + u * st) * EPV);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float x[EPV];
        unpack16(raw[u], x, rowp);
#pragma unroll
        for (int c = 0; c < EPV; ++c) f((i + u * st) * EPV + c, x[c]);
      }
    }
    for (; i < nvec; i += st) {
      const uint4 raw = *reinterpret_cast<const uint4*>(rowp + i * EPV);
      float x[EPV];
      unpack16(raw, x, rowp);
#pragma unroll
      for (int c = 0; c < EPV; ++c) f(i * EPV + c, x[c]);
    }
    j0 = nvec * EPV;
  }
  for (int j = j0 + threadIdx.x; j < V; j += blockDim.x) f(j, to_f32(rowp[j]));
}

// Block-wide search over a histogram of nb bins scanned from the highest bin
// down (bin order = value order): the bin d with above < rem <= above + w[d],
// where above is the weight of the bins higher than d. Returns d (or -1), with
// the weight and count above it.
template <class Sh>
__device__ int hist_find_desc(Sh& sh, int nb, uint64_t rem, uint64_t* above_w, uint64_t* above_c) {
  const int G = (nb + blockDim.x - 1) / blockDim.x;
  uint64_t lw = 0, lc = 0;
  for (int g = 0; g < G; ++g) {
    const int i = threadIdx.x * G + g;
    if (i < nb) {
      lw += sh.hw[nb - 1 - i];
      lc += sh.hc[nb - 1 - i];
    }
  }
  uint64_t tw, tc;
  const uint64_t iw = block_scan_incl(lw, sh.r64, &tw);
  const uint64_t ic = block_scan_incl(lc, sh.r64, &tc);
  if (threadIdx.x == 0) sh.b32[0] = -1;
  __syncthreads();
  uint64_t ew = iw - lw, ec = ic - lc;
  for (int g = 0; g < G; ++g) {
    const int i = threadIdx.x * G + g;
    if (i < nb) {
      const int d = nb - 1 - i;
      const uint64_t w = sh.hw[d];
      if (ew < rem && rem <= ew + w) {
        sh.b32[0] = d;
        sh.b64[0] = ew;
        sh.b64[1] = ec;
      }
      ew += w;
      ec += sh.hc[d];
    }
  }
  __syncthreads();
  const int d = sh.b32[0];
  *above_w = sh.b64[0];
  *above_c = sh.b64[1];
  __syncthreads();
  return d;
}

// Exact weighted selection over the ordered keys of s = x / T for the ids that
// `pick` accepts (pick(j, s, key, &w) returns whether j takes part, with its
// weight w; equal keys must have equal weights). Finds the key tau of the
// element at which the cumulative weight, in the order (key desc, id asc),
// first reaches rem. Three digit passes (11, 11, 10 bits). Outputs the weight
// and count strictly above tau and the weight of one tau element.
template <typename E, class Sh, typename Pick>
__device__ void radix_select(const E* __restrict__ rowp, int V, bool aligned, float T, uint64_t rem,
                             Pick pick, Sh& sh, uint32_t* tau, uint64_t* w_above,
                             uint64_t* c_above, uint64_t* w_tau) {
  static_assert(Sh::kBinCap >= 2048, "radix select needs 2048 bins");
  uint32_t prefix = 0, pmask = 0;
  uint64_t wa = 0, ca = 0;
  const int shifts[3] = {21, 10, 0};
  const int nbits[3] = {11, 11, 10};
  int d = 0;
  for (int pass = 0; pass < 3; ++pass) {
    const int shf = shifts[pass], nb = 1 << nbits[pass];
    for (int i = threadIdx.x; i < nb; i += blockDim.x) {
      sh.hw[i] = 0;
      sh.hc[i] = 0;
    }
    __syncthreads();
    row_visit(rowp, V, aligned, [&](int j, float x) {
      const float s = scaled(x, T);
      const uint32_t key = f2key(s);
      if ((key & pmask) != prefix) return;
      uint64_t w;
      if (!pick(j, s, key, &w)) return;
      const uint32_t dd = (key >> shf) & static_cast<uint32_t>(nb - 1);
      atomicAdd(reinterpret_cast<unsigned long long*>(&sh.hw[dd]), static_cast<unsigned long long>(w));
      atomicAdd(&sh.hc[dd], 1u);
    });
    __syncthreads();
    uint64_t aw, ac;
    d = hist_find_desc(sh, nb, rem, &aw, &ac);
    if (d < 0) d = 0;  // unreachable when rem <= total weight
    rem -= aw;
    wa += aw;
    ca += ac;
    prefix |= static_cast<uint32_t>(d) << shf;
    pmask |= static_cast<uint32_t>(nb - 1) << shf;
  }
  const uint32_t cnt = sh.hc[d];
  *w_tau = cnt ? sh.hw[d] / cnt : 0;
  *tau = prefix;
  *w_above = wa;
  *c_above = ca;
  __syncthreads();
}

// The id of the need-th (1-based) element, in increasing id order, whose key
// equals tau and that `pick` accepts.
template <typename E, class Sh, typename Pick>
__device__ int32_t tie_cut(const E* __restrict__ rowp, int V, float T, uint32_t tau, uint64_t need,
                           Pick pick, Sh& sh) {
  constexpr int PER = 16;
  if (threadIdx.x == 0) sh.b32[1] = -1;
  __syncthreads();
  uint64_t base = 0;
  for (int c0 = 0; c0 < V; c0 += blockDim.x * PER) {
    const int j0 = c0 + threadIdx.x * PER;
    uint32_t cnt = 0;
    for (int e = 0; e < PER; ++e) {
      const int j = j0 + e;
      if (j < V) {
        const float s = scaled(to_f32(rowp[j]), T);
        const uint32_t key = f2key(s);
        uint64_t w;
        if (key == tau && pick(j, s, key, &w)) ++cnt;
      }
    }
    uint64_t tot;
    const uint64_t incl = block_scan_incl(static_cast<uint64_t>(cnt), sh.r64, &tot);
    const uint64_t excl = incl - cnt;
    if (cnt && base + excl < need && need <= base + incl) {
      uint64_t want = need - base - excl;
      for (int e = 0; e < PER; ++e) {
        const int j = j0 + e;
        if (j < V) {
          const float s = scaled(to_f32(rowp[j]), T);
          const uint32_t key = f2key(s);
          uint64_t w;
          if (key == tau && pick(j, s, key, &w) && --want == 0) {
            sh.b32[1] = j;
            break;
          }
        }
      }
    }
    base += tot;
    if (base >= need) break;
  }
  __syncthreads();
  const int32_t r = sh.b32[1];
  __syncthreads();
  return r;
}

// Sort the first n entries of a (shared) array, larger first; pads to a power
// of two no larger than cap.
__device__ __forceinline__ void sort_desc(uint64_t* a, int n) {
  const int np = next_pow2(n < 2 ? 2 : n);
  for (int i = n + threadIdx.x; i < np; i += blockDim.x) a[i] = 0ull;
  __syncthreads();
  block_sort_desc(a, np);
}

// The min(n, 64) largest of n values in shared memory, sorted descending into
// a[0..), by the block's waves with no block-wide network: wave w sorts the
// 64-entry chunks w, w + (waves), ... in registers and keeps the 64 best of
// them (a chunk sorted ascending merged into the best so far, descending);
// the other waves leave their best in a, reversed, and wave 0 merges them
// into its own. Entries of a past the result are left unspecified.
__device__ __forceinline__ void top64_sorted(uint64_t* a, int n) {
  const int w = static_cast<int>(threadIdx.x) / kWave;
  const int l = lane();
  const int nw = static_cast<int>(blockDim.x) / kWave;
  const int nchunk = (n + kWave - 1) / kWave;
  uint64_t v = 0ull;
  if (w < nchunk) {  // uniform per wave
    v = (w * kWave + l < n) ? a[w * kWave + l] : 0ull;
    v = wave_sort_u64<true>(v);
    for (int c = w + nw; c < nchunk; c += nw) {
      const uint64_t b = (c * kWave + l < n) ? a[c * kWave + l] : 0ull;
      v = wave_merge_top_u64(v, wave_sort_u64<false>(b));
    }
  }
  __syncthreads();  // every chunk is read
  if (w > 0 && w < nchunk) a[w * kWave + (kWave - 1 - l)] = v;  // ascending
  __syncthreads();
  if (w == 0) {
    for (int q = 1; q < nw && q < nchunk; ++q) v = wave_merge_top_u64(v, a[q * kWave + l]);
    a[l] = v;
  }
  __syncthreads();
}

// Exact k-th largest of n distinct packed values in shared memory: MSB-first
// radix select with 8-bit digits. Stops early once the remaining rank equals
// the size of the chosen bucket (the whole bucket is then selected and the
// prefix alone is a valid threshold). Every value >= the result is selected,
// exactly k of them (k <= n).
template <class Sh>
__device__ uint64_t block_kth_largest(const uint64_t* a, int n, int k, Sh& sh) {
  uint64_t prefix = 0, pmask = 0;
  int rem = k;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) sh.hc[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const uint64_t v = a[i];
      if ((v & pmask) == prefix) atomicAdd(&sh.hc[(v >> shift) & 255u], 1u);
    }
    __syncthreads();
    const int G = (256 + blockDim.x - 1) / blockDim.x;
    int lc = 0;
    for (int g = 0; g < G; ++g) {
      const int i = threadIdx.x * G + g;
      if (i < 256) lc += static_cast<int>(sh.hc[255 - i]);
    }
    int tot;
    int run = block_scan_incl(lc, sh.ri, &tot) - lc;
    if (threadIdx.x == 0) sh.b32[0] = -1;
    __syncthreads();
    for (int g = 0; g < G; ++g) {
      const int i = threadIdx.x * G + g;
      if (i < 256) {
        const int d = 255 - i;
        const int c = static_cast<int>(sh.hc[d]);
        if (run < rem && rem <= run + c) {
          sh.b32[0] = d;
          sh.b32[1] = run;
          sh.b32[2] = c;
        }
        run += c;
      }
    }
    __syncthreads();
    const int d = sh.b32[0] < 0 ? 0 : sh.b32[0];
    const int above = sh.b32[1], c = sh.b32[2];
    __syncthreads();
    rem -= above;
    prefix |= static_cast<uint64_t>(d) << shift;
    pmask |= 0xffull << shift;
    if (c == rem) break;
  }
  return prefix;
}

// union_topk for a row whose segments' words and candidate slots were loaded
// into LDS at the kernel's entry (stage: every slot of every segment, valid
// below each segment's count; segm and segk: the meta words and k-th keys):
// the same entries are gathered, with no global load. Every thread reads the
// few segments' words itself, so the early return is uniform.
template <class Sh>
__device__ __forceinline__ int union_topk_staged(const uint64_t* stage, const uint32_t* segm,
                                                 const uint32_t* segk, int ntile, int shift,
                                                 uint32_t ovf_flag, int k, Sh& sh) {
  uint32_t ovf = 0u, lp = 0u;
  for (int s = 0; s < ntile; ++s) {
    ovf |= segm[s] & ovf_flag;
    lp = segk[s] > lp ? segk[s] : lp;
  }
  if (ovf) return -1;
  const uint64_t pstar = static_cast<uint64_t>(lp) << 32;
  if (threadIdx.x == 0) sh.n = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < ntile * kSelCap; i += blockDim.x) {
    const int c = static_cast<int>((segm[i / kSelCap] >> shift) & 0xffu);
    const uint64_t v = stage[i];
    if ((i % kSelCap) < c && v >= pstar && v != 0ull) {
      const int pos = atomicAdd(&sh.n, 1);
      if (pos < Sh::kBufCap) sh.buf[pos] = v;
    }
  }
  __syncthreads();
  const int n = sh.n;
  __syncthreads();
  if (n > Sh::kBufCap) return -1;
  // n <= ntile * kSelCap <= kTopChunkMax: the k best sorted, without a block sort
  top64_sorted(sh.buf, n);
  return n < k ? n : k;
}

// The exact top k (order: key desc, id asc) of the union of one candidate list
// over the row's tiles, sorted into sh.buf[0..min(k, total)). Returns the
// count, or -1 when a tile overflowed or the union does not fit. Only entries
// whose key reaches P* = the largest per-tile exact k-th key are gathered: that
// tile alone holds k values >= P*, so no entry below it is in the row's top k.
template <class Sh>
__device__ __forceinline__ int union_topk(const uint32_t* __restrict__ mrow,
                                          const uint64_t* __restrict__ crow,
                                          const uint32_t* __restrict__ kth_row, int ntile,
                                          int shift, uint32_t ovf_flag, int k, Sh& sh) {
  // tile counts -> offsets (each thread owns consecutive tiles), and P*
  const int G = (ntile + blockDim.x - 1) / blockDim.x;
  int lc = 0, ovf = 0;
  uint32_t lp = 0;
  for (int g = 0; g < G; ++g) {
    const int t = threadIdx.x * G + g;
    if (t < ntile) {
      const uint32_t m = mrow[t];
      if (m & ovf_flag) ovf = 1;
      lc += static_cast<int>((m >> shift) & 0xffu);
      const uint32_t kt = kth_row[t];
      lp = kt > lp ? kt : lp;
    }
  }
  ovf = block_max(ovf, sh.ri);
  if (ovf) return -1;
  const uint64_t pstar = static_cast<uint64_t>(block_max(lp, reinterpret_cast<uint32_t*>(sh.ri)))
                         << 32;
  int total;
  int off = block_scan_incl(lc, sh.ri, &total) - lc;
  for (int g = 0; g < G; ++g) {
    const int t = threadIdx.x * G + g;
    if (t < ntile) {
      sh.toff[t] = off;
      off += static_cast<int>((mrow[t] >> shift) & 0xffu);
    }
  }
  if (threadIdx.x == 0) {
    sh.toff[ntile] = total;
    sh.n = 0;
  }
  __syncthreads();
  // Read the valid entries with all threads: entry g lives in the tile t with
  // toff[t] <= g < toff[t+1] (binary search in LDS). Four loads are issued
  // before any is used so their latencies overlap.
  constexpr int U = 4;
  for (int g0 = threadIdx.x; g0 < total; g0 += U * blockDim.x) {
    uint64_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = g0 + u * static_cast<int>(blockDim.x);
      v[u] = 0ull;
      if (g < total) {
        int lo = 0, hi = ntile - 1;  // last t with toff[t] <= g
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (sh.toff[mid] <= g) lo = mid; else hi = mid - 1;
        }
        v[u] = crow[static_cast<size_t>(lo) * kSelCap + (g - sh.toff[lo])];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (v[u] >= pstar && v[u] != 0ull) {
        const int pos = atomicAdd(&sh.n, 1);
        if (pos < Sh::kBufCap) sh.buf[pos] = v[u];
      }
    }
  }
  __syncthreads();
  int n = sh.n;
  __syncthreads();
  if (n > Sh::kBufCap) return -1;
  if (n > kTopChunkMax && n > k) {
    const uint64_t thr = block_kth_largest(sh.buf, n, k, sh);
    uint64_t* tmp = sh.hw;  // at least 2048 slots
    if (threadIdx.x == 0) sh.n = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const uint64_t v = sh.buf[i];
      if (v >= thr) tmp[atomicAdd(&sh.n, 1)] = v;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < k; i += blockDim.x) sh.buf[i] = tmp[i];
    __syncthreads();
    n = k;
  }
  // n <= kTopChunkMax here (k <= 64): the k best sorted, without a block sort
  top64_sorted(sh.buf, n);
  return n < k ? n : k;
}

// Exact top k of s = x / T over the row data (k <= 1024); sorted into sh.buf.
template <typename E, class Sh>
__device__ int slow_topk(const E* __restrict__ rowp, int V, bool aligned, float T, int k, Sh& sh) {
  auto all = [](int, float, uint32_t, uint64_t* w) {
    *w = 1;
    return true;
  };
  uint32_t tau;
  uint64_t wa, ca, wt;
  radix_select(rowp, V, aligned, T, static_cast<uint64_t>(k), all, sh, &tau, &wa, &ca, &wt);
  const uint64_t need = static_cast<uint64_t>(k) - ca;
  const int32_t idc = tie_cut(rowp, V, T, tau, need, all, sh);
  if (threadIdx.x == 0) sh.n = 0;
  __syncthreads();
  row_visit(rowp, V, aligned, [&](int j, float x) {
    const uint32_t key = f2key(scaled(x, T));
    if (key > tau || (key == tau && j <= idc)) {
      const int pos = atomicAdd(&sh.n, 1);
      if (pos < Sh::kBufCap) sh.buf[pos] = pack(key, j);
    }
  });
  __syncthreads();
  int n = sh.n;
  __syncthreads();
  if (n > k) n = k;  // cannot happen: exactly k ids pass
  sort_desc(sh.buf, n);
  return n;
}

// Truncate and draw over the n (<= 4 * blockDim) sorted candidates L. Returns
// the status (0, or VS_ROW_BAD_PARAM when x / T overflowed to +inf).
template <class Sh>
__device__ int block_draw(const uint64_t* L, int n, const RowCfg& c, int row, int32_t* id_out,
                          int32_t* kept_out, uint32_t* mask_row, Sh& sh) {
  constexpr int PER = 4;
  if (n <= 0) return VS_ROW_BAD_LOGITS;  // no candidate: never read an id from it
  const uint64_t top = L[0];
  if (pkey(top) == kKeyPosInf) return VS_ROW_BAD_PARAM;
  const float m = key2f(pkey(top));
  float e[PER];
  bool in_s[PER], kept[PER];
  uint64_t W[PER];
  uint64_t lsum = 0;
  for (int q = 0; q < PER; ++q) {
    const int i = threadIdx.x * PER + q;
    const bool has = i < n;
    e[q] = has ? pinned_exp(key2f(pkey(L[i])) - m) : 0.0f;
    in_s[q] = has && (e[q] >= c.mp);  // a prefix of the order: e is monotone in s
    W[q] = in_s[q] ? mass_of(e[q]) : 0ull;
    lsum += W[q];
  }
  if (c.p < 1.0f) {
    uint64_t tw;
    uint64_t run = block_scan_incl(lsum, sh.r64, &tw) - lsum;
    const double thr = static_cast<double>(c.p) * static_cast<double>(tw);
    int first = 0x7fffffff;
    for (int q = 0; q < PER; ++q) {
      run += W[q];
      if (in_s[q] && static_cast<double>(run) >= thr && first == 0x7fffffff)
        first = threadIdx.x * PER + q;
    }
    const int cut = block_min(first, sh.ri);
    for (int q = 0; q < PER; ++q) kept[q] = in_s[q] && (static_cast<int>(threadIdx.x) * PER + q) <= cut;
  } else {
    for (int q = 0; q < PER; ++q) kept[q] = in_s[q];
  }
  const uint64_t rs = row_stream(c.seed, row);
  double best = -1.0;
  int best_id = 0x7fffffff, nk = 0;
  for (int q = 0; q < PER; ++q) {
    if (!kept[q]) continue;
    const int i = threadIdx.x * PER + q;
    const int id = pid(L[i]);
    ++nk;
    const double sc = gumbel_score(e[q], rs, id);
    if (sc > best || (sc == best && id < best_id)) {
      best = sc;
      best_id = id;
    }
    if (mask_row) atomicOr(&mask_row[id >> 5], 1u << (id & 31));
  }
  const double bb = block_max(best, sh.rd);
  const int win = block_min(best == bb ? best_id : 0x7fffffff, sh.ri);
  const int total = block_sum(nk, sh.ri);
  *id_out = win;
  *kept_out = total;
  return 0;
}

template <typename E>
__device__ __forceinline__ float logit_at(const Job& j, int row, int id) {
  return to_f32(static_cast<const E*>(j.logits)[static_cast<int64_t>(row) * j.ld + id]);
}

// The loads the row kernel's work begins with (light_row), issued apart so
// that a caller can start them before it knows the row's route. A row of few
// segments has every per-segment word and every candidate slot loaded, before
// its parameters are known: the loads are independent, so their latencies
// overlap instead of following one another, and the steps that follow read
// LDS (stale slots past a segment's count included: they are never used).
// kPer: candidate slots per thread (kStageMax / the block size).
template <int kPer>
struct LightLoads {
  uint64_t sa[kPer], sb[kPer];
  uint32_t m0, kA0, kB0;
  LsePart lp0;
};
template <int kPer>
__device__ __forceinline__ void light_load(const Job& j, int row, LightLoads<kPer>& L) {
  const int ntile = j.nseg;
  const int t0 = static_cast<int>(threadIdx.x);
  L.m0 = L.kA0 = L.kB0 = 0u;
  L.lp0 = LsePart{-kInf, 0.0f};
  if (ntile <= kStageSegs) {  // uniform
    const size_t s0 = static_cast<size_t>(row) * ntile;
    const uint64_t* crowA = j.candA + s0 * kSelCap;
    const uint64_t* crowB = j.candB + s0 * kSelCap;
    const bool lists_b = j.lse && j.k_lp > 0;
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = t0 + r * static_cast<int>(blockDim.x);
      L.sa[r] = i < ntile * kSelCap ? crowA[i] : 0ull;
      L.sb[r] = (lists_b && i < ntile * kSelCap) ? crowB[i] : 0ull;
    }
    if (t0 < ntile) {
      L.m0 = j.meta[s0 + t0];
      L.kA0 = j.kthA[s0 + t0];
      L.kB0 = j.kthB[s0 + t0];
      if (j.lse) L.lp0 = j.lpart[s0 + t0];
    }
  }
}

// The row kernel's work for one row (a block of kStageMax / kPer threads,
// the loads of light_load in L): the row's draw, status, log-sum-exp and
// log-probs from the streaming pass's per-segment words, for every row the
// streaming pass did not finish and the full-vocabulary passes do not take.
template <typename E, int kPer>
__device__ __forceinline__ void light_row(const Job& j, int row, LightSh& sh,
                                          const LightLoads<kPer>& L) {
  if (j.nseg == 1 && (j.meta[row] & kMetaFinal)) return;  // finished by the streaming pass
  const int ntile = j.nseg;  // candidate lists and partials come per segment
  const uint32_t* mrow = j.meta + static_cast<size_t>(row) * ntile;
  const uint64_t* crowA = j.candA + static_cast<size_t>(row) * ntile * kSelCap;
  const uint64_t* crowB = j.candB + static_cast<size_t>(row) * ntile * kSelCap;
  const uint32_t* kthA = j.kthA + static_cast<size_t>(row) * ntile;
  const uint32_t* kthB = j.kthB + static_cast<size_t>(row) * ntile;
  const LsePart* lrow = j.lpart + static_cast<size_t>(row) * ntile;
  const E* rowp = static_cast<const E*>(j.logits) + static_cast<int64_t>(row) * j.ld;
  const bool aligned = j.aligned;
  const float nanv = __builtin_nanf("");
  const bool staged = ntile <= kStageSegs;  // uniform
  const int t0 = static_cast<int>(threadIdx.x);
  const int NT = static_cast<int>(blockDim.x);
  const uint32_t m0 = L.m0;
  const LsePart lp0 = L.lp0;
  const Plan pl = plan_row(j, row);
  const RowCfg& c = pl.c;
  if (staged) {
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int i = t0 + r * NT;
      if (i < kStageMax) {
        sh.stage[0][i] = L.sa[r];
        sh.stage[1][i] = L.sb[r];
      }
    }
    if (t0 < ntile) {
      sh.segm[t0] = m0;
      sh.segk[0][t0] = L.kA0;
      sh.segk[1][t0] = L.kB0;
      sh.segl[t0] = lp0;
    }
  }

  // flags over the tiles, the row argmax when list A holds argmaxes, and the
  // log-sum-exp from the tile partials: a staged row's few segments are
  // combined by every thread from LDS (in segment order, no block
  // reductions), a longer row's by the block
  uint32_t fl = 0;
  uint64_t top = 0;
  float M = -kInf, logS = nanv;
  if (staged) {
    __syncthreads();  // the staged words are visible
    for (int t = 0; t < ntile; ++t) {
      const uint32_t mt = sh.segm[t];
      fl |= mt;
      if (pl.kA == 1 && (mt & kMetaCountA)) {
        const uint64_t v = sh.stage[0][t * kSelCap];
        top = v > top ? v : top;
      }
    }
    if (j.lse) {
      for (int t = 0; t < ntile; ++t) M = fmaxf(M, sh.segl[t].m);
      float ls = 0.0f;
      if (M > -kInf) {
        for (int t = 0; t < ntile; ++t) {
          const LsePart pt = sh.segl[t];
          if (pt.m > -kInf) ls += pt.s * __expf(pt.m - M);
        }
      }
      logS = logf(ls);
    }
  } else {
    if (threadIdx.x == 0) sh.flags = 0u;
    __syncthreads();
    for (int t = threadIdx.x; t < ntile; t += blockDim.x) {
      const uint32_t m = mrow[t];
      fl |= m;
      if (pl.kA == 1 && (m & kMetaCountA)) {
        const uint64_t v = crowA[static_cast<size_t>(t) * kSelCap];
        top = v > top ? v : top;
      }
    }
    if (fl) atomicOr(&sh.flags, fl & (kMetaBadLogits | kMetaHasFinite));
    top = block_max(top, sh.r64);  // also orders the atomicOr above
    fl = sh.flags;
    if (j.lse) {
      float lm = -kInf;
      for (int t = threadIdx.x; t < ntile; t += blockDim.x) lm = fmaxf(lm, lrow[t].m);
      M = block_max(lm, sh.rf);
      float ls = 0.0f;
      if (M > -kInf) {
        for (int t = threadIdx.x; t < ntile; t += blockDim.x) {
          const LsePart pt = lrow[t];
          if (pt.m > -kInf) ls += pt.s * __expf(pt.m - M);
        }
      }
      logS = logf(block_sum(ls, sh.rf));
    }
  }
  const bool bad_logits = (fl & kMetaBadLogits) || !(fl & kMetaHasFinite);
  if (j.lse) {
    if (threadIdx.x == 0)
      j.rlse[row] = bad_logits ? make_float2(nanv, nanv) : make_float2(M, logS);
  }

  // the draw
  int sorted_shared = 0;  // entries of list A's exact top k left sorted in sh.buf
  if (j.sample) {
    const int mwords = (j.V + 31) / 32;
    uint32_t* mask_row = j.out_mask ? j.out_mask + static_cast<size_t>(row) * mwords : nullptr;
    if (mask_row) {
      for (int i = threadIdx.x; i < mwords; i += blockDim.x) mask_row[i] = 0u;
      __syncthreads();
    }
    int status = c.status | (bad_logits ? VS_ROW_BAD_LOGITS : 0);
    if (pl.kA == 1 && top == 0ull) status |= VS_ROW_BAD_LOGITS;  // no argmax was found
    if (status == 0) {
      if ((j.hints & VS_HINT_ALL_GREEDY) && c.mode != kModeGreedy) status = VS_ROW_HINT_VIOLATED;
      if ((j.hints & VS_HINT_NO_GREEDY) && c.mode == kModeGreedy) status = VS_ROW_HINT_VIOLATED;
      if ((j.hints & VS_HINT_NO_FULLVOCAB) && c.mode == kModeFull) status = VS_ROW_HINT_VIOLATED;
      if ((j.hints & VS_HINT_SMALL_TOPK) && c.mode != kModeGreedy && c.mode != kModeKFast)
        status = VS_ROW_HINT_VIOLATED;
    }
    int32_t id = -1, kept = 0;
    uint32_t next = kRowDone;
    if (status == 0) {
      if (c.mode == kModeGreedy) {
        id = pid(top);
        kept = 1;
        if (mask_row && threadIdx.x == 0) atomicOr(&mask_row[id >> 5], 1u << (id & 31));
      } else if (c.mode == kModeKFast || c.mode == kModeKSlow) {
        int n = -1;
        if (pl.kA > 1)
          n = staged ? union_topk_staged(sh.stage[0], sh.segm, sh.segk[0], ntile, 0, kMetaOverflowA, c.k, sh)
                     : union_topk(mrow, crowA, kthA, ntile, 0, kMetaOverflowA, c.k, sh);
        if (n < 0) n = slow_topk(rowp, j.V, aligned, c.T, c.k, sh);
        if (c.T == 1.0f) sorted_shared = n;
        if (n <= kWave) {
          if (threadIdx.x < kWave) {
            const int st = wave_draw(sh.buf, n, c, row, &id, &kept, mask_row);
            if (threadIdx.x == 0) {
              sh.b32[0] = st;
              sh.b32[1] = id;
              sh.b32[2] = kept;
            }
          }
          __syncthreads();
          status = sh.b32[0];
          id = sh.b32[1];
          kept = sh.b32[2];
          __syncthreads();
        } else {
          status = block_draw(sh.buf, n, c, row, &id, &kept, mask_row, sh);
        }
      } else {  // full vocabulary: the cut and the draw come later
        const float m = scaled(key2f(pkey(top)), c.T);
        if (m == kInf) {
          status = VS_ROW_BAD_PARAM;
        } else {
          // (the passes ran already: this is the cut kernel's entry, and
          // the streaming pass cleared their counters)
          next = kRowFull;
          if (threadIdx.x == 0) j.desc[row].m = m;
        }
      }
    }
    if (status) {
      id = -1;
      kept = 0;
      next = kRowDone;
    }
    if (threadIdx.x == 0) {
      j.desc[row].mode = next;
      if (next == kRowDone) {
        if (id >= j.V) {  // unreachable: every id comes from a tile of [0, V)
          id = -1;
          kept = 0;
          status = VS_ROW_BAD_LOGITS;
        }
        j.out_ids[row] = id;
        if (j.out_kept) j.out_kept[row] = kept;
        if (j.tok_sampled)
          j.out_tok_lp[row] = (id < 0 || bad_logits) ? nanv : (logit_at<E>(j, row, id) - M) - logS;
      }
      if (j.out_status) j.out_status[row] = status;
    }
    if (status && mask_row) {  // a row that failed reports an empty kept set
      __syncthreads();
      for (int i = threadIdx.x; i < mwords; i += blockDim.x) mask_row[i] = 0u;
    }
    __syncthreads();
  }

  // top-k log-probabilities
  if (j.lse && j.k_lp > 0) {
    const int k = j.k_lp;
    int32_t* ids = j.out_lp_ids + static_cast<size_t>(row) * k;
    float* lps = j.out_lp + static_cast<size_t>(row) * k;
    if (bad_logits) {
      for (int i = threadIdx.x; i < k; i += blockDim.x) {
        ids[i] = -1;
        lps[i] = nanv;
      }
    } else {
      int n;
      const uint64_t* src = sh.buf;
      if (pl.shared && pl.kA == 1) {  // k == 1 and list A holds the argmax
        n = 1;
        if (threadIdx.x == 0) sh.b64[2] = top;
        __syncthreads();
        src = &sh.b64[2];
      } else if (pl.shared && sorted_shared >= k) {
        n = sorted_shared;
      } else {
        if (staged)
          n = pl.shared ? union_topk_staged(sh.stage[0], sh.segm, sh.segk[0], ntile, 0, kMetaOverflowA,
                                            k, sh)
                        : union_topk_staged(sh.stage[1], sh.segm, sh.segk[1], ntile,
                                            kMetaCountBShift, kMetaOverflowB, k, sh);
        else
          n = pl.shared
                  ? union_topk(mrow, crowA, kthA, ntile, 0, kMetaOverflowA, k, sh)
                  : union_topk(mrow, crowB, kthB, ntile, kMetaCountBShift, kMetaOverflowB, k, sh);
        if (n < 0) n = slow_topk(rowp, j.V, aligned, lse_T(j, row), k, sh);
      }
      for (int i = threadIdx.x; i < k; i += blockDim.x) {
        if (i < n) {
          const uint64_t P = src[i];
          ids[i] = pid(P);
          lps[i] = (key2f(pkey(P)) - M) - logS;
        } else {
          ids[i] = -1;
          lps[i] = nanv;
        }
      }
    }
  }

  // log-probabilities of given ids (vs_logprobs)
  if (j.lse && !j.sample && threadIdx.x == 0) {
    int st = bad_logits ? VS_ROW_BAD_LOGITS : 0;
    if (j.tok) {
      const int tok = j.tok[row];
      const bool badtok = tok < 0 || tok >= j.V;
      if (badtok) st |= VS_ROW_BAD_TOKEN_ID;
      j.out_tok_lp[row] = (bad_logits || badtok)
                              ? nanv
                              : (lse_scaled(logit_at<E>(j, row, tok), lse_T(j, row)) - M) - logS;
    }
    if (j.out_lp_status) j.out_lp_status[row] = st;
  }
}

template <typename E>
__global__ __launch_bounds__(kLightThreads) void k_row_light(Job j) {
  __shared__ LightSh sh;
  const int row = static_cast<int>(blockIdx.x);
  LightLoads<kStageMax / kLightThreads> L;
  light_load(j, row, L);
  light_row<E>(j, row, sh, L);
}

template <typename E>
__device__ void full_topp_cut(const E* __restrict__ rowp, int V, bool aligned, float T, float p,
                              float mp, float m, FullSh& sh, RowDesc* d) {
  const FullTerms ft{m, mp};
  for (int i = threadIdx.x; i < kBuckets; i += blockDim.x) {
    sh.hw[i] = 0;
    sh.hc[i] = 0;
  }
  __syncthreads();
  row_visit(rowp, V, aligned, [&](int, float x) {
    uint64_t w;
    int b;
    if (ft.mass(scaled(x, T), &w, &b)) {
      atomicAdd(reinterpret_cast<unsigned long long*>(&sh.hw[b]), static_cast<unsigned long long>(w));
      atomicAdd(&sh.hc[b], 1u);
    }
  });
  __syncthreads();
  uint64_t lt = 0;
  for (int i = threadIdx.x; i < kBuckets; i += blockDim.x) lt += sh.hw[i];
  const uint64_t total = block_sum(lt, sh.r64);
  // The kept prefix is the shortest whose mass reaches thr; masses are
  // integers, so "cum >= thr" is "cum >= ceil(thr)".
  const double thr = static_cast<double>(p) * static_cast<double>(total);
  const uint64_t target = ceil(thr) >= 1.0 ? static_cast<uint64_t>(ceil(thr)) : 1ull;
  // Bucket 0 holds the largest s; hist_find_desc scans from the highest index
  // down, so present the buckets in reverse.
  for (int i = threadIdx.x; i < kBuckets / 2; i += blockDim.x) {
    const int o = kBuckets - 1 - i;
    const uint64_t tw = sh.hw[i];
    sh.hw[i] = sh.hw[o];
    sh.hw[o] = tw;
    const uint32_t tc = sh.hc[i];
    sh.hc[i] = sh.hc[o];
    sh.hc[o] = tc;
  }
  __syncthreads();
  uint64_t aw, ac;
  const int dr = hist_find_desc(sh, kBuckets, target, &aw, &ac);
  const int bstar = kBuckets - 1 - (dr < 0 ? kBuckets - 1 : dr);
  const uint32_t nb = sh.hc[kBuckets - 1 - bstar];
  const uint64_t rem = target - aw;
  __syncthreads();

  auto in_bucket = [&](int, float s, uint32_t, uint64_t* w) {
    int b;
    return ft.mass(s, w, &b) && b == bstar;
  };
  uint32_t tau;
  int32_t idc;
  int32_t kept;
  if (nb <= static_cast<uint32_t>(FullSh::kBufCap)) {
    if (threadIdx.x == 0) sh.n = 0;
    __syncthreads();
    row_visit(rowp, V, aligned, [&](int jj, float x) {
      const float s = scaled(x, T);
      uint64_t w;
      int b;
      if (ft.mass(s, &w, &b) && b == bstar) {
        const int pos = atomicAdd(&sh.n, 1);
        if (pos < FullSh::kBufCap) sh.buf[pos] = pack(f2key(s), jj);
      }
    });
    __syncthreads();
    const int n = sh.n < FullSh::kBufCap ? sh.n : FullSh::kBufCap;
    __syncthreads();
    sort_desc(sh.buf, n);
    // Cumulative mass inside the bucket, in order; the cut is the first index
    // where it reaches rem.
    constexpr int PER = FullSh::kBufCap / kFullThreads;
    uint64_t loc[PER];
    uint64_t lsum = 0;
    for (int e = 0; e < PER; ++e) {
      const int i = threadIdx.x * PER + e;
      uint64_t w = 0;
      int b;
      if (i < n) ft.mass(key2f(pkey(sh.buf[i])), &w, &b);
      loc[e] = w;
      lsum += w;
    }
    uint64_t tot;
    uint64_t run = block_scan_incl(lsum, sh.r64, &tot) - lsum;
    int first = 0x7fffffff;
    for (int e = 0; e < PER; ++e) {
      run += loc[e];
      const int i = threadIdx.x * PER + e;
      if (i < n && run >= rem && first == 0x7fffffff) first = i;
    }
    const int cut = block_min(first, sh.ri);
    const int cc = cut < n ? cut : (n > 0 ? n - 1 : 0);
    tau = pkey(sh.buf[cc]);
    idc = pid(sh.buf[cc]);
    kept = static_cast<int32_t>(ac) + cc + 1;
  } else {
    uint64_t wa, ca, wt;
    radix_select(rowp, V, aligned, T, rem, in_bucket, sh, &tau, &wa, &ca, &wt);
    const uint64_t r2 = rem - wa;
    const uint64_t need = wt ? (r2 + wt - 1) / wt : 1;
    idc = tie_cut(rowp, V, T, tau, need, in_bucket, sh);
    kept = static_cast<int32_t>(ac + ca + need);
  }
  if (threadIdx.x == 0) {
    set_cut(d, sh, kRowFullTopP, tau, idc, kept);
  }
}

// The top-p cut from the ids of the cut bucket, gathered by the parallel
// passes: the first entry, in the order (key desc, id asc), at which the mass
// inside the bucket reaches the remainder. For a list of at most one entry
// per thread: a bitonic sort of the packed values (whose descending order is
// that order), then a prefix sum of the masses in sorted order; the cut is
// the first entry whose running mass reaches the remainder. The sort runs
// each wave's 64 entries through an in-register network (runs of 64,
// descending in even waves and ascending in odd ones), then merges runs of
// 128, 256, ...: partner distances of 64 and more through LDS (two buffers
// in turn, so one barrier per step), the last six steps inside the wave.
// Masses are formed after the sort, from the keys. Called by every thread
// with its entry (v = 0 past the list: below every packed value, which holds
// ~id in its low half); xa and xb are two LDS buffers of blockDim entries.
// Returns false when the masses fall short of the remainder (not expected:
// the list holds the whole bucket). The result is the same in every thread.
__device__ __forceinline__ bool sort_cut_from_list(const FullCut& fc, int n, uint64_t v,
                                                   const FullTerms& ft, uint64_t* xa,
                                                   uint64_t* xb, FullSh& sh, RowDesc* d,
                                                   uint32_t mode) {
  const int t = static_cast<int>(threadIdx.x);
  const int wv = t / kWave;  // uniform per wave
  if (n <= kWave) {  // uniform: one wave sorts, scans and cuts; one barrier shares the outcome
    if (wv == 0) {
      v = wave_sort_u64<true>(v);
      uint32_t w = 0u;
      if (v != 0ull) {
        uint64_t wt;
        int b;
        w = ft.mass(key2f(pkey(v)), &wt, &b) ? static_cast<uint32_t>(wt) : 0u;
      }
      // masses (at most 2^31) scanned as 16-bit halves, whose sums over 64
      // lanes fit in 32 bits
      const uint32_t lo = wave_scan_incl_u32(w & 0xffffu);
      const uint32_t hi = wave_scan_incl_u32(w >> 16);
      const uint64_t cum = (static_cast<uint64_t>(hi) << 16) + lo;
      const int rank = __popcll(__ballot(cum < fc.rem));  // the running mass is nondecreasing
      if (rank < n && lane() == rank) {
        set_cut(d, sh, mode, pkey(v), pid(v), static_cast<int32_t>(fc.above_c) + rank + 1);
      }
      if (lane() == 0) sh.b32[3] = rank < n ? 1 : 0;
    }
    __syncthreads();
    return sh.b32[3] != 0;
  }
  // only the first P entries (P the power of two >= n) need sorting: every
  // entry past them is padding, and so is every sorted entry past n. Each
  // wave sorts its 64 in registers (descending); then runs of L merge
  // pairwise into 2L through two LDS buffers in turn, one barrier a level: an
  // entry's place in the merged run is its index in its own run plus the
  // entries of the partner run that come before it (a binary search; on
  // equal values, padding, those of the left run first).
  const int P = n <= 1 ? 1 : 1 << (32 - __clz(n - 1));
  if (wv * kWave < P) v = wave_sort_u64<true>(v);
  uint64_t* src = xa;
  uint64_t* dst = xb;
  if (t < P) src[t] = v;
  __syncthreads();
  for (int L = kWave; L < P; L <<= 1) {  // uniform
    if (t < P) {
      const int run = t / L, i = t - run * L;
      const uint64_t* pr = src + (run ^ 1) * L;
      const bool left = (run & 1) == 0;
      int lo = 0, hi = L;  // the partner entries before v: larger, or equal from the left run
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const uint64_t o = pr[mid];
        if (o > v || (!left && o == v)) lo = mid + 1;
        else hi = mid;
      }
      dst[(run & ~1) * L + i + lo] = v;
    }
    __syncthreads();
    uint64_t* tmp = src;
    src = dst;
    dst = tmp;
    if (t < P) v = src[t];
  }
  // thread t holds the entry of rank t; the running mass (in-wave DPP scans
  // of 16-bit halves, then the waves' totals: one barrier) first reaches the
  // remainder at the cut, whose rank is its thread's index
  uint32_t w = 0u;
  if (v != 0ull) {
    uint64_t wt;
    int b;
    w = ft.mass(key2f(pkey(v)), &wt, &b) ? static_cast<uint32_t>(wt) : 0u;
  }
  const uint32_t slo = wave_scan_incl_u32(w & 0xffffu);
  const uint32_t shi = wave_scan_incl_u32(w >> 16);
  const uint64_t in_w = (static_cast<uint64_t>(shi) << 16) + slo;
  if (lane() == kWave - 1) sh.r64[wv] = in_w;
  __syncthreads();
  uint64_t cum = in_w, total = 0ull;
  for (int q = 0; q < kFullThreads / kWave; ++q) {
    const uint64_t tq = sh.r64[q];
    cum += q < wv ? tq : 0ull;
    total += tq;
  }
  if (total < fc.rem) return false;  // uniform: the list's masses fall short of the remainder
  if (cum >= fc.rem && cum - w < fc.rem)  // (one thread: the running mass is nondecreasing)
    set_cut(d, sh, mode, pkey(v), pid(v), static_cast<int32_t>(fc.above_c) + t + 1);
  return true;
}

// The same select over the whole workgroup, for long lists: a radix select on
// the packed values, with 10-bit digits taken just below the highest bit in
// which the remaining entries still differ (bits they all share are skipped:
// the bitwise AND and OR of the chosen digit's entries give the next such
// bit). Each round is one counting pass over the list by every wave and one
// scan of the digits' masses and counts over the workgroup (a digit per
// thread, largest first: in-wave DPP scans, then the waves' totals), with
// three barriers a round; each thread clears its own digit for the next
// round once it has read it, and the round's result alternates between two
// LDS records. Called by every thread; the result is the same in every
// thread. lo and hi: the list's smallest and largest entry.
__device__ __forceinline__ bool block_cut_from_list(const FullCut& fc, int n, uint64_t lo,
                                                    uint64_t hi, const uint32_t* mw, FullSh& sh,
                                                    RowDesc* d, uint32_t mode) {
  constexpr int kDig = 10;
  constexpr int kBins = 1 << kDig;
  static_assert(3 * kBins <= FullSh::kBinCap && kBins <= FullSh::kBinCap, "digit tables");
  uint64_t* bw = sh.hw;               // each digit's mass
  uint64_t* band = sh.hw + kBins;     // the AND of its entries
  uint64_t* bor = sh.hw + 2 * kBins;  // their OR
  uint32_t* bc = sh.hc;               // their count
  static_assert(kBins == kFullThreads, "one digit per thread");
  uint64_t rem = fc.rem;
  int rank = 0;
  uint64_t cutv = hi;
  uint64_t diff = lo ^ hi;  // the bits in which the remaining entries differ
  uint64_t same = hi;       // (their common bits, above the highest of those)
  const int t = static_cast<int>(threadIdx.x);
  const int wv = t / kWave, ln = lane();
  const int dgt = kBins - 1 - t;  // this thread's digit
  bw[dgt] = 0ull;
  band[dgt] = ~0ull;
  bor[dgt] = 0ull;
  bc[dgt] = 0u;
  __syncthreads();
  int par = 0;  // the round's result record
  while (diff != 0ull) {  // uniform
    const int hb = 63 - __clzll(diff);
    const int shift = hb >= kDig - 1 ? hb - (kDig - 1) : 0;
    const uint64_t pmask = hb >= 63 ? 0ull : (~0ull << (hb + 1));
    const uint64_t prefix = same & pmask;
    // (whole waves per step: when every counted entry of a wave falls in one
    // digit, as when the entries share their key, the wave combines them and
    // one lane updates the digit, instead of 64 atomics on one address; the
    // lanes of a wave take entries 67 apart, a permutation of each 1024, so
    // that neighbouring entries, often neighbouring ids, spread over waves)
    static_assert(kFullThreads == 1024, "the entry permutation covers 1024 threads");
#pragma unroll 1
    for (int i0 = 0; i0 < n; i0 += kFullThreads) {
      const int i = i0 + ((t * 67) & (kFullThreads - 1));
      const uint64_t v = i < n ? sh.buf[i] : 0ull;
      const bool in = i < n && (v & pmask) == prefix;
      const int dg = static_cast<int>((v >> shift) & (kBins - 1));
      const uint64_t vb = __ballot(in);
      if (vb == 0ull) continue;  // uniform per wave
      const int first = __ffsll(static_cast<unsigned long long>(vb)) - 1;
      const int d0 = __builtin_amdgcn_readlane(dg, first);
      const uint64_t w = in ? static_cast<uint64_t>(mw[i]) : 0ull;
      if (__ballot(in && dg != d0) == 0ull) {  // uniform per wave
        const uint64_t ws = wave_sum(w);
        const uint64_t wa = wave_reduce(in ? v : ~0ull, [](uint64_t a, uint64_t b) { return a & b; });
        const uint64_t wo = wave_reduce(in ? v : 0ull, [](uint64_t a, uint64_t b) { return a | b; });
        if (lane() == first) {
          atomicAdd(reinterpret_cast<unsigned long long*>(&bw[d0]), static_cast<unsigned long long>(ws));
          atomicAdd(&bc[d0], static_cast<uint32_t>(__popcll(vb)));
          atomicAnd(reinterpret_cast<unsigned long long*>(&band[d0]), static_cast<unsigned long long>(wa));
          atomicOr(reinterpret_cast<unsigned long long*>(&bor[d0]), static_cast<unsigned long long>(wo));
        }
      } else if (in) {
        atomicAdd(reinterpret_cast<unsigned long long*>(&bw[dg]), static_cast<unsigned long long>(w));
        atomicAdd(&bc[dg], 1u);
        atomicAnd(reinterpret_cast<unsigned long long*>(&band[dg]), static_cast<unsigned long long>(v));
        atomicOr(reinterpret_cast<unsigned long long*>(&bor[dg]), static_cast<unsigned long long>(v));
      }
    }
    __syncthreads();
    // the masses (at most 2^31 an entry, 2^13 entries: below 2^44 a digit)
    // scanned as 22-bit halves and the counts, each below 2^32 over a wave
    const uint64_t w = bw[dgt];
    const uint32_t cn = bc[dgt];
    const uint32_t s_lo = wave_scan_incl_u32(static_cast<uint32_t>(w & 0x3fffffull));
    const uint32_t s_hi = wave_scan_incl_u32(static_cast<uint32_t>(w >> 22));
    const uint32_t s_cn = wave_scan_incl_u32(cn);
    const uint64_t w_in = (static_cast<uint64_t>(s_hi) << 22) + s_lo;
    if (ln == kWave - 1) {
      sh.r64[wv] = w_in;
      sh.ri[wv] = static_cast<int32_t>(s_cn);
    }
    if (t == 0) sh.cr32[par][0] = -1;
    __syncthreads();
    uint64_t wb = w_in - w;
    uint32_t cb = s_cn - cn;
    for (int q = 0; q < wv; ++q) {
      wb += sh.r64[q];
      cb += static_cast<uint32_t>(sh.ri[q]);
    }
    if (cn > 0u && wb < rem && rem <= wb + w) {  // one digit of one thread
      sh.cr32[par][0] = dgt;
      sh.cr32[par][1] = static_cast<int32_t>(cb);
      sh.cr32[par][2] = static_cast<int32_t>(cn);
      sh.cr64[par][0] = wb;
      sh.cr64[par][1] = band[dgt];
      sh.cr64[par][2] = bor[dgt];
    }
    bw[dgt] = 0ull;  // (read: cleared for the next round)
    band[dgt] = ~0ull;
    bor[dgt] = 0ull;
    bc[dgt] = 0u;
    __syncthreads();
    const int dg = sh.cr32[par][0];
    const int above = sh.cr32[par][1], cnt = sh.cr32[par][2];
    const uint64_t wabove = sh.cr64[par][0], dand = sh.cr64[par][1], dor = sh.cr64[par][2];
    par ^= 1;
    if (dg < 0) return false;  // the list's masses fall short of the remainder
    rem -= wabove;
    rank += above;
    if (cnt == 1) {
      cutv = dand;
      break;
    }
    diff = dand ^ dor;  // nonzero: the entries are distinct
    same = dand;
  }
  if (threadIdx.x == 0) {
    set_cut(d, sh, mode, pkey(cutv), pid(cutv), static_cast<int32_t>(fc.above_c) + rank + 1);
  }
  return true;
}

constexpr int kRejectThreads = 1024;
static_assert(2 * kRejectThreads >= (VS_MAX_V / kFullSegMin) * kCandM, "two candidates per thread");

// The rejection draw of a full-vocabulary top-p row whose cut (tau, id_cut,
// kept) is in *d: of the row's kCandM best Gumbel candidates (the union of its
// histogram segments' best kCandM holds them), taken in the order (score
// desc, id asc), the first that lies inside the cut is the Gumbel-max draw
// over the kept set: every id that scores higher is one of the candidates
// taken before it, all outside the cut. The row's outputs are then written
// and the row is done; when none of the kCandM lies inside the cut, the row is
// left to the Gumbel pass over its kept set. One workgroup per row, after the
// cut kernel (rows that are not full-vocabulary top-p rows return at once).
template <typename E>
__global__ __launch_bounds__(kRejectThreads) void k_topp_reject(Job j) {
  __shared__ double rd[kRejectThreads / kWave];
  __shared__ int32_t ri[kRejectThreads / kWave];
  __shared__ uint32_t s_key;
  const int row = blockIdx.x;
  RowDesc* d = j.desc + row;
  if (d->mode != kRowFullTopP) return;  // uniform over the block
  const uint32_t tau = d->tau;
  const int32_t idc = d->id_cut;
  const int32_t kept = d->kept;
  const GCand* cand = j.fcand + static_cast<size_t>(row) * j.ntile3 * kCandM;
  const int n = j.fseg * kCandM;
  // this thread's candidates: slots t, t + blockDim.x (n <= 2 blockDim.x:
  // at most 2048 for 2^21 ids of 4096-id segments; fewer segments than
  // compute units otherwise)
  const int t = static_cast<int>(threadIdx.x);
  const int t2 = t + static_cast<int>(blockDim.x);
  double as = -1.0, bsc = -1.0;
  int32_t ai = 0x7fffffff, bi2 = 0x7fffffff;
  uint32_t ak = 0u, bk = 0u;
  if (t < n) {
    const GCand g = cand[t];
    as = g.score;
    ai = g.id;
    ak = g.key;
  }
  if (t2 < n) {
    const GCand g = cand[t2];
    bsc = g.score;
    bi2 = g.id;
    bk = g.key;
  }
  for (int r = 0; r < kCandM; ++r) {
    // this thread's best remaining candidate
    const bool first = as > bsc || (as == bsc && ai < bi2);
    const double hs = first ? as : bsc;
    const int32_t hi = first ? ai : bi2;
    const uint32_t hk = first ? ak : bk;
    const double bs = block_max(hs, rd);
    if (bs < 0.0) return;  // uniform: no candidate left (the Gumbel pass draws)
    const int bi = block_min(hs == bs ? hi : 0x7fffffff, ri);
    const bool mine = hs == bs && hi == bi;
    if (mine) s_key = hk;
    __syncthreads();
    const uint32_t key = s_key;
    __syncthreads();
    if (key > tau || (key == tau && bi <= idc)) {  // uniform: inside the cut
      if (threadIdx.x == 0) {
        j.out_ids[row] = bi;
        if (j.out_kept) j.out_kept[row] = kept;
        if (j.tok_sampled) {
          const float2 ml = j.rlse[row];
          j.out_tok_lp[row] = (logit_at<E>(j, row, bi) - ml.x) - ml.y;
        }
        d->mode = kRowDone;
      }
      return;
    }
    if (mine) {  // taken: outside the cut
      if (first)
        as = -1.0;
      else
        bsc = -1.0;
    }
  }
}

// What the row kernel writes for a row it routes to the full-vocabulary path
// (when it has no top-k log-probs to write): the descriptor's m, status 0,
// the row's (max, log sum) from the segment partials (combined as the row
// kernel combines them: in segment order for a few segments, whose partials
// wave 0's lanes hold from light_load), an empty kept-mask row.
template <int kPer>
__device__ __forceinline__ void full_row_writes(const Job& j, int row, float m, FullSh& sh,
                                                const LightLoads<kPer>& L) {
  if (threadIdx.x == 0) {
    j.desc[row].m = m;
    if (j.out_status) j.out_status[row] = 0;
  }
  if (j.lse) {  // uniform
    const int ntile = j.nseg;
    float M = -kInf, ls = 0.0f;
    if (ntile <= kStageSegs) {  // uniform
      if (threadIdx.x < kWave) {
        for (int t = 0; t < ntile; ++t) M = fmaxf(M, __shfl(L.lp0.m, t));
        for (int t = 0; t < ntile; ++t) {
          const float pm = __shfl(L.lp0.m, t), ps = __shfl(L.lp0.s, t);
          if (M > -kInf && pm > -kInf) ls += ps * __expf(pm - M);
        }
        if (threadIdx.x == 0) j.rlse[row] = make_float2(M, logf(ls));
      }
    } else {
      const LsePart* lrow = j.lpart + static_cast<size_t>(row) * ntile;
      float lm = -kInf;
      for (int t = threadIdx.x; t < ntile; t += blockDim.x) lm = fmaxf(lm, lrow[t].m);
      M = block_max(lm, sh.rf);
      if (M > -kInf) {
        for (int t = threadIdx.x; t < ntile; t += blockDim.x) {
          const LsePart pt = lrow[t];
          if (pt.m > -kInf) ls += pt.s * __expf(pt.m - M);
        }
      }
      ls = block_sum(ls, sh.rf);
      if (threadIdx.x == 0) j.rlse[row] = make_float2(M, logf(ls));
    }
  }
  if (j.out_mask) {  // uniform
    const int mwords = (j.V + 31) / 32;
    uint32_t* mask_row = j.out_mask + static_cast<size_t>(row) * mwords;
    for (int i = threadIdx.x; i < mwords; i += blockDim.x) mask_row[i] = 0u;
  }
}

// The draw of a full-vocabulary row in a call whose gather pass drew (no kept
// mask asked for), finished here, after the cut. The gather pass left one
// record per segment: for a top-p row the best (score desc, id asc) over its
// ids above the cut bucket, for a row without the cut (top_p >= 1) the best
// over all of its members and their count (kFinWhole). A top-p row cut from
// its list adds the list's kept entries, those at or above the cut entry
// (kFinListed: nlist entries, entry t in thread t's v0 for a list of at most
// one entry per thread, all of them in sh.buf otherwise); a top-p row cut from
// the row itself draws over its whole kept set in one pass over the row
// (kFinRow; rare: the cut bucket did not fit the list). Each id's score, the
// skip test and the tie order are those of the Gumbel pass over the kept set
// (an id is skipped only when it provably scores below a best already found),
// so the draw is the same. Then the row's outputs: the sampled id, the kept
// count and, in the fused call, the sampled id's log-probability (from ml,
// thread 0's (max, log-sum-exp) of the row, and the sampled id's logit, which
// at T = 1 is its s). Every wave reads the records (g0: lane l's record l,
// loaded by the caller ahead of the cut), so each holds their best without a
// barrier; the cut comes from LDS (set_cut, published by the caller's
// barrier).
enum : int { kFinWhole = 0, kFinListed = 1, kFinRow = 2 };
template <typename E>
__device__ __forceinline__ void finish_full_draw(const Job& j, int row, float T, uint64_t seed,
                                                  float m, int how, int nlist, uint64_t v0,
                                                  const GPart& g0, float2 ml, FullSh& sh) {
  constexpr int kNT = kFullThreads, kNW = kFullThreads / kWave;
  const E* rowp = static_cast<const E*>(j.logits) + static_cast<int64_t>(row) * j.ld;
  const uint64_t rs = row_stream(seed, row);
  const int t0 = static_cast<int>(threadIdx.x);
  const int ln = lane(), wv = t0 / kWave;
  double best = -1.0;
  int best_id = 0x7fffffff;
  float best_s = 0.0f;
  int kept = 0;
  const auto take = [&](double sc, int id, float sv) {
    if (sc > best || (sc == best && id < best_id)) {
      best = sc;
      best_id = id;
      best_s = sv;
    }
  };
  if (how != kFinRow) {  // uniform
    const GPart* g = j.gpart + static_cast<size_t>(row) * j.ntile3;
    for (int t = ln; t < j.fseg; t += kWave) {
      const GPart p = t == ln ? g0 : g[t];
      if (wv == 0) kept += p.kept;  // (counted once)
      if (p.score >= 0.0) take(p.score, p.id, p.s);
    }
  }
  if (how != kFinWhole) {  // uniform
    const uint64_t cutv = sh.cut_v;
    kept = t0 == 0 ? sh.cut_kept : 0;
    // every thread's bound starts from the records' best
    const double b0 = how == kFinListed ? wave_max(best) : -1.0;
    double lim = b0 > 0.0 ? (1.0 + 0x1p-40) / b0 : __builtin_inf();
    uint64_t skip = skip_below(lim);
    const auto score = [&](float sv, int id) {
      const uint64_t b = random_bits(rs, id);
      if (b < skip) return;  // e <= 1: below the bound
      const double sc = gumbel_score(pinned_exp(sv - m), rs, id);
      if (sc > best || (sc == best && id < best_id)) {
        best = sc;
        best_id = id;
        best_s = sv;
        lim = fmin(lim, (1.0 + 0x1p-40) / best);
        skip = skip_below(lim);
      }
    };
    if (how == kFinListed) {  // uniform
      for (int i = t0; i < nlist; i += kNT) {
        const uint64_t v = i == t0 ? v0 : sh.buf[i];
        if (v >= cutv) score(key2f(pkey(v)), pid(v));  // at or above the cut entry
      }
    } else {
      // key > tau, or key == tau and id <= id_cut
      for (int id = t0; id < j.V; id += kNT) {
        const float x = to_f32(rowp[id]);
        const float sv = T == 1.0f ? x : x / T;
        if (pack(f2key(sv), id) >= cutv) score(sv, id);
      }
    }
  }
  // the block's best and kept count with one barrier: each wave's through
  // slots of its own, read by thread 0
  {
    const double wb = wave_max(best);
    const int wi = wave_min(best == wb ? best_id : 0x7fffffff);
    const int wk = wave_sum(kept);
    const uint64_t own = __ballot(best == wb && best_id == wi);  // the lane holding it
    const float ws = own ? __shfl(best_s, __ffsll(static_cast<unsigned long long>(own)) - 1) : 0.0f;
    if (ln == 0) {
      sh.rd[wv] = wb;
      sh.ri[wv] = wi;
      sh.rk[wv] = wk;
      sh.rf[wv] = ws;
    }
  }
  __syncthreads();
  if (wv != 0) return;  // uniform per wave: wave 0 combines the waves' slots
  const bool slot = ln < kNW;
  const double sd = slot ? sh.rd[ln] : -1.0;
  const int si = slot ? sh.ri[ln] : 0x7fffffff;
  const double bb = wave_max(sd);
  const int bid = wave_min(sd == bb ? si : 0x7fffffff);
  const int bk = wave_sum(slot ? sh.rk[ln] : 0);
  const uint64_t own = __ballot(slot && sd == bb && si == bid);
  const float bs = own ? __shfl(slot ? sh.rf[ln] : 0.0f, __ffsll(static_cast<unsigned long long>(own)) - 1) : 0.0f;
  if (ln == 0) {
    if (bid < 0 || bid >= j.V) {  // unreachable: the row maximum is always kept
      j.out_ids[row] = -1;
      if (j.out_kept) j.out_kept[row] = 0;
      if (j.out_status) j.out_status[row] = VS_ROW_BAD_LOGITS;
      if (j.tok_sampled) j.out_tok_lp[row] = __builtin_nanf("");
      return;
    }
    j.out_ids[row] = bid;
    if (j.out_kept) j.out_kept[row] = bk;
    if (j.tok_sampled) {
      const float x = T == 1.0f ? bs : to_f32(rowp[bid]);
      j.out_tok_lp[row] = (x - ml.x) - ml.y;
    }
  }
}

// The cut kernel, after the full-vocabulary passes: a full-vocabulary row
// (route_row, the histogram and gather passes' own decision) gets its cut,
// which sets the draw's mode for the Gumbel kernels; in a call whose gather
// pass drew (j.fdraw) this kernel then finishes the draw of every such row
// itself (finish_full_draw) and the Gumbel kernels do not run. The row kernel
// is not launched in a call that runs these passes: this kernel does its work,
// a full-vocabulary row's status, log-sum-exp and kept-mask row before the
// cut, and every other row the streaming pass did not finish gets the row
// kernel's work (light_row), in parallel with the cuts.
union RowFullSh {
  FullSh full;
  LightSh light;
};

template <typename E>
__global__ __launch_bounds__(kFullThreads) void k_row_full(Job j) {
  __shared__ RowFullSh sm;
  FullSh& sh = sm.full;
  const int row = blockIdx.x;
  RowDesc* d = j.desc + row;
  // every load the row may need is issued before any is used (the cut record
  // and this thread's list slot are read whatever the row's route, and used
  // only for rows with a cut): their latencies overlap
  const RoutePre rp = route_preload(j, row);
  const FullCut fc = j.fcut[row];
  const uint32_t got = j.fcnt[row];
  const uint64_t* lst = j.flist + static_cast<size_t>(row) * kFullListCap;
  const uint64_t v0 = lst[threadIdx.x];  // (kFullThreads <= kFullListCap)
  // and the row kernel's first loads, for the rows that take its work
  LightLoads<kStageMax / kFullThreads> L;
  light_load(j, row, L);
  const RowRoute rt = route_row(j, row, rp);
  if (!rt.full) {  // uniform over the block
    light_row<E>(j, row, sm.light, L);
    return;
  }
  const RowCfg& c = rt.c;
  const float m = rt.m;
  // the gather pass's record of segment l for lane l of every wave, for the
  // draw at the end (in flight during the cut)
  GPart g0{-1.0, 0x7fffffff, 0};
  if (j.fdraw && lane() < j.fseg)  // (j.fdraw uniform)
    g0 = j.gpart[static_cast<size_t>(row) * j.ntile3 + lane()];
  if (j.lse && j.k_lp > 0) {  // uniform
    // the row kernel's writes for the row, its top-k log-probs included (the
    // same route: the row kernel sends it to the full-vocabulary path)
    light_row<E>(j, row, sm.light, L);
    __syncthreads();  // (the cut reuses the LDS)
  } else {
    full_row_writes(j, row, m, sh, L);
  }
  // the row's (max, log-sum-exp) for the sampled id's log-prob (thread 0
  // wrote it above; in flight during the cut)
  float2 ml = make_float2(0.0f, 0.0f);
  if (j.fdraw && j.tok_sampled && threadIdx.x == 0) ml = j.rlse[row];
  if (c.p < 1.0f) {
    // the gathered list, when it holds the whole cut bucket: a short list
    // (one entry per thread) sorted and cut by the whole workgroup, a longer
    // one loaded with its masses into LDS for the workgroup's radix select
    const bool listed = fc.bucket >= 0 && got == fc.count && got > 0u &&
                        got <= static_cast<uint32_t>(FullSh::kBufCap);  // uniform
    int fin = kFinRow;  // the draw's source once the cut is known (j.fdraw)
    if (listed) {
      __shared__ __align__(16) uint32_t mw[kFullListCap];
      // the draw then comes from the list and the gather pass's bests when
      // the gather pass drew over the ids above the bucket
      const uint32_t mode = j.fdraw ? kRowFullListed : kRowFullTopP;
      const int n = static_cast<int>(got);
      const FullTerms ft{m, c.mp};
      if (n <= kSortCutMax) {  // uniform
        const uint64_t v = static_cast<int>(threadIdx.x) < n ? v0 : 0ull;
        if (sort_cut_from_list(fc, n, v, ft, sh.buf, reinterpret_cast<uint64_t*>(mw), sh, d, mode))
          fin = kFinListed;  // uniform
      } else {
        // (kLB entries per thread in flight at once; the list's least and
        // largest entries through per-wave slots and one barrier, which
        // also publishes buf and mw)
        constexpr int kLB = 4;
        const int t = static_cast<int>(threadIdx.x);
        uint64_t lo = ~0ull, hi = 0ull;
        for (int i0 = 0; i0 < n; i0 += kLB * kFullThreads) {
          uint64_t vb[kLB];
#pragma unroll
          for (int k = 0; k < kLB; ++k) {
            const int i = i0 + k * kFullThreads + t;
            vb[k] = (i0 == 0 && k == 0) ? v0 : (i < n ? lst[i] : 0ull);
          }
#pragma unroll
          for (int k = 0; k < kLB; ++k) {
            const int i = i0 + k * kFullThreads + t;
            if (i < n) {
              uint64_t w;
              int b;
              if (!ft.mass(key2f(pkey(vb[k])), &w, &b)) w = 0;
              sh.buf[i] = vb[k];
              mw[i] = static_cast<uint32_t>(w);
              lo = vb[k] < lo ? vb[k] : lo;
              hi = vb[k] > hi ? vb[k] : hi;
            }
          }
        }
        lo = wave_min(lo);
        hi = wave_max(hi);
        if (lane() == 0) {
          sh.r64[t / kWave] = lo;
          sh.r64b[t / kWave] = hi;
        }
        __syncthreads();
        for (int w = 0; w < kFullThreads / kWave; ++w) {
          lo = sh.r64[w] < lo ? sh.r64[w] : lo;
          hi = sh.r64b[w] > hi ? sh.r64b[w] : hi;
        }
        if (block_cut_from_list(fc, n, lo, hi, mw, sh, d, mode)) fin = kFinListed;  // uniform
      }
      __syncthreads();  // (else, a list short of the remainder, the full path)
    }
    if (fin == kFinRow) {  // uniform
      const E* rowp = static_cast<const E*>(j.logits) + static_cast<int64_t>(row) * j.ld;
      full_topp_cut(rowp, j.V, j.aligned, c.T, c.p, c.mp, m, sh, d);
      __syncthreads();  // (the cut's record)
    }
    if (j.fdraw)  // uniform
      finish_full_draw<E>(j, row, c.T, c.seed, m, fin, static_cast<int>(got), v0, g0, ml, sh);
  } else {
    if (threadIdx.x == 0) d->mode = (c.mp > 0.0f) ? kRowFullMinP : kRowFullNone;
    if (j.fdraw)  // uniform
      finish_full_draw<E>(j, row, c.T, c.seed, m, kFinWhole, 0, 0ull, g0, ml, sh);
  }
}

}  // namespace

hipError_t launch_row_light(const Job& j, hipStream_t st) {
  if (j.dt == VS_F32)
    hipLaunchKernelGGL(k_row_light<float>, dim3(j.B), dim3(kLightThreads), 0, st, j);
  else
    hipLaunchKernelGGL(k_row_light<uint16_t>, dim3(j.B), dim3(kLightThreads), 0, st, j);
  return hipGetLastError();
}

hipError_t launch_row_full(const Job& j, hipStream_t st) {
  if (j.dt == VS_F32)
    hipLaunchKernelGGL(k_row_full<float>, dim3(j.B), dim3(kFullThreads), 0, st, j);
  else
    hipLaunchKernelGGL(k_row_full<uint16_t>, dim3(j.B), dim3(kFullThreads), 0, st, j);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !j.topp_reject) return e;
  if (j.dt == VS_F32)
    hipLaunchKernelGGL(k_topp_reject<float>, dim3(j.B), dim3(kRejectThreads), 0, st, j);
  else
    hipLaunchKernelGGL(k_topp_reject<uint16_t>, dim3(j.B), dim3(kRejectThreads), 0, st, j);
  return hipGetLastError();
}

}  // namespace vsk
