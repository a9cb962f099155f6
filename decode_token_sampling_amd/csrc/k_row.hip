// K2: one 1024-thread workgroup per row, after the streaming pass.
//
//  - greedy rows: the lowest id of the row maximum, from the tiles' argmaxes;
//  - top-k rows (k <= 64): merge the tiles' sorted candidate lists, then
//    truncate (min-p, top-p over the survivors) and draw among at most k ids;
//  - larger k, or a tile whose candidates overflowed: an exact radix select of
//    the k-th key over the whole row (three digit passes), a pass that finds the
//    last kept id inside a tie group, and a gather of exactly k ids;
//  - full-vocabulary rows: the row maximum m of s = x / T, and for top-p < 1 the
//    cut: a histogram of fixed-point masses over buckets of (s - m) (128 per
//    unit, monotone in s), the bucket where the cumulative mass reaches
//    top_p * total, then the exact cut inside that bucket (gathered and sorted
//    in LDS, or, if it holds more than 8192 ids, a mass-weighted radix select).
//    The Gumbel kernels then draw over the kept set.
// The log-softmax row kernel (vs_logprobs) shares the candidate merge and the
// slow top-k path.
#include "vs_device.h"
#include "vs_kernels.h"

namespace vsk {
namespace {

constexpr int kRowThreads = 1024;
constexpr int kBufCap = 8192;
constexpr int kBuckets = 4096;
constexpr float kBucketsPerUnit = 128.0f;

struct RowShared {
  uint64_t buf[kBufCap];   // gathered candidates (packed key, id)
  uint64_t hw[kBuckets];   // histogram weights
  uint32_t hc[kBuckets];   // histogram counts
  uint64_t r64[16];
  double rd[16];
  int32_t ri[16];
  int n;
  uint64_t b64[4];
  int32_t b32[4];
};

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
__device__ __forceinline__ int hist_find_desc(RowShared& sh, int nb, uint64_t rem,
                                              uint64_t* above_w, uint64_t* above_c) {
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
template <typename E, typename Pick>
__device__ void radix_select(const E* __restrict__ rowp, int V, bool aligned, float T, uint64_t rem,
                             Pick pick, RowShared& sh, uint32_t* tau, uint64_t* w_above,
                             uint64_t* c_above, uint64_t* w_tau) {
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
template <typename E, typename Pick>
__device__ int32_t tie_cut(const E* __restrict__ rowp, int V, float T, uint32_t tau, uint64_t need,
                           Pick pick, RowShared& sh) {
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

// Sort the first n entries of sh.buf (larger first); pads to a power of two.
__device__ __forceinline__ void sort_buf(RowShared& sh, int n) {
  const int np = next_pow2(n < 2 ? 2 : n);
  for (int i = n + threadIdx.x; i < np; i += blockDim.x) sh.buf[i] = 0ull;
  __syncthreads();
  block_sort_desc(sh.buf, np);
}

// Merge the tiles' sorted top-k lists of one row into sh.buf, sorted; returns
// min(k, total candidates), or -1 when a tile overflowed or too many survive.
// Only entries >= P* can be in the row's top k, where P* is the largest k-th
// entry of a full tile list (that tile alone has k entries >= P*).
__device__ int merge_tiles(const uint32_t* __restrict__ mrow, const uint64_t* __restrict__ crow,
                           int ntile, int k, RowShared& sh) {
  uint64_t pl = 0;
  int ovf = 0;
  for (int t = threadIdx.x; t < ntile; t += blockDim.x) {
    const uint32_t m = mrow[t];
    if (m & kMetaOverflow) ovf = 1;
    if (static_cast<int>(m & kMetaCountMask) == k) {
      const uint64_t v = crow[static_cast<size_t>(t) * kFastK + k - 1];
      pl = v > pl ? v : pl;
    }
  }
  ovf = block_max(ovf, sh.ri);
  if (ovf) return -1;
  const uint64_t pstar = block_max(pl, sh.r64);
  if (threadIdx.x == 0) sh.n = 0;
  __syncthreads();
  for (int f = threadIdx.x; f < ntile * k; f += blockDim.x) {
    const int t = f / k, i = f - t * k;
    if (i < static_cast<int>(mrow[t] & kMetaCountMask)) {
      const uint64_t v = crow[static_cast<size_t>(t) * kFastK + i];
      if (v >= pstar) {
        const int pos = atomicAdd(&sh.n, 1);
        if (pos < kBufCap) sh.buf[pos] = v;
      }
    }
  }
  __syncthreads();
  const int n = sh.n;
  __syncthreads();
  if (n > kBufCap) return -1;
  sort_buf(sh, n);
  return n < k ? n : k;
}

// Exact top-k of the row by radix select; leaves the k entries sorted in sh.buf.
template <typename E>
__device__ int slow_topk(const E* __restrict__ rowp, int V, bool aligned, float T, int k,
                         RowShared& sh) {
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
      if (pos < kBufCap) sh.buf[pos] = pack(key, j);
    }
  });
  __syncthreads();
  int n = sh.n;
  __syncthreads();
  if (n > k) n = k;  // cannot happen: exactly k ids pass
  sort_buf(sh, n);
  return n;
}

// Truncate and draw over the n (<= blockDim) sorted candidates in sh.buf.
// Returns the status (0, or VS_ROW_BAD_PARAM when x / T overflowed).
__device__ int draw_sorted(RowShared& sh, int n, const RowCfg& c, int row, int32_t* id_out,
                           int32_t* kept_out, uint32_t* mask_row) {
  const int i = threadIdx.x;
  const uint64_t top = sh.buf[0];
  if (pkey(top) == kKeyPosInf) return VS_ROW_BAD_PARAM;
  const float m = key2f(pkey(top));
  const bool has = i < n;
  const uint64_t P = has ? sh.buf[i] : 0ull;
  const float e = has ? pinned_exp(key2f(pkey(P)) - m) : 0.0f;
  const bool in_s = has && (e >= c.mp);  // a prefix of the order: e is monotone in s
  bool kept = in_s;
  if (c.p < 1.0f) {
    const uint64_t W = in_s ? mass_of(e) : 0ull;
    uint64_t tw;
    const uint64_t cum = block_scan_incl(W, sh.r64, &tw);
    const double thr = static_cast<double>(c.p) * static_cast<double>(tw);
    const int first = (in_s && static_cast<double>(cum) >= thr) ? i : 0x7fffffff;
    const int cut = block_min(first, sh.ri);
    kept = in_s && i <= cut;
  }
  const int nk = block_sum(kept ? 1 : 0, sh.ri);
  const uint64_t rs = row_stream(c.seed, row);
  const int id = has ? pid(P) : 0x7fffffff;
  const double score = kept ? gumbel_score(e, rs, id) : -1.0;
  const double best = block_max(score, sh.rd);
  const int win = block_min((kept && score == best) ? id : 0x7fffffff, sh.ri);
  if (kept && mask_row) atomicOr(&mask_row[id >> 5], 1u << (id & 31));
  *id_out = win;
  *kept_out = nk;
  return 0;
}

// Per-element quantities of a full-vocabulary top-p row.
struct FullTerms {
  float m, T, mp;
  __device__ __forceinline__ bool mass(float s, uint64_t* w, int* bucket) const {
    const float t = s - m;
    const float e = pinned_exp(t);
    if (!(e >= mp)) return false;
    const uint64_t W = mass_of(e);
    if (W == 0) return false;
    *w = W;
    int b = static_cast<int>(-t * kBucketsPerUnit);
    *bucket = b < kBuckets - 1 ? b : kBuckets - 1;
    return true;
  }
};

template <typename E>
__device__ void full_topp_cut(const E* __restrict__ rowp, int V, bool aligned, const RowCfg& c,
                              float m, RowShared& sh, RowDesc* d) {
  const FullTerms ft{m, c.T, c.mp};
  for (int i = threadIdx.x; i < kBuckets; i += blockDim.x) {
    sh.hw[i] = 0;
    sh.hc[i] = 0;
  }
  __syncthreads();
  row_visit(rowp, V, aligned, [&](int, float x) {
    uint64_t w;
    int b;
    if (ft.mass(scaled(x, c.T), &w, &b)) {
      atomicAdd(reinterpret_cast<unsigned long long*>(&sh.hw[b]), static_cast<unsigned long long>(w));
      atomicAdd(&sh.hc[b], 1u);
    }
  });
  __syncthreads();
  uint64_t lt = 0;
  for (int i = threadIdx.x; i < kBuckets; i += blockDim.x) lt += sh.hw[i];
  const uint64_t total = block_sum(lt, sh.r64);
  // The kept prefix is the shortest whose mass reaches thr; masses are integers,
  // so "cum >= thr" is "cum >= ceil(thr)".
  const double thr = static_cast<double>(c.p) * static_cast<double>(total);
  const uint64_t target = static_cast<uint64_t>(ceil(thr)) > 0 ? static_cast<uint64_t>(ceil(thr)) : 1;
  // Bucket 0 holds the largest s: scan buckets upwards == values downwards.
  // hist_find_desc scans bins from the top index down, so present the buckets
  // reversed by swapping the arrays in place.
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
  if (nb <= static_cast<uint32_t>(kBufCap)) {
    if (threadIdx.x == 0) sh.n = 0;
    __syncthreads();
    row_visit(rowp, V, aligned, [&](int j, float x) {
      const float s = scaled(x, c.T);
      uint64_t w;
      int b;
      if (ft.mass(s, &w, &b) && b == bstar) {
        const int pos = atomicAdd(&sh.n, 1);
        if (pos < kBufCap) sh.buf[pos] = pack(f2key(s), j);
      }
    });
    __syncthreads();
    const int n = sh.n < kBufCap ? sh.n : kBufCap;
    __syncthreads();
    sort_buf(sh, n);
    // Cumulative mass inside the bucket, in order; the cut is the first index
    // where it reaches rem.
    constexpr int PER = kBufCap / kRowThreads;
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
    radix_select(rowp, V, aligned, c.T, rem, in_bucket, sh, &tau, &wa, &ca, &wt);
    const uint64_t r2 = rem - wa;
    const uint64_t need = wt ? (r2 + wt - 1) / wt : 1;
    idc = tie_cut(rowp, V, c.T, tau, need, in_bucket, sh);
    kept = static_cast<int32_t>(ac + ca + need);
  }
  if (threadIdx.x == 0) {
    d->mode = kFullTopP;
    d->m = m;
    d->tau = tau;
    d->id_cut = idc;
    d->kept = kept;
  }
}

template <typename E>
__global__ __launch_bounds__(kRowThreads) void k_row(
    const E* __restrict__ logits, int B, int V, int64_t ld, bool aligned,
    const float* __restrict__ temperature, const int32_t* __restrict__ top_k,
    const float* __restrict__ top_p, const float* __restrict__ min_p,
    const uint64_t* __restrict__ seeds, uint32_t hints, int ntile,
    const uint32_t* __restrict__ meta, const uint64_t* __restrict__ cand,
    RowDesc* __restrict__ desc, int32_t* __restrict__ out_ids, int32_t* __restrict__ out_kept,
    uint32_t* __restrict__ out_mask, int32_t* __restrict__ out_status) {
  __shared__ RowShared sh;
  const int row = blockIdx.x;
  const RowCfg c = load_cfg(row, V, temperature, top_k, top_p, min_p, seeds);
  const uint32_t* mrow = meta + static_cast<size_t>(row) * ntile;
  const uint64_t* crow = cand + static_cast<size_t>(row) * ntile * kFastK;
  const E* rowp = logits + static_cast<int64_t>(row) * ld;
  const int mwords = (V + 31) / 32;
  uint32_t* mask_row = out_mask ? out_mask + static_cast<size_t>(row) * mwords : nullptr;

  int bad = 0, finite = 0;
  uint64_t top = 0;
  for (int t = threadIdx.x; t < ntile; t += blockDim.x) {
    const uint32_t m = mrow[t];
    if (m & kMetaBadLogits) bad = 1;
    if (m & kMetaHasFinite) finite = 1;
    if (m & kMetaCountMask) {
      const uint64_t v = crow[static_cast<size_t>(t) * kFastK];
      top = v > top ? v : top;
    }
  }
  bad = block_max(bad, sh.ri);
  finite = block_max(finite, sh.ri);
  top = block_max(top, sh.r64);
  if (mask_row) {
    for (int i = threadIdx.x; i < mwords; i += blockDim.x) mask_row[i] = 0u;
    __syncthreads();
  }

  int status = c.status;
  if (bad || !finite) status |= VS_ROW_BAD_LOGITS;
  if (status == 0) {
    if ((hints & VS_HINT_ALL_GREEDY) && c.mode != kModeGreedy) status = VS_ROW_HINT_VIOLATED;
    if ((hints & VS_HINT_NO_FULLVOCAB) && c.mode == kModeFull) status = VS_ROW_HINT_VIOLATED;
  }
  int32_t id = -1, kept = 0;
  bool full = false;
  RowDesc* d = desc + row;
  if (status == 0) {
    if (c.mode == kModeGreedy) {
      id = pid(top);
      kept = 1;
      if (mask_row && threadIdx.x == 0) atomicOr(&mask_row[id >> 5], 1u << (id & 31));
    } else if (c.mode == kModeKFast || c.mode == kModeKSlow) {
      int n = (c.mode == kModeKFast) ? merge_tiles(mrow, crow, ntile, c.k, sh) : -1;
      if (n < 0) n = slow_topk(rowp, V, aligned, c.T, c.k, sh);
      status = draw_sorted(sh, n, c, row, &id, &kept, mask_row);
    } else {  // full vocabulary
      const float m = scaled(key2f(pkey(top)), c.T);
      if (m == kInf) {
        status = VS_ROW_BAD_PARAM;
      } else {
        full = true;
        if (c.p < 1.0f) {
          full_topp_cut(rowp, V, aligned, c, m, sh, d);
        } else if (threadIdx.x == 0) {
          d->mode = (c.mp > 0.0f) ? kFullMinP : kFullNone;
          d->m = m;
          d->tau = 0;
          d->id_cut = 0;
          d->kept = 0;
        }
      }
    }
  }
  if (threadIdx.x == 0) {
    if (!full) d->mode = kFullSkip;
    if (status) {
      id = -1;
      kept = 0;
    }
    if (!full) {
      out_ids[row] = id;
      if (out_kept) out_kept[row] = kept;
    }
    if (out_status) out_status[row] = status;
  }
  if (status && mask_row) {  // a row that failed after setting bits reports an empty set
    __syncthreads();
    for (int i = threadIdx.x; i < mwords; i += blockDim.x) mask_row[i] = 0u;
  }
}

template <typename E>
__global__ __launch_bounds__(kRowThreads) void k_lse_row(
    const E* __restrict__ logits, int B, int V, int64_t ld, bool aligned, int k,
    const int32_t* __restrict__ token_ids, int ntile, const uint32_t* __restrict__ meta,
    const uint64_t* __restrict__ cand, const LsePart* __restrict__ lpart,
    float2* __restrict__ rlse, float* __restrict__ out_tok, int32_t* __restrict__ out_ids,
    float* __restrict__ out_lp, int32_t* __restrict__ out_status) {
  __shared__ RowShared sh;
  const int row = blockIdx.x;
  const uint32_t* mrow = meta + static_cast<size_t>(row) * ntile;
  const uint64_t* crow = cand + static_cast<size_t>(row) * ntile * kFastK;
  const LsePart* lrow = lpart + static_cast<size_t>(row) * ntile;
  const E* rowp = logits + static_cast<int64_t>(row) * ld;

  int bad = 0;
  float M = -kInf;
  for (int t = threadIdx.x; t < ntile; t += blockDim.x) {
    if (mrow[t] & kMetaBadLogits) bad = 1;
    M = fmaxf(M, lrow[t].m);
  }
  bad = block_max(bad, sh.ri);
  M = block_max(M, reinterpret_cast<float*>(sh.rd));
  float S = 0.0f;
  if (M != -kInf) {
    for (int t = threadIdx.x; t < ntile; t += blockDim.x) {
      const LsePart p = lrow[t];
      if (p.m != -kInf) S += p.s * __expf(p.m - M);
    }
  }
  S = block_sum(S, reinterpret_cast<float*>(sh.rd));
  int status = (bad || M == -kInf) ? VS_ROW_BAD_LOGITS : 0;
  const float nanv = __builtin_nanf("");
  const float logS = logf(S);
  if (threadIdx.x == 0) {
    rlse[row] = status ? make_float2(nanv, nanv) : make_float2(M, logS);
  }
  if (token_ids) {
    const int tok = token_ids[row];
    const bool badtok = tok < 0 || tok >= V;
    if (badtok) status |= VS_ROW_BAD_TOKEN_ID;
    if (threadIdx.x == 0)
      out_tok[row] = (status & VS_ROW_BAD_LOGITS) || badtok ? nanv : (to_f32(rowp[tok]) - M) - logS;
  }
  if (k > 0) {
    int32_t* ids = out_ids + static_cast<size_t>(row) * k;
    float* lps = out_lp + static_cast<size_t>(row) * k;
    if (status & VS_ROW_BAD_LOGITS) {
      for (int i = threadIdx.x; i < k; i += blockDim.x) {
        ids[i] = -1;
        lps[i] = nanv;
      }
    } else {
      int n = merge_tiles(mrow, crow, ntile, k, sh);
      if (n < 0) n = slow_topk(rowp, V, aligned, 1.0f, k, sh);
      for (int i = threadIdx.x; i < k; i += blockDim.x) {
        if (i < n) {
          const uint64_t P = sh.buf[i];
          ids[i] = pid(P);
          lps[i] = (key2f(pkey(P)) - M) - logS;
        } else {
          ids[i] = -1;
          lps[i] = nanv;
        }
      }
    }
  }
  if (threadIdx.x == 0 && out_status) out_status[row] = status;
}

}  // namespace

hipError_t launch_row(const SampleArgs& a, const WsLayout& L, char* ws, hipStream_t st) {
  const auto* meta = reinterpret_cast<const uint32_t*>(ws + L.meta);
  const auto* cand = reinterpret_cast<const uint64_t*>(ws + L.cand);
  auto* desc = reinterpret_cast<RowDesc*>(ws + L.desc);
  if (a.dt == VS_F32)
    hipLaunchKernelGGL(k_row<float>, dim3(a.B), dim3(kRowThreads), 0, st,
                       static_cast<const float*>(a.logits), a.B, a.V, a.ld, a.aligned, a.temperature,
                       a.top_k, a.top_p, a.min_p, a.seeds, a.hints, L.ntile1, meta, cand, desc,
                       a.out_ids, a.out_kept, a.out_mask, a.out_status);
  else
    hipLaunchKernelGGL(k_row<uint16_t>, dim3(a.B), dim3(kRowThreads), 0, st,
                       static_cast<const uint16_t*>(a.logits), a.B, a.V, a.ld, a.aligned,
                       a.temperature, a.top_k, a.top_p, a.min_p, a.seeds, a.hints, L.ntile1, meta,
                       cand, desc, a.out_ids, a.out_kept, a.out_mask, a.out_status);
  return hipGetLastError();
}

hipError_t launch_lse_row(const LogprobArgs& a, const WsLayout& L, char* ws, hipStream_t st) {
  const auto* meta = reinterpret_cast<const uint32_t*>(ws + L.meta);
  const auto* cand = reinterpret_cast<const uint64_t*>(ws + L.cand);
  const auto* lp = reinterpret_cast<const LsePart*>(ws + L.lpart);
  auto* rl = reinterpret_cast<float2*>(ws + L.rlse);
  if (a.dt == VS_F32)
    hipLaunchKernelGGL(k_lse_row<float>, dim3(a.B), dim3(kRowThreads), 0, st,
                       static_cast<const float*>(a.logits), a.B, a.V, a.ld, a.aligned, a.k,
                       a.token_ids, L.ntile1, meta, cand, lp, rl, a.out_token_lp, a.out_topk_ids,
                       a.out_topk_lp, a.out_status);
  else
    hipLaunchKernelGGL(k_lse_row<uint16_t>, dim3(a.B), dim3(kRowThreads), 0, st,
                       static_cast<const uint16_t*>(a.logits), a.B, a.V, a.ld, a.aligned, a.k,
                       a.token_ids, L.ntile1, meta, cand, lp, rl, a.out_token_lp, a.out_topk_ids,
                       a.out_topk_lp, a.out_status);
  return hipGetLastError();
}

}  // namespace vsk
