// K1: the single streaming pass over the logits.
//
// Each wave owns a tile of 4096 consecutive logits of one row (64 lanes x 64
// values held in registers after 16-byte loads). Per tile it writes:
//  - a validity flag (a NaN or +inf logit makes the row invalid);
//  - for top-k rows (0 < k <= 64): the tile's k best (s desc, id asc) as packed
//    (key, id), where s = x / T;
//  - for every other row: the tile's best x with its lowest id (greedy argmax,
//    and the row maximum the full-vocabulary and slow paths need);
//  - in log-sum-exp mode (vs_logprobs): the tile max and sum of exp(x - max),
//    plus the tile's top-k of x.
// The top-k of a tile uses a threshold: tau = k-th largest of the 64 lane
// maxima (of the 128 lane top-2 values when k > 32). At least k values are
// >= tau, so the tile's top-k is among them; a ballot compacts those few
// candidates into LDS, where one wave sorts them. A tile whose candidates do
// not fit (heavy ties at the threshold) is flagged, and the row-level kernel
// then selects over the whole row instead.
#include "vs_device.h"
#include "vs_kernels.h"

namespace vsk {
namespace {

constexpr int kVals = 64;            // values per lane
constexpr int kCap = 128;            // candidate slots per wave

template <typename E>
__device__ __forceinline__ int elem_index(int tile_base, int q) {
  constexpr int EPV = Epv<E>::n;
  return tile_base + ((q / EPV) * kWave + lane()) * EPV + (q % EPV);
}

template <typename E>
__device__ __forceinline__ void load_tile(const E* __restrict__ rowp, int tile_base, int V,
                                          bool vec, float (&v)[kVals]) {
  constexpr int EPV = Epv<E>::n;
  constexpr int NV = kVals / EPV;
  const int l = lane();
  if (vec) {
    uint4 raw[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i)
      raw[i] = *reinterpret_cast<const uint4*>(rowp + tile_base + (i * kWave + l) * EPV);
#pragma unroll
    for (int i = 0; i < NV; ++i) unpack16(raw[i], &v[i * EPV], rowp);
  } else {
#pragma unroll
    for (int q = 0; q < kVals; ++q) {
      const int idx = elem_index<E>(tile_base, q);
      v[q] = (idx < V) ? to_f32(rowp[idx]) : -kInf;
    }
  }
}

// k-th largest (1-based, k <= 64) of the union of two lane-sorted descending
// sequences a and b: max over i in [0,k] of min(a[i-1], b[k-i-1]).
__device__ __forceinline__ uint32_t kth_of_union(uint32_t sa, uint32_t sb, int k) {
  const int i = lane();
  const uint32_t a_prev = __shfl(sa, i > 0 ? i - 1 : 0);
  const int bj = k - i - 1;
  const uint32_t b_at = __shfl(sb, bj >= 0 ? (bj < kWave ? bj : kWave - 1) : 0);
  uint32_t ai = (i == 0) ? 0xffffffffu : a_prev;
  uint32_t bi = (bj < 0) ? 0xffffffffu : b_at;
  uint32_t c = (i <= k) ? (ai < bi ? ai : bi) : 0u;
  c = wave_max(c);
  if (k == kWave) {  // the i = 64 term: a[63]
    const uint32_t a63 = __shfl(sa, kWave - 1);
    c = (a63 > c) ? a63 : c;
  }
  return c;
}

// Returns the tile's candidate count (<= k) written to out, or -1 on overflow.
// v: the lane's values; k in [2, 64]; T > 0 the row temperature.
template <typename E>
__device__ __forceinline__ int tile_topk(const float (&v)[kVals], float lmax, int tile_base,
                                         int V, bool vec, int k, float T,
                                         uint64_t* __restrict__ sb, uint64_t* __restrict__ out) {
  const int l = lane();
  uint32_t tau_key;
  if (k <= 32) {
    const uint32_t s = wave_sort_desc(f2key(lmax));
    tau_key = __shfl(s, k - 1);
  } else {
    float a = -kInf, b = -kInf;
#pragma unroll
    for (int q = 0; q < kVals; ++q) {
      b = fmaxf(b, fminf(a, v[q]));
      a = fmaxf(a, v[q]);
    }
    tau_key = kth_of_union(wave_sort_desc(f2key(a)), wave_sort_desc(f2key(b)), k);
  }
  const float tau = key2f(tau_key);
  const bool t1 = (T == 1.0f);
  float pre = tau;           // prefilter on x
  uint32_t sig_key = tau_key;  // exact filter on the key of s = x / T
  if (!t1) {
    sig_key = f2key(tau / T);
    // Any x with fl(x/T) >= fl(tau/T) satisfies x >= tau - 2^-22 |tau| - T 2^-149;
    // the bound below is looser still and rounded down.
    const double lb = static_cast<double>(tau) - __builtin_ldexp(fabs(static_cast<double>(tau)), -21) -
                      static_cast<double>(T) * 0x1p-148;
    pre = static_cast<float>(lb);
    if (static_cast<double>(pre) > lb) pre = nextafterf(pre, -kInf);
  }

  int n = 0;
#pragma unroll
  for (int q = 0; q < kVals; ++q) {
    const int idx = elem_index<E>(tile_base, q);
    bool pred = (v[q] >= pre) && (vec || idx < V);
    uint64_t bal = __ballot(pred);
    if (bal) {
      uint32_t key = f2key(v[q]);
      if (!t1) {
        if (pred) {
          key = f2key(v[q] / T);
          pred = key >= sig_key;
        }
        bal = __ballot(pred);
      }
      if (pred) {
        const int pos = n + lanes_below(bal);
        if (pos < kCap) sb[pos] = pack(key, idx);
      }
      n += __popcll(bal);
    }
  }
  wave_lds_sync();
  if (n > kCap) return -1;
  uint64_t a = (l < n) ? sb[l] : 0ull;
  a = wave_sort_desc(a);
  if (n > kWave) {
    uint64_t b = (l + kWave < n) ? sb[l + kWave] : 0ull;
    b = wave_sort_desc(b);
    a = wave_merge_top_desc(a, b);
  }
  const int cnt = n < k ? n : k;
  if (l < cnt) out[l] = a;
  wave_lds_sync();
  return cnt;
}

template <typename E, bool kLse>
__global__ __launch_bounds__(256) void k_select(
    const E* __restrict__ logits, int B, int V, int64_t ld, bool aligned,
    const float* __restrict__ temperature, const int32_t* __restrict__ top_k,
    const float* __restrict__ top_p, const float* __restrict__ min_p, int lp_k, uint32_t hints,
    int ntile, int wpr, uint32_t* __restrict__ meta, uint64_t* __restrict__ cand,
    LsePart* __restrict__ lpart) {
  __shared__ uint64_t sbuf[kSelWaves][kCap];
  int row, wg;
  if (!xcd_row_tile(blockIdx.x, B, wpr, &row, &wg)) return;
  const int w = threadIdx.x / kWave;
  const int tile = wg * kSelWaves + w;
  if (tile >= ntile) return;  // no block-level barrier below this point
  const int l = lane();

  int kk;
  float T = 1.0f;
  if (kLse) {
    kk = lp_k;
  } else {
    const RowCfg c = load_cfg(row, V, temperature, top_k, top_p, min_p, nullptr);
    const bool fast = (c.mode == kModeKFast) && !(hints & VS_HINT_ALL_GREEDY);
    kk = fast ? c.k : 1;
    if (fast) T = c.T;
  }

  const E* rowp = logits + static_cast<int64_t>(row) * ld;
  const int tile_base = tile * kSelTile;
  const bool vec = aligned && (tile_base + kSelTile <= V);
  float v[kVals];
  load_tile<E>(rowp, tile_base, V, vec, v);

  float lmax = -kInf;
  bool bad = false;
#pragma unroll
  for (int q = 0; q < kVals; ++q) {
    lmax = fmaxf(lmax, v[q]);
    bad = bad || __builtin_amdgcn_classf(v[q], 0x203);  // signalling/quiet NaN or +inf
  }
  uint32_t flags = (__ballot(bad) != 0ull) ? kMetaBadLogits : 0u;
  if (__ballot(lmax > -kInf) != 0ull) flags |= kMetaHasFinite;
  const size_t slot = static_cast<size_t>(row) * ntile + tile;
  uint64_t* out = cand + slot * kFastK;

  if (kLse) {
    const float M = wave_max(lmax);
    float s = 0.0f;
    if (M != -kInf) {
#pragma unroll
      for (int q = 0; q < kVals; ++q) s += __expf(v[q] - M);
    }
    s = wave_sum(s);
    if (l == 0) lpart[slot] = LsePart{M, s};
  }

  int cnt = 0;
  if (kk == 1) {
    const float M = wave_max(lmax);
    int best = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < kVals; ++q) {
      const int idx = elem_index<E>(tile_base, q);
      if (v[q] == M && (vec || idx < V)) best = idx < best ? idx : best;
    }
    best = wave_min(best);
    if (best != 0x7fffffff) {
      cnt = 1;
      if (l == 0) out[0] = pack(f2key(M), best);
    }
  } else if (kk > 1) {
    cnt = tile_topk<E>(v, lmax, tile_base, V, vec, kk, T, sbuf[w], out);
    if (cnt < 0) {
      flags |= kMetaOverflow;
      cnt = 0;
    }
  }
  if (l == 0) meta[slot] = static_cast<uint32_t>(cnt) | flags;
}

template <typename E, bool kLse>
hipError_t launch_select_t(const void* logits, int B, int V, int64_t ld, bool aligned,
                           const float* T, const int32_t* k, const float* p, const float* mp,
                           int lp_k, uint32_t hints, const WsLayout& L, char* ws, hipStream_t st) {
  const int grid = xcd_grid(B, L.wpr1);
  hipLaunchKernelGGL((k_select<E, kLse>), dim3(grid), dim3(256), 0, st,
                     static_cast<const E*>(logits), B, V, ld, aligned, T, k, p, mp, lp_k, hints,
                     L.ntile1, L.wpr1, reinterpret_cast<uint32_t*>(ws + L.meta),
                     reinterpret_cast<uint64_t*>(ws + L.cand),
                     reinterpret_cast<LsePart*>(ws + L.lpart));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const SampleArgs& a, const WsLayout& L, char* ws, hipStream_t st) {
  if (a.dt == VS_F32)
    return launch_select_t<float, false>(a.logits, a.B, a.V, a.ld, a.aligned, a.temperature,
                                         a.top_k, a.top_p, a.min_p, 0, a.hints, L, ws, st);
  return launch_select_t<uint16_t, false>(a.logits, a.B, a.V, a.ld, a.aligned, a.temperature,
                                          a.top_k, a.top_p, a.min_p, 0, a.hints, L, ws, st);
}

hipError_t launch_select_lse(const LogprobArgs& a, const WsLayout& L, char* ws, hipStream_t st) {
  if (a.dt == VS_F32)
    return launch_select_t<float, true>(a.logits, a.B, a.V, a.ld, a.aligned, nullptr, nullptr,
                                        nullptr, nullptr, a.k, 0u, L, ws, st);
  return launch_select_t<uint16_t, true>(a.logits, a.B, a.V, a.ld, a.aligned, nullptr, nullptr,
                                         nullptr, nullptr, a.k, 0u, L, ws, st);
}

}  // namespace vsk
