// K1: the single streaming pass over the logits.
//
// Each wave owns a tile of 4096 consecutive logits of one row: 64 lanes x 64
// values, loaded with 16-byte vector loads and held in registers. Per tile it
// writes a meta word (candidate counts and flags) and up to two candidate
// lists of packed (ordered key << 32 | ~id):
//  - list A, for the draw: the tile's argmax of x with its lowest id (greedy
//    rows, and the row maximum the full-vocabulary and slow paths need), or
//    for top-k rows (2 <= k <= 64) a superset of the tile's top k of
//    s = x / T: every value >= tau, where tau is the k-th largest of the 64
//    lane maxima (of the 128 lane top-two values when k > 32). At least k
//    values reach tau, so nothing below it can be among the row's top k;
//  - list B, for top-k log-probabilities of x when list A cannot serve them.
// In log-probability mode it also writes the tile's max and sum of exp(x - max).
// tau comes from a ballot radix select over the lane maxima and candidates are
// compacted by ballot and written directly, so the pass has no sorting network
// and no LDS traffic. A tile with more than 128 candidates (heavy ties at the
// threshold) sets an overflow flag; the row kernels then select exactly from
// the row itself.
#include "vs_device.h"
#include "vs_kernels.h"

namespace vsk {
namespace {

constexpr int kVals = 64;  // values per lane

template <typename E>
__device__ __forceinline__ int elem_index(int tile_base, int q) {
  constexpr int EPV = Epv<E>::n;
  return tile_base + ((q / EPV) * kWave + lane()) * EPV + (q % EPV);
}

template <typename E>
__device__ __forceinline__ void load_tile(const E* __restrict__ rowp, int tile_base, int V,
                                          bool vec, bool stream, float (&v)[kVals]) {
  constexpr int EPV = Epv<E>::n;
  constexpr int NV = kVals / EPV;
  const int l = lane();
  if (vec) {
    uint4 raw[NV];
    if (stream) {
#pragma unroll
      for (int i = 0; i < NV; ++i) raw[i] = load16_stream(rowp + tile_base + (i * kWave + l) * EPV);
    } else {
#pragma unroll
      for (int i = 0; i < NV; ++i) raw[i] = load16(rowp + tile_base + (i * kWave + l) * EPV);
    }
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

// Stages in LDS (sk: keys, si: ids; one region per wave) every value of the
// tile that reaches the threshold: v >= pre, and for T != 1 also
// key(v / T) >= sig_key. Returns the count (only the first kSelCap are stored).
template <typename E, bool kVec, bool kT1>
__device__ __forceinline__ int extract(const float (&v)[kVals], int tile_base, int V, float pre,
                                       uint32_t sig_key, float T, uint32_t* __restrict__ sk,
                                       int32_t* __restrict__ si) {
  int n = 0;
#pragma unroll
  for (int q = 0; q < kVals; ++q) {
    bool p = v[q] >= pre;
    if (!kVec) p = p && elem_index<E>(tile_base, q) < V;
    uint64_t bal = __builtin_amdgcn_ballot_w64(p);
    if (bal) {  // uniform: taken only when some lane has a candidate here
      uint32_t key = f2key(v[q]);
      if (!kT1) {
        if (p) {
          key = f2key(v[q] / T);
          p = key >= sig_key;
        }
        bal = __builtin_amdgcn_ballot_w64(p);
      }
      if (p) {
        const int pos = n + lanes_below(bal);
        if (pos < kSelCap) {
          sk[pos] = key;
          si[pos] = elem_index<E>(tile_base, q);
        }
      }
      n += __popcll(bal);
    }
  }
  return n;
}

// Writes a superset of the tile's top-k (2 <= k <= 64) of s = x / T (T > 0) to
// out and returns its size, or -1 when more than kSelCap values qualify. The
// exact k-th largest key of the tile (0 when the tile holds fewer than k
// values) goes to *kth: at least k values of the row reach it.
template <typename E>
__device__ __forceinline__ int tile_topk(const float (&v)[kVals], float lmax, int tile_base,
                                         int V, bool vec, int k, float T,
                                         uint64_t* __restrict__ out, uint32_t* __restrict__ sk,
                                         int32_t* __restrict__ si, uint32_t* kth) {
  uint32_t tau_key;
  if (k <= 32) {
    tau_key = wave_kth_largest(f2key(lmax), k);
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
    tau_key = wave_kth_largest2(f2key(lmax), f2key(b), k);
  }
  const float tau = key2f(tau_key);
  int n;
  if (T == 1.0f) {
    n = vec ? extract<E, true, true>(v, tile_base, V, tau, tau_key, T, sk, si)
            : extract<E, false, true>(v, tile_base, V, tau, tau_key, T, sk, si);
  } else {
    const uint32_t sig_key = f2key(tau / T);
    // fl(x/T) >= fl(tau/T) implies x >= tau - 2^-22 |tau| - T 2^-149 (both
    // quotients round to the same float, so they differ by at most one ulp of
    // it); the bound used is looser still and rounded down.
    const double lb = static_cast<double>(tau) -
                      __builtin_ldexp(fabs(static_cast<double>(tau)), -21) -
                      static_cast<double>(T) * 0x1p-148;
    float pre = static_cast<float>(lb);
    if (static_cast<double>(pre) > lb) pre = nextafterf(pre, -kInf);
    n = vec ? extract<E, true, false>(v, tile_base, V, pre, sig_key, T, sk, si)
            : extract<E, false, false>(v, tile_base, V, pre, sig_key, T, sk, si);
  }
  if (n > kSelCap) return -1;
  wave_lds_wait();
  // one coalesced write of the staged candidates, and the exact k-th key
  const int l = lane();
  const uint32_t ka = l < n ? sk[l] : 0u;
  if (l < n) out[l] = pack(ka, si[l]);
  if (n > kWave) {
    const uint32_t kb = l + kWave < n ? sk[l + kWave] : 0u;
    if (l + kWave < n) out[l + kWave] = pack(kb, si[l + kWave]);
    *kth = wave_kth_largest2(ka, kb, k);
  } else {
    *kth = (n >= k) ? wave_kth_largest(ka, k) : 0u;
  }
  wave_lds_wait();
  return n;
}

template <typename E>
__global__ __launch_bounds__(256) void k_select(Job j) {
  __shared__ uint32_t stage_key[kSelWaves][kSelCap];
  __shared__ int32_t stage_id[kSelWaves][kSelCap];
  int row, wg;
  if (!xcd_row_tile(blockIdx.x, j.B, j.wpr, &row, &wg)) return;
  const int w = threadIdx.x / kWave;
  const int tile = wg * kSelWaves + w;
  if (tile >= j.ntile) return;  // the kernel has no block-level barrier
  const int l = lane();
  const Plan pl = plan_row(j, row);

  const E* rowp = static_cast<const E*>(j.logits) + static_cast<int64_t>(row) * j.ld;
  const int tile_base = tile * kSelTile;
  const bool vec = j.aligned && (tile_base + kSelTile <= j.V);
  // Rows finished from this pass alone are read once: stream them past the
  // caches. Rows whose logits are read again later keep the normal policy.
  const bool stream = !j.out_full && j.sample &&
                      (pl.c.mode == kModeGreedy || pl.c.mode == kModeKFast);
  float v[kVals];
  load_tile<E>(rowp, tile_base, j.V, vec, stream, v);

  float lmax = -kInf;
  bool bad = false;
#pragma unroll
  for (int q = 0; q < kVals; ++q) {
    lmax = fmaxf(lmax, v[q]);
    bad = bad || __builtin_amdgcn_classf(v[q], 0x203);  // NaN or +inf
  }
  uint32_t meta = (__ballot(bad) != 0ull) ? kMetaBadLogits : 0u;
  const float M = wave_max_dpp(lmax);
  if (M > -kInf) meta |= kMetaHasFinite;
  const size_t slot = static_cast<size_t>(row) * j.ntile + tile;

  if (j.lse) {
    float s = 0.0f;
    if (M > -kInf) {
#pragma unroll
      for (int q = 0; q < kVals; ++q) s += __expf(v[q] - M);
    }
    s = wave_sum_dpp(s);
    if (l == 0) j.lpart[slot] = LsePart{M, s};
  }

  uint64_t* outA = j.candA + slot * kSelCap;
  if (pl.kA == 1) {
    const uint64_t best = tile_argmax<E>(v, M, tile_base, j.V, vec);
    if (best) meta |= 1u;
    if (l == 0) {
      if (best) outA[0] = best;
      j.kthA[slot] = pkey(best);  // the tile maximum: its 1st-largest key
    }
  } else if (pl.kA > 1) {
    uint32_t kth = 0;
    const int n = tile_topk<E>(v, lmax, tile_base, j.V, vec, pl.kA, pl.TA, outA, stage_key[w],
                               stage_id[w], &kth);
    meta |= (n < 0) ? kMetaOverflowA : static_cast<uint32_t>(n);
    if (l == 0) j.kthA[slot] = kth;
  }
  if (pl.kB > 1) {
    uint32_t kth = 0;
    const int n = tile_topk<E>(v, lmax, tile_base, j.V, vec, pl.kB, 1.0f,
                               j.candB + slot * kSelCap, stage_key[w], stage_id[w], &kth);
    meta |= (n < 0) ? kMetaOverflowB : (static_cast<uint32_t>(n) << kMetaCountBShift);
    if (l == 0) j.kthB[slot] = kth;
  } else if (pl.kB == 1) {
    const uint64_t best = tile_argmax<E>(v, M, tile_base, j.V, vec);
    if (best) meta |= 1u << kMetaCountBShift;
    if (l == 0) {
      if (best) j.candB[slot * kSelCap] = best;
      j.kthB[slot] = pkey(best);
    }
  }
  if (l == 0) j.meta[slot] = meta;
}

}  // namespace

hipError_t launch_select(const Job& j, hipStream_t st) {
  const int grid = xcd_grid(j.B, j.wpr);
  if (j.dt == VS_F32)
    hipLaunchKernelGGL(k_select<float>, dim3(grid), dim3(256), 0, st, j);
  else
    hipLaunchKernelGGL(k_select<uint16_t>, dim3(grid), dim3(256), 0, st, j);
  return hipGetLastError();
}

}  // namespace vsk
