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
//  - for a list that wants the argmax of x: each lane's best value and its
//    first id;
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
// A segment that is a whole row finishes the row itself when its draw needs
// nothing beyond its candidates (see the closing steps below), and when it
// finishes every row of a call that asks for the full log-softmax, its waves
// then write the row's log-probabilities, reading the row a second time.
#include "vs_device.h"
#include "vs_kernels.h"
#include "vs_penalty.h"

namespace vsk {
namespace {

constexpr int kVals = kSelTile / kWave;  // values per lane and tile (32)
constexpr int kGroup = 4;         // values per group (a lane's maxima are kept per group)
constexpr int kGroups = kVals / kGroup;
static_assert(kGroup == 4 && kVals % kGroup == 0 && kGroups <= 32, "groups of 4 values, a bit each");

constexpr int kPoolCap = 512;     // candidates per segment and list (the shared pool)
constexpr int kCheck = 32;        // the pool's bound is recomputed every kCheck entries
static_assert(kPoolCap % 16 == 0, "rank_counts reads the pool in batches of up to 16");
constexpr float kL2E = 1.44269504088896340736f;
// s_waitcnt operand for "vector memory count 0", other counters left at their
// maxima (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVmcnt0 = 0x0F70;

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
// The 16-byte loads of the tile at base; stride 0 makes each load read 16
// bytes of the first tile in every lane (a placeholder load that keeps the
// load count fixed).
template <typename E, bool kStream>
__device__ __forceinline__ void load_raw(const E* __restrict__ base, int stride, Raw<E>& raw) {
  constexpr int EPV = Epv<E>::n;
  // one lane address, the loads at fixed offsets from it (a placeholder reads
  // the same 16 bytes in every lane, at each load's offset)
  const E* p = base + lane() * EPV * stride;
#pragma unroll
  for (int i = 0; i < Raw<E>::n; ++i) {
    raw.r[i] = kStream ? load16_stream(p + i * kWave * EPV) : load16(p + i * kWave * EPV);
  }
}

// Tl: the log-prob temperature of the row (1: the values as they are).
template <typename E>
__device__ __forceinline__ void unpack_raw(const Raw<E>& raw, const E* rowp, float (&v)[kVals],
                                           float Tl) {
  constexpr int EPV = Epv<E>::n;
#pragma unroll
  for (int i = 0; i < Raw<E>::n; ++i) unpack16(raw.r[i], &v[i * EPV], rowp);
  if (Tl != 1.0f) {  // uniform
#pragma unroll
    for (int q = 0; q < kVals; ++q) v[q] = v[q] / Tl;
  }
}

// A tile that ends past V: element loads, -inf beyond V.
template <typename E>
__device__ __forceinline__ void load_tail(const E* __restrict__ rowp, int tile_base, int V,
                                          float (&v)[kVals], float Tl) {
#pragma unroll
  for (int q = 0; q < kVals; ++q) {
    const int idx = elem_index<E>(tile_base, q);
    v[q] = (idx < V) ? lse_scaled(to_f32(rowp[idx]), Tl) : -kInf;
  }
}

// The smallest float pre such that key(fl(x / T)) >= thr implies x >= pre:
// fl(x / T) >= s forces x / T >= pred(s), so x >= T * pred(s) (exact in
// double), rounded down to float. Keys at or below key(-inf) stand for -inf
// or for negative NaNs: every value passes.
__device__ __forceinline__ float prefilter(uint32_t thr, float T) {
  if (thr <= kKeyNegInf) return -kInf;
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
  float b = -kInf;
  if (k > 32) {
    // the lane's second largest value: the largest value below the lane
    // maximum, or the maximum itself when it occurs twice
    int nmax = 0;
#pragma unroll
    for (int q = 0; q < kVals; ++q) {
      b = fmaxf(b, v[q] < lmax ? v[q] : -kInf);
      nmax += (v[q] == lmax) ? 1 : 0;
    }
    if (nmax > 1) b = lmax;
  }
  const uint32_t tk = (k <= 32) ? wave_kth_largest(f2key(lmax), k)
                                : wave_kth_largest2(f2key(lmax), f2key(b), k);
  return (T == 1.0f) ? tk : f2key(key2f(tk) / T);
}

// Appends to the list's shared pool the values of group gi (values 4 gi ..
// 4 gi + 3 of every lane) that reach its threshold: v >= pre (pre =
// prefilter(thr, T)), and for T != 1 also key(v / T) >= thr. The group
// reserves its space in the pool with one atomic add and writes its entries
// packed. Returns -1 when the pool is full (the caller then flags the
// overflow), else 1 when the reservation crossed a multiple of kCheck entries
// (*end: the pool size after it), else 0.
template <typename E, int gi>
__device__ __forceinline__ int extract_group(const float (&v)[kVals], int tile_base, int V,
                                             bool vec, uint32_t thr, float pre, float T,
                                             int* pool_n, uint64_t* __restrict__ pool, int* end) {
  constexpr int EPV = Epv<E>::n;
  const int l = lane();
  bool p[kGroup];
  uint32_t key[kGroup];
  uint64_t bal[kGroup];
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < kGroup; ++u) {
    // value q = gi * 4 + u of the lane: vector q / EPV, component q % EPV
    constexpr int q0 = gi * kGroup;
    const int q = q0 + u;
    const int id = tile_base + ((q / EPV) * kWave + l) * EPV + (q % EPV);
    const float x = v[q];
    p[u] = x >= pre && (vec || id < V);
    key[u] = f2key(x);
    if (T != 1.0f && p[u]) {
      key[u] = f2key(x / T);
      p[u] = key[u] >= thr;
    }
    bal[u] = __builtin_amdgcn_ballot_w64(p[u]);
    cnt += __popcll(bal[u]);
  }
  if (cnt == 0) return 0;
  int base = 0;
  if (l == 0) base = atomicAdd(pool_n, cnt);
  base = __builtin_amdgcn_readfirstlane(base);
  if (base + cnt > kPoolCap) return -1;
  const int crossed = (base + cnt) / kCheck > base / kCheck ? 1 : 0;
  if (crossed) *end = base + cnt;
#pragma unroll
  for (int u = 0; u < kGroup; ++u) {
    const int q = gi * kGroup + u;
    const int id = tile_base + ((q / EPV) * kWave + l) * EPV + (q % EPV);
    if (p[u]) pool[base + lanes_below(bal[u])] = pack(key[u], id);
    base += __popcll(bal[u]);
  }
  return crossed;
}

// The active groups of the tile from group G on (a bit per group whose
// maximum reaches the prefilter in some lane), each through extract_group.
// Same result codes.
template <typename E, int G = 0>
__device__ __forceinline__ int extract(const float (&v)[kVals], uint32_t active, int tile_base,
                                       int V, bool vec, uint32_t thr, float pre, float T,
                                       int* pool_n, uint64_t* __restrict__ pool, int* end) {
  if constexpr (G == kGroups) {
    return 0;
  } else {
    int crossed = 0;
    if (active & (1u << G)) {
      crossed = extract_group<E, G>(v, tile_base, V, vec, thr, pre, T, pool_n, pool, end);
      if (crossed < 0) return -1;
    }
    const int rest = extract<E, G + 1>(v, active, tile_base, V, vec, thr, pre, T, pool_n, pool, end);
    return rest < 0 ? -1 : (crossed | rest);
  }
}

// Adds to r[i] the number of the first n pool entries larger than e[i]. The
// pool is read kBatch entries at a time, all lanes reading the same words, so
// that the reads overlap instead of each waiting on the one before; entries
// from n on count as 0. n <= kPoolCap, a multiple of kBatch.
template <int R, int kBatch>
__device__ __forceinline__ void rank_counts(const uint64_t* pool, int n, const uint64_t (&e)[R],
                                            int (&r)[R]) {
  for (int m0 = 0; m0 < n; m0 += kBatch) {  // uniform
    uint64_t o[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) o[u] = pool[m0 + u];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const uint64_t x = (m0 + u < n) ? o[u] : 0ull;
#pragma unroll
      for (int i = 0; i < R; ++i) r[i] += (x > e[i]) ? 1 : 0;
    }
  }
}

// The k-th largest key among the n packed entries of an LDS pool, with one
// wave: each entry's rank is the number of larger entries, and the entry of
// rank k - 1 holds the key. Entries still being written read as 0 (below every
// value), which can only lower the result: it stays a valid bound. 0 when the
// pool has fewer than k entries.
__device__ __forceinline__ uint32_t pool_kth(const uint64_t* pool, int n, int k) {
  constexpr int R = 2;  // entries per lane and pass (the passes cover 128 entries each)
  const int l = lane();
  uint32_t best = 0u;
  for (int c0 = 0; c0 < n; c0 += R * kWave) {  // uniform
    uint64_t e[R];
    int r[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int at = c0 + i * kWave + l;
      e[i] = at < n ? pool[at] : 0ull;
      r[i] = 0;
    }
    rank_counts<R, 8>(pool, n, e, r);
#pragma unroll
    for (int i = 0; i < R; ++i)
      if (r[i] == k - 1 && e[i] != 0ull) best = pkey(e[i]);
  }
  return wave_max_u32_dpp(best);
}

// A wave's view of one top-k list.
struct List {
  int li;        // 0: list A, 1: list B
  int k;
  float T;
  uint32_t thr;  // the bound this wave uses (a lower bound on the segment's k-th key)
  float pre;     // prefilter(thr, T): values of x below it cannot reach thr
  __device__ __forceinline__ void set_thr(uint32_t t) {
    thr = t;
    pre = prefilter(t, T);
  }
};


// The penalty step's table: 2^12 slots of id and count.
constexpr int kPenLog2 = 12;

struct SegSh {
  // The arrays of the streaming loop and its closing steps share their memory
  // with the penalty step's table, which is done with before they are first
  // written.
  union {
    struct {
      uint64_t pool[2][kPoolCap];  // each list's candidates (packed), appended by all waves
      double q[kPoolCap];          // list A's pool: -log(u) of the entries reaching the bound
      uint32_t rank[2][kPoolCap];  // each pool entry's rank, summed over the waves' slices
      uint64_t stage[kSelMaxWaves][kWave];  // per-wave staging of a list rescan
    };
    struct {
      uint32_t pen_keys[1 << kPenLog2];
      uint32_t pen_counts[1 << kPenLog2];
    };
  };
  int next_tile;  // the segment's next unclaimed tile (claimed by whole waves)
  int next_out;   // the next tile of the full log-softmax write
  uint32_t thr[2];
  int merge_n[2];
  int ovf[2];
  uint32_t kth_key[2];
  uint32_t flags;
  uint32_t hist[256];
  uint32_t prefix;
  int krem;
  int out_n[2];
  float wm[16];
  float ws[16];
  uint64_t best[2][16];
  uint64_t top[2][kSelCap];  // each list's segment candidates
  uint64_t srt[2][kWave];    // a list's 64 best, sorted (segments handed on; rescans)
  float tot_m, tot_s;        // the segment's log-sum-exp partial
  uint64_t tot_b[2];         // the segment's argmax per argmax list
  PenSh pen;                 // the penalty step's scalars
};


// Finishes list `li` in LDS: leaves the 64 best entries sorted in sh.srt and,
// when `out` is set, gathers in sh.top every entry whose key reaches the
// segment's exact k-th largest key (*kth, 0 with fewer than k entries). An
// entry's rank is the number of larger entries (packed values are distinct),
// so it is the entry's sorted position, and the entry of rank k - 1 holds the
// k-th key. Every wave counts one slice of the pool against all entries and
// adds its counts to sh.rank (zero at the start), so the count is spread over
// the block. Returns the number gathered (without `out`: the number of sorted
// entries the list needs, min(n, k)), or -1 on overflow. Called by the whole
// block (W waves) after the streaming loop; nothing here touches global
// memory, so no wait on the memory system is taken.
__device__ __forceinline__ int merge_list(SegSh& sh, int li, int k, int W, bool out,
                                          uint32_t* kth) {
  const int l = lane();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int NT = W * kWave;
  const int n = sh.merge_n[li];
  *kth = 0u;
  if (sh.ovf[li] || n > kPoolCap) return -1;
  const uint64_t* pool = sh.pool[li];
  uint32_t* rank = sh.rank[li];
  // slices of a multiple of 8 entries (clamped to the pool, whose unused
  // entries read as 0 and count as smaller than every entry), read 8 at a
  // time with no condition, so that the reads overlap
  const int C = (((n + W - 1) / W) + 7) & ~7;
  const int c0 = w * C;
  const int c1 = min(c0 + C, kPoolCap);
  for (int i0 = 0; i0 < n && c0 < n; i0 += kWave) {  // uniform
    const int i = i0 + l;
    const uint64_t e = pool[i < kPoolCap ? i : kPoolCap - 1];
    int cnt = 0;
    for (int m0 = c0; m0 < c1; m0 += 8) {  // uniform
      uint64_t o[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] = pool[m0 + u];
#pragma unroll
      for (int u = 0; u < 8; ++u) cnt += (o[u] > e) ? 1 : 0;
    }
    if (i < n && cnt) atomicAdd(&rank[i], static_cast<uint32_t>(cnt));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += NT) {
    const int r = static_cast<int>(rank[i]);
    const uint64_t e = pool[i];
    if (r < kWave) sh.srt[li][r] = e;
    if (r == k - 1) sh.kth_key[li] = pkey(e);
  }
  __syncthreads();
  if (!out) return n < k ? n : k;
  const uint32_t kt = (n >= k) ? sh.kth_key[li] : 0u;
  uint64_t* keep = sh.top[li];
  for (int i0 = 0; i0 < n; i0 += NT) {
    const int i = i0 + static_cast<int>(threadIdx.x);
    const uint64_t e = i < n ? pool[i] : 0ull;
    const bool take = i < n && pkey(e) >= kt;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(take);
    int b0 = 0;
    if (l == 0 && bal) b0 = atomicAdd(&sh.out_n[li], __popcll(bal));
    b0 = __shfl(b0, 0);
    if (take) {
      const int pos = b0 + lanes_below(bal);
      if (pos < kSelCap) keep[pos] = e;
    }
  }
  __syncthreads();
  const int c = sh.out_n[li];
  *kth = kt;
  return c > kSelCap ? -1 : c;
}

// Per-lane maxima of the 4-value groups and of the lane, NaN-propagating: a
// lane maximum is NaN or +inf exactly when the lane holds a NaN or a +inf,
// which make the row invalid.
__device__ __forceinline__ void tile_maxima(const float (&v)[kVals], float (&g)[kGroups],
                                            float& lmax) {
#pragma unroll
  for (int gi = 0; gi < kGroups; ++gi) {
    float m = v[gi * kGroup];
#pragma unroll
    for (int u = 1; u < kGroup; ++u) m = __builtin_elementwise_maximum(m, v[gi * kGroup + u]);
    g[gi] = m;
  }
  lmax = g[0];
#pragma unroll
  for (int gi = 1; gi < kGroups; ++gi) lmax = __builtin_elementwise_maximum(lmax, g[gi]);
}

// Adds one tile's candidates to the list's shared pool (in LDS). shv is the
// workgroup's shared bound, read from LDS when the tile's processing began (a
// stale value is still a valid bound). Each time the pool grows past a
// multiple of kCheck entries, the wave that crossed it recomputes the exact
// k-th largest key of the pool and raises the shared bound: the pool holds
// every value seen so far that reached the bound in force, so that key is the
// running k-th largest value of the segment.
template <typename E>
__device__ __forceinline__ void list_tile(const float (&v)[kVals], const float (&g)[kGroups],
                                          float lmax, int tile_base, int V, bool vec, List& L,
                                          uint32_t shv, SegSh& sh, uint64_t* pool) {
  shv = __builtin_amdgcn_readfirstlane(shv);
  if (shv > L.thr) L.set_thr(shv);  // another wave raised the bound
  // no value of the tile reaches this wave's bound: nothing to do (no LDS)
  if (L.thr != 0u && __builtin_amdgcn_ballot_w64(lmax >= L.pre) == 0ull) return;
  if (L.thr == 0u) {  // no bound yet: this tile's own k-th lane maximum
    L.set_thr(tile_bound(v, lmax, L.k, L.T));
    if (lane() == 0) atomicMax(&sh.thr[L.li], L.thr);
  }
  uint32_t active = 0;
#pragma unroll
  for (int gi = 0; gi < kGroups; ++gi)
    if (__builtin_amdgcn_ballot_w64(g[gi] >= L.pre) != 0ull) active |= 1u << gi;
  if (!active) return;
  int end = 0;
  const int r = extract<E>(v, active, tile_base, V, vec, L.thr, L.pre, L.T, &sh.merge_n[L.li],
                           pool, &end);
  if (r < 0) {  // the pool is full: the row is selected the slow way
    if (lane() == 0) sh.ovf[L.li] = 1;
    return;
  }
  if (r > 0) {
    const uint32_t nb = pool_kth(pool, end, L.k);
    if (nb > L.thr) {
      L.set_thr(nb);
      if (lane() == 0) atomicMax(&sh.thr[L.li], nb);
    }
  }
}

// A lower bound on the k-th largest of the block's keys, one per thread
// (1 <= k <= blockDim): the top 16 bits of that key, found by two 8-bit digit
// passes over an LDS histogram (at least k keys reach the result). Called by
// the whole block (NT threads); inline, so that the loads in flight around it
// are not waited for.
__device__ __forceinline__ uint32_t block_kth_u32(uint32_t key, int k, int NT, SegSh& sh) {
  uint32_t prefix = 0;
  for (int d = 3; d >= 2; --d) {
    __syncthreads();  // the previous pass's readers are done with sh
    for (int i = threadIdx.x; i < 256; i += NT) sh.hist[i] = 0u;
    __syncthreads();
    const uint32_t hmask = (d == 3) ? 0u : (0xffffffffu << (8 * (d + 1)));
    if ((key & hmask) == prefix) atomicAdd(&sh.hist[(key >> (8 * d)) & 0xffu], 1u);
    __syncthreads();
    if (threadIdx.x < kWave) {
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
  }
  __syncthreads();
  return prefix;
}

// The exact 64 best entries of one list (packed keys of s = x / T with their
// ids) over the whole row, for a row whose candidate pool overflowed. Each
// wave rescans its slices of the row (64 lanes x one 16-byte vector: 256 fp32
// or 512 bf16 values, every W-th slice) keeping its 64 best entries sorted
// across its lanes, lane 0 the best. A slice contributes at most its own 64
// best: when more than 64 of its entries beat the wave's 64th best, they are
// cut to the keys above the slice's exact 64th largest key plus, of the keys
// equal to it, the lowest ids (larger packed values) up to 64 in all. The
// survivors are compacted through the wave's LDS stage, sorted and merged in.
// The waves' lists then merge pairwise through LDS, and the block's 64 best
// land in srt. Packed entries are distinct, so the result depends on no
// order. Small slices keep the code and its registers small: the path is
// rare. Called by the whole block (W waves, every lane active).
template <typename E>
__device__ __forceinline__ void rescan_list(const E* __restrict__ rowp, int V, bool aligned,
                                            float T, int W, uint64_t (*stage)[kWave],
                                            uint64_t* srt) {
  constexpr int EPV = Epv<E>::n;
  constexpr int kSlice = kWave * EPV;
  const int l = lane();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int nslice = (V + kSlice - 1) / kSlice;
  uint64_t top = 0ull;   // this wave's 64 best, descending across lanes
  uint64_t tmin = 0ull;  // its 64th best: entries must beat it
  for (int t = w; t < nslice; t += W) {
    const int id0 = t * kSlice + l * EPV;  // this lane's first id; ids follow the lane, then u
    float v[EPV];
    if (aligned && (t + 1) * kSlice <= V) {
      unpack16(load16(rowp + id0), v, rowp);
    } else {
#pragma unroll
      for (int u = 0; u < EPV; ++u) v[u] = (id0 + u < V) ? to_f32(rowp[id0 + u]) : -kInf;
    }
    uint32_t key[EPV];
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < EPV; ++u) {
      key[u] = (id0 + u < V) ? f2key((T == 1.0f) ? v[u] : v[u] / T) : 0u;
      cnt += (key[u] != 0u && pack(key[u], id0 + u) > tmin) ? 1 : 0;
    }
    cnt = wave_sum_dpp_i32(cnt);
    if (cnt == 0) continue;
    uint32_t kt = 0u;  // with more than 64 entries: the slice's 64th largest key
    int need = kWave;  // entries equal to kt still wanted, lowest ids first
    if (cnt > kWave) {
      // the largest t with at least 64 keys >= t, one bit at a time
      for (int b = 31; b >= 0; --b) {
        const uint32_t c = kt | (1u << b);
        int ge = 0;
#pragma unroll
        for (int u = 0; u < EPV; ++u) ge += key[u] >= c ? 1 : 0;
        if (wave_sum_dpp_i32(ge) >= kWave) kt = c;
      }
      int gt = 0;
#pragma unroll
      for (int u = 0; u < EPV; ++u) gt += key[u] > kt ? 1 : 0;
      need = kWave - wave_sum_dpp_i32(gt);
    }
    // rank of a key equal to kt among those of the slice, in id order: ties in
    // lower lanes, then in this lane before it
    int rank = 0;
#pragma unroll
    for (int u = 0; u < EPV; ++u) rank += lanes_below(__ballot(key[u] != 0u && key[u] == kt));
    int n = 0;  // entries staged (uniform)
#pragma unroll
    for (int u = 0; u < EPV; ++u) {
      const bool tie = key[u] != 0u && key[u] == kt;
      const bool sel = key[u] != 0u && (key[u] > kt || (tie && rank < need)) &&
                       pack(key[u], id0 + u) > tmin;
      rank += tie ? 1 : 0;
      const uint64_t bs = __ballot(sel);
      if (sel) stage[w][n + lanes_below(bs)] = pack(key[u], id0 + u);
      n += __popcll(bs);
    }
    wave_lds_sync();
    const uint64_t b = l < n ? stage[w][l] : 0ull;
    top = wave_merge_top_desc(top, wave_sort_desc(b));
    tmin = __shfl(top, kWave - 1);
    wave_lds_sync();
  }
  for (int h = 1; h < W; h <<= 1) {
    __syncthreads();
    if ((w & (2 * h - 1)) == h) stage[w][l] = top;
    __syncthreads();
    if ((w & (2 * h - 1)) == 0 && w + h < W) top = wave_merge_top_desc(top, stage[w + h][l]);
  }
  if (w == 0) srt[l] = top;
  __syncthreads();
}

// A pool entry with its pool position i in the low bits, ordered as the entry:
// the key, then 0x1fffff - id (ids are below 2^21), then i (11 bits).
constexpr int kTagBits = 11;
static_assert(kPoolCap <= (1 << kTagBits), "pool positions fit the tag");
__device__ __forceinline__ uint64_t tag_entry(uint64_t e, int i) {
  const uint32_t rid = 0x1fffffu - static_cast<uint32_t>(pid(e));
  return (static_cast<uint64_t>(pkey(e)) << 32) | (static_cast<uint64_t>(rid) << kTagBits) |
         static_cast<uint32_t>(i);
}
__device__ __forceinline__ uint64_t untag_entry(uint64_t t) {
  if (t == 0ull) return 0ull;
  const int32_t id = static_cast<int32_t>(0x1fffffu - ((static_cast<uint32_t>(t) >> kTagBits) & 0x1fffffu));
  return pack(static_cast<uint32_t>(t >> 32), id);
}
__device__ __forceinline__ int tag_pos(uint64_t t) {
  return static_cast<int>(static_cast<uint32_t>(t) & ((1u << kTagBits) - 1u));
}

// The best entries of a list's pool (n entries, unused slots 0) whose key
// reaches the bound thr, sorted descending across the lanes of one wave (lane
// i the i-th; 0 past the end), as tagged entries (tag_entry) when kTag; *cnt
// gets how many reach thr. Every entry of the row's top k reaches a valid
// bound, and every value that reaches the final bound entered the pool, so the
// result starts with the row's top k. Usually at most 64 entries reach it:
// they are compacted through the wave's LDS stage and sorted in registers.
// Otherwise the pool's chunks are sorted and merged one by one. Called by a
// whole wave, every lane active.
template <bool kTag>
__device__ __forceinline__ uint64_t wave_top_of_pool(const uint64_t* pool, int n, uint32_t thr,
                                                     uint64_t* stage, int* cnt) {
  const int l = lane();
  int total = 0;
  for (int c0 = 0; c0 < n; c0 += kWave) {  // uniform
    const int i = c0 + l;
    uint64_t e = i < n ? pool[i] : 0ull;
    const bool keep = e != 0ull && pkey(e) >= thr;
    if (kTag && keep) e = tag_entry(e, i);
    const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
    const int at = total + lanes_below(bal);
    if (keep && at < kWave) stage[at] = e;
    total += __popcll(bal);
  }
  *cnt = total;
  if (total <= kWave) {
    wave_lds_wait();
    return wave_sort_u64<true>(l < total ? stage[l] : 0ull);
  }
  uint64_t top = 0ull;
  for (int c0 = 0; c0 < n; c0 += kWave) {  // uniform
    const int i = c0 + l;
    uint64_t e = i < n ? pool[i] : 0ull;
    if (e == 0ull || pkey(e) < thr) e = 0ull;
    if (kTag && e != 0ull) e = tag_entry(e, i);
    if (__builtin_amdgcn_ballot_w64(e != 0ull) == 0ull) continue;
    top = wave_merge_top_u64(top, wave_sort_u64<false>(e));
  }
  return top;
}

// Writes the row's full log-softmax, lp = (x - M) - logS for every id (NaN
// throughout for a row that failed its checks), with the formula and inputs of
// the separate write pass. Whole waves claim 2048-id tiles from an LDS counter
// as they arrive; a tile is read with 16-byte loads (a second read of the row
// this workgroup has just streamed, mostly served by the caches) and written
// with non-temporal 16-byte stores, or element by element at the row's end
// and for unaligned rows or outputs.
template <typename E, bool kStream>
__device__ __forceinline__ void write_full_row(const Job& j, const E* __restrict__ rowp,
                                               float* __restrict__ orow, int t_begin, int t_end,
                                               float M, float logS, float Tl, int* next) {
  constexpr int EPV = Epv<E>::n;
  const int l = lane();
  for (;;) {
    int t = 0;
    if (l == 0) t = atomicAdd(next, 1);
    t = __builtin_amdgcn_readfirstlane(t);
    if (t >= t_end) break;
    // last tiles first: the streaming pass read them last, so more of them
    // are still in the caches
    t = t_end - 1 - (t - t_begin);
    const int base = t * kSelTile;
    if (j.aligned && j.full_vec && base + kSelTile <= j.V) {  // uniform
      Raw<E> X;
      load_raw<E, kStream>(rowp + base, 1, X);
#pragma unroll
      for (int i = 0; i < Raw<E>::n; ++i) {
        float x[EPV];
        unpack16(X.r[i], x, rowp);
        if (Tl != 1.0f) {  // uniform
#pragma unroll
          for (int c = 0; c < EPV; ++c) x[c] = x[c] / Tl;
        }
        const int j0 = base + (i * kWave + l) * EPV;
#pragma unroll
        for (int c = 0; c < EPV; c += 4) {
          f32x4 o;
          o.x = (x[c] - M) - logS;
          o.y = (x[c + 1] - M) - logS;
          o.z = (x[c + 2] - M) - logS;
          o.w = (x[c + 3] - M) - logS;
          __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(orow + j0 + c));
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < kVals; ++q) {
        const int id = elem_index<E>(base, q);
        if (id < j.V) orow[id] = (lse_scaled(to_f32(rowp[id]), Tl) - M) - logS;
      }
    }
  }
}

// Finishes a row with one wave: the same outputs the row kernel writes (draw,
// kept count, status, log-sum-exp, the log-probs of the sampled or given id and
// the top-k log-probs). LA and LB hold the lists' best entries sorted across
// the lanes (lane i the i-th, nA and nB of them); (M, S) is the row's
// log-sum-exp partial and bA, bB its argmax for argmax lists; qA, when given,
// holds -log(u) of list A's entries by lane. Every load comes before the first
// store: a load issued after stores waits for them too.
template <typename E>
__device__ __forceinline__ void finish_row(const Job& j, int row, const Plan& pl, uint32_t flags,
                                           uint64_t LA, int nA, uint64_t LB, int nB, float M,
                                           float S, uint64_t bA, uint64_t bB, const double* qA) {
  const int l = lane();
  const float nanv = __builtin_nanf("");
  const RowCfg& c = pl.c;
  const bool bad_logits = (flags & kMetaBadLogits) || !(flags & kMetaHasFinite);
  const float logS = j.lse ? logf(S) : nanv;
  const E* rowp = static_cast<const E*>(j.logits) + static_cast<int64_t>(row) * j.ld;

  // the draw
  int status = 0;
  int32_t id = -1, kept = 0;
  float x_id = nanv;
  if (j.sample) {
    status = c.status | (bad_logits ? VS_ROW_BAD_LOGITS : 0);
    if (pl.kA == 1 && bA == 0ull) status |= VS_ROW_BAD_LOGITS;
    if (status == 0) {
      if ((j.hints & VS_HINT_ALL_GREEDY) && c.mode != kModeGreedy) status = VS_ROW_HINT_VIOLATED;
      if ((j.hints & VS_HINT_NO_GREEDY) && c.mode == kModeGreedy) status = VS_ROW_HINT_VIOLATED;
      if ((j.hints & VS_HINT_SMALL_TOPK) && c.mode != kModeGreedy && c.mode != kModeKFast)
        status = VS_ROW_HINT_VIOLATED;
    }
    if (status == 0) {
      if (c.mode == kModeGreedy) {
        id = pid(bA);
        kept = 1;
      } else {  // top-k <= 64
        status = wave_draw_lanes(LA, nA < pl.kA ? nA : pl.kA, c, row, &id, &kept, nullptr, qA);
      }
    }
    if (status || id < 0 || id >= j.V) {
      if (!status) status = VS_ROW_BAD_LOGITS;  // unreachable: ids come from the row
      id = -1;
      kept = 0;
    }
    // the sampled id's logit: its key when the list holds keys of x itself
    bool x_known = false;
    if (id >= 0) {
      if (c.mode == kModeGreedy) {
        x_id = key2f(pkey(bA));
        x_known = true;
      } else if (pl.TA == 1.0f) {
        const uint64_t hit = __ballot(l < nA && LA != 0ull && pid(LA) == id);
        if (hit) {
          x_id = key2f(pkey(readlane_u64(LA, __ffsll(static_cast<unsigned long long>(hit)) - 1)));
          x_known = true;
        }
      }
    }
    if (j.tok_sampled && id >= 0 && !x_known) x_id = to_f32(rowp[id]);
  }
  // the given id (vs_logprobs)
  int lp_st = bad_logits ? VS_ROW_BAD_LOGITS : 0;
  float x_tok = nanv;
  if (j.lse && !j.sample && j.tok) {
    const int tok = j.tok[row];
    if (tok < 0 || tok >= j.V)
      lp_st |= VS_ROW_BAD_TOKEN_ID;
    else if (!bad_logits)
      x_tok = lse_scaled(to_f32(rowp[tok]), lse_T(j, row));
  }
  // the top-k log-probabilities' source
  uint64_t P = 0ull;
  int n = 0;
  if (j.lse && j.k_lp > 0 && !bad_logits) {
    if (pl.shared && pl.kA == 1) {  // k == 1: the argmax of list A
      n = 1;
      P = bA;
    } else if (pl.shared) {
      n = nA;
      P = LA;
    } else if (pl.kB == 1) {
      n = 1;
      P = bB;
    } else {
      n = nB;
      P = LB;
    }
  }

  // stores
  if (l == 0) {
    if (j.lse) j.rlse[row] = bad_logits ? make_float2(nanv, nanv) : make_float2(M, logS);
    if (j.sample) {
      j.desc[row].mode = kRowDone;
      j.out_ids[row] = id;
      if (j.out_kept) j.out_kept[row] = kept;
      if (j.out_status) j.out_status[row] = status;
      if (j.tok_sampled) j.out_tok_lp[row] = (id < 0 || bad_logits) ? nanv : (x_id - M) - logS;
    } else if (j.lse) {
      if (j.tok) j.out_tok_lp[row] = (lp_st != 0) ? nanv : (x_tok - M) - logS;
      if (j.out_lp_status) j.out_lp_status[row] = lp_st;
    }
  }
  if (j.lse && j.k_lp > 0 && l < j.k_lp) {
    const int k = j.k_lp;
    const bool has = l < n && P != 0ull;
    j.out_lp_ids[static_cast<size_t>(row) * k + l] = has ? pid(P) : -1;
    j.out_lp[static_cast<size_t>(row) * k + l] = has ? (key2f(pkey(P)) - M) - logS : nanv;
  }
}

template <typename E, bool kStream, bool kScaled>
__global__ __launch_bounds__(1024) void k_select(Job j) {
  __shared__ SegSh sh;
  int row, seg;
  if (!xcd_row_tile(blockIdx.x, j.B, j.nseg, &row, &seg)) return;  // uniform per block
  // the block size as a kernel argument: reading blockDim costs a memory load
  const int W = j.nwave;
  const int NT = W * kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = lane();
  const Plan pl = plan_row(j, row);
  // the log-prob temperature (kScaled: vs_logprobs_ex; 1 otherwise, known at
  // compile time): every value is read as x / Tl, so the log-sum-exp, the
  // lists and the writes see s
  const float Tl = kScaled ? lse_T(j, row) : 1.0f;
  const int t_begin = seg * j.tps;
  const int t_end = min(t_begin + j.tps, j.ntile);

  if (j.full_chain && pl.c.mode == kModeFull && pl.c.p < 1.0f) {
    // A full-vocabulary top-p row's histogram, list counter and cut counts
    // start at zero for the histogram and gather passes: this segment's share
    // of the buckets, and the counters with the first segment (the passes
    // route the row themselves; clearing a row they do not take is harmless).
    uint64_t* hw = j.fhw + static_cast<size_t>(row) * kFullBuckets;
    const int per = (kFullBuckets + j.nseg - 1) / j.nseg;
    const int b1 = min(kFullBuckets, (seg + 1) * per);
    for (int i = seg * per + static_cast<int>(threadIdx.x); i < b1; i += NT) hw[i] = 0ull;
    if (seg == 0 && threadIdx.x == 0) {
      j.fcnt[row] = 0u;
      j.fcut[row].count = 0u;
      j.fcut[row].above_c = 0ull;
    }
  }

  if (j.pen) {
    // Occurrence penalties of the ids of this segment, in place, before the
    // segment is read (every id lies in one segment, so each is penalised
    // once; the first segment also reports ids outside [0, V)). The barrier
    // orders the writes before the reads below, and before the table's
    // memory is reused.
    const PenRow pr = pen_row(row, j.pen_pids, j.pen_poff, j.pen_oids, j.pen_ooff, j.pen_pres,
                              j.pen_freq, j.pen_rep, j.pen_ign);
    E* rw = const_cast<E*>(static_cast<const E*>(j.logits)) + static_cast<int64_t>(row) * j.ld;
    const bool bad_id = penalize_range<E, kPenLog2>(
        rw, pr, j.V, t_begin * kSelTile, min(t_end * kSelTile, j.V), seg == 0, sh.pen_keys,
        sh.pen_counts, sh.pen, NT);
    if (seg == 0 && threadIdx.x == 0 && j.out_pen_status)
      j.out_pen_status[row] = (pr.bad ? VS_ROW_BAD_PARAM : 0) | (bad_id ? VS_ROW_BAD_TOKEN_ID : 0);
    __syncthreads();
  }

  if (threadIdx.x == 0) {
    sh.next_tile = t_begin + W;  // the first W tiles go to the waves in order
    sh.thr[0] = sh.thr[1] = 0u;
    sh.ovf[0] = sh.ovf[1] = 0;
    sh.merge_n[0] = sh.merge_n[1] = 0;
    sh.out_n[0] = sh.out_n[1] = 0;
    sh.kth_key[0] = sh.kth_key[1] = 0u;
    sh.flags = 0u;
    sh.next_out = t_begin;
  }
  // empty pool slots read as 0, below every candidate; ranks start at 0
  for (int i = threadIdx.x; i < 2 * kPoolCap; i += NT) {
    (&sh.pool[0][0])[i] = 0ull;
    (&sh.rank[0][0])[i] = 0u;
  }
  __syncthreads();

  List LA{0, pl.kA, pl.TA, 0u, -kInf};
  List LB{1, pl.kB, 1.0f, 0u, -kInf};
  const E* rowp = static_cast<const E*>(j.logits) + static_cast<int64_t>(row) * j.ld;

  // log-sum-exp state per lane: running maximum lm, its shift lc = fl(lm
  // log2 e) (-inf while lm is), and the sum ls of 2^(x log2 e - lc); in
  // "huge" mode (a maximum of 2^120 or more seen by the wave) ls is the sum of
  // exp(x - lm) instead
  float lm = -kInf, lc = -kInf, ls = 0.0f;
  bool huge = false;
  // argmax lists: each lane's best value of x so far (ordered key) and the
  // lowest id holding it
  uint32_t arg_key = 0u;
  int32_t arg_id = -1;
  bool bad_l = false, fin_l = false;
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
  auto step = [&](const float (&v)[kVals], const float (&g)[kGroups], float lmax, int tt,
                  bool vec) __attribute__((always_inline)) {
    const int tile_base = tt * kSelTile;
    // the shared bounds, read now so that the LDS latency hides behind the work below
    const uint32_t shvA =
        pl.kA > 1 ? __hip_atomic_load(&sh.thr[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) : 0u;
    const uint32_t shvB =
        pl.kB > 1 ? __hip_atomic_load(&sh.thr[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) : 0u;
    bad_l = bad_l || !(lmax < kInf);
    fin_l = fin_l || lmax > -kInf;

    if (j.lse) {
      // Each lane keeps sum 2^(x log2 e - c) over its values, c = fl(m log2 e)
      // for its running maximum m (one fma and one exp2 per value); a new
      // maximum rescales the sum by 2^(c_old - c_new). The wave and the
      // workgroup combine the lanes once, at the end.
      if (!huge && __ballot(fabsf(lmax) >= 0x1p120f && fabsf(lmax) < kInf) != 0ull) {
        // a maximum too large for c: from here on sums of exp(x - m)
        huge = true;
        if (lm > -kInf) ls *= __builtin_amdgcn_exp2f(-fmaf(lm, kL2E, -lc));
      }
      const float mn = fmaxf(lm, lmax);  // (a NaN lmax leaves m: the row is invalid anyway)
      if (!huge) {
        const float cn = mn * kL2E;
        ls *= (mn > -kInf) ? __builtin_amdgcn_exp2f(lc - cn) : 1.0f;
        const float cu = (mn > -kInf) ? cn : 0.0f;  // all -inf so far: terms of 0
        float s2[4] = {0.0f, 0.0f, 0.0f, 0.0f};    // independent partial sums
#pragma unroll
        for (int q = 0; q < kVals; ++q) s2[q & 3] += __builtin_amdgcn_exp2f(fmaf(v[q], kL2E, -cu));
        ls += (s2[0] + s2[1]) + (s2[2] + s2[3]);
        lc = cn;
      } else {
        const float mu = (mn > -kInf) ? mn : 0.0f;
        ls *= (mn > -kInf && lm > -kInf) ? __expf(lm - mn) : 1.0f;
        float s1 = 0.0f;
#pragma unroll
        for (int q = 0; q < kVals; ++q) s1 += __expf(v[q] - mu);
        ls += s1;
      }
      lm = mn;
    }

    if (pl.kA == 1 || pl.kB == 1) {
      // a lane whose maximum beats its best so far finds the first position
      // of that maximum (ids grow with q in a lane and with the tiles a wave
      // takes, so the earliest one is the lowest id); rare after a few tiles
      const uint32_t lk = f2key(lmax);
      if (__builtin_amdgcn_ballot_w64(lk > arg_key) != 0ull) {
        if (lk > arg_key) {
          int first = kVals;
#pragma unroll
          for (int q = kVals - 1; q >= 0; --q)
            if (v[q] == lmax && (vec || elem_index<E>(tile_base, q) < j.V)) first = q;
          if (first < kVals) {
            arg_key = lk;
            arg_id = elem_index<E>(tile_base, first);
          }
        }
      }
    }
    if (pl.kA > 1) list_tile<E>(v, g, lmax, tile_base, j.V, vec, LA, shvA, sh, sh.pool[0]);
    if (pl.kB > 1) list_tile<E>(v, g, lmax, tile_base, j.V, vec, LB, shvB, sh, sh.pool[1]);
  };
  const bool pf = j.aligned && j.V >= kSelTile;  // full tiles exist: element 0 starts one
  const int tf_end = pf ? min(t_end, j.V / kSelTile) : t_begin;  // this segment's full tiles
  // Tiles go to waves as they need them (a wave that is ahead takes more): the
  // first round gives wave w tile t_begin + w, later ones come from an LDS
  // counter. Claims increase, so at most one wave draws the row's partial last
  // tile (the only tile in [tf_end, t_end)).
  auto claim = [&]() __attribute__((always_inline)) {
    int c = 0;
    if (l == 0) c = atomicAdd(&sh.next_tile, 1);
    return __builtin_amdgcn_readfirstlane(c);
  };
  const int t0 = t_begin + w;
  int ta = t0;
  int tb = pf ? claim() : t_end;
  Raw<E> A, Bf;
  if (pf) {
    issue(A, ta);
    issue(Bf, tb);
  }
  // First round: the maxima of every wave's first two tiles (both buffers),
  // where they are full ones. The k-th largest lane maximum over the
  // workgroup bounds each list's k-th key from below (k distinct values reach
  // it) and is the pools' starting bound; two tiles make it tighter, which
  // saves more extraction later than the wait for the second one costs. (A
  // key of 0 stands for no value; a bound of 0 means no bound yet.)
  {
    uint32_t key0 = 0u;
    if (t0 < tf_end) {
      float v[kVals], g[kGroups], lmax;
      unpack_raw<E>(A, rowp, v, Tl);
      tile_maxima(v, g, lmax);
      if (tb < tf_end) {  // the second buffer's tile too (uniform per wave)
        float v2[kVals], g2[kGroups], lmax2;
        unpack_raw<E>(Bf, rowp, v2, Tl);
        tile_maxima(v2, g2, lmax2);
        lmax = __builtin_elementwise_maximum(lmax, lmax2);
      }
      key0 = f2key(lmax);
    } else if (pf) {
      // the placeholder loads finish here, so that no path reaches the loop
      // below with the buffers' loads outstanding
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    // (a bound of 0 means fewer than k lanes held data: no bound yet)
    // The 16-bit prefix can fall below key(-inf), into keys of negative NaNs,
    // when the k-th lane maximum is -inf: key(-inf) is then the bound (only a
    // NaN, which fails the row anyway, lies below it).
    if (pl.kA > 1) {
      uint32_t tk = block_kth_u32(key0, pl.kA, NT, sh);
      if (tk != 0u && tk < kKeyNegInf) tk = kKeyNegInf;
      LA.set_thr((pl.TA == 1.0f || tk == 0u) ? tk : f2key(key2f(tk) / pl.TA));
    }
    if (pl.kB > 1) {
      uint32_t tk = block_kth_u32(key0, pl.kB, NT, sh);
      if (tk != 0u && tk < kKeyNegInf) tk = kKeyNegInf;
      LB.set_thr(tk);
    }
    if (threadIdx.x == 0) {
      atomicMax(&sh.thr[0], LA.thr);
      atomicMax(&sh.thr[1], LB.thr);
    }
  }
  if (pf) {
    // Two buffers in turn: process one, then refill it with a newly claimed
    // tile while the other one's loads are in flight. The buffer processed is
    // always the one holding the smaller tile index.
    while (ta < tf_end) {
      {
        float v[kVals], g[kGroups], lmax;
        unpack_raw<E>(A, rowp, v, Tl);
        tile_maxima(v, g, lmax);
        step(v, g, lmax, ta, true);
      }
      ta = claim();
      issue(A, ta);
      if (tb >= tf_end) break;
      {
        float v[kVals], g[kGroups], lmax;
        unpack_raw<E>(Bf, rowp, v, Tl);
        tile_maxima(v, g, lmax);
        step(v, g, lmax, tb, true);
      }
      tb = claim();
      issue(Bf, tb);
    }
  }
  // Element loads: the row's partial last tile, if this wave drew it, or every
  // tile of a row that is not 16-byte aligned or is shorter than a tile (then
  // the waves take them in turn).
  int tt = pf ? ((ta >= tf_end && ta < t_end) ? ta : ((tb >= tf_end && tb < t_end) ? tb : t_end))
              : t0;
  for (; tt < t_end; tt = pf ? t_end : tt + W) {
    float v[kVals], g[kGroups], lmax;
    load_tail<E>(rowp, tt * kSelTile, j.V, v, Tl);
    tile_maxima(v, g, lmax);
    step(v, g, lmax, tt, false);
  }

  // this wave's log-sum-exp partial (Mw, Sw): Sw = sum of exp(x - Mw)
  float Mw = -kInf, Sw = 0.0f;
  if (j.lse) {
    const float s_l = (!huge && lm > -kInf) ? ls * __builtin_amdgcn_exp2f(-fmaf(lm, kL2E, -lc)) : ls;
    Mw = wave_max_dpp(lm);
    Sw = wave_sum_dpp((lm > -kInf && Mw > -kInf) ? s_l * __expf(lm - Mw) : 0.0f);
  }
  const bool bad = __ballot(bad_l) != 0ull;
  const bool fin = __ballot(fin_l) != 0ull;
  uint64_t best = 0ull;
  if (pl.kA == 1 || pl.kB == 1) best = wave_max_u64_dpp(arg_id >= 0 ? pack(arg_key, arg_id) : 0ull);
  if (l == 0) {
    sh.wm[w] = Mw;
    sh.ws[w] = Sw;
    sh.best[0][w] = pl.kA == 1 ? best : 0ull;
    sh.best[1][w] = pl.kB == 1 ? best : 0ull;
    uint32_t f = bad ? kMetaBadLogits : 0u;
    if (fin) f |= kMetaHasFinite;
    if (f) atomicOr(&sh.flags, f);
  }
  __syncthreads();

  const size_t slot = static_cast<size_t>(row) * j.nseg + seg;
  // A row read whole by this workgroup whose draw needs nothing beyond its
  // candidates (greedy, top-k <= 64, or rows that fail their checks, and every
  // row when the caller's hints promise that; no kept mask asked for) is
  // finished here, from LDS; the row kernel then skips it, or is not launched.
  // A list whose pool overflowed is then rebuilt by a rescan of the row. Other
  // segments hand their lists and partials on through the workspace.
  const bool hinted = (j.hints & (VS_HINT_SMALL_TOPK | VS_HINT_ALL_GREEDY)) != 0u;
  const bool finish = j.nseg == 1 && !j.out_mask &&
                      (!j.sample || hinted || pl.c.mode == kModeGreedy ||
                       pl.c.mode == kModeKFast || pl.c.mode == kModeInvalid);
  uint32_t meta = sh.flags;
  if (finish) {
    // A list whose pool overflowed is rebuilt by a rescan of the row (every
    // wave). Then the waves split the closing work: wave 0 sorts each list's
    // best entries in registers; wave 1 reduces the row totals; the others
    // compute the draw's exponential noise of list A's entries that reach the
    // final bound, by pool position. After one barrier wave 0 draws and writes
    // the row; the other waves are done.
    const bool rsA = pl.kA > 1 && (sh.ovf[0] || sh.merge_n[0] > kPoolCap);
    const bool rsB = pl.kB > 1 && (sh.ovf[1] || sh.merge_n[1] > kPoolCap);
    if (rsA || rsB) {  // rare: one copy of the rescan serves both lists
#pragma unroll 1
      for (int li = 0; li < 2; ++li) {
        if (li == 0 ? rsA : rsB)
          // (Tl is 1 in a sampling call and TA is 1 in a log-prob call: the
          // product is the one of them that applies, exactly)
          rescan_list<E>(rowp, j.V, j.aligned, (li == 0 ? pl.TA : 1.0f) * Tl, W, sh.stage,
                         sh.srt[li]);
      }
    }
    const bool noise = j.sample && pl.kA > 1 && !rsA && W > 2;  // the table is filled
    const int wt = W > 1 ? 1 : 0;                               // the wave reducing the totals
    uint64_t LA = 0ull, LB = 0ull;
    int nA = 0, nB = 0;
    if (w == 0) {
      if (pl.kA > 1) {
        int cnt = pl.kA;
        if (rsA)
          LA = sh.srt[0][l];
        else if (noise)
          LA = wave_top_of_pool<true>(sh.pool[0], sh.merge_n[0], sh.thr[0], sh.stage[0], &cnt);
        else
          LA = wave_top_of_pool<false>(sh.pool[0], sh.merge_n[0], sh.thr[0], sh.stage[0], &cnt);
        nA = cnt < pl.kA ? cnt : pl.kA;
      }
      if (pl.kB > 1) {
        int cnt = pl.kB;
        LB = rsB ? sh.srt[1][l]
                 : wave_top_of_pool<false>(sh.pool[1], sh.merge_n[1], sh.thr[1], sh.stage[1], &cnt);
        nB = cnt < pl.kB ? cnt : pl.kB;
      }
    }
    if (w == wt) {
      const float mi = l < W ? sh.wm[l] : -kInf;
      const float M = wave_max_dpp(mi);
      const float S = wave_sum_dpp((j.lse && mi > -kInf) ? sh.ws[l] * __expf(mi - M) : 0.0f);
      const uint64_t bA = (pl.kA == 1) ? wave_max_u64_dpp(l < W ? sh.best[0][l] : 0ull) : 0ull;
      const uint64_t bB = (pl.kB == 1) ? wave_max_u64_dpp(l < W ? sh.best[1][l] : 0ull) : 0ull;
      if (l == 0) {
        sh.tot_m = M;
        sh.tot_s = S;
        sh.tot_b[0] = bA;
        sh.tot_b[1] = bB;
      }
    }
    if (noise && w >= 2) {
      const uint64_t rs = row_stream(pl.c.seed, row);
      const uint32_t thr = sh.thr[0];
      const int n = sh.merge_n[0];
      for (int i = (w - 2) * kWave + l; i < n; i += (W - 2) * kWave) {
        const uint64_t e = sh.pool[0][i];
        if (pkey(e) >= thr) sh.q[i] = -log(uniform_of(rs, pid(e)));
      }
    }
    __syncthreads();
    if (w == 0) {
      double q = 1.0;
      if (noise) {
        q = (LA != 0ull) ? sh.q[tag_pos(LA)] : 1.0;
        LA = untag_entry(LA);
      }
      const float M = sh.tot_m, S = sh.tot_s;
      const uint64_t bA = sh.tot_b[0], bB = sh.tot_b[1];
      if (pl.kA > 1) meta |= static_cast<uint32_t>(nA);
      if (pl.kB > 1) meta |= static_cast<uint32_t>(nB) << kMetaCountBShift;
      if (pl.kA == 1 && bA) meta |= 1u;
      if (pl.kB == 1 && bB) meta |= 1u << kMetaCountBShift;
      sh.stage[0][l] = __double_as_longlong(q);  // the noise by lane, for the draw
      wave_lds_wait();
      finish_row<E>(j, row, pl, meta, LA, nA, LB, nB, M, S, bA, bB,
                    noise ? reinterpret_cast<const double*>(sh.stage[0]) : nullptr);
      if (l == 0) j.meta[slot] = meta | kMetaFinal;
    }
    if (j.full_in_select) {  // every wave, wave 0 once the row's outputs are written
      const bool bad = (meta & kMetaBadLogits) || !(meta & kMetaHasFinite);
      const float nanv = __builtin_nanf("");
      const float M = bad ? nanv : sh.tot_m;
      const float logS = bad ? nanv : logf(sh.tot_s);
      write_full_row<E, true>(j, rowp, j.out_full + static_cast<int64_t>(row) * j.ld_out, t_begin, t_end, M,
                              logS, Tl, &sh.next_out);
    }
    return;
  }
  uint32_t kthA = 0u, kthB = 0u;
  int nA = 0, nB = 0;
  // the segment totals, by the last wave while the others start the merge
  if (w == W - 1) {
    const float mi = l < W ? sh.wm[l] : -kInf;
    const float M = wave_max_dpp(mi);
    const float S = wave_sum_dpp((j.lse && mi > -kInf) ? sh.ws[l] * __expf(mi - M) : 0.0f);
    uint64_t bA = 0ull, bB = 0ull;
    if (pl.kA == 1) bA = wave_max_u64_dpp(l < W ? sh.best[0][l] : 0ull);
    if (pl.kB == 1) bB = wave_max_u64_dpp(l < W ? sh.best[1][l] : 0ull);
    if (l == 0) {
      sh.tot_m = M;
      sh.tot_s = S;
      sh.tot_b[0] = bA;
      sh.tot_b[1] = bB;
    }
  }
  if (pl.kA > 1) nA = merge_list(sh, 0, pl.kA, W, true, &kthA);
  if (pl.kB > 1) nB = merge_list(sh, 1, pl.kB, W, true, &kthB);
  __syncthreads();  // the totals are visible to every wave
  if (pl.kA > 1) meta |= (nA < 0) ? kMetaOverflowA : static_cast<uint32_t>(nA);
  if (pl.kB > 1) meta |= (nB < 0) ? kMetaOverflowB : (static_cast<uint32_t>(nB) << kMetaCountBShift);
  const float M = sh.tot_m, S = sh.tot_s;
  const uint64_t bA = sh.tot_b[0], bB = sh.tot_b[1];
  if (pl.kA == 1 && bA) meta |= 1u;
  if (pl.kB == 1 && bB) meta |= 1u << kMetaCountBShift;
  if (w == 0 && l == 0) {
    if (j.lse) j.lpart[slot] = LsePart{M, S};
    if (pl.kA == 1) {
      if (bA) j.candA[slot * kSelCap] = bA;
      j.kthA[slot] = pkey(bA);  // the segment maximum: its 1st-largest key
    }
    if (pl.kB == 1) {
      if (bB) j.candB[slot * kSelCap] = bB;
      j.kthB[slot] = pkey(bB);
    }
    j.meta[slot] = meta;
  }
  // the lists' candidates, for the row kernel
  for (int i = threadIdx.x; i < nA; i += NT) j.candA[slot * kSelCap + i] = sh.top[0][i];
  for (int i = threadIdx.x; i < nB; i += NT) j.candB[slot * kSelCap + i] = sh.top[1][i];
  if (threadIdx.x == 0) {
    if (pl.kA > 1) j.kthA[slot] = kthA;
    if (pl.kB > 1) j.kthB[slot] = kthB;
  }
}

// The greedy call with the full log-softmax written, one read of the logits:
// one 1024-thread workgroup per row keeps the whole row on chip, 23 of each
// thread's 16-byte vectors in registers and 9 in LDS (rows of 94,209 to
// 131,072 fp32 values: the register part is then always whole), so the write
// reads nothing again (the streaming pass re-reads each row for it, mostly
// from beyond L2). Vector g = r * 1024 + t is thread t's r-th. Each thread
// forms its own maximum and sum of exponentials (the streaming pass's shifted
// base-2 form; a NaN or +inf value leaves a NaN sum), and each wave bounds the
// top-k: the k-th largest of its threads' maxima, and the ceil(k/16)-th (k
// values reach the larger of the first's maximum over the waves and the
// second's minimum). One barrier combines them; the log-softmax
// (x - M) - log S is written from the resident values, the values at or above
// the bound are gathered in LDS and the threads whose maximum is M find the
// argmax (lowest id among equal values); after a second barrier one wave keeps
// the k best of the gathered values by sorts and merges 64 at a time (with
// more than kResPool of them, k rounds of a block maximum over the row read
// again, below the last one taken). The outputs and their edge cases are the
// streaming pass's for greedy rows.
constexpr int kResT = 1024;
constexpr int kResW = kResT / kWave;
constexpr int kResReg = 23;  // 16-byte vectors a thread keeps in registers
constexpr int kResLds = 9;   // and in LDS
constexpr int kResFirst = 14;  // register vectors loaded with the LDS part's
constexpr int kResPool = 1024;
constexpr int kResMinV = kResReg * 4 * kResT + 1;          // 94,209 values
constexpr int kResMaxV = (kResReg + kResLds) * 4 * kResT;  // 131,072 values
struct ResSh {
  f32x4 lv[kResLds * kResT];  // 144 KB
  uint64_t pool[kResPool];
  uint64_t wx[kResW];
  float wm[kResW], ws[kResW];
  uint32_t wta[kResW], wtb[kResW];
  int pool_n, amin;
};
// (non-temporal: the row is read once; measured 3 % faster than plain loads)
__device__ __forceinline__ f32x4 res_load(const float* p) {
  const uint4 u = load16_stream(p);
  f32x4 x;
  x.x = __uint_as_float(u.x);
  x.y = __uint_as_float(u.y);
  x.z = __uint_as_float(u.z);
  x.w = __uint_as_float(u.w);
  return x;
}
__device__ __forceinline__ float res_max4(const f32x4& x) {
  return fmaxf(fmaxf(x.x, x.y), fmaxf(x.z, x.w));
}
// sum over the vector of 2^(x log2 e - c), or exp(x - c) in huge mode
template <bool kHuge>
__device__ __forceinline__ float res_exp4(const f32x4& x, float c) {
  if (kHuge) return (__expf(x.x - c) + __expf(x.y - c)) + (__expf(x.z - c) + __expf(x.w - c));
  return (__builtin_amdgcn_exp2f(fmaf(x.x, kL2E, -c)) + __builtin_amdgcn_exp2f(fmaf(x.y, kL2E, -c))) +
         (__builtin_amdgcn_exp2f(fmaf(x.z, kL2E, -c)) + __builtin_amdgcn_exp2f(fmaf(x.w, kL2E, -c)));
}

__global__ __launch_bounds__(kResT) void k_select_resident(Job j) {
  __shared__ ResSh sh;
  const int row = blockIdx.x;
  const int t = static_cast<int>(threadIdx.x), ln = lane();
  const int wv = __builtin_amdgcn_readfirstlane(t / kWave);
  const float* rowp = static_cast<const float*>(j.logits) + static_cast<int64_t>(row) * j.ld;
  const int nvec = j.V / 4;
  const float nanv = __builtin_nanf("");
  const int kl = j.k_lp;
  // the LDS part's loads first (their registers are free again once stored)
  f32x4 tmp[kResLds];
  // (vectors past the row load its last one and read as -inf when used: a
  // value written over a load in flight would wait for it)
#pragma unroll
  for (int r = 0; r < kResLds; ++r) tmp[r] = res_load(rowp + 4 * min((kResReg + r) * kResT + t, nvec - 1));
  f32x4 rv[kResReg];
#pragma unroll
  for (int r = 0; r < kResFirst; ++r) rv[r] = res_load(rowp + 4 * (r * kResT + t));
  // this thread's maximum m and sum s of 2^(x log2 e - c), c = fl(m log2 e),
  // taken vector by vector as the loads land (a larger maximum rescales s by
  // 2^(c_old - c_new)); a NaN value, or m = +inf, leaves s NaN
  float m = -kInf, cs = -kInf, s = 0.0f;
  const auto acc = [&](const f32x4& x) __attribute__((always_inline)) {
    const float mn = fmaxf(m, res_max4(x));
    const float cn = mn * kL2E;
    const bool fin = mn > -kInf;
    s *= fin ? __builtin_amdgcn_exp2f(cs - cn) : 1.0f;
    s += res_exp4<false>(x, fin ? cn : 0.0f);
    m = mn;
    cs = cn;
  };
#pragma unroll
  for (int r = 0; r < kResLds; ++r) {
    f32x4 x = tmp[r];
    if ((kResReg + r) * kResT + t >= nvec) x.x = x.y = x.z = x.w = -kInf;
    acc(x);
    sh.lv[r * kResT + t] = x;  // (each thread reads back its own)
  }
  // (the values above are taken and stored here, before the remaining loads,
  // so their registers are free for them)
  asm volatile("" : "+v"(m), "+v"(s), "+v"(cs) : : "memory");
#pragma unroll
  for (int r = kResFirst; r < kResReg; ++r) rv[r] = res_load(rowp + 4 * (r * kResT + t));
  if (t == 0) {
    sh.pool_n = 0;
    sh.amin = 0x7fffffff;
  }
#pragma unroll
  for (int r = 0; r < kResReg; ++r) {
    acc(rv[r]);
    // (each vector's terms as it lands, not after the last one)
    asm volatile("" : "+v"(m), "+v"(s), "+v"(cs));
  }
  // s relative to m; with a maximum of 2^120 or more in the wave (m log2 e
  // near overflow) the sum again as exp(x - m)
  if (__ballot(fabsf(m) >= 0x1p120f && fabsf(m) < kInf) != 0ull) {
    const float cu = m > -kInf ? m : 0.0f;
    float s2[2] = {0.0f, 0.0f};
#pragma unroll
    for (int r = 0; r < kResReg; ++r) s2[r & 1] += res_exp4<true>(rv[r], cu);
#pragma unroll 3
    for (int r = 0; r < kResLds; ++r) s2[r & 1] += res_exp4<true>(sh.lv[r * kResT + t], cu);
    s = s2[0] + s2[1];
  } else if (m > -kInf) {
    s *= __builtin_amdgcn_exp2f(-fmaf(m, kL2E, -cs));
  }
  {
    const float wm = wave_max(m);
    const float ws = wave_sum((m > -kInf) ? s * __expf(m - wm) : s);
    uint32_t ta = 0u, tb = 0u;
    if (kl > 0) {
      const uint32_t key = f2key(m);
      ta = wave_kth_largest(key, kl);
      tb = wave_kth_largest(key, (kl + kResW - 1) / kResW);
    }
    if (ln == 0) {
      sh.wm[wv] = wm;
      sh.ws[wv] = ws;
      sh.wta[wv] = ta;
      sh.wtb[wv] = tb;
    }
  }
  __syncthreads();
  const float wmi = ln < kResW ? sh.wm[ln] : -kInf;
  const float M = wave_max(wmi);
  const float wsi = ln < kResW ? sh.ws[ln] : 0.0f;
  const float S = wave_sum((wmi > -kInf) ? wsi * __expf(wmi - M) : wsi);
  const uint32_t tau = kl > 0 ? max(wave_max(ln < kResW ? sh.wta[ln] : 0u),
                                    wave_min(ln < kResW ? sh.wtb[ln] : 0xffffffffu))
                              : 0u;
  const bool rowbad = __builtin_isnan(S) || !(M > -kInf) || !(M < kInf);
  const float Mo = rowbad ? nanv : M;
  const float logS = rowbad ? nanv : logf(S);
  // the argmax: the lowest id holding M, from the threads whose maximum it is
  if (!rowbad && m == M) {
    int aid = 0x7fffffff;
#pragma unroll 1
    for (int r = kResLds - 1; r >= 0; --r) {
      const f32x4 x = sh.lv[r * kResT + t];
      const int id = 4 * ((kResReg + r) * kResT + t);
      aid = x.w == M ? id + 3 : aid;
      aid = x.z == M ? id + 2 : aid;
      aid = x.y == M ? id + 1 : aid;
      aid = x.x == M ? id : aid;
    }
#pragma unroll
    for (int r = kResReg - 1; r >= 0; --r) {
      const int id = 4 * (r * kResT + t);
      aid = rv[r].w == M ? id + 3 : aid;
      aid = rv[r].z == M ? id + 2 : aid;
      aid = rv[r].y == M ? id + 1 : aid;
      aid = rv[r].x == M ? id : aid;
    }
    atomicMin(&sh.amin, aid);
  }
  // the candidates for the top-k log-probs
  const bool gather = kl > 0 && !rowbad;
  const float tauf = key2f(tau);
  const auto take = [&](const f32x4& x, int g) __attribute__((always_inline)) {
    // (four compares: a maximum here would be the first pass's, kept live)
    if (((x.x >= tauf) | (x.y >= tauf) | (x.z >= tauf) | (x.w >= tauf)) && g < nvec) {
      const float e[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (e[q] >= tauf) {
          const int at = atomicAdd(&sh.pool_n, 1);
          if (at < kResPool) sh.pool[at] = pack(f2key(e[q]), 4 * g + q);
        }
      }
    }
  };
  // the log-softmax from the resident values
  float* orow = j.out_full + static_cast<int64_t>(row) * j.ld_out;
#pragma unroll
  for (int r = 0; r < kResReg; ++r) {
    const int g = r * kResT + t;
    if (gather) take(rv[r], g);
    f32x4 o;
    o.x = (rv[r].x - Mo) - logS;
    o.y = (rv[r].y - Mo) - logS;
    o.z = (rv[r].z - Mo) - logS;
    o.w = (rv[r].w - Mo) - logS;
    __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(orow + 4 * g));
  }
#pragma unroll 3
  for (int r = 0; r < kResLds; ++r) {
    const int g = (kResReg + r) * kResT + t;
    const f32x4 x = sh.lv[r * kResT + t];
    if (gather) take(x, g);
    if (g < nvec) {
      f32x4 o;
      o.x = (x.x - Mo) - logS;
      o.y = (x.y - Mo) - logS;
      o.z = (x.z - Mo) - logS;
      o.w = (x.w - Mo) - logS;
      __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(orow + 4 * g));
    }
  }
  __syncthreads();
  // the row's outputs (a greedy row's, as the streaming pass writes them)
  // (by wave 1: wave 0 keeps the top-k meanwhile)
  if (t == kWave) {
    const RowCfg c = load_cfg(row, j.V, j.T, j.k, j.p, j.mp, j.seeds);
    int status = c.status | (rowbad ? VS_ROW_BAD_LOGITS : 0);
    if (status == 0) {
      if ((j.hints & VS_HINT_ALL_GREEDY) && c.mode != kModeGreedy) status = VS_ROW_HINT_VIOLATED;
      if ((j.hints & VS_HINT_NO_GREEDY) && c.mode == kModeGreedy) status = VS_ROW_HINT_VIOLATED;
      if ((j.hints & VS_HINT_SMALL_TOPK) && c.mode != kModeGreedy && c.mode != kModeKFast)
        status = VS_ROW_HINT_VIOLATED;
    }
    const int32_t id = status ? -1 : sh.amin;
    j.rlse[row] = rowbad ? make_float2(nanv, nanv) : make_float2(M, logS);
    j.desc[row].mode = kRowDone;
    j.out_ids[row] = id;
    if (j.out_kept) j.out_kept[row] = status ? 0 : 1;
    if (j.out_status) j.out_status[row] = status;
    if (j.tok_sampled) j.out_tok_lp[row] = (id < 0 || rowbad) ? nanv : (M - M) - logS;
  }
  if (kl == 0) return;
  if (rowbad) {
    if (t < kl) {
      j.out_lp_ids[static_cast<size_t>(row) * kl + t] = -1;
      j.out_lp[static_cast<size_t>(row) * kl + t] = nanv;
    }
    return;
  }
  const int np = sh.pool_n;
  if (np <= kResPool) {  // uniform
    if (wv != 0) return;
    uint64_t top = 0ull;  // the 64 best so far, descending
    for (int c0 = 0; c0 < np; c0 += kWave) {
      uint64_t v = c0 + ln < np ? sh.pool[c0 + ln] : 0ull;
      v = wave_sort_u64<false>(v);
      top = wave_merge_top_u64(top, v);
    }
    if (ln < kl) {
      j.out_lp_ids[static_cast<size_t>(row) * kl + ln] = top ? pid(top) : -1;
      j.out_lp[static_cast<size_t>(row) * kl + ln] = top ? (key2f(pkey(top)) - M) - logS : nanv;
    }
    return;
  }
  // rare (many equal values): one block maximum a rank, below the last
  uint64_t last = ~0ull;
  for (int q = 0; q < kl; ++q) {
    uint64_t b = 0ull;
    for (int i = t; i < j.V; i += kResT) {
      const uint64_t pk = pack(f2key(rowp[i]), i);
      b = (pk < last && pk > b) ? pk : b;
    }
    const uint64_t wb = wave_max(b);
    if (ln == 0) sh.wx[wv] = wb;
    __syncthreads();
    b = wave_max(ln < kResW ? sh.wx[ln] : 0ull);
    __syncthreads();  // (the slots are written again next rank)
    if (t == 0) {
      j.out_lp_ids[static_cast<size_t>(row) * kl + q] = b ? pid(b) : -1;
      j.out_lp[static_cast<size_t>(row) * kl + q] = b ? (key2f(pkey(b)) - M) - logS : nanv;
    }
    last = b;
  }
}

}  // namespace

hipError_t launch_select(const Job& j, hipStream_t st) {
  // greedy rows with the full log-softmax written, small enough to keep on
  // chip: one read (k_select_resident)
  if (j.full_in_select && j.sample && (j.hints & VS_HINT_ALL_GREEDY) && j.dt == VS_F32 &&
      j.V % 4 == 0 && j.V >= kResMinV && j.V <= kResMaxV && j.aligned && j.full_vec && !j.pen && !j.out_mask &&
      j.k_lp <= kWave && !j.lpT) {
    hipLaunchKernelGGL(k_select_resident, dim3(j.B), dim3(kResT), 0, st, j);
    return hipGetLastError();
  }
  const int grid = xcd_grid(j.B, j.nseg);
  const dim3 block(kWave * j.nwave);
  const size_t lds = 0;
  // Logits read once (no later kernel reads them again: no full log-softmax
  // output, and no full-vocabulary rows) stream past the caches, and so do
  // logits too large for the last-level cache to keep for a second reader
  // (more than half of its 256 MB).
  const int64_t bytes = static_cast<int64_t>(j.B) * j.V * (j.dt == VS_F32 ? 4 : 2);
  // When the pass also writes the full log-softmax it reads each row a second
  // time right away: the first read then goes through the caches (measured
  // faster overall than streaming it past them).
  const bool stream = !j.full_in_select &&
                      (bytes > (int64_t{128} << 20) ||
                       (!j.out_full &&
                        (!j.sample || (j.hints & (VS_HINT_NO_FULLVOCAB | VS_HINT_ALL_GREEDY |
                                                  VS_HINT_SMALL_TOPK)))));
  // (instances with the log-prob temperature only for calls that pass one)
  const bool scaled = j.lpT != nullptr && !j.sample;
  if (j.dt == VS_F32) {
    if (scaled && stream)
      hipLaunchKernelGGL((k_select<float, true, true>), dim3(grid), block, lds, st, j);
    else if (scaled)
      hipLaunchKernelGGL((k_select<float, false, true>), dim3(grid), block, lds, st, j);
    else if (stream)
      hipLaunchKernelGGL((k_select<float, true, false>), dim3(grid), block, lds, st, j);
    else
      hipLaunchKernelGGL((k_select<float, false, false>), dim3(grid), block, lds, st, j);
  } else {
    if (scaled && stream)
      hipLaunchKernelGGL((k_select<uint16_t, true, true>), dim3(grid), block, lds, st, j);
    else if (scaled)
      hipLaunchKernelGGL((k_select<uint16_t, false, true>), dim3(grid), block, lds, st, j);
    else if (stream)
      hipLaunchKernelGGL((k_select<uint16_t, true, false>), dim3(grid), block, lds, st, j);
    else
      hipLaunchKernelGGL((k_select<uint16_t, false, false>), dim3(grid), block, lds, st, j);
  }
  return hipGetLastError();
}

}  // namespace vsk
