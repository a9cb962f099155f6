// What one ABI call asks of the kernels, and the per-row plan all kernels
// derive from it identically.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "vs_device.h"

namespace vsk {

constexpr int kSelTile = 2048;    // one wave's tile in the streaming pass
constexpr int kSegMin = 4096;     // values per segment, at least (bounds the segment count)
constexpr int kSelMaxWaves = 16;  // waves per streaming-pass workgroup, at most
constexpr int kSelCap = 128;      // candidate slots per segment and list
constexpr int kGumTile = 4096;    // Gumbel tile: 256 threads x 16 values
constexpr int kFullTile = 4096;   // full log-softmax write tile
// Full-vocabulary top-p: fixed-point masses histogrammed over buckets of
// t = s - m (kFullPerUnit buckets per unit, bucket 0 holding the largest s),
// and the ids of the bucket holding the cut gathered into a list per row.
constexpr int kFullBuckets = 4096;
constexpr float kFullPerUnit = 128.0f;
constexpr int kFullListCap = 8192;
constexpr int kFullSegMin = 4096;  // ids per segment of the histogram and gather passes, at least
static_assert(kFullSegMin >= kGumTile, "a histogram segment spans at least one Gumbel tile");

// Segment meta word (a segment is the run of tiles of one row that one
// streaming-pass workgroup reads).
constexpr uint32_t kMetaCountA = 0xffu;
constexpr int kMetaCountBShift = 8;
constexpr uint32_t kMetaBadLogits = 1u << 16;
constexpr uint32_t kMetaHasFinite = 1u << 17;
constexpr uint32_t kMetaOverflowA = 1u << 18;
constexpr uint32_t kMetaOverflowB = 1u << 19;
constexpr uint32_t kMetaFinal = 1u << 20;  // the streaming pass finished the row itself

// Row descriptor states (written for every row by the row kernel each call).
enum : uint32_t {
  kRowDone = 0,       // id final (or the row failed)
  kRowFullNone = 1,   // full vocabulary, no truncation: Gumbel kernels draw
  kRowFullMinP = 2,   // full vocabulary, min-p only
  kRowFullTopP = 3,   // full vocabulary, top-p cut given by (tau, id_cut)
  kRowFull = 4,       // full vocabulary, the cut still to be found (heavy kernel)
  kRowFullListed = 5, // top-p cut (tau, id_cut) found in the row's list; the cut kernel drew
                      // from the list's kept entries and the gather pass's bests over the
                      // ids above the list's bucket (no Gumbel pass over the kept set)
};
// In a call whose gather pass draws (j.fdraw), the cut kernel finishes every
// full-vocabulary row, whatever its state above, and the Gumbel pass over the
// kept sets does not run.

// The top-p cut of a full-vocabulary row, found from its mass histogram.
// bucket and rem come from the first segment's gather workgroup; count and
// above_c are sums over all of the row's gather workgroups (zeroed by the row
// kernel with the histogram).
struct FullCut {
  int32_t bucket;     // the bucket holding the cut (-1: not found)
  uint32_t count;     // ids in that bucket
  uint64_t rem;       // mass still needed inside it (>= 1)
  uint64_t above_c;   // ids in the buckets above it
  uint64_t pad;
};

// Per-id terms of a full-vocabulary row: the relative weight e = E(s - m),
// the fixed-point mass W and the bucket of t = s - m; false for ids outside
// the kept candidates (e < min_p, or zero mass). The one definition every
// full-vocabulary kernel uses.
struct FullTerms {
  float m, mp;
  __device__ __forceinline__ bool mass(float s, uint64_t* w, int* bucket) const {
    float e;
    return mass_e(s, w, bucket, &e);
  }
  // the same, with e = E(s - m) itself
  __device__ __forceinline__ bool mass_e(float s, uint64_t* w, int* bucket, float* e_out) const {
    const float t = s - m;
    const float e = pinned_exp(t);
    *e_out = e;
    if (!(e >= mp)) return false;
    const uint64_t W = mass_of(e);
    if (W == 0) return false;
    *w = W;
    *bucket = bucket_of(t);
    return true;
  }
  __device__ __forceinline__ static int bucket_of(float t) {
    const int b = static_cast<int>(-t * kFullPerUnit);
    return b < kFullBuckets - 1 ? b : kFullBuckets - 1;
  }
};

// The rejection draw of full-vocabulary top-p rows: each histogram workgroup
// keeps the kCandM best Gumbel scores of its segment's candidates (every id of
// positive mass that passes min-p), and once the cut is known the first of
// the row's kCandM best that lies inside it is the draw.
constexpr int kCandM = 4;
struct GCand {
  double score;  // e / -log(u); negative: no candidate
  int32_t id;
  uint32_t key;  // ordered key of s = x / T
};

struct Job {
  const void* logits;
  int dt;  // vs_dtype
  int B, V;
  int64_t ld;
  int aligned;
  // sampling
  int sample;
  const float* T;
  const int32_t* k;
  const float* p;
  const float* mp;
  const uint64_t* seeds;
  uint32_t hints;
  int32_t* out_ids;
  int32_t* out_kept;
  uint32_t* out_mask;
  int32_t* out_status;
  // log-probabilities
  int lse;                 // log-sum-exp wanted
  int k_lp;                // top-k log-probs (0..64)
  const int32_t* tok;      // ids whose log-prob is wanted (vs_logprobs), or NULL
  int tok_sampled;         // the log-prob of the sampled id is wanted (fused call)
  float* out_tok_lp;
  int32_t* out_lp_ids;
  float* out_lp;
  float* out_full;
  int64_t ld_out;
  int32_t* out_lp_status;  // vs_logprobs status
  const float* lpT;        // [B] temperature of the log-probs (vs_logprobs_ex), or NULL
  // occurrence penalties applied by the streaming pass before it reads its
  // segment (vs_penalize_sample_logprobs); the logits are then written in place
  int pen;
  const int32_t* pen_pids;
  const int32_t* pen_poff;
  const int32_t* pen_oids;
  const int32_t* pen_ooff;
  const float* pen_pres;
  const float* pen_freq;
  const float* pen_rep;
  const int32_t* pen_ign;
  int32_t* out_pen_status;
  // full-vocabulary top-p (per row): mass histogram, the cut bucket's ids
  uint64_t* fhw;       // [B][kFullBuckets] masses
  uint64_t* flist;     // [B][kFullListCap] packed (key, id) of the cut bucket
  uint32_t* fcnt;      // [B] entries appended to flist (may exceed the capacity)
  FullCut* fcut;       // [B] the cut bucket and the mass needed inside it
  GCand* fcand;        // [B][ntile3][kCandM]: each histogram segment's best candidates
  int topp_reject;     // full-vocabulary top-p rows draw by rejection (no kept mask asked for)
  int fdraw;           // else the gather pass and the cut kernel draw them (no kept mask asked for)
  int fseg;            // segments per row of the histogram and gather passes
  int fseg_len;        // ids per segment (a multiple of 8)
  int full_in_select;      // the streaming pass writes out_full itself (it finishes every row)
  int full_chain;          // the full-vocabulary passes run: the streaming pass clears their
                           // counters and the cut kernel does the row kernel's work (the
                           // row kernel is not launched)
  int full_vec;            // out_full rows take 16-byte stores
  // workspace; streaming-pass geometry
  int ntile;  // tiles per row
  int nseg;   // segments per row (<= ceil(V / kSegMin), the workspace's slots per row)
  int tps;    // tiles per segment
  int nwave;  // waves per streaming-pass workgroup
  int ntile3;
  int gseg;  // Gumbel-pass tiles per workgroup
  uint32_t* meta;
  uint64_t* candA;
  uint64_t* candB;
  uint32_t* kthA;   // per segment: exact k-th key of list A's candidates (0: fewer than k)
  uint32_t* kthB;
  LsePart* lpart;
  float2* rlse;
  RowDesc* desc;
  GPart* gpart;
};

struct Plan {
  RowCfg c;
  int kA;       // list A: 1 = argmax of x, 2..64 = top-k of s = x / TA, 0 = none
  float TA;
  int kB;       // list B: top-k of x for log-probs, when list A cannot serve
  bool shared;  // the log-prob top-k comes from list A
};

__device__ __forceinline__ Plan plan_row(const Job& j, int row) {
  Plan pl;
  pl.kB = 0;
  pl.shared = true;
  if (j.sample) {
    pl.c = load_cfg(row, j.V, j.T, j.k, j.p, j.mp, j.seeds);
    const bool fast = pl.c.mode == kModeKFast && !(j.hints & VS_HINT_ALL_GREEDY);
    pl.kA = fast ? pl.c.k : 1;
    pl.TA = fast ? pl.c.T : 1.0f;
    if (j.lse && j.k_lp > 0) {
      pl.shared = (pl.kA == 1) ? (j.k_lp == 1) : (pl.TA == 1.0f && j.k_lp <= pl.kA);
      pl.kB = pl.shared ? 0 : j.k_lp;
    }
  } else {
    pl.c = RowCfg{kModeInvalid, 0, 1.0f, 0, 1.0f, 0.0f, 0ull};
    pl.kA = j.k_lp;
    pl.TA = 1.0f;
  }
  return pl;
}

// The route of a sampling row that the streaming pass did not finish: a
// full-vocabulary row (mode kModeFull) whose checks pass goes through the
// histogram, gather and cut passes with m = its largest s = x / T; any other
// row is the row kernel's. The checks are the row kernel's for such a row:
// no NaN or +inf logit and some finite one, an argmax found, no hint that
// rules the row out, and a finite m. The histogram and gather passes and the
// cut kernel each decide it with this one function from the same inputs (the
// row's parameters and the streaming pass's per-segment words). Called with
// every lane of the wave active (the segments' words are combined across it).
struct RowRoute {
  RowCfg c;
  float m;    // the largest s of a full-vocabulary row
  bool full;  // a full-vocabulary row whose checks pass
};
// The first 64 segments' words for route_row, one per lane: loads a caller
// issues ahead of its other loads, so that they return first.
struct RoutePre {
  uint32_t mt;  // the segment's meta word
  uint64_t v;   // its list-A slot 0 (the segment argmax when it found one)
};
__device__ __forceinline__ RoutePre route_preload(const Job& j, int row) {
  RoutePre p{0u, 0ull};
  const int ntile = j.nseg;
  const size_t s0 = static_cast<size_t>(row) * ntile;
  const int t = lane();
  if (t < ntile) {  // (the slot is read whether or not the segment found one)
    p.mt = j.meta[s0 + t];
    p.v = j.candA[(s0 + t) * kSelCap];
  }
  return p;
}
__device__ __forceinline__ RowRoute route_row(const Job& j, int row, const RoutePre& p) {
  RowRoute r;
  r.c = load_cfg(row, j.V, j.T, j.k, j.p, j.mp, j.seeds);
  r.m = 0.0f;
  r.full = false;
  if (r.c.mode != kModeFull) return r;  // uniform
  const int ntile = j.nseg;
  const size_t s0 = static_cast<size_t>(row) * ntile;
  uint32_t fl = p.mt;
  uint64_t top = (p.mt & kMetaCountA) ? p.v : 0ull;  // the row argmax: the best segment argmax
  for (int t = lane() + kWave; t < ntile; t += kWave) {
    const uint32_t mt = j.meta[s0 + t];
    const uint64_t v = j.candA[(s0 + t) * kSelCap];
    fl |= mt;
    if (mt & kMetaCountA) top = v > top ? v : top;
  }
  fl = wave_reduce(fl, [](uint32_t a, uint32_t b) { return a | b; });
  top = wave_max(top);
  const bool bad_logits = (fl & kMetaBadLogits) || !(fl & kMetaHasFinite);
  if (r.c.status || bad_logits || top == 0ull) return r;
  if (j.hints & (VS_HINT_ALL_GREEDY | VS_HINT_NO_FULLVOCAB | VS_HINT_SMALL_TOPK)) return r;
  const float x = key2f(pkey(top));
  const float m = (r.c.T == 1.0f) ? x : x / r.c.T;
  if (m == kInf) return r;  // x / T overflowed
  r.m = m;
  r.full = true;
  return r;
}

// The temperature the log-probs of a row are taken at: vs_logprobs_ex's per-row
// temperature when it is positive and finite, else 1 (never in a sampling
// call). Every read of the logits in the log-prob path divides by it, so that
// the log-softmax is that of s = x / T rounded to fp32.
__device__ __forceinline__ float lse_T(const Job& j, int row) {
  if (!j.lpT || j.sample) return 1.0f;
  const float t = j.lpT[row];
  return (t > 0.0f && t <= 3.40282347e38f) ? t : 1.0f;
}
__device__ __forceinline__ float lse_scaled(float x, float T) { return T == 1.0f ? x : x / T; }

struct WsLayout {
  int ntile, ntile3;
  size_t meta, candA, candB, kthA, kthB, desc, gpart, lpart, rlse, fhw, flist, fcnt, fcut, fcand,
      total;
};
// The workspace layout for B rows of V ids with nslot segment slots per row
// (the streaming pass uses min(nslot, its segment count) of them per row).
WsLayout ws_layout(int B, int V, int nslot);
// Segment slots per row that covers every device: one per kSegMin ids.
inline int ws_slots_any(int V) { return (V + kSegMin - 1) / kSegMin; }
// Streaming-pass segments per row on the current device.
int stream_segments(int B, int V);

hipError_t launch_select(const Job& j, hipStream_t st);
hipError_t launch_row_light(const Job& j, hipStream_t st);
hipError_t launch_row_full(const Job& j, hipStream_t st);
hipError_t launch_full_prep(const Job& j, hipStream_t st);
hipError_t launch_gumbel(const Job& j, hipStream_t st);
hipError_t launch_lse_full(const Job& j, hipStream_t st);
hipError_t launch_topp_decay(int B, float* top_p, const float* top_p_init, const float* decay,
                             const float* top_p_min, const int32_t* reset_ids,
                             const int32_t* sampled, int32_t* out_status, hipStream_t st);
hipError_t launch_seed_advance(int B, uint64_t* seeds, const int32_t* sampled, hipStream_t st);
hipError_t launch_slot_remap(int B, int B_src, const int32_t* remap, const void* src, void* dst,
                             int elem_bytes, int32_t* out_status, hipStream_t st);
hipError_t launch_penalize(void* logits, int dt, int B, int V, int64_t ld,
                           const int32_t* prompt_ids, const int32_t* prompt_off,
                           const int32_t* output_ids, const int32_t* output_off,
                           const float* presence, const float* frequency,
                           const float* repetition, const int32_t* prompt_ignore,
                           int32_t* out_status, hipStream_t st);

}  // namespace vsk
