// K3/K4: the Gumbel-max draw over full-vocabulary kept sets, and the full
// log-softmax write of vs_logprobs.
//
// K3 (grid: rows x runs of gseg 4096-id tiles, all of a row on one XCD; each
// run reports in its first tile's record, the others empty): for every id
// of the tile it recomputes s = x / T, tests membership (everything; e >=
// min_p; or for top-p "key > tau, or key == tau and id <= id_cut"), and for
// kept ids forms score = e / -log(u(seed, row, id)) with e = E(s - m). Each
// tile keeps its best (score desc, id asc) and its kept count. A thread skips
// the logarithm and the division for an id that provably scores below its
// best so far: -log u > 1 - u for u < 1, so 1 - u >= e / best (with margins
// for the rounding of both sides) means e / -log u < best; e <= 1 gives a
// first test before e itself is computed (an integer compare of the id's
// random word with a threshold derived from the bound, no floating point),
// a hardware-exponential upper bound on e a second one. Any kept id's score
// bounds the row's maximum from below, so each workgroup first scores one id
// per thread and shares the best (one barrier), and after each tile its waves
// share their bests again through LDS (plain stores and loads: a stale value
// is only a looser bound). Skipped ids cannot be the argmax, so the result is
// the exact one. The next tile's loads are issued before the current tile is
// scored, and rows at T = 1 take a copy of the loop without the division.
// K4 (one workgroup per row) reduces the tiles: the sampled id, the kept count
// and, in the fused call, the sampled id's log-probability. The argmax compares
// true ids, never thread or tile order, so the result does not depend on the
// partition (vllm.cpp pull request #1997, "The kernel (#1984)").
#include <type_traits>

#include "vs_device.h"
#include "vs_kernels.h"

namespace vsk {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = kGumTile / kThreads;  // 16
constexpr float kLog2E = 1.44269504088896340736f;

__device__ __forceinline__ bool full_row(uint32_t mode) {
  return mode == kRowFullNone || mode == kRowFullMinP || mode == kRowFullTopP;
}

template <typename E>
__global__ __launch_bounds__(kThreads) void k_gumbel_partial(Job j) {
  __shared__ double sd[kThreads / kWave];
  __shared__ int si[kThreads / kWave];
  __shared__ uint64_t swb[kThreads / kWave];  // each wave's best score bits so far
  int row, run;
  const int nrun = (j.ntile3 + j.gseg - 1) / j.gseg;
  if (!xcd_row_tile(blockIdx.x, j.B, nrun, &row, &run)) return;
  const RowDesc d = j.desc[row];
  if (!full_row(d.mode)) return;  // uniform over the block
  constexpr int EPV = Epv<E>::n;
  constexpr int NV = kPerThread / EPV;
  const float T = j.T ? j.T[row] : 1.0f;
  const float mp = j.mp ? j.mp[row] : 0.0f;
  const uint64_t rs = row_stream(j.seeds ? j.seeds[row] : 0ull, row);
  const E* rowp = static_cast<const E*>(j.logits) + static_cast<int64_t>(row) * j.ld;
  const int mwords = (j.V + 31) / 32;
  uint32_t* mask_row = j.out_mask ? j.out_mask + static_cast<size_t>(row) * mwords : nullptr;
  const int t0 = run * j.gseg;
  const int t1 = min(j.ntile3, t0 + j.gseg);
  const int wv = static_cast<int>(threadIdx.x) / kWave;

  double best = -1.0;
  int best_id = 0x7fffffff;
  // (1 + 2^-40) / (the largest kept id's score known here): an id whose 1 - u
  // reaches lim * e scores below it (infinite, so that no id is skipped,
  // until a score is known); skip: the random words that reach it for any e
  double lim = __builtin_inf();
  uint64_t skip = 0ull;
  float lim_up = __builtin_inff();  // a float at or above lim
  int kept = 0;

  // the 16-byte vectors of a tile this thread reads, when the tile is whole
  // and the row aligned
  const auto vec_of = [&](int tile) { return j.aligned && (tile + 1) * kGumTile <= j.V; };
  const auto first_id = [&](int tile, int i) {
    return tile * kGumTile + (i * kThreads + static_cast<int>(threadIdx.x)) * EPV;
  };

  // The draw's score of a kept id whose random word b passed the integer
  // test, unless a finer bound test shows it cannot beat the best; e < 0:
  // E(s - m) not computed yet.
  const auto score = [&](int id, float s, float e, uint64_t b) {
    const double u = uniform_of_bits(b);
    const double one_u = (1.0 - u) * (1.0 - 0x1p-50);  // rounded down past any rounding error
    if (one_u >= lim) return;                          // e <= 1: below the bound
    if (e < 0.0f) {
      // an upper bound on e from the hardware exponential first: for
      // s - m >= -87 the fp32 constant and product move the exponent by
      // at most 9e-6 (2^x by 6.3e-6 relative), the instruction adds
      // about 1 ulp, and 2^-16 covers both; below -87 e is 0
      const float eub = __builtin_amdgcn_exp2f((s - d.m) * kLog2E) * (1.0f + 0x1p-16f);
      if (one_u >= lim * static_cast<double>(eub)) return;  // below the bound
      e = pinned_exp(s - d.m);
    }
    if (one_u >= lim * static_cast<double>(e)) return;  // below the bound
    const double sc = static_cast<double>(e) / -log(u);  // as gumbel_score
    if (sc > best || (sc == best && id < best_id)) {
      best = sc;
      best_id = id;
      lim = fmin(lim, (1.0 + 0x1p-40) / best);
      skip = skip_below(lim);
      lim_up = up_of(lim);
    }
  };

  // Membership of the ids v[c] = s of ids j0 + c (c < n, n <= EPV) as a bit
  // mask; e[c] gets E(s - m) where membership needed it, else -1.
  const auto members = [&](int j0, int n, const float* v, float* e) {
    uint32_t km = 0;
    if (d.mode == kRowFullMinP) {  // uniform
#pragma unroll
      for (int c = 0; c < EPV; ++c) {
        e[c] = pinned_exp(v[c] - d.m);
        km |= (c < n && e[c] >= mp) ? 1u << c : 0u;
      }
    } else if (d.mode == kRowFullNone) {  // uniform
#pragma unroll
      for (int c = 0; c < EPV; ++c) {
        e[c] = -1.0f;
        km |= c < n ? 1u << c : 0u;
      }
    } else {
#pragma unroll
      for (int c = 0; c < EPV; ++c) {
        e[c] = -1.0f;
        const uint32_t key = f2key(v[c]);
        km |= (c < n && (key > d.tau || (key == d.tau && j0 + c <= d.id_cut))) ? 1u << c : 0u;
      }
    }
    return km;
  };

  // the workgroup's best so far into every thread's bound (scores are
  // nonnegative: their bits order as integers)
  const auto share = [&](bool barrier) {
    uint64_t wb = wave_max_u64_dpp(best >= 0.0 ? static_cast<uint64_t>(__double_as_longlong(best)) : 0ull);
    if (barrier) __syncthreads();
    if (lane() == 0) __hip_atomic_store(&swb[wv], wb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (barrier) __syncthreads();
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) {
      const uint64_t o = __hip_atomic_load(&swb[w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      wb = o > wb ? o : wb;
    }
    const double sbest = __longlong_as_double(static_cast<long long>(wb));
    if (sbest > 0.0 && (1.0 + 0x1p-40) / sbest < lim) {
      lim = (1.0 + 0x1p-40) / sbest;
      skip = skip_below(lim);
      lim_up = up_of(lim);
    }
  };

  const auto run_tiles = [&](auto div) {
    constexpr bool kDiv = decltype(div)::value;
    const auto scaled = [&](float x) { return kDiv ? x / T : x; };
    uint4 cur[NV];
    if (vec_of(t0)) {
#pragma unroll
      for (int i = 0; i < NV; ++i) cur[i] = *reinterpret_cast<const uint4*>(rowp + first_id(t0, i));
    }
    // First one id per thread, the first of its first vector: the workgroup
    // then starts from the best of up to 256 scores rather than each thread
    // from its own. (The id is scored again, and counted, with its tile.)
    {
      const int id = first_id(t0, 0);
      float v[EPV], e[EPV];
#pragma unroll
      for (int c = 0; c < EPV; ++c) v[c] = -kInf;
      if (id < j.V) {
        if (vec_of(t0)) {
          float x[EPV];
          unpack16(cur[0], x, rowp);
          v[0] = scaled(x[0]);
        } else {
          v[0] = scaled(to_f32(rowp[id]));
        }
      }
      const uint32_t km = members(id, id < j.V ? 1 : 0, v, e);
      if (km & 1u) {
        const uint64_t b = random_bits(rs, id);
        if (b >= skip) score(id, v[0], e[0], b);
      }
      share(true);
    }
    for (int tile = t0; tile < t1; ++tile) {
      const bool vec = vec_of(tile);
      uint4 nxt[NV];
      if (tile + 1 < t1 && vec_of(tile + 1)) {
#pragma unroll
        for (int i = 0; i < NV; ++i) nxt[i] = *reinterpret_cast<const uint4*>(rowp + first_id(tile + 1, i));
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int j0 = first_id(tile, i);
        const int n = min(EPV, max(0, j.V - j0));
        float v[EPV], e[EPV];
        if (vec) {
          unpack16(cur[i], v, rowp);
        } else {
#pragma unroll
          for (int c = 0; c < EPV; ++c) v[c] = (c < n) ? to_f32(rowp[j0 + c]) : -kInf;
        }
#pragma unroll
        for (int c = 0; c < EPV; ++c) v[c] = scaled(v[c]);
        const uint32_t km = members(j0, n, v, e);
        kept += __popc(km);
        // EPV divides 32: the vector's ids share one mask word
        if (mask_row && km) atomicOr(&mask_row[j0 >> 5], km << (j0 & 31));
        if (__ballot(km != 0u)) {  // uniform: some lane keeps an id here
          // the integer test for this vector, on the high halves of the
          // random words, from an upper bound on its ids' e (the
          // hardware-exponential bound of score at the vector's largest s,
          // at most 1; tighter than e <= 1 wherever that is small)
          float vmax = v[0];
#pragma unroll
          for (int c = 1; c < EPV; ++c) vmax = fmaxf(vmax, v[c]);
          const float veub =
              fminf(__builtin_amdgcn_exp2f((vmax - d.m) * kLog2E) * (1.0f + 0x1p-16f), 1.0f);
          const uint32_t vskip = skip_hi(lim_up, veub);
          uint32_t need = 0;
#pragma unroll
          for (int c = 0; c < EPV; ++c)
            need |= ((km >> c) & 1u) && random_hi(rs, j0 + c) >= vskip ? 1u << c : 0u;
          if (__ballot(need != 0u)) {  // rare once a bound is known (the words are formed again)
#pragma unroll
            for (int c = 0; c < EPV; ++c)
              if ((need >> c) & 1u) score(j0 + c, v[c], e[c], random_bits(rs, j0 + c));
          }
        }
      }
      share(false);
#pragma unroll
      for (int i = 0; i < NV; ++i) cur[i] = nxt[i];
    }
  };
  if (T == 1.0f)  // uniform; x / 1 is x
    run_tiles(std::false_type{});
  else
    run_tiles(std::true_type{});

  const double bb = block_max(best, sd);
  const int bid = block_min(best == bb ? best_id : 0x7fffffff, si);
  const int bk = block_sum(kept, si);
  if (threadIdx.x == 0) {
    GPart* g = j.gpart + static_cast<size_t>(row) * j.ntile3;
    g[t0] = GPart{bb, bid, bk};
    for (int t = t0 + 1; t < t1; ++t) g[t] = GPart{-1.0, 0x7fffffff, 0};
  }
}

template <typename E>
__global__ __launch_bounds__(kThreads) void k_gumbel_final(Job j) {
  __shared__ double sd[kThreads / kWave];
  __shared__ int si[kThreads / kWave];
  const int row = blockIdx.x;
  const GPart* g = j.gpart + static_cast<size_t>(row) * j.ntile3;
  // the descriptor and this thread's first record, loaded together
  const RowDesc d = j.desc[row];
  const int t0 = static_cast<int>(threadIdx.x);
  const GPart p0 = t0 < j.ntile3 ? g[t0] : GPart{-1.0, 0x7fffffff, 0};
  if (!full_row(d.mode)) return;  // uniform over the block
  double best = -1.0;
  int best_id = 0x7fffffff;
  int kept = 0;
  for (int t = t0; t < j.ntile3; t += blockDim.x) {
    const GPart p = t == t0 ? p0 : g[t];
    kept += p.kept;
    if (p.kept && (p.score > best || (p.score == best && p.id < best_id))) {
      best = p.score;
      best_id = p.id;
    }
  }
  const double bb = block_max(best, sd);
  const int bid = block_min(best == bb ? best_id : 0x7fffffff, si);
  const int bk = block_sum(kept, si);
  if (threadIdx.x == 0) {
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
      const float2 ml = j.rlse[row];
      const float x = to_f32(static_cast<const E*>(j.logits)[static_cast<int64_t>(row) * j.ld + bid]);
      j.out_tok_lp[row] = (x - ml.x) - ml.y;
    }
  }
}

// lp = (x - max) - log(sum exp(x - max)) for every id of the row.
template <typename E, bool kScaled>
__global__ __launch_bounds__(kThreads) void k_lse_full(Job j, int ntile, bool out_vec) {
  int row, tile;
  if (!xcd_row_tile(blockIdx.x, j.B, ntile, &row, &tile)) return;
  constexpr int EPV = Epv<E>::n;
  constexpr int NV = kPerThread / EPV;
  const float2 ml = j.rlse[row];
  const float Tl = kScaled ? lse_T(j, row) : 1.0f;  // the log-prob temperature (1: none)
  const E* rowp = static_cast<const E*>(j.logits) + static_cast<int64_t>(row) * j.ld;
  float* orow = j.out_full + static_cast<int64_t>(row) * j.ld_out;
  const int base = tile * kFullTile;
  const bool vec = j.aligned && out_vec && (base + kFullTile <= j.V);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j0 = base + (i * kThreads + static_cast<int>(threadIdx.x)) * EPV;
    if (vec) {
      // read once, written once: both streamed past the caches
      const uint4 raw = load16_stream(rowp + j0);
      float x[EPV];
      unpack16(raw, x, rowp);
      if (Tl != 1.0f) {  // uniform
#pragma unroll
        for (int c = 0; c < EPV; ++c) x[c] = x[c] / Tl;
      }
#pragma unroll
      for (int c = 0; c < EPV; c += 4) {
        f32x4 o;
        o.x = (x[c] - ml.x) - ml.y;
        o.y = (x[c + 1] - ml.x) - ml.y;
        o.z = (x[c + 2] - ml.x) - ml.y;
        o.w = (x[c + 3] - ml.x) - ml.y;
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(orow + j0 + c));
      }
    } else {
#pragma unroll
      for (int c = 0; c < EPV; ++c) {
        const int id = j0 + c;
        if (id < j.V) orow[id] = (lse_scaled(to_f32(rowp[id]), Tl) - ml.x) - ml.y;
      }
    }
  }
}

}  // namespace

hipError_t launch_gumbel(const Job& j, hipStream_t st) {
  const int grid = xcd_grid(j.B, (j.ntile3 + j.gseg - 1) / j.gseg);
  if (j.dt == VS_F32)
    hipLaunchKernelGGL(k_gumbel_partial<float>, dim3(grid), dim3(kThreads), 0, st, j);
  else
    hipLaunchKernelGGL(k_gumbel_partial<uint16_t>, dim3(grid), dim3(kThreads), 0, st, j);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (j.dt == VS_F32)
    hipLaunchKernelGGL(k_gumbel_final<float>, dim3(j.B), dim3(kThreads), 0, st, j);
  else
    hipLaunchKernelGGL(k_gumbel_final<uint16_t>, dim3(j.B), dim3(kThreads), 0, st, j);
  return hipGetLastError();
}

hipError_t launch_lse_full(const Job& j, hipStream_t st) {
  const int ntile = (j.V + kFullTile - 1) / kFullTile;
  const int grid = xcd_grid(j.B, ntile);
  const bool out_vec = (reinterpret_cast<uintptr_t>(j.out_full) % 16 == 0) && (j.ld_out % 4 == 0);
  const bool scaled = j.lpT != nullptr && !j.sample;  // the log-prob temperature's instances
  const dim3 g(grid), b(kThreads);
  if (j.dt == VS_F32 && scaled)
    hipLaunchKernelGGL((k_lse_full<float, true>), g, b, 0, st, j, ntile, out_vec);
  else if (j.dt == VS_F32)
    hipLaunchKernelGGL((k_lse_full<float, false>), g, b, 0, st, j, ntile, out_vec);
  else if (scaled)
    hipLaunchKernelGGL((k_lse_full<uint16_t, true>), g, b, 0, st, j, ntile, out_vec);
  else
    hipLaunchKernelGGL((k_lse_full<uint16_t, false>), g, b, 0, st, j, ntile, out_vec);
  return hipGetLastError();
}

}  // namespace vsk
