// K3/K4: the Gumbel-max draw over full-vocabulary kept sets, and the full
// log-softmax write of vs_logprobs.
//
// K3 (grid: rows x 4096-id tiles, all tiles of a row on one XCD): for every id
// of the tile it recomputes s = x / T and e = exp(s - m), tests membership
// (everything; e >= min_p; or for top-p "key > tau, or key == tau and
// id <= id_cut"), and for kept ids forms score = e / -log(u(seed, row, id)).
// Each tile keeps its best (score desc, id asc) and its kept count.
// K4 (one workgroup per row) reduces the tiles: the sampled id and the kept
// count. The argmax compares the true id, never thread or tile order, so the
// result does not depend on the partition (vllm.cpp #1997, "The kernel").
#include "vs_device.h"
#include "vs_kernels.h"

namespace vsk {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = kGumTile / kThreads;  // 16

template <typename E>
__global__ __launch_bounds__(kThreads) void k_gumbel_partial(
    const E* __restrict__ logits, int B, int V, int64_t ld, bool aligned,
    const float* __restrict__ temperature, const float* __restrict__ min_p,
    const uint64_t* __restrict__ seeds, const RowDesc* __restrict__ desc, int ntile,
    GPart* __restrict__ gpart, uint32_t* __restrict__ out_mask) {
  __shared__ double sd[kThreads / kWave];
  __shared__ int si[kThreads / kWave];
  int row, tile;
  if (!xcd_row_tile(blockIdx.x, B, ntile, &row, &tile)) return;
  const RowDesc d = desc[row];
  if (d.mode == kFullSkip) return;  // uniform over the block
  constexpr int EPV = Epv<E>::n;
  constexpr int NV = kPerThread / EPV;
  const float T = temperature ? temperature[row] : 1.0f;
  const float mp = min_p ? min_p[row] : 0.0f;
  const uint64_t rs = row_stream(seeds ? seeds[row] : 0ull, row);
  const E* rowp = logits + static_cast<int64_t>(row) * ld;
  const int base = tile * kGumTile;
  const bool vec = aligned && (base + kGumTile <= V);
  const int mwords = (V + 31) / 32;
  uint32_t* mask_row = out_mask ? out_mask + static_cast<size_t>(row) * mwords : nullptr;

  double best = -1.0;
  int best_id = 0x7fffffff;
  int kept = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j0 = base + (i * kThreads + static_cast<int>(threadIdx.x)) * EPV;
    float x[EPV];
    if (vec) {
      const uint4 raw = *reinterpret_cast<const uint4*>(rowp + j0);
      unpack16(raw, x, rowp);
    } else {
#pragma unroll
      for (int c = 0; c < EPV; ++c) x[c] = (j0 + c < V) ? to_f32(rowp[j0 + c]) : -kInf;
    }
    uint32_t bits = 0;
#pragma unroll
    for (int c = 0; c < EPV; ++c) {
      const int j = j0 + c;
      if (j >= V) continue;
      const float s = (T == 1.0f) ? x[c] : x[c] / T;
      const float e = pinned_exp(s - d.m);
      bool keep;
      if (d.mode == kFullNone) {
        keep = true;
      } else if (d.mode == kFullMinP) {
        keep = e >= mp;
      } else {
        const uint32_t key = f2key(s);
        keep = key > d.tau || (key == d.tau && j <= d.id_cut);
      }
      if (keep) {
        ++kept;
        bits |= 1u << (j & 31);
        const double sc = gumbel_score(e, rs, j);
        if (sc > best || (sc == best && j < best_id)) {
          best = sc;
          best_id = j;
        }
      }
    }
    if (mask_row && bits) atomicOr(&mask_row[j0 >> 5], bits);
  }
  const double bb = block_max(best, sd);
  const int bid = block_min(best == bb ? best_id : 0x7fffffff, si);
  const int bk = block_sum(kept, si);
  if (threadIdx.x == 0) gpart[static_cast<size_t>(row) * ntile + tile] = GPart{bb, bid, bk};
}

__global__ __launch_bounds__(kThreads) void k_gumbel_final(
    int B, int ntile, const RowDesc* __restrict__ desc, const GPart* __restrict__ gpart,
    int32_t* __restrict__ out_ids, int32_t* __restrict__ out_kept) {
  __shared__ double sd[kThreads / kWave];
  __shared__ int si[kThreads / kWave];
  const int row = blockIdx.x;
  if (desc[row].mode == kFullSkip) return;
  const GPart* g = gpart + static_cast<size_t>(row) * ntile;
  double best = -1.0;
  int best_id = 0x7fffffff;
  int kept = 0;
  for (int t = threadIdx.x; t < ntile; t += blockDim.x) {
    const GPart p = g[t];
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
    out_ids[row] = bid;
    if (out_kept) out_kept[row] = bk;
  }
}

// lp = (x - max) - log(sum exp(x - max)) for every id of the row.
template <typename E>
__global__ __launch_bounds__(kThreads) void k_lse_full(
    const E* __restrict__ logits, int B, int V, int64_t ld, bool aligned,
    const float2* __restrict__ rlse, int ntile, float* __restrict__ out, int64_t ld_out,
    bool out_vec) {
  int row, tile;
  if (!xcd_row_tile(blockIdx.x, B, ntile, &row, &tile)) return;
  constexpr int EPV = Epv<E>::n;
  constexpr int NV = kPerThread / EPV;
  const float2 ml = rlse[row];
  const E* rowp = logits + static_cast<int64_t>(row) * ld;
  float* orow = out + static_cast<int64_t>(row) * ld_out;
  const int base = tile * kFullTile;
  const bool vec = aligned && out_vec && (base + kFullTile <= V);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j0 = base + (i * kThreads + static_cast<int>(threadIdx.x)) * EPV;
    if (vec) {
      const uint4 raw = *reinterpret_cast<const uint4*>(rowp + j0);
      float x[EPV];
      unpack16(raw, x, rowp);
#pragma unroll
      for (int c = 0; c < EPV; c += 4) {
        float4 o;
        o.x = (x[c] - ml.x) - ml.y;
        o.y = (x[c + 1] - ml.x) - ml.y;
        o.z = (x[c + 2] - ml.x) - ml.y;
        o.w = (x[c + 3] - ml.x) - ml.y;
        *reinterpret_cast<float4*>(orow + j0 + c) = o;
      }
    } else {
#pragma unroll
      for (int c = 0; c < EPV; ++c) {
        const int j = j0 + c;
        if (j < V) orow[j] = (to_f32(rowp[j]) - ml.x) - ml.y;
      }
    }
  }
}

}  // namespace

hipError_t launch_gumbel(const SampleArgs& a, const WsLayout& L, char* ws, hipStream_t st) {
  const auto* desc = reinterpret_cast<const RowDesc*>(ws + L.desc);
  auto* gp = reinterpret_cast<GPart*>(ws + L.gpart);
  const int grid = xcd_grid(a.B, L.ntile3);
  if (a.dt == VS_F32)
    hipLaunchKernelGGL(k_gumbel_partial<float>, dim3(grid), dim3(kThreads), 0, st,
                       static_cast<const float*>(a.logits), a.B, a.V, a.ld, a.aligned,
                       a.temperature, a.min_p, a.seeds, desc, L.ntile3, gp, a.out_mask);
  else
    hipLaunchKernelGGL(k_gumbel_partial<uint16_t>, dim3(grid), dim3(kThreads), 0, st,
                       static_cast<const uint16_t*>(a.logits), a.B, a.V, a.ld, a.aligned,
                       a.temperature, a.min_p, a.seeds, desc, L.ntile3, gp, a.out_mask);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_gumbel_final, dim3(a.B), dim3(kThreads), 0, st, a.B, L.ntile3, desc, gp,
                     a.out_ids, a.out_kept);
  return hipGetLastError();
}

hipError_t launch_lse_full(const LogprobArgs& a, const WsLayout& L, char* ws, hipStream_t st) {
  const auto* rl = reinterpret_cast<const float2*>(ws + L.rlse);
  const int ntile = (a.V + kFullTile - 1) / kFullTile;
  const int grid = xcd_grid(a.B, ntile);
  const bool out_vec = (reinterpret_cast<uintptr_t>(a.out_full) % 16 == 0) && (a.ld_out % 4 == 0);
  if (a.dt == VS_F32)
    hipLaunchKernelGGL(k_lse_full<float>, dim3(grid), dim3(kThreads), 0, st,
                       static_cast<const float*>(a.logits), a.B, a.V, a.ld, a.aligned, rl, ntile,
                       a.out_full, a.ld_out, out_vec);
  else
    hipLaunchKernelGGL(k_lse_full<uint16_t>, dim3(grid), dim3(kThreads), 0, st,
                       static_cast<const uint16_t*>(a.logits), a.B, a.V, a.ld, a.aligned, rl, ntile,
                       a.out_full, a.ld_out, out_vec);
  return hipGetLastError();
}

}  // namespace vsk
