// Host-side launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/vs.h"

namespace vsk {

// One select/log-sum-exp tile is one wave's 64 lanes x 64 values.
constexpr int kSelTile = 4096;
constexpr int kSelWaves = 4;      // tiles per 256-thread workgroup
constexpr int kGumTile = 4096;    // Gumbel tile: 256 threads x 16 values
constexpr int kFullTile = 4096;   // full log-softmax write tile

struct WsLayout {
  int B, V;
  int ntile1;   // select tiles per row
  int wpr1;     // select workgroups per row
  int ntile3;   // Gumbel tiles per row
  size_t meta, cand, desc, gpart, lpart, rlse, total;
};

WsLayout ws_layout(int B, int V);

struct SampleArgs {
  const void* logits;
  vs_dtype dt;
  int B, V;
  int64_t ld;
  bool aligned;
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;
  const float* min_p;
  const uint64_t* seeds;
  uint32_t hints;
  int32_t* out_ids;
  int32_t* out_kept;
  uint32_t* out_mask;
  int32_t* out_status;
};

struct LogprobArgs {
  const void* logits;
  vs_dtype dt;
  int B, V;
  int64_t ld;
  bool aligned;
  const int32_t* token_ids;
  float* out_token_lp;
  int k;
  int32_t* out_topk_ids;
  float* out_topk_lp;
  float* out_full;
  int64_t ld_out;
  int32_t* out_status;
};

hipError_t launch_select(const SampleArgs& a, const WsLayout& L, char* ws, hipStream_t st);
hipError_t launch_select_lse(const LogprobArgs& a, const WsLayout& L, char* ws, hipStream_t st);
hipError_t launch_row(const SampleArgs& a, const WsLayout& L, char* ws, hipStream_t st);
hipError_t launch_gumbel(const SampleArgs& a, const WsLayout& L, char* ws, hipStream_t st);
hipError_t launch_lse_row(const LogprobArgs& a, const WsLayout& L, char* ws, hipStream_t st);
hipError_t launch_lse_full(const LogprobArgs& a, const WsLayout& L, char* ws, hipStream_t st);
hipError_t launch_penalize(void* logits, vs_dtype dt, int B, int V, int64_t ld,
                           const int32_t* prompt_ids, const int32_t* prompt_off,
                           const int32_t* output_ids, const int32_t* output_off,
                           const float* presence, const float* frequency,
                           const float* repetition, int32_t* out_status, hipStream_t st);

}  // namespace vsk
