/*
 * CPU oracle for batched decode-step token sampling.
 *
 * TEST INFRASTRUCTURE ONLY. This library is the slow, plain, single-threaded
 * definition that the GPU library is checked against. Only the test suite, the
 * package smoke check and the CPU-baseline leg of the benchmark may load it.
 * It shares no code, header, table or constant generator with the GPU path.
 *
 * Every function follows the definitions on the source pages:
 *  - occurrence penalties: TensorRT-LLM "Sampling" page, section "LLM API
 *    sampling behavior when using Torch Sampler", the occurrence-penalty bullets;
 *  - temperature, min-p, top-k, top-p and the greedy triggers: the same section;
 *  - the Gumbel-max draw (SplitMix64 uniforms, f64 exponential noise, score
 *    prob/q, lowest-index argmax): vllm.cpp pull request #1997, sections
 *    "The kernel (#1984)" and "What the 236 ms is";
 *  - log-softmax log-probabilities: the TT sampling README, "Key Components"
 *    (LogProbsCalculator), and the Tunix sampler page, the greedy/top-p answer.
 * Points the pages leave open follow the readings listed in the repository's
 * design notes (non-finite logits, penalty rounding, pinned exp, fixed-point
 * top-p masses, the (seed,row,id) mixing of the random stream).
 *
 * Row status bits written by the oracle have the same meaning as those of the
 * GPU library: 1 bad parameter, 2 bad logits, 4 bad token id, 8 top-k larger
 * than the supported maximum.
 */
#ifndef DTS_ORACLE_H
#define DTS_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype: 0 = fp32, 1 = bf16 (stored as raw uint16). ld = row stride in elements. */

/* prompt_ignore: [B] int32 or NULL (TensorRT-LLM "Sampling" page, the
 * prompt_ignore_length bullet): the first n prompt ids of row r, n =
 * clamp(prompt_ignore[r], 0, prompt length), count for the repetition penalty
 * but not for presence and frequency. */
int oracle_penalize(void* logits, int dtype, int B, int V, int64_t ld,
                    const int32_t* prompt_ids, const int32_t* prompt_off,
                    const int32_t* output_ids, const int32_t* output_off,
                    const float* presence, const float* frequency,
                    const float* repetition, const int32_t* prompt_ignore,
                    int32_t* row_status);

/* out_kept_mask: B*V bytes or NULL; out_top2: B*2 doubles (best and second-best
 * Gumbel score, -1 where fewer than two kept ids) or NULL. */
int oracle_sample(const void* logits, int dtype, int B, int V, int64_t ld,
                  const float* temperature, const int32_t* top_k,
                  const float* top_p, const float* min_p, const uint64_t* seeds,
                  int32_t* out_ids, int32_t* out_kept_count,
                  uint8_t* out_kept_mask, double* out_top2, int32_t* row_status);

/* Same as oracle_sample for the single row r of a batch (for bounded timing
 * samples); arrays are the full-batch arrays. */
int oracle_sample_row(const void* logits, int dtype, int B, int V, int64_t ld,
                      int r, const float* temperature, const int32_t* top_k,
                      const float* top_p, const float* min_p,
                      const uint64_t* seeds, int32_t* out_ids,
                      int32_t* out_kept_count, uint8_t* out_kept_mask,
                      double* out_top2, int32_t* row_status);

/* The same at a temperature per row: the log-softmax of s = x / T (fp32
 * division); temperature NULL, or a T that is not positive and finite, means
 * T = 1. */
int oracle_logprobs_t(const void* logits, int dtype, int B, int V, int64_t ld,
                      const float* temperature, const int32_t* token_ids, double* out_token_lp,
                      int k, int32_t* out_topk_ids, double* out_topk_lp, double* out_full,
                      int32_t* row_status);
/* token_ids/out_token_lp may be NULL; out_full (B*V doubles) may be NULL. */
int oracle_logprobs(const void* logits, int dtype, int B, int V, int64_t ld,
                    const int32_t* token_ids, double* out_token_lp, int k,
                    int32_t* out_topk_ids, double* out_topk_lp,
                    double* out_full, int32_t* row_status);

/* Top-p decay after one sampled token (TensorRT-LLM "Sampling" page, the
 * Top-P decay bullets). Row r with sampled[r] >= 0: top_p[r] = top_p_init[r]
 * when reset_ids[r] >= 0 and sampled[r] == reset_ids[r], else
 * max(top_p[r] * decay[r] rounded to fp32, top_p_min[r]). top_p_min NULL:
 * 1e-6 for every row; reset_ids NULL: no reset id. decay or top_p_min outside
 * (0, 1], top_p_init outside [0, 1] or a reset id below -1: row unchanged,
 * status 1 (bad parameter). */
int oracle_topp_decay(int B, float* top_p, const float* top_p_init, const float* decay,
                      const float* top_p_min, const int32_t* reset_ids,
                      const int32_t* sampled, int32_t* row_status);

/* One new seed per row per sampled token: seeds[r] += 0x9E3779B97F4A7C15
 * (mod 2^64), the SplitMix64 increment, for rows with sampled[r] >= 0 (every
 * row when sampled is NULL). */
int oracle_seed_advance(int B, uint64_t* seeds, const int32_t* sampled);

/* Slot remap: dst[i] = src[remap[i]] (elements of elem_bytes, 4 or 8) for
 * 0 <= remap[i] < B_src; a negative entry leaves dst[i]; an entry >= B_src
 * leaves it and sets status 1. */
int oracle_slot_remap(int B, int B_src, const int32_t* remap, const void* src, void* dst,
                      int elem_bytes, int32_t* row_status);

/* Building blocks exposed for the pin tests. */
float oracle_exp_pinned(float t);
uint64_t oracle_splitmix64(uint64_t x);
double oracle_uniform(uint64_t seed, int row, int id);
uint16_t oracle_f32_to_bf16(float f);
/* got[i] against E(the float with bits lo_bits + i), i < n: returns the number
 * of results whose bits differ; *first_bad (if not NULL) receives the first
 * such i, or n. */
long oracle_exp_compare(uint32_t lo_bits, uint32_t n, const float* got, uint32_t* first_bad);
/* Exhaustive checks of the pinned exp over every float in [lo, hi] (lo <= hi <= 0):
 * returns the number of monotonicity violations; *max_ulp receives the largest
 * error in fp32 ulps against libm's double exp rounded to float. */
long oracle_exp_scan(float lo, float hi, double* max_ulp);

#ifdef __cplusplus
}
#endif
#endif
