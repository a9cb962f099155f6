/*
 * vs.h — batched decode-step token sampling on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libvs.so. Three calls make up one decode step over a row-major
 * [B, ld] matrix of fp32 or bf16 logits (only columns [0, V) are read):
 *
 *   vs_penalize  presence / frequency / repetition penalties, in place
 *   vs_sample    temperature, min-p, top-k, top-p, then a seeded Gumbel-max draw
 *   vs_logprobs  log-softmax log-probabilities (given ids, top-k, full rows)
 *   vs_sample_logprobs  the last two fused: the logits are read once
 *
 * Conventions shared by every call:
 *  - All array arguments are DEVICE pointers unless stated otherwise; sizes and
 *    scalars are host values. The caller owns every buffer. The library keeps no
 *    pointer after a call returns, and no call allocates or frees memory (the
 *    one device array the library owns, the scratch of
 *    vs_sample_logprobs_noalloc, exists from load to process end).
 *  - Mutable state kept by the library: cached device properties (compute-unit
 *    count per device), the per-device address of that scratch, and the
 *    profiling record of vs_profile_begin/_end, which is thread-local (one per
 *    calling host thread, empty unless that thread turned it on) and so never
 *    shared between callers.
 *  - Each call checks its host-visible arguments, enqueues kernels on `stream`
 *    and returns without waiting. Outputs are valid once the stream reaches that
 *    point; inputs must stay alive until then. No call synchronises, copies to
 *    the host or allocates, so every call can be captured into a HIP graph.
 *  - Host-detectable errors (NULL required pointer, B <= 0, V <= 0,
 *    V > VS_MAX_V, ld < V, unknown dtype, bad k, workspace too small) return an
 *    error status and enqueue nothing. A failed launch returns VS_ERR_HIP.
 *  - Problems found on the device (per-row parameters, non-finite logits, token
 *    ids out of range) are reported per row in `out_row_status` (bits VS_ROW_*)
 *    when that pointer is not NULL; see each call for what such a row outputs.
 *  - A workspace may serve one call at a time: two calls that overlap in time
 *    (on different streams) need different workspaces.
 *  - Logits rows are 16-byte aligned (base pointer and ld * element size) for the
 *    fast load path; other layouts are accepted and take a slower path.
 */
#ifndef VS_H
#define VS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum vs_dtype { VS_F32 = 0, VS_BF16 = 1 } vs_dtype;

typedef enum vs_status {
  VS_OK = 0,
  VS_ERR_INVALID_ARGUMENT = 1,
  VS_ERR_WORKSPACE_TOO_SMALL = 2,
  VS_ERR_UNSUPPORTED = 3,
  VS_ERR_HIP = 4
} vs_status;

/* Per-row status bits (device-written int32 per row). */
#define VS_ROW_BAD_PARAM 1        /* temperature < 0, NaN or inf; top_k < 0; top_p or min_p
                                     outside [0,1]; repetition <= 0 or non-finite penalties;
                                     logits / temperature overflowing to +inf */
#define VS_ROW_BAD_LOGITS 2       /* a NaN or +inf logit in [0,V), or every logit is -inf */
#define VS_ROW_BAD_TOKEN_ID 4     /* a history id (vs_penalize) or query id (vs_logprobs)
                                     outside [0,V) */
#define VS_ROW_TOPK_UNSUPPORTED 8 /* VS_TOPK_MAX < top_k < V */
#define VS_ROW_HINT_VIOLATED 16   /* the row needs a stage the caller's hints switched off */

/* vs_sample hints: promises by the caller that let the library skip kernels.
 * A row that breaks a promise gets VS_ROW_HINT_VIOLATED and id -1 (it is never
 * sampled wrongly). With hints = 0 every row is handled. */
#define VS_HINT_NONE 0u
#define VS_HINT_NO_FULLVOCAB 1u   /* no row samples over the full vocabulary: every row is
                                     greedy or has 0 < top_k < V */
#define VS_HINT_NO_FULLVOCAB_TRUNCATION VS_HINT_NO_FULLVOCAB
#define VS_HINT_ALL_GREEDY 2u     /* every row is greedy */
#define VS_HINT_NO_GREEDY 4u      /* no row is greedy. Checked, but it lets nothing be
                                     skipped here: a greedy row costs no kernel of its own
                                     (its argmax comes with the streaming pass's lists) */
#define VS_HINT_SMALL_TOPK 8u     /* every row is greedy or has 1 < top_k <= 64 (and
                                     top_k < V): no full-vocabulary row, no larger top-k */
/* Not promises but a choice of method for full-vocabulary top-p rows, passed in
 * the same word; every method gives identical results, and all are ignored
 * when a kept mask is asked for (the Gumbel pass over the kept set writes it).
 *  VS_OPT_TOPP_REJECTION: draw by rejection. The histogram pass of the top-p
 *    cut also keeps each segment's best Gumbel candidates over all ids that
 *    pass min-p; once the cut is known, the first of the row's best candidates
 *    (score order) that lies inside it is the draw (every higher score belongs
 *    to a candidate outside it), with no pass over the kept set; a row whose
 *    best candidates all lie outside falls back to that pass.
 *  VS_OPT_TOPP_GATHER_DRAW: the pass that gathers the ids of the cut's bucket
 *    also draws over the ids above that bucket (all kept, wherever the cut
 *    falls inside it), and the kernel that finds the cut scores the kept ids
 *    of the bucket and finishes the row (a bucket that overflowed its list:
 *    one pass over the row's kept set in that kernel); no pass over the kept
 *    sets, and rows without the cut (top_p = 1) drawn in the gather pass too.
 *  VS_OPT_TOPP_KEPT_PASS: the Gumbel pass over the kept set after the cut.
 * Without one of them (or with more than one: the first listed wins), the
 * gather draw is taken, the fastest of the three on every measured workload. */
#define VS_OPT_TOPP_REJECTION 256u
#define VS_OPT_TOPP_GATHER_DRAW 512u
#define VS_OPT_TOPP_KEPT_PASS 1024u

#define VS_MAX_V (1 << 21)        /* largest vocabulary */
#define VS_TOPK_MAX 1024          /* largest top_k below V */
#define VS_LOGPROB_K_MAX 64       /* largest top-k for vs_logprobs */

/* Bytes of device workspace that vs_sample and vs_logprobs need for B rows of
 * V logits of type dt. Returns VS_ERR_INVALID_ARGUMENT for bad sizes. */
vs_status vs_workspace_size(int B, int V, vs_dtype dt, size_t* bytes);

/* Static English text for a status code (host pointer, never NULL). */
const char* vs_status_string(vs_status s);

/*
 * vs_penalize — occurrence penalties, in place.
 *
 * Defined by the TensorRT-LLM "Sampling" page (section "LLM API sampling
 * behavior when using Torch Sampler", occurrence-penalty bullets). With c the
 * number of times id j occurs in the row's prompt ids plus its output ids, every
 * j with c > 0 becomes, each step one rounded fp32 operation:
 *     y = x >= 0 ? x / repetition : x * repetition;  y = y - presence;
 *     y = y - frequency * c
 * bf16 logits are widened exactly, penalised in fp32 and rounded once to
 * nearest-even. Ids with c = 0 are not touched.
 *
 *  logits      [B, ld] fp32 or bf16, modified in place
 *  prompt_ids  int32 token ids, CSR by row: row r owns
 *  prompt_off  prompt_ids[prompt_off[r] .. prompt_off[r+1]); prompt_off has B+1
 *              entries. Both NULL: no prompt history.
 *  output_ids, output_off: the generated tokens so far, same layout (or both NULL).
 *  presence, frequency, repetition: [B] fp32 each; NULL means 0, 0 and 1.
 *  out_row_status [B] int32 or NULL. A row with a bad parameter is left
 *              unchanged (VS_ROW_BAD_PARAM); ids outside [0,V) are skipped
 *              (VS_ROW_BAD_TOKEN_ID).
 */
vs_status vs_penalize(void* logits, vs_dtype dt, int B, int V, int64_t ld,
                      const int32_t* prompt_ids, const int32_t* prompt_off,
                      const int32_t* output_ids, const int32_t* output_off,
                      const float* presence, const float* frequency,
                      const float* repetition, int32_t* out_row_status,
                      hipStream_t stream);

/*
 * vs_penalize_ex — vs_penalize with a prompt ignore length per row.
 *
 * The TensorRT-LLM "Sampling" page's prompt_ignore_length bullet: the first n
 * prompt ids of a row, n = prompt_ignore_len[r] clamped to [0, the row's prompt
 * length], are left out of the presence and frequency counts and still count
 * for the repetition penalty. So an id that occurs only there gets the
 * repetition step alone; values <= 0 change nothing; a value at or past the
 * prompt length counts presence and frequency over the output ids only.
 *
 *  prompt_ignore_len [B] int32 device pointer, or NULL (every n = 0: exactly
 *              vs_penalize). Every other argument, and the errors, as
 *              vs_penalize.
 */
vs_status vs_penalize_ex(void* logits, vs_dtype dt, int B, int V, int64_t ld,
                         const int32_t* prompt_ids, const int32_t* prompt_off,
                         const int32_t* output_ids, const int32_t* output_off,
                         const float* presence, const float* frequency,
                         const float* repetition, const int32_t* prompt_ignore_len,
                         int32_t* out_row_status, hipStream_t stream);

/*
 * vs_topp_decay — the effective top-p after one sampled token, in place.
 *
 * The TensorRT-LLM "Sampling" page's Top-P decay bullets: after every sampled
 * token the effective top_p is multiplied by top_p_decay (one rounded fp32
 * product), bounded from below by top_p_min, and reset to the initial top_p
 * when the token top_p_reset_ids is sampled. With top_p = 1 and an active
 * decay the state starts from 1. The caller passes the state as vs_sample's
 * top_p on the next step; a greedy row ignores it there (greedy takes
 * precedence).
 *
 *  top_p        [B] fp32, the state, updated in place (device).
 *  top_p_init   [B] fp32 in [0, 1]; decay [B] fp32 in (0, 1].
 *  top_p_min    [B] fp32 in (0, 1], or NULL (1e-6 for every row).
 *  reset_ids    [B] int32, -1 for none, or NULL (none).
 *  sampled_ids  [B] int32, the step's ids; a row with a negative id (nothing
 *               sampled) keeps its state.
 *  out_row_status [B] int32 or NULL: VS_ROW_BAD_PARAM for a parameter out of
 *               range (also a reset id below -1); that row keeps its state.
 * Errors: VS_ERR_INVALID_ARGUMENT for B <= 0 or a required NULL pointer.
 */
vs_status vs_topp_decay(int B, float* top_p, const float* top_p_init, const float* decay,
                        const float* top_p_min, const int32_t* reset_ids,
                        const int32_t* sampled_ids, int32_t* out_row_status, hipStream_t stream);

/*
 * vs_seed_advance — one new seed per row per sampled token, in place.
 *
 * The TT sampling README's seed contract asks for new seed values exactly once
 * per sampled token; the Tunix sampler folds the decoding step into its key.
 * Here seeds[r] += 0x9E3779B97F4A7C15 (mod 2^64), the SplitMix64 increment,
 * so successive seeds are that generator's successive states and each step's
 * draw (keyed by seed, row and id) is a fresh stream.
 *
 *  seeds        [B] uint64, device, updated in place.
 *  sampled_ids  [B] int32 or NULL: only rows with an id >= 0 advance (NULL:
 *               every row).
 * Errors: VS_ERR_INVALID_ARGUMENT for B <= 0 or seeds NULL.
 */
vs_status vs_seed_advance(int B, uint64_t* seeds, const int32_t* sampled_ids, hipStream_t stream);

/*
 * vs_slot_remap — per-row state follows its request to a new batch slot.
 *
 * The TT sampling README's decode update contract: slot_remap[i] = j means
 * new slot i takes the state of the continuing request from old slot j,
 * applied once per decode that carries the remap (the caller's duty). Here
 * one per-row array at a time (seeds, the top-p decay state, parameters):
 * dst[i] = src[slot_remap[i]] for 0 <= slot_remap[i] < B_src. A negative
 * entry leaves dst[i] as it is (a new request, which the caller initialises);
 * an entry >= B_src leaves it too and reports VS_ROW_BAD_PARAM.
 *
 *  slot_remap  [B] int32, device.
 *  src         [B_src] elements of elem_bytes (4 or 8), device.
 *  dst         [B] elements, device, not src (the old state is read whole).
 *  out_row_status [B] int32 or NULL.
 * Errors: VS_ERR_INVALID_ARGUMENT for B or B_src <= 0, a NULL pointer, src ==
 * dst, or elem_bytes other than 4 and 8.
 */
vs_status vs_slot_remap(int B, int B_src, const int32_t* slot_remap, const void* src, void* dst,
                        int elem_bytes, int32_t* out_row_status, hipStream_t stream);

/*
 * vs_sample — one token per row.
 *
 * Truncation follows the TensorRT-LLM "Sampling" page (same section): greedy
 * when temperature = 0, top_k = 1, top_p = 0 or min_p = 1; otherwise
 * s = x / temperature (correctly rounded fp32), then min-p (keep relative
 * weight >= min_p, applied first) and top-k (top_k = 0 or >= V: no top-k), then
 * top-p on the survivors renormalised (shortest prefix reaching top_p of their
 * mass). The draw follows vllm.cpp pull request #1997 ("The kernel (#1984)"):
 * per kept id j a SplitMix64 uniform u(seed, row, j), q = -log(u) in double,
 * score = prob / q, and the largest score wins with ties to the lowest id.
 * Order everywhere is larger s first, lower id first among equals. Relative
 * weights are e = exp(s - max s) rounded to fp32 (0 below -87); top-p masses are
 * floor(e * 2^31) summed exactly; the top-p threshold is top_p * total in double.
 *
 *  logits       [B, ld] fp32 or bf16 (read only)
 *  temperature  [B] fp32 or NULL (all 1)       top_k [B] int32 or NULL (all 0)
 *  top_p        [B] fp32 or NULL (all 1)       min_p [B] fp32 or NULL (all 0)
 *               with temperature, top_k and top_p all NULL every row is greedy
 *               (the page: none of the three set means greedy sampling)
 *  seeds        [B] uint64 or NULL (all 0): the caller's per-row seed, advanced by
 *               the caller once per sampled token
 *  hints        VS_HINT_* promises (0 = none)
 *  out_ids      [B] int32: the sampled id, -1 for a row with a nonzero status
 *  out_kept_count [B] int32 or NULL: size of the kept set (1 for greedy)
 *  out_kept_mask  [B, ceil(V/32)] uint32 or NULL: bit j%32 of word j/32 set for
 *               every kept id (for tests; costs an extra write)
 *  out_row_status [B] int32 or NULL
 *  ws, ws_bytes  device workspace of at least vs_workspace_size() bytes
 */
vs_status vs_sample(const void* logits, vs_dtype dt, int B, int V, int64_t ld,
                    const float* temperature, const int32_t* top_k,
                    const float* top_p, const float* min_p,
                    const uint64_t* seeds, uint32_t hints, int32_t* out_ids,
                    int32_t* out_kept_count, uint32_t* out_kept_mask,
                    int32_t* out_row_status, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/*
 * vs_sample_logprobs — vs_sample and the log-probabilities of the same logits
 * in one pass over them: the result equals vs_sample followed by vs_logprobs
 * with token_ids = out_ids (a row whose id is -1 gets a NaN log-prob), but the
 * logits are read once (the streaming pass also forms the log-sum-exp partials
 * and the top-k candidates of the raw logits).
 *
 *  out_token_logprob [B] fp32 or NULL: log-prob of the sampled id
 *  k, out_topk_ids, out_topk_logprobs, out_full, ld_out: as in vs_logprobs
 *  other arguments and out_row_status: as in vs_sample (the status of the draw;
 *  a row with bad logits also gets NaN log-probs and top-k ids -1)
 */
vs_status vs_sample_logprobs(const void* logits, vs_dtype dt, int B, int V, int64_t ld,
                             const float* temperature, const int32_t* top_k,
                             const float* top_p, const float* min_p,
                             const uint64_t* seeds, uint32_t hints, int32_t* out_ids,
                             int32_t* out_kept_count, uint32_t* out_kept_mask,
                             int32_t* out_row_status, float* out_token_logprob, int k,
                             int32_t* out_topk_ids, float* out_topk_logprobs, float* out_full,
                             int64_t ld_out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * vs_penalize_sample_logprobs — vs_penalize_ex followed by vs_sample_logprobs
 * in one call: the streaming pass that reads each row segment first applies
 * the occurrence penalties (TensorRT-LLM "Sampling", occurrence-penalty and
 * prompt_ignore_length bullets; the same arithmetic, rounding and row checks
 * as vs_penalize_ex) to the segment's history ids, in place, then reads the
 * segment. The result equals the two calls in sequence, without the separate
 * penalty launch and its second pass over each history.
 *
 *  logits      [B, ld] fp32 or bf16, modified in place: on return it holds the
 *              penalised logits, as after vs_penalize_ex (later passes of the
 *              same call, for full-vocabulary rows, read them from there).
 *  prompt_ids .. prompt_ignore_len: as vs_penalize_ex (NULL pairs: no history;
 *              NULL parameters: 0, 0, 1; NULL ignore lengths: 0).
 *  out_penalty_status [B] int32 or NULL: the penalty step's status per row, as
 *              vs_penalize_ex's out_row_status.
 *  every other argument, and the errors: as vs_sample_logprobs.
 */
vs_status vs_penalize_sample_logprobs(void* logits, vs_dtype dt, int B, int V, int64_t ld,
                                      const int32_t* prompt_ids, const int32_t* prompt_off,
                                      const int32_t* output_ids, const int32_t* output_off,
                                      const float* presence, const float* frequency,
                                      const float* repetition, const int32_t* prompt_ignore_len,
                                      int32_t* out_penalty_status, const float* temperature,
                                      const int32_t* top_k, const float* top_p,
                                      const float* min_p, const uint64_t* seeds, uint32_t hints,
                                      int32_t* out_ids, int32_t* out_kept_count,
                                      uint32_t* out_kept_mask, int32_t* out_row_status,
                                      float* out_token_logprob, int k, int32_t* out_topk_ids,
                                      float* out_topk_logprobs, float* out_full, int64_t ld_out,
                                      void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * vs_sample_logprobs_noalloc — vs_sample_logprobs without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops that must not call hipMalloc, harnesses that
 * forbid allocation). The call allocates nothing: its kernels use a scratch
 * array that the library holds in device memory, VS_NOALLOC_SCRATCH_BYTES
 * per device, for as long as the process runs.
 *
 *  Arguments, outputs and per-row errors: as vs_sample_logprobs (minus ws and
 *  ws_bytes). The scratch is laid out for the current device's geometry; a
 *  batch whose layout exceeds VS_NOALLOC_SCRATCH_BYTES (about 100 KB per row
 *  plus 2 KB per row segment: B = 1024 rows of 128,256 ids do not fit, 256 rows
 *  of 248,320 do) returns VS_ERR_WORKSPACE_TOO_SMALL and enqueues nothing: use
 *  vs_sample_logprobs with a workspace instead.
 *  Every call on one device shares that device's scratch, whatever the stream:
 *  calls that may overlap in time on one device race and give wrong results;
 *  order them on one stream (or with events). Nothing in the scratch needs
 *  clearing between calls.
 * Errors: as vs_sample_logprobs; VS_ERR_HIP if the scratch's device address
 * cannot be obtained.
 */
#define VS_NOALLOC_SCRATCH_BYTES (64u << 20)
vs_status vs_sample_logprobs_noalloc(const void* logits, vs_dtype dt, int B, int V, int64_t ld,
                                     const float* temperature, const int32_t* top_k,
                                     const float* top_p, const float* min_p,
                                     const uint64_t* seeds, uint32_t hints, int32_t* out_ids,
                                     int32_t* out_kept_count, uint32_t* out_kept_mask,
                                     int32_t* out_row_status, float* out_token_logprob, int k,
                                     int32_t* out_topk_ids, float* out_topk_logprobs,
                                     float* out_full, int64_t ld_out, hipStream_t stream);

/*
 * vs_logprobs — log-softmax log-probabilities of the buffer given (temperature
 * 1, no truncation), as the TT sampling README's LogProbsCalculator ("Key
 * Components": numerically stable log-softmax via the max and the sum of
 * exponentials) and the Tunix sampler page (greedy argmax plus a log-softmax)
 * describe. Computed in fp32: lp_j = (x_j - max) - log(sum exp(x - max)).
 *
 *  token_ids, out_token_logprob: [B] each, or both NULL; lp of the given id.
 *  k            0 <= k <= min(VS_LOGPROB_K_MAX, V)
 *  out_topk_ids, out_topk_logprobs: [B, k] (NULL when k = 0): the k largest
 *               logits, larger first and lower id first among equals.
 *  out_full     [B, ld_out] fp32 or NULL: every lp of the row (ld_out >= V)
 *  out_row_status [B] int32 or NULL. A row with bad logits gets NaN log-probs and
 *               top-k ids -1; an id outside [0,V) gets NaN.
 */
vs_status vs_logprobs(const void* logits, vs_dtype dt, int B, int V, int64_t ld,
                      const int32_t* token_ids, float* out_token_logprob, int k,
                      int32_t* out_topk_ids, float* out_topk_logprobs,
                      float* out_full, int64_t ld_out, int32_t* out_row_status,
                      void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * vs_logprobs_ex — vs_logprobs at a temperature per row ("processed"
 * log-probs): the log-softmax of s = x / T, with s rounded to fp32 as the
 * sampling step forms it (the TensorRT-LLM page: temperature divides the
 * logits; the Tunix sampler divides by the temperature before its softmax).
 * lp_j = (s_j - max s) - log(sum exp(s - max s)); the top-k are the k largest
 * s. A row whose T is not positive and finite takes T = 1; a row where x / T
 * overflows to +inf is a row with bad logits.
 *
 *  temperature [B] fp32, device, or NULL (exactly vs_logprobs). Every other
 *              argument, and the errors, as vs_logprobs.
 */
vs_status vs_logprobs_ex(const void* logits, vs_dtype dt, int B, int V, int64_t ld,
                         const float* temperature, const int32_t* token_ids,
                         float* out_token_logprob, int k, int32_t* out_topk_ids,
                         float* out_topk_logprobs, float* out_full, int64_t ld_out,
                         int32_t* out_row_status, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/*
 * Profiling aid (not part of the sampling step). While active on the calling
 * host thread, every kernel stage that a vs_* call enqueues is bracketed by
 * hipEventRecord(events[2i]) and hipEventRecord(events[2i+1]) on that call's
 * stream, i = 0, 1, ... in enqueue order, until `capacity` events are used.
 * `events` is a host array of events the caller created (hipEventCreate) and
 * owns. Stage names: "select", "row", "full_prep", "row_full", "gumbel",
 * "lse_select", "lse_row", "lse_full", "penalize", "topp_decay",
 * "seed_advance", "slot_remap". vs_profile_end stops recording on this thread,
 * copies up to max_names stage-name pointers (static strings) to `names` (may
 * be NULL) and returns the number of stages recorded.
 */
vs_status vs_profile_begin(hipEvent_t* events, int capacity);
int vs_profile_end(const char** names, int max_names);

#ifdef __cplusplus
}
#endif
#endif /* VS_H */
