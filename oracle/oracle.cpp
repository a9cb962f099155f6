// CPU oracle for batched decode-step token sampling.
//
// TEST INFRASTRUCTURE ONLY: loaded by the test suite, the package smoke check
// and the CPU-baseline leg of the benchmark, never by the product path. It is
// a plain, slow, single-threaded statement of what the sampling step computes,
// written from the source pages and sharing nothing with the GPU library.
// Build: g++ -O2 -ffp-contract=off (no fast-math, no FTZ/DAZ).
//
// Readings of points the pages leave open are stated next to the code they
// govern; each one is also listed in the repository's design notes.

#include "oracle.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <vector>

namespace {

constexpr int kRowBadParam = 1;
constexpr int kRowBadLogits = 2;
constexpr int kRowBadTokenId = 4;
constexpr int kRowTopkUnsupported = 8;
// Largest top-k the library supports (rows with a larger k below V are rejected).
constexpr int kTopKMax = 1024;

float bits_to_float(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
uint32_t float_to_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

float load_logit(const void* base, int dtype, int64_t idx) {
  if (dtype == 0) return static_cast<const float*>(base)[idx];
  // bf16 is the high half of an fp32: widening is exact.
  uint16_t h = static_cast<const uint16_t*>(base)[idx];
  return bits_to_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16 with round-to-nearest-even on the dropped 16 bits.
uint16_t to_bf16(float f) {
  uint32_t u = float_to_bits(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);  // NaN stays NaN
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return static_cast<uint16_t>(u >> 16);
}

void store_logit(void* base, int dtype, int64_t idx, float v) {
  if (dtype == 0)
    static_cast<float*>(base)[idx] = v;
  else
    static_cast<uint16_t*>(base)[idx] = to_bf16(v);
}

// Pinned relative weight E(t) = exp(t) rounded to fp32, and 0 below -87 (so no
// fp32 subnormal ever enters a mass). The pages give probabilities only as the
// softmax of the scaled logits; the rounding of this one function decides
// min-p and top-p membership, so both implementations must agree on it to the
// bit. The definition here is the plain one: libm's double exp, rounded once.
float pinned_exp(float t) {
  if (!(t >= -87.0f)) return 0.0f;
  return static_cast<float>(std::exp(static_cast<double>(t)));
}

// SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014, in the widely used variant with Stafford's Mix13
// finaliser): one output for state x is mix13(x + golden gamma).
uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Uniform in (0,1) for (seed, row, id): two SplitMix64 rounds per element, the
// first keyed by seed and row, the second by the token id (vllm.cpp #1997,
// "two SplitMix64 rounds ... per element", GumbelScore(prob, seed, row, j)).
// The 52 high bits plus one half give an exact double strictly inside (0,1).
double uniform01(uint64_t seed, int row, int id) {
  uint64_t a = splitmix64(seed ^ (static_cast<uint64_t>(static_cast<uint32_t>(row)) << 32));
  uint64_t b = splitmix64(a + static_cast<uint64_t>(static_cast<uint32_t>(id)));
  return (static_cast<double>(b >> 12) + 0.5) * 0x1p-52;
}

bool row_logits_bad(const void* logits, int dtype, int64_t base, int V) {
  bool all_neg_inf = true;
  for (int j = 0; j < V; ++j) {
    float x = load_logit(logits, dtype, base + j);
    if (std::isnan(x) || x == std::numeric_limits<float>::infinity()) return true;
    if (x != -std::numeric_limits<float>::infinity()) all_neg_inf = false;
  }
  return all_neg_inf;
}

bool sample_params_bad(float T, int k, float p, float mp) {
  if (!(T >= 0.0f && T <= std::numeric_limits<float>::max())) return true;
  if (k < 0) return true;
  if (!(p >= 0.0f && p <= 1.0f)) return true;
  if (!(mp >= 0.0f && mp <= 1.0f)) return true;
  return false;
}

// One row of the sampling step. Returns the row status.
int sample_one_row(const void* logits, int dtype, int V, int64_t ld, int r,
                   float T, int k, float p, float mp, uint64_t seed,
                   int32_t* out_id, int32_t* out_kept, uint8_t* mask,
                   double* top2) {
  const int64_t base = static_cast<int64_t>(r) * ld;
  *out_id = -1;
  *out_kept = 0;
  if (mask) std::memset(mask, 0, static_cast<size_t>(V));
  if (top2) { top2[0] = -1.0; top2[1] = -1.0; }

  int status = 0;
  const bool bad_param = sample_params_bad(T, k, p, mp);
  if (bad_param) status |= kRowBadParam;
  if (row_logits_bad(logits, dtype, base, V)) status |= kRowBadLogits;
  // Greedy whenever temperature = 0, top_p = 0, top_k = 1 or min_p = 1,
  // whatever the other parameters say (TensorRT-LLM "Sampling", the
  // Torch Sampler bullets).
  const bool greedy = !bad_param && (T == 0.0f || k == 1 || p == 0.0f || mp == 1.0f);
  const int keff = (k >= V) ? 0 : k;  // top_k = vocab size means no top-k
  if (!bad_param && !greedy && keff > kTopKMax) status |= kRowTopkUnsupported;
  if (status) return status;

  std::vector<float> x(V);
  for (int j = 0; j < V; ++j) x[j] = load_logit(logits, dtype, base + j);

  if (greedy) {
    // Lowest index among the maximal logits.
    int best = 0;
    for (int j = 1; j < V; ++j)
      if (x[j] > x[best]) best = j;
    *out_id = best;
    *out_kept = 1;
    if (mask) mask[best] = 1;
    return 0;
  }

  // Temperature: the logits are divided by T (one correctly rounded fp32
  // division per element).
  std::vector<float> s(V);
  for (int j = 0; j < V; ++j) s[j] = x[j] / T;
  for (int j = 0; j < V; ++j)
    if (s[j] == std::numeric_limits<float>::infinity()) return kRowBadParam;  // x/T overflowed

  // One total order: larger scaled logit first, lower id first among equals.
  std::vector<int> order(V);
  for (int j = 0; j < V; ++j) order[j] = j;
  std::sort(order.begin(), order.end(), [&](int a, int b) {
    if (s[a] != s[b]) return s[a] > s[b];
    return a < b;
  });

  const float m = s[order[0]];
  std::vector<float> e(V);
  for (int j = 0; j < V; ++j) e[j] = pinned_exp(s[j] - m);

  // min-p keeps probability >= min_p * p_max, i.e. e >= min_p because the
  // softmax normaliser cancels and e of the top token is exactly 1. top-k keeps
  // the first keff ids of the order. Both keep a prefix, so they commute.
  const int n0 = (keff > 0) ? keff : V;
  std::vector<int> S;
  for (int i = 0; i < n0; ++i) {
    int j = order[i];
    if (e[j] >= mp) S.push_back(j);
  }

  // top-p on the survivors, renormalised over them: the shortest prefix whose
  // mass reaches p of the survivors' mass. Masses are fixed point,
  // W = floor(e * 2^31), summed exactly; the threshold is one double multiply.
  std::vector<int> K;
  if (p < 1.0f) {
    uint64_t total = 0;
    for (int j : S) total += static_cast<uint64_t>(e[j] * 2147483648.0f);
    const double thr = static_cast<double>(p) * static_cast<double>(total);
    uint64_t cum = 0;
    for (int j : S) {
      K.push_back(j);
      cum += static_cast<uint64_t>(e[j] * 2147483648.0f);
      if (static_cast<double>(cum) >= thr) break;
    }
  } else {
    K = S;
  }

  *out_kept = static_cast<int32_t>(K.size());
  if (mask)
    for (int j : K) mask[j] = 1;

  if (K.size() == 1) {
    *out_id = K[0];
    return 0;
  }

  // Gumbel-max: score = e / q with q = -log(u) in double; the largest score
  // wins and ties go to the lowest id.
  double g1 = -1.0, g2 = -1.0;
  int best = -1;
  for (int j : K) {
    const double q = -std::log(uniform01(seed, r, j));
    const double score = static_cast<double>(e[j]) / q;
    if (score > g1 || (score == g1 && j < best)) {
      g2 = g1;
      g1 = score;
      best = j;
    } else if (score > g2) {
      g2 = score;
    }
  }
  *out_id = best;
  if (top2) { top2[0] = g1; top2[1] = g2; }
  return 0;
}

}  // namespace

extern "C" {

float oracle_exp_pinned(float t) { return pinned_exp(t); }
uint64_t oracle_splitmix64(uint64_t x) { return splitmix64(x); }
double oracle_uniform(uint64_t seed, int row, int id) { return uniform01(seed, row, id); }
uint16_t oracle_f32_to_bf16(float f) { return to_bf16(f); }

long oracle_exp_scan(float lo, float hi, double* max_ulp) {
  long violations = 0;
  double worst = 0.0;
  float prev = 0.0f;
  bool first = true;
  for (float t = lo; t <= hi; t = std::nextafter(t, 1.0f)) {
    const float e = pinned_exp(t);
    if (!first && e < prev) ++violations;
    first = false;
    prev = e;
    // Error against an 80-bit reference, in units of the fp32 spacing there.
    const long double ref = std::exp(static_cast<long double>(t));
    const float rf = static_cast<float>(ref);
    const float up = std::nextafter(rf, std::numeric_limits<float>::infinity());
    const double err = static_cast<double>(std::fabs(static_cast<long double>(e) - ref) /
                                           static_cast<long double>(up - rf));
    if (t >= -87.0f && err > worst) worst = err;
    if (t == hi) break;
  }
  if (max_ulp) *max_ulp = worst;
  return violations;
}

int oracle_penalize(void* logits, int dtype, int B, int V, int64_t ld,
                    const int32_t* prompt_ids, const int32_t* prompt_off,
                    const int32_t* output_ids, const int32_t* output_off,
                    const float* presence, const float* frequency,
                    const float* repetition, const int32_t* prompt_ignore,
                    int32_t* row_status) {
  std::vector<int> count(V);   // every occurrence: the repetition penalty
  std::vector<int> pcount(V);  // occurrences past the ignored prompt prefix
  for (int r = 0; r < B; ++r) {
    int status = 0;
    const float pres = presence ? presence[r] : 0.0f;
    const float freq = frequency ? frequency[r] : 0.0f;
    const float rep = repetition ? repetition[r] : 1.0f;
    // repetition_penalty must be > 0; the other two must be finite.
    const bool bad = !(rep > 0.0f && std::isfinite(rep)) || !std::isfinite(pres) ||
                     !std::isfinite(freq);
    if (bad) status |= kRowBadParam;

    // c = occurrences in the prompt plus occurrences in the generated output.
    // The first n prompt ids (prompt_ignore_length, clamped to [0, prompt
    // length]) count for repetition only.
    std::fill(count.begin(), count.end(), 0);
    std::fill(pcount.begin(), pcount.end(), 0);
    auto add = [&](const int32_t* ids, const int32_t* off, int32_t skip) {
      if (!ids || !off) return;
      for (int32_t i = off[r]; i < off[r + 1]; ++i) {
        const int32_t t = ids[i];
        if (t < 0 || t >= V) {
          status |= kRowBadTokenId;
          continue;
        }
        ++count[t];
        if (i - off[r] >= skip) ++pcount[t];
      }
    };
    const int32_t ign = prompt_ignore ? prompt_ignore[r] : 0;
    add(prompt_ids, prompt_off, ign > 0 ? ign : 0);
    add(output_ids, output_off, 0);

    if (!bad) {
      const int64_t base = static_cast<int64_t>(r) * ld;
      for (int j = 0; j < V; ++j) {
        if (count[j] == 0) continue;
        const float x = load_logit(logits, dtype, base + j);
        // repetition: divide a non-negative logit, multiply a negative one;
        // then presence; then frequency times the count. Each step is one
        // rounded fp32 operation, no fused multiply-add.
        float y = (x >= 0.0f) ? x / rep : x * rep;
        if (pcount[j] > 0) {
          y = y - pres;
          const float fc = freq * static_cast<float>(pcount[j]);
          y = y - fc;
        }
        store_logit(logits, dtype, base + j, y);
      }
    }
    if (row_status) row_status[r] = status;
  }
  return 0;
}

long oracle_exp_compare(uint32_t lo_bits, uint32_t n, const float* got, uint32_t* first_bad) {
  long bad = 0;
  uint32_t first = n;
  for (uint32_t i = 0; i < n; ++i) {
    uint32_t b = lo_bits + i;
    float t;
    std::memcpy(&t, &b, sizeof t);
    const float want = oracle_exp_pinned(t);
    uint32_t wb, gb;
    std::memcpy(&wb, &want, sizeof wb);
    std::memcpy(&gb, &got[i], sizeof gb);
    if (wb != gb) {
      if (first == n) first = i;
      ++bad;
    }
  }
  if (first_bad) *first_bad = first;
  return bad;
}

int oracle_slot_remap(int B, int B_src, const int32_t* remap, const void* src, void* dst,
                      int elem_bytes, int32_t* row_status) {
  for (int i = 0; i < B; ++i) {
    const int32_t j = remap[i];  // new slot i continues the request of old slot j
    if (row_status) row_status[i] = (j >= B_src) ? kRowBadParam : 0;
    if (j < 0 || j >= B_src) continue;
    std::memcpy(static_cast<char*>(dst) + static_cast<int64_t>(i) * elem_bytes,
                static_cast<const char*>(src) + static_cast<int64_t>(j) * elem_bytes, elem_bytes);
  }
  return 0;
}

int oracle_topp_decay(int B, float* top_p, const float* top_p_init, const float* decay,
                      const float* top_p_min, const int32_t* reset_ids,
                      const int32_t* sampled, int32_t* row_status) {
  for (int r = 0; r < B; ++r) {
    const float d = decay[r];
    const float lo = top_p_min ? top_p_min[r] : 1e-6f;
    const float p0 = top_p_init[r];
    const int32_t reset = reset_ids ? reset_ids[r] : -1;
    // the page rejects a decay or floor outside (0, 1] and a negative reset
    // id other than the "no reset id" value -1
    const bool bad = !(d > 0.0f && d <= 1.0f) || !(lo > 0.0f && lo <= 1.0f) ||
                     !(p0 >= 0.0f && p0 <= 1.0f) || reset < -1;
    if (row_status) row_status[r] = bad ? kRowBadParam : 0;
    if (bad || sampled[r] < 0) continue;  // no token was sampled: nothing decays
    if (reset >= 0 && sampled[r] == reset) {
      top_p[r] = p0;  // the reset id was sampled: back to the initial top_p
    } else {
      const float p = top_p[r] * d;  // one rounded fp32 product
      top_p[r] = p > lo ? p : lo;    // bounded from below
    }
  }
  return 0;
}

int oracle_seed_advance(int B, uint64_t* seeds, const int32_t* sampled) {
  for (int r = 0; r < B; ++r)
    if (!sampled || sampled[r] >= 0) seeds[r] += 0x9E3779B97F4A7C15ull;
  return 0;
}

int oracle_sample_row(const void* logits, int dtype, int B, int V, int64_t ld,
                      int r, const float* temperature, const int32_t* top_k,
                      const float* top_p, const float* min_p,
                      const uint64_t* seeds, int32_t* out_ids,
                      int32_t* out_kept_count, uint8_t* out_kept_mask,
                      double* out_top2, int32_t* row_status) {
  if (r < 0 || r >= B) return 1;
  // A parameter array left out (NULL) gives every row its neutral value
  // (T = 1, top_k = 0, top_p = 1, min_p = 0, seed 0); with temperature, top_k
  // and top_p all left out the rows are greedy (TensorRT-LLM "Sampling", LLM
  // API sampling behavior: none of the three set means greedy), here T = 0.
  const bool unset = !temperature && !top_k && !top_p;
  const float T = temperature ? temperature[r] : (unset ? 0.0f : 1.0f);
  int32_t kept = 0;
  const int status = sample_one_row(
      logits, dtype, V, ld, r, T, top_k ? top_k[r] : 0, top_p ? top_p[r] : 1.0f,
      min_p ? min_p[r] : 0.0f, seeds ? seeds[r] : 0ull, &out_ids[r], &kept,
      out_kept_mask ? out_kept_mask + static_cast<int64_t>(r) * V : nullptr,
      out_top2 ? out_top2 + 2 * r : nullptr);
  if (out_kept_count) out_kept_count[r] = kept;
  if (row_status) row_status[r] = status;
  return 0;
}

int oracle_sample(const void* logits, int dtype, int B, int V, int64_t ld,
                  const float* temperature, const int32_t* top_k,
                  const float* top_p, const float* min_p, const uint64_t* seeds,
                  int32_t* out_ids, int32_t* out_kept_count,
                  uint8_t* out_kept_mask, double* out_top2, int32_t* row_status) {
  for (int r = 0; r < B; ++r)
    oracle_sample_row(logits, dtype, B, V, ld, r, temperature, top_k, top_p, min_p,
                      seeds, out_ids, out_kept_count, out_kept_mask, out_top2,
                      row_status);
  return 0;
}

int oracle_logprobs(const void* logits, int dtype, int B, int V, int64_t ld,
                    const int32_t* token_ids, double* out_token_lp, int k,
                    int32_t* out_topk_ids, double* out_topk_lp,
                    double* out_full, int32_t* row_status) {
  return oracle_logprobs_t(logits, dtype, B, V, ld, nullptr, token_ids, out_token_lp, k,
                           out_topk_ids, out_topk_lp, out_full, row_status);
}

int oracle_logprobs_t(const void* logits, int dtype, int B, int V, int64_t ld,
                      const float* temperature, const int32_t* token_ids, double* out_token_lp,
                      int k, int32_t* out_topk_ids, double* out_topk_lp, double* out_full,
                      int32_t* row_status) {
  const double nan = std::numeric_limits<double>::quiet_NaN();
  std::vector<double> z(V);
  std::vector<int> order(V);
  for (int r = 0; r < B; ++r) {
    const int64_t base = static_cast<int64_t>(r) * ld;
    int status = 0;
    // The log-probs are those of s = x / T, one rounded fp32 division as the
    // sampling step forms s; a temperature that is not positive and finite
    // means T = 1. The row checks apply to s (x / T may overflow).
    float T = temperature ? temperature[r] : 1.0f;
    if (!(T > 0.0f && T <= std::numeric_limits<float>::max())) T = 1.0f;
    bool all_neg_inf = true, bad = false;
    for (int j = 0; j < V; ++j) {
      const float x = load_logit(logits, dtype, base + j);
      const float s = (T == 1.0f) ? x : x / T;
      if (std::isnan(s) || s == std::numeric_limits<float>::infinity()) bad = true;
      if (s != -std::numeric_limits<float>::infinity()) all_neg_inf = false;
      z[j] = static_cast<double>(s);
    }
    if (bad || all_neg_inf) status |= kRowBadLogits;
    if (token_ids && (token_ids[r] < 0 || token_ids[r] >= V)) status |= kRowBadTokenId;
    if (row_status) row_status[r] = status;
    if (status & kRowBadLogits) {
      if (out_token_lp) out_token_lp[r] = nan;
      for (int i = 0; i < k; ++i) {
        out_topk_ids[static_cast<int64_t>(r) * k + i] = -1;
        out_topk_lp[static_cast<int64_t>(r) * k + i] = nan;
      }
      if (out_full)
        for (int j = 0; j < V; ++j) out_full[static_cast<int64_t>(r) * V + j] = nan;
      continue;
    }
    // Numerically stable log-softmax: subtract the row max, sum the
    // exponentials, subtract the log of the sum.
    double M = z[0];
    for (int j = 1; j < V; ++j) M = std::max(M, z[j]);
    double S = 0.0;
    for (int j = 0; j < V; ++j) S += std::exp(z[j] - M);
    const double logS = std::log(S);
    auto lp = [&](int j) { return (z[j] - M) - logS; };

    if (out_token_lp) out_token_lp[r] = (status & kRowBadTokenId) ? nan : lp(token_ids[r]);
    if (k > 0) {
      for (int j = 0; j < V; ++j) order[j] = j;
      std::sort(order.begin(), order.end(), [&](int a, int b) {
        if (z[a] != z[b]) return z[a] > z[b];
        return a < b;
      });
      for (int i = 0; i < k; ++i) {
        out_topk_ids[static_cast<int64_t>(r) * k + i] = order[i];
        out_topk_lp[static_cast<int64_t>(r) * k + i] = lp(order[i]);
      }
    }
    if (out_full)
      for (int j = 0; j < V; ++j) out_full[static_cast<int64_t>(r) * V + j] = lp(j);
  }
  return 0;
}

}  // extern "C"
