// Device-side building blocks shared by the sampling kernels (gfx950, wave64).
//
// Numeric conventions (the same ones the C ABI documents):
//  - order: larger value first, lower id first among equals; -0 equals +0;
//  - ordered key of an fp32 value: a uint32 whose unsigned order is the float
//    order (-0 canonicalised to +0), packed with the id as
//    (key << 32) | ~id so that one uint64 comparison gives the full order;
//  - relative weight e = exp(t) rounded to fp32 for t >= -87, else 0;
//  - Gumbel uniforms from SplitMix64 keyed by (seed, row, id).
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

#include "../../include/vs.h"

namespace vsk {

constexpr int kWave = 64;
constexpr int kFastK = 64;     // top-k handled by the per-tile fast path
constexpr float kInf = __builtin_inff();

// ---------------------------------------------------------------- keys
__device__ __forceinline__ uint32_t f2key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t pack(uint32_t key, int32_t id) {
  return (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(id));
}
__device__ __forceinline__ uint32_t pkey(uint64_t p) { return static_cast<uint32_t>(p >> 32); }
__device__ __forceinline__ int32_t pid(uint64_t p) {
  return static_cast<int32_t>(~static_cast<uint32_t>(p));
}
constexpr uint32_t kKeyNegInf = 0x007fffffu;  // f2key(-inf)
constexpr uint32_t kKeyPosInf = 0xff800000u;  // f2key(+inf)

// ---------------------------------------------------------------- element access
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// 16-byte vector loads: elements per vector and unpacking to fp32.
template <typename E>
struct Epv;
template <>
struct Epv<float> {
  static constexpr int n = 4;
};
template <>
struct Epv<uint16_t> {
  static constexpr int n = 8;
};

__device__ __forceinline__ void unpack16(const uint4& u, float* x, const float*) {
  x[0] = __uint_as_float(u.x);
  x[1] = __uint_as_float(u.y);
  x[2] = __uint_as_float(u.z);
  x[3] = __uint_as_float(u.w);
}
__device__ __forceinline__ void unpack16(const uint4& u, float* x, const uint16_t*) {
  x[0] = __uint_as_float(u.x << 16);
  x[1] = __uint_as_float(u.x & 0xffff0000u);
  x[2] = __uint_as_float(u.y << 16);
  x[3] = __uint_as_float(u.y & 0xffff0000u);
  x[4] = __uint_as_float(u.z << 16);
  x[5] = __uint_as_float(u.z & 0xffff0000u);
  x[6] = __uint_as_float(u.w << 16);
  x[7] = __uint_as_float(u.w & 0xffff0000u);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16(const void* p) {
  const u32x4 t = *reinterpret_cast<const u32x4*>(p);
  return make_uint4(t.x, t.y, t.z, t.w);
}
// Streaming read hint (non-temporal): data read once need not stay in L2.
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// ---------------------------------------------------------------- pinned exp
// exp(t) rounded once to fp32 for t >= -87, 0 below. Evaluated in double:
// Cody & Waite range reduction t = n*ln2 + r with ln2 split into a high part
// (low 11 mantissa bits cleared, so n*hi is exact) and a low part, a degree-13
// Taylor polynomial for e^r on |r| <= ln2/2 (truncation error < 5e-18), and an
// exact scaling by 2^n. Its double result is within a few 1e-17 of e^t, so the
// final fp32 rounding is the correctly rounded value; the oracle states this
// function as libm's exp rounded to fp32 and the tests compare the two.
//
// c + a * b in double with the constant c read from scalar registers: one
// VALU instruction per step. (Left to itself the compiler copies each 64-bit
// constant into a vector register first, since the VOP3 form cannot take a
// 64-bit literal; that doubles the instruction count of the polynomial.)
// Only the named constant operand goes to scalar registers: every other
// operand is a per-lane value.
__device__ __forceinline__ double fma_k(double a, double b, double c) {
  double d;
  asm("v_fma_f64 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "s"(c));
  return d;
}
// c - n * k with the constant k from scalar registers.
__device__ __forceinline__ double fnma_k(double n, double k, double c) {
  double d;
  asm("v_fma_f64 %0, -%1, %2, %3" : "=v"(d) : "v"(n), "s"(k), "v"(c));
  return d;
}
// pinned_exp of N values at once, the same operations on each, issued in
// turn across the N values (the constant-operand FMAs are inline asm, which
// the compiler keeps in source order: written value by value, the N
// dependent chains would run one after the other).
template <int N>
__device__ __forceinline__ void pinned_exp_n(const float* tf, float* out) {
  // the Taylor coefficients of exp after the leading 1/13!, highest first
  constexpr double kC[13] = {1.0 / 479001600.0, 1.0 / 39916800.0, 1.0 / 3628800.0,
                             1.0 / 362880.0,    1.0 / 40320.0,    1.0 / 5040.0,
                             1.0 / 720.0,       1.0 / 120.0,      1.0 / 24.0,
                             1.0 / 6.0,         0.5,              1.0,
                             1.0};
  double r[N], p[N], n[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const double t = static_cast<double>(fminf(fmaxf(tf[i], -87.5f), 128.0f));
    n[i] = rint(t * 1.4426950408889634);
    r[i] = fnma_k(n[i], 0x1.62e42fefa3800p-1, t);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) r[i] = fnma_k(n[i], 0x1.ef35793c76730p-45, r[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) p[i] = fma_k(1.0 / 6227020800.0, r[i], kC[0]);
#pragma unroll
  for (int k = 1; k < 13; ++k) {
#pragma unroll
    for (int i = 0; i < N; ++i) p[i] = fma_k(p[i], r[i], kC[k]);
  }
  // n is an integer in [-127, 185]; p * 2^n is exact in double (and above
  // the fp32 range from t = 88.73 on, where the conversion gives +inf)
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float y = static_cast<float>(ldexp(p[i], static_cast<int>(n[i])));
    out[i] = tf[i] >= -87.0f ? y : 0.0f;  // below -87 (and NaN): 0
  }
}
__device__ __forceinline__ float pinned_exp(float tf) {
  float e;
  pinned_exp_n<1>(&tf, &e);
  return e;
}

// Fixed-point top-p mass of a relative weight e in [0,1]: floor(e * 2^31).
__device__ __forceinline__ uint64_t mass_of(float e) {
  return static_cast<uint64_t>(static_cast<uint32_t>(e * 2147483648.0f));
}

// ---------------------------------------------------------------- random stream
// SplitMix64 (Steele, Lea, Flood 2014; Mix13 finaliser): output for state x.
__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
__device__ __forceinline__ uint64_t row_stream(uint64_t seed, int row) {
  return splitmix64(seed ^ (static_cast<uint64_t>(static_cast<uint32_t>(row)) << 32));
}
// The random word of an id, and the uniform strictly inside (0,1) made from
// it: its top 52 bits plus one half, times 2^-52.
__device__ __forceinline__ uint64_t random_bits(uint64_t row_state, int id) {
  return splitmix64(row_state + static_cast<uint64_t>(static_cast<uint32_t>(id)));
}
__device__ __forceinline__ double uniform_of_bits(uint64_t b) {
  return (static_cast<double>(b >> 12) + 0.5) * 0x1p-52;
}
__device__ __forceinline__ double uniform_of(uint64_t row_state, int id) {
  return uniform_of_bits(random_bits(row_state, id));
}
// The high half of an id's random word (the compiler leaves out what only
// the low half needs).
__device__ __forceinline__ uint32_t random_hi(uint64_t row_state, int id) {
  return static_cast<uint32_t>(random_bits(row_state, id) >> 32);
}
// The Gumbel draw's skip test on the high half of a random word. A kept id
// with e <= eub and random word b cannot beat a best score S when
// 1 - u >= (1 + 2^-40) e / S (-log u > 1 - u; the margin covers the
// rounding of the scores); the integer form of that test takes the words
// below (1 - L) 2^64 (up to a few units of 2^12), L = lim * eub with
// lim = (1 + 2^-40) / S. skip_hi returns a bound H on the high half such that
// b >> 32 < H implies that test, evaluated in fp32: lim_up is a float at or
// above lim (up_of), the product is raised past its rounding, and 1 - L,
// scaled by 2^32, is lowered by 256 units past the rounding of the
// subtraction (NaN and L >= 1 give 0: nothing skipped).
__device__ __forceinline__ float up_of(double lim) {
  // float(lim) is within 2^-24 of lim; 2^-21 above it stays above lim after
  // the product's own rounding (and is infinite past the float range)
  return static_cast<float>(lim) * (1.0f + 0x1p-21f);
}
__device__ __forceinline__ uint32_t skip_hi(float lim_up, float eub) {
  const float L = lim_up * eub;                  // >= lim * eub (1 + 2^-23)
  const float t = (1.0f - L) * 4294967296.0f;    // within 2^7 of (1 - L) 2^32
  const uint32_t h = t >= 4294967040.0f ? 4294967040u : (t > 256.0f ? static_cast<uint32_t>(t) : 256u);
  return h - 256u;
}

// The random words b below which an id cannot beat the score bound lim:
// with u = ((b >> 12) + 1/2) 2^-52, every b < skip_below(lim) has
// 1 - u >= lim (1 + 2^-45) + 2^-52, so (1 - u)(1 - 2^-50) rounded stays
// >= lim and the id scores below the bound (0: no b, while lim >= 1).
__device__ __forceinline__ uint64_t skip_below(double lim) {
  if (!(lim < 1.0)) return 0ull;
  // (1 - lim (1 + 2^-45)) 2^52 - 2, whose rounding errors stay below 1.5
  const double v = (1.0 - lim * (1.0 + 0x1p-45)) * 0x1p52 - 2.0;
  if (!(v > 0.0)) return 0ull;
  return static_cast<uint64_t>(v) << 12;  // floor(v) < 2^52
}

// Gumbel-max score prob / q with q = -log(u) (exponential noise), in double.
__device__ __forceinline__ double gumbel_score(float e, uint64_t row_state, int id) {
  const double q = -log(uniform_of(row_state, id));
  return static_cast<double>(e) / q;
}

// ---------------------------------------------------------------- row modes
enum : int { kModeInvalid = 0, kModeGreedy = 1, kModeKFast = 2, kModeKSlow = 3, kModeFull = 4 };

struct RowCfg {
  int mode;
  int status;
  float T;
  int k;      // effective top-k (0 = none)
  float p;
  float mp;
  uint64_t seed;
};

// A row's parameters as the caller's arrays give them: arrays left out take
// neutral values; temperature, top_k and top_p all left out make every row
// greedy (TensorRT-LLM "Sampling": none of the three set means greedy), as T = 0.
struct RowParams {
  float T, p, mp;
  int k;
  uint64_t seed;
};
__device__ __forceinline__ RowParams load_params(int r, const float* temperature,
                                                 const int32_t* top_k, const float* top_p,
                                                 const float* min_p, const uint64_t* seeds) {
  RowParams a;
  a.T = temperature ? temperature[r] : ((!top_k && !top_p) ? 0.0f : 1.0f);
  a.k = top_k ? top_k[r] : 0;
  a.p = top_p ? top_p[r] : 1.0f;
  a.mp = min_p ? min_p[r] : 0.0f;
  a.seed = seeds ? seeds[r] : 0ull;
  return a;
}
// The row's mode and status from its parameters.
__device__ __forceinline__ RowCfg cfg_of(const RowParams& a, int V) {
  RowCfg c;
  c.T = a.T;
  const int k = a.k;
  c.p = a.p;
  c.mp = a.mp;
  c.seed = a.seed;
  c.mode = kModeInvalid;
  c.status = 0;
  c.k = k;
  const bool bad = !(c.T >= 0.0f && c.T <= 3.40282347e38f) || k < 0 ||
                   !(c.p >= 0.0f && c.p <= 1.0f) || !(c.mp >= 0.0f && c.mp <= 1.0f);
  if (bad) {
    c.status = VS_ROW_BAD_PARAM;
    return c;
  }
  if (c.T == 0.0f || k == 1 || c.p == 0.0f || c.mp == 1.0f) {
    c.mode = kModeGreedy;
    return c;
  }
  c.k = (k >= V) ? 0 : k;
  if (c.k > VS_TOPK_MAX) {
    c.status = VS_ROW_TOPK_UNSUPPORTED;
    return c;
  }
  c.mode = (c.k == 0) ? kModeFull : (c.k <= kFastK ? kModeKFast : kModeKSlow);
  return c;
}
__device__ __forceinline__ RowCfg load_cfg(int r, int V, const float* temperature,
                                           const int32_t* top_k, const float* top_p,
                                           const float* min_p, const uint64_t* seeds) {
  return cfg_of(load_params(r, temperature, top_k, top_p, min_p, seeds), V);
}

// ---------------------------------------------------------------- workspace records
// Per-row record handed from the row kernel to the full-vocabulary kernels.
struct RowDesc {
  uint32_t mode;
  float m;         // max over the row of s = x / T
  uint32_t tau;    // top-p: ordered key of the last kept value
  int32_t id_cut;  // top-p: largest kept id among those whose key equals tau
  int32_t kept;    // kept-set size as found by the cut (top-p)
  uint32_t pad[3];
};

struct GPart {  // Gumbel partial result of one tile
  double score;
  int32_t id;
  int32_t kept;
  float s;  // the best id's s = x / T, where the gather pass drew (else 0)
};

struct LsePart {  // log-sum-exp partial of one tile: max and sum of exp(x - max)
  float m;
  float s;
};

// ---------------------------------------------------------------- wave primitives
__device__ __forceinline__ int lane() { return static_cast<int>(__lane_id()); }

// The value of lane (this lane XOR J) for J = 1, 2, 4, 8, 16, 32, every lane
// active: DPP quad permutations for 1 and 2, row shifts into alternate banks
// for 4, a row rotation by 8, and the gfx950 row-pair and half-wave swaps for
// 16 and 32 (a copy of the value in both operands, so each lane finds its
// partner in one of the two results).
template <int J>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t x) {
  const int v = static_cast<int>(x);
  // (the moves below write every lane, so no old value is set up first; for
  // J = 4 the second move writes the lanes the first one leaves)
  if constexpr (J == 1) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));
  } else if constexpr (J == 2) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));
  } else if constexpr (J == 4) {
    const int t = __builtin_amdgcn_mov_dpp(v, 0x104, 0xF, 0x5, false);  // row_shl:4, banks 0, 2
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(t, v, 0x114, 0xF, 0xA, false));  // row_shr:4
  } else if constexpr (J == 8) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false));  // row_ror:8
  } else if constexpr (J == 16) {
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    // lanes with bit 4 set, as a wave mask (no per-lane test)
    return __builtin_amdgcn_inverse_ballot_w64(0xFFFF0000FFFF0000ull) ? a[0] : a[1];
  } else {
    static_assert(J == 32, "lane_xor_u32: J in {1, 2, 4, 8, 16, 32}");
    const auto a = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return __builtin_amdgcn_inverse_ballot_w64(0xFFFFFFFF00000000ull) ? a[0] : a[1];
  }
}
template <int J>
__device__ __forceinline__ uint64_t lane_xor_u64(uint64_t x) {
  const uint32_t lo = lane_xor_u32<J>(static_cast<uint32_t>(x));
  const uint32_t hi = lane_xor_u32<J>(static_cast<uint32_t>(x >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
// The value of lane (this lane XOR J) for a 32- or 64-bit value of any type.
template <int J, typename T>
__device__ __forceinline__ T lane_xor(T v) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "lane_xor: 32- or 64-bit values");
  if constexpr (sizeof(T) == 4) {
    const uint32_t u = lane_xor_u32<J>(__builtin_bit_cast(uint32_t, v));
    return __builtin_bit_cast(T, u);
  } else {
    const uint64_t u = lane_xor_u64<J>(__builtin_bit_cast(uint64_t, v));
    return __builtin_bit_cast(T, u);
  }
}


// lane_xor for a partner distance known only at run time (uniform over the
// wave: a scalar branch picks the exchange).
template <typename T>
__device__ __forceinline__ T lane_xor_rt(T v, int j) {
  switch (j) {
    case 1: return lane_xor<1>(v);
    case 2: return lane_xor<2>(v);
    case 4: return lane_xor<4>(v);
    case 8: return lane_xor<8>(v);
    case 16: return lane_xor<16>(v);
    default: return lane_xor<32>(v);
  }
}
// Butterfly reductions over the wave (every lane gets the result), the
// exchanges by DPP and gfx950 lane swaps rather than through LDS.
template <typename T, typename F>
__device__ __forceinline__ T wave_reduce(T v, F op) {
  v = op(v, lane_xor<32>(v));
  v = op(v, lane_xor<16>(v));
  v = op(v, lane_xor<8>(v));
  v = op(v, lane_xor<4>(v));
  v = op(v, lane_xor<2>(v));
  v = op(v, lane_xor<1>(v));
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
  return wave_reduce(v, [](T a, T b) { return (b > a) ? b : a; });
}
template <typename T>
__device__ __forceinline__ T wave_min(T v) {
  return wave_reduce(v, [](T a, T b) { return (b < a) ? b : a; });
}
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  return wave_reduce(v, [](T a, T b) { return a + b; });
}
// Number of set bits of a ballot below this lane.
__device__ __forceinline__ int lanes_below(uint64_t ballot) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(ballot >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(ballot), 0u));
}
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}
// Cross-lane exchange through LDS inside one wave: wait for this wave's LDS
// operations only (lgkmcnt(0); vector-memory and export counters left at their
// maxima, gfx9 encoding) and keep the compiler from moving memory operations
// across. Outstanding global stores are not waited for.
__device__ __forceinline__ void wave_lds_wait() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_wave_barrier();
  __asm__ volatile("" ::: "memory");
}

// DPP lane movement within rows of 16 lanes (gfx9 encodings): quad_perm,
// row_ror. Every lane has a valid source for these controls.
constexpr int kDppXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRor4 = 0x124;   // row_ror:4
constexpr int kDppRor8 = 0x128;   // row_ror:8
// (every lane is written, so no old value is set up first)
template <int kCtrl>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_mov_dpp(v, kCtrl, 0xF, 0xF, false);
}
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(dpp_i32<kCtrl>(__float_as_int(v)));
}
__device__ __forceinline__ float readlane_f32(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// Wave-wide max of a u32, max / sum of an fp32 (uniform result): all-reduce
// inside each row of 16 lanes with DPP, then combine the four rows through
// scalar reads. fmaxf ignores NaN. The summation order is fixed, so results are
// reproducible.
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
  v = max(v, static_cast<uint32_t>(dpp_i32<kDppXor1>(static_cast<int>(v))));
  v = max(v, static_cast<uint32_t>(dpp_i32<kDppXor2>(static_cast<int>(v))));
  v = max(v, static_cast<uint32_t>(dpp_i32<kDppRor4>(static_cast<int>(v))));
  v = max(v, static_cast<uint32_t>(dpp_i32<kDppRor8>(static_cast<int>(v))));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}
template <int kCtrl>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = static_cast<uint32_t>(dpp_i32<kCtrl>(static_cast<int>(static_cast<uint32_t>(v))));
  const uint32_t hi = static_cast<uint32_t>(dpp_i32<kCtrl>(static_cast<int>(static_cast<uint32_t>(v >> 32))));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), l);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
// Wave-wide max of a u64 (every lane active).
__device__ __forceinline__ uint64_t wave_max_u64_dpp(uint64_t v) {
  uint64_t o = dpp_u64<kDppXor1>(v);
  v = o > v ? o : v;
  o = dpp_u64<kDppXor2>(v);
  v = o > v ? o : v;
  o = dpp_u64<kDppRor4>(v);
  v = o > v ? o : v;
  o = dpp_u64<kDppRor8>(v);
  v = o > v ? o : v;
  const uint64_t a = readlane_u64(v, 0), b = readlane_u64(v, 16);
  const uint64_t c = readlane_u64(v, 32), d = readlane_u64(v, 48);
  const uint64_t ab = a > b ? a : b, cd = c > d ? c : d;
  return ab > cd ? ab : cd;
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppRor4>(v));
  v = fmaxf(v, dpp_f32<kDppRor8>(v));
  return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)),
               fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppRor4>(v);
  v += dpp_f32<kDppRor8>(v);
  return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}
__device__ __forceinline__ int wave_sum_dpp_i32(int v) {
  v += dpp_i32<kDppXor1>(v);
  v += dpp_i32<kDppXor2>(v);
  v += dpp_i32<kDppRor4>(v);
  v += dpp_i32<kDppRor8>(v);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}
__device__ __forceinline__ int wave_min_dpp(int v) {
  v = min(v, dpp_i32<kDppXor1>(v));
  v = min(v, dpp_i32<kDppXor2>(v));
  v = min(v, dpp_i32<kDppRor4>(v));
  v = min(v, dpp_i32<kDppRor8>(v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Inclusive prefix sum of a u32 over the 64 lanes in lane order (every lane
// active; the caller keeps the sums below 2^32). Within each row of 16 lanes:
// the shifts by 1, 2 and 3 of the inputs give 4-lane window sums, then the
// shifts by 4 (banks 1-3) and by 8 (banks 2-3) of the running sums complete
// the row; the row broadcasts of lane 15 (into rows 1 and 3) and of lane 31
// (into rows 2 and 3) carry the totals across rows (gfx9 DPP encodings).
__device__ __forceinline__ uint32_t wave_scan_incl_u32(uint32_t v) {
  const int x0 = static_cast<int>(v);
  int x = x0;
  x += __builtin_amdgcn_update_dpp(0, x0, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x0, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x0, 0x113, 0xF, 0xF, false);  // row_shr:3
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xE, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xC, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return static_cast<uint32_t>(x);
}

// The same inclusive prefix sum for a u64 (sums below 2^64): each step moves
// both halves with the same DPP control (masked lanes read 0) and adds with
// carry.
template <int kCtrl, int kRowMask, int kBankMask>
__device__ __forceinline__ uint64_t dpp_mv_u64(uint64_t x) {
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(x)), kCtrl,
                                             kRowMask, kBankMask, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(x >> 32)),
                                             kCtrl, kRowMask, kBankMask, false);
  return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}
__device__ __forceinline__ uint64_t wave_scan_incl_u64(uint64_t v) {
  const uint64_t x0 = v;
  uint64_t x = x0;
  x += dpp_mv_u64<0x111, 0xF, 0xF>(x0);  // row_shr:1..3 of the inputs
  x += dpp_mv_u64<0x112, 0xF, 0xF>(x0);
  x += dpp_mv_u64<0x113, 0xF, 0xF>(x0);
  x += dpp_mv_u64<0x114, 0xF, 0xE>(x);   // row_shr:4, banks 1-3
  x += dpp_mv_u64<0x118, 0xF, 0xC>(x);   // row_shr:8, banks 2-3
  x += dpp_mv_u64<0x142, 0xA, 0xF>(x);   // row_bcast:15 into rows 1 and 3
  x += dpp_mv_u64<0x143, 0xC, 0xF>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}

// The lanes that keep the larger value of their pair in a bitonic step (block
// size K, partner distance J), as a wave mask fixed at compile time.
template <int K, int J, bool kDesc>
__host__ __device__ constexpr uint64_t keep_max_lanes() {
  uint64_t m = 0;
  for (int i = 0; i < 64; ++i)
    if ((((i & K) == 0) == ((i & J) == 0)) == kDesc) m |= 1ull << i;
  return m;
}
// One compare-exchange step of a bitonic network over the 64 lanes (block
// size K, partner distance J); kDesc: the finished sequence is descending. A
// lane takes its partner's value when the partner's is larger and the lane
// keeps the larger one, or not larger and it keeps the smaller (equal values
// are the same either way): one compare, the lane pattern as a scalar mask.
template <int K, int J, bool kDesc>
__device__ __forceinline__ uint64_t bitonic_step(uint64_t v) {
  const uint64_t o = lane_xor_u64<J>(v);
  constexpr uint64_t kKeepMax = keep_max_lanes<K, J, kDesc>();
  const bool keep_max = __builtin_amdgcn_inverse_ballot_w64(kKeepMax);
  return (o > v) == keep_max ? o : v;
}
// The last six steps of a bitonic merge whose runs are longer than the wave:
// a bitonic sequence over the 64 lanes comes out sorted (descending with
// kDesc, else ascending).
template <bool kDesc>
__device__ __forceinline__ uint64_t wave_merge_steps(uint64_t v) {
  v = bitonic_step<64, 32, kDesc>(v);
  v = bitonic_step<64, 16, kDesc>(v);
  v = bitonic_step<64, 8, kDesc>(v);
  v = bitonic_step<64, 4, kDesc>(v);
  v = bitonic_step<64, 2, kDesc>(v);
  v = bitonic_step<64, 1, kDesc>(v);
  return v;
}
// Sorts one u64 per lane across the wave in registers (lane 0 first).
template <bool kDesc>
__device__ __forceinline__ uint64_t wave_sort_u64(uint64_t v) {
  v = bitonic_step<2, 1, kDesc>(v);
  v = bitonic_step<4, 2, kDesc>(v);
  v = bitonic_step<4, 1, kDesc>(v);
  v = bitonic_step<8, 4, kDesc>(v);
  v = bitonic_step<8, 2, kDesc>(v);
  v = bitonic_step<8, 1, kDesc>(v);
  v = bitonic_step<16, 8, kDesc>(v);
  v = bitonic_step<16, 4, kDesc>(v);
  v = bitonic_step<16, 2, kDesc>(v);
  v = bitonic_step<16, 1, kDesc>(v);
  v = bitonic_step<32, 16, kDesc>(v);
  v = bitonic_step<32, 8, kDesc>(v);
  v = bitonic_step<32, 4, kDesc>(v);
  v = bitonic_step<32, 2, kDesc>(v);
  v = bitonic_step<32, 1, kDesc>(v);
  v = bitonic_step<64, 32, kDesc>(v);
  v = bitonic_step<64, 16, kDesc>(v);
  v = bitonic_step<64, 8, kDesc>(v);
  v = bitonic_step<64, 4, kDesc>(v);
  v = bitonic_step<64, 2, kDesc>(v);
  v = bitonic_step<64, 1, kDesc>(v);
  return v;
}
// The 64 largest of a (descending across the lanes) and b (ascending),
// descending: the lane-wise maxima form a bitonic sequence holding them,
// which the last six steps sort.
__device__ __forceinline__ uint64_t wave_merge_top_u64(uint64_t a_desc, uint64_t b_asc) {
  return wave_merge_steps<true>(a_desc > b_asc ? a_desc : b_asc);
}

// k-th largest (1-based, 1 <= k <= 64) of one uint32 per lane, every lane of
// the wave active: MSB-first radix select on ballots (32 rounds of one vector
// compare and scalar bit counts; no LDS traffic).
__device__ __forceinline__ uint32_t wave_kth_largest(uint32_t key, int k) {
  uint64_t cand = ~0ull;
  uint32_t prefix = 0;
#pragma unroll 4
  for (int b = 31; b >= 0; --b) {
    const uint64_t ones = __ballot((key >> b) & 1u) & cand;
    const int c = __popcll(ones);
    if (c >= k) {
      cand = ones;
      prefix |= 1u << b;
    } else {
      k -= c;
      cand &= ~ones;
    }
  }
  return prefix;
}
// Same over two uint32 per lane (k <= 128).
// The k-th largest of the 64 * N keys held N per lane (1 <= k <= 64 * N),
// MSB-first with one ballot per key slot and bit.
template <int N>
__device__ __forceinline__ uint32_t wave_kth_largest_n(const uint32_t (&key)[N], int k) {
  uint64_t cand[N];
#pragma unroll
  for (int i = 0; i < N; ++i) cand[i] = ~0ull;
  uint32_t prefix = 0;
#pragma unroll 4
  for (int b = 31; b >= 0; --b) {
    uint64_t ones[N];
    int c = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      ones[i] = __ballot((key[i] >> b) & 1u) & cand[i];
      c += __popcll(ones[i]);
    }
    if (c >= k) {
#pragma unroll
      for (int i = 0; i < N; ++i) cand[i] = ones[i];
      prefix |= 1u << b;
    } else {
      k -= c;
#pragma unroll
      for (int i = 0; i < N; ++i) cand[i] &= ~ones[i];
    }
  }
  return prefix;
}
__device__ __forceinline__ uint32_t wave_kth_largest2(uint32_t ka, uint32_t kb, int k) {
  uint64_t ca = ~0ull, cb = ~0ull;
  uint32_t prefix = 0;
#pragma unroll 4
  for (int b = 31; b >= 0; --b) {
    const uint64_t oa = __ballot((ka >> b) & 1u) & ca;
    const uint64_t ob = __ballot((kb >> b) & 1u) & cb;
    const int c = __popcll(oa) + __popcll(ob);
    if (c >= k) {
      ca = oa;
      cb = ob;
      prefix |= 1u << b;
    } else {
      k -= c;
      ca &= ~oa;
      cb &= ~ob;
    }
  }
  return prefix;
}

// Bitonic sort of one value per lane across the wave, larger first.
template <typename T>
__device__ __forceinline__ T wave_sort_desc(T v) {
  const int l = lane();
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const T o = lane_xor_rt(v, j);
      const bool keep_max = (((l & k) == 0) == ((l & j) == 0));
      v = keep_max ? (o > v ? o : v) : (o < v ? o : v);
    }
  }
  return v;
}
// Given two descending lane-sorted sequences a and b, the 64 largest of their
// union, descending (bitonic half-cleaner, then a bitonic merge).
template <typename T>
__device__ __forceinline__ T wave_merge_top_desc(T a, T b) {
  const int l = lane();
  const T br = __shfl(b, kWave - 1 - l);
  T v = (a > br) ? a : br;
#pragma unroll
  for (int j = kWave >> 1; j > 0; j >>= 1) {
    const T o = lane_xor_rt(v, j);
    v = ((l & j) == 0) ? (o > v ? o : v) : (o < v ? o : v);
  }
  return v;
}

// The cut and the draw over the n <= 64 sorted candidates (lane i holds the
// i-th, P, packed with the key of s = x / T), given each candidate's relative
// weight e = E(s - m) (m the largest s) and Gumbel score sc = e / -log(u):
// min-p keeps e >= min_p; top-p keeps the shortest prefix whose fixed-point
// mass reaches p times the kept mass; the draw is the largest score over the
// kept set, ties to the lowest id. Returns the status (VS_ROW_BAD_LOGITS for
// an empty list, VS_ROW_BAD_PARAM when s = +inf). Called by a whole wave,
// every lane active; lanes from n on are ignored.
__device__ inline int wave_cut_draw(uint64_t P, int n, float e, double sc, const RowCfg& c,
                                    int32_t* id_out, int32_t* kept_out, uint32_t* mask_row) {
  const int i = lane();
  if (n <= 0) return VS_ROW_BAD_LOGITS;  // no candidate: never read an id from it
  if (pkey(readlane_u64(P, 0)) == kKeyPosInf) return VS_ROW_BAD_PARAM;
  const bool has = i < n;
  const bool in_s = has && (e >= c.mp);
  const int id = has ? pid(P) : 0x7fffffff;
  bool kept = in_s;
  if (c.p < 1.0f) {
    // fixed-point masses (< 2^31 + 1) scanned as 16-bit halves, whose sums
    // over 64 lanes fit in 32 bits
    const uint32_t w = in_s ? static_cast<uint32_t>(mass_of(e)) : 0u;
    const uint32_t lo = wave_scan_incl_u32(w & 0xffffu);
    const uint32_t hi = wave_scan_incl_u32(w >> 16);
    const uint64_t cum = (static_cast<uint64_t>(hi) << 16) + lo;
    const uint64_t tw = readlane_u64(cum, kWave - 1);
    const double thr = static_cast<double>(c.p) * static_cast<double>(tw);
    const uint64_t hit = __ballot(in_s && static_cast<double>(cum) >= thr);
    const int cut = hit ? __ffsll(static_cast<unsigned long long>(hit)) - 1 : kWave;
    kept = in_s && i <= cut;
  }
  // scores are nonnegative, so their bits order as integers
  const uint64_t sb = kept ? static_cast<uint64_t>(__double_as_longlong(sc)) : 0ull;
  const uint64_t best = wave_max_u64_dpp(sb);
  const int win = wave_min_dpp((kept && sb == best) ? id : 0x7fffffff);
  if (kept && mask_row) atomicOr(&mask_row[id >> 5], 1u << (id & 31));
  *id_out = win;
  *kept_out = __popcll(__ballot(kept));
  return 0;
}

// Truncation and the draw over the n <= 64 sorted candidates P (lane i the
// i-th) with one wave, no block barrier: each lane forms its candidate's
// weight and score (q, when given, holds -log(u) of the candidates by lane,
// the same values this function would compute), then wave_cut_draw. Called by
// a whole wave, every lane active.
__device__ inline int wave_draw_lanes(uint64_t P, int n, const RowCfg& c, int row,
                                      int32_t* id_out, int32_t* kept_out, uint32_t* mask_row,
                                      const double* q) {
  const int i = lane();
  if (n <= 0) return VS_ROW_BAD_LOGITS;
  const float m = key2f(pkey(readlane_u64(P, 0)));
  const bool has = i < n;
  const float e = has ? pinned_exp(key2f(pkey(P)) - m) : 0.0f;
  // every candidate's score, computed before the cut is known so that the two
  // overlap
  double sc = 0.0;
  if (has) sc = q ? static_cast<double>(e) / q[i] : gumbel_score(e, row_stream(c.seed, row), pid(P));
  return wave_cut_draw(has ? P : 0ull, n, e, sc, c, id_out, kept_out, mask_row);
}
// The same with the sorted candidates in memory (LDS).
__device__ inline int wave_draw(const uint64_t* L, int n, const RowCfg& c, int row,
                                int32_t* id_out, int32_t* kept_out, uint32_t* mask_row,
                                const double* q = nullptr) {
  const int i = lane();
  const uint64_t P = (i < n) ? L[i] : 0ull;
  return wave_draw_lanes(P, n, c, row, id_out, kept_out, mask_row, q);
}

// ---------------------------------------------------------------- block primitives
// All take a shared scratch array with at least (blockDim.x / 64) slots and
// must be called by every thread of the block.
template <typename T>
__device__ __forceinline__ T block_max(T v, T* scratch) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  __syncthreads();
  if (lane() == 0) scratch[w] = v;
  __syncthreads();
  v = scratch[0];
  for (int i = 1; i < nw; ++i) v = (scratch[i] > v) ? scratch[i] : v;
  __syncthreads();
  return v;
}
template <typename T>
__device__ __forceinline__ T block_min(T v, T* scratch) {
  v = wave_min(v);
  const int w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  __syncthreads();
  if (lane() == 0) scratch[w] = v;
  __syncthreads();
  v = scratch[0];
  for (int i = 1; i < nw; ++i) v = (scratch[i] < v) ? scratch[i] : v;
  __syncthreads();
  return v;
}
template <typename T>
__device__ __forceinline__ T block_sum(T v, T* scratch) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  __syncthreads();
  if (lane() == 0) scratch[w] = v;
  __syncthreads();
  v = scratch[0];
  for (int i = 1; i < nw; ++i) v += scratch[i];
  __syncthreads();
  return v;
}
// Inclusive prefix sum over the block in thread order; *total gets the block sum.
template <typename T>
__device__ __forceinline__ T block_scan_incl(T v, T* scratch, T* total) {
  const int l = lane();
  if constexpr (std::is_same<T, uint64_t>::value) {  // in-wave: DPP row shifts and broadcasts
    v = wave_scan_incl_u64(v);
  } else if constexpr (std::is_integral<T>::value && sizeof(T) == 4) {
    v = static_cast<T>(wave_scan_incl_u32(static_cast<uint32_t>(v)));
  } else {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const T w = __shfl_up(v, o);
      if (l >= o) v += w;
    }
  }
  const int w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  __syncthreads();
  if (l == kWave - 1) scratch[w] = v;
  __syncthreads();
  T before = 0, all = 0;
  for (int i = 0; i < nw; ++i) {
    if (i < w) before += scratch[i];
    all += scratch[i];
  }
  __syncthreads();
  if (total) *total = all;
  return v + before;
}

// Bitonic sort of n (a power of two) uint64 values in shared memory, larger first.
__device__ __forceinline__ void block_sort_desc(uint64_t* buf, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < (n >> 1); i += blockDim.x) {
        const int lo = ((i / j) * 2 * j) + (i % j);
        const int hi = lo + j;
        const bool desc = ((lo & k) == 0);
        const uint64_t a = buf[lo], b = buf[hi];
        if (desc ? (a < b) : (a > b)) {
          buf[lo] = b;
          buf[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int next_pow2(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// XCD-aware placement: workgroups are dispatched round-robin over the 8 XCDs,
// so workgroup L runs on XCD L % 8. Placing every tile of row r on XCD r % 8
// keeps a row's re-reads in one L2. Returns false for padding workgroups.
constexpr int kXcds = 8;
__device__ __forceinline__ bool xcd_row_tile(int L, int B, int tiles_per_row, int* row, int* tile) {
  const int x = L % kXcds;
  const int q = L / kXcds;
  const int a = q / tiles_per_row;
  *tile = q - a * tiles_per_row;
  *row = x + kXcds * a;
  return *row < B;
}
__host__ __device__ inline int xcd_grid(int B, int tiles_per_row) {
  return kXcds * ((B + kXcds - 1) / kXcds) * tiles_per_row;
}

}  // namespace vsk
