// C ABI of libvs.so: argument checks, workspace layout, kernel sequence.
#include <stdint.h>

#include <cstring>
#include <mutex>

#include "vs_device.h"
#include "vs_kernels.h"

namespace vsk {

namespace {
size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Compute units of the current device (cached per device).
int device_cus() {
  constexpr int kMaxDev = 64;
  static int cache[kMaxDev] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
  int n = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    __atomic_store_n(&cache[dev], n, __ATOMIC_RELAXED);
  }
  return n;
}
}  // namespace

WsLayout ws_layout(int B, int V, int nslot) {
  WsLayout L{};
  L.ntile = (V + kSelTile - 1) / kSelTile;
  L.ntile3 = (V + kGumTile - 1) / kGumTile;
  const size_t tiles = static_cast<size_t>(B) * nslot;
  size_t off = 0;
  L.meta = off;
  off = align_up(off + tiles * sizeof(uint32_t));
  L.candA = off;
  off = align_up(off + tiles * kSelCap * sizeof(uint64_t));
  L.candB = off;
  off = align_up(off + tiles * kSelCap * sizeof(uint64_t));
  L.kthA = off;
  off = align_up(off + tiles * sizeof(uint32_t));
  L.kthB = off;
  off = align_up(off + tiles * sizeof(uint32_t));
  L.desc = off;
  off = align_up(off + static_cast<size_t>(B) * sizeof(RowDesc));
  L.gpart = off;
  off = align_up(off + static_cast<size_t>(B) * L.ntile3 * sizeof(GPart));
  L.lpart = off;
  off = align_up(off + tiles * sizeof(LsePart));
  L.rlse = off;
  off = align_up(off + static_cast<size_t>(B) * sizeof(float2));
  L.fhw = off;
  off = align_up(off + static_cast<size_t>(B) * kFullBuckets * sizeof(uint64_t));
  L.flist = off;
  off = align_up(off + static_cast<size_t>(B) * kFullListCap * sizeof(uint64_t));
  L.fcnt = off;
  off = align_up(off + static_cast<size_t>(B) * sizeof(uint32_t));
  L.fcut = off;
  off = align_up(off + static_cast<size_t>(B) * sizeof(FullCut));
  L.fcand = off;  // a histogram segment is at least one Gumbel tile long
  off = align_up(off + static_cast<size_t>(B) * L.ntile3 * kCandM * sizeof(GCand));
  L.total = off;
  return L;
}

int stream_segments(int B, int V) {
  const int cus = device_cus();
  const int nslot = ws_slots_any(V);
  int S = (cus + B - 1) / B;
  S = S < 1 ? 1 : (S > nslot ? nslot : S);
  const int ntile = (V + kSelTile - 1) / kSelTile;
  const int tps = (ntile + S - 1) / S;
  return (ntile + tps - 1) / tps;
}

// nslot: the workspace's segment slots per row (ws_slots_any(V) for a
// caller's workspace, the device's segment count for the library's scratch).
Job make_job(const void* logits, int dt, int B, int V, int64_t ld, void* ws, int nslot) {
  const WsLayout L = ws_layout(B, V, nslot);
  char* w = static_cast<char*>(ws);
  Job j{};
  j.logits = logits;
  j.dt = dt;
  j.B = B;
  j.V = V;
  j.ld = ld;
  const int64_t es = (dt == VS_F32) ? 4 : 2;
  j.aligned = (reinterpret_cast<uintptr_t>(logits) % 16 == 0) && ((ld * es) % 16 == 0);
  j.ntile = L.ntile;
  j.ntile3 = L.ntile3;
  // Streaming-pass geometry: enough segments per row that the batch gives
  // every compute unit a workgroup, each segment read by up to 16 waves. When
  // the batch alone holds more rows than compute units, workgroups shrink
  // (down to 4 waves) so that several share a compute unit and one row's
  // closing steps overlap other rows' streaming.
  const int cus = device_cus();
  int S = (cus + B - 1) / B;
  S = S < 1 ? 1 : (S > ws_slots_any(V) ? ws_slots_any(V) : S);
  j.tps = (L.ntile + S - 1) / S;
  j.nseg = (L.ntile + j.tps - 1) / j.tps;
  int wmax = kSelMaxWaves;
  while (wmax > 4 && static_cast<int64_t>(B) * wmax > static_cast<int64_t>(cus) * kSelMaxWaves)
    wmax >>= 1;
  j.nwave = j.tps < wmax ? j.tps : wmax;
  j.meta = reinterpret_cast<uint32_t*>(w + L.meta);
  j.candA = reinterpret_cast<uint64_t*>(w + L.candA);
  j.candB = reinterpret_cast<uint64_t*>(w + L.candB);
  j.kthA = reinterpret_cast<uint32_t*>(w + L.kthA);
  j.kthB = reinterpret_cast<uint32_t*>(w + L.kthB);
  j.desc = reinterpret_cast<RowDesc*>(w + L.desc);
  j.gpart = reinterpret_cast<GPart*>(w + L.gpart);
  j.lpart = reinterpret_cast<LsePart*>(w + L.lpart);
  j.rlse = reinterpret_cast<float2*>(w + L.rlse);
  j.fhw = reinterpret_cast<uint64_t*>(w + L.fhw);
  j.flist = reinterpret_cast<uint64_t*>(w + L.flist);
  j.fcnt = reinterpret_cast<uint32_t*>(w + L.fcnt);
  j.fcut = reinterpret_cast<FullCut*>(w + L.fcut);
  j.fcand = reinterpret_cast<GCand*>(w + L.fcand);
  // Gumbel pass of full-vocabulary rows: up to 8 tiles per workgroup (the
  // pruning bound tightens along them) while the grid keeps about 1024
  // workgroups (four waves per SIMD to hide the loads' latency).
  {
    const int64_t t = static_cast<int64_t>(B) * L.ntile3 / 1024;
    j.gseg = t < 1 ? 1 : (t > 8 ? 8 : static_cast<int>(t));
  }
  // Histogram and gather passes of full-vocabulary rows (1024-thread
  // workgroups): enough segments per row that the batch gives every compute
  // unit about one workgroup, each at least kFullSegMin ids (a multiple of 8,
  // so segments start 16-byte aligned). Fewer, longer segments mean fewer
  // flushes of per-segment histograms into the row's.
  {
    const int smax = (V + kFullSegMin - 1) / kFullSegMin;
    int fs = (cus + B - 1) / B;
    fs = fs < 1 ? 1 : (fs > smax ? smax : fs);
    const int len = ((V + fs - 1) / fs + 7) & ~7;
    j.fseg_len = len;
    j.fseg = (V + len - 1) / len;
  }
  return j;
}

}  // namespace vsk

using vsk::WsLayout;

namespace {

// Per-thread stage profiling (vs_profile_begin / vs_profile_end).
constexpr int kMaxProfiled = 4096;
thread_local hipEvent_t* g_prof_ev = nullptr;
thread_local int g_prof_cap = 0;
thread_local int g_prof_n = 0;
thread_local const char* g_prof_names[kMaxProfiled];

// Runs one launch function, bracketed by profiling events when active.
template <typename F>
hipError_t stage(const char* name, hipStream_t st, F&& launch) {
  const bool rec = g_prof_ev && 2 * g_prof_n + 1 < g_prof_cap && g_prof_n < kMaxProfiled;
  if (rec && hipEventRecord(g_prof_ev[2 * g_prof_n], st) != hipSuccess) return hipErrorUnknown;
  const hipError_t e = launch();
  if (rec) {
    if (hipEventRecord(g_prof_ev[2 * g_prof_n + 1], st) != hipSuccess) return hipErrorUnknown;
    g_prof_names[g_prof_n++] = name;
  }
  return e;
}

// Full log-softmax rows that take 16-byte stores.
int full_vec(const float* out_full, int64_t ld_out) {
  return (out_full && reinterpret_cast<uintptr_t>(out_full) % 16 == 0 && ld_out % 4 == 0) ? 1 : 0;
}

// The integer a caller passed in an enum parameter, read without loading a
// value of the enum type (a C caller may pass any int there; loading one
// outside the enumerators' range as the enum would be undefined in C++).
template <typename Enum>
int raw(const Enum* p) {
  static_assert(sizeof(Enum) == sizeof(int), "the C enums are passed as int");
  int v;
  std::memcpy(&v, p, sizeof v);
  return v;
}

bool sizes_ok(int dt, int B, int V, int64_t ld) {
  return (dt == VS_F32 || dt == VS_BF16) && B > 0 && V > 0 && V <= VS_MAX_V && ld >= V;
}

// With the full log-softmax written by the streaming pass, workgroups of at
// least 8 waves: fewer rows in flight between a row's read and its re-read for
// the write, so more of the re-read comes from the caches (measured on 1024
// rows of 128,256: 8 waves 4 % faster than 4; 16 slower).
void widen_for_full_write(vsk::Job& j) {
  if (j.full_in_select && j.nwave < 8) j.nwave = j.tps < 8 ? j.tps : 8;
}

}  // namespace

extern "C" {

vs_status vs_workspace_size(int B, int V, vs_dtype dt, size_t* bytes) {
  if (!bytes || !sizes_ok(raw(&dt), B, V, V)) return VS_ERR_INVALID_ARGUMENT;
  *bytes = vsk::ws_layout(B, V, vsk::ws_slots_any(V)).total;
  return VS_OK;
}

const char* vs_status_string(vs_status s) {
  switch (raw(&s)) {
    case VS_OK: return "ok";
    case VS_ERR_INVALID_ARGUMENT: return "invalid argument";
    case VS_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case VS_ERR_UNSUPPORTED: return "unsupported";
    case VS_ERR_HIP: return "HIP launch failure";
  }
  return "unknown status";
}

}  // extern "C"

namespace {
vs_status penalize_impl(void* logits, int dt, int B, int V, int64_t ld,
                        const int32_t* prompt_ids, const int32_t* prompt_off,
                        const int32_t* output_ids, const int32_t* output_off,
                        const float* presence, const float* frequency, const float* repetition,
                        const int32_t* prompt_ignore_len, int32_t* out_row_status,
                        hipStream_t stream) {
  if (!logits || !sizes_ok(dt, B, V, ld)) return VS_ERR_INVALID_ARGUMENT;
  if ((prompt_ids == nullptr) != (prompt_off == nullptr)) return VS_ERR_INVALID_ARGUMENT;
  if ((output_ids == nullptr) != (output_off == nullptr)) return VS_ERR_INVALID_ARGUMENT;
  const hipError_t e = stage("penalize", stream, [&] {
    return vsk::launch_penalize(logits, dt, B, V, ld, prompt_ids, prompt_off, output_ids,
                                output_off, presence, frequency, repetition, prompt_ignore_len,
                                out_row_status, stream);
  });
  return e == hipSuccess ? VS_OK : VS_ERR_HIP;
}

}  // namespace

extern "C" {

vs_status vs_penalize_ex(void* logits, vs_dtype dt, int B, int V, int64_t ld,
                         const int32_t* prompt_ids, const int32_t* prompt_off,
                         const int32_t* output_ids, const int32_t* output_off,
                         const float* presence, const float* frequency,
                         const float* repetition, const int32_t* prompt_ignore_len,
                         int32_t* out_row_status, hipStream_t stream) {
  return penalize_impl(logits, raw(&dt), B, V, ld, prompt_ids, prompt_off, output_ids, output_off,
                       presence, frequency, repetition, prompt_ignore_len, out_row_status, stream);
}

vs_status vs_penalize(void* logits, vs_dtype dt, int B, int V, int64_t ld,
                      const int32_t* prompt_ids, const int32_t* prompt_off,
                      const int32_t* output_ids, const int32_t* output_off,
                      const float* presence, const float* frequency,
                      const float* repetition, int32_t* out_row_status,
                      hipStream_t stream) {
  return penalize_impl(logits, raw(&dt), B, V, ld, prompt_ids, prompt_off, output_ids, output_off,
                       presence, frequency, repetition, nullptr, out_row_status, stream);
}

vs_status vs_topp_decay(int B, float* top_p, const float* top_p_init, const float* decay,
                        const float* top_p_min, const int32_t* reset_ids,
                        const int32_t* sampled_ids, int32_t* out_row_status, hipStream_t stream) {
  if (B <= 0 || !top_p || !top_p_init || !decay || !sampled_ids) return VS_ERR_INVALID_ARGUMENT;
  const hipError_t e = stage("topp_decay", stream, [&] {
    return vsk::launch_topp_decay(B, top_p, top_p_init, decay, top_p_min, reset_ids, sampled_ids,
                                  out_row_status, stream);
  });
  return e == hipSuccess ? VS_OK : VS_ERR_HIP;
}

vs_status vs_slot_remap(int B, int B_src, const int32_t* slot_remap, const void* src, void* dst,
                        int elem_bytes, int32_t* out_row_status, hipStream_t stream) {
  if (B <= 0 || B_src <= 0 || !slot_remap || !src || !dst || src == dst ||
      (elem_bytes != 4 && elem_bytes != 8))
    return VS_ERR_INVALID_ARGUMENT;
  const hipError_t e = stage("slot_remap", stream, [&] {
    return vsk::launch_slot_remap(B, B_src, slot_remap, src, dst, elem_bytes, out_row_status, stream);
  });
  return e == hipSuccess ? VS_OK : VS_ERR_HIP;
}

vs_status vs_seed_advance(int B, uint64_t* seeds, const int32_t* sampled_ids, hipStream_t stream) {
  if (B <= 0 || !seeds) return VS_ERR_INVALID_ARGUMENT;
  const hipError_t e = stage("seed_advance", stream, [&] {
    return vsk::launch_seed_advance(B, seeds, sampled_ids, stream);
  });
  return e == hipSuccess ? VS_OK : VS_ERR_HIP;
}


}  // extern "C"

namespace {

// The occurrence penalties a fused call applies in its streaming pass.
struct PenArgs {
  const int32_t *prompt_ids, *prompt_off, *output_ids, *output_off;
  const float *presence, *frequency, *repetition;
  const int32_t* prompt_ignore_len;
  int32_t* out_status;
};

// vs_sample_logprobs on a workspace laid out with nslot segment slots per
// row; with pen, the streaming pass first applies those penalties in place.
vs_status sample_logprobs_impl(const PenArgs* pen, const void* logits, int dt, int B, int V,
                               int64_t ld,
                               const float* temperature, const int32_t* top_k,
                               const float* top_p, const float* min_p,
                               const uint64_t* seeds, uint32_t hints, int32_t* out_ids,
                               int32_t* out_kept_count, uint32_t* out_kept_mask,
                               int32_t* out_row_status, float* out_token_logprob, int k,
                               int32_t* out_topk_ids, float* out_topk_logprobs, float* out_full,
                               int64_t ld_out, void* ws, size_t ws_bytes, int nslot,
                               hipStream_t stream) {
  if (!logits || !out_ids || !ws || !sizes_ok(dt, B, V, ld)) return VS_ERR_INVALID_ARGUMENT;
  if (hints & ~(VS_HINT_NO_FULLVOCAB | VS_HINT_ALL_GREEDY | VS_HINT_NO_GREEDY | VS_HINT_SMALL_TOPK |
                VS_OPT_TOPP_REJECTION | VS_OPT_TOPP_GATHER_DRAW | VS_OPT_TOPP_KEPT_PASS))
    return VS_ERR_INVALID_ARGUMENT;
  if (k < 0 || k > VS_LOGPROB_K_MAX || k > V) return VS_ERR_INVALID_ARGUMENT;
  if (k > 0 && (!out_topk_ids || !out_topk_logprobs)) return VS_ERR_INVALID_ARGUMENT;
  if (out_full && ld_out < V) return VS_ERR_INVALID_ARGUMENT;
  if (ws_bytes < vsk::ws_layout(B, V, nslot).total) return VS_ERR_WORKSPACE_TOO_SMALL;
  if (pen && ((pen->prompt_ids == nullptr) != (pen->prompt_off == nullptr) ||
              (pen->output_ids == nullptr) != (pen->output_off == nullptr)))
    return VS_ERR_INVALID_ARGUMENT;
  vsk::Job j = vsk::make_job(logits, dt, B, V, ld, ws, nslot);
  if (pen) {
    j.pen = 1;
    j.pen_pids = pen->prompt_ids;
    j.pen_poff = pen->prompt_off;
    j.pen_oids = pen->output_ids;
    j.pen_ooff = pen->output_off;
    j.pen_pres = pen->presence;
    j.pen_freq = pen->frequency;
    j.pen_rep = pen->repetition;
    j.pen_ign = pen->prompt_ignore_len;
    j.out_pen_status = pen->out_status;
  }
  j.sample = 1;
  // full-vocabulary top-p rows draw by rejection when the caller chooses it
  // and asks for no kept mask (the Gumbel pass over the kept set writes that)
  j.topp_reject = ((hints & VS_OPT_TOPP_REJECTION) && !out_kept_mask) ? 1 : 0;
  // otherwise, without a kept mask, the gather pass and the cut kernel draw
  // them unless the Gumbel pass over the kept set is chosen (measured: the
  // gather draw, two launches shorter, is the faster on w4x32000 too)
  const bool gather_draw =
      (hints & VS_OPT_TOPP_GATHER_DRAW) || !(hints & VS_OPT_TOPP_KEPT_PASS);
  j.fdraw = (!j.topp_reject && !out_kept_mask && gather_draw) ? 1 : 0;
  j.T = temperature;
  j.k = top_k;
  j.p = top_p;
  j.mp = min_p;
  j.seeds = seeds;
  j.hints = hints;
  j.out_ids = out_ids;
  j.out_kept = out_kept_count;
  j.out_mask = out_kept_mask;
  j.out_status = out_row_status;
  j.lse = (out_token_logprob != nullptr || k > 0 || out_full != nullptr) ? 1 : 0;
  j.k_lp = k;
  j.tok_sampled = out_token_logprob != nullptr;
  j.out_tok_lp = out_token_logprob;
  j.out_lp_ids = out_topk_ids;
  j.out_lp = out_topk_logprobs;
  j.out_full = out_full;
  j.ld_out = ld_out;
  // With one segment per row, no kept mask and hints that rule out every row
  // the streaming pass cannot finish (top-k above 64, full vocabulary), the
  // streaming pass finishes every row and the row kernel has nothing to do;
  // it then also writes the full log-softmax, right after reading each row.
  const bool select_finishes =
      j.nseg == 1 && !out_kept_mask && (hints & (VS_HINT_SMALL_TOPK | VS_HINT_ALL_GREEDY));
  j.full_in_select = (out_full && select_finishes) ? 1 : 0;
  widen_for_full_write(j);
  j.full_vec = full_vec(out_full, ld_out);
  // Unless a hint rules out full-vocabulary rows, their passes run (each
  // returns at once for rows it does not take), and the row kernel's work
  // then moves into the cut kernel after them, which saves a launch and its
  // wait on the path: the streaming pass clears the passes' counters, and
  // every pass routes the rows itself (measured: w32x151936 91.6 -> 84.3 us,
  // w64x262144 111.3 -> 107.2 us; w4x32000 43.4 -> 40.8 us once the cut
  // kernel also finished the draw).
  const bool full_passes = !(hints & (VS_HINT_NO_FULLVOCAB | VS_HINT_ALL_GREEDY | VS_HINT_SMALL_TOPK));
  j.full_chain = full_passes ? 1 : 0;
  if (stage("select", stream, [&] { return vsk::launch_select(j, stream); }) != hipSuccess)
    return VS_ERR_HIP;
  if (!select_finishes && !j.full_chain &&
      stage("row", stream, [&] { return vsk::launch_row_light(j, stream); }) != hipSuccess)
    return VS_ERR_HIP;
  if (full_passes) {
    if (stage("full_prep", stream, [&] { return vsk::launch_full_prep(j, stream); }) != hipSuccess)
      return VS_ERR_HIP;
    if (stage("row_full", stream, [&] { return vsk::launch_row_full(j, stream); }) != hipSuccess)
      return VS_ERR_HIP;
    // (when the gather pass drew, the cut kernel finished every
    // full-vocabulary row: no Gumbel pass over the kept sets)
    if (!j.fdraw &&
        stage("gumbel", stream, [&] { return vsk::launch_gumbel(j, stream); }) != hipSuccess)
      return VS_ERR_HIP;
  }
  if (out_full && !j.full_in_select) {
    if (stage("lse_full", stream, [&] { return vsk::launch_lse_full(j, stream); }) != hipSuccess)
      return VS_ERR_HIP;
  }
  return VS_OK;
}

vs_status logprobs_impl(const void* logits, int dt, int B, int V, int64_t ld,
                        const float* temperature, const int32_t* token_ids,
                        float* out_token_logprob, int k, int32_t* out_topk_ids,
                        float* out_topk_logprobs, float* out_full, int64_t ld_out,
                        int32_t* out_row_status, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!logits || !ws || !sizes_ok(dt, B, V, ld)) return VS_ERR_INVALID_ARGUMENT;
  if ((token_ids == nullptr) != (out_token_logprob == nullptr)) return VS_ERR_INVALID_ARGUMENT;
  if (k < 0 || k > VS_LOGPROB_K_MAX || k > V) return VS_ERR_INVALID_ARGUMENT;
  if (k > 0 && (!out_topk_ids || !out_topk_logprobs)) return VS_ERR_INVALID_ARGUMENT;
  if (out_full && ld_out < V) return VS_ERR_INVALID_ARGUMENT;
  if (ws_bytes < vsk::ws_layout(B, V, vsk::ws_slots_any(V)).total) return VS_ERR_WORKSPACE_TOO_SMALL;
  vsk::Job j = vsk::make_job(logits, dt, B, V, ld, ws, vsk::ws_slots_any(V));
  j.lse = 1;
  j.k_lp = k;
  j.tok = token_ids;
  j.out_tok_lp = out_token_logprob;
  j.out_lp_ids = out_topk_ids;
  j.out_lp = out_topk_logprobs;
  j.out_full = out_full;
  j.ld_out = ld_out;
  j.out_lp_status = out_row_status;
  j.lpT = temperature;
  // with one segment per row the streaming pass finishes every row (and then
  // writes the full log-softmax itself)
  j.full_in_select = (out_full && j.nseg == 1) ? 1 : 0;
  widen_for_full_write(j);
  j.full_vec = full_vec(out_full, ld_out);
  if (stage("lse_select", stream, [&] { return vsk::launch_select(j, stream); }) != hipSuccess)
    return VS_ERR_HIP;
  if (j.nseg > 1 &&
      stage("lse_row", stream, [&] { return vsk::launch_row_light(j, stream); }) != hipSuccess)
    return VS_ERR_HIP;
  if (out_full && !j.full_in_select) {
    if (stage("lse_full", stream, [&] { return vsk::launch_lse_full(j, stream); }) != hipSuccess)
      return VS_ERR_HIP;
  }
  return VS_OK;
}

// The library's own scratch for vs_sample_logprobs_noalloc: one array per
// device (each device that loads the library's code holds its own copy until
// the process ends). Host code never uses the array's name as an address: the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[VS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The current device's scratch address (NULL if it cannot be had).
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  void* p = __atomic_load_n(&g_scratch_ptr[dev], __ATOMIC_ACQUIRE);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev];
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    __atomic_store_n(&g_scratch_ptr[dev], p, __ATOMIC_RELEASE);
  }
  return p;
}

}  // namespace

extern "C" {

vs_status vs_sample(const void* logits, vs_dtype dt, int B, int V, int64_t ld,
                    const float* temperature, const int32_t* top_k,
                    const float* top_p, const float* min_p,
                    const uint64_t* seeds, uint32_t hints, int32_t* out_ids,
                    int32_t* out_kept_count, uint32_t* out_kept_mask,
                    int32_t* out_row_status, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  return sample_logprobs_impl(nullptr, logits, raw(&dt), B, V, ld, temperature, top_k, top_p,
                              min_p, seeds, hints, out_ids, out_kept_count, out_kept_mask,
                              out_row_status, nullptr, 0, nullptr, nullptr, nullptr, 0, ws,
                              ws_bytes, vsk::ws_slots_any(V), stream);
}

vs_status vs_sample_logprobs(const void* logits, vs_dtype dt, int B, int V, int64_t ld,
                             const float* temperature, const int32_t* top_k,
                             const float* top_p, const float* min_p,
                             const uint64_t* seeds, uint32_t hints, int32_t* out_ids,
                             int32_t* out_kept_count, uint32_t* out_kept_mask,
                             int32_t* out_row_status, float* out_token_logprob, int k,
                             int32_t* out_topk_ids, float* out_topk_logprobs, float* out_full,
                             int64_t ld_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return sample_logprobs_impl(nullptr, logits, raw(&dt), B, V, ld, temperature, top_k, top_p, min_p,
                              seeds, hints, out_ids, out_kept_count, out_kept_mask, out_row_status,
                              out_token_logprob, k, out_topk_ids, out_topk_logprobs, out_full,
                              ld_out, ws, ws_bytes, vsk::ws_slots_any(V), stream);
}

vs_status vs_sample_logprobs_noalloc(const void* logits, vs_dtype dt, int B, int V, int64_t ld,
                                     const float* temperature, const int32_t* top_k,
                                     const float* top_p, const float* min_p,
                                     const uint64_t* seeds, uint32_t hints, int32_t* out_ids,
                                     int32_t* out_kept_count, uint32_t* out_kept_mask,
                                     int32_t* out_row_status, float* out_token_logprob, int k,
                                     int32_t* out_topk_ids, float* out_topk_logprobs,
                                     float* out_full, int64_t ld_out, hipStream_t stream) {
  if (!logits || !out_ids || !sizes_ok(raw(&dt), B, V, ld)) return VS_ERR_INVALID_ARGUMENT;
  // laid out for the segments this device's streaming pass uses, not for every device
  const int nslot = vsk::stream_segments(B, V);
  if (vsk::ws_layout(B, V, nslot).total > VS_NOALLOC_SCRATCH_BYTES) return VS_ERR_WORKSPACE_TOO_SMALL;
  void* ws = scratch_ptr();
  if (!ws) return VS_ERR_HIP;
  return sample_logprobs_impl(nullptr, logits, raw(&dt), B, V, ld, temperature, top_k, top_p, min_p,
                              seeds, hints, out_ids, out_kept_count, out_kept_mask, out_row_status,
                              out_token_logprob, k, out_topk_ids, out_topk_logprobs, out_full,
                              ld_out, ws, VS_NOALLOC_SCRATCH_BYTES, nslot, stream);
}

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
                                      void* ws, size_t ws_bytes, hipStream_t stream) {
  const PenArgs pen{prompt_ids, prompt_off, output_ids, output_off, presence,
                    frequency,  repetition, prompt_ignore_len, out_penalty_status};
  return sample_logprobs_impl(&pen, logits, raw(&dt), B, V, ld, temperature, top_k, top_p, min_p, seeds,
                              hints, out_ids, out_kept_count, out_kept_mask, out_row_status,
                              out_token_logprob, k, out_topk_ids, out_topk_logprobs, out_full,
                              ld_out, ws, ws_bytes, vsk::ws_slots_any(V), stream);
}

vs_status vs_logprobs(const void* logits, vs_dtype dt, int B, int V, int64_t ld,
                      const int32_t* token_ids, float* out_token_logprob, int k,
                      int32_t* out_topk_ids, float* out_topk_logprobs,
                      float* out_full, int64_t ld_out, int32_t* out_row_status,
                      void* ws, size_t ws_bytes, hipStream_t stream) {
  return logprobs_impl(logits, raw(&dt), B, V, ld, nullptr, token_ids, out_token_logprob, k,
                       out_topk_ids, out_topk_logprobs, out_full, ld_out, out_row_status, ws,
                       ws_bytes, stream);
}

vs_status vs_logprobs_ex(const void* logits, vs_dtype dt, int B, int V, int64_t ld,
                         const float* temperature, const int32_t* token_ids,
                         float* out_token_logprob, int k, int32_t* out_topk_ids,
                         float* out_topk_logprobs, float* out_full, int64_t ld_out,
                         int32_t* out_row_status, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  return logprobs_impl(logits, raw(&dt), B, V, ld, temperature, token_ids, out_token_logprob, k,
                       out_topk_ids, out_topk_logprobs, out_full, ld_out, out_row_status, ws,
                       ws_bytes, stream);
}

vs_status vs_profile_begin(hipEvent_t* events, int capacity) {
  if (!events || capacity < 2) return VS_ERR_INVALID_ARGUMENT;
  g_prof_ev = events;
  g_prof_cap = capacity;
  g_prof_n = 0;
  return VS_OK;
}

int vs_profile_end(const char** names, int max_names) {
  const int n = g_prof_n;
  if (names)
    for (int i = 0; i < n && i < max_names; ++i) names[i] = g_prof_names[i];
  g_prof_ev = nullptr;
  g_prof_cap = 0;
  g_prof_n = 0;
  return n;
}

}  // extern "C"
