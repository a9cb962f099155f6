#!/usr/bin/env python3
"""Benchmark of the batched decode-step sampling path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|all] [--no-cpu]

A step is one pass of the whole sampling path over one batch of synthetic
logits already resident in HBM: the draw and the log-probabilities the
workload asks for in one call (vs_sample_logprobs, one read of the logits),
with the occurrence penalties applied by the same call's streaming pass when
the workload has them (vs_penalize_sample_logprobs; the separate vs_penalize
launch before vs_sample_logprobs is timed beside it).

The headline is the 256 x 248,320 fp32 workload (temperature 1, top-k 20,
top-p 0.95, sampled-id and top-20 log-probs): its K steps are timed exactly,
as graph replays of steps over rotated input copies (together larger than the
256 MB Infinity Cache, so every step reads cold logits), bracketed by a
device synchronisation on both sides. Every other workload is measured the
same way and reported under "configs", each with percentiles over replays,
per-stage kernel times, the roofline of its kernels and a streaming-read
reference on the same buffers. Inputs that a step penalises in place are
restored from a pristine copy between replays, outside the timed region, so
that every timed step penalises fresh logits once.

The CPU oracle is timed on the host (one pinned thread on a bounded row
sample, and the same per-row function on all host cores over the whole
batch); the all-core run also checks the GPU's ids and kept counts of one
fresh step per workload and counts near-tie rows. Prints one JSON line.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "rows/sec + achieved logits GB/s (% HBM peak), B=256 V=248,320 top-k/top-p"
HBM_PEAK_GBPS = 8000.0
HEADLINE = "w256x248320_f32"
ALL_WORKLOADS = ["w256x248320_f32", "w4x32000_f32", "w32x151936_bf16", "w1024x128256_f32",
                 "w64x262144_bf16"]
# The vector ALUs' issue ceiling: 256 CUs x 4 SIMDs x 16 lanes per cycle x
# 2.4 GHz (every VALU instruction at the non-packed fp32 rate, 32-bit integer
# multiplies included), and one SplitMix64 word as the compiler builds it for
# gfx950: 19 VALU instructions per lane (two 64-bit products by constants as
# 2 v_mad_u64_u32 + 4 v_mul_lo_u32, and 13 adds, shifts and xors).
VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9
SPLITMIX_OPS_PER_WORD = 19
SPLITMIX_PEAK_WORDS = VALU_LANE_OPS / SPLITMIX_OPS_PER_WORD
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {"select": "k_select.hip", "lse_select": "k_select.hip", "row": "k_row.hip",
                  "full_prep": "k_full.hip",
                  "lse_row": "k_row.hip", "row_full": "k_row.hip", "gumbel": "k_gumbel.hip",
                  "lse_full": "k_gumbel.hip", "penalize": "k_penalize.hip"}
MAX_POOL = 16   # host threads for the all-core oracle run, at most


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch has loaded."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = h
        return arr

    def record(self, ev, stream):
        if self.lib.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b):
        self.lib.hipEventSynchronize(b)
        out = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(out), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def destroy(self, arr):
        for h in arr:
            self.lib.hipEventDestroy(h)


def selftest_lib():
    """The measurement aids (a plain streaming read, a plain SplitMix64 stream)."""
    lib = ctypes.CDLL(os.path.join(ROOT, "decode_token_sampling_amd", "libvs_selftest.so"))
    P = ctypes.c_void_p
    lib.vs_selftest_read_rows.argtypes = [P, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int, P, P]
    lib.vs_selftest_read_rows.restype = ctypes.c_int
    lib.vs_selftest_splitmix.argtypes = [ctypes.c_int, ctypes.c_int, P, P]
    lib.vs_selftest_splitmix.restype = ctypes.c_int
    return lib


def kernel_hash(stage: str) -> str:
    src = os.path.join(ROOT, "decode_token_sampling_amd", "csrc")
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[stage], "vs_device.h", "vs_kernels.h"):
        with open(os.path.join(src, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, stage: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[workload][stage]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_hash") != kernel_hash(stage):
        return None
    return rec.get("bytes_per_launch")


def pct(v, q):
    return float(np.percentile(np.asarray(v, np.float64), q)) if len(v) else None


class Bench:
    """Device buffers and the step closure for one workload."""

    def __init__(self, vs, torch, wl, steps, dev, copies=0):
        self.vs, self.torch, self.wl, self.dev = vs, torch, wl, dev
        B, V = wl.B, wl.V
        d = lambda a, dt: None if a is None else torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(dev)
        if wl.dtype == "f32":
            self.base = torch.from_numpy(wl.logits).to(dev)
        else:
            self.base = torch.from_numpy(wl.logits.view(np.int16)).to(dev).view(torch.bfloat16)
        self.logit_bytes = B * V * wl.elem_bytes
        if not copies:
            copies = min(64, max(3, math.ceil(768e6 / self.logit_bytes)))
            if wl.has_penalties:   # each replay penalises every copy once: more copies, fewer restores
                copies = max(copies, 16)
            copies = min(copies, max(3, steps // 4))   # at least four replays for the percentiles
        self.copies = max(1, min(copies, steps))
        self.xs = [self.base.clone() for _ in range(self.copies)]
        self.T = d(wl.temperature, np.float32)
        self.K = d(wl.top_k, np.int32)
        self.P = d(wl.top_p, np.float32)
        self.MP = d(wl.min_p, np.float32)
        self.S = d(np.asarray(wl.seeds, np.uint64), np.int64)
        self.pen = None
        if wl.has_penalties:
            self.pen = [d(wl.prompt_ids, np.int32), d(wl.prompt_off, np.int32),
                        d(wl.output_ids, np.int32), d(wl.output_off, np.int32),
                        d(wl.presence, np.float32), d(wl.frequency, np.float32),
                        d(wl.repetition, np.float32)]
        self.ws = vs.workspace(B, V, self.base.dtype, dev)
        self.ids = torch.empty(B, dtype=torch.int32, device=dev)
        self.kept = torch.empty(B, dtype=torch.int32, device=dev)
        self.st = torch.empty(B, dtype=torch.int32, device=dev)
        self.pst = torch.empty(B, dtype=torch.int32, device=dev)
        self.full = torch.empty((B, V), dtype=torch.float32, device=dev) if wl.full_logprobs else None
        # the promise a serving engine derives from its batch's parameters
        self.hints = vs.hints_for(wl.temperature, wl.top_k, wl.top_p, wl.min_p, V)
        self.want_token_lp = not wl.full_logprobs
        self.tlp = torch.empty(B, dtype=torch.float32, device=dev) if self.want_token_lp else None
        k = wl.logprob_k
        self.tids = torch.empty((B, k), dtype=torch.int32, device=dev) if k else None
        self.tlps = torch.empty((B, k), dtype=torch.float32, device=dev) if k else None

    def step(self, i, hints=None, separate=False):
        """One step on input copy i: with penalties, the fused call (the
        streaming pass applies them) or, separate, vs_penalize first."""
        vs = self.vs
        x = self.xs[i % self.copies]
        kw = dict(hints=self.hints if hints is None else hints, k=self.wl.logprob_k,
                  token_logprob=self.want_token_lp, ws=self.ws, out_ids=self.ids, kept=self.kept,
                  row_status=self.st, out_token_lp=self.tlp, out_topk_ids=self.tids,
                  out_topk_lp=self.tlps, out_full=self.full)
        if self.pen is not None and not separate:
            vs.penalize_sample_logprobs(x, *self.pen, penalty_status=self.pst, temperature=self.T,
                                        top_k=self.K, top_p=self.P, min_p=self.MP, seeds=self.S, **kw)
            return
        if self.pen is not None:
            vs.penalize(x, *self.pen, row_status=self.pst)
        vs.sample_logprobs(x, self.T, self.K, self.P, self.MP, self.S, **kw)

    def restore(self):
        """Fresh logits in every copy (only workloads that penalise in place need it)."""
        if self.pen is not None:
            for x in self.xs:
                x.copy_(self.base)

    def describe(self, hints=None, separate=False):
        h = self.hints if hints is None else hints
        wl = self.wl
        outs = ", ".join(p for p in [
            "sampled-id lp" if self.want_token_lp else "",
            f"top-{wl.logprob_k}" if wl.logprob_k else "",
            "full [B,V] write" if wl.full_logprobs else ""] if p)
        if self.pen is not None and not separate:
            return f"vs_penalize_sample_logprobs(hints={h}; {outs})"
        parts = (["vs_penalize"] if self.pen is not None else []) + [
            f"vs_sample_logprobs(hints={h}; {outs})"]
        return " + ".join(parts)


def capture(torch, dev, fn, n):
    """A HIP graph of fn(0) .. fn(n - 1) (the library allocates and synchronises
    nothing, so its calls are capturable)."""
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for i in range(n):
            fn(i)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def time_steps(torch, dev, hip, b: Bench, K, hints=None, eager=False, separate=False):
    """Exactly K steps: graph replays of `copies` steps (plus one shorter graph
    for the remainder), each replay bracketed by HIP events on the stream the
    kernels run on; inputs restored between replays outside the events. Returns
    (total ms, per-step ms of each full replay)."""
    fn = lambda i: b.step(i, hints, separate)
    stream = torch.cuda.current_stream(dev).cuda_stream
    g = b.copies
    plan = [g] * (K // g) + ([K % g] if K % g else [])
    graphs = {}
    if not eager:
        for n in set(plan):
            graphs[n] = capture(torch, dev, fn, n)
            b.restore()
    torch.cuda.synchronize()
    ev = hip.create(2 * len(plan))
    for r, n in enumerate(plan):
        b.restore()
        hip.record(ev[2 * r], stream)
        if eager:
            for i in range(n):
                fn(i)
        else:
            graphs[n].replay()
        hip.record(ev[2 * r + 1], stream)
    torch.cuda.synchronize()
    spans = [hip.ms(ev[2 * r], ev[2 * r + 1]) for r in range(len(plan))]
    hip.destroy(ev)
    per_step = [s / n for s, n in zip(spans, plan) if n == g]
    del graphs
    return float(sum(spans)), per_step


def stage_profile(torch, dev, hip, lib, b: Bench, n, separate=False):
    """Per-stage durations: eager steps with every kernel stage bracketed by HIP
    events on its stream, queued behind a spin kernel so that the events time
    the GPU, not the host's enqueue rate."""
    cap = 2 * 8 * n
    pev = hip.create(cap)
    b.restore()
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2.4e9 * 0.02))
    if lib.vs_profile_begin(pev, cap) != 0:
        raise RuntimeError("vs_profile_begin failed")
    for i in range(n):
        b.step(i, separate=separate)
    names = (ctypes.c_char_p * (cap // 2))()
    m = lib.vs_profile_end(names, cap // 2)
    torch.cuda.synchronize()
    stage_ms = {}
    for i in range(m):
        stage_ms.setdefault(names[i].decode(), []).append(hip.ms(pev[2 * i], pev[2 * i + 1]))
    hip.destroy(pev)
    return stage_ms


def read_reference(torch, dev, hip, st, b: Bench, reps=20):
    """A plain streaming read of the same logits copies (one 1024-thread
    workgroup per row, non-temporal 16-byte loads), rotated like the steps."""
    wl = b.wl
    out = torch.empty(wl.B, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    row_bytes = wl.V * wl.elem_bytes

    def one(i):
        x = b.xs[i % b.copies]
        rc = st.vs_selftest_read_rows(x.data_ptr(), wl.B, row_bytes, row_bytes, 1, out.data_ptr(), stream)
        if rc:
            raise RuntimeError(f"vs_selftest_read_rows failed ({rc})")

    for i in range(3):
        one(i)
    torch.cuda.synchronize()
    ev = hip.create(2)
    hip.record(ev[0], stream)
    for i in range(reps):
        one(i)
    hip.record(ev[1], stream)
    torch.cuda.synchronize()
    ms = hip.ms(ev[0], ev[1]) / reps
    hip.destroy(ev)
    return {"kernel": "stream read, one 1024-thread workgroup per row (vs_selftest_read_rows)",
            "us": ms * 1e3, "GBps": b.logit_bytes / (ms * 1e-3) / 1e9}


def splitmix_reference(torch, dev, hip, st):
    """Words per second of a plain SplitMix64 stream over the whole chip."""
    blocks, n = 8192, 256
    out = torch.empty(blocks * 256, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    for _ in range(2):
        if st.vs_selftest_splitmix(blocks, n, out.data_ptr(), stream):
            raise RuntimeError("vs_selftest_splitmix failed")
    torch.cuda.synchronize()
    ev = hip.create(2)
    reps = 10
    hip.record(ev[0], stream)
    for _ in range(reps):
        st.vs_selftest_splitmix(blocks, n, out.data_ptr(), stream)
    hip.record(ev[1], stream)
    torch.cuda.synchronize()
    ms = hip.ms(ev[0], ev[1]) / reps
    hip.destroy(ev)
    return blocks * 256 * n / (ms * 1e-3)


def full_vocab_words(wl, kept):
    """Random words the Gumbel pass computes: one per kept id of every
    full-vocabulary row (not greedy, no top-k)."""
    greedy = (wl.temperature == 0) | (wl.top_k == 1) | (wl.top_p == 0) | (wl.min_p == 1)
    full = ~greedy & ((wl.top_k == 0) | (wl.top_k >= wl.V))
    return int(kept[full].astype(np.int64).sum())


def topp_method(wl, hints):
    """The method the library takes for full-vocabulary top-p rows without a
    kept mask (the rule its header states)."""
    import decode_token_sampling_amd as vs
    if hints & vs.OPT_TOPP_REJECTION:
        return "rejection"
    if hints & vs.OPT_TOPP_GATHER_DRAW:
        return "gather_draw"
    if hints & vs.OPT_TOPP_KEPT_PASS:
        return "kept_pass"
    return "gather_draw"


def rooflines(wl, b: Bench, stage_avg, ms_per_step, kept, splitmix_rate):
    """The roofline of each kernel stage that ran: HBM-bound passes against
    8 TB/s from their algorithmic bytes, the pass that forms the draw's random
    words against the vector ALUs' issue ceiling for them."""
    out = {}
    gather = topp_method(wl, b.hints) == "gather_draw"
    one_launch = set(stage_avg) == {"select"}
    for stage, ms in stage_avg.items():
        if stage == "select":
            by = b.logit_bytes + (wl.B * wl.V * 4 if (wl.full_logprobs and "lse_full" not in stage_avg) else 0)
            t = ms_per_step if one_launch else ms
            out[stage] = {"bound": "hbm", "achieved": by / (t * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                          "unit": "GB/s", "frac": by / (t * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                          "algorithmic_bytes_per_launch": by, "launch_ms": t,
                          "duration_source": "timed region, one launch per step" if one_launch
                          else "per-stage HIP events (eager steps)",
                          "traffic": load_traffic(wl.name, stage)}
        elif stage in ("full_prep", "lse_full"):
            by = 2 * b.logit_bytes if stage == "full_prep" else b.logit_bytes + wl.B * wl.V * 4
            out[stage] = {"bound": "hbm", "achieved": by / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS,
                          "unit": "GB/s", "frac": by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                          "algorithmic_bytes_per_launch": by, "launch_ms": ms,
                          "traffic": load_traffic(wl.name, stage)}
            if stage == "full_prep" and gather:  # the gather pass also forms the draw's words
                words = full_vocab_words(wl, kept)
                rate = words / (ms * 1e-3)
                out[stage]["draw_words"] = {
                    "bound": "alu", "achieved": rate / 1e12, "peak": SPLITMIX_PEAK_WORDS / 1e12,
                    "unit": "T SplitMix64 words/s", "frac": rate / SPLITMIX_PEAK_WORDS,
                    "words_per_launch": words,
                    "measured_splitmix_stream_Twords": splitmix_rate / 1e12}
        elif stage == "gumbel" and gather:  # finishing the rows: the list's kept ids
            out[stage] = {"bound": "latency", "launch_ms": ms,
                          "note": "the kept set's words were formed by the gather pass"}
        elif stage == "gumbel":
            words = full_vocab_words(wl, kept)
            rate = words / (ms * 1e-3)
            out[stage] = {"bound": "alu", "achieved": rate / 1e12, "peak": SPLITMIX_PEAK_WORDS / 1e12,
                          "unit": "T SplitMix64 words/s", "frac": rate / SPLITMIX_PEAK_WORDS,
                          "words_per_launch": words, "launch_ms": ms,
                          "measured_splitmix_stream_Twords": splitmix_rate / 1e12}
    return out


def measure(vs, torch, dev, hip, st, wl, steps, warmup, eager, splitmix_rate):
    b = Bench(vs, torch, wl, steps, dev)
    for i in range(warmup):
        b.step(i)
    torch.cuda.synchronize()
    total_ms, per_step = time_steps(torch, dev, hip, b, steps, eager=eager)
    ms_per_step = total_ms / steps
    if int((b.st != 0).sum().item()):
        raise RuntimeError(f"{wl.name}: rows reported a nonzero status")
    stage_ms = stage_profile(torch, dev, hip, vs.load(), b, min(steps, 32))
    stage_avg = {k: float(np.mean(v)) for k, v in stage_ms.items()}
    # one fresh step for the oracle's check
    b.restore()
    b.step(0)
    torch.cuda.synchronize()
    res_ids, res_kept = b.ids.cpu().numpy(), b.kept.cpu().numpy()
    side = 4 * ((len(wl.prompt_ids) if wl.prompt_ids is not None else 0) +
                (len(wl.output_ids) if wl.output_ids is not None else 0))
    alg = b.logit_bytes + side + (wl.B * wl.V * 4 if wl.full_logprobs else 0)
    rec = {
        "B": wl.B, "V": wl.V, "dtype": wl.dtype, "step": b.describe(), "input_copies": b.copies,
        "launch": "eager" if eager else "hipGraph replay", "steps": steps,
        "ms_per_step": ms_per_step, "rows_per_s": wl.B / (ms_per_step * 1e-3),
        "ms_per_step_p10_p50_p90": [pct(per_step, 10), pct(per_step, 50), pct(per_step, 90)],
        "percentiles_over": f"{len(per_step)} replays of {b.copies} steps",
        "algorithmic_bytes_per_step": alg,
        "logits_GBps": alg / (ms_per_step * 1e-3) / 1e9,
        "hbm_peak_frac": alg / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "stages_ms": stage_avg,
        "roofline": rooflines(wl, b, stage_avg, ms_per_step, res_kept, splitmix_rate),
        "read_reference": read_reference(torch, dev, hip, st, b),
        "description": wl.description,
    }
    rr = rec["read_reference"]
    rec["read_reference"]["step_vs_read"] = rr["us"] / (ms_per_step * 1e3)
    if b.pen is not None:
        t1, _ = time_steps(torch, dev, hip, b, steps, eager=eager, separate=True)
        sep_stages = stage_profile(torch, dev, hip, vs.load(), b, min(steps, 32), separate=True)
        rec["separate_penalize"] = {
            "ms_per_step": t1 / steps, "step": b.describe(separate=True),
            "stages_ms": {k: float(np.mean(v)) for k, v in sep_stages.items()}}
    full_topp = (~((wl.temperature == 0) | (wl.top_k == 1) | (wl.top_p == 0) | (wl.min_p == 1)) &
                 ((wl.top_k == 0) | (wl.top_k >= wl.V)) & (wl.top_p < 1)).any()
    if full_topp:  # each method for full-vocabulary top-p rows, timed beside the default
        rec["topp_methods"] = {}
        for name, bit in (("rejection", vs.OPT_TOPP_REJECTION),
                          ("gather_draw", vs.OPT_TOPP_GATHER_DRAW),
                          ("kept_pass", vs.OPT_TOPP_KEPT_PASS)):
            hr = b.hints | bit
            tr, _ = time_steps(torch, dev, hip, b, steps, hints=hr, eager=eager)
            rec["topp_methods"][name] = {"ms_per_step": tr / steps, "step": b.describe(hr)}
    if wl.name == HEADLINE and b.hints != 0:
        t0, _ = time_steps(torch, dev, hip, b, steps, hints=0, eager=eager)
        rec["no_hint"] = {"ms_per_step": t0 / steps, "step": b.describe(0),
                          "hbm_peak_frac": alg / (t0 / steps * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    del b
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec, res_ids, res_kept


def host_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = sorted(os.sched_getaffinity(0))
    except AttributeError:
        avail = list(range(os.cpu_count() or 1))
    return model, avail


def oracle_rows(oracle, wl, x, rows):
    """The whole step of the given rows: the draw, then the log-probs the
    workload asks for (a greedy row's log-prob at temperature 1)."""
    o = oracle.sample(x, wl.V, wl.temperature, wl.top_k, wl.top_p, wl.min_p, wl.seeds, rows=rows)
    for r in rows:
        oracle.logprobs(np.ascontiguousarray(x[r:r + 1]), wl.V,
                        None if wl.full_logprobs else o["ids"][r:r + 1], k=wl.logprob_k,
                        full=wl.full_logprobs)
    return o


def cpu_leg(wl, gpu_ids, gpu_kept, budget_s, pinned):
    """The oracle as it stands on the host. pinned: one thread pinned to one
    core over a bounded row sample (rows/s). Always: the same per-row function
    on every available core (at most MAX_POOL threads) over the whole batch,
    whose ids and kept counts are compared with the GPU's and whose near-tie
    rows are counted."""
    import oracle

    oracle.build(force=False)
    model, avail = host_info()
    x = wl.logits
    t_pen = 0.0
    if wl.has_penalties:
        x = x.copy()
        t0 = time.perf_counter()
        oracle.penalize(x, wl.V, wl.prompt_ids, wl.prompt_off, wl.output_ids, wl.output_off,
                        wl.presence, wl.frequency, wl.repetition)
        t_pen = time.perf_counter() - t0
    res = {"host_cpu": model, "host_cores_available": len(avail)}
    if pinned:
        saved = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {avail[0]})
        try:
            n, t = 0, 0.0
            while n < wl.B and (t < budget_s or n < 2):
                t0 = time.perf_counter()
                oracle_rows(oracle, wl, x, [n])
                t += time.perf_counter() - t0
                n += 1
        finally:
            os.sched_setaffinity(0, saved)
        total = t + t_pen * n / wl.B
        res["pinned"] = {"value": n / total, "unit": "rows/s", "cores": 1, "rows": n,
                         "seconds": total}
    nthreads = max(1, min(MAX_POOL, len(avail)))
    B = wl.B
    chunks = [list(range(i, B, nthreads)) for i in range(nthreads)]
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=nthreads) as ex:
        outs = list(ex.map(lambda rows: (rows, oracle_rows(oracle, wl, x, rows)), chunks))
    t_all = time.perf_counter() - t0 + t_pen
    ids = np.full(B, -1, np.int32)
    kept = np.zeros(B, np.int32)
    top2 = np.full((B, 2), -1.0)
    for rows, o in outs:
        ids[rows], kept[rows], top2[rows] = o["ids"][rows], o["kept"][rows], o["top2"][rows]
    g1, g2 = top2[:, 0], top2[:, 1]
    near = (g2 >= 0) & (g1 - g2 < 1e-6 * g1)
    res["all_cores"] = {"value": B / t_all, "unit": "rows/s", "cores": nthreads, "rows": B,
                        "seconds": t_all}
    res["near_tie_rows"] = int(near.sum())
    res["id_mismatch_rows"] = int(((ids != gpu_ids) & ~near).sum())
    res["kept_mismatch_rows"] = int((kept != gpu_kept).sum())
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="all", help="a workload name, or 'all' (headline first)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--eager", action="store_true", help="time eager launches, not HIP graphs")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of pinned one-thread oracle work on the headline")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first copy this many MiB device to device three times (HIP's copy "
                         "kernel), the known-size reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): every row of the "
              "sampling step stays on one device, and no multi-GPU path is built.", file=sys.stderr)
        sys.exit(2)

    import torch

    import decode_token_sampling_amd as vs
    import synth

    vs.load()
    st = selftest_lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hip = HipEvents()
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        a.fill_(1)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    names = ALL_WORKLOADS if args.workload == "all" else [args.workload]
    splitmix_rate = splitmix_reference(torch, dev, hip, st)

    configs, checks = {}, {}
    for name in names:
        wl = synth.make(name)
        t0 = time.time()
        rec, ids, kept = measure(vs, torch, dev, hip, st, wl, args.steps, args.warmup, args.eager,
                                 splitmix_rate)
        configs[name] = rec
        checks[name] = (wl, ids, kept)
        print(f"# {name}: {rec['ms_per_step'] * 1e3:.1f} us/step, {rec['rows_per_s']:.4g} rows/s "
              f"({time.time() - t0:.1f} s)", file=sys.stderr, flush=True)

    head_name = names[0]
    head = configs[head_name]
    wl_head = checks[head_name][0]
    dom = "select" if "select" in head["roofline"] else sorted(head["roofline"])[0]
    roof = dict(head["roofline"][dom])
    roof["kernel"] = dom
    result = {
        "metric": METRIC,
        "value": head["rows_per_s"],
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if wl_head.dtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": head_name, "B": wl_head.B, "V": wl_head.V, "logits": wl_head.dtype,
                   "step": head["step"], "input_copies": head["input_copies"],
                   "launch": head["launch"], "description": wl_head.description},
        "logits_GBps": head["logits_GBps"],
        "hbm_peak_frac": head["hbm_peak_frac"],
        "roofline": roof,
        "configs": configs,
    }
    if not args.no_cpu:
        for i, name in enumerate(names):
            wl, ids, kept = checks[name]
            t0 = time.time()
            c = cpu_leg(wl, ids, kept, args.cpu_budget, pinned=(i == 0))
            configs[name]["oracle"] = c
            print(f"# oracle {name}: {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
        c = configs[head_name]["oracle"]
        result["cpu_baseline"] = {
            "value": c["pinned"]["value"], "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{c['pinned']['rows']} of {wl_head.B} rows of {head_name}, whole step per "
                      f"row, one thread pinned to one core of {c['host_cpu']} "
                      f"({c['host_cores_available']} cores available), {c['pinned']['seconds']:.1f} s",
            "all_cores": c["all_cores"],
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
