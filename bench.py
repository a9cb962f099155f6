#!/usr/bin/env python3
"""Benchmark of the batched decode-step sampling path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole sampling path over one batch of synthetic
logits already resident in HBM: occurrence penalties when the workload has
them (vs_penalize), then the draw and the log-probabilities the workload asks
for in one call (vs_sample_logprobs, one read of the logits). Rotated copies of the inputs (together larger than the 256 MB
Infinity Cache) keep repeat reads from being served on chip. Prints one JSON
line: rows/s for the whole step, the logits bandwidth it implies, the roofline
of the dominant kernel (timed with HIP events on the stream it runs on) and
the CPU oracle timed on a bounded sample of the same work.
"""
from __future__ import annotations

import argparse
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
DEFAULT_WORKLOAD = "w256x248320_f32"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {"select": "k_select.hip", "lse_select": "k_select.hip", "row": "k_row.hip",
                  "full_prep": "k_full.hip",
                  "lse_row": "k_row.hip", "row_full": "k_row.hip", "gumbel": "k_gumbel.hip",
                  "lse_full": "k_gumbel.hip", "penalize": "k_penalize.hip"}


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


def build_step(vs, torch, wl, copies, dev):
    """Device buffers and the step closure for one workload."""
    import synth  # noqa: F401  (data already generated)

    B, V = wl.B, wl.V
    d = lambda a, dt: None if a is None else torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(dev)
    if wl.dtype == "f32":
        base = torch.from_numpy(wl.logits).to(dev)
    else:
        base = torch.from_numpy(wl.logits.view(np.int16)).to(dev).view(torch.bfloat16)
    xs = [base] + [base.clone() for _ in range(copies - 1)]
    T = d(wl.temperature, np.float32)
    K = d(wl.top_k, np.int32)
    P = d(wl.top_p, np.float32)
    MP = d(wl.min_p, np.float32)
    S = d(np.asarray(wl.seeds, np.uint64), np.int64)
    pen = None
    if wl.has_penalties:
        pen = [d(wl.prompt_ids, np.int32), d(wl.prompt_off, np.int32), d(wl.output_ids, np.int32),
               d(wl.output_off, np.int32), d(wl.presence, np.float32), d(wl.frequency, np.float32),
               d(wl.repetition, np.float32)]
    ws = vs.workspace(B, V, base.dtype, dev)
    ids = torch.empty(B, dtype=torch.int32, device=dev)
    kept = torch.empty(B, dtype=torch.int32, device=dev)
    st = torch.empty(B, dtype=torch.int32, device=dev)
    pst = torch.empty(B, dtype=torch.int32, device=dev)
    full = torch.empty((B, V), dtype=torch.float32, device=dev) if wl.full_logprobs else None
    # the promises a serving engine derives from its batch's parameters
    hints = vs.hints_for(wl.temperature, wl.top_k, wl.top_p, wl.min_p, V)
    want_token_lp = not wl.full_logprobs

    tlp = torch.empty(B, dtype=torch.float32, device=dev) if want_token_lp else None
    tids = torch.empty((B, wl.logprob_k), dtype=torch.int32, device=dev) if wl.logprob_k else None
    tlps = torch.empty((B, wl.logprob_k), dtype=torch.float32, device=dev) if wl.logprob_k else None

    def step(i):
        x = xs[i % copies]
        if pen is not None:
            vs.penalize(x, *pen, row_status=pst)
        vs.sample_logprobs(x, T, K, P, MP, S, hints=hints, k=wl.logprob_k,
                           token_logprob=want_token_lp, ws=ws, out_ids=ids, kept=kept,
                           row_status=st, out_token_lp=tlp, out_topk_ids=tids, out_topk_lp=tlps,
                           out_full=full)

    parts = (["vs_penalize"] if pen is not None else []) + [
        f"vs_sample_logprobs(hints={hints}; " + ", ".join(p for p in [
            "sampled-id lp" if want_token_lp else "", f"top-{wl.logprob_k}" if wl.logprob_k else "",
            "full [B,V] write" if wl.full_logprobs else ""] if p) + ")"]
    outs = dict(ids=ids, kept=kept, status=st)
    return step, " + ".join(parts), outs, base.dtype


def cpu_baseline(wl, budget_s=12.0):
    """The oracle as it stands, single-threaded, on a bounded row sample."""
    import oracle

    oracle.build(force=False)
    B, V = wl.B, wl.V
    x = wl.logits
    t_pen = 0.0
    if wl.has_penalties:
        x = x.copy()
        t0 = time.perf_counter()
        oracle.penalize(x, V, wl.prompt_ids, wl.prompt_off, wl.output_ids, wl.output_off,
                        wl.presence, wl.frequency, wl.repetition)
        t_pen = time.perf_counter() - t0
    n = 0
    t_rows = 0.0
    while n < B and (t_rows < budget_s or n < 2):
        r = n
        t0 = time.perf_counter()
        o = oracle.sample(x, V, wl.temperature, wl.top_k, wl.top_p, wl.min_p, wl.seeds, rows=[r])
        oracle.logprobs(np.ascontiguousarray(x[r:r + 1]), V,
                        None if wl.full_logprobs else o["ids"][r:r + 1], k=wl.logprob_k,
                        full=wl.full_logprobs)
        t_rows += time.perf_counter() - t0
        n += 1
    total = t_rows + t_pen * n / B
    return {"value": n / total, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} of {B} rows of {wl.name}, whole step per row (penalties scaled from "
                      f"the full batch) on one host thread, {total:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--copies", type=int, default=0, help="rotated input copies (0: auto)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--eager", action="store_true", help="time eager launches, not a HIP graph")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the sampling path keeps "
              "each row on one device and this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import decode_token_sampling_amd as vs
    import synth

    vs.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.make(args.workload)
    elem = wl.elem_bytes
    logit_bytes = wl.B * wl.V * elem
    copies = args.copies or min(64, max(3, math.ceil(768e6 / logit_bytes)))
    step, step_desc, outs, _ = build_step(vs, torch, wl, copies, dev)
    hip = HipEvents()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # Headline timing: the step for every input copy captured once into a HIP
    # graph (the library allocates and synchronises nothing, so the calls are
    # capturable), replayed back to back.
    graph = None
    if not args.eager:
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            for i in range(copies):
                step(i)
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(copies):
                step(i)
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
    replays = max(1, math.ceil(args.steps / copies))
    steps = replays * copies if graph is not None else args.steps
    stream = torch.cuda.current_stream(dev).cuda_stream
    ev = hip.create(2)
    hip.record(ev[0], stream)
    if graph is not None:
        for _ in range(replays):
            graph.replay()
    else:
        for i in range(steps):
            step(i)
    hip.record(ev[1], stream)
    torch.cuda.synchronize()
    total_ms = hip.ms(ev[0], ev[1])
    ms_per_step = total_ms / steps
    hip.destroy(ev)
    assert int((outs["status"] != 0).sum().item()) == 0, "rows reported a nonzero status"

    # Per-stage durations: eager steps with every kernel stage bracketed by HIP
    # events on its own stream, queued behind a spin kernel so that the events
    # time the GPU, not the host's enqueue rate.
    nprof = min(args.steps, 64)
    cap = 2 * 8 * nprof
    pev = hip.create(cap)
    lib = vs.load()
    torch.cuda._sleep(int(2.4e9 * 0.02))
    if lib.vs_profile_begin(pev, cap) != 0:
        raise RuntimeError("vs_profile_begin failed")
    for i in range(nprof):
        step(i)
    names = (ctypes.c_char_p * (cap // 2))()
    n = lib.vs_profile_end(names, cap // 2)
    torch.cuda.synchronize()
    stage_ms = {}
    for i in range(n):
        stage_ms.setdefault(names[i].decode(), []).append(hip.ms(pev[2 * i], pev[2 * i + 1]))
    hip.destroy(pev)
    stage_avg = {k: float(np.mean(v)) for k, v in stage_ms.items()}

    # Dominant kernel: the streaming pass (one read of the logits, plus the
    # full log-softmax write when the workload asks for it and the pass writes
    # it itself), or the separate full log-softmax write when one ran.
    dom = "lse_full" if (wl.full_logprobs and "lse_full" in stage_avg) else "select"
    dom_bytes = logit_bytes + (wl.B * wl.V * 4 if wl.full_logprobs else 0)
    dom_ms = stage_avg[dom]
    duration_source = "per-stage HIP events (eager steps)"
    if set(stage_ms) == {dom} and len(stage_ms[dom]) == nprof:
        # the step is this one launch: its average duration is the timed
        # region's (HIP events around the graph replays on the kernel's
        # stream, including the gap between consecutive launches)
        dom_ms = ms_per_step
        duration_source = "timed region, one launch per step (HIP events)"
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    side = 0
    if wl.has_penalties:
        side += 4 * (len(wl.prompt_ids) if wl.prompt_ids is not None else 0)
        side += 4 * (len(wl.output_ids) if wl.output_ids is not None else 0)
    alg_bytes = logit_bytes + side + (wl.B * wl.V * 4 if wl.full_logprobs else 0)
    step_gbps = alg_bytes / (ms_per_step * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": wl.B / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "V": wl.V, "logits": wl.dtype,
                   "step": step_desc, "input_copies": copies,
                   "launch": "eager" if graph is None else "hipGraph replay",
                   "description": wl.description},
        "logits_GBps": step_gbps,
        "hbm_peak_frac": step_gbps / HBM_PEAK_GBPS,
        "stages_ms": stage_avg,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "algorithmic_bytes_per_launch": dom_bytes, "launch_ms": dom_ms,
                     "duration_source": duration_source,
                     "traffic": load_traffic(wl.name, dom)},
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
