"""Helpers for GPU-vs-oracle parity tests: run both sides on the same host bytes.

The GPU side goes through the C ABI (via the package's ctypes binding); the
oracle side through oracle/. Inputs come from synth (data only).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

NEAR_TIE_REL = 1e-6      # rows whose two best Gumbel scores are closer are exempt for the id
LOGPROB_ATOL = 1e-5


def to_device(x: np.ndarray, ld: int | None = None, pad_value=None) -> torch.Tensor:
    """Host logits (float32, or uint16 bf16 bits) -> device tensor [B, ld] (columns >= V padded)."""
    B, V = x.shape
    ld = ld or V
    if x.dtype == np.float32:
        t = torch.empty((B, ld), dtype=torch.float32, device="cuda")
        if ld > V:
            t.fill_(float("nan") if pad_value is None else pad_value)
        t[:, :V] = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    else:
        t = torch.empty((B, ld), dtype=torch.bfloat16, device="cuda")
        if ld > V:
            t.fill_(float("nan") if pad_value is None else pad_value)
        t[:, :V] = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return t


def from_device(t: torch.Tensor, V: int) -> np.ndarray:
    """Device logits -> host array in the oracle's format ([B, V] float32 or uint16 bits)."""
    t = t[:, :V].contiguous()
    if t.dtype == torch.float32:
        return t.cpu().numpy()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host_pad(x: np.ndarray, ld: int) -> np.ndarray:
    """Host copy with row stride ld (the oracle reads only the first V columns)."""
    B, V = x.shape
    out = np.zeros((B, ld), x.dtype)
    out[:, :V] = x
    return out


def mask_bits(mask: torch.Tensor, V: int) -> np.ndarray:
    m = mask.cpu().numpy().astype(np.uint32).view(np.uint8)
    bits = np.unpackbits(m, axis=1, bitorder="little")
    return bits[:, :V]


def dev(a, dtype):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=dtype)).cuda()


def gpu_sample(xd: torch.Tensor, V: int, w, hints=0, mask=True):
    import decode_token_sampling_amd as vs
    out = vs.sample(xd, temperature=dev(w["temperature"], np.float32),
                    top_k=dev(w["top_k"], np.int32), top_p=dev(w["top_p"], np.float32),
                    min_p=dev(w["min_p"], np.float32),
                    seeds=dev(np.asarray(w["seeds"], np.uint64).view(np.int64), np.int64),
                    hints=hints, V=V, mask=mask)
    torch.cuda.synchronize()
    res = dict(ids=out["ids"].cpu().numpy(), kept=out["kept"].cpu().numpy(),
               status=out["status"].cpu().numpy())
    if mask:
        res["mask"] = mask_bits(out["mask"], V)
    return res


def compare_sample(g, o, rows=None, check_mask=True):
    """Assert GPU == oracle: status, kept counts and kept sets bit-exact; ids
    bit-exact except near-tie rows. Returns the number of near-tie rows."""
    rows = np.arange(len(o["ids"])) if rows is None else np.asarray(rows)
    assert np.array_equal(g["status"][rows], o["status"][rows]), (
        rows[g["status"][rows] != o["status"][rows]][:10], g["status"][rows][:10], o["status"][rows][:10])
    assert np.array_equal(g["kept"][rows], o["kept"][rows]), (
        rows[g["kept"][rows] != o["kept"][rows]][:10],
        g["kept"][rows][g["kept"][rows] != o["kept"][rows]][:10],
        o["kept"][rows][g["kept"][rows] != o["kept"][rows]][:10])
    if check_mask and "mask" in o and "mask" in g:
        bad = [r for r in rows if not np.array_equal(g["mask"][r], o["mask"][r])]
        assert not bad, f"kept sets differ on rows {bad[:10]}"
    g1, g2 = o["top2"][rows, 0], o["top2"][rows, 1]
    near = (g2 >= 0) & (g1 - g2 < NEAR_TIE_REL * g1)
    diff = (g["ids"][rows] != o["ids"][rows]) & ~near
    assert not diff.any(), (rows[diff][:10], g["ids"][rows][diff][:10], o["ids"][rows][diff][:10])
    return int(near.sum())


def oracle_sample(x: np.ndarray, V: int, w, mask=True, rows=None):
    return oracle.sample(x, V, w["temperature"], w["top_k"], w["top_p"], w["min_p"],
                         np.asarray(w["seeds"], np.uint64), want_mask=mask, rows=rows)


def params_from(wl: synth.Workload):
    return dict(temperature=wl.temperature, top_k=wl.top_k, top_p=wl.top_p, min_p=wl.min_p,
                seeds=wl.seeds)


def random_params(rng: np.random.Generator, B: int, V: int, kinds=None):
    """Per-row parameters that cover every path: greedy (all four triggers),
    top-k fast (k <= 64) and slow (k <= 1024), full vocabulary without
    truncation, with min-p, with top-p, and combinations."""
    kinds = kinds or ["greedy", "kfast", "kslow", "none", "minp", "topp", "topp_minp", "k_topp",
                      "k_minp_topp"]
    T = np.empty(B, np.float32)
    k = np.zeros(B, np.int32)
    p = np.ones(B, np.float32)
    mp = np.zeros(B, np.float32)
    for r in range(B):
        kind = kinds[r % len(kinds)]
        T[r] = rng.choice([1.0, 0.7, 1.3, float(np.float32(rng.uniform(0.2, 3.0)))])
        if kind == "greedy":
            trig = r // len(kinds) % 4
            if trig == 0:
                T[r] = 0.0
            elif trig == 1:
                k[r] = 1
            elif trig == 2:
                p[r] = 0.0
            else:
                mp[r] = 1.0
        elif kind == "kfast":
            k[r] = rng.integers(2, 65)
        elif kind == "kslow":
            k[r] = rng.integers(65, 1025)
        elif kind == "minp":
            mp[r] = rng.choice([0.01, 0.1, 0.5])
        elif kind == "topp":
            p[r] = rng.uniform(0.05, 0.999)
        elif kind == "topp_minp":
            p[r] = rng.uniform(0.3, 0.99)
            mp[r] = rng.choice([0.001, 0.05])
        elif kind == "k_topp":
            k[r] = rng.choice([2, 20, 50, 64, 300])
            p[r] = rng.uniform(0.2, 0.99)
        elif kind == "k_minp_topp":
            k[r] = rng.choice([8, 40, 200])
            p[r] = rng.uniform(0.2, 0.99)
            mp[r] = 0.02
    return dict(temperature=T, top_k=k, top_p=p, min_p=mp,
                seeds=rng.integers(0, 2**63, B, dtype=np.int64).astype(np.uint64))
