"""Seeded synthetic workloads for the sampling step.

This module only generates inputs (logits, per-row parameters, token
histories). It contains none of the sampling arithmetic, so both the GPU
library's tests and the CPU oracle can be fed the same bytes from it.

Logit construction (per workload): a Gaussian term plus a Zipf-like rank term
``scale * N(0,1) - 1.5 * ln(rank_j)``, where ``rank`` is one seeded permutation
of 1..V shared by every row; "N(mu, s)" is read with ``s`` the standard
deviation. bf16 logits are produced by rounding the fp32 values to nearest-even
and are returned as raw ``uint16`` bits. Zipf(a) token ids are ``k - 1`` with
``k`` drawn from P(k) proportional to k**-a on 1..V by inverse CDF.

Workload names describe their shapes:
  w4x32000_f32     4 rows, fp32, mixed greedy / top-k+top-p / top-p / untruncated
  w32x151936_bf16  32 rows, bf16, random per-row parameters and penalties
  w256x248320_f32  256 rows, fp32, temperature 1, top-k 20, top-p 0.95
  w1024x128256_f32 1024 rows, fp32, greedy, full log-softmax output
  w64x262144_bf16  64 rows, bf16, peaked and flat rows, top-p 0.99, penalties
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np


@dataclass
class Workload:
    name: str
    B: int
    V: int
    dtype: str                      # "f32" or "bf16"
    logits: np.ndarray              # [B, V] float32, or uint16 bf16 bits
    temperature: np.ndarray         # [B] float32
    top_k: np.ndarray               # [B] int32
    top_p: np.ndarray               # [B] float32
    min_p: np.ndarray               # [B] float32
    seeds: np.ndarray               # [B] uint64
    prompt_ids: Optional[np.ndarray] = None   # CSR token history
    prompt_off: Optional[np.ndarray] = None
    output_ids: Optional[np.ndarray] = None
    output_off: Optional[np.ndarray] = None
    presence: Optional[np.ndarray] = None
    frequency: Optional[np.ndarray] = None
    repetition: Optional[np.ndarray] = None
    logprob_k: int = 0              # top-k log-probs wanted
    full_logprobs: bool = False     # full [B, V] log-softmax wanted
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def has_penalties(self) -> bool:
        return self.repetition is not None or self.presence is not None or self.frequency is not None

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest-even); returns uint16 bits. Input data prep only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + (0x7FFF + ((u >> 16) & 1))) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32)


def zipf_ids(rng: np.random.Generator, n: int, V: int, a: float = 1.1) -> np.ndarray:
    k = np.arange(1, V + 1, dtype=np.float64)
    cdf = np.cumsum(k ** (-a))
    cdf /= cdf[-1]
    u = rng.random(n)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, V - 1).astype(np.int32)


def gaussian_rank_logits(rng: np.random.Generator, B: int, V: int, scale: float) -> np.ndarray:
    """scale * N(0,1) - 1.5 * ln(rank_j); one rank permutation shared by all rows."""
    rank = rng.permutation(V).astype(np.float64) + 1.0
    rank_term = (1.5 * np.log(rank)).astype(np.float32)
    out = np.empty((B, V), np.float32)
    for r in range(B):
        g = rng.standard_normal(V, dtype=np.float32)
        out[r] = np.float32(scale) * g - rank_term
    return out


def _csr(lists):
    off = np.zeros(len(lists) + 1, np.int32)
    off[1:] = np.cumsum([len(l) for l in lists])
    ids = np.concatenate(lists).astype(np.int32) if lists else np.zeros(0, np.int32)
    return ids, off


def w4x32000_f32() -> Workload:
    rng = np.random.default_rng(101)
    B, V = 4, 32000
    x = gaussian_rank_logits(rng, B, V, 2.0)
    return Workload(
        "w4x32000_f32", B, V, "f32", x,
        temperature=np.array([0.0, 1.0, 0.7, 1.0], np.float32),
        top_k=np.array([0, 8, 0, 0], np.int32),
        top_p=np.array([1.0, 0.5, 0.9, 1.0], np.float32),
        min_p=np.zeros(B, np.float32),
        seeds=np.full(B, 1234, np.uint64),
        logprob_k=0,
        description="B=4 V=32000 fp32; greedy, (T1 k8 p0.5), (T0.7 p0.9), untruncated; seed 1234",
    )


def w32x151936_bf16() -> Workload:
    rng = np.random.default_rng(102)
    B, V = 32, 151936
    x = gaussian_rank_logits(rng, B, V, 2.0)
    T = rng.uniform(0.5, 1.5, B).astype(np.float32)
    k = rng.choice(np.array([0, 20, 50], np.int32), B).astype(np.int32)
    p = rng.uniform(0.8, 1.0, B).astype(np.float32)
    mp = rng.choice(np.array([0.0, 0.05], np.float32), B).astype(np.float32)
    plen = rng.integers(32, 1025, B)
    olen = rng.integers(32, 257, B)
    pids, poff = _csr([zipf_ids(rng, int(n), V) for n in plen])
    oids, ooff = _csr([zipf_ids(rng, int(n), V) for n in olen])
    return Workload(
        "w32x151936_bf16", B, V, "bf16", f32_to_bf16_bits(x),
        temperature=T, top_k=k, top_p=p, min_p=mp,
        seeds=(1234 + np.arange(B)).astype(np.uint64),
        prompt_ids=pids, prompt_off=poff, output_ids=oids, output_off=ooff,
        presence=rng.uniform(0, 1, B).astype(np.float32),
        frequency=rng.uniform(0, 1, B).astype(np.float32),
        repetition=rng.uniform(1.0, 1.3, B).astype(np.float32),
        logprob_k=0,
        description="B=32 V=151936 bf16; random T/k/p/min-p; prompt+output Zipf(1.1) penalties",
    )


def w256x248320_f32() -> Workload:
    rng = np.random.default_rng(103)
    B, V = 256, 248320
    x = gaussian_rank_logits(rng, B, V, 3.0)
    return Workload(
        "w256x248320_f32", B, V, "f32", x,
        temperature=np.ones(B, np.float32),
        top_k=np.full(B, 20, np.int32),
        top_p=np.full(B, 0.95, np.float32),
        min_p=np.zeros(B, np.float32),
        seeds=(1234 + np.arange(B)).astype(np.uint64),
        logprob_k=20,
        description="B=256 V=248320 fp32; T 1.0, top-k 20, top-p 0.95; id + logprob + top-20 logprobs",
    )


def w1024x128256_f32() -> Workload:
    rng = np.random.default_rng(104)
    B, V = 1024, 128256
    x = np.empty((B, V), np.float32)
    for r in range(B):
        x[r] = np.float32(4.0) * rng.standard_normal(V, dtype=np.float32)
        peaks = rng.choice(V, 50, replace=False)
        x[r, peaks] += np.float32(8.0)
    return Workload(
        "w1024x128256_f32", B, V, "f32", x,
        temperature=np.zeros(B, np.float32),
        top_k=np.zeros(B, np.int32),
        top_p=np.ones(B, np.float32),
        min_p=np.zeros(B, np.float32),
        seeds=(1234 + np.arange(B)).astype(np.uint64),
        logprob_k=20, full_logprobs=True,
        description="B=1024 V=128256 fp32 N(0,4) + 50 peaks at +8; greedy; full log-softmax + top-20",
    )


def w64x262144_bf16() -> Workload:
    rng = np.random.default_rng(105)
    B, V = 64, 262144
    x = np.empty((B, V), np.float32)
    for r in range(B):
        if r < B // 2:
            x[r] = rng.standard_normal(V, dtype=np.float32)
            x[r, rng.integers(0, V)] += np.float32(15.0)
        else:
            x[r] = np.float32(0.1) * rng.standard_normal(V, dtype=np.float32)
    rows = np.arange(B)
    T = np.where(rows % 8 == 0, 0.0, 1.0).astype(np.float32)
    mp = np.where(rows % 4 == 0, 0.01, 0.0).astype(np.float32)
    oids, ooff = _csr([zipf_ids(rng, 2048, V) for _ in range(B)])
    return Workload(
        "w64x262144_bf16", B, V, "bf16", f32_to_bf16_bits(x),
        temperature=T, top_k=np.zeros(B, np.int32), top_p=np.full(B, 0.99, np.float32),
        min_p=mp, seeds=(1234 + np.arange(B)).astype(np.uint64),
        output_ids=oids, output_off=ooff,
        repetition=np.full(B, 1.2, np.float32),
        presence=np.zeros(B, np.float32), frequency=np.zeros(B, np.float32),
        logprob_k=0,
        description="B=64 V=262144 bf16; peaked/flat rows; top-p 0.99, min-p 0.01 every 4th row, "
                    "greedy every 8th; repetition 1.2 from 2048 Zipf output ids",
    )


WORKLOADS = {
    "w4x32000_f32": w4x32000_f32,
    "w32x151936_bf16": w32x151936_bf16,
    "w256x248320_f32": w256x248320_f32,
    "w1024x128256_f32": w1024x128256_f32,
    "w64x262144_bf16": w64x262144_bf16,
}


def make(name: str) -> Workload:
    return WORKLOADS[name]()


def random_rows(seed: int, B: int, V: int, dtype: str = "f32", kind: str = "rank",
                scale: float = 2.0) -> np.ndarray:
    """Small seeded logits for parity and edge cases. kind: rank | normal | ties | flat."""
    rng = np.random.default_rng(seed)
    if kind == "rank":
        x = gaussian_rank_logits(rng, B, V, scale)
    elif kind == "normal":
        x = (np.float32(scale) * rng.standard_normal((B, V), dtype=np.float32))
    elif kind == "ties":
        # few distinct values: heavy ties everywhere, including at any cut-off
        x = rng.integers(-4, 5, (B, V)).astype(np.float32) * np.float32(0.5)
    elif kind == "flat":
        x = np.float32(0.1) * rng.standard_normal((B, V), dtype=np.float32)
    else:
        raise ValueError(kind)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x
