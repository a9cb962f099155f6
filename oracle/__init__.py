"""CPU oracle for batched decode-step token sampling (ctypes over liboracle.so).

TEST INFRASTRUCTURE ONLY. The tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use this module; the product package
never imports it. The oracle is a plain single-threaded C++ statement of the
sampling step (see ``oracle.cpp`` for the page passages each part follows).

All array arguments are numpy arrays on the host. bf16 logits are passed as
``uint16`` arrays holding the raw bf16 bits.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("DTS_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

ROW_BAD_PARAM = 1
ROW_BAD_LOGITS = 2
ROW_BAD_TOKEN_ID = 4
ROW_TOPK_UNSUPPORTED = 8


def build(force: bool = True, path: str | None = None, sanitize: bool = False) -> str:
    """Compile liboracle.so with g++ (no fast-math, no FP contraction).

    ``path``: where to write it (default: the library this module loads).
    ``sanitize``: build with AddressSanitizer and UndefinedBehaviorSanitizer,
    every report fatal (load it with gcc's libasan and libubsan preloaded)."""
    path = path or LIB_PATH
    if force or not os.path.exists(path):
        san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
               "-g"] if sanitize else []
        cmd = [
            "g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
            "-fPIC", "-shared", "-Wall", "-Wextra", *san,
            os.path.join(_HERE, "oracle.cpp"), "-o", path + ".tmp",
        ]
        subprocess.run(cmd, check=True)
        os.replace(path + ".tmp", path)
    return path


def _configure(lib):
    """Argument and result types of the library's entry points."""
    P = ctypes.c_void_p
    i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.oracle_penalize.argtypes = [P, i32, i32, i32, i64, P, P, P, P, P, P, P, P, P]
    lib.oracle_sample.argtypes = [P, i32, i32, i32, i64, P, P, P, P, P, P, P, P, P, P]
    lib.oracle_sample_row.argtypes = [P, i32, i32, i32, i64, i32, P, P, P, P, P, P, P, P, P, P]
    lib.oracle_logprobs.argtypes = [P, i32, i32, i32, i64, P, P, i32, P, P, P, P]
    lib.oracle_logprobs_t.argtypes = [P, i32, i32, i32, i64, P, P, P, i32, P, P, P, P]
    lib.oracle_topp_decay.argtypes = [i32, P, P, P, P, P, P, P]
    lib.oracle_seed_advance.argtypes = [i32, P, P]
    lib.oracle_slot_remap.argtypes = [i32, i32, P, P, P, i32, P]
    lib.oracle_exp_pinned.argtypes = [f32]
    lib.oracle_exp_pinned.restype = f32
    lib.oracle_splitmix64.argtypes = [ctypes.c_uint64]
    lib.oracle_splitmix64.restype = ctypes.c_uint64
    lib.oracle_uniform.argtypes = [ctypes.c_uint64, i32, i32]
    lib.oracle_uniform.restype = ctypes.c_double
    lib.oracle_f32_to_bf16.argtypes = [f32]
    lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.oracle_exp_scan.argtypes = [f32, f32, ctypes.POINTER(ctypes.c_double)]
    lib.oracle_exp_scan.restype = ctypes.c_long
    lib.oracle_exp_compare.argtypes = [ctypes.c_uint32, ctypes.c_uint32, P,
                                       ctypes.POINTER(ctypes.c_uint32)]
    lib.oracle_exp_compare.restype = ctypes.c_long
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = _configure(ctypes.CDLL(LIB_PATH))
    return _lib


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _dtype_code(logits: np.ndarray) -> int:
    if logits.dtype == np.float32:
        return 0
    if logits.dtype == np.uint16:
        return 1
    raise TypeError("logits must be float32 or uint16 (bf16 bits)")


def _as(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


def penalize(logits, V, prompt_ids=None, prompt_off=None, output_ids=None,
             output_off=None, presence=None, frequency=None, repetition=None,
             prompt_ignore=None):
    """Apply occurrence penalties in place on a [B, ld] array; returns row status.
    prompt_ignore: per-row prompt_ignore_length (None: 0)."""
    lib = _load()
    B, ld = logits.shape
    st = np.zeros(B, np.int32)
    args = [_as(prompt_ids, np.int32), _as(prompt_off, np.int32), _as(output_ids, np.int32),
            _as(output_off, np.int32), _as(presence, np.float32), _as(frequency, np.float32),
            _as(repetition, np.float32), _as(prompt_ignore, np.int32)]
    lib.oracle_penalize(_ptr(logits), _dtype_code(logits), B, V, ld, *[_ptr(a) for a in args],
                        _ptr(st))
    return st


def sample(logits, V, temperature, top_k, top_p, min_p, seeds, want_mask=False, rows=None):
    """Sample one id per row. Returns dict(ids, kept, status, top2[, mask]).

    ``rows`` restricts the work to a subset of rows (others are left as -1)."""
    lib = _load()
    B, ld = logits.shape
    T = _as(temperature, np.float32)
    K = _as(top_k, np.int32)
    Pp = _as(top_p, np.float32)
    Mp = _as(min_p, np.float32)
    S = _as(seeds, np.uint64)
    ids = np.full(B, -1, np.int32)
    kept = np.zeros(B, np.int32)
    st = np.zeros(B, np.int32)
    top2 = np.full((B, 2), -1.0, np.float64)
    mask = np.zeros((B, V), np.uint8) if want_mask else None
    dt = _dtype_code(logits)
    if rows is None:
        lib.oracle_sample(_ptr(logits), dt, B, V, ld, _ptr(T), _ptr(K), _ptr(Pp), _ptr(Mp),
                          _ptr(S), _ptr(ids), _ptr(kept), _ptr(mask), _ptr(top2), _ptr(st))
    else:
        for r in rows:
            lib.oracle_sample_row(_ptr(logits), dt, B, V, ld, int(r), _ptr(T), _ptr(K), _ptr(Pp),
                                  _ptr(Mp), _ptr(S), _ptr(ids), _ptr(kept), _ptr(mask),
                                  _ptr(top2), _ptr(st))
    out = dict(ids=ids, kept=kept, status=st, top2=top2)
    if want_mask:
        out["mask"] = mask
    return out


def logprobs(logits, V, token_ids=None, k=0, full=False, temperature=None):
    """Log-softmax log-probs in fp64 (of x / T per row when temperature is given).
    Returns dict(token_lp, topk_ids, topk_lp, full, status)."""
    lib = _load()
    B, ld = logits.shape
    tok = _as(token_ids, np.int32)
    tlp = np.zeros(B, np.float64) if tok is not None else None
    tids = np.zeros((B, max(k, 0)), np.int32)
    tlps = np.zeros((B, max(k, 0)), np.float64)
    fullo = np.zeros((B, V), np.float64) if full else None
    st = np.zeros(B, np.int32)
    Tv = _as(temperature, np.float32)
    lib.oracle_logprobs_t(_ptr(logits), _dtype_code(logits), B, V, ld, _ptr(Tv), _ptr(tok),
                          _ptr(tlp), k, _ptr(tids), _ptr(tlps), _ptr(fullo), _ptr(st))
    return dict(token_lp=tlp, topk_ids=tids, topk_lp=tlps, full=fullo, status=st)


def topp_decay(top_p, top_p_init, decay, sampled, top_p_min=None, reset_ids=None):
    """Top-p decay after one sampled token, in place on the fp32 array top_p;
    returns row status."""
    lib = _load()
    B = len(top_p)
    st = np.zeros(B, np.int32)
    args = [_as(top_p_init, np.float32), _as(decay, np.float32), _as(top_p_min, np.float32),
            _as(reset_ids, np.int32), _as(sampled, np.int32)]
    lib.oracle_topp_decay(B, _ptr(top_p), *[_ptr(a) for a in args], _ptr(st))
    return st


def seed_advance(seeds, sampled=None):
    """One new seed per row per sampled token, in place on the uint64 array seeds."""
    lib = _load()
    lib.oracle_seed_advance(len(seeds), _ptr(seeds), _ptr(_as(sampled, np.int32)))


def slot_remap(remap, src, dst):
    """dst[i] = src[remap[i]] in place on dst (4- or 8-byte elements); returns row status."""
    lib = _load()
    remap = _as(remap, np.int32)
    assert src.dtype == dst.dtype and src.itemsize in (4, 8) and dst.flags["C_CONTIGUOUS"]
    st = np.zeros(len(remap), np.int32)
    lib.oracle_slot_remap(len(remap), len(src), _ptr(remap), _ptr(np.ascontiguousarray(src)),
                          _ptr(dst), src.itemsize, _ptr(st))
    return st


def exp_pinned(t: float) -> float:
    return _load().oracle_exp_pinned(float(t))


def splitmix64(x: int) -> int:
    return _load().oracle_splitmix64(x)


def uniform(seed: int, row: int, idx: int) -> float:
    return _load().oracle_uniform(seed, row, idx)


def f32_to_bf16(f: float) -> int:
    return _load().oracle_f32_to_bf16(float(f))


def exp_compare(lo_bits: int, got: np.ndarray):
    """Number of got[i] (fp32) whose bits differ from E(float bits lo_bits + i),
    and the first such i (len(got) if none)."""
    lib = _load()
    got = np.ascontiguousarray(got, np.float32)
    first = ctypes.c_uint32(0)
    bad = lib.oracle_exp_compare(lo_bits, len(got), _ptr(got), ctypes.byref(first))
    return int(bad), int(first.value)


def exp_scan(lo: float, hi: float):
    """(monotonicity violations, max ulp error vs an 80-bit exp) over all floats in [lo, hi]."""
    mu = ctypes.c_double(0.0)
    v = _load().oracle_exp_scan(float(lo), float(hi), ctypes.byref(mu))
    return v, mu.value
