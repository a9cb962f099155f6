"""Batched decode-step token sampling on AMD MI355X (gfx950).

A thin ctypes binding over ``libvs.so``, whose C ABI is declared in
``include/vs.h``. This module only marshals arguments: torch tensors supply
device memory and the current HIP stream; every step of the computation runs
in the library's HIP kernels. There is no CPU fallback: a missing library
raises ``RuntimeError``.

    import decode_token_sampling_amd as vs
    ws = vs.workspace(B, V, torch.float32)
    status = vs.penalize(logits, prompt_ids=..., prompt_off=..., repetition=...)
    out = vs.sample(logits, temperature=T, top_k=k, top_p=p, min_p=mp, seeds=seeds, ws=ws)
    lp = vs.logprobs(logits, token_ids=out["ids"], k=20, ws=ws)
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LIB_PATH", "VsError", "load", "workspace_size", "workspace", "penalize", "sample",
    "logprobs", "sample_logprobs", "ROW_BAD_PARAM", "ROW_BAD_LOGITS", "ROW_BAD_TOKEN_ID", "ROW_TOPK_UNSUPPORTED",
    "ROW_HINT_VIOLATED", "HINT_NONE", "HINT_NO_FULLVOCAB", "HINT_ALL_GREEDY", "HINT_NO_GREEDY",
    "HINT_SMALL_TOPK",
    "OPT_TOPP_REJECTION", "OPT_TOPP_GATHER_DRAW", "OPT_TOPP_KEPT_PASS", "MAX_V",
    "TOPK_MAX", "LOGPROB_K_MAX", "EXPORTED_SYMBOLS", "hints_for", "sample_logprobs_noalloc",
    "NOALLOC_SCRATCH_BYTES", "penalize_sample_logprobs",
]

# the in-tree build; VS_LIBRARY names another build of the same library (a
# host-sanitised one, say)
LIB_PATH = os.environ.get("VS_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                        "libvs.so")

ROW_BAD_PARAM = 1
ROW_BAD_LOGITS = 2
ROW_BAD_TOKEN_ID = 4
ROW_TOPK_UNSUPPORTED = 8
ROW_HINT_VIOLATED = 16
HINT_NONE = 0
HINT_NO_FULLVOCAB = 1
HINT_ALL_GREEDY = 2
HINT_NO_GREEDY = 4
HINT_SMALL_TOPK = 8
OPT_TOPP_REJECTION = 256
OPT_TOPP_GATHER_DRAW = 512
OPT_TOPP_KEPT_PASS = 1024
MAX_V = 1 << 21
TOPK_MAX = 1024
LOGPROB_K_MAX = 64
NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTED_SYMBOLS = ("vs_workspace_size", "vs_status_string", "vs_penalize", "vs_penalize_ex",
                    "vs_sample", "vs_logprobs", "vs_logprobs_ex", "vs_sample_logprobs", "vs_topp_decay",
                    "vs_seed_advance", "vs_slot_remap", "vs_profile_begin", "vs_profile_end",
                    "vs_sample_logprobs_noalloc", "vs_penalize_sample_logprobs")

_STATUS = {0: "ok", 1: "invalid argument", 2: "workspace too small", 3: "unsupported",
           4: "HIP launch failure"}
_lib = None


class VsError(RuntimeError):
    def __init__(self, call: str, code: int):
        super().__init__(f"{call}: {_STATUS.get(code, code)} (status {code})")
        self.code = code


def load() -> ctypes.CDLL:
    """Load libvs.so (raises RuntimeError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m decode_token_sampling_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, u32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
    lib.vs_workspace_size.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
    lib.vs_status_string.argtypes = [i32]
    lib.vs_status_string.restype = ctypes.c_char_p
    lib.vs_penalize.argtypes = [P, i32, i32, i32, i64, P, P, P, P, P, P, P, P, P]
    lib.vs_penalize_ex.argtypes = [P, i32, i32, i32, i64, P, P, P, P, P, P, P, P, P, P]
    lib.vs_topp_decay.argtypes = [i32, P, P, P, P, P, P, P, P]
    lib.vs_seed_advance.argtypes = [i32, P, P, P]
    lib.vs_slot_remap.argtypes = [i32, i32, P, P, P, i32, P, P]
    lib.vs_sample.argtypes = [P, i32, i32, i32, i64, P, P, P, P, P, u32, P, P, P, P, P, sz, P]
    lib.vs_logprobs.argtypes = [P, i32, i32, i32, i64, P, P, i32, P, P, P, i64, P, P, sz, P]
    lib.vs_logprobs_ex.argtypes = [P, i32, i32, i32, i64, P, P, P, i32, P, P, P, i64, P, P, sz, P]
    lib.vs_sample_logprobs.argtypes = [P, i32, i32, i32, i64, P, P, P, P, P, u32, P, P, P, P, P,
                                       i32, P, P, P, i64, P, sz, P]
    lib.vs_sample_logprobs_noalloc.argtypes = [P, i32, i32, i32, i64, P, P, P, P, P, u32, P, P, P,
                                               P, P, i32, P, P, P, i64, P]
    lib.vs_penalize_sample_logprobs.argtypes = [P, i32, i32, i32, i64, P, P, P, P, P, P, P, P, P,
                                                P, P, P, P, P, u32, P, P, P, P, P, i32, P, P, P,
                                                i64, P, sz, P]
    lib.vs_profile_begin.argtypes = [P, i32]
    lib.vs_profile_end.argtypes = [ctypes.POINTER(ctypes.c_char_p), i32]
    for f in ("vs_workspace_size", "vs_penalize", "vs_penalize_ex", "vs_topp_decay",
              "vs_seed_advance", "vs_slot_remap", "vs_sample", "vs_logprobs", "vs_logprobs_ex",
              "vs_sample_logprobs", "vs_sample_logprobs_noalloc", "vs_penalize_sample_logprobs",
              "vs_profile_begin", "vs_profile_end"):
        getattr(lib, f).restype = i32
    _lib = lib
    return lib


def hints_for(temperature, top_k, top_p, min_p, V: int) -> int:
    """The strongest VS_HINT_* promise that a batch's parameters (host arrays,
    one entry per row; None means the call's default for every row) support:
    every row greedy; every row greedy or 1 < top_k <= 64; every row greedy or
    0 < top_k < V; else none. Host bookkeeping only: it reads no logits."""
    import numpy as np

    def arr(a, default, dt):
        return np.full(1, default, dt) if a is None else np.asarray(a, dt)

    T = arr(temperature, 1.0, np.float32)
    k = arr(top_k, 0, np.int64)
    p = arr(top_p, 1.0, np.float32)
    mp = arr(min_p, 0.0, np.float32)
    greedy = (T == 0) | (k == 1) | (p == 0) | (mp == 1)
    if bool(greedy.all()):
        return HINT_ALL_GREEDY
    if bool((greedy | ((k > 1) & (k <= 64) & (k < V))).all()):
        return HINT_SMALL_TOPK
    if bool((greedy | ((k > 0) & (k < V))).all()):
        return HINT_NO_FULLVOCAB
    return HINT_NONE


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return 0
    if t.dtype == torch.bfloat16:
        return 1
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _ptr(t, dtype=None, n=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if n is not None and t.numel() < n:
        raise ValueError(f"{name} needs at least {n} elements")
    return t.data_ptr()


def _logits_args(logits: torch.Tensor, V):
    if logits.dim() != 2 or not logits.is_cuda:
        raise ValueError("logits must be a 2-D device tensor [B, ld]")
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    B = logits.shape[0]
    V = logits.shape[1] if V is None else int(V)
    return B, V, logits.stride(0) if B > 1 else max(logits.shape[1], 1)


def _stream(stream):
    return (stream or torch.cuda.current_stream(torch.cuda.current_device())).cuda_stream


def workspace_size(B: int, V: int, dtype: torch.dtype = torch.float32) -> int:
    out = ctypes.c_size_t(0)
    code = load().vs_workspace_size(int(B), int(V), 0 if dtype == torch.float32 else 1,
                                    ctypes.byref(out))
    if code:
        raise VsError("vs_workspace_size", code)
    return out.value


def workspace(B: int, V: int, dtype: torch.dtype = torch.float32, device=None) -> torch.Tensor:
    """Device workspace for vs_sample / vs_logprobs (uint8 tensor)."""
    return torch.empty(workspace_size(B, V, dtype), dtype=torch.uint8, device=device or "cuda")


def penalize(logits, prompt_ids=None, prompt_off=None, output_ids=None, output_off=None,
             presence=None, frequency=None, repetition=None, V=None, row_status=None,
             stream=None, prompt_ignore=None) -> torch.Tensor:
    """Occurrence penalties in place (vs_penalize, or vs_penalize_ex with a per-row
    prompt_ignore_length tensor). Returns the per-row status tensor."""
    B, V, ld = _logits_args(logits, V)
    st = row_status if row_status is not None else torch.empty(B, dtype=torch.int32,
                                                                device=logits.device)
    args = [logits.data_ptr(), _dtype_code(logits), B, V, ld,
            _ptr(prompt_ids, torch.int32, name="prompt_ids"), _ptr(prompt_off, torch.int32, B + 1, "prompt_off"),
            _ptr(output_ids, torch.int32, name="output_ids"), _ptr(output_off, torch.int32, B + 1, "output_off"),
            _ptr(presence, torch.float32, B, "presence"), _ptr(frequency, torch.float32, B, "frequency"),
            _ptr(repetition, torch.float32, B, "repetition")]
    tail = [_ptr(st, torch.int32, B, "row_status"), _stream(stream)]
    if prompt_ignore is None:
        name, code = "vs_penalize", load().vs_penalize(*args, *tail)
    else:
        name = "vs_penalize_ex"
        code = load().vs_penalize_ex(*args, _ptr(prompt_ignore, torch.int32, B, "prompt_ignore"), *tail)
    if code:
        raise VsError(name, code)
    return st


def topp_decay(top_p, top_p_init, decay, sampled_ids, top_p_min=None, reset_ids=None,
               row_status=None, stream=None) -> torch.Tensor:
    """Top-p decay after one sampled token, in place on the fp32 state tensor
    top_p (vs_topp_decay). Returns the per-row status tensor."""
    B = top_p.shape[0]
    st = row_status if row_status is not None else torch.empty(B, dtype=torch.int32,
                                                                device=top_p.device)
    code = load().vs_topp_decay(
        B, _ptr(top_p, torch.float32, B, "top_p"), _ptr(top_p_init, torch.float32, B, "top_p_init"),
        _ptr(decay, torch.float32, B, "decay"), _ptr(top_p_min, torch.float32, B, "top_p_min"),
        _ptr(reset_ids, torch.int32, B, "reset_ids"), _ptr(sampled_ids, torch.int32, B, "sampled_ids"),
        _ptr(st, torch.int32, B, "row_status"), _stream(stream))
    if code:
        raise VsError("vs_topp_decay", code)
    return st


def seed_advance(seeds, sampled_ids=None, stream=None) -> None:
    """One new seed per row per sampled token, in place on the int64 (uint64
    bits) seed tensor (vs_seed_advance)."""
    B = seeds.shape[0]
    code = load().vs_seed_advance(B, _ptr(seeds, torch.int64, B, "seeds"),
                                  _ptr(sampled_ids, torch.int32, B, "sampled_ids"), _stream(stream))
    if code:
        raise VsError("vs_seed_advance", code)


def slot_remap(slot_remap, src, dst, row_status=None, stream=None) -> torch.Tensor:
    """New slot i takes src[slot_remap[i]] into dst[i] (vs_slot_remap); src and dst
    are 4- or 8-byte per-row tensors. Returns the per-row status tensor."""
    B, B_src = slot_remap.shape[0], src.shape[0]
    if src.element_size() != dst.element_size() or src.element_size() not in (4, 8):
        raise TypeError("src and dst must hold 4- or 8-byte elements of one size")
    st = row_status if row_status is not None else torch.empty(B, dtype=torch.int32,
                                                                device=dst.device)
    code = load().vs_slot_remap(B, B_src, _ptr(slot_remap, torch.int32, B, "slot_remap"),
                                _ptr(src, src.dtype, B_src, "src"), _ptr(dst, dst.dtype, B, "dst"),
                                src.element_size(), _ptr(st, torch.int32, B, "row_status"),
                                _stream(stream))
    if code:
        raise VsError("vs_slot_remap", code)
    return st


def sample(logits, temperature=None, top_k=None, top_p=None, min_p=None, seeds=None, hints=0,
           V=None, ws=None, out_ids=None, kept=None, mask=False, row_status=None,
           stream=None) -> dict:
    """One token per row (vs_sample). Returns dict(ids, kept, status[, mask])."""
    B, V, ld = _logits_args(logits, V)
    dev = logits.device
    if ws is None:
        ws = workspace(B, V, logits.dtype, dev)
    ids = out_ids if out_ids is not None else torch.empty(B, dtype=torch.int32, device=dev)
    kc = kept if kept is not None else torch.empty(B, dtype=torch.int32, device=dev)
    st = row_status if row_status is not None else torch.empty(B, dtype=torch.int32, device=dev)
    mk = None
    if mask is True:
        mk = torch.empty((B, (V + 31) // 32), dtype=torch.int32, device=dev)
    elif isinstance(mask, torch.Tensor):
        mk = mask
    code = load().vs_sample(
        logits.data_ptr(), _dtype_code(logits), B, V, ld,
        _ptr(temperature, torch.float32, B, "temperature"), _ptr(top_k, torch.int32, B, "top_k"),
        _ptr(top_p, torch.float32, B, "top_p"), _ptr(min_p, torch.float32, B, "min_p"),
        _ptr(seeds, torch.int64, B, "seeds"), int(hints), _ptr(ids, torch.int32, B, "out_ids"),
        _ptr(kc, torch.int32, B, "kept"), _ptr(mk, torch.int32, name="mask"),
        _ptr(st, torch.int32, B, "row_status"), _ptr(ws, torch.uint8, name="ws"), ws.numel(),
        _stream(stream))
    if code:
        raise VsError("vs_sample", code)
    out = dict(ids=ids, kept=kc, status=st)
    if mk is not None:
        out["mask"] = mk
    return out


def logprobs(logits, token_ids=None, k=0, full=False, V=None, ws=None, out_full=None,
             row_status=None, stream=None, temperature=None) -> dict:
    """Log-softmax log-probs (vs_logprobs; vs_logprobs_ex at a per-row temperature when
    one is given). Returns dict(token_lp, topk_ids, topk_lp, full, status)."""
    B, V, ld = _logits_args(logits, V)
    dev = logits.device
    if ws is None:
        ws = workspace(B, V, logits.dtype, dev)
    tlp = torch.empty(B, dtype=torch.float32, device=dev) if token_ids is not None else None
    tids = torch.empty((B, k), dtype=torch.int32, device=dev) if k > 0 else None
    tlps = torch.empty((B, k), dtype=torch.float32, device=dev) if k > 0 else None
    fo = out_full
    if full and fo is None:
        fo = torch.empty((B, V), dtype=torch.float32, device=dev)
    ld_out = fo.stride(0) if fo is not None else 0
    st = row_status if row_status is not None else torch.empty(B, dtype=torch.int32, device=dev)
    head = [logits.data_ptr(), _dtype_code(logits), B, V, ld]
    tail = [_ptr(token_ids, torch.int32, B, "token_ids"), _ptr(tlp, torch.float32, B, "token_lp"),
            int(k), _ptr(tids, torch.int32, name="topk_ids"), _ptr(tlps, torch.float32, name="topk_lp"),
            fo.data_ptr() if fo is not None else None, ld_out, _ptr(st, torch.int32, B, "row_status"),
            _ptr(ws, torch.uint8, name="ws"), ws.numel(), _stream(stream)]
    if temperature is None:
        name, code = "vs_logprobs", load().vs_logprobs(*head, *tail)
    else:
        name = "vs_logprobs_ex"
        code = load().vs_logprobs_ex(*head, _ptr(temperature, torch.float32, B, "temperature"), *tail)
    if code:
        raise VsError(name, code)
    return dict(token_lp=tlp, topk_ids=tids, topk_lp=tlps, full=fo, status=st)


def sample_logprobs(logits, temperature=None, top_k=None, top_p=None, min_p=None, seeds=None,
                    hints=0, k=0, token_logprob=True, full=False, V=None, ws=None, out_ids=None,
                    kept=None, mask=False, row_status=None, out_token_lp=None, out_topk_ids=None,
                    out_topk_lp=None, out_full=None, stream=None) -> dict:
    """vs_sample and the log-probs of the sampled ids (and top-k) in one pass over the
    logits (vs_sample_logprobs). Returns dict(ids, kept, status, token_lp, topk_ids,
    topk_lp, full[, mask])."""
    return _sample_logprobs(False, logits, temperature, top_k, top_p, min_p, seeds, hints, k,
                            token_logprob, full, V, ws, out_ids, kept, mask, row_status,
                            out_token_lp, out_topk_ids, out_topk_lp, out_full, stream)


def sample_logprobs_noalloc(logits, temperature=None, top_k=None, top_p=None, min_p=None,
                            seeds=None, hints=0, k=0, token_logprob=True, full=False, V=None,
                            out_ids=None, kept=None, mask=False, row_status=None,
                            out_token_lp=None, out_topk_ids=None, out_topk_lp=None,
                            out_full=None, stream=None) -> dict:
    """sample_logprobs through vs_sample_logprobs_noalloc: no workspace, the
    library's per-device scratch instead (the library allocates nothing; calls
    on one device must not overlap). Outputs the caller does not pass are
    still allocated here, by torch."""
    return _sample_logprobs(True, logits, temperature, top_k, top_p, min_p, seeds, hints, k,
                            token_logprob, full, V, None, out_ids, kept, mask, row_status,
                            out_token_lp, out_topk_ids, out_topk_lp, out_full, stream)


def penalize_sample_logprobs(logits, prompt_ids=None, prompt_off=None, output_ids=None,
                             output_off=None, presence=None, frequency=None, repetition=None,
                             prompt_ignore=None, penalty_status=None, temperature=None, top_k=None,
                             top_p=None, min_p=None, seeds=None, hints=0, k=0, token_logprob=True,
                             full=False, V=None, ws=None, out_ids=None, kept=None, mask=False,
                             row_status=None, out_token_lp=None, out_topk_ids=None,
                             out_topk_lp=None, out_full=None, stream=None) -> dict:
    """Occurrence penalties in place and sample_logprobs in one call
    (vs_penalize_sample_logprobs): the streaming pass penalises each segment's
    history ids before reading it. Returns sample_logprobs' dict plus
    penalty_status."""
    B = logits.shape[0]
    pst = penalty_status if penalty_status is not None else torch.empty(
        B, dtype=torch.int32, device=logits.device)
    pen = [_ptr(prompt_ids, torch.int32, name="prompt_ids"),
           _ptr(prompt_off, torch.int32, B + 1, "prompt_off"),
           _ptr(output_ids, torch.int32, name="output_ids"),
           _ptr(output_off, torch.int32, B + 1, "output_off"),
           _ptr(presence, torch.float32, B, "presence"), _ptr(frequency, torch.float32, B, "frequency"),
           _ptr(repetition, torch.float32, B, "repetition"),
           _ptr(prompt_ignore, torch.int32, B, "prompt_ignore"), _ptr(pst, torch.int32, B, "penalty_status")]
    out = _sample_logprobs(False, logits, temperature, top_k, top_p, min_p, seeds, hints, k,
                           token_logprob, full, V, ws, out_ids, kept, mask, row_status,
                           out_token_lp, out_topk_ids, out_topk_lp, out_full, stream, pen=pen)
    out["penalty_status"] = pst
    return out


def _sample_logprobs(noalloc, logits, temperature, top_k, top_p, min_p, seeds, hints, k,
                     token_logprob, full, V, ws, out_ids, kept, mask, row_status, out_token_lp,
                     out_topk_ids, out_topk_lp, out_full, stream, pen=None) -> dict:
    B, V, ld = _logits_args(logits, V)
    dev = logits.device
    if ws is None and not noalloc:
        ws = workspace(B, V, logits.dtype, dev)
    ids = out_ids if out_ids is not None else torch.empty(B, dtype=torch.int32, device=dev)
    kc = kept if kept is not None else torch.empty(B, dtype=torch.int32, device=dev)
    st = row_status if row_status is not None else torch.empty(B, dtype=torch.int32, device=dev)
    tlp = out_token_lp
    if token_logprob and tlp is None:
        tlp = torch.empty(B, dtype=torch.float32, device=dev)
    tids = out_topk_ids if out_topk_ids is not None else (
        torch.empty((B, k), dtype=torch.int32, device=dev) if k > 0 else None)
    tlps = out_topk_lp if out_topk_lp is not None else (
        torch.empty((B, k), dtype=torch.float32, device=dev) if k > 0 else None)
    fo = out_full
    if full and fo is None:
        fo = torch.empty((B, V), dtype=torch.float32, device=dev)
    mk = None
    if mask is True:
        mk = torch.empty((B, (V + 31) // 32), dtype=torch.int32, device=dev)
    elif isinstance(mask, torch.Tensor):
        mk = mask
    args = [logits.data_ptr(), _dtype_code(logits), B, V, ld,
            _ptr(temperature, torch.float32, B, "temperature"), _ptr(top_k, torch.int32, B, "top_k"),
            _ptr(top_p, torch.float32, B, "top_p"), _ptr(min_p, torch.float32, B, "min_p"),
            _ptr(seeds, torch.int64, B, "seeds"), int(hints), _ptr(ids, torch.int32, B, "out_ids"),
            _ptr(kc, torch.int32, B, "kept"), _ptr(mk, torch.int32, name="mask"),
            _ptr(st, torch.int32, B, "row_status"), _ptr(tlp, torch.float32, B, "token_lp"), int(k),
            _ptr(tids, torch.int32, name="topk_ids"), _ptr(tlps, torch.float32, name="topk_lp"),
            fo.data_ptr() if fo is not None else None, fo.stride(0) if fo is not None else 0]
    if pen is not None:
        name = "vs_penalize_sample_logprobs"
        code = load().vs_penalize_sample_logprobs(*args[:5], *pen, *args[5:],
                                                  _ptr(ws, torch.uint8, name="ws"), ws.numel(),
                                                  _stream(stream))
    elif noalloc:
        name = "vs_sample_logprobs_noalloc"
        code = load().vs_sample_logprobs_noalloc(*args, _stream(stream))
    else:
        name = "vs_sample_logprobs"
        code = load().vs_sample_logprobs(*args, _ptr(ws, torch.uint8, name="ws"), ws.numel(),
                                         _stream(stream))
    if code:
        raise VsError(name, code)
    out = dict(ids=ids, kept=kc, status=st, token_lp=tlp, topk_ids=tids, topk_lp=tlps, full=fo)
    if mk is not None:
        out["mask"] = mk
    return out
