"""CPU checks of the boundary: libvs.so loads and exports every call that
include/vs.h declares; host-side argument checks return errors without a GPU
call; the binding refuses host tensors."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "vs.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^(?:vs_status|const char\*|int)\s+(vs_\w+)\(", text, re.M)))


def test_header_declares_the_boundary():
    assert _declared() == sorted(["vs_workspace_size", "vs_status_string", "vs_penalize",
                                  "vs_penalize_ex", "vs_sample", "vs_logprobs", "vs_logprobs_ex",
                                  "vs_sample_logprobs", "vs_sample_logprobs_noalloc",
                                  "vs_penalize_sample_logprobs",
                                  "vs_topp_decay", "vs_seed_advance", "vs_slot_remap",
                                  "vs_profile_begin", "vs_profile_end"])


def test_library_exports_every_declared_symbol():
    import decode_token_sampling_amd as vs
    lib = vs.load()
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(_declared()) == set(vs.EXPORTED_SYMBOLS)


def test_host_checks_without_gpu():
    import decode_token_sampling_amd as vs
    lib = vs.load()
    n = ctypes.c_size_t(0)
    assert lib.vs_workspace_size(256, 248320, 0, ctypes.byref(n)) == 0 and n.value > 0
    assert lib.vs_workspace_size(0, 10, 0, ctypes.byref(n)) == 1
    assert lib.vs_workspace_size(4, vs.MAX_V + 1, 0, ctypes.byref(n)) == 1
    assert lib.vs_workspace_size(4, 10, 7, ctypes.byref(n)) == 1
    assert lib.vs_status_string(2) == b"workspace too small"
    # null logits / bad sizes are rejected before any launch
    assert lib.vs_sample(None, 0, 4, 10, 10, *([None] * 5), 0, None, None, None, None,
                         None, 0, None) == 1
    assert lib.vs_penalize(None, 0, 4, 10, 10, *([None] * 9)) == 1
    assert lib.vs_penalize_ex(None, 0, 4, 10, 10, *([None] * 10)) == 1
    assert lib.vs_topp_decay(0, *([None] * 8)) == 1
    assert lib.vs_topp_decay(4, None, *([None] * 7)) == 1
    assert lib.vs_seed_advance(4, None, None, None) == 1
    assert lib.vs_slot_remap(4, 4, None, None, None, 4, None, None) == 1
    p16, p32 = ctypes.c_void_p(16), ctypes.c_void_p(32)  # never dereferenced
    assert lib.vs_slot_remap(4, 4, p16, p16, p16, 4, None, None) == 1   # src == dst
    assert lib.vs_slot_remap(4, 4, p16, p16, p32, 2, None, None) == 1   # 2-byte elements
    assert lib.vs_logprobs(None, 0, 4, 10, 10, None, None, 0, None, None, None, 0, None,
                           None, 0, None) == 1
    assert lib.vs_logprobs_ex(None, 0, 4, 10, 10, None, None, None, 0, None, None, None, 0,
                              None, None, 0, None) == 1
    dummy = ctypes.c_void_p(16)  # never dereferenced: the checks fail first
    assert lib.vs_sample(dummy, 0, 4, 10, 9, *([None] * 5), 0, dummy, None, None, None,
                         dummy, 1 << 30, None) == 1          # ld < V
    assert lib.vs_sample(dummy, 0, 4, 10, 10, *([None] * 5), 0, dummy, None, None, None,
                         dummy, 8, None) == 2                # workspace too small
    assert lib.vs_logprobs(dummy, 0, 4, 10, 10, None, None, 65, dummy, dummy, None, 0, None,
                           dummy, 1 << 30, None) == 1        # k > 64
    assert lib.vs_sample(dummy, 0, 4, 10, 10, *([None] * 5), 16, dummy, None, None, None,
                         dummy, 1 << 30, None) == 1          # unknown hint bit


def test_fused_penalty_host_checks_without_gpu():
    import decode_token_sampling_amd as vs
    lib = vs.load()
    d = ctypes.c_void_p(16)  # never dereferenced: the checks fail first
    # a prompt id array without its offsets
    assert lib.vs_penalize_sample_logprobs(d, 0, 4, 10, 10, d, None, None, None, None, None, None,
                                           None, None, *([None] * 5), 0, d, None, None, None, None,
                                           0, None, None, None, 0, d, 1 << 30, None) == 1
    # workspace too small
    assert lib.vs_penalize_sample_logprobs(d, 0, 4, 10, 10, *([None] * 9), *([None] * 5), 0, d,
                                           None, None, None, None, 0, None, None, None, 0, d, 8,
                                           None) == 2


def test_binding_refuses_host_tensors():
    import torch
    import decode_token_sampling_amd as vs
    with pytest.raises(ValueError):
        vs.sample(torch.zeros(2, 10))


def test_binding_constants_match_the_header():
    """Every VS_HINT_*, VS_OPT_*, VS_ROW_* and size constant the binding
    exports has the header's value (the binding has no other source)."""
    import decode_token_sampling_amd as vs
    with open(os.path.join(ROOT, "include", "vs.h")) as f:
        text = f.read()
    defs = {m[0]: int(m[1]) << int(m[2] or 0)
            for m in re.findall(r"^#define VS_(\w+)\s+\(?(\d+)u?(?:\s*<<\s*(\d+))?", text, re.M)}
    checked = 0
    for name, value in defs.items():
        if hasattr(vs, name):
            assert getattr(vs, name) == value, name
            checked += 1
    assert checked >= 12, checked
    assert defs["HINT_SMALL_TOPK"] == 8 and defs["HINT_NO_GREEDY"] == 4
