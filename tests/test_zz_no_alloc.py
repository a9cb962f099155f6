"""vs_sample_logprobs_noalloc (the library's own scratch, no workspace
argument) against vs_sample_logprobs with a workspace: two calls in a row on
one device, the second on a smaller batch (the scratch keeps the first call's
contents), each compared to the workspace call on the same inputs: ids, kept
counts, kept sets and row status bit-exact, log-probs within 1e-5 (their
summation order is free). A batch too large for the scratch is refused
before anything is enqueued."""
import numpy as np
import pytest
import torch

import synth
from parity import LOGPROB_ATOL, dev, random_params, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_token_sampling_amd as vs
    vs.load()


def _args(w):
    return [dev(w["temperature"], np.float32), dev(w["top_k"], np.int32),
            dev(w["top_p"], np.float32), dev(w["min_p"], np.float32),
            dev(np.asarray(w["seeds"], np.uint64).view(np.int64), np.int64)]


def _same(a, b, full=False):
    for key in ("ids", "kept", "status"):
        assert torch.equal(a[key], b[key]), key
    if "mask" in a:
        assert torch.equal(a["mask"], b["mask"])
    for key in ("token_lp", "topk_lp") + (("full",) if full else ()):
        if a[key] is None:
            continue
        x, y = a[key].cpu().numpy(), b[key].cpu().numpy()
        assert np.array_equal(np.isnan(x), np.isnan(y)), key
        assert np.array_equal(np.isinf(x), np.isinf(y)), key
        fin = np.isfinite(y)
        assert np.array_equal(x[~fin & ~np.isnan(y)], y[~fin & ~np.isnan(y)]), key
        if fin.any():
            assert np.abs(x[fin] - y[fin]).max() <= LOGPROB_ATOL, key
    if "topk_ids" in a and a["topk_ids"] is not None:
        assert torch.equal(a["topk_ids"], b["topk_ids"])


def test_noalloc_matches_workspace_call_twice():
    import decode_token_sampling_amd as vs
    # call 1: the headline batch (256 rows of 248,320 fp32, top-k 20, top-p
    # 0.95, sampled-id and top-20 log-probs), as benchmarked
    wl = synth.make("w256x248320_f32")
    xd = to_device(wl.logits)
    w = dict(temperature=wl.temperature, top_k=wl.top_k, top_p=wl.top_p, min_p=wl.min_p,
             seeds=wl.seeds)
    hints = vs.hints_for(wl.temperature, wl.top_k, wl.top_p, wl.min_p, wl.V)
    a = vs.sample_logprobs_noalloc(xd, *_args(w), hints=hints, k=20)
    b = vs.sample_logprobs(xd, *_args(w), hints=hints, k=20)
    torch.cuda.synchronize()
    _same(a, b)
    assert (a["status"] == 0).all()
    # call 2: a smaller batch through every row mode (greedy, top-k up to 1024,
    # full-vocabulary top-p and min-p), several segments per row, kept masks,
    # top-5 log-probs and the full log-softmax; bf16 and masked ids
    V, B = 70001, 27
    x = synth.random_rows(90, B, V, "bf16", kind="rank")
    x[3, :100] = synth.f32_to_bf16_bits(np.array([-np.inf], np.float32))[0]
    w2 = random_params(np.random.default_rng(91), B, V)
    xd2 = to_device(x)
    a2 = vs.sample_logprobs_noalloc(xd2, *_args(w2), k=5, full=True, mask=True, V=V)
    b2 = vs.sample_logprobs(xd2, *_args(w2), k=5, full=True, mask=True, V=V)
    torch.cuda.synchronize()
    _same(a2, b2, full=True)
    # and once more without masks (rows finished in the streaming pass where
    # they can be), after the masked call left its scratch contents behind
    a3 = vs.sample_logprobs_noalloc(xd2, *_args(w2), k=5, V=V)
    b3 = vs.sample_logprobs(xd2, *_args(w2), k=5, V=V)
    torch.cuda.synchronize()
    _same(a3, b3)


def test_noalloc_refuses_batches_beyond_the_scratch():
    import decode_token_sampling_amd as vs
    lib = vs.load()
    B, V = 1024, 128256   # about 100 MB of scratch: more than the library holds
    x = torch.empty(16, dtype=torch.float32, device="cuda")   # never read: the call refuses first
    ids = torch.empty(16, dtype=torch.int32, device="cuda")
    code = lib.vs_sample_logprobs_noalloc(x.data_ptr(), 0, B, V, V, None, None, None, None, None, 0,
                                          ids.data_ptr(), None, None, None, None, 0, None, None,
                                          None, 0, torch.cuda.current_stream().cuda_stream)
    assert code == 2  # VS_ERR_WORKSPACE_TOO_SMALL, nothing enqueued
    assert lib.vs_status_string(code) == b"workspace too small"
