"""GPU parity on the five benchmark workloads at full size, against the oracle.

Each workload runs the call bench.py times (one vs_sample_logprobs call with
the hint its parameters support, the log-prob outputs the workload asks for
and no kept mask; for the penalised workloads vs_penalize_sample_logprobs,
and vs_penalize then vs_sample_logprobs as the separate path bench.py times
beside it), and every row of every output is compared: penalised logits and
row status bit-exact, ids and kept counts bit-exact, sampled-id and top-k
log-probs within 1e-5, the full log-softmax within 1e-5 on every fourth row
and normalised on every row. The same logits then go through the path that
writes kept masks (the row kernels), whose kept sets must equal the oracle's
bit for bit. Near-tie rows (two best Gumbel scores within 1e-6 relative) would
be exempt from the id check; the oracle finds none on these workloads, and
the tests require that count to be 0, so the id check covers every row.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import LOGPROB_ATOL, compare_sample, dev, from_device, gpu_sample, oracle_sample, \
    params_from, to_device

pytestmark = pytest.mark.gpu

WORKLOADS = ["w4x32000_f32", "w32x151936_bf16", "w256x248320_f32", "w1024x128256_f32",
             "w64x262144_bf16"]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_token_sampling_amd as vs
    vs.load()
    oracle.build(force=False)


@functools.lru_cache(maxsize=None)
def _oracle(name):
    """The oracle's step on one workload: penalised logits and their status,
    the draw with kept masks, and the log-probs of its sampled ids (the full
    log-softmax on every fourth row when the workload asks for it)."""
    wl = synth.make(name)
    x = wl.logits
    pst = None
    if wl.has_penalties:
        x = x.copy()
        pst = oracle.penalize(x, wl.V, wl.prompt_ids, wl.prompt_off, wl.output_ids,
                              wl.output_off, wl.presence, wl.frequency, wl.repetition)
    o = oracle_sample(x, wl.V, params_from(wl), mask=True)
    assert (o["status"] == 0).all()
    lp = oracle.logprobs(x, wl.V, o["ids"], k=wl.logprob_k)
    full_rows = np.arange(0, wl.B, 4)
    full = None
    if wl.full_logprobs:
        full = oracle.logprobs(np.ascontiguousarray(x[full_rows]), wl.V, k=0, full=True)["full"]
    return wl, x, pst, o, lp, full_rows, full


def _penalised_device(wl, x_oracle, pst):
    """The workload's logits on the device with vs_penalize applied, checked
    against the oracle's penalised logits and status."""
    import decode_token_sampling_amd as vs
    xd = to_device(wl.logits)
    if wl.has_penalties:
        st = vs.penalize(xd, dev(wl.prompt_ids, np.int32), dev(wl.prompt_off, np.int32),
                         dev(wl.output_ids, np.int32), dev(wl.output_off, np.int32),
                         dev(wl.presence, np.float32), dev(wl.frequency, np.float32),
                         dev(wl.repetition, np.float32)).cpu().numpy()
        assert np.array_equal(st, pst)
        assert np.array_equal(from_device(xd, wl.V).view(np.uint8), x_oracle.view(np.uint8))
    return xd


def _check_lp(got, want):
    got = got.cpu().numpy()
    assert got.shape == want.shape
    assert np.isfinite(got).all() and np.isfinite(want).all()
    err = np.abs(got - want).max()
    assert err <= LOGPROB_ATOL, err


@pytest.mark.parametrize("name", WORKLOADS)
def test_workload_benched_call(name):
    """The call bench.py times (for penalised workloads, its separate-launch
    variant), every row of every output against the oracle."""
    import decode_token_sampling_amd as vs
    wl, x, pst, o, lp, full_rows, full = _oracle(name)
    xd = _penalised_device(wl, x, pst)
    w = params_from(wl)
    hints = vs.hints_for(wl.temperature, wl.top_k, wl.top_p, wl.min_p, wl.V)
    out = vs.sample_logprobs(xd, dev(w["temperature"], np.float32), dev(w["top_k"], np.int32),
                             dev(w["top_p"], np.float32), dev(w["min_p"], np.float32),
                             dev(np.asarray(w["seeds"], np.uint64).view(np.int64), np.int64),
                             hints=hints, k=wl.logprob_k, token_logprob=not wl.full_logprobs,
                             full=wl.full_logprobs)
    torch.cuda.synchronize()
    g = dict(ids=out["ids"].cpu().numpy(), kept=out["kept"].cpu().numpy(),
             status=out["status"].cpu().numpy())
    near = compare_sample(g, o, check_mask=False)
    assert near == 0, f"{name}: {near} near-tie rows (the oracle finds none)"
    if not wl.full_logprobs:
        _check_lp(out["token_lp"], lp["token_lp"])
    if wl.logprob_k:
        assert np.array_equal(out["topk_ids"].cpu().numpy(), lp["topk_ids"])
        _check_lp(out["topk_lp"], lp["topk_lp"])
    if wl.full_logprobs:
        _check_lp(out["full"][torch.from_numpy(full_rows).cuda()], full)
        s = torch.logsumexp(out["full"].double(), dim=1).cpu().numpy()
        assert np.abs(s).max() < 1e-5
    if name == "w1024x128256_f32":
        assert np.array_equal(g["ids"], np.argmax(wl.logits, axis=1))  # greedy: first maximum


@pytest.mark.parametrize("name", WORKLOADS)
def test_workload_kept_sets(name):
    """The same draw with kept masks (and no hint): every row's kept set."""
    wl, x, pst, o, lp, full_rows, full = _oracle(name)
    xd = _penalised_device(wl, x, pst)
    g = gpu_sample(xd, wl.V, params_from(wl), mask=True)
    assert compare_sample(g, o) == 0


@pytest.mark.parametrize("name", ["w256x248320_f32", "w1024x128256_f32"])
def test_workload_separate_calls(name):
    """vs_sample then vs_logprobs on the sampled ids (two reads of the logits)."""
    import decode_token_sampling_amd as vs
    wl, x, pst, o, lp, full_rows, full = _oracle(name)
    xd = to_device(wl.logits)
    g = gpu_sample(xd, wl.V, params_from(wl), mask=False)
    assert compare_sample(g, o, check_mask=False) == 0
    out = vs.logprobs(xd, dev(g["ids"], np.int32), k=wl.logprob_k, full=wl.full_logprobs)
    torch.cuda.synchronize()
    _check_lp(out["token_lp"], lp["token_lp"])
    assert np.array_equal(out["topk_ids"].cpu().numpy(), lp["topk_ids"])
    _check_lp(out["topk_lp"], lp["topk_lp"])
    if wl.full_logprobs:
        _check_lp(out["full"][torch.from_numpy(full_rows).cuda()], full)


@pytest.mark.parametrize("name", ["w32x151936_bf16", "w64x262144_bf16"])
def test_workload_fused_penalties(name):
    """The penalised workloads through vs_penalize_sample_logprobs (the
    penalties applied by the streaming pass, the call bench.py times for
    them): penalised logits, penalty status, ids, kept counts and sampled-id
    log-probs of every row against the oracle."""
    import decode_token_sampling_amd as vs
    wl, x, pst, o, lp, full_rows, full = _oracle(name)
    xd = to_device(wl.logits)
    w = params_from(wl)
    hints = vs.hints_for(wl.temperature, wl.top_k, wl.top_p, wl.min_p, wl.V)
    out = vs.penalize_sample_logprobs(
        xd, dev(wl.prompt_ids, np.int32), dev(wl.prompt_off, np.int32), dev(wl.output_ids, np.int32),
        dev(wl.output_off, np.int32), dev(wl.presence, np.float32), dev(wl.frequency, np.float32),
        dev(wl.repetition, np.float32), temperature=dev(w["temperature"], np.float32),
        top_k=dev(w["top_k"], np.int32), top_p=dev(w["top_p"], np.float32),
        min_p=dev(w["min_p"], np.float32),
        seeds=dev(np.asarray(w["seeds"], np.uint64).view(np.int64), np.int64), hints=hints,
        k=wl.logprob_k)
    torch.cuda.synchronize()
    assert np.array_equal(out["penalty_status"].cpu().numpy(), pst)
    assert np.array_equal(from_device(xd, wl.V).view(np.uint8), x.view(np.uint8))
    g = dict(ids=out["ids"].cpu().numpy(), kept=out["kept"].cpu().numpy(),
             status=out["status"].cpu().numpy())
    assert compare_sample(g, o, check_mask=False) == 0
    _check_lp(out["token_lp"], lp["token_lp"])


@pytest.mark.parametrize("method", ["rejection", "gather", "kept_pass"])
@pytest.mark.parametrize("name", ["w4x32000_f32", "w32x151936_bf16", "w64x262144_bf16"])
def test_workload_topp_methods(name, method):
    """The workloads with full-vocabulary top-p rows through each method for
    them (VS_OPT_TOPP_REJECTION, VS_OPT_TOPP_GATHER_DRAW, VS_OPT_TOPP_KEPT_PASS;
    the benchmarked call takes the default): ids, kept counts and sampled-id
    log-probs of every row against the oracle."""
    import decode_token_sampling_amd as vs
    wl, x, pst, o, lp, full_rows, full = _oracle(name)
    xd = _penalised_device(wl, x, pst)
    w = params_from(wl)
    h = {"rejection": vs.OPT_TOPP_REJECTION, "gather": vs.OPT_TOPP_GATHER_DRAW,
         "kept_pass": vs.OPT_TOPP_KEPT_PASS}[method]
    out = vs.sample_logprobs(xd, dev(w["temperature"], np.float32), dev(w["top_k"], np.int32),
                             dev(w["top_p"], np.float32), dev(w["min_p"], np.float32),
                             dev(np.asarray(w["seeds"], np.uint64).view(np.int64), np.int64),
                             hints=h, k=wl.logprob_k)
    torch.cuda.synchronize()
    g = dict(ids=out["ids"].cpu().numpy(), kept=out["kept"].cpu().numpy(),
             status=out["status"].cpu().numpy())
    assert compare_sample(g, o, check_mask=False) == 0
    _check_lp(out["token_lp"], lp["token_lp"])
