"""GPU parity: the HIP library, called through the C ABI, against the CPU oracle.

Bar: token ids, kept counts, kept sets and row status bit-exact (ids of rows
whose two best Gumbel scores are within 1e-6 relative are exempt and counted);
penalised logits bit-exact (0 ulp fp32, and the single rounding of bf16);
log-probs within 1e-5 absolute.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import (LOGPROB_ATOL, compare_sample, dev, from_device, gpu_sample, host_pad,
                    mask_bits, oracle_sample, params_from, random_params, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_token_sampling_amd as vs
    vs.load()
    oracle.build(force=False)


# ---------------------------------------------------------------- sampling grid
# Widths around the 4096-id tile edges and the workload widths, several row
# shapes (ties, flat rows, masked -inf ids) and parameters covering every path.
WIDTHS = [1, 2, 7, 63, 64, 100, 1000, 4095, 4096, 4097, 8191, 12345, 32000, 70001, 151936,
          248320]


def _row_shapes(seed, B, V, dtype):
    kinds = ["rank", "ties", "normal", "flat"]
    x = np.concatenate([synth.random_rows(seed + i, (B + 3) // 4, V, dtype, kind=k)
                        for i, k in enumerate(kinds)])[:B]
    x = np.ascontiguousarray(x)
    rng = np.random.default_rng(seed)
    if V > 4:  # masked ids (-inf) on a few rows
        neg = np.float32(-np.inf)
        for r in range(0, B, 5):
            cols = rng.choice(V, V // 3, replace=False)
            if dtype == "bf16":
                x[r, cols] = synth.f32_to_bf16_bits(np.array([neg]))[0]
            else:
                x[r, cols] = neg
    return x


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", WIDTHS)
def test_sample_grid(V, dtype, seed):
    B = 27
    x = _row_shapes(1000 + V + 7919 * seed, B, V, dtype)
    rng = np.random.default_rng(V + 104729 * seed)
    w = random_params(rng, B, V)
    g = gpu_sample(to_device(x), V, w)
    o = oracle_sample(x, V, w)
    assert compare_sample(g, o) <= 1


@pytest.mark.parametrize("seed", range(2))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [100, 4097, 32000, 70001, 151936, 262144])
def test_topp_draw_methods(V, dtype, seed):
    """The three methods for full-vocabulary top-p rows without a kept mask
    (rejection; the gather pass's draw over the ids above the cut bucket plus
    the bucket's kept ids; the Gumbel pass over the kept set): ids, kept
    counts and status equal the oracle's and each other's, on rows of every
    mode; the top-p rows cover tight and loose cuts (p from 0.05 to 0.999)
    with min-p, ties, flat rows and masked ids."""
    import decode_token_sampling_amd as vs
    B = 27
    x = _row_shapes(3100 + V + 31 * seed, B, V, dtype)
    w = random_params(np.random.default_rng(V + 7 * seed), B, V,
                      kinds=["topp", "topp_minp", "topp", "greedy", "kfast", "none", "minp"])
    xd = to_device(x)
    o = oracle_sample(x, V, w, mask=False)
    res = {}
    for name, h in (("rejection", vs.OPT_TOPP_REJECTION), ("gather", vs.OPT_TOPP_GATHER_DRAW),
                    ("kept_pass", vs.OPT_TOPP_KEPT_PASS), ("default", 0)):
        res[name] = gpu_sample(xd, V, w, hints=h, mask=False)
        assert compare_sample(res[name], o) <= 1, name
    for name in ("rejection", "gather", "default"):
        for key in ("ids", "kept", "status"):
            assert np.array_equal(res[name][key], res["kept_pass"][key]), (name, key)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sample_padded_and_unaligned_rows(dtype):
    V = 5000
    x = _row_shapes(77, 18, V, dtype)
    w = random_params(np.random.default_rng(5), 18, V)
    o = oracle_sample(x, V, w)
    for ld in (V + 1, V + 8, V + 37):  # padding columns hold NaN: never read
        g = gpu_sample(to_device(x, ld=ld), V, w)
        compare_sample(g, o)


def test_sample_seeds_change_draw_and_repeat():
    V, B = 3000, 16
    x = synth.random_rows(3, B, V, kind="flat")
    w = dict(temperature=np.ones(B, np.float32), top_k=np.zeros(B, np.int32),
             top_p=np.ones(B, np.float32), min_p=np.zeros(B, np.float32),
             seeds=np.arange(B, dtype=np.uint64))
    xd = to_device(x)
    a = gpu_sample(xd, V, w)
    b = gpu_sample(xd, V, w)
    assert np.array_equal(a["ids"], b["ids"])
    w2 = dict(w, seeds=np.arange(B, dtype=np.uint64) + 1000)
    c = gpu_sample(xd, V, w2)
    assert (a["ids"] != c["ids"]).sum() > B // 2
    compare_sample(c, oracle_sample(x, V, w2))


@pytest.mark.parametrize("given", ["none", "temperature", "top_k", "top_p", "min_p"])
def test_sample_unset_parameters(given):
    """Parameter arrays left out (NULL): neutral values, and greedy rows when
    temperature, top_k and top_p are all left out; ids, kept counts and kept
    sets against the oracle given the same NULLs."""
    import decode_token_sampling_amd as vs
    V, B = 5000, 12
    x = synth.random_rows(21, B, V, kind="normal")
    vals = dict(temperature=np.full(B, 0.8, np.float32), top_k=np.full(B, 40, np.int32),
                top_p=np.full(B, 0.7, np.float32), min_p=np.full(B, 0.02, np.float32))
    w = {k: (v if k == given else None) for k, v in vals.items()}
    xd = to_device(x)
    out = vs.sample(xd, **{k: (None if v is None else dev(v, v.dtype)) for k, v in w.items()},
                    mask=True, V=V)
    torch.cuda.synchronize()
    g = dict(ids=out["ids"].cpu().numpy(), kept=out["kept"].cpu().numpy(),
             status=out["status"].cpu().numpy(), mask=mask_bits(out["mask"], V))
    o = oracle.sample(x, V, w["temperature"], w["top_k"], w["top_p"], w["min_p"], None, want_mask=True)
    compare_sample(g, o)
    if given in ("none", "min_p"):
        assert (g["kept"] == 1).all() and np.array_equal(g["ids"], np.argmax(x, axis=1))


def test_sample_invalid_rows():
    V, B = 300, 9
    x = synth.random_rows(4, B, V)
    x[1, 7] = np.nan
    x[2, 299] = np.inf
    x[3, :] = -np.inf
    x[8, :] = 3e38
    w = dict(temperature=np.array([1, 1, 1, 1, -1, np.nan, 1, 1, 1e-3], np.float32),
             top_k=np.array([0, 0, 0, 0, 0, 0, -1, 0, 0], np.int32),
             top_p=np.array([1, 1, 1, 1, 1, 1, 1, 1.5, 1], np.float32),
             min_p=np.zeros(B, np.float32), seeds=np.zeros(B, np.uint64))
    g = gpu_sample(to_device(x), V, w)
    o = oracle_sample(x, V, w)
    compare_sample(g, o)
    assert g["status"].tolist() == [0, 2, 2, 2, 1, 1, 1, 1, 1]
    assert (g["ids"][1:] == -1).all()


def test_sample_topk_unsupported_and_k_at_least_v():
    V, B = 3000, 3
    x = synth.random_rows(6, B, V)
    w = dict(temperature=np.ones(B, np.float32), top_k=np.array([1025, 3000, 5000], np.int32),
             top_p=np.full(B, 0.9, np.float32), min_p=np.zeros(B, np.float32),
             seeds=np.zeros(B, np.uint64))
    g = gpu_sample(to_device(x), V, w)
    compare_sample(g, oracle_sample(x, V, w))
    assert g["status"].tolist() == [8, 0, 0]


def test_sample_hints():
    import decode_token_sampling_amd as vs
    V, B = 9000, 12
    x = synth.random_rows(8, B, V)
    w = random_params(np.random.default_rng(1), B, V, kinds=["greedy", "kfast", "kslow", "topp"])
    o = oracle_sample(x, V, w)
    g = gpu_sample(to_device(x), V, w, hints=vs.HINT_NO_FULLVOCAB)
    full = np.arange(B) % 4 == 3
    assert (g["status"][full] == vs.ROW_HINT_VIOLATED).all() and (g["ids"][full] == -1).all()
    compare_sample(g, o, rows=np.nonzero(~full)[0])
    g = gpu_sample(to_device(x), V, w, hints=vs.HINT_ALL_GREEDY)
    greedy = np.arange(B) % 4 == 0
    assert (g["status"][~greedy] == vs.ROW_HINT_VIOLATED).all()
    compare_sample(g, o, rows=np.nonzero(greedy)[0])
    g = gpu_sample(to_device(x), V, w, hints=vs.HINT_NO_GREEDY)
    assert (g["status"][greedy] == vs.ROW_HINT_VIOLATED).all() and (g["ids"][greedy] == -1).all()
    compare_sample(g, o, rows=np.nonzero(~greedy)[0])


def test_sample_heavy_ties_take_exact_path():
    """Rows of a handful of distinct values: tile candidate lists overflow and
    the exact row-level selection decides (ties to the lowest ids)."""
    V, B = 20000, 12
    x = (np.random.default_rng(2).integers(0, 3, (B, V)).astype(np.float32))
    w = dict(temperature=np.ones(B, np.float32),
             top_k=np.array([2, 20, 64, 65, 500, 1024, 0, 0, 0, 7, 33, 0], np.int32),
             top_p=np.array([1, 1, 1, 1, 0.5, 0.9, 0.3, 0.01, 1, 0.7, 0.6, 0.999], np.float32),
             min_p=np.array([0, 0, 0, 0, 0, 0, 0, 0, 0.5, 0, 0, 0.2], np.float32),
             seeds=np.arange(B, dtype=np.uint64))
    compare_sample(gpu_sample(to_device(x), V, w), oracle_sample(x, V, w))


def test_sample_constant_rows_fallback_inside_bucket():
    """Every id in one top-p bucket (> 8192 ids): the mass-weighted radix
    select and tie cut inside the bucket decide."""
    V, B = 50000, 4
    x = np.zeros((B, V), np.float32)
    x[1] = np.float32(0.25) * (np.arange(V) % 2)   # two values
    x[2, ::7] = 1e-6
    w = dict(temperature=np.ones(B, np.float32), top_k=np.zeros(B, np.int32),
             top_p=np.array([0.37, 0.8, 0.5, 0.999], np.float32), min_p=np.zeros(B, np.float32),
             seeds=np.arange(B, dtype=np.uint64))
    xd = to_device(x)
    compare_sample(gpu_sample(xd, V, w), oracle_sample(x, V, w))
    _every_draw_method(xd, x, V, w)


def _every_draw_method(xd, x, V, w):
    """Without a kept mask, each method for full-vocabulary top-p rows against
    the oracle (a cut bucket beyond the list: the gather draw falls back to
    the Gumbel pass over the kept set)."""
    import decode_token_sampling_amd as vs
    o = oracle_sample(x, V, w, mask=False)
    for h in (vs.OPT_TOPP_REJECTION, vs.OPT_TOPP_GATHER_DRAW, vs.OPT_TOPP_KEPT_PASS):
        compare_sample(gpu_sample(xd, V, w, hints=h, mask=False), o)


def test_full_topp_gather_overflows_lds_but_fits_list():
    """A cut bucket of 3000 tied ids inside one gather segment: the segment's
    LDS staging (2048 ids) overflows into direct appends while the row's list
    (<= 8192) still feeds the radix-select cut; ties go to the lowest ids."""
    V, B = 32768, 3
    x = np.full((B, V), -4.0, np.float32)
    x[0, :3000] = 2.0                      # one segment holds the whole bucket
    x[1, 100:3100] = 2.0
    x[1, 5] = 2.5                          # a larger id above the bucket
    x[2, 4096:7096] = 1.0                  # the bucket in the second segment
    w = dict(temperature=np.ones(B, np.float32), top_k=np.zeros(B, np.int32),
             top_p=np.array([0.5, 0.7, 0.3], np.float32), min_p=np.zeros(B, np.float32),
             seeds=np.arange(B, dtype=np.uint64))
    xd = to_device(x)
    compare_sample(gpu_sample(xd, V, w), oracle_sample(x, V, w))
    _every_draw_method(xd, x, V, w)


# ---------------------------------------------------------------- penalties
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_penalize_parity(dtype):
    import decode_token_sampling_amd as vs
    rng = np.random.default_rng(11)
    B, V = 24, 40000
    x = synth.random_rows(12, B, V, dtype, kind="rank")
    pl = rng.integers(0, 1500, B)
    ol = rng.integers(0, 300, B)
    pl[3] = 0
    ol[4] = 0
    pids, poff = synth._csr([synth.zipf_ids(rng, int(n), V) for n in pl])
    oids, ooff = synth._csr([synth.zipf_ids(rng, int(n), V) for n in ol])
    oids = oids.copy()
    if len(oids) > 5:
        oids[2] = -3            # bad ids are skipped and reported
        oids[5] = V
    pres = rng.uniform(-0.5, 1.0, B).astype(np.float32)
    freq = rng.uniform(-0.2, 1.0, B).astype(np.float32)
    rep = rng.uniform(0.7, 1.5, B).astype(np.float32)
    rep[7] = 0.0                # bad parameter: row untouched
    xd = to_device(x)
    st = vs.penalize(xd, dev(pids, np.int32), dev(poff, np.int32), dev(oids, np.int32),
                     dev(ooff, np.int32), dev(pres, np.float32), dev(freq, np.float32),
                     dev(rep, np.float32)).cpu().numpy()
    xo = x.copy()
    so = oracle.penalize(xo, V, pids, poff, oids, ooff, pres, freq, rep)
    assert np.array_equal(st, so)
    got = from_device(xd, V)
    assert np.array_equal(got.view(np.uint8), xo.view(np.uint8))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_penalize_prompt_ignore_parity(dtype):
    """vs_penalize_ex: per-row prompt_ignore_length of 0, negative, inside the
    prompt, the whole prompt and past it, on rows with and without a prompt."""
    import decode_token_sampling_amd as vs
    rng = np.random.default_rng(17)
    B, V = 24, 40000
    x = synth.random_rows(18, B, V, dtype, kind="rank")
    pl = rng.integers(0, 1500, B)
    ol = rng.integers(0, 300, B)
    pl[3] = 0
    ol[4] = 0
    pids, poff = synth._csr([synth.zipf_ids(rng, int(n), V) for n in pl])
    oids, ooff = synth._csr([synth.zipf_ids(rng, int(n), V) for n in ol])
    ign = np.array([rng.integers(0, n + 1) if n else 0 for n in pl], np.int32)
    ign[0], ign[1], ign[2], ign[5] = 0, -7, int(pl[2]), int(pl[5]) + 100
    pres = rng.uniform(-0.5, 1.0, B).astype(np.float32)
    freq = rng.uniform(-0.2, 1.0, B).astype(np.float32)
    rep = rng.uniform(0.7, 1.5, B).astype(np.float32)
    xd = to_device(x)
    st = vs.penalize(xd, dev(pids, np.int32), dev(poff, np.int32), dev(oids, np.int32),
                     dev(ooff, np.int32), dev(pres, np.float32), dev(freq, np.float32),
                     dev(rep, np.float32), prompt_ignore=dev(ign, np.int32)).cpu().numpy()
    xo = x.copy()
    so = oracle.penalize(xo, V, pids, poff, oids, ooff, pres, freq, rep, prompt_ignore=ign)
    assert np.array_equal(st, so)
    assert np.array_equal(from_device(xd, V).view(np.uint8), xo.view(np.uint8))


def test_penalize_prompt_ignore_many_classes():
    """A prompt long enough for several hash classes: the ignored prefix is
    decided by history position in every class pass."""
    import decode_token_sampling_amd as vs
    rng = np.random.default_rng(19)
    B, V = 2, 300000
    x = synth.random_rows(20, B, V)
    plists = [rng.integers(0, V, 60000).astype(np.int32), np.arange(0, V, 5, dtype=np.int32)]
    olists = [rng.integers(0, V, 500).astype(np.int32), np.arange(0, V, 11, dtype=np.int32)]
    pids, poff = synth._csr(plists)
    oids, ooff = synth._csr(olists)
    ign = np.array([31000, 20000], np.int32)
    pres = np.full(B, 0.25, np.float32)
    freq = np.full(B, 0.01, np.float32)
    rep = np.full(B, 1.3, np.float32)
    xd = to_device(x)
    vs.penalize(xd, dev(pids, np.int32), dev(poff, np.int32), dev(oids, np.int32),
                dev(ooff, np.int32), dev(pres, np.float32), dev(freq, np.float32),
                dev(rep, np.float32), prompt_ignore=dev(ign, np.int32))
    xo = x.copy()
    oracle.penalize(xo, V, pids, poff, oids, ooff, pres, freq, rep, prompt_ignore=ign)
    assert np.array_equal(from_device(xd, V), xo)


def test_penalize_bad_id_in_every_wave():
    """Thread i of the penalty workgroup reads history ids i, i + 1024, ...;
    row r holds its one bad id at position 64 r + 5, which wave r reads. The
    row status reports it whichever wave finds it, and the valid ids are
    still applied."""
    import decode_token_sampling_amd as vs
    rng = np.random.default_rng(23)
    B, V = 16, 5000
    x = synth.random_rows(24, B, V, kind="rank")
    lists = []
    for r in range(B):
        ids = rng.integers(0, V, 1100).astype(np.int32)
        ids[64 * r + 5] = -1 if r % 2 else V
        lists.append(ids)
    oids, ooff = synth._csr(lists)
    rep = np.full(B, 1.25, np.float32)
    pres = np.full(B, 0.5, np.float32)
    xd = to_device(x)
    st = vs.penalize(xd, output_ids=dev(oids, np.int32), output_off=dev(ooff, np.int32),
                     presence=dev(pres, np.float32), repetition=dev(rep, np.float32)).cpu().numpy()
    xo = x.copy()
    so = oracle.penalize(xo, V, None, None, oids, ooff, pres, None, rep)
    assert (so == vs.ROW_BAD_TOKEN_ID).all()
    assert np.array_equal(st, so), st
    assert np.array_equal(from_device(xd, V), xo)


def test_penalize_long_history_many_classes():
    import decode_token_sampling_amd as vs
    rng = np.random.default_rng(13)
    B, V = 3, 300000
    x = synth.random_rows(14, B, V)
    lists = [rng.integers(0, V, 60000).astype(np.int32), np.arange(0, V, 7, dtype=np.int32),
             np.zeros(5, np.int32)]
    oids, ooff = synth._csr(lists)
    rep = np.full(B, 1.3, np.float32)
    freq = np.full(B, 0.01, np.float32)
    xd = to_device(x)
    vs.penalize(xd, output_ids=dev(oids, np.int32), output_off=dev(ooff, np.int32),
                frequency=dev(freq, np.float32), repetition=dev(rep, np.float32))
    xo = x.copy()
    oracle.penalize(xo, V, None, None, oids, ooff, None, freq, rep)
    assert np.array_equal(from_device(xd, V), xo)


# ---------------------------------------------------------------- penalties fused into the draw
def _histories(rng, B, V, with_bad=True):
    pl = rng.integers(0, 1500, B)
    ol = rng.integers(0, 300, B)
    pl[min(3, B - 1)] = 0
    pids, poff = synth._csr([synth.zipf_ids(rng, int(n), V) for n in pl])
    # output ids: Zipf plus uniform ids, so that every segment of a row has some
    oids, ooff = synth._csr([np.concatenate([synth.zipf_ids(rng, int(n) // 2, V),
                                             rng.integers(0, V, int(n) - int(n) // 2).astype(np.int32)])
                             for n in ol])
    oids = oids.copy()
    if with_bad and len(oids) > 9:
        oids[2], oids[9] = -3, V          # bad ids: skipped and reported
    ign = np.array([rng.integers(-5, n + 50) if n else 0 for n in pl], np.int32)
    pres = rng.uniform(-0.5, 1.0, B).astype(np.float32)
    freq = rng.uniform(-0.2, 1.0, B).astype(np.float32)
    rep = rng.uniform(0.7, 1.5, B).astype(np.float32)
    if B > 5:
        rep[5] = 0.0                      # a bad parameter: that row is left unpenalised
    return pids, poff, oids, ooff, pres, freq, rep, ign


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,V", [(24, 40000), (7, 70001), (320, 9000)])
def test_fused_penalties_equal_separate_calls_and_oracle(B, V, dtype):
    """vs_penalize_sample_logprobs against vs_penalize_ex then
    vs_sample_logprobs on a copy, and against the oracle's penalties then draw:
    penalised logits, penalty status, ids, kept counts and row status bit-exact;
    log-probs within 1e-5. Rows take one segment each (320 rows: the streaming
    pass finishes them) or several (the row and full-vocabulary kernels read
    the penalised logits the streaming pass wrote)."""
    import decode_token_sampling_amd as vs
    rng = np.random.default_rng(B + V)
    x = _row_shapes(60 + V, B, V, dtype)
    pids, poff, oids, ooff, pres, freq, rep, ign = _histories(rng, B, V)
    w = random_params(np.random.default_rng(V - B), B, V)
    hist = [dev(pids, np.int32), dev(poff, np.int32), dev(oids, np.int32), dev(ooff, np.int32),
            dev(pres, np.float32), dev(freq, np.float32), dev(rep, np.float32)]
    args = [dev(w["temperature"], np.float32), dev(w["top_k"], np.int32), dev(w["top_p"], np.float32),
            dev(w["min_p"], np.float32), dev(np.asarray(w["seeds"], np.uint64).view(np.int64), np.int64)]
    xa, xb = to_device(x), to_device(x)
    f = vs.penalize_sample_logprobs(xa, *hist, prompt_ignore=dev(ign, np.int32), temperature=args[0],
                                    top_k=args[1], top_p=args[2], min_p=args[3], seeds=args[4],
                                    k=5, V=V)
    pst = vs.penalize(xb, *hist, prompt_ignore=dev(ign, np.int32), V=V)
    s2 = vs.sample_logprobs(xb, *args, k=5, V=V)
    torch.cuda.synchronize()
    assert torch.equal(xa, xb) if dtype == "f32" else torch.equal(xa.view(torch.int16), xb.view(torch.int16))
    assert torch.equal(f["penalty_status"], pst)
    for key in ("ids", "kept", "status", "topk_ids"):
        assert torch.equal(f[key], s2[key]), key
    for key in ("token_lp", "topk_lp"):
        a, b = f[key].cpu().numpy(), s2[key].cpu().numpy()
        assert np.array_equal(np.isnan(a), np.isnan(b))
        ok = ~np.isnan(b)
        assert np.abs(a[ok] - b[ok]).max() <= LOGPROB_ATOL
    xo = x.copy()
    so = oracle.penalize(xo, V, pids, poff, oids, ooff, pres, freq, rep, prompt_ignore=ign)
    assert np.array_equal(f["penalty_status"].cpu().numpy(), so)
    assert np.array_equal(from_device(xa, V).view(np.uint8), xo.view(np.uint8))
    g = dict(ids=f["ids"].cpu().numpy(), kept=f["kept"].cpu().numpy(), status=f["status"].cpu().numpy())
    compare_sample(g, oracle_sample(xo, V, w, mask=False))
    _check_fused_logprobs(xo, V, f, 5)


@pytest.mark.parametrize("B", [9, 300])
def test_fused_penalties_move_the_argmax(B):
    """Greedy rows whose largest logit (at a segment's first, middle or last id,
    or the row's last) is in the history with a large presence penalty: the
    draw must see the penalised value that the same pass wrote, so the argmax
    moves to the runner-up, as the oracle's penalties-then-draw says."""
    import decode_token_sampling_amd as vs
    V = 50000
    rng = np.random.default_rng(B)
    x = synth.random_rows(70 + B, B, V, kind="normal")
    spots = [0, 2047, 2048, 4096 * 3 + 5, V // 2, V - 1]
    lists = []
    for r in range(B):
        top = spots[r % len(spots)]
        x[r, top] = 50.0
        lists.append(np.array([top, int(rng.integers(0, V))], np.int32))
    oids, ooff = synth._csr(lists)
    pres = np.full(B, 100.0, np.float32)
    T = np.zeros(B, np.float32)
    w = dict(temperature=T, top_k=np.zeros(B, np.int32), top_p=np.ones(B, np.float32),
             min_p=np.zeros(B, np.float32), seeds=np.arange(B, dtype=np.uint64))
    xd = to_device(x)
    f = vs.penalize_sample_logprobs(xd, output_ids=dev(oids, np.int32), output_off=dev(ooff, np.int32),
                                    presence=dev(pres, np.float32), temperature=dev(T, np.float32),
                                    k=1, V=V)
    torch.cuda.synchronize()
    xo = x.copy()
    oracle.penalize(xo, V, None, None, oids, ooff, pres, None, None)
    o = oracle_sample(xo, V, w, mask=False)
    ids = f["ids"].cpu().numpy()
    assert np.array_equal(ids, o["ids"])
    assert not np.any(ids == np.array([spots[r % len(spots)] for r in range(B)]))
    assert np.array_equal(from_device(xd, V), xo)


# ---------------------------------------------------------------- log-probs
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [1, 5, 64, 4097, 33333])
def test_logprobs_parity(V, dtype):
    import decode_token_sampling_amd as vs
    B = 9
    x = _row_shapes(50 + V, B, V, dtype)
    rng = np.random.default_rng(V)
    tok = rng.integers(0, V, B).astype(np.int32)
    k = min(V, 20)
    g = vs.logprobs(to_device(x), dev(tok, np.int32), k=k, full=True, V=V)
    torch.cuda.synchronize()
    o = oracle.logprobs(x, V, tok, k=k, full=True)
    assert np.array_equal(g["status"].cpu().numpy(), o["status"])
    assert np.allclose(g["token_lp"].cpu().numpy(), o["token_lp"], atol=LOGPROB_ATOL, rtol=0)
    assert np.array_equal(g["topk_ids"].cpu().numpy(), o["topk_ids"])
    assert np.allclose(g["topk_lp"].cpu().numpy(), o["topk_lp"], atol=LOGPROB_ATOL, rtol=0)
    full = g["full"].cpu().numpy()
    of = o["full"]
    fin = np.isfinite(of)
    assert np.array_equal(np.isfinite(full), fin) and np.array_equal(full[~fin], of[~fin])
    assert np.abs(full[fin] - of[fin]).max() <= LOGPROB_ATOL


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_maximum_vocabulary(dtype):
    """V = 2^21, the largest vocabulary the library takes: every row mode for
    the draw (ids, kept sets, status) and the log-probs (sampled-id, top-20,
    full row) against the oracle."""
    import decode_token_sampling_amd as vs
    V, B = 1 << 21, 9
    x = _row_shapes(77, B, V, dtype)
    rng = np.random.default_rng(78)
    w = random_params(rng, B, V)
    xd = to_device(x)
    compare_sample(gpu_sample(xd, V, w), oracle_sample(x, V, w))
    tok = rng.integers(0, V, B).astype(np.int32)
    g = vs.logprobs(xd, dev(tok, np.int32), k=20, full=True, V=V)
    torch.cuda.synchronize()
    o = oracle.logprobs(x, V, tok, k=20, full=True)
    assert np.array_equal(g["status"].cpu().numpy(), o["status"])
    assert np.allclose(g["token_lp"].cpu().numpy(), o["token_lp"], atol=LOGPROB_ATOL, rtol=0)
    assert np.array_equal(g["topk_ids"].cpu().numpy(), o["topk_ids"])
    assert np.allclose(g["topk_lp"].cpu().numpy(), o["topk_lp"], atol=LOGPROB_ATOL, rtol=0)
    full = g["full"].cpu().numpy()
    of = o["full"]
    fin = np.isfinite(of)
    assert np.array_equal(np.isfinite(full), fin) and np.array_equal(full[~fin], of[~fin])
    assert np.abs(full[fin] - of[fin]).max() <= LOGPROB_ATOL


def test_large_batch_short_rows():
    """2048 rows of 1000 ids: more rows than compute units, every row mode."""
    V, B = 1000, 2048
    x = _row_shapes(79, B, V, "f32")
    w = random_params(np.random.default_rng(80), B, V)
    compare_sample(gpu_sample(to_device(x), V, w), oracle_sample(x, V, w))


def _temperatures(rng, B):
    T = rng.choice([1.0, 0.5, 0.7, 1.3, 2.5], B).astype(np.float32)
    T[0], T[1 % B], T[2 % B] = 0.0, -1.0, np.nan
    if B > 3:
        T[3] = np.inf
    return T


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V,B", [(64, 9), (4097, 9), (33333, 9), (70001, 9), (9000, 320), (40000, 320)])
def test_logprobs_at_temperature(V, B, dtype):
    """vs_logprobs_ex: the log-softmax of x / T per row (T not positive and
    finite: 1) against the oracle; 9 rows take several segments each (the row
    kernel merges them), 320 rows one segment each (the streaming pass finishes
    them and writes the full row itself)."""
    import decode_token_sampling_amd as vs
    x = _row_shapes(90 + V, B, V, dtype)
    rng = np.random.default_rng(V + B)
    T = _temperatures(rng, B)
    if dtype == "f32" and B > 5:
        x[5, 7] = np.float32(3e38)   # x / T overflows on a row with T < 1
        T[5] = np.float32(0.5)
    tok = rng.integers(0, V, B).astype(np.int32)
    k = min(V, 20)
    g = vs.logprobs(to_device(x), dev(tok, np.int32), k=k, full=True, V=V, temperature=dev(T, np.float32))
    torch.cuda.synchronize()
    o = oracle.logprobs(x, V, tok, k=k, full=True, temperature=T)
    assert np.array_equal(g["status"].cpu().numpy(), o["status"])
    assert np.allclose(g["token_lp"].cpu().numpy(), o["token_lp"], atol=LOGPROB_ATOL, rtol=0,
                       equal_nan=True)
    assert np.array_equal(g["topk_ids"].cpu().numpy(), o["topk_ids"])
    assert np.allclose(g["topk_lp"].cpu().numpy(), o["topk_lp"], atol=LOGPROB_ATOL, rtol=0,
                       equal_nan=True)
    full, of = g["full"].cpu().numpy(), o["full"]
    finf = np.isfinite(of)
    assert np.array_equal(np.isfinite(full), finf)
    assert np.array_equal(np.isnan(full), np.isnan(of))
    assert np.abs(full[finf] - of[finf]).max() <= LOGPROB_ATOL


def test_logprobs_ties_and_bad_rows():
    import decode_token_sampling_amd as vs
    V, B = 9000, 5
    x = np.random.default_rng(3).integers(0, 2, (B, V)).astype(np.float32)
    x[1, 5] = np.nan
    x[2, :] = -np.inf
    tok = np.array([0, 1, 2, V + 3, -1], np.int32)
    g = vs.logprobs(to_device(x), dev(tok, np.int32), k=64, V=V)
    torch.cuda.synchronize()
    o = oracle.logprobs(x, V, tok, k=64)
    assert np.array_equal(g["status"].cpu().numpy(), o["status"])
    assert np.array_equal(g["topk_ids"].cpu().numpy(), o["topk_ids"])
    gl, ol = g["token_lp"].cpu().numpy(), o["token_lp"]
    assert np.array_equal(np.isnan(gl), np.isnan(ol))
    ok = ~np.isnan(ol)
    assert np.allclose(gl[ok], ol[ok], atol=LOGPROB_ATOL, rtol=0)


# ---------------------------------------------------------------- fused draw + log-probs
def _check_fused_logprobs(x, V, out, k):
    ids = out["ids"].cpu().numpy()
    o = oracle.logprobs(x, V, ids, k=k)
    tlp = out["token_lp"].cpu().numpy()
    ok = ~np.isnan(o["token_lp"])
    assert np.array_equal(np.isnan(tlp), ~ok)
    assert np.allclose(tlp[ok], o["token_lp"][ok], atol=LOGPROB_ATOL, rtol=0)
    if k:
        assert np.array_equal(out["topk_ids"].cpu().numpy(), o["topk_ids"])
        gl, ol = out["topk_lp"].cpu().numpy(), o["topk_lp"]
        assert np.array_equal(np.isnan(gl), np.isnan(ol))
        fin = ~np.isnan(ol)
        assert np.allclose(gl[fin], ol[fin], atol=LOGPROB_ATOL, rtol=0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [7, 4097, 32000, 70001])
@pytest.mark.parametrize("k", [0, 1, 5, 64])
def test_sample_logprobs_fused(V, dtype, k):
    import decode_token_sampling_amd as vs
    B = 27
    k = min(k, V)
    x = _row_shapes(2000 + V, B, V, dtype)
    x[3, 1] = np.nan if dtype == "f32" else 0x7FC0   # a bad row
    w = random_params(np.random.default_rng(V + k), B, V)
    out = vs.sample_logprobs(to_device(x), dev(w["temperature"], np.float32),
                             dev(w["top_k"], np.int32), dev(w["top_p"], np.float32),
                             dev(w["min_p"], np.float32),
                             dev(np.asarray(w["seeds"], np.uint64).view(np.int64), np.int64),
                             k=k, mask=True, V=V)
    torch.cuda.synchronize()
    g = dict(ids=out["ids"].cpu().numpy(), kept=out["kept"].cpu().numpy(),
             status=out["status"].cpu().numpy(), mask=mask_bits(out["mask"], V))
    compare_sample(g, oracle_sample(x, V, w))
    _check_fused_logprobs(x, V, out, k)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("k", [0, 5])
def test_gather_draw_finish_with_logprobs(dtype, k):
    """The default draw of full-vocabulary rows (the gather pass draws, the cut
    kernel finishes each row) with the sampled ids' log-probs and no kept mask,
    on every way the cut kernel finishes a row: a cut from the gathered list,
    a cut bucket beyond the list (a row of one value: the one-pass draw over
    the kept set), rows without the cut (top_p = 1) with and without min-p; at
    T = 1 (where the sampled id's logit is its s) and T != 1; a batch below
    and one above 16 rows. Ids, kept counts, status and log-probs against the
    oracle."""
    import decode_token_sampling_amd as vs
    V = 40000
    for B in (6, 20):
        x = _row_shapes(4000 + B + 13 * k, B, V, dtype)
        one = synth.f32_to_bf16_bits(np.array([np.float32(0.5)]))[0] if dtype == "bf16" else np.float32(0.5)
        x[1] = one                                   # one value: the bucket holds every id
        x[B - 2] = one
        rows = np.arange(B)
        T = np.where(rows % 2 == 0, 1.0, 0.7).astype(np.float32)
        p = np.array([0.9, 0.6, 1.0, 0.99, 1.0, 0.3], np.float32)[rows % 6]
        mp = np.where(rows % 3 == 2, 0.05, 0.0).astype(np.float32)
        w = dict(temperature=T, top_k=np.zeros(B, np.int32), top_p=p, min_p=mp,
                 seeds=(900 + rows).astype(np.uint64))
        out = vs.sample_logprobs(to_device(x), dev(T, np.float32), dev(w["top_k"], np.int32),
                                 dev(p, np.float32), dev(mp, np.float32),
                                 dev(np.asarray(w["seeds"], np.uint64).view(np.int64), np.int64),
                                 k=k, mask=False, V=V)
        torch.cuda.synchronize()
        g = dict(ids=out["ids"].cpu().numpy(), kept=out["kept"].cpu().numpy(),
                 status=out["status"].cpu().numpy())
        assert compare_sample(g, oracle_sample(x, V, w, mask=False), check_mask=False) == 0
        _check_fused_logprobs(x, V, out, k)


def test_fused_equals_separate_calls():
    import decode_token_sampling_amd as vs
    V, B = 50000, 24
    x = _row_shapes(31, B, V, "f32")
    w = random_params(np.random.default_rng(4), B, V)
    args = [dev(w["temperature"], np.float32), dev(w["top_k"], np.int32), dev(w["top_p"], np.float32),
            dev(w["min_p"], np.float32), dev(np.asarray(w["seeds"], np.uint64).view(np.int64), np.int64)]
    xd = to_device(x)
    f = vs.sample_logprobs(xd, *args, k=20, full=True)
    s = vs.sample(xd, *args)
    l = vs.logprobs(xd, s["ids"], k=20, full=True)
    torch.cuda.synchronize()
    assert torch.equal(f["ids"], s["ids"]) and torch.equal(f["kept"], s["kept"])
    assert torch.equal(f["status"], s["status"])
    good = s["ids"] >= 0
    assert torch.equal(f["token_lp"][good], l["token_lp"][good])
    assert torch.equal(f["topk_ids"], l["topk_ids"]) and torch.equal(f["topk_lp"], l["topk_lp"])
    assert torch.equal(f["full"], l["full"])


# ---------------------------------------------------------------- rows finished by the streaming pass
# With at least one row per compute unit every row gets a workgroup of its
# own, which also finishes the row (draw, log-probs) when no kept mask is asked
# for; rows that need the row kernels (top-k > 64, full vocabulary, ties that
# overflow the candidate pool) still go there. These tests run such batches
# without a mask, against the oracle and against the row-kernel path (the
# same call with a mask).
FIN_B = 320


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [7, 2048, 4097, 70001])
def test_finish_in_stream_sample(V, dtype):
    x = _row_shapes(3000 + V, FIN_B, V, dtype)
    w = random_params(np.random.default_rng(V + 7), FIN_B, V)
    xd = to_device(x)
    g = gpu_sample(xd, V, w, mask=False)
    compare_sample(g, oracle_sample(x, V, w, mask=False))
    gm = gpu_sample(xd, V, w, mask=True)
    for key in ("ids", "kept", "status"):
        assert np.array_equal(g[key], gm[key]), key


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [4097, 32000])
@pytest.mark.parametrize("k", [0, 1, 5, 20, 64])
def test_finish_in_stream_fused(V, dtype, k):
    import decode_token_sampling_amd as vs
    x = _row_shapes(4000 + V, FIN_B, V, dtype)
    x[3, 1] = np.nan if dtype == "f32" else 0x7FC0   # a bad row
    w = random_params(np.random.default_rng(V + 3 * k), FIN_B, V)
    out = vs.sample_logprobs(to_device(x), dev(w["temperature"], np.float32),
                             dev(w["top_k"], np.int32), dev(w["top_p"], np.float32),
                             dev(w["min_p"], np.float32),
                             dev(np.asarray(w["seeds"], np.uint64).view(np.int64), np.int64),
                             k=k, V=V)
    torch.cuda.synchronize()
    g = dict(ids=out["ids"].cpu().numpy(), kept=out["kept"].cpu().numpy(),
             status=out["status"].cpu().numpy())
    compare_sample(g, oracle_sample(x, V, w, mask=False))
    _check_fused_logprobs(x, V, out, k)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [4097, 32000])
def test_finish_in_stream_full_logsoftmax(V, dtype):
    """Rows the streaming pass finishes (greedy and small top-k rows, promised
    by the hint): the pass writes the full log-softmax itself. It agrees with
    the separate write pass that runs when a kept mask sends the rows to the
    row kernel (to the log-prob tolerance: the waves' log-sum-exp partials are
    summed in the order their dynamically claimed tiles give, so the last bit
    of log S can differ from call to call) and with the oracle; a bad row is
    NaN throughout."""
    import decode_token_sampling_amd as vs
    x = _row_shapes(7000 + V, FIN_B, V, dtype)
    x[3, 1] = np.nan if dtype == "f32" else 0x7FC0
    rng = np.random.default_rng(V + 11)
    T = rng.uniform(0.5, 1.5, FIN_B).astype(np.float32)
    T[::5] = 0.0
    top_k = rng.integers(2, 65, FIN_B).astype(np.int32)
    top_p = rng.uniform(0.5, 1.0, FIN_B).astype(np.float32)
    seeds = np.arange(99, 99 + FIN_B, dtype=np.uint64)
    args = [dev(T, np.float32), dev(top_k, np.int32), dev(top_p, np.float32),
            dev(np.zeros(FIN_B, np.float32), np.float32), dev(seeds.view(np.int64), np.int64)]
    xd = to_device(x)
    f = vs.sample_logprobs(xd, *args, hints=vs.HINT_SMALL_TOPK, k=20, full=True, V=V)
    r = vs.sample_logprobs(xd, *args, k=20, full=True, mask=True, V=V)
    torch.cuda.synchronize()
    assert torch.equal(f["ids"], r["ids"]) and torch.equal(f["status"], r["status"])
    ff, rf = f["full"], r["full"]
    assert torch.equal(torch.isnan(ff), torch.isnan(rf)) and bool(torch.isnan(ff[3]).all())
    inf = torch.isinf(ff)
    assert torch.equal(inf, torch.isinf(rf)) and torch.equal(ff[inf], rf[inf])
    fin = torch.isfinite(ff)
    assert torch.equal(fin, torch.isfinite(rf))
    assert (ff[fin] - rf[fin]).abs().max().item() <= LOGPROB_ATOL
    rows = np.array([0, 1, 3, 100, FIN_B - 1])
    o = oracle.logprobs(np.ascontiguousarray(x[rows]), V, f["ids"].cpu().numpy()[rows], k=20,
                        full=True)
    got = f["full"][torch.from_numpy(rows).cuda()].cpu().numpy()
    fin = np.isfinite(o["full"])
    assert np.array_equal(np.isfinite(got), fin)
    assert np.abs(got[fin] - o["full"][fin]).max() <= LOGPROB_ATOL


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("k", [0, 1, 20, 64])
def test_finish_in_stream_logprobs(dtype, k):
    import decode_token_sampling_amd as vs
    V = 33333
    x = _row_shapes(5000 + k, FIN_B, V, dtype)
    x[7, 3] = np.nan if dtype == "f32" else 0x7FC0
    tok = np.random.default_rng(k).integers(0, V, FIN_B).astype(np.int32)
    tok[5], tok[6] = -1, V  # bad ids
    g = vs.logprobs(to_device(x), dev(tok, np.int32), k=k, V=V)
    torch.cuda.synchronize()
    o = oracle.logprobs(x, V, tok, k=k)
    assert np.array_equal(g["status"].cpu().numpy(), o["status"])
    gl, ol = g["token_lp"].cpu().numpy(), o["token_lp"]
    assert np.array_equal(np.isnan(gl), np.isnan(ol))
    ok = ~np.isnan(ol)
    assert np.allclose(gl[ok], ol[ok], atol=LOGPROB_ATOL, rtol=0)
    if k:
        assert np.array_equal(g["topk_ids"].cpu().numpy(), o["topk_ids"])
        gk, ok_ = g["topk_lp"].cpu().numpy(), o["topk_lp"]
        assert np.array_equal(np.isnan(gk), np.isnan(ok_))
        fin = ~np.isnan(ok_)
        assert np.allclose(gk[fin], ok_[fin], atol=LOGPROB_ATOL, rtol=0)


# ---------------------------------------------------------------- pool overflow: the rescan
# Rows that overflow the streaming pass's candidate pool: ascending or
# descending values (the running bound trails every new value), constant rows
# and a handful of levels (ties at the k-th value), a few finite values among
# -inf (fewer than k finite ids). A row finished by the streaming pass then
# rebuilds its lists by a rescan of the row; with a kept mask the row kernel's
# exact path does it instead. Both must equal the oracle.
def _overflow_rows(seed, B, V, dtype):
    rng = np.random.default_rng(seed)
    x = np.empty((B, V), np.float32)
    for r in range(B):
        kind = r % 6
        if kind == 0:
            x[r] = np.linspace(-6, 6, V, dtype=np.float32)
        elif kind == 1:
            x[r] = np.linspace(6, -6, V, dtype=np.float32)
        elif kind == 2:
            x[r] = np.float32(0.5)
        elif kind == 3:
            x[r] = -np.inf
            n = int(rng.integers(1, 12))
            x[r, rng.choice(V, min(n, V), replace=False)] = rng.normal(size=min(n, V))
        elif kind == 4:
            x[r] = rng.integers(0, 4, V).astype(np.float32)
        else:
            x[r] = rng.normal(size=V).astype(np.float32)
    return synth.f32_to_bf16_bits(x) if dtype == "bf16" else x


def _small_topk_params(rng, B):
    """Greedy rows and rows with 1 < top_k <= 64, some with top-p and min-p."""
    T = rng.choice(np.array([1.0, 0.7, 1.3], np.float32), B).astype(np.float32)
    k = rng.choice(np.array([2, 5, 20, 64], np.int32), B).astype(np.int32)
    p = np.where(rng.random(B) < 0.5, np.float32(1.0), rng.uniform(0.2, 0.99, B)).astype(np.float32)
    mp = np.where(rng.random(B) < 0.25, np.float32(0.05), np.float32(0)).astype(np.float32)
    T[::7] = 0.0  # greedy rows
    return dict(temperature=T, top_k=k, top_p=p, min_p=mp,
                seeds=rng.integers(0, 2**63, B, dtype=np.int64).astype(np.uint64))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [4097, 8192, 70001, 70004])
def test_finish_in_stream_overflow_rescan(V, dtype):
    import decode_token_sampling_amd as vs
    x = _overflow_rows(6000 + V, FIN_B, V, dtype)
    w = _small_topk_params(np.random.default_rng(V), FIN_B)
    xd = to_device(x)
    o = oracle_sample(x, V, w, mask=False)
    for hints in (vs.HINT_SMALL_TOPK, 0):  # without the row kernel, and with it launched
        compare_sample(gpu_sample(xd, V, w, hints=hints, mask=False), o)
    g = gpu_sample(xd, V, w, mask=True)  # the row kernel's exact path
    compare_sample(g, oracle_sample(x, V, w, mask=True))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [12344, 12345])
@pytest.mark.parametrize("k", [1, 20, 64])
def test_finish_in_stream_overflow_fused(dtype, V, k):
    import decode_token_sampling_amd as vs
    x = _overflow_rows(7000 + k, FIN_B, V, dtype)
    w = _small_topk_params(np.random.default_rng(k), FIN_B)
    out = vs.sample_logprobs(to_device(x), dev(w["temperature"], np.float32),
                             dev(w["top_k"], np.int32), dev(w["top_p"], np.float32),
                             dev(w["min_p"], np.float32),
                             dev(np.asarray(w["seeds"], np.uint64).view(np.int64), np.int64),
                             hints=vs.HINT_SMALL_TOPK, k=k, V=V)
    torch.cuda.synchronize()
    g = dict(ids=out["ids"].cpu().numpy(), kept=out["kept"].cpu().numpy(),
             status=out["status"].cpu().numpy())
    compare_sample(g, oracle_sample(x, V, w, mask=False))
    _check_fused_logprobs(x, V, out, k)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("k", [20, 64])
def test_finish_in_stream_overflow_logprobs(dtype, k):
    import decode_token_sampling_amd as vs
    V = 9000
    x = _overflow_rows(8000 + k, FIN_B, V, dtype)
    tok = np.random.default_rng(k).integers(0, V, FIN_B).astype(np.int32)
    g = vs.logprobs(to_device(x), dev(tok, np.int32), k=k, V=V)
    torch.cuda.synchronize()
    o = oracle.logprobs(x, V, tok, k=k)
    assert np.array_equal(g["status"].cpu().numpy(), o["status"])
    gl, ol = g["token_lp"].cpu().numpy(), o["token_lp"]
    assert np.array_equal(np.isnan(gl), np.isnan(ol))
    fin = ~np.isnan(ol)
    assert np.allclose(gl[fin], ol[fin], atol=LOGPROB_ATOL, rtol=0)
    assert np.array_equal(g["topk_ids"].cpu().numpy(), o["topk_ids"])
    gk, ok_ = g["topk_lp"].cpu().numpy(), o["topk_lp"]
    assert np.array_equal(np.isnan(gk), np.isnan(ok_))
    fin = ~np.isnan(ok_)
    assert np.allclose(gk[fin], ok_[fin], atol=LOGPROB_ATOL, rtol=0)


@pytest.mark.parametrize("B", [12, FIN_B])
def test_sample_hint_small_topk(B):
    """Rows that break the small top-k promise (full vocabulary, top-k above
    64) report it and draw nothing; the others match the oracle, whether the
    streaming pass finishes every row (one segment per row) or not."""
    import decode_token_sampling_amd as vs
    V = 9000
    x = synth.random_rows(9 + B, B, V)
    w = random_params(np.random.default_rng(B), B, V, kinds=["greedy", "kfast", "kslow", "topp"])
    o = oracle_sample(x, V, w, mask=False)
    g = gpu_sample(to_device(x), V, w, hints=vs.HINT_SMALL_TOPK, mask=False)
    bad = (np.arange(B) % 4 == 2) | (np.arange(B) % 4 == 3)
    assert (g["status"][bad] == vs.ROW_HINT_VIOLATED).all() and (g["ids"][bad] == -1).all()
    assert (g["kept"][bad] == 0).all()
    compare_sample(g, o, rows=np.nonzero(~bad)[0])


# ---------------------------------------------------------------- greedy rows kept on chip
# Greedy batches with the full log-softmax, fp32 rows of 94,209 to 131,072
# values and one row per workgroup: one kernel keeps each row in registers and
# LDS and writes every output from there.
@pytest.mark.parametrize("V", [94212, 128256, 131072])
@pytest.mark.parametrize("k", [0, 1, 20, 64])
def test_resident_greedy_full(V, k):
    """Edge rows first: a constant row (ties everywhere: the top-k from the row
    read again), a NaN, a +inf, all -inf, ten finite values among -inf (the
    top-k runs into -inf), huge values (one maximum near the fp32 limit: exact
    differences), a maximum held twice, -0 and +0 as the maximum, the maximum in
    the last vector (the LDS part); then random rows. Ids, kept counts and
    status against the oracle; log-probs, top-k and the full log-softmax against
    the oracle on the edge rows and a few random ones, and on every row against
    the same call with a kept mask (the row kernels' path)."""
    import decode_token_sampling_amd as vs
    B = 256
    rng = np.random.default_rng(V + 7 * k)
    x = (np.float32(4.0) * rng.standard_normal((B, V), dtype=np.float32))
    x[0] = np.float32(0.5)
    x[1, 77] = np.nan
    x[2, V // 2] = np.inf
    x[3] = -np.inf
    x[4] = -np.inf
    x[4, rng.choice(V, 10, replace=False)] = rng.standard_normal(10).astype(np.float32)
    x[5] = np.float32(2e38) - np.float32(2.0 ** 110) * rng.integers(0, 1000, V).astype(np.float32)
    x[5, 12345] = np.float32(3e38)
    x[6, 100] = x[6, 5000] = np.float32(50.0)
    x[7] = -np.abs(x[7]) - np.float32(1.0)
    x[7, 300] = np.float32(0.0)
    x[7, 200] = np.float32(-0.0)
    x[8, V - 1] = np.float32(60.0)
    T = np.zeros(B, np.float32)
    top_k = np.zeros(B, np.int32)
    T[9], top_k[9] = 1.0, 1                      # greedy by top_k = 1
    w = dict(temperature=T, top_k=top_k, top_p=np.ones(B, np.float32),
             min_p=np.zeros(B, np.float32), seeds=np.arange(B, dtype=np.uint64))
    args = [dev(T, np.float32), dev(top_k, np.int32), dev(w["top_p"], np.float32),
            dev(w["min_p"], np.float32), dev(w["seeds"].view(np.int64), np.int64)]
    xd = to_device(x)
    f = vs.sample_logprobs(xd, *args, hints=vs.HINT_ALL_GREEDY, k=k, full=True, V=V)
    r = vs.sample_logprobs(xd, *args, k=k, full=True, mask=True, V=V)
    torch.cuda.synchronize()
    g = dict(ids=f["ids"].cpu().numpy(), kept=f["kept"].cpu().numpy(),
             status=f["status"].cpu().numpy())
    assert compare_sample(g, oracle_sample(x, V, w, mask=False), check_mask=False) == 0
    assert g["ids"][0] == 0 and g["ids"][6] == 100 and g["ids"][7] == 200 and g["ids"][8] == V - 1
    assert torch.equal(f["ids"], r["ids"]) and torch.equal(f["status"], r["status"])
    ff, rf = f["full"], r["full"]
    assert torch.equal(torch.isnan(ff), torch.isnan(rf))
    assert torch.equal(torch.isinf(ff), torch.isinf(rf))
    fin = torch.isfinite(ff)
    assert (ff[fin] - rf[fin]).abs().max().item() <= LOGPROB_ATOL
    if k:
        assert torch.equal(f["topk_ids"], r["topk_ids"])
    rows = np.array(list(range(10)) + [10, 100, B - 1])
    xs = np.ascontiguousarray(x[rows])
    ids = g["ids"][rows]
    out = {key: (f[key][torch.from_numpy(rows).cuda()] if f.get(key) is not None else None)
           for key in ("ids", "token_lp", "topk_ids", "topk_lp")}
    _check_fused_logprobs(xs, V, out, k)
    o = oracle.logprobs(xs, V, ids, k=k, full=True)
    got = ff[torch.from_numpy(rows).cuda()].cpu().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(o["full"]))
    finf = np.isfinite(o["full"])
    assert np.array_equal(np.isfinite(got), finf)
    assert np.abs(got[finf] - o["full"][finf]).max() <= LOGPROB_ATOL
