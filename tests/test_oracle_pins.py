"""Pins for the CPU oracle: each check ties it to something other than itself.

Sources: the page fixtures under tests/golden (each carries its citation),
closed forms, brute force on tiny inputs, published known answers, and
statistics. Runs on the CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32_MAX = np.finfo(np.float32).max


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- random stream
def test_splitmix64_known_answers(orc):
    g = _golden("splitmix64_known_answers.json")
    gamma = 0x9E3779B97F4A7C15
    for n, want in enumerate(g["state0_outputs"]):
        assert orc.splitmix64((n * gamma) % 2**64) == int(want, 16)


def test_seed_advance_walks_the_splitmix64_states(orc):
    """Advancing a seed of 0 n times gives the generator's state n * gamma, so its
    mixed value is the published output n + 1; rows without a sampled token
    keep their seed."""
    g = _golden("splitmix64_known_answers.json")
    seeds = np.zeros(2, np.uint64)
    for n, want in enumerate(g["state0_outputs"]):
        assert orc.splitmix64(int(seeds[0])) == int(want, 16)
        orc.seed_advance(seeds, np.array([5, -1], np.int32))
    assert int(seeds[1]) == 0
    s = np.array([2**64 - 1], np.uint64)
    orc.seed_advance(s)
    assert int(s[0]) == (2**64 - 1 + 0x9E3779B97F4A7C15) % 2**64


def test_slot_remap_hand_case(orc):
    g = _golden("slot_remap_hand.json")
    src = np.array(g["old"], np.uint64)
    dst = np.array(g["dst_before"], np.uint64)
    st = orc.slot_remap(np.array(g["remap"], np.int32), src, dst)
    assert dst.tolist() == g["expected"] and st.tolist() == [0, 0, 0, 0]
    # an entry past the old batch is reported and leaves the slot
    d2 = np.full(3, 7, np.float32)
    st = orc.slot_remap(np.array([1, 5, 0], np.int32), np.array([0.5, 0.25], np.float32), d2)
    assert d2.tolist() == [0.25, 7.0, 0.5] and st.tolist() == [0, 1, 0]


def test_topp_decay_hand_sequence(orc):
    g = _golden("topp_decay_hand.json")
    p = np.array([g["top_p_init"]], np.float32)
    got = []
    for t in g["tokens"]:
        st = orc.topp_decay(p, [g["top_p_init"]], [g["decay"]], np.array([t], np.int32),
                            top_p_min=[g["top_p_min"]], reset_ids=[g["reset_id"]])
        assert st[0] == 0
        got.append(float(p[0]))
    assert got == [float(np.float32(v)) for v in g["expected"]]


def test_topp_decay_defaults_and_rejections(orc):
    # an initial top_p of 1 with an active decay: the first token already decays it
    p = np.array([1.0], np.float32)
    orc.topp_decay(p, [1.0], [0.75], np.array([0], np.int32))
    assert p[0] == np.float32(0.75)
    # the default floor is 1e-6 and no reset id matches by default
    p = np.array([0.5], np.float32)
    for _ in range(60):
        orc.topp_decay(p, [0.5], [0.5], np.array([0], np.int32))
    assert p[0] == np.float32(1e-6)
    # out-of-range parameters: the row is rejected and unchanged
    bad = [dict(decay=0.0), dict(decay=1.5), dict(top_p_min=0.0), dict(top_p_min=2.0),
           dict(reset=-2), dict(init=1.5)]
    for b in bad:
        p = np.array([0.3], np.float32)
        st = orc.topp_decay(p, [b.get("init", 0.3)], [b.get("decay", 0.5)], np.array([4], np.int32),
                            top_p_min=[b.get("top_p_min", 0.1)], reset_ids=[b.get("reset", -1)])
        assert st[0] == 1 and p[0] == np.float32(0.3), b


def test_uniform_range_and_distribution(orc):
    u = np.array([orc.uniform(s, r, j) for s in (0, 1234, 2**63 + 5) for r in range(8)
                  for j in range(0, 4000, 3)])
    assert np.all(u > 0.0) and np.all(u < 1.0)
    # 20-bin histogram chi-square against the flat density (19 dof; 99.99% point ~ 50)
    h, _ = np.histogram(u, bins=20, range=(0, 1))
    e = len(u) / 20
    assert ((h - e) ** 2 / e).sum() < 50
    # mean of -log(u) is 1 for an exponential
    assert abs(np.mean(-np.log(u)) - 1.0) < 0.02


def test_uniform_rows_and_ids_uncorrelated(orc):
    a = np.array([orc.uniform(77, 0, j) for j in range(20000)])
    b = np.array([orc.uniform(77, 1, j) for j in range(20000)])
    assert abs(np.corrcoef(a, b)[0, 1]) < 0.03           # neighbouring rows
    assert abs(np.corrcoef(a[:-1], a[1:])[0, 1]) < 0.03   # neighbouring ids
    c = np.array([orc.uniform(78, 0, j) for j in range(20000)])
    assert abs(np.corrcoef(a, c)[0, 1]) < 0.03           # neighbouring seeds


def test_uniform_is_exact_dyadic_midpoint(orc):
    # u = (m + 1/2) * 2^-52 for an integer m in [0, 2^52): 2^53 * u is odd
    for s, r, j in [(0, 0, 0), (1, 2, 3), (2**64 - 1, 255, 248319)]:
        v = orc.uniform(s, r, j) * 2.0**53
        assert v == math.floor(v) and int(v) % 2 == 1


# ---------------------------------------------------------------- pinned exp
def test_exp_special_values(orc):
    assert orc.exp_pinned(0.0) == 1.0
    assert orc.exp_pinned(-0.0) == 1.0
    assert orc.exp_pinned(-87.5) == 0.0
    assert orc.exp_pinned(float("-inf")) == 0.0
    assert orc.exp_pinned(-87.0) > 0.0
    # e^(-n ln2) = 2^-n (to the rounding of the argument)
    for n in (1, 2, 10, 40, 100, 125):
        t = np.float32(-n * math.log(2.0))
        assert abs(orc.exp_pinned(float(t)) / 2.0**-n - 1.0) < 1e-5


def test_exp_monotone_and_correctly_rounded_large_arguments(orc):
    # every float in [-87, -1]: monotone, and within half an fp32 ulp of an 80-bit exp
    viol, ulp = orc.exp_scan(-87.0, -1.0)
    assert viol == 0
    assert ulp <= 0.5000001


def test_exp_monotone_small_arguments_sampled(orc):
    for lo, hi in [(-1.0, -0.999), (-0.5, -0.4995), (-0.01, -0.00999), (-2.0**-20, -2.0**-21)]:
        viol, ulp = orc.exp_scan(lo, hi)
        assert viol == 0 and ulp <= 0.5000001
    # below half an ulp of 1 the value is exactly 1
    for t in (-2.0**-25, -2.0**-40, -1e-30, -1e-45):
        assert orc.exp_pinned(t) == 1.0


@pytest.mark.slow
def test_exp_monotone_small_arguments_exhaustive(orc):
    viol, ulp = orc.exp_scan(-1.0, -(2.0 ** -26))
    assert viol == 0 and ulp <= 0.5000001


# ---------------------------------------------------------------- bf16 rounding
def test_bf16_round_to_nearest_even(orc):
    one = 0x3F80
    assert orc.f32_to_bf16(1.0) == one
    assert orc.f32_to_bf16(1.0 + 2.0**-8) == one            # halfway, even stays
    assert orc.f32_to_bf16(1.0 + 3 * 2.0**-8) == one + 2    # halfway, odd rounds up
    assert orc.f32_to_bf16(1.0 + 2.0**-8 + 2.0**-20) == one + 1
    assert orc.f32_to_bf16(-1.0 - 2.0**-8 - 2.0**-20) == 0xBF81
    assert orc.f32_to_bf16(float("inf")) == 0x7F80
    assert orc.f32_to_bf16(3.3895e38) == 0x7F7F              # the largest bf16
    assert orc.f32_to_bf16(3.398e38) == 0x7F80               # past the midpoint to 2^128


# ---------------------------------------------------------------- penalties
def _pen_csr(lists):
    off = np.zeros(len(lists) + 1, np.int32)
    off[1:] = np.cumsum([len(l) for l in lists])
    ids = np.array([i for l in lists for i in l], np.int32)
    return ids, off


def test_penalty_hand_case(orc):
    g = _golden("penalties_hand.json")
    x = np.array([g["logits"]], np.float32)
    pids, poff = _pen_csr([g["prompt_ids"]])
    oids, ooff = _pen_csr([g["output_ids"]])
    st = orc.penalize(x, g["V"], pids, poff, oids, ooff,
                      np.array([g["presence"]], np.float32), np.array([g["frequency"]], np.float32),
                      np.array([g["repetition"]], np.float32))
    assert st[0] == 0
    assert x[0].tolist() == g["expected"]


def test_penalty_prompt_ignore_hand_case(orc):
    """prompt_ignore_length on a hand-derived case; 0, negative and past-the-prompt
    values behave as the page says (no effect, no effect, clamped)."""
    g = _golden("penalties_ignore_hand.json")
    pids, poff = _pen_csr([g["prompt_ids"]])
    oids, ooff = _pen_csr([g["output_ids"]])
    par = [np.array([g[k]], np.float32) for k in ("presence", "frequency", "repetition")]
    for n, key in [(g["prompt_ignore"], "expected"), (0, "expected_no_ignore"), (-5, "expected_no_ignore")]:
        x = np.array([g["logits"]], np.float32)
        st = orc.penalize(x, g["V"], pids, poff, oids, ooff, *par, prompt_ignore=np.array([n], np.int32))
        assert st[0] == 0
        assert x[0].tolist() == g[key], n


def test_penalty_prompt_ignore_properties(orc):
    """N past the prompt equals N = prompt length (every prompt id counts for
    repetition only); N = 0 equals no argument; an id seen only in the ignored
    prefix gets the repetition step alone."""
    rng = np.random.default_rng(11)
    B, V = 6, 300
    plist = [rng.integers(0, V, rng.integers(0, 40)).tolist() for _ in range(B)]
    olist = [rng.integers(0, V, rng.integers(0, 20)).tolist() for _ in range(B)]
    pids, poff = _pen_csr(plist)
    oids, ooff = _pen_csr(olist)
    par = [rng.uniform(-1, 1, B).astype(np.float32), rng.uniform(-1, 1, B).astype(np.float32),
           rng.uniform(0.5, 2, B).astype(np.float32)]
    base = rng.normal(0, 3, (B, V)).astype(np.float32)
    lens = np.diff(poff)

    def run(ign):
        x = base.copy()
        orc.penalize(x, V, pids, poff, oids, ooff, *par, prompt_ignore=ign)
        return x
    assert np.array_equal(run(None).view(np.uint32), run(np.zeros(B, np.int32)).view(np.uint32))
    assert np.array_equal(run(lens.astype(np.int32)).view(np.uint32),
                          run((lens + 7).astype(np.int32)).view(np.uint32))
    full = run(lens.astype(np.int32))
    for r in range(B):
        only_prompt = set(plist[r]) - set(olist[r])
        rep = par[2][r]
        for j in only_prompt:
            x = base[r, j]
            want = np.float32(x / rep) if x >= 0 else np.float32(x * rep)
            assert full[r, j] == want
        for j in set(range(V)) - set(plist[r]) - set(olist[r]):
            assert full[r, j] == base[r, j]


def test_penalty_neutral_is_identity_and_unseen_untouched(orc):
    for dt in ("f32", "bf16"):
        x = synth.random_rows(5, 3, 500, dt)
        x0 = x.copy()
        ids, off = _pen_csr([[1, 2, 2, 499], [], [0] * 10])
        st = orc.penalize(x, 500, ids, off, None, None, np.zeros(3, np.float32),
                          np.zeros(3, np.float32), np.ones(3, np.float32))
        assert (st == 0).all()
        assert np.array_equal(x.view(np.uint8), x0.view(np.uint8))
        x = x0.copy()
        orc.penalize(x, 500, ids, off, None, None, np.full(3, 0.3, np.float32),
                     np.full(3, 0.1, np.float32), np.full(3, 1.7, np.float32))
        seen = [{1, 2, 499}, set(), {0}]
        for r in range(3):
            for j in range(500):
                if j not in seen[r]:
                    assert x[r, j] == x0[r, j]


def test_penalty_directions(orc):
    # repetition > 1 pushes a seen token down on both signs; < 1 pulls it up;
    # presence does not depend on the count; frequency is linear in it.
    x = np.array([[3.0, -3.0, 3.0, -3.0]], np.float32)
    ids, off = _pen_csr([[0, 1]])
    orc.penalize(x, 4, ids, off, None, None, None, None, np.array([1.5], np.float32))
    assert x[0, 0] < 3.0 and x[0, 1] < -3.0
    x = np.array([[3.0, -3.0]], np.float32)
    orc.penalize(x, 2, ids, off, None, None, None, None, np.array([0.5], np.float32))
    assert x[0, 0] > 3.0 and x[0, 1] > -3.0
    x = np.zeros((1, 4), np.float32)
    ids, off = _pen_csr([[0, 1, 1, 1]])
    orc.penalize(x, 4, ids, off, None, None, np.array([0.7], np.float32), None, None)
    assert x[0, 0] == x[0, 1] == np.float32(-0.7)
    x = np.zeros((1, 4), np.float32)
    orc.penalize(x, 4, ids, off, None, None, None, np.array([0.5], np.float32), None)
    assert x[0, 0] == -0.5 and x[0, 1] == -1.5


def test_penalty_bf16_store_is_nearest_even(orc):
    x = synth.random_rows(9, 1, 300, "bf16", scale=3.0)
    x0 = synth.bf16_bits_to_f32(x.copy())
    ids, off = _pen_csr([list(range(0, 300, 2))])
    orc.penalize(x, 300, ids, off, None, None, np.array([0.013], np.float32),
                 np.array([0.0071], np.float32), np.array([1.19], np.float32))
    got = synth.bf16_bits_to_f32(x)[0]
    for j in range(0, 300, 2):
        a = float(x0[0, j])
        y = np.float32(a / np.float32(1.19)) if a >= 0 else np.float32(a * np.float32(1.19))
        y = np.float32(y - np.float32(0.013))
        y = np.float32(y - np.float32(np.float32(0.0071) * np.float32(1)))
        # candidates: the two bf16 values around y; the stored one must be the nearer
        # (the even one when exactly halfway)
        lo = np.float32(np.frombuffer((np.float32(y).view(np.uint32) & 0xFFFF0000).tobytes(), np.float32)[0])
        step = np.float32(np.frombuffer(((np.float32(lo).view(np.uint32) + 0x10000)).tobytes(), np.float32)[0])
        cands = sorted({float(lo), float(step)}, key=lambda c: (abs(c - float(y)),
                       (np.float32(c).view(np.uint32) >> 16) & 1))
        assert float(got[j]) == cands[0]


def test_penalty_bad_params_and_ids(orc):
    x = synth.random_rows(3, 4, 50)
    x0 = x.copy()
    ids, off = _pen_csr([[1, 2], [1, -1, 50], [3], [4]])
    st = orc.penalize(x, 50, ids, off, None, None, np.array([0, 0, float("nan"), 0], np.float32),
                      None, np.array([0.0, 1.2, 1.2, -1.0], np.float32))
    assert st.tolist() == [1, 4, 1, 1]
    assert np.array_equal(x[0], x0[0]) and np.array_equal(x[2], x0[2]) and np.array_equal(x[3], x0[3])
    assert x[1, 1] != x0[1, 1]


# ---------------------------------------------------------------- truncation
def _sample1(orc, logits, T, k, p, mp, seed=1, V=None):
    x = np.ascontiguousarray(np.atleast_2d(np.asarray(logits, np.float32)))
    B, n = x.shape
    V = V or n
    return orc.sample(x, V, np.full(B, T, np.float32), np.full(B, k, np.int32),
                      np.full(B, p, np.float32), np.full(B, mp, np.float32),
                      np.arange(seed, seed + B, dtype=np.uint64), want_mask=True)


def test_truncation_hand_cases(orc):
    g = _golden("truncation_hand.json")
    for c in g["cases"]:
        logits = np.log(np.array(c["probs"], np.float64)).astype(np.float32)
        out = _sample1(orc, logits, c["temperature"], c["top_k"], c["top_p"], c["min_p"])
        kept = np.nonzero(out["mask"][0])[0].tolist()
        assert kept == c["kept"], c["name"]
        assert out["kept"][0] == len(c["kept"])
        assert out["ids"][0] in c["kept"]


def test_greedy_triggers(orc):
    x = np.array([1.0, 3.0, 3.0, 2.0, -1.0], np.float32)
    for T, k, p, mp in [(0.0, 0, 0.9, 0.0), (1.0, 1, 0.9, 0.0), (1.0, 0, 0.0, 0.0),
                        (1.0, 0, 0.9, 1.0), (0.0, 5, 0.5, 0.5)]:
        out = _sample1(orc, x, T, k, p, mp)
        assert out["ids"][0] == 1 and out["kept"][0] == 1 and out["status"][0] == 0


def test_unset_parameters(orc):
    """Arrays left out take neutral values (T 1, top_k 0, top_p 1, min_p 0,
    seed 0); temperature, top_k and top_p all left out make the row greedy
    (TensorRT-LLM "Sampling", LLM API sampling behavior: none of the three
    set means greedy)."""
    x = np.array([[1.0, 3.0, 3.0, 2.0, -1.0]], np.float32)
    out = orc.sample(x, 5, None, None, None, None, None, want_mask=True)
    assert out["ids"][0] == 1 and out["kept"][0] == 1 and out["status"][0] == 0
    assert out["mask"][0].tolist() == [0, 1, 0, 0, 0]
    # one of the three given: the others neutral, untruncated (every id kept)
    out = orc.sample(x, 5, np.ones(1, np.float32), None, None, None, None, want_mask=True)
    assert out["kept"][0] == 5 and out["mask"][0].all()
    out = orc.sample(x, 5, None, np.array([2], np.int32), None, None, None, want_mask=True)
    assert out["kept"][0] == 2 and out["mask"][0].tolist() == [0, 1, 1, 0, 0]
    explicit = orc.sample(x, 5, np.ones(1, np.float32), np.array([2], np.int32),
                          np.ones(1, np.float32), np.zeros(1, np.float32), np.zeros(1, np.uint64))
    assert out["ids"][0] == explicit["ids"][0]  # seed 0 when left out


def _brute_rank(s):
    """rank_j = #{i : s_i > s_j or (s_i == s_j and i < j)} by pairwise counting."""
    n = len(s)
    return np.array([sum(1 for i in range(n) if s[i] > s[j] or (s[i] == s[j] and i < j))
                     for j in range(n)])


@pytest.mark.parametrize("kind", ["rank", "ties", "normal"])
def test_topk_matches_pairwise_ranks(orc, kind):
    for seed in range(6):
        x = synth.random_rows(100 + seed, 1, 48, kind=kind)[0]
        for T in (1.0, 0.7, 3.0):
            s = (x / np.float32(T)).astype(np.float32)
            rk = _brute_rank(s)
            for k in (2, 5, 13, 47, 48):
                out = _sample1(orc, x, T, k, 1.0, 0.0, seed=seed)
                want = (rk < min(k, 48)).astype(np.uint8)
                assert np.array_equal(out["mask"][0], want)
                assert out["mask"][0][out["ids"][0]] == 1


def test_topp_matches_subset_brute_force(orc):
    """Kept set = the smallest set of highest-probability tokens (lowest ids
    first within a tie) whose probability reaches top_p, found by enumerating
    subsets with float64 probabilities; cases whose masses sit within 1e-6 of the
    threshold are skipped."""
    checked = 0
    rng = np.random.default_rng(7)
    for trial in range(60):
        V = int(rng.integers(3, 10))
        x = (rng.standard_normal(V) * 1.5).astype(np.float32)
        if trial % 3 == 0:
            x[rng.integers(0, V)] = x[0]  # a tie
        p = float(np.float32(rng.uniform(0.05, 0.99)))
        k = int(rng.choice([0, 2, 3, V]))
        mp = float(np.float32(rng.choice([0.0, 0.2])))
        probs = np.exp(x.astype(np.float64) - x.max())
        rk = _brute_rank(x)
        n0 = k if 0 < k < V else V
        S = [j for j in range(V) if rk[j] < n0 and probs[j] >= mp]
        tot = probs[S].sum()
        best = None
        for size in range(1, len(S) + 1):
            for sub in itertools.combinations(S, size):
                outside = [j for j in S if j not in sub]
                if any(rk[o] < rk[i] for o in outside for i in sub):
                    continue  # not a top set in the order
                if probs[list(sub)].sum() >= p * tot:
                    best = sorted(sub)
                    break
            if best is not None:
                break
        cums = np.cumsum(sorted(probs[S], reverse=True)) / tot
        if np.min(np.abs(cums - p)) < 1e-6:
            continue
        out = _sample1(orc, x, 1.0, k, p, mp, seed=trial)
        assert np.nonzero(out["mask"][0])[0].tolist() == best, (trial, x, p, k, mp)
        checked += 1
    assert checked > 40


def test_pipeline_invariants_random_rows(orc):
    B, V = 24, 3000
    x = synth.random_rows(11, B, V, kind="rank")
    rng = np.random.default_rng(3)
    T = rng.uniform(0.3, 2.0, B).astype(np.float32)
    k = rng.choice([0, 1, 5, 50, 400], B).astype(np.int32)
    p = rng.uniform(0.1, 1.0, B).astype(np.float32)
    mp = rng.choice([0.0, 0.01, 0.3], B).astype(np.float32)
    out = orc.sample(x, V, T, k, p, mp, np.arange(B, dtype=np.uint64), want_mask=True)
    for r in range(B):
        if k[r] == 1:
            assert out["ids"][r] == int(np.argmax(x[r]))
            continue
        s = (x[r] / T[r]).astype(np.float32)
        order = np.lexsort((np.arange(V), -s))       # numpy's sort, not the oracle's
        m = out["mask"][r]
        n = int(m.sum())
        assert n == out["kept"][r] >= 1
        assert m[order[:n]].all()                      # kept set is a prefix of the order
        if k[r] > 0:
            assert n <= k[r]
        e = np.exp(s.astype(np.float64) - s.max())
        assert (e[m == 1] >= mp[r] * (1 - 1e-6)).all()
        assert m[out["ids"][r]] == 1


def test_gumbel_frequencies_follow_renormalised_softmax(orc):
    """The distribution check (vllm.cpp #1997, 'Red before green': the large-N
    empirical frequency case owns the score formula prob / q)."""
    V, N = 8, 100000
    probs = np.array([8, 7, 6, 5, 4, 3, 2, 1], np.float64)
    probs /= probs.sum()
    row = np.log(probs).astype(np.float32)
    x = np.tile(row, (N, 1))
    for k, p in [(0, 1.0), (4, 1.0), (0, 0.6)]:
        out = orc.sample(x, V, np.ones(N, np.float32), np.full(N, k, np.int32),
                         np.full(N, p, np.float32), np.zeros(N, np.float32),
                         np.arange(N, dtype=np.uint64) * 7919 + 11)
        counts = np.bincount(out["ids"], minlength=V)
        keep = np.zeros(V, bool)
        keep[: (k if k else V)] = True
        if p < 1:
            keep[:] = np.cumsum(probs) - probs < p   # 0.22, 0.42, 0.61 -> 3 kept
        q = np.where(keep, probs, 0.0)
        q /= q.sum()
        assert counts[~keep].sum() == 0
        exp_c = q[keep] * N
        chi2 = ((counts[keep] - exp_c) ** 2 / exp_c).sum()
        assert chi2 < 30, (k, p, counts, exp_c)      # <= 7 dof, far beyond the 99.99% point


def test_gumbel_top_two_scores_brute_force(orc):
    """The two best Gumbel scores the oracle reports (they decide which rows are
    near-ties, exempt from the id comparison) against a brute force over the
    kept set: every kept id's score e / (-log u) from the pinned exponential and
    uniform, sorted by numpy. The drawn id is the lowest id of the best score
    (vllm.cpp #1997, 'The kernel (#1984)': score = prob / q, argmax with ties to
    the lowest index); a row of one kept id reports no scores (-1, -1)."""
    rng = np.random.default_rng(41)
    B, V = 60, 48
    x = np.concatenate([synth.random_rows(42, 20, V, kind="rank"),
                        synth.random_rows(43, 20, V, kind="normal"),
                        synth.random_rows(44, 20, V, kind="flat")])
    T = rng.choice([1.0, 0.5, 1.7], B).astype(np.float32)
    k = rng.choice([0, 2, 3, 10, 30], B).astype(np.int32)
    p = rng.choice([1.0, 0.9, 0.5, 0.05], B).astype(np.float32)
    mp = rng.choice([0.0, 0.0, 0.1], B).astype(np.float32)
    seeds = rng.integers(0, 2**63, B, dtype=np.int64).astype(np.uint64)
    out = orc.sample(x, V, T, k, p, mp, seeds, want_mask=True)
    seen_two = 0
    for r in range(B):
        kept = np.nonzero(out["mask"][r])[0]
        assert len(kept) == out["kept"][r] >= 1
        if len(kept) == 1:
            assert out["ids"][r] == kept[0]
            assert out["top2"][r].tolist() == [-1.0, -1.0]
            continue
        s = (x[r] / T[r]).astype(np.float32)
        m = s.max()
        sc = np.array([orc.exp_pinned(np.float32(s[j] - m)) / -math.log(orc.uniform(int(seeds[r]), r, int(j)))
                       for j in kept])
        order = np.lexsort((kept, -sc))            # best score first, lower id first
        assert out["ids"][r] == kept[order[0]]
        assert out["top2"][r, 0] == sc[order[0]]
        assert out["top2"][r, 1] == sc[order[1]]
        seen_two += 1
    assert seen_two >= B // 2


# ---------------------------------------------------------------- status rows
def test_invalid_rows(orc):
    V = 16
    x = synth.random_rows(1, 6, V)
    x[1, 3] = np.nan
    x[2, 5] = np.inf
    x[3, :] = -np.inf
    T = np.array([1, 1, 1, 1, -1, 1], np.float32)
    k = np.array([0, 0, 0, 0, 0, 0], np.int32)
    out = orc.sample(x, V, T, k, np.ones(6, np.float32), np.zeros(6, np.float32),
                     np.zeros(6, np.uint64))
    assert out["status"].tolist() == [0, 2, 2, 2, 1, 0]
    assert out["ids"].tolist()[1:5] == [-1, -1, -1, -1]
    # top-k beyond the supported 1024 (but below V) is rejected; k >= V means no top-k
    x = synth.random_rows(2, 2, 3000)
    out = orc.sample(x, 3000, np.ones(2, np.float32), np.array([1025, 3000], np.int32),
                     np.ones(2, np.float32), np.zeros(2, np.float32), np.zeros(2, np.uint64))
    assert out["status"].tolist() == [8, 0] and out["kept"][1] == 3000
    # x / T overflowing to +inf is a bad parameter
    x = np.array([[3e38, 1.0]], np.float32)
    out = _sample1(orc, x, 1e-3, 0, 1.0, 0.0)
    assert out["status"][0] == 1 and out["ids"][0] == -1
    # -inf logits are allowed and never kept by top-p
    x = np.array([[0.0, -np.inf, 1.0, -np.inf]], np.float32)
    out = _sample1(orc, x, 1.0, 0, 0.999, 0.0)
    assert out["status"][0] == 0 and out["mask"][0].tolist() == [1, 0, 1, 0]


# ---------------------------------------------------------------- log-softmax
def test_logsoftmax_closed_forms(orc):
    V = 1000
    x = np.full((1, V), 2.5, np.float32)
    out = orc.logprobs(x, V, np.array([7], np.int32), k=3, full=True)
    assert np.allclose(out["full"][0], -math.log(V), atol=1e-12)
    assert out["topk_ids"][0].tolist() == [0, 1, 2]
    # two levels: na values a, nb values b
    na, nb, a, b = 3, 997, 4.0, -1.0
    x = np.full((1, V), b, np.float32)
    x[0, [10, 500, 999]] = a
    out = orc.logprobs(x, V, np.array([500], np.int32), k=4, full=True)
    lse = a + math.log(na + nb * math.exp(b - a))
    assert abs(out["token_lp"][0] - (a - lse)) < 1e-12
    assert out["topk_ids"][0].tolist() == [10, 500, 999, 0]
    assert abs(out["topk_lp"][0][3] - (b - lse)) < 1e-12


def test_logsoftmax_normalised_and_topk_brute(orc):
    x = synth.random_rows(21, 4, 64, kind="ties")
    out = orc.logprobs(x, 64, np.array([0, 1, 2, 63], np.int32), k=10, full=True)
    for r in range(4):
        lp = out["full"][r]
        assert abs(math.fsum(np.exp(lp)) - 1.0) < 1e-12
        rk = _brute_rank(x[r])
        assert out["topk_ids"][r].tolist() == [int(np.nonzero(rk == i)[0][0]) for i in range(10)]
    x = np.array([[0.0, -np.inf, 1.0]], np.float32)
    out = orc.logprobs(x, 3, np.array([1], np.int32), k=3, full=True)
    assert out["token_lp"][0] == -np.inf and out["topk_ids"][0].tolist() == [2, 0, 1]


def test_logsoftmax_at_temperature(orc):
    """Processed log-probs (vs_logprobs_ex): T = 1, T <= 0 and NaN give the plain
    log-softmax bit for bit; logits doubled at T = 2 give exactly the plain
    result (2x / 2 = x in fp32); a two-level row matches its closed form; an
    overflow of x / T makes the row invalid."""
    rng = np.random.default_rng(41)
    B, V = 5, 700
    x = (rng.normal(0, 3, (B, V))).astype(np.float32)
    plain = orc.logprobs(x, V, k=7, full=True)
    for T in (1.0, 0.0, -2.0, float("nan")):
        got = orc.logprobs(x, V, k=7, full=True, temperature=np.full(B, T, np.float32))
        assert np.array_equal(got["full"], plain["full"]) and np.array_equal(got["topk_ids"], plain["topk_ids"]), T
    doubled = orc.logprobs(2 * x, V, k=7, full=True, temperature=np.full(B, 2.0, np.float32))
    assert np.array_equal(doubled["full"], plain["full"])
    assert np.array_equal(doubled["topk_ids"], plain["topk_ids"])
    # two levels a (n1 ids) and b (n2 ids): lp_a = -log(n1 + n2 exp((b - a) / T))
    a, b, n1, T = 3.0, 1.0, 4, 0.5
    row = np.full((1, V), b, np.float32)
    row[0, :n1] = a
    o = orc.logprobs(row, V, full=True, temperature=np.array([T], np.float32))
    want_a = -np.log(n1 + (V - n1) * np.exp((b - a) / T))
    assert abs(o["full"][0, 0] - want_a) < 1e-12
    assert abs(o["full"][0, -1] - (want_a + (b - a) / T)) < 1e-12
    big = np.full((1, V), 1.0, np.float32)
    big[0, 3] = 3e38
    o = orc.logprobs(big, V, k=1, temperature=np.array([1e-3], np.float32))
    assert o["status"][0] == 2 and o["topk_ids"][0, 0] == -1


def test_logsoftmax_bad_rows(orc):
    x = np.array([[0.0, np.nan], [-np.inf, -np.inf], [1.0, 2.0]], np.float32)
    out = orc.logprobs(x, 2, np.array([0, 0, 5], np.int32), k=1)
    assert out["status"].tolist() == [2, 2, 4]
    assert np.isnan(out["token_lp"]).all()
