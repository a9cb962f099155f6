"""GPU parity of the per-row state updates between decode steps (vs_topp_decay,
vs_seed_advance) against the oracle, bit-exact, and a short decode loop that
chains vs_sample with both updates."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import compare_sample, dev, gpu_sample, oracle_sample, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_token_sampling_amd as vs
    vs.load()
    oracle.build(force=False)


def test_topp_decay_parity_over_steps():
    import decode_token_sampling_amd as vs
    rng = np.random.default_rng(21)
    B = 1000
    p0 = rng.uniform(0.0, 1.0, B).astype(np.float32)
    p0[::9] = 1.0
    decay = rng.uniform(0.3, 1.0, B).astype(np.float32)
    floor = rng.uniform(1e-6, 0.4, B).astype(np.float32)
    reset = rng.integers(-1, 20, B).astype(np.int32)
    decay[5], floor[6], reset[7], p0[8] = 0.0, 1.5, -3, 2.0  # rejected rows
    state = p0.copy()
    sd = dev(state, np.float32)
    args = [dev(p0, np.float32), dev(decay, np.float32)]
    for step in range(12):
        ids = rng.integers(-1, 20, B).astype(np.int32)
        st = vs.topp_decay(sd, *args, dev(ids, np.int32), top_p_min=dev(floor, np.float32),
                           reset_ids=dev(reset, np.int32)).cpu().numpy()
        so = oracle.topp_decay(state, p0, decay, ids, top_p_min=floor, reset_ids=reset)
        assert np.array_equal(st, so), step
        assert np.array_equal(sd.cpu().numpy().view(np.uint32), state.view(np.uint32)), step
    # default floor and no reset ids
    s2 = p0.copy()
    sd2 = dev(s2, np.float32)
    ids = np.zeros(B, np.int32)
    for _ in range(30):
        vs.topp_decay(sd2, args[0], args[1], dev(ids, np.int32))
        oracle.topp_decay(s2, p0, decay, ids)
    assert np.array_equal(sd2.cpu().numpy().view(np.uint32), s2.view(np.uint32))


def test_seed_advance_parity():
    import decode_token_sampling_amd as vs
    rng = np.random.default_rng(22)
    B = 777
    seeds = rng.integers(0, 2**63, B, dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    seeds[:3] = [0, 2**64 - 1, 2**63]
    sd = dev(seeds.view(np.int64), np.int64)
    for step in range(5):
        ids = rng.integers(-1, 3, B).astype(np.int32)
        vs.seed_advance(sd, dev(ids, np.int32))
        oracle.seed_advance(seeds, ids)
        assert np.array_equal(sd.cpu().numpy().view(np.uint64), seeds), step
    vs.seed_advance(sd)
    oracle.seed_advance(seeds)
    assert np.array_equal(sd.cpu().numpy().view(np.uint64), seeds)


def test_decode_loop_with_state():
    """Four decode steps: draw with the current top-p state and seeds, then decay
    the state and advance the seeds from the step's ids. Every step matches the
    oracle's loop (ids, kept sets, status); the state updates take the GPU's ids
    so that an exempt near-tie row cannot desynchronise the two loops."""
    import decode_token_sampling_amd as vs
    rng = np.random.default_rng(23)
    B, V = 24, 6000
    x = synth.random_rows(24, B, V, kind="rank")
    xd = to_device(x)
    T = rng.choice([1.0, 0.8, 1.2], B).astype(np.float32)
    T[0] = 0.0                                   # greedy takes precedence over the decay
    k = np.where(np.arange(B) % 3 == 0, 40, 0).astype(np.int32)
    p0 = np.ones(B, np.float32)                  # active decay with top_p 1: starts at 1
    p0[1::2] = 0.95
    decay = np.full(B, 0.8, np.float32)
    floor = np.full(B, 0.3, np.float32)
    reset = rng.integers(0, 50, B).astype(np.int32)
    seeds = (1000 + np.arange(B)).astype(np.uint64)
    state = p0.copy()
    sd, seedd = dev(state, np.float32), dev(seeds.view(np.int64), np.int64)
    mp = np.zeros(B, np.float32)
    near = 0
    for step in range(4):
        w = dict(temperature=T, top_k=k, top_p=state.copy(), min_p=mp, seeds=seeds.copy())
        g = gpu_sample(xd, V, w)
        assert np.array_equal(sd.cpu().numpy().view(np.uint32), state.view(np.uint32))
        assert np.array_equal(seedd.cpu().numpy().view(np.uint64), seeds)
        o = oracle_sample(x, V, w)
        near += compare_sample(g, o)
        ids = dev(g["ids"], np.int32)
        vs.topp_decay(sd, dev(p0, np.float32), dev(decay, np.float32), ids,
                      top_p_min=dev(floor, np.float32), reset_ids=dev(reset, np.int32))
        vs.seed_advance(seedd, ids)
        oracle.topp_decay(state, p0, decay, g["ids"], top_p_min=floor, reset_ids=reset)
        oracle.seed_advance(seeds, g["ids"])
    assert near <= 2


def test_slot_remap_parity():
    import decode_token_sampling_amd as vs
    rng = np.random.default_rng(25)
    for B, B_src, dt in [(300, 300, np.uint64), (257, 400, np.float32), (64, 10, np.int32)]:
        remap = rng.integers(-1, B_src + 2, B).astype(np.int32)
        src = rng.integers(0, 2**31, B_src).astype(dt) if dt != np.float32 else rng.random(B_src).astype(dt)
        dst = np.zeros(B, dt) + dt(3)
        tdt = {np.uint64: torch.int64, np.float32: torch.float32, np.int32: torch.int32}[dt]
        sv = torch.from_numpy(src.view(np.int64) if dt == np.uint64 else src).cuda()
        dv = torch.from_numpy(dst.view(np.int64) if dt == np.uint64 else dst.copy()).cuda()
        st = vs.slot_remap(dev(remap, np.int32), sv, dv).cpu().numpy()
        so = oracle.slot_remap(remap, src, dst)
        assert np.array_equal(st, so)
        got = dv.cpu().numpy()
        assert np.array_equal(got.view(np.uint8), dst.view(np.uint8)), (B, B_src, dt)
        assert sv.dtype == tdt
