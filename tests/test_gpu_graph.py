"""A whole decode step captured in a HIP graph: penalties in place, the draw
with its log-probs, top-p decay and the seed advance. The library allocates
and synchronises nothing and records no memset, so the step is capturable.

The eager step is checked against the oracle's step (penalised logits, ids,
kept counts, status, decay state and seeds bit-exact; log-probs within 1e-5).
The graph is then replayed several times, with eager work between replays,
and every replay is checked against the eager step (ids, kept counts,
status, penalised logits and state bit-exact; log-probs within the tolerance,
their summation order being free) and so against the oracle. Finally the graph
is replayed three times in a row without resetting anything, a three-step
decode loop (each step penalises the logits again, draws with the decayed
top-p and the advanced seeds), and each step is compared with the oracle's
loop."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import LOGPROB_ATOL, compare_sample, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_token_sampling_amd as vs
    vs.load()
    oracle.build(force=False)


class OracleLoop:
    """The oracle's decode loop over the same host inputs."""

    def __init__(self, x0, hist, T, K, MP, p_init, decay, seeds0, k_lp):
        self.x = x0.copy()
        self.hist, self.T, self.K, self.MP = hist, T, K, MP
        self.p_init, self.decay = p_init, decay
        self.p = p_init.copy()
        self.seeds = seeds0.copy()
        self.k_lp = k_lp

    def step(self):
        B, V = self.x.shape
        pst = oracle.penalize(self.x, V, *self.hist)
        o = oracle.sample(self.x, V, self.T, self.K, self.p, self.MP, self.seeds)
        lp = oracle.logprobs(self.x, V, o["ids"], k=self.k_lp)
        out = dict(x=self.x.copy(), pst=pst, ids=o["ids"], kept=o["kept"], st=o["status"],
                   top2=o["top2"], tlp=lp["token_lp"], tids=lp["topk_ids"], tlps=lp["topk_lp"],
                   p_used=self.p.copy(), seeds_used=self.seeds.copy())
        out["dst"] = oracle.topp_decay(self.p, self.p_init, self.decay, o["ids"])
        oracle.seed_advance(self.seeds, o["ids"])
        out["p"] = self.p.copy()
        out["seeds"] = self.seeds.copy()
        return out


def _check_against_oracle(got, want, tag):
    assert np.array_equal(got["x"].cpu().numpy(), want["x"]), tag
    for key in ("pst", "dst"):
        assert np.array_equal(got[key].cpu().numpy(), want[key]), (tag, key)
    g = dict(ids=got["ids"].cpu().numpy(), kept=got["kept"].cpu().numpy(),
             status=got["st"].cpu().numpy())
    o = dict(ids=want["ids"], kept=want["kept"], status=want["st"], top2=want["top2"])
    assert compare_sample(g, o, check_mask=False) == 0, tag
    assert np.array_equal(got["p"].cpu().numpy(), want["p"]), tag
    assert np.array_equal(got["seeds"].cpu().numpy().view(np.uint64), want["seeds"]), tag
    assert np.array_equal(got["tids"].cpu().numpy(), want["tids"]), tag
    for key in ("tlp", "tlps"):
        a = got[key].cpu().numpy()
        assert np.isfinite(a).all() and a.shape == want[key].shape, (tag, key)
        assert np.abs(a - want[key]).max() <= LOGPROB_ATOL, (tag, key)


def test_captured_decode_step_matches_eager_and_oracle():
    import decode_token_sampling_amd as vs
    rng = np.random.default_rng(31)
    B, V, KLP = 40, 50000, 5
    x0h = synth.random_rows(32, B, V, kind="rank")
    pids, poff = synth._csr([synth.zipf_ids(rng, int(n), V) for n in rng.integers(0, 300, B)])
    oids, ooff = synth._csr([synth.zipf_ids(rng, int(n), V) for n in rng.integers(0, 100, B)])
    pres = rng.uniform(0, 0.5, B).astype(np.float32)
    freq = rng.uniform(0, 0.2, B).astype(np.float32)
    rep = rng.uniform(1.0, 1.3, B).astype(np.float32)
    Th = rng.choice([0.0, 0.7, 1.0, 1.3], B).astype(np.float32)
    Kh = rng.choice([0, 1, 20, 50, 200], B).astype(np.int32)
    MPh = np.where(np.arange(B) % 5 == 0, 0.05, 0.0).astype(np.float32)
    p_inith = rng.uniform(0.6, 1.0, B).astype(np.float32)
    decayh = np.full(B, 0.9, np.float32)
    seeds0h = (7000 + np.arange(B)).astype(np.uint64)

    x0 = torch.from_numpy(x0h).cuda()
    pen = [dev(pids, np.int32), dev(poff, np.int32), dev(oids, np.int32), dev(ooff, np.int32),
           dev(pres, np.float32), dev(freq, np.float32), dev(rep, np.float32)]
    T, K, MP = dev(Th, np.float32), dev(Kh, np.int32), dev(MPh, np.float32)
    p_init, decay = dev(p_inith, np.float32), dev(decayh, np.float32)
    seeds0 = dev(seeds0h.view(np.int64), np.int64)
    ws = vs.workspace(B, V, torch.float32, x0.device)

    # buffers the step reads and writes (fixed addresses for the graph)
    x = x0.clone()
    p_state = p_init.clone()
    seeds = seeds0.clone()
    ids = torch.empty(B, dtype=torch.int32, device="cuda")
    kept = torch.empty_like(ids)
    st = torch.empty_like(ids)
    pst = torch.empty_like(ids)
    dst = torch.empty_like(ids)
    tlp = torch.empty(B, dtype=torch.float32, device="cuda")
    tids = torch.empty((B, KLP), dtype=torch.int32, device="cuda")
    tlps = torch.empty((B, KLP), dtype=torch.float32, device="cuda")

    def step():
        vs.penalize(x, *pen, row_status=pst)
        vs.sample_logprobs(x, T, K, p_state, MP, seeds, k=KLP, ws=ws, out_ids=ids, kept=kept,
                           row_status=st, out_token_lp=tlp, out_topk_ids=tids, out_topk_lp=tlps)
        vs.topp_decay(p_state, p_init, decay, ids, row_status=dst)
        vs.seed_advance(seeds, ids)

    def reset():
        x.copy_(x0)
        p_state.copy_(p_init)
        seeds.copy_(seeds0)

    def snapshot():
        torch.cuda.synchronize()
        return {k: v.clone() for k, v in dict(x=x, p=p_state, seeds=seeds, ids=ids, kept=kept, st=st,
                                               pst=pst, dst=dst, tlp=tlp, tids=tids, tlps=tlps).items()}

    def oracle_loop():
        return OracleLoop(x0h, (pids, poff, oids, ooff, pres, freq, rep), Th, Kh, MPh, p_inith,
                          decayh, seeds0h, KLP)

    first = oracle_loop().step()
    reset()
    step()
    want = snapshot()
    _check_against_oracle(want, first, "eager")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset()
        step()  # warm the stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()

    for rep_i in range(4):
        reset()
        torch.cuda.synchronize()
        graph.replay()
        got = snapshot()
        for k in ("x", "p", "seeds", "ids", "kept", "st", "pst", "dst", "tids"):
            assert torch.equal(got[k], want[k]), (rep_i, k)
        for k in ("tlp", "tlps"):
            a, b = got[k].cpu().numpy(), want[k].cpu().numpy()
            fin = np.isfinite(b)
            assert np.array_equal(np.isfinite(a), fin), (rep_i, k)
            assert np.abs(a[fin] - b[fin]).max() <= LOGPROB_ATOL, (rep_i, k)
        _check_against_oracle(got, first, f"replay {rep_i}")
        # eager work between replays
        reset()
        step()
        torch.cuda.synchronize()

    # a three-step decode loop: replays back to back on the graph's own state
    loop = oracle_loop()
    reset()
    torch.cuda.synchronize()
    for t in range(3):
        graph.replay()
        got = snapshot()
        _check_against_oracle(got, loop.step(), f"loop step {t}")
