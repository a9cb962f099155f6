"""A whole decode step captured in a HIP graph: penalties in place, the draw
with its log-probs, top-p decay and the seed advance. The library allocates
and synchronises nothing and records no memset, so the step is capturable;
the graph is replayed several times, with eager work between the replays, and
every replay is checked against an eager run of the same step from the same
inputs (ids, kept counts, status, penalised logits and state bit-exact;
log-probs within the tolerance, their summation order being free)."""
import numpy as np
import pytest
import torch

import synth
from parity import LOGPROB_ATOL, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_token_sampling_amd as vs
    vs.load()


def test_captured_decode_step_matches_eager():
    import decode_token_sampling_amd as vs
    rng = np.random.default_rng(31)
    B, V = 40, 50000
    x0 = torch.from_numpy(synth.random_rows(32, B, V, kind="rank")).cuda()
    pids, poff = synth._csr([synth.zipf_ids(rng, int(n), V) for n in rng.integers(0, 300, B)])
    oids, ooff = synth._csr([synth.zipf_ids(rng, int(n), V) for n in rng.integers(0, 100, B)])
    pen = [dev(pids, np.int32), dev(poff, np.int32), dev(oids, np.int32), dev(ooff, np.int32),
           dev(rng.uniform(0, 0.5, B), np.float32), dev(rng.uniform(0, 0.2, B), np.float32),
           dev(rng.uniform(1.0, 1.3, B), np.float32)]
    T = dev(rng.choice([0.0, 0.7, 1.0, 1.3], B), np.float32)
    K = dev(rng.choice([0, 1, 20, 50, 200], B), np.int32)
    MP = dev(np.where(np.arange(B) % 5 == 0, 0.05, 0.0), np.float32)
    p_init = dev(rng.uniform(0.6, 1.0, B), np.float32)
    decay = dev(np.full(B, 0.9), np.float32)
    seeds0 = dev((7000 + np.arange(B)).astype(np.uint64).view(np.int64), np.int64)
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
    tids = torch.empty((B, 5), dtype=torch.int32, device="cuda")
    tlps = torch.empty((B, 5), dtype=torch.float32, device="cuda")

    def step():
        vs.penalize(x, *pen, row_status=pst)
        vs.sample_logprobs(x, T, K, p_state, MP, seeds, k=5, ws=ws, out_ids=ids, kept=kept,
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

    reset()
    step()
    want = snapshot()

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

    for rep in range(4):
        reset()
        torch.cuda.synchronize()
        graph.replay()
        got = snapshot()
        for k in ("x", "p", "seeds", "ids", "kept", "st", "pst", "dst", "tids"):
            assert torch.equal(got[k], want[k]), (rep, k)
        for k in ("tlp", "tlps"):
            a, b = got[k].cpu().numpy(), want[k].cpu().numpy()
            fin = np.isfinite(b)
            assert np.array_equal(np.isfinite(a), fin), (rep, k)
            assert np.abs(a[fin] - b[fin]).max() <= LOGPROB_ATOL, (rep, k)
        # eager work between replays
        reset()
        step()
        torch.cuda.synchronize()
