"""Closed-loop greedy decoding on the device: each step's argmax selects the next input embedding
from the tied fp16 table and advances the position, so that replays of one captured step graph
decode successive tokens with no host round trip.  Checked against the oracle running the same
greedy loop (its own argmax, the same table lookup and stop rule), token by token, up to the
first step whose top-2 logit gap falls under 1e-3 (after a near-tie either token is valid and the
two runs may part)."""
import numpy as np
import pytest

from oracle import vv_oracle as O
from int4_blockwise_gemv_amd import synth
from gpu_util import STEP_PATHS, host
from helpers import oracle_model

pytestmark = pytest.mark.gpu

TINY = synth.TinyShape(layers=2, hidden=256, n_q=4, n_kv=2, head_dim=128, inter=512, vocab=1000)


def _oracle_loop(m, table, emb, pos, K, V, steps, stops, cap):
    """The oracle's greedy loop: returns history [B][cap] (-1 = none), the step at which each
    sequence's comparison stops being binding (first near-tie), and the done flags."""
    B = len(pos)
    emb, pos = emb.copy(), np.array(pos, np.int64)
    hist = np.full((B, cap), -1, np.int64)
    done = np.zeros(B, bool)
    binding = np.full(B, steps)
    for t in range(steps):
        logits, tok, gap, _ = O.decode_step(m, emb, pos, K, V)
        for b in range(B):
            if gap[b] < 1e-3 and binding[b] == steps:
                binding[b] = t
            if done[b]:
                continue
            hist[b, pos[b]] = tok[b]
            if tok[b] in stops:
                done[b] = True
            elif pos[b] + 1 < cap:
                emb[b] = table[tok[b]]
                pos[b] += 1
    return hist, binding, done, pos


@pytest.mark.parametrize("path", STEP_PATHS)
def test_closed_loop_greedy_graph(cuda, path):
    import torch
    from int4_blockwise_gemv_amd.model import DeviceModel, DeviceState
    steps, cap = 8, 40
    pos0 = [5, 17, 0] if path == "layered" else [5]   # the chained path serves batch 1
    if path == "chained":
        cap = 80                                        # >= 2 attention splits
    B = len(pos0)
    w = synth.Workload("loop", TINY, B, max(pos0), cap, (3,))
    glob = synth.model_globals(TINY, 3, B, True)
    table = glob["lm"]
    m = oracle_model(TINY, 3, range(2), glob=glob)
    caches = [synth.layer_cache(w, 3, li, np.asarray(pos0)) for li in range(2)]
    # pick a stop id that sequence 0 actually emits (at its third step), so stopping is exercised
    Ks, Vs = [c[0].copy() for c in caches], [c[1].copy() for c in caches]
    free, _, _, _ = _oracle_loop(m, table, glob["emb"], pos0, Ks, Vs, steps, set(), cap)
    stop = int(free[0, pos0[0] + 2])
    stops = [stop, 151645]
    Ks, Vs = [c[0].copy() for c in caches], [c[1].copy() for c in caches]
    ref, binding, done_ref, pos_ref = _oracle_loop(m, table, glob["emb"], pos0, Ks, Vs, steps, set(stops), cap)

    dm = DeviceModel(TINY, 3, range(2), max_batch=B, lm=glob["lm"], gf=glob["gf"])
    ds = DeviceState(dm, B, cap, path=path)
    for li in range(2):
        ds.load_cache_layer(li, *caches[li])
    ds.emb.copy_(torch.from_numpy(glob["emb"].view(np.int16)).view(torch.float16).cuda())
    ds.pos.copy_(torch.from_numpy(np.asarray(pos0, np.int32)).cuda())
    ds.enable_feedback(stop_ids=stops)
    torch.cuda.synchronize()
    g = ds.graph()
    try:
        for _ in range(steps):
            g.launch()
        torch.cuda.synchronize()
    finally:
        g.close()
    assert ds.status() == 0
    hist = host(ds.history).astype(np.int64)
    for b in range(B):
        n = int(binding[b])
        want = [int(t) for t in ref[b] if t >= 0][:n]
        got = [int(t) for t in hist[b] if t >= 0][:n]
        assert got == want, (b, got, want)
        if n == steps:   # no near-tie on the way: the stop flags and final positions agree too
            assert bool(host(ds.done)[b]) == bool(done_ref[b])
            assert int(host(ds.pos)[b]) == int(pos_ref[b])
    if binding[0] == steps:
        assert done_ref[0] and host(ds.done)[0] == 1   # sequence 0 reached its stop token
