"""End-to-end parity of the benchmark workloads at full size, run as the benchmark runs them (the
captured graph of the step): the 1.5B-shaped step at P = 4096, the 7B-shaped step at P = 4000, the
7B shape with general int4 weights over a 16384-position cache with 1% outlier positions, and the
1.5B shape with 16 ragged sequences (past lengths 512..8192).

The oracle packs every layer itself from the seeded fp32 masters (in worker processes: the
oracle's packing is plain numpy and takes seconds per layer) and runs its own whole step from the
same input embeddings and caches.  Compared: the residual stream after every layer, the K/V each
layer writes at the new position (and the rest of every cache untouched), the logits and the
greedy token ("VibeVoice-1.5B — Current Status", Inference: incremental decoding reproduces the
full computation; "vibevoice-asr-bitnet-onnx", tier table: int4 tiers token-exact against the
reference)."""
import numpy as np
import pytest

from oracle import vv_oracle as O
from int4_blockwise_gemv_amd import synth
from gpu_util import STEP_PATHS, host, rel_err
from helpers import oracle_model, oracle_packs_parallel

pytestmark = pytest.mark.gpu
TOL = 2e-3
DRIFT_TOL = 1e-2

_PACKS = {}


def _packs(shape, seed):
    """Oracle packs of every layer, kept for the session (the 1.5B weights serve two workloads)."""
    key = (shape.name, seed)
    if key not in _PACKS:
        _PACKS.clear()
        _PACKS[key] = oracle_packs_parallel(shape, seed, range(shape.layers))
    return _PACKS[key]


def _check_tokens(tok, ref_logits):
    for b in range(ref_logits.shape[0]):
        i, gap = O.argmax_with_gap(ref_logits[b])
        if gap >= 1e-3:
            assert int(tok[b]) == i, (b, int(tok[b]), i, gap)
        else:
            top2 = np.argsort(ref_logits[b])[-2:]
            assert int(tok[b]) in set(int(t) for t in top2)


def _end_to_end(wl_name, seed, path):
    import torch
    from int4_blockwise_gemv_amd.model import DeviceModel, DeviceState
    wl = synth.WORKLOADS[wl_name]
    s = wl.shape
    lens = synth.past_lengths(wl, seed)
    glob = synth.model_globals(s, seed, wl.batch, with_lm=True)
    dm = DeviceModel(s, seed, max_batch=wl.batch, lm=glob["lm"], gf=glob["gf"])
    ds = DeviceState(dm, wl.batch, wl.cap, trace=True, logits=True, path=path)
    caches = []
    for li in range(s.layers):
        K, V = synth.layer_cache(wl, seed, li, lens)
        ds.load_cache_layer(li, K, V)
        caches.append((K, V))
    ds.emb.copy_(torch.from_numpy(glob["emb"].view(np.int16)).view(torch.float16).cuda())
    ds.pos.copy_(torch.from_numpy(lens).cuda())
    torch.cuda.synchronize()
    g = ds.graph()
    try:
        g.launch()
        torch.cuda.synchronize()
    finally:
        g.close()
    assert ds.status() == 0
    gtr = host(ds.trace).astype(np.float64)
    glog = host(ds.logits).astype(np.float64)
    gtok = host(ds.token)
    assert np.all(np.isfinite(gtr))

    m = oracle_model(s, seed, range(s.layers), glob=glob, packs=_packs(s, seed))
    # (1) every layer on the GPU's own input residual: the layer's GEMV and attention outputs on
    #     identical inputs (the output residual and the K/V written at the new position)
    local = 0.0
    for li in range(s.layers):
        K0, V0 = caches[li]
        Kl, Vl = K0.copy(), V0.copy()
        hl = O.layer_step(m.layers[li], m, gtr[li], lens, Kl, Vl)
        gk = host(ds.k[li]).astype(np.float64)
        gv = host(ds.v[li]).astype(np.float64)
        for b in range(wl.batch):
            p = int(lens[b])
            errs = (rel_err(gtr[li + 1][b], hl[b]), rel_err(gk[b, :, p], Kl[b, :, p]),
                    rel_err(gv[b, :, p], Vl[b, :, p]))
            local = max(local, *errs)
            assert max(errs) <= TOL, (li, b, errs)
            keep = np.ones(wl.cap, bool)
            keep[p] = False
            assert np.array_equal(gk[b][:, keep], K0[b][:, keep].astype(np.float64)), (li, b)
            assert np.array_equal(gv[b][:, keep], V0[b][:, keep].astype(np.float64)), (li, b)
        del gk, gv, Kl, Vl
    # (2) the whole step against the oracle's own step over all layers from the same embeddings:
    #     logits and token, the residual stream after every layer; the K/V written at every layer
    #     are reported (deep layers' K/V inherit the residual stream's drift over the layers before)
    Kc = [K.copy() for K, _ in caches]
    Vc = [V.copy() for _, V in caches]
    tr = {}
    logits, _, _, _ = O.decode_step(m, glob["emb"], lens, Kc, Vc, tr)
    drift = 0.0
    for li in range(s.layers + 1):
        for b in range(wl.batch):
            drift = max(drift, rel_err(gtr[li][b], tr["h"][li][b]))
    kv_drift = 0.0
    for li in range(s.layers):
        gk = host(ds.k[li]).astype(np.float64)
        gv = host(ds.v[li]).astype(np.float64)
        for b in range(wl.batch):
            p = int(lens[b])
            kv_drift = max(kv_drift, rel_err(gk[b, :, p], Kc[li][b, :, p]), rel_err(gv[b, :, p], Vc[li][b, :, p]))
        del gk, gv
    lerr = max(rel_err(glog[b], logits[b]) for b in range(wl.batch))
    print(f"{wl_name} seed {seed} [{path}]: layer-local worst {local:.2e}; whole step: residual drift {drift:.2e}, "
          f"K/V drift {kv_drift:.2e}, logits {lerr:.2e}")
    assert drift <= DRIFT_TOL and kv_drift <= DRIFT_TOL
    assert lerr <= TOL
    _check_tokens(gtok, logits)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("path", STEP_PATHS)
def test_end_to_end_1p5b_p4096(cuda, path):
    _end_to_end("decode-1.5b-p4096", 0, path)


@pytest.mark.timeout(600)
def test_end_to_end_1p5b_batch16_ragged(cuda):
    _end_to_end("decode-1.5b-b16-ragged", 0, "layered")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("path", STEP_PATHS)
def test_end_to_end_7b_p4000(cuda, path):
    _end_to_end("decode-7b-p4000", 0, path)


@pytest.mark.timeout(900)
def test_end_to_end_7b_absmax_p16384_outliers(cuda):
    _end_to_end("decode-7b-absmax-p16384", 0, "layered")
