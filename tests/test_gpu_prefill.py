"""GPU parity of the prefill (vv_prefill, the decoder_init contract) against the oracle's prefill:
the present K/V of every prompt position of every layer, the untouched rest of the cache, the last
position's logits and its greedy token; then decode steps continuing from the prefilled cache
against the oracle's decode steps from its own prefilled cache."""
import dataclasses

import numpy as np
import pytest

from oracle import vv_oracle as O
from int4_blockwise_gemv_amd import synth
from gpu_util import dev, host, rel_err
from helpers import oracle_model

pytestmark = pytest.mark.gpu
TOL = 2e-3
TINY = synth.TinyShape(layers=2, hidden=256, n_q=4, n_kv=2, head_dim=128, inter=512, vocab=1000)


def _prompt(shape, seed, S):
    return synth.fp16_normal(seed, synth.GLOBAL_LAYER, synth.T_X, (S, shape.hidden))


class PrefillCase:
    def __init__(self, shape, seed, layer_ids, S, cap, kv="f16"):
        from int4_blockwise_gemv_amd.model import DeviceModel, DeviceState
        self.shape, self.seed, self.layer_ids, self.S, self.cap = shape, seed, list(layer_ids), S, cap
        self.kv_np = np.float32 if kv == "f32" else np.float16
        self.glob = synth.model_globals(shape, seed, 1)
        self.dm = DeviceModel(shape, seed, self.layer_ids, max_batch=1, lm=self.glob["lm"], gf=self.glob["gf"])
        self.ds = DeviceState(self.dm, 1, cap, kv=kv)
        self.emb = _prompt(shape, seed, S)

    def run(self):
        import torch
        print(f"prefill {self.shape.name} layers {self.layer_ids} S={self.S} cap={self.cap}", flush=True)
        self.ds.prefill(dev(self.emb))
        torch.cuda.synchronize()

    def oracle(self):
        m = oracle_model(self.shape, self.seed, self.layer_ids, glob=self.glob)
        s = self.shape
        Kp = [np.zeros((s.n_kv, self.cap, s.head_dim), self.kv_np) for _ in self.layer_ids]
        Vp = [np.zeros((s.n_kv, self.cap, s.head_dim), self.kv_np) for _ in self.layer_ids]
        logits, tok, gap = O.prefill(m, self.emb, Kp, Vp)
        return m, logits, tok, gap, Kp, Vp


def _check_token(tok, logits):
    i, gap = O.argmax_with_gap(logits)
    if gap >= 1e-3:
        assert int(tok) == i, (int(tok), i, gap)
    else:
        assert int(tok) in set(int(t) for t in np.argsort(logits)[-2:])


def _compare(case, ref):
    _, logits, tok, gap, Kp, Vp = ref
    gl = host(case.ds.logits)[0].astype(np.float64)
    e = rel_err(gl, logits)
    print(f"last-position logits rel err {e:.2e} (top-2 gap {gap:.2e})")
    assert e <= TOL
    _check_token(host(case.ds.token)[0], logits)
    gk = host(case.ds.k).astype(np.float64)
    gv = host(case.ds.v).astype(np.float64)
    S = case.S
    for i in range(len(case.layer_ids)):
        ek = rel_err(gk[i, 0][:, :S], Kp[i][:, :S])
        ev = rel_err(gv[i, 0][:, :S], Vp[i][:, :S])
        print(f"layer {case.layer_ids[i]}: K rel err {ek:.2e}, V rel err {ev:.2e}")
        assert ek <= TOL and ev <= TOL
        # every position is checked on its own scale too (early positions are not drowned out)
        for t in sorted({0, S // 2, S - 1}):
            assert rel_err(gk[i, 0][:, t], Kp[i][:, t]) <= TOL
            assert rel_err(gv[i, 0][:, t], Vp[i][:, t]) <= TOL
        assert not np.any(gk[i, 0][:, S:]) and not np.any(gv[i, 0][:, S:])   # the rest stays zero


@pytest.mark.parametrize("S", [1, 2, 17, 64, 130, 200])
def test_prefill_tiny(cuda, S):
    """Prompt lengths on both sides of the 16-token MFMA groups, the 128-token GEMM blocks and the
    64-position attention splits."""
    case = PrefillCase(TINY, 0, range(2), S, S + 8)
    case.run()
    _compare(case, case.oracle())


def test_prefill_tiny_absmax_group7(cuda):
    """General int4 (per-block absmax scales) and 7 query heads per KV head."""
    shp = dataclasses.replace(TINY, n_q=7, n_kv=1, mode="absmax", name="tiny-absmax-g7")
    case = PrefillCase(shp, 2, range(2), 77, 96)
    case.run()
    _compare(case, case.oracle())


def test_prefill_zero_layers(cuda):
    shp = dataclasses.replace(TINY, layers=0, name="tiny-0")
    case = PrefillCase(shp, 3, [], 5, 8)
    case.run()
    m, logits, tok, gap, _, _ = case.oracle()
    assert rel_err(host(case.ds.logits)[0].astype(np.float64), logits) <= TOL
    _check_token(host(case.ds.token)[0], logits)


@pytest.mark.parametrize("S", [300, 700])
@pytest.mark.timeout(600)
def test_prefill_1p5b_width(cuda, S):
    """Two layers at 1.5B width (H 1536, 12/2 heads, I 8960); 700 tokens take two attention
    launches of the token chunking."""
    case = PrefillCase(synth.QWEN2_1P5B, 0, [0, 27], S, S + 64)
    case.run()
    _compare(case, case.oracle())


@pytest.mark.timeout(600)
def test_prefill_7b_width(cuda):
    """One layer at 7B width (H 3584, 28/4 heads, I 18944)."""
    case = PrefillCase(synth.QWEN2_7B, 1, [5], 160, 200)
    case.run()
    _compare(case, case.oracle())


@pytest.mark.parametrize("S", [17, 130])
def test_prefill_tiny_fp32_kv(cuda, S):
    """The fp32-KV variant: k and v written to fp32 caches unrounded."""
    case = PrefillCase(TINY, 7, range(2), S, S + 8, kv="f32")
    case.run()
    _compare(case, case.oracle())


@pytest.mark.parametrize("kv", ["f16", "f32"])
def test_prefill_then_decode(cuda, kv):
    """decoder_init then decoder_step: decode steps at positions S, S+1, S+2 over the prefilled
    cache equal the oracle's decode steps over its own prefilled cache."""
    import torch
    S, cap = 40, 48
    case = PrefillCase(TINY, 5, range(2), S, cap, kv=kv)
    case.run()
    m, _, _, _, Kp, Vp = case.oracle()
    Kc = [k[None].copy() for k in Kp]
    Vc = [v[None].copy() for v in Vp]
    nxt = synth.fp16_normal(6, synth.GLOBAL_LAYER, synth.T_X, (3, TINY.hidden))
    for i in range(3):
        case.ds.emb.copy_(dev(nxt[i:i + 1]))
        case.ds.pos.fill_(S + i)
        case.ds.step()
        torch.cuda.synchronize()
        logits, tok, gap, _ = O.decode_step(m, nxt[i:i + 1], np.array([S + i]), Kc, Vc)
        e = rel_err(host(case.ds.logits)[0].astype(np.float64), logits[0])
        print(f"decode at {S + i}: logits rel err {e:.2e}")
        assert e <= TOL
        _check_token(host(case.ds.token)[0], logits[0])


def test_prefill_deterministic(cuda):
    import torch
    case = PrefillCase(TINY, 4, range(2), 90, 96)
    case.run()
    k1, l1 = host(case.ds.k).copy(), host(case.ds.logits).copy()
    case.ds.k.zero_()
    case.ds.v.zero_()
    case.run()
    assert np.array_equal(host(case.ds.k), k1) and np.array_equal(host(case.ds.logits), l1)


@pytest.mark.timeout(900)
def test_prefill_7b_full_prompt(cuda):
    """The benchmarked prompt length at 7B width: one layer, S = 2048 (32 query blocks of the causal
    attention, 32 token blocks of the GEMMs), every position's K/V and the last logits against the
    oracle."""
    import time
    case = PrefillCase(synth.QWEN2_7B, 0, [3], 2048, 2048)
    case.run()
    t = time.time()
    ref = case.oracle()
    print(f"oracle prefill {time.time() - t:.1f} s")
    _compare(case, ref)


@pytest.mark.timeout(600)
def test_prefill_0p5b_width(cuda):
    """Two layers at the 0.5B width (H 896 = 28 blocks: the GEMMs over K = H end on a partial group of
    4 blocks; 14/2 heads, I 4864)."""
    case = PrefillCase(synth.QWEN2_0P5B, 2, [0, 19], 300, 320)
    case.run()
    _compare(case, case.oracle())


@pytest.mark.timeout(600)
def test_prefill_1p5b_width_fp32_kv(cuda):
    """fp32 caches at 1.5B width: the causal attention reads K and V as fp16 hi + lo parts."""
    case = PrefillCase(synth.QWEN2_1P5B, 1, [0, 27], 300, 364, kv="f32")
    case.run()
    _compare(case, case.oracle())


def test_prefill_workspace_reused_for_a_shorter_prompt(cuda):
    """One state (and so one prefill workspace, sized by the first, longer prompt) serves a 64-token
    prompt and then a 17-token one: the argmax keys sit at an offset that does not depend on S, so
    the second call finds them cleared, and both results match the oracle."""
    import torch
    case = PrefillCase(TINY, 12, range(2), 64, 96)
    case.run()
    _compare(case, case.oracle())
    short = PrefillCase.__new__(PrefillCase)
    short.__dict__.update(case.__dict__)
    short.S = 17
    short.emb = _prompt(TINY, 13, 17)
    case.ds.k.zero_()
    case.ds.v.zero_()
    torch.cuda.synchronize()
    short.run()
    _compare(short, short.oracle())
