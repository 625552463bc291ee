"""GPU parity: split-KV GQA decode attention and the lm_head GEMV + argmax against the oracle."""
import math

import numpy as np
import pytest

from oracle import vv_oracle as O
from int4_blockwise_gemv_amd import synth
from gpu_util import dev, host, rel_err

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _gqa_gpu(q, K, V, lens, q_f16=False, out_f16=False):
    import torch
    from int4_blockwise_gemv_amd import vv
    B, nq, d = q.shape
    _, nkv, cap, _ = K.shape
    ws = torch.zeros(vv.gqa_workspace(B, nq, nkv, cap), dtype=torch.uint8, device="cuda")
    qd = dev(q.astype(np.float16) if q_f16 else q.astype(np.float32))
    out = torch.empty((B, nq, d), dtype=torch.float16 if out_f16 else torch.float32, device="cuda")
    vv.gqa_decode(qd, dev(K), dev(V), dev(np.asarray(lens, np.int32)), 1 / math.sqrt(d), out, ws)
    torch.cuda.synchronize()
    return host(out).astype(np.float64)


def _gqa_ref(q, K, V, lens):
    d = q.shape[-1]
    return np.stack([O.gqa_decode(q[b].astype(np.float64), K[b], V[b], int(lens[b]), 1 / math.sqrt(d))
                     for b in range(q.shape[0])])


@pytest.mark.parametrize("q_f16,out_f16", [(True, False), (False, True), (False, False)])
def test_gqa_single_layer_256(cuda, q_f16, out_f16):
    """One GQA decode step: 12 query heads, 2 KV heads, head_dim 128, cache length 256."""
    q = synth.fp16_normal(0, 0, synth.T_QATT, (1, 12, 128))
    K = synth.fp16_normal(0, 0, synth.T_KC, (1, 2, 256, 128))
    V = synth.fp16_normal(0, 0, synth.T_VC, (1, 2, 256, 128))
    ref = _gqa_ref(q, K, V, [256])
    got = _gqa_gpu(q, K, V, [256], q_f16, out_f16)
    assert rel_err(got, ref) <= TOL


def test_gqa_tiny_brute_shape(cuda):
    """2 KV heads, cache length 3 (the brute-force shape of the oracle pins)."""
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 4, 128)).astype(np.float32)
    K = rng.standard_normal((1, 2, 5, 128)).astype(np.float16)
    V = rng.standard_normal((1, 2, 5, 128)).astype(np.float16)
    assert rel_err(_gqa_gpu(q, K, V, [3]), _gqa_ref(q, K, V, [3])) <= 1e-5


@pytest.mark.parametrize("nq,nkv,cap,lens", [
    (28, 4, 4001, [4001]),            # 7B group of 7, P + 1 = 4001
    (12, 2, 4097, [1, 4097]),         # length 1 and full
    (12, 2, 700, [513, 1, 77, 700]),  # ragged batch
    (8, 8, 64, [64, 31]),             # group of 1
    (16, 2, 300, [300]),              # group of 8
    (8, 8, 17000, [17000, 5]),        # > 2048 workgroups at 64 positions: 128-position splits
    (8, 1, 65536, [65536, 3]),        # 1024 splits of 64 positions: the merge's 16 waves
    (8, 1, 131072, [131072]),         # largest capacity, one KV head: 1024 splits of 128
])
def test_gqa_shapes_and_ragged(cuda, nq, nkv, cap, lens):
    B = len(lens)
    q = synth.fp16_normal(1, B, synth.T_QATT, (B, nq, 128)).astype(np.float32)
    K = synth.fp16_normal(1, B, synth.T_KC, (B, nkv, cap, 128))
    V = synth.fp16_normal(1, B, synth.T_VC, (B, nkv, cap, 128))
    assert rel_err(_gqa_gpu(q, K, V, lens), _gqa_ref(q, K, V, lens)) <= TOL


def test_gqa_long_context_outliers(cuda):
    """16384 + 1 positions, 1% of positions scaled x8 (softmax range stress)."""
    w = synth.WORKLOADS["decode-7b-absmax-p16384"]
    lens = np.array([w.past], np.int32)
    K, V = synth.layer_cache(w, 0, 0, lens)
    q = synth.fp16_normal(0, 0, synth.T_QATT, (1, 28, 128)).astype(np.float32)
    assert rel_err(_gqa_gpu(q, K, V, lens), _gqa_ref(q, K, V, lens)) <= TOL


def test_gqa_constant_v_per_group(cuda):
    """A constant V per KV head comes back on exactly the query heads of its group."""
    q = synth.fp16_normal(3, 0, synth.T_QATT, (1, 12, 128)).astype(np.float32)
    K = synth.fp16_normal(3, 0, synth.T_KC, (1, 2, 100, 128))
    V = np.zeros((1, 2, 100, 128), np.float16)
    V[0, 0], V[0, 1] = 1.5, -2.0
    out = _gqa_gpu(q, K, V, [100])
    assert np.allclose(out[0, :6], 1.5, rtol=1e-6) and np.allclose(out[0, 6:], -2.0, rtol=1e-6)


# ---------------------------------------------------------------------------------------------
# lm_head + argmax
# ---------------------------------------------------------------------------------------------

def _lm_gpu(W, x, with_logits=True):
    import torch
    from int4_blockwise_gemv_amd import vv
    V, H = W.shape
    B = x.shape[0]
    ws = torch.zeros(vv.lm_workspace(B, V, H), dtype=torch.uint8, device="cuda")
    logits = torch.empty((B, V), dtype=torch.float32, device="cuda") if with_logits else None
    tok = torch.empty(B, dtype=torch.int32, device="cuda")
    vv.lm_head_argmax(dev(W), dev(x), logits, tok, ws)
    torch.cuda.synchronize()
    return (host(logits).astype(np.float64) if with_logits else None), host(tok)


def _check_tokens(tok, ref_logits):
    for b in range(ref_logits.shape[0]):
        i, gap = O.argmax_with_gap(ref_logits[b])
        if gap >= 1e-3:
            assert int(tok[b]) == i, (b, int(tok[b]), i, gap)
        else:  # a near-tie: either of the top two is acceptable
            top2 = np.argsort(ref_logits[b])[-2:]
            assert int(tok[b]) in set(int(t) for t in top2)


@pytest.mark.parametrize("H", [1536, 3584])
@pytest.mark.parametrize("B", [1, 3, 8, 16])
def test_lm_head_full_vocab(cuda, H, B):
    W = synth.fp16_normal(0, 0, synth.T_LM, (151936, H), std=0.02)
    x = synth.fp16_normal(0, 1, synth.T_EMB, (B, H)).astype(np.float32)
    ref, _, _ = O.lm_head_argmax(W, x)
    logits, tok = _lm_gpu(W, x)
    assert rel_err(logits, ref) <= TOL
    _check_tokens(tok, ref)
    _, tok2 = _lm_gpu(W, x, with_logits=False)
    assert np.array_equal(tok, tok2)


def test_lm_head_ties_pick_smallest_index(cuda):
    H, V = 256, 5000
    W = synth.fp16_normal(1, 0, synth.T_LM, (V, H), std=0.02)
    x = np.abs(synth.fp16_normal(1, 0, synth.T_EMB, (1, H))).astype(np.float32)
    W[[4321, 17, 999]] = np.float16(0.5)  # three identical rows with the largest dot
    _, tok = _lm_gpu(W, x)
    assert int(tok[0]) == 17


def test_lm_head_fp16_activation_and_odd_sizes(cuda):
    H, V = 200, 1001
    W = synth.fp16_normal(2, 0, synth.T_LM, (V, H), std=0.02)
    x = synth.fp16_normal(2, 0, synth.T_EMB, (2, H))
    ref, _, _ = O.lm_head_argmax(W, x)
    logits, tok = _lm_gpu(W, x)
    assert rel_err(logits, ref) <= TOL
    _check_tokens(tok, ref)


def test_lm_head_batch16_keeps_fp32_input_precision(cuda):
    """Batches of 3..16 run on the matrix cores with the fp32 activation split into two fp16
    parts: the logits stay within fp32 accumulation error of the fp64 result (far inside the
    2e-3 budget), including inputs that fp16 alone would round."""
    H, V, B = 1536, 4096, 16
    W = synth.fp16_normal(4, 0, synth.T_LM, (V, H), std=0.02)
    x = synth.fp16_normal(4, 1, synth.T_EMB, (B, H)).astype(np.float32)
    x = x * np.float32(1.0 + 1.0 / 3000.0)          # not representable in fp16
    ref, _, _ = O.lm_head_argmax(W, x)
    logits, tok = _lm_gpu(W, x)
    err = rel_err(logits, ref)
    print(f"batch-16 lm_head rel err {err:.2e}")
    assert err <= 2e-5
    _check_tokens(tok, ref)


def test_lm_head_batched_ties_and_fp16_input(cuda):
    """Matrix-core path: equal rows tie to the smallest index in every batch row; fp16 input."""
    H, V, B = 512, 1001, 4
    W = synth.fp16_normal(5, 0, synth.T_LM, (V, H), std=0.02)
    x = np.abs(synth.fp16_normal(5, 0, synth.T_EMB, (B, H)))
    W[[999, 17, 640]] = np.float16(0.5)
    logits, tok = _lm_gpu(W, x)
    assert list(tok) == [17] * B
    ref, _, _ = O.lm_head_argmax(W, x.astype(np.float32))
    assert rel_err(logits, ref) <= TOL


@pytest.mark.parametrize("B", [1, 3])
def test_lm_head_nan_rows_never_win(cuda, B):
    """NaN logits (rows of NaN weights, one of them where the true maximum would be) never win:
    the token is the argmax over the finite logits (VALU path at B = 1, matrix cores at B = 3)."""
    H, V = 256, 3000
    W = synth.fp16_normal(6, 0, synth.T_LM, (V, H), std=0.02)
    x = synth.fp16_normal(6, 1, synth.T_EMB, (B, H)).astype(np.float32)
    ref, _, _ = O.lm_head_argmax(W, x)
    best = [int(np.argmax(ref[b])) for b in range(B)]
    nan_rows = sorted(set(best + [0, 5, 2999]))
    W[nan_rows] = np.float16(np.nan)
    ref[:, nan_rows] = -np.inf
    logits, tok = _lm_gpu(W, x)
    assert np.isnan(logits[:, nan_rows]).all()
    keep = np.setdiff1d(np.arange(V), nan_rows)
    assert rel_err(logits[:, keep], ref[:, keep]) <= TOL
    _check_tokens(tok, ref)
    assert all(int(t) not in nan_rows for t in tok)
