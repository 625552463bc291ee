"""Pins of the oracle's decode step: wiring special cases with closed forms, and
KV-incremental decoding == an independently written full causal forward (the
incremental-equals-full check the 1.5B STATUS page reports for its ONNX decoder)."""
import math

import numpy as np
import pytest

from oracle import vv_oracle as O
from int4_blockwise_gemv_amd import synth
from helpers import oracle_model, zero_proj, scaled_identity_proj

# codes 15 -> q - 8 = 7; scale 1/16 (0x2C00) -> 7/16; scale 1/32 (0x2800) -> 7/32
C716 = (15, 0x2C00, 7 / 16)
C732 = (15, 0x2800, 7 / 32)


def _tiny_layer(H, nq, nkv, d, I, **over):
    L = O.OLayer(q=zero_proj(nq * d, H), k=zero_proj(nkv * d, H), v=zero_proj(nkv * d, H),
                 o=zero_proj(H, nq * d), gate=zero_proj(I, H), up=zero_proj(I, H), down=zero_proj(H, I),
                 g1=np.ones(H, np.float16), g2=np.ones(H, np.float16))
    for k, v in over.items():
        setattr(L, k, v)
    return L


def _model(layers, H, nq, nkv, d, lm=None, gf=None, theta=1e6):
    return O.OModel(layers=layers, gf=np.ones(H, np.float16) if gf is None else gf, lm=lm, n_q=nq, n_kv=nkv,
                    head_dim=d, eps=1e-6, rope_theta=theta)


def _caches(nkv, cap, d, P, seed=0):
    K = np.zeros((1, nkv, cap, d), np.float16)
    V = np.zeros((1, nkv, cap, d), np.float16)
    K[0, :, :P] = synth.fp16_normal(seed, 0, synth.T_KC, (nkv, P, d))
    V[0, :, :P] = synth.fp16_normal(seed, 0, synth.T_VC, (nkv, P, d))
    return K, V


def test_zero_layer_is_identity_and_writes_zero_kv():
    H, nq, nkv, d, I, P = 64, 2, 1, 32, 64, 5
    m = _model([_tiny_layer(H, nq, nkv, d, I)], H, nq, nkv, d)
    K, V = _caches(nkv, 8, d, P)
    K0, V0 = K.copy(), V.copy()
    x = synth.fp16_normal(0, 0, synth.T_EMB, (1, H))
    _, _, _, h = O.decode_step(m, x, np.array([P]), [K], [V])
    assert np.array_equal(h, x.astype(np.float64))
    assert np.all(K[0, :, P] == 0) and np.all(V[0, :, P] == 0)
    assert np.array_equal(K[0, :, :P], K0[0, :, :P]) and np.array_equal(V[0, :, :P], V0[0, :, :P])


def test_bias_only_kv_append_with_rope():
    """Zero weights: new k = RoPE(b_k, P), v = b_v are written (fp16) at slot P."""
    H, nq, nkv, d, I, P = 64, 2, 1, 32, 64, 5
    bk = synth.bias(0, 0, synth.T_BK, nkv * d)
    bv = synth.bias(0, 0, synth.T_BV, nkv * d)
    m = _model([_tiny_layer(H, nq, nkv, d, I, bk=bk, bv=bv)], H, nq, nkv, d, theta=10000.0)
    K, V = _caches(nkv, 8, d, P)
    O.decode_step(m, synth.fp16_normal(0, 0, synth.T_EMB, (1, H)), np.array([P]), [K], [V])
    b = bk.astype(np.float64)
    inv = 10000.0 ** (-np.arange(0, d, 2) / d)
    want = np.empty(d)
    for i in range(d // 2):
        a = P * inv[i]
        want[i] = b[i] * math.cos(a) - b[i + d // 2] * math.sin(a)
        want[i + d // 2] = b[i + d // 2] * math.cos(a) + b[i] * math.sin(a)
    assert np.array_equal(K[0, 0, P], want.astype(np.float16))
    assert np.array_equal(V[0, 0, P], bv)


def test_uniform_attention_through_o_proj():
    """q = 0 -> uniform softmax over the P+1 positions (including the new v = b_v);
    W_o = (7/16) I, zero MLP -> h' = h + 7/16 * mean_{j<=P} V[g(h), j] per head."""
    H, nq, nkv, d, I, P = 128, 4, 2, 32, 64, 6
    bv = synth.bias(1, 0, synth.T_BV, nkv * d)
    o_proj = scaled_identity_proj(H, C716[0], C716[1])
    m = _model([_tiny_layer(H, nq, nkv, d, I, bv=bv, o=o_proj)], H, nq, nkv, d)
    K, V = _caches(nkv, 10, d, P, seed=3)
    x = synth.fp16_normal(2, 0, synth.T_EMB, (1, H))
    _, _, _, h = O.decode_step(m, x, np.array([P]), [K], [V])
    Vf = V[0].astype(np.float64)  # slot P now holds fp16(b_v)
    assert np.array_equal(V[0, :, P], bv.reshape(nkv, d))
    want = x.astype(np.float64)[0].copy()
    for hh in range(nq):
        kv = hh // (nq // nkv)
        want[hh * d:(hh + 1) * d] += 7 / 16 * Vf[kv, :P + 1].mean(axis=0)
    assert np.allclose(h[0], want, rtol=0, atol=1e-13)


def test_mlp_closed_form():
    """Zero attention; gate = 7/16 I, up = 7/32 I, down = 7/16 I:
    h' = h + 7/16 * silu(7/16 m) * (7/32 m), m = RMSNorm(h; g2)."""
    H, nq, nkv, d, P = 64, 2, 1, 32, 3
    g2 = synth.gamma(0, 0, synth.T_G2, H)
    L = _tiny_layer(H, nq, nkv, d, H, g2=g2, gate=scaled_identity_proj(H, *C716[:2]),
                    up=scaled_identity_proj(H, *C732[:2]), down=scaled_identity_proj(H, *C716[:2]))
    m = _model([L], H, nq, nkv, d)
    K, V = _caches(nkv, 4, d, P)
    x = synth.fp16_normal(5, 0, synth.T_EMB, (1, H))
    _, _, _, h = O.decode_step(m, x, np.array([P]), [K], [V])
    h0 = x.astype(np.float64)[0]
    mm = h0 / math.sqrt(np.mean(h0 * h0) + 1e-6) * g2.astype(np.float64)
    a = 7 / 16 * mm
    want = h0 + 7 / 16 * (a / (1 + np.exp(-a))) * (7 / 32 * mm)
    assert np.allclose(h[0], want, rtol=1e-14, atol=1e-15)


def test_zero_layers_reduce_to_lm_head_argmax():
    H, V = 64, 300
    lm = synth.fp16_normal(0, 0, synth.T_LM, (V, H), std=0.02)
    gf = synth.gamma(0, 0, synth.T_GF, H)
    m = _model([], H, 2, 1, 32, lm=lm, gf=gf)
    x = synth.fp16_normal(1, 0, synth.T_EMB, (2, H))
    logits, tok, gap, _ = O.decode_step(m, x, np.array([0, 0]), [], [])
    f = x.astype(np.float64)
    f = f / np.sqrt(np.mean(f * f, axis=1, keepdims=True) + 1e-6) * gf.astype(np.float64)
    want = f @ lm.astype(np.float64).T
    assert np.allclose(logits, want, rtol=1e-13, atol=1e-15)
    assert list(tok) == list(np.argmax(want, axis=1))


@pytest.mark.parametrize("kv_dtype", [np.float16, np.float32])
def test_incremental_decode_equals_full_forward(kv_dtype):
    """T decode steps from a prefix cache == one full causal forward over the same tokens, with
    fp16 caches and with the fp32-KV variant."""
    shape = synth.TinyShape(layers=2, hidden=256, n_q=4, n_kv=2, head_dim=64, inter=384, vocab=500)
    m = oracle_model(shape, seed=0)
    T, P0, cap = 4, 3, 8
    L = shape.layers
    K0 = synth.fp16_normal(0, 0, synth.T_KC, (L, shape.n_kv, P0, shape.head_dim)).astype(kv_dtype)
    V0 = synth.fp16_normal(0, 0, synth.T_VC, (L, shape.n_kv, P0, shape.head_dim)).astype(kv_dtype)
    emb = synth.fp16_normal(9, 0, synth.T_EMB, (T, shape.hidden))
    full = O.full_forward(m, emb, K0, V0, kv_dtype=kv_dtype)
    Kc = [np.zeros((1, shape.n_kv, cap, shape.head_dim), kv_dtype) for _ in range(L)]
    Vc = [np.zeros((1, shape.n_kv, cap, shape.head_dim), kv_dtype) for _ in range(L)]
    for li in range(L):
        Kc[li][0, :, :P0] = K0[li]
        Vc[li][0, :, :P0] = V0[li]
    for t in range(T):
        logits, tok, _, _ = O.decode_step(m, emb[t:t + 1], np.array([P0 + t]), Kc, Vc)
        assert np.allclose(logits[0], full[t], rtol=1e-12, atol=1e-12)
        assert tok[0] == int(np.argmax(full[t]))


def test_prefill_equals_token_by_token_decode():
    """The prefill (decoder_init) oracle == T decode steps from an empty cache: the same present
    K/V at every position and the same logits at the last one (two independent formulations)."""
    shape = synth.TinyShape(layers=2, hidden=256, n_q=4, n_kv=2, head_dim=64, inter=384, vocab=500)
    m = oracle_model(shape, seed=3)
    T, cap = 5, 8
    L = shape.layers
    emb = synth.fp16_normal(4, 0, synth.T_EMB, (T, shape.hidden))
    Kp = [np.zeros((shape.n_kv, cap, shape.head_dim), np.float16) for _ in range(L)]
    Vp = [np.zeros((shape.n_kv, cap, shape.head_dim), np.float16) for _ in range(L)]
    logits, tok, gap = O.prefill(m, emb, Kp, Vp)
    Kc = [np.zeros((1, shape.n_kv, cap, shape.head_dim), np.float16) for _ in range(L)]
    Vc = [np.zeros((1, shape.n_kv, cap, shape.head_dim), np.float16) for _ in range(L)]
    for t in range(T):
        step_logits, step_tok, _, _ = O.decode_step(m, emb[t:t + 1], np.array([t]), Kc, Vc)
    assert np.allclose(logits, step_logits[0], rtol=1e-12, atol=1e-12)
    assert tok == int(step_tok[0])
    for li in range(L):
        # fp16 stores of the same float64 values: allow a rounding-boundary flip of one ulp
        a = Kp[li].astype(np.float64)
        b = Kc[li][0].astype(np.float64)
        assert np.max(np.abs(a - b) / np.maximum(np.abs(b), 1e-3)) <= 2 ** -10
        assert np.array_equal(Kp[li][:, T:], Kc[li][0][:, T:])   # untouched positions stay zero
        assert np.max(np.abs(Vp[li].astype(np.float64) - Vc[li][0].astype(np.float64))) <= 2 ** -10 * 8


def test_fp32_kv_stores_unrounded_keys():
    """The fp32-KV variant keeps k and v unrounded: its stored keys differ from the fp16 cache's by
    the fp16 rounding only, and its attention output equals the fp16 cache's within that rounding."""
    shape = synth.TinyShape(layers=1, hidden=256, n_q=4, n_kv=2, head_dim=64, inter=384, vocab=500)
    m = oracle_model(shape, seed=2)
    emb = synth.fp16_normal(5, 0, synth.T_EMB, (3, shape.hidden))
    K16 = [np.zeros((shape.n_kv, 4, shape.head_dim), np.float16)]
    V16 = [np.zeros((shape.n_kv, 4, shape.head_dim), np.float16)]
    K32 = [np.zeros((shape.n_kv, 4, shape.head_dim), np.float32)]
    V32 = [np.zeros((shape.n_kv, 4, shape.head_dim), np.float32)]
    l16, _, _ = O.prefill(m, emb, K16, V16)
    l32, _, _ = O.prefill(m, emb, K32, V32)
    assert np.array_equal(K32[0].astype(np.float16), K16[0])      # fp16(fp32 value) is the fp16 store
    assert not np.array_equal(K32[0], K16[0].astype(np.float32))  # and fp32 keeps more bits
    assert np.allclose(l32, l16, rtol=0, atol=1e-2 * np.max(np.abs(l16)))


def test_batched_step_equals_per_sequence_steps():
    """Sequences in a batch are independent (ragged positions)."""
    shape = synth.TinyShape(layers=1, hidden=128, n_q=2, n_kv=1, head_dim=64, inter=128, vocab=200)
    m = oracle_model(shape, seed=1, batch=3)
    pos = np.array([2, 5, 0])
    cap = 8
    K = synth.fp16_normal(1, 0, synth.T_KC, (1, 3, 1, cap, 64))
    V = synth.fp16_normal(1, 0, synth.T_VC, (1, 3, 1, cap, 64))
    emb = synth.fp16_normal(1, 0, synth.T_EMB, (3, 128))
    Kb, Vb = [K[0].copy()], [V[0].copy()]
    logits, tok, _, _ = O.decode_step(m, emb, pos, Kb, Vb)
    for b in range(3):
        Ks, Vs = [K[0, b:b + 1].copy()], [V[0, b:b + 1].copy()]
        lb, tb, _, _ = O.decode_step(m, emb[b:b + 1], pos[b:b + 1], Ks, Vs)
        assert np.allclose(lb[0], logits[b], rtol=1e-12, atol=1e-13) and tb[0] == tok[b]
        assert np.array_equal(Ks[0][0], Kb[0][b])
