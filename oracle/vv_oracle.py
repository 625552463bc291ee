"""fp64 CPU oracle for the int4 block-32 (ternary) decode step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library (``int4_blockwise_gemv_amd``) and imports nothing from it;
both sides receive the same seeded arrays from ``int4_blockwise_gemv_amd.synth``,
a module that draws random numbers and holds none of the arithmetic below.

It is written to be slow and obviously correct: numpy float64 throughout,
except at the storage points the pages' tensor contracts fix as 16-bit
(block scales, K/V cache entries, input embeddings, the lm_head table).

Sources (pages, cited by title and section):

* "vibevoice-asr-bitnet-onnx" model page (Masterx), in four places:
  - ternarisation paragraph: s = 1/mean(|W|), W' = round(clamp(W*s, -1, 1))/s on
    the q/k/v/o/gate/up/down projections; ternary x scale values are exact in
    fp16 and in block-32 symmetric int4; activations stay in float;
  - MatMulNBits note under the tier table: q = w/s + 8 in {7, 8, 9}, block
    32, symmetric, one scale per block equal to the ternary scale;
    lm_head/embeddings stay fp16;
  - graph contracts: decoder_step(input_embeds[1,1,H], position_ids[1,1],
    past K/V [28,1,kv,P,128]) -> logits[1,1,V], present K/V [...,P+1,128];
    decoder_init (the prompt's S tokens) -> logits and present K/V [...,S,128];
  - decoding note: greedy argmax, stop tokens 151645 / 151643.
* "VibeVoice-1.5B -- Current Status", Architecture section: the backbone is
  Qwen2.5-1.5B (hidden 1536, 28 layers, 12 heads, 2 KV heads, q/k/v bias,
  embeddings tied to the head); Inference section: KV-incremental decoding
  equals full recomputation.

Readings where the pages are silent (the plainest reading the rest of the pages support):

* the stored block scale is mean(|W|) = 1/s (the only reading that puts the
  codes in {7,8,9}); mean(|W|) is per projection tensor, the same value in
  every block;
* mean(|W|) is the correctly rounded fp64 sum of |W| (math.fsum) divided by
  the element count in fp64; round() is half-to-even; the fp16 scale is one
  correctly rounded conversion from fp64;
* general (non-ternary) int4: per-block scale fp16(absmax/7), q =
  clip(rint(w / scale) + 8, 0, 15), an all-zero block (scale 0) gives q = 8;
* nibble order: byte j of a block holds element 2j in the low nibble and 2j+1
  in the high nibble; packed shape [N][K/32][16], scales [N][K/32];
* Qwen2 layer: pre-RMSNorm (eps 1e-6), q/k/v bias, NeoX rotate-half RoPE with
  theta 1e6 applied to q and the new k, GQA head h -> KV head h // (nq/nkv),
  softmax scale 1/sqrt(head_dim), SiLU-gated MLP, residual adds;
* the decode step writes fp16(k), fp16(v) at slot P, then attends over P+1
  positions (past P -> present P+1 in the decoder_step contract).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

BLOCK = 32
ZERO_POINT = 8


# ---------------------------------------------------------------------------
# 16-bit storage
# ---------------------------------------------------------------------------

def fp16_bits(x) -> np.ndarray:
    """IEEE binary16 bits of x (float64), one round-to-nearest-even step."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def fp16_value(bits) -> np.ndarray:
    """float64 value of binary16 bits."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# ---------------------------------------------------------------------------
# quantisation (bitnet-onnx page: ternarisation paragraph and MatMulNBits note)
# ---------------------------------------------------------------------------

def exact_mean_abs(W: np.ndarray) -> float:
    """mean(|W|): correctly rounded fp64 sum of |W|, divided by the count in fp64."""
    a = np.abs(np.asarray(W, dtype=np.float32)).astype(np.float64).ravel()
    n = a.size
    if n == 0:
        return 0.0
    step = 1 << 20
    s = math.fsum(v for i in range(0, n, step) for v in a[i:i + step].tolist())
    return s / float(n)


def ternary_codes(W: np.ndarray, m: Optional[float] = None):
    """Ternarise one projection tensor.

    s = 1/m with m = mean(|W|); t = round(clamp(W*s, -1, 1)) evaluated in exact
    arithmetic; the code is q = t + 8.  In exact arithmetic |W*s| > 1/2 is
    |W| > m/2 (m/2 is exact in fp64), a tie |W*s| = 1/2 rounds to even (0),
    and anything past the clamp rounds to +-1.

    Returns (codes uint8 [N,K], scale_bits uint16 [N,K/32], m).
    """
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    assert K % BLOCK == 0
    if m is None:
        m = exact_mean_abs(W)
    W64 = W.astype(np.float64)
    if m == 0.0:
        t = np.zeros((N, K), np.int64)
    else:
        t = np.where(np.abs(W64) > 0.5 * m, np.sign(W64), 0.0).astype(np.int64)
    codes = (t + ZERO_POINT).astype(np.uint8)
    sbits = np.full((N, K // BLOCK), fp16_bits(m), dtype=np.uint16)
    return codes, sbits, m


def ternary_codes_literal(W: np.ndarray):
    """The pages' formula evaluated literally in fp64: rint(clip(W * (1/m), -1, 1)).

    Used only as a cross-check of the exact reading above (they agree except
    when W*s lands within fp64 rounding of 1/2).
    """
    W64 = np.asarray(W, dtype=np.float32).astype(np.float64)
    m = exact_mean_abs(W)
    s = 1.0 / m
    t = np.rint(np.clip(W64 * s, -1.0, 1.0)).astype(np.int64)
    return (t + ZERO_POINT).astype(np.uint8)


def absmax_codes(W: np.ndarray):
    """General symmetric int4 block-32: scale = fp16(absmax/7), q = clip(rint(w/scale) + 8, 0, 15).

    Returns (codes uint8 [N,K], scale_bits uint16 [N,K/32]).
    """
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    assert K % BLOCK == 0
    Wb = W.astype(np.float64).reshape(N, K // BLOCK, BLOCK)
    amax = np.abs(Wb).max(axis=2)
    sbits = fp16_bits(amax / 7.0)
    scale = fp16_value(sbits)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint(Wb / scale[:, :, None])
    r = np.where(scale[:, :, None] == 0.0, 0.0, r)
    r = np.where(np.isfinite(r), r, 0.0)
    codes = np.clip(r + ZERO_POINT, 0, 15).astype(np.uint8).reshape(N, K)
    return codes, sbits.astype(np.uint16)


def quantize(W: np.ndarray, mode: str):
    if mode == "ternary":
        c, s, _ = ternary_codes(W)
        return c, s
    if mode == "absmax":
        return absmax_codes(W)
    raise ValueError(mode)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[N,K] codes 0..15 -> [N, K/32, 16] bytes; byte j = code[2j] | code[2j+1] << 4."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, K = codes.shape
    c = codes.reshape(N, K // BLOCK, BLOCK // 2, 2)
    return (c[..., 0] | (c[..., 1] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[N, K/32, 16] bytes -> [N, K] codes."""
    p = np.asarray(packed, dtype=np.uint8)
    N, nb, _ = p.shape
    out = np.empty((N, nb, 16, 2), np.uint8)
    out[..., 0] = p & 0x0F
    out[..., 1] = p >> 4
    return out.reshape(N, nb * BLOCK)


def dequant(packed: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """w = (q - 8) * scale, float64 [N, K] (exact: a 4-bit integer times an fp16 value)."""
    q = unpack_nibbles(packed).astype(np.float64) - ZERO_POINT
    N, K = q.shape
    s = fp16_value(scale_bits)
    return (q.reshape(N, K // BLOCK, BLOCK) * s[:, :, None]).reshape(N, K)


def pack(W: np.ndarray, mode: str):
    """fp32 master -> (packed uint8 [N, K/32, 16], scale bits uint16 [N, K/32])."""
    c, s = quantize(W, mode)
    return pack_nibbles(c), s


# ---------------------------------------------------------------------------
# GEMV on packed weights
# ---------------------------------------------------------------------------

def gemv(packed, scale_bits, x, bias=None, row_chunk: int = 4096) -> np.ndarray:
    """y[m, n] = sum_k deq(W)[n, k] * x[m, k] (+ bias[n]), float64.

    x is [M, K] (any float dtype, taken as float64).  Dequantises row chunks so
    that large matrices never exist in fp64 at once.
    """
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    N = packed.shape[0]
    y = np.empty((x.shape[0], N), np.float64)
    for r0 in range(0, N, row_chunk):
        r1 = min(N, r0 + row_chunk)
        Wd = dequant(packed[r0:r1], scale_bits[r0:r1])
        y[:, r0:r1] = x @ Wd.T
    if bias is not None:
        y += np.asarray(bias, dtype=np.float64)[None, :]
    return y


# ---------------------------------------------------------------------------
# Qwen2 layer pieces
# ---------------------------------------------------------------------------

def rmsnorm(h, g, eps: float) -> np.ndarray:
    """h / sqrt(mean(h^2) + eps) * g over the last axis."""
    h = np.asarray(h, dtype=np.float64)
    r = np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    return h / r * np.asarray(g, dtype=np.float64)


def silu(z) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    return np.power(float(theta), -np.arange(0, head_dim, 2, dtype=np.float64) / head_dim)


def rope(x, pos, theta: float) -> np.ndarray:
    """Rotate-half RoPE on the last axis (head_dim), pairs (i, i + d/2), angle pos * theta^(-2i/d).

    x: [..., heads, d]; pos: scalar or array broadcastable to x.shape[:-2].
    theta <= 0 leaves x unchanged.
    """
    x = np.asarray(x, dtype=np.float64)
    if theta <= 0:
        return x.copy()
    d = x.shape[-1]
    half = d // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None, None] * rope_inv_freq(d, theta)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def gqa_decode(q, K, V, length: int, scale: float) -> np.ndarray:
    """One sequence: q [nq, d]; K, V [nkv, >=length, d]; attention over positions [0, length).

    o_h = sum_j softmax_j(q_h . K[g(h), j] * scale) V[g(h), j], g(h) = h // (nq / nkv).
    """
    q = np.asarray(q, dtype=np.float64)
    nq, d = q.shape
    nkv = K.shape[0]
    grp = nq // nkv
    out = np.empty((nq, d), np.float64)
    for h in range(nq):
        kh = h // grp
        k = np.asarray(K[kh, :length], dtype=np.float64)
        v = np.asarray(V[kh, :length], dtype=np.float64)
        s = (k @ q[h]) * scale
        s = s - s.max()
        p = np.exp(s)
        out[h] = (p @ v) / p.sum()
    return out


def argmax_with_gap(logits) -> tuple:
    """(first index of the maximum, gap between the largest and second-largest value)."""
    z = np.asarray(logits, dtype=np.float64)
    i = int(np.argmax(z))
    if z.size < 2:
        return i, math.inf
    top2 = np.partition(z, -2)[-2:]
    return i, float(top2[1] - top2[0])


def lm_head_argmax(W16, x):
    """logits = W x for an fp16 table W [V, H] and x [B, H]; token = first argmax per row."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    V = W16.shape[0]
    logits = np.empty((x.shape[0], V), np.float64)
    step = 16384
    for r0 in range(0, V, step):
        r1 = min(V, r0 + step)
        logits[:, r0:r1] = x @ np.asarray(W16[r0:r1], dtype=np.float64).T
    toks, gaps = zip(*(argmax_with_gap(row) for row in logits))
    return logits, np.array(toks, np.int64), np.array(gaps)


# ---------------------------------------------------------------------------
# decode step (decoder_step contract)
# ---------------------------------------------------------------------------

@dataclass
class OLayer:
    q: tuple   # (packed, scale_bits) per projection
    k: tuple
    v: tuple
    o: tuple
    gate: tuple
    up: tuple
    down: tuple
    g1: np.ndarray
    g2: np.ndarray
    bq: Optional[np.ndarray] = None
    bk: Optional[np.ndarray] = None
    bv: Optional[np.ndarray] = None


@dataclass
class OModel:
    layers: Sequence[OLayer]
    gf: np.ndarray
    lm: Optional[np.ndarray]   # fp16 [V, H]
    n_q: int
    n_kv: int
    head_dim: int
    eps: float = 1e-6
    rope_theta: float = 1e6


def layer_step(L: OLayer, m: OModel, h, pos, Kc, Vc, trace: Optional[dict] = None):
    """One Qwen2 decoder layer for B sequences at positions pos[b].

    h: [B, H] float64 residual stream.  Kc, Vc: this layer's fp16 caches
    [B, nkv, cap, d], updated in place at slot pos[b].  Returns the new h.
    """
    B, H = h.shape
    d, nq, nkv = m.head_dim, m.n_q, m.n_kv
    a = rmsnorm(h, L.g1, m.eps)
    q = gemv(*L.q, a, L.bq).reshape(B, nq, d)
    k = gemv(*L.k, a, L.bk).reshape(B, nkv, d)
    v = gemv(*L.v, a, L.bv).reshape(B, nkv, d)
    pos = np.asarray(pos, dtype=np.int64)
    q = rope(q, pos, m.rope_theta)
    k = rope(k, pos, m.rope_theta)
    o = np.empty((B, nq, d), np.float64)
    for b in range(B):
        p = int(pos[b])
        Kc[b, :, p] = k[b].astype(Kc.dtype)     # fp16 caches, or fp32 in the fp32-KV variant
        Vc[b, :, p] = v[b].astype(Vc.dtype)
        o[b] = gqa_decode(q[b], Kc[b], Vc[b], p + 1, 1.0 / math.sqrt(d))
    h = h + gemv(*L.o, o.reshape(B, nq * d))
    mm = rmsnorm(h, L.g2, m.eps)
    act = silu(gemv(*L.gate, mm)) * gemv(*L.up, mm)
    h = h + gemv(*L.down, act)
    if trace is not None:
        trace.setdefault("k_new", []).append(k)
        trace.setdefault("v_new", []).append(v)
        trace.setdefault("o", []).append(o)
    return h


def decode_step(m: OModel, input_embeds, pos, Kcaches, Vcaches, trace: Optional[dict] = None):
    """decoder_step: input_embeds [B, H] (fp16 values) at positions pos [B] with per-layer
    caches -> (logits [B, V] or None, token [B] or None, gap [B] or None, final h [B, H]).

    Kcaches[l], Vcaches[l]: fp16 [B, nkv, cap, d], updated in place at slot pos[b].
    """
    h = np.asarray(input_embeds, dtype=np.float16).astype(np.float64)
    if trace is not None:
        trace["h"] = [h.copy()]
    for li, L in enumerate(m.layers):
        h = layer_step(L, m, h, pos, Kcaches[li], Vcaches[li], trace)
        if trace is not None:
            trace["h"].append(h.copy())
    if m.lm is None:
        return None, None, None, h
    f = rmsnorm(h, m.gf, m.eps)
    logits, tok, gap = lm_head_argmax(m.lm, f)
    return logits, tok, gap, h


def full_forward(m: OModel, embeds, K0=None, V0=None, kv_out=None, last_only: bool = False,
                 kv_dtype=np.float16):
    """Independent full causal forward over T tokens (for the incremental == full check, and the
    decoder_init / prefill contract of the bitnet-onnx page's graph contracts).

    embeds [T, H] fp16 values; optional prefix caches K0/V0 [L, nkv, P0, d] fp16 that the
    T tokens attend to (positions 0..P0-1), new tokens at positions P0..P0+T-1.  The new
    keys/values are rounded to kv_dtype (fp16, or fp32 for the fp32-KV variant of the ASR-ONNX
    card) before use, as the decode step stores them.  With kv_out
    (a sequence of (K, V) fp16 arrays [nkv, cap, d], one pair per layer), the new keys/values
    are also stored at their positions there (the present K/V of the contract).
    Returns logits [T, V] of every position (with last_only, [1, V] of the last one).
    """
    x = np.asarray(embeds, dtype=np.float16).astype(np.float64)
    T, H = x.shape
    d, nq, nkv = m.head_dim, m.n_q, m.n_kv
    grp = nq // nkv
    P0 = 0 if K0 is None else K0.shape[2]
    pos = np.arange(P0, P0 + T)
    for li, L in enumerate(m.layers):
        a = rmsnorm(x, L.g1, m.eps)
        q = rope(gemv(*L.q, a, L.bq).reshape(T, nq, d), pos, m.rope_theta)
        k = rope(gemv(*L.k, a, L.bk).reshape(T, nkv, d), pos, m.rope_theta)
        v = gemv(*L.v, a, L.bv).reshape(T, nkv, d)
        k = k.astype(kv_dtype).astype(np.float64)
        v = v.astype(kv_dtype).astype(np.float64)
        if kv_out is not None:
            Kc, Vc = kv_out[li]
            Kc[:, P0:P0 + T] = k.transpose(1, 0, 2).astype(kv_dtype)
            Vc[:, P0:P0 + T] = v.transpose(1, 0, 2).astype(kv_dtype)
        if P0:
            kall = np.concatenate([np.asarray(K0[li], np.float64).transpose(1, 0, 2), k], axis=0)
            vall = np.concatenate([np.asarray(V0[li], np.float64).transpose(1, 0, 2), v], axis=0)
        else:
            kall, vall = k, v
        o = np.empty((T, nq, d))
        for h in range(nq):
            kh = h // grp
            s = (q[:, h, :] @ kall[:, kh, :].T) / math.sqrt(d)        # [T, P0+T]
            mask = np.arange(P0 + T)[None, :] > pos[:, None]
            s = np.where(mask, -np.inf, s)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            o[:, h, :] = (p @ vall[:, kh, :]) / p.sum(axis=1, keepdims=True)
        x = x + gemv(*L.o, o.reshape(T, nq * d))
        mm = rmsnorm(x, L.g2, m.eps)
        x = x + gemv(*L.down, silu(gemv(*L.gate, mm)) * gemv(*L.up, mm))
    f = rmsnorm(x[-1:] if last_only else x, m.gf, m.eps)
    return f @ np.asarray(m.lm, np.float64).T


def prefill(m: OModel, embeds, Kc, Vc):
    """decoder_init (bitnet-onnx page, graph contracts): the T prompt embeddings at positions
    0..T-1 of an empty cache -> present K/V of those positions (written into Kc[l], Vc[l],
    fp16 [nkv, cap, d]) and the logits of the last position, which greedy decoding needs to
    pick the first generated token.  The caches' dtype (fp16, or fp32 for the fp32-KV variant)
    is the storage precision of k and v.  Returns (logits [V], token, top-2 gap)."""
    kv_dtype = Kc[0].dtype if len(Kc) else np.float16
    logits = full_forward(m, embeds, kv_out=list(zip(Kc, Vc)), last_only=True, kv_dtype=kv_dtype)
    tok, gap = argmax_with_gap(logits[-1])
    return logits[-1], tok, gap


# ---------------------------------------------------------------------------
# tolerance helpers used by the parity tests
# ---------------------------------------------------------------------------

def max_rel_err(y, ref) -> float:
    """Normwise max relative error: max_i |y_i - r_i| / max_i |r_i|."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(y - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den
