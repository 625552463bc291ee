"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Every test here checks the oracle against something other than itself: hand-computed
blocks (tests/golden/), exact rational arithmetic, closed forms, invariants the pages
state, and pure-Python brute force on tiny inputs.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import vv_oracle as O
from int4_blockwise_gemv_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    d = {}
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            d[k.strip()] = v.split()
    return d


def _frac_list(tokens):
    return [Fraction(t) for t in tokens]


def _x_pattern(n):
    return np.array([(i % 5) - 2 for i in range(n)], dtype=np.float16)


# ---------------------------------------------------------------------------
# fp16 rounding
# ---------------------------------------------------------------------------

def _rne_fp16_exact(v: Fraction) -> int:
    """Correctly rounded binary16 bits of a rational (normal and subnormal range)."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -14)
    ulp = Fraction(2) ** (e - 10)
    q = a / ulp
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * ulp
    if val >= 65520:
        return sign | 0x7C00
    bits = int(np.float16(float(val)).view(np.uint16))  # val is exactly representable here
    return sign | bits


def test_fp16_rounding_matches_exact_rne():
    rng = np.random.default_rng(123)
    vals = []
    # exact midpoints between adjacent fp16 values (ties), and points just off them
    for b in rng.integers(0x0001, 0x7BFF, size=400):
        lo = Fraction(float(np.uint16(b).view(np.float16)))
        hi = Fraction(float(np.uint16(b + 1).view(np.float16)))
        mid = (lo + hi) / 2
        vals += [mid, mid + (hi - lo) / 2 ** 20, mid - (hi - lo) / 2 ** 20]
    vals += [Fraction(float(v)) for v in rng.standard_normal(300) * 0.02]
    for v in vals:
        f = float(v)
        assert Fraction(f) == v or abs(Fraction(f) - v) < abs(v) * Fraction(1, 2 ** 50)
        got = int(O.fp16_bits(f))
        want = _rne_fp16_exact(Fraction(f))
        assert got == want, (v, hex(got), hex(want))


# ---------------------------------------------------------------------------
# ternary quantisation
# ---------------------------------------------------------------------------

def test_ternary_hand_block():
    g = _read_golden("ternary_hand_block.txt")
    Wf = _frac_list(g["W"])
    assert sum(abs(w) for w in Wf) / len(Wf) == Fraction(1, 16)
    W = np.array([[float(w) for w in Wf]], dtype=np.float32)
    codes, sbits, m = O.ternary_codes(W)
    assert m == 1.0 / 16
    assert [int(c) for c in codes[0]] == [int(c) for c in g["codes"]]
    assert int(sbits[0, 0]) == int(g["scale_bits"][0], 16)
    packed = O.pack_nibbles(codes)
    assert packed.shape == (1, 1, 16)
    assert [int(b) for b in packed[0, 0]] == [int(b, 16) for b in g["bytes"]]
    assert [int(b) for b in packed[0, 0]] != [int(b, 16) for b in g["bytes_half_away"]]
    x = _x_pattern(32)
    y = O.gemv(packed, sbits, x[None, :])
    assert Fraction(float(y[0, 0])) == Fraction(g["dot"][0])
    # unpack is the inverse of pack
    assert np.array_equal(O.unpack_nibbles(packed), codes)


def test_ternary_exact_reading_matches_literal_formula():
    W = synth.master_weight(7, 0, 0, 96, 256)
    c_exact, _, _ = O.ternary_codes(W)
    c_lit = O.ternary_codes_literal(W)
    assert np.array_equal(c_exact, c_lit)


def test_exact_mean_abs_is_correctly_rounded():
    rng = np.random.default_rng(5)
    for n in (1, 7, 32, 1000):
        W = (rng.standard_normal(n) * rng.choice([1e-30, 1e-3, 1.0, 1e20], size=n)).astype(np.float32)
        exact = sum((Fraction(float(abs(w))) for w in W), Fraction(0))
        want = float(exact) / n  # float(Fraction) is correctly rounded
        assert O.exact_mean_abs(W.reshape(1, -1)) == want


def test_ternary_invariants_and_fp16_exactness():
    """codes in {7,8,9}; one scale per tensor; deq values in {-s, 0, s} and exact in fp16."""
    W = synth.master_weight(0, 0, synth.T_Q, 192, 1536)
    packed, sbits = O.pack(W, "ternary")
    codes = O.unpack_nibbles(packed)
    assert set(np.unique(codes).tolist()) <= {7, 8, 9}
    assert np.unique(sbits).size == 1
    deq = O.dequant(packed, sbits)
    s = float(O.fp16_value(sbits[0, 0]))
    assert set(np.unique(deq).tolist()) <= {-s, 0.0, s}
    assert np.array_equal(deq.astype(np.float16).astype(np.float64), deq)


def test_ternary_statistics_closed_forms():
    """E|W| = 0.02 sqrt(2/pi); P(t != 0) = P(|Z| > sqrt(2/pi)/2) = erfc(1/(2 sqrt(pi)))."""
    W = synth.master_weight(1, 0, synth.T_GATE, 1536, 1536)  # 2.36 M weights
    m = O.exact_mean_abs(W)
    assert abs(m / (0.02 * math.sqrt(2 / math.pi)) - 1) < 2e-3
    codes, _, _ = O.ternary_codes(W, m)
    frac_nz = float(np.mean(codes != 8))
    p = math.erfc(0.5 * math.sqrt(2 / math.pi) / math.sqrt(2))
    assert abs(p - 0.68994) < 1e-4
    assert abs(frac_nz - p) < 1e-3
    # sign symmetry
    assert abs(float(np.mean(codes == 9)) - float(np.mean(codes == 7))) < 2e-3


def test_ternary_all_zero_tensor():
    W = np.zeros((2, 64), np.float32)
    codes, sbits, m = O.ternary_codes(W)
    assert m == 0.0 and np.all(codes == 8) and np.all(sbits == 0)


# ---------------------------------------------------------------------------
# general int4 (absmax) quantisation
# ---------------------------------------------------------------------------

def test_absmax_hand_block():
    g = _read_golden("absmax_hand_block.txt")
    W = np.array([[float(Fraction(w)) for w in g["W"]]], dtype=np.float32)
    codes, sbits = O.absmax_codes(W)
    assert int(sbits[0, 0]) == int(g["scale_bits"][0], 16)
    assert [int(c) for c in codes[0]] == [int(c) for c in g["codes"]]
    packed = O.pack_nibbles(codes)
    assert [int(b) for b in packed[0, 0]] == [int(b, 16) for b in g["bytes"]]
    y = O.gemv(packed, sbits, _x_pattern(32)[None, :])
    assert Fraction(float(y[0, 0])) == Fraction(g["dot"][0])


def test_absmax_invariants():
    W = synth.master_weight(0, 0, synth.T_DOWN, 128, 2048)
    W[3, :32] = 0.0  # an all-zero block
    codes, sbits = O.absmax_codes(W)
    assert codes.min() >= 1 and codes.max() <= 15
    assert np.all(codes[3, :32] == 8) and sbits[3, 0] == 0
    cb = codes.reshape(128, 64, 32).astype(np.int64) - 8
    nz = sbits != 0
    assert np.all(np.abs(cb).max(axis=2)[nz] == 7)
    deq = O.dequant(O.pack_nibbles(codes), sbits)
    s = O.fp16_value(sbits)
    err = np.abs(deq - W.astype(np.float64)).reshape(128, 64, 32).max(axis=2)
    assert np.all(err <= s / 2 * (1 + 1e-12))
    # scale is the single correctly rounded fp16 of absmax/7
    amax = np.abs(W.astype(np.float64)).reshape(128, 64, 32).max(axis=2)
    for i, j in [(0, 0), (5, 17), (127, 63)]:
        assert int(sbits[i, j]) == _rne_fp16_exact(Fraction(float(amax[i, j])) / 7)


def test_absmax_exact_against_fractions():
    """Every code equals the exact rational rint(w/scale) + 8 (ties to even), clamped."""
    rng = np.random.default_rng(9)
    W = (rng.standard_normal((4, 64)) * 0.02).astype(np.float32)
    # plant exact ties: w = (k + 1/2) * scale for the block's own scale
    codes, sbits = O.absmax_codes(W)
    for i in range(4):
        for b in range(2):
            s = Fraction(float(O.fp16_value(sbits[i, b])))
            for j in range(32):
                w = Fraction(float(W[i, 32 * b + j]))
                r = w / s
                fl = math.floor(r)
                rem = r - fl
                t = fl + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2) else 0)
                assert int(codes[i, 32 * b + j]) == min(15, max(0, t + 8))


# ---------------------------------------------------------------------------
# GEMV
# ---------------------------------------------------------------------------

def test_gemv_exact_rationals():
    rng = np.random.default_rng(11)
    N, K = 5, 96
    codes = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    sb = np.array([[0x2C00, 0x3400, 0x2000], [0x3C00, 0x3800, 0x1C00], [0x2C00] * 3, [0x3000] * 3,
                   [0x0001, 0x3C00, 0x4000]], dtype=np.uint16)  # includes a subnormal scale
    x = (rng.integers(-64, 64, size=(2, K)) / 16.0).astype(np.float16)
    bias = np.array([0.5, -0.25, 0, 1, 2], dtype=np.float16)
    y = O.gemv(O.pack_nibbles(codes), sb, x, bias)
    for m in range(2):
        for n in range(N):
            acc = Fraction(float(bias[n]))
            for k in range(K):
                s = Fraction(float(np.uint16(sb[n, k // 32]).view(np.float16)))
                acc += (int(codes[n, k]) - 8) * s * Fraction(float(x[m, k]))
            assert Fraction(float(y[m, n])) == acc


def test_gemv_one_hot_returns_columns():
    W = synth.master_weight(3, 0, synth.T_O, 64, 128)
    packed, sb = O.pack(W, "absmax")
    deq = O.dequant(packed, sb)
    for k in (0, 31, 32, 127):
        x = np.zeros((1, 128), np.float16)
        x[0, k] = 1
        assert np.array_equal(O.gemv(packed, sb, x)[0], deq[:, k])


def test_gemv_all_codes_nine_gives_scaled_sum():
    codes = np.full((3, 64), 9, np.uint8)
    sb = np.full((3, 2), 0x3555, np.uint16)
    x = synth.fp16_normal(0, 0, synth.T_X, (1, 64))
    y = O.gemv(O.pack_nibbles(codes), sb, x)
    s = float(O.fp16_value(0x3555))
    assert np.allclose(y[0], s * float(np.sum(x.astype(np.float64))), rtol=1e-15, atol=0)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def _brute_gqa(q, K, V, length, scale):
    nq, d = len(q), len(q[0])
    nkv = len(K)
    out = []
    for h in range(nq):
        kh = h * nkv // nq
        sc = [sum(float(q[h][i]) * float(K[kh][j][i]) for i in range(d)) * scale for j in range(length)]
        mx = max(sc)
        w = [math.exp(s - mx) for s in sc]
        tot = sum(w)
        out.append([sum(w[j] * float(V[kh][j][i]) for j in range(length)) / tot for i in range(d)])
    return out


def test_gqa_brute_force_2kv_len3():
    rng = np.random.default_rng(2)
    nq, nkv, d, L = 4, 2, 128, 3
    q = rng.standard_normal((nq, d))
    K = rng.standard_normal((nkv, 5, d)).astype(np.float16)
    V = rng.standard_normal((nkv, 5, d)).astype(np.float16)
    got = O.gqa_decode(q, K, V, L, 1 / math.sqrt(d))
    want = np.array(_brute_gqa(q.tolist(), K.astype(np.float64).tolist(), V.astype(np.float64).tolist(), L,
                               1 / math.sqrt(d)))
    assert np.max(np.abs(got - want)) < 1e-12


def test_gqa_special_cases():
    rng = np.random.default_rng(4)
    nq, nkv, d = 6, 2, 128
    K = rng.standard_normal((nkv, 8, d)).astype(np.float16)
    V = rng.standard_normal((nkv, 8, d)).astype(np.float16)
    q = rng.standard_normal((nq, d))
    # length 1 -> v0
    o = O.gqa_decode(q, K, V, 1, 0.1)
    for h in range(nq):
        assert np.array_equal(o[h], V[h // 3, 0].astype(np.float64))
    # identical keys -> mean of V
    K2 = np.repeat(K[:, :1], 8, axis=1)
    o = O.gqa_decode(q, K2, V, 8, 0.1)
    for h in range(nq):
        assert np.allclose(o[h], V[h // 3].astype(np.float64).mean(axis=0), atol=1e-14)
    # one key dominant by a score margin of 40 -> that value vector
    qd = np.zeros((nq, d))
    qd[:, 0] = 1.0
    K3 = np.zeros((nkv, 8, d), np.float16)
    K3[:, 5, 0] = 40.0
    o = O.gqa_decode(qd, K3, V, 8, 1.0)
    for h in range(nq):
        assert np.allclose(o[h], V[h // 3, 5].astype(np.float64), rtol=0, atol=1e-14)
    # constant V per KV head -> that constant on exactly the heads of its group (head mapping)
    V4 = np.zeros((nkv, 8, d), np.float16)
    V4[0] = 1.5
    V4[1] = -2.0
    o = O.gqa_decode(q, K, V4, 8, 0.1)
    assert np.allclose(o[:3], 1.5, atol=1e-14) and np.allclose(o[3:], -2.0, atol=1e-14)


# ---------------------------------------------------------------------------
# norm / activation / rope closed forms
# ---------------------------------------------------------------------------

def test_rmsnorm_constant_vector():
    g = synth.gamma(0, 0, synth.T_G1, 64)
    for c in (0.0, 1e-3, 2.5, -7.0):
        r = O.rmsnorm(np.full(64, c), g, 1e-6)
        assert np.allclose(r, g.astype(np.float64) * c / math.sqrt(c * c + 1e-6), rtol=1e-14, atol=0)


def test_silu_closed_forms():
    assert O.silu(0.0) == 0.0
    z = np.linspace(-3, 20, 93)
    assert np.allclose(O.silu(z), z * 0.5 * (1 + np.tanh(z / 2)), rtol=1e-13, atol=0)
    zn = np.linspace(-40, -0.5, 80)  # sigmoid(z) = e^z / (1 + e^z), stable for z < 0
    assert np.allclose(O.silu(zn), zn * np.exp(zn) / (1 + np.exp(zn)), rtol=1e-13, atol=0)
    assert abs(float(O.silu(math.log(3))) - 0.75 * math.log(3)) < 1e-15


def test_rope_closed_forms():
    d = 128
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, d))
    assert np.array_equal(O.rope(x, 0, 1e6), x)
    for p in (1, 17, 4000):
        r = O.rope(x, p, 1e6)
        assert np.allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    # pair (0, 64) rotates by angle p (frequency theta^0 = 1); pair (i, i+64) by p * theta^(-2i/d)
    e0 = np.zeros((1, d))
    e0[0, 0] = 1.0
    r = O.rope(e0, 5, 1e6)[0]
    assert abs(r[0] - math.cos(5)) < 1e-15 and abs(r[64] - math.sin(5)) < 1e-15
    assert np.count_nonzero(np.abs(r) > 1e-15) == 2
    e1 = np.zeros((1, d))
    e1[0, 64 + 3] = 1.0
    r = O.rope(e1, 7, 1e6)[0]
    ang = 7 * 1e6 ** (-6 / 128)
    assert abs(r[3] + math.sin(ang)) < 1e-15 and abs(r[67] - math.cos(ang)) < 1e-15
    # relative position: q(p+s) . k(r+s) independent of s
    q = rng.standard_normal((1, d))
    k = rng.standard_normal((1, d))
    dots = [float(np.sum(O.rope(q, 10 + s, 1e6) * O.rope(k, 3 + s, 1e6))) for s in (0, 100, 5000)]
    assert max(dots) - min(dots) < 1e-10


# ---------------------------------------------------------------------------
# lm_head + argmax
# ---------------------------------------------------------------------------

def test_argmax_ties_and_gap():
    z = np.array([0.5, 2.0, -1.0, 2.0, 1.999])
    i, gap = O.argmax_with_gap(z)
    assert i == 1 and gap == 0.0
    i, gap = O.argmax_with_gap(np.array([1.0, 3.0, 2.5]))
    assert i == 1 and gap == 0.5
    W = np.zeros((6, 32), np.float16)
    W[2, 0] = 1
    W[4, 0] = 1
    x = np.zeros((1, 32))
    x[0, 0] = 3.0
    logits, tok, gap = O.lm_head_argmax(W, x)
    assert tok[0] == 2 and gap[0] == 0.0 and logits[0, 4] == 3.0
