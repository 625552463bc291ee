"""Host check of the in-register dequantisation used by the int4 GEMV kernel: in the tiled
layout (include/vv.h) pair i of a dword sits in nibbles i and 4+i; after a shift by 4-4i bits
and an AND-OR with the fp16 bits of 64.0 (ulp 1/16), each half reads 64 + q exactly, and the
per-block correction 72 * sum(x) removes the offset and the zero point 8."""
import numpy as np

from gpu_util import codes_to_tiled


def _halves(u):
    return np.array([u & 0xFFFF, u >> 16], dtype=np.uint16).view(np.float16).astype(np.float64)


def _pairs(dw):
    return [((dw << 4) & 0x00F000F0) | 0x54005400, (dw & 0x00F000F0) | 0x54005400,
            ((dw >> 4) & 0x00F000F0) | 0x54005400, ((dw >> 8) & 0x00F000F0) | 0x54005400]


def test_magic_pairs_read_64_plus_code_in_every_slot():
    for q in range(16):
        for slot in range(8):
            dw = q << (4 * slot)
            pair, half = slot % 4, slot // 4
            vals = _halves(_pairs(dw)[pair])
            assert vals[half] == 64 + q and vals[1 - half] == 64


def test_one_hot_block_dot_equals_code_minus_zero_point():
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 16, size=(64, 32)).astype(np.uint8)
    q, _ = codes_to_tiled(codes, np.full((64, 1), 0x3C00, np.uint16))
    d = np.frombuffer(q.tobytes(), "<u4").reshape(64, 4)
    for lane in (0, 17, 63):
        for k in range(32):
            x = np.zeros(32, np.float16)
            x[k] = 1
            xu = np.frombuffer(x.tobytes(), "<u4")
            acc = sum((_halves(p) * _halves(int(xu[4 * w + j]))).sum()
                      for w in range(4) for j, p in enumerate(_pairs(int(d[lane, w]))))
            assert acc - 72 * float(x.astype(np.float64).sum()) == int(codes[lane, k]) - 8


# ---- exact code pairs and the 8-bit digit form of fp32 activations ----------------------------

def _exact_pairs(dw):
    """The exact code pairs: nibbles 0/4 and (after a byte shift) 2/6 under fp16 1024.0 less 1032,
    nibbles 1/5 and 3/7 under fp16 64.0 less 72 (element order (0,1), (2,3), (4,5), (6,7))."""
    d8 = dw >> 8
    raw = [(dw & 0x000F000F) | 0x64006400, (dw & 0x00F000F0) | 0x54005400,
           (d8 & 0x000F000F) | 0x64006400, (d8 & 0x00F000F0) | 0x54005400]
    off = [1032.0, 72.0, 1032.0, 72.0]
    return [_halves(r) - o for r, o in zip(raw, off)]


def test_exact_code_pairs_read_code_minus_8_in_every_slot():
    for q in range(16):
        for slot in range(8):
            dw = q << (4 * slot)
            elem = 2 * slot if slot < 4 else 2 * (slot - 4) + 1
            vals = np.concatenate(_exact_pairs(dw))
            want = np.full(8, -8.0)
            want[elem] = q - 8
            assert np.array_equal(vals, want), (q, slot)


def _perm(s0, s1, sel):
    """v_perm_b32: byte i of the result is byte sel_i of the 64-bit value (s0 << 32) | s1."""
    c = ((int(s0) & 0xFFFFFFFF) << 32) | (int(s1) & 0xFFFFFFFF)
    out = 0
    for i in range(4):
        b = (sel >> (8 * i)) & 0xFF
        out |= ((c >> (8 * b)) & 0xFF) << (8 * i)
    return out


def _sbytes(u):
    return [((int(u) >> (8 * i)) & 0xFF) - (256 if (int(u) >> (8 * i)) & 0x80 else 0) for i in range(4)]


def _stage_block(x):
    """The LDS image that the kernels' digit staging writes for one 32-element fp32 block, lane by
    lane as the 8 lanes compute it (lane r holds elements 4r..4r+3)."""
    x = np.asarray(x, np.float32)
    a = float(np.max(np.abs(x)))
    e = int(np.frexp(np.float32(a))[1]) if a > 0 else 0
    sh = 22 - e
    off = 128 * (1 + 256 + 65536)
    L = []
    for r in range(8):
        u = [int(np.rint(np.ldexp(np.float64(x[4 * r + i]), sh))) + off for i in range(4)]
        p01, p23 = _perm(u[1], u[0], 0x05010400), _perm(u[3], u[2], 0x05010400)
        q01, q23 = _perm(u[1], u[0], 0x06020602), _perm(u[3], u[2], 0x06020602)
        L.append([_perm(p23, p01, 0x05040100) ^ 0x80808080, _perm(p23, p01, 0x07060302) ^ 0x80808080,
                  _perm(q23, q01, 0x05040100) ^ 0x80808080])
    blk = [0] * 28
    for r in range(8):
        sel = 0x03070206 if r & 1 else 0x05010400
        for k in range(3):
            blk[8 * k + r] = _perm(L[r ^ 1][k], L[r][k], sel)
    for k in range(3):
        blk[25 + k] = -8 * sum(sum(_sbytes(L[r][k])) for r in range(8))
    scale = float(np.ldexp(np.float32(1.0), e - 22))
    return blk, scale, sh


def _block_dot(codes_dw, blk):
    """The kernels' integer block dot: per level, sdot4 of (codes & 0x0F0F0F0F) and
    ((codes >> 4) & 0x0F0F0F0F) with the staged digit dwords, started at -8 sum(d)."""
    S = []
    for k in range(3):
        t = blk[25 + k]
        for w in range(4):
            lo, hi = codes_dw[w] & 0x0F0F0F0F, (codes_dw[w] >> 4) & 0x0F0F0F0F
            t += sum(a * b for a, b in zip(_sbytes(lo), _sbytes(blk[8 * k + 2 * w])))
            t += sum(a * b for a, b in zip(_sbytes(hi), _sbytes(blk[8 * k + 2 * w + 1])))
        S.append(t)
    return S


def test_digit_staging_and_integer_block_dot_are_exact():
    """Random blocks over many magnitudes (zeros, single non-zero, all equal, negative, huge and
    tiny): the digits decode to X_i = rint(x_i 2^(22-e)) with |X_i| <= 2^22 and every digit a
    signed byte; the integer block dot equals sum_i (q_i - 8) X_i exactly, for codes in the tiled
    layout's nibble order."""
    rng = np.random.default_rng(7)
    blocks = [rng.standard_normal(32) * 10.0 ** rng.integers(-30, 30) for _ in range(60)]
    blocks += [np.zeros(32), np.eye(32)[5] * -3.5, np.full(32, 0.75), -np.abs(rng.standard_normal(32)),
               np.full(32, 2.0 ** 100), np.full(32, 2.0 ** -120), np.array([2.0 ** 22 - 1] + [1.0] * 31)]
    for x in blocks:
        x = np.asarray(x, np.float32)
        blk, scale, sh = _stage_block(x)
        X = np.rint(np.ldexp(x.astype(np.float64), sh)).astype(np.int64)
        assert np.max(np.abs(X)) <= 2 ** 22
        # decode the image back to X, element by element
        order = [(0, 4, 1, 5), (2, 6, 3, 7)]
        dec = np.zeros(32, np.int64)
        for k in range(3):
            for w in range(4):
                for h in range(2):
                    for j, el in enumerate(order[h]):
                        dec[8 * w + el] += _sbytes(blk[8 * k + 2 * w + h])[j] * 256 ** k
        assert np.array_equal(dec, X)
        codes = rng.integers(0, 16, 32)
        q, _ = codes_to_tiled(codes[None, :].astype(np.uint8).repeat(64, 0), np.zeros((64, 1), np.uint16))
        dw = [int(v) for v in np.frombuffer(q.tobytes(), "<u4").reshape(64, 4)[0]]
        S = _block_dot(dw, blk)
        assert S[0] + 256 * S[1] + 65536 * S[2] == int(np.sum((codes - 8) * X))
        assert all(abs(s) <= 32 * 15 * 128 + 8 * 32 * 128 for s in S)
        # the kernel's fp32 combination: one rounding of the exact sum, then an exact power of two
        t = np.float32(np.float32(S[2]) * np.float32(65536) + np.float32(np.float32(S[1]) * 256 + S[0]))
        exact = float(np.sum((codes - 8) * X))
        assert abs(float(t) - exact) <= abs(exact) * 2.0 ** -24 + 1e-30
        assert scale == 2.0 ** (-sh)
