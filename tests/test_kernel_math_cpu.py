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
