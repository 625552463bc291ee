"""GPU parity: packer / repacker / dequantiser (bit-exact) and the int4 GEMV (2e-3) against the
fp64 oracle, on the projection shapes of the 1.5B- and 7B-shaped decoders and on edge cases."""
import numpy as np
import pytest

from oracle import vv_oracle as O
from int4_blockwise_gemv_amd import synth
from gpu_util import dev, host, host_u16, codes_to_tiled, rel_err

pytestmark = pytest.mark.gpu

# (N, K): every projection shape of the 1.5B- and 7B-shaped layers, plus ragged edge cases
PROJ_SHAPES = [(1536, 1536), (256, 1536), (8960, 1536), (1536, 8960),
               (3584, 3584), (512, 3584), (18944, 3584), (3584, 18944)]
EDGE_SHAPES = [(1, 32), (100, 96), (65, 64), (130, 288), (7, 1024)]
TOL = 2e-3


def _pack_gpu(W, mode, tiled=False):
    import torch
    from int4_blockwise_gemv_amd import vv
    N, K = W.shape
    Wd = dev(W)
    ws = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    lay = vv.VV_LAYOUT_TILED if tiled else vv.VV_LAYOUT_ROWMAJOR
    q = torch.empty(vv.packed_bytes(N, K, lay), dtype=torch.uint8, device="cuda")
    s = torch.empty(vv.scale_bytes(N, K, lay) // 2, dtype=torch.int16, device="cuda")
    if tiled:
        vv.pack_int4_tiled(Wd, mode, 64, 64, 0, 64 * -(-N // 64), q, s, ws)
    else:
        vv.pack_int4(Wd, mode, q, s, ws)
    torch.cuda.synchronize()
    return q, s


@pytest.mark.parametrize("mode", ["ternary", "absmax"])
@pytest.mark.parametrize("shape", PROJ_SHAPES + EDGE_SHAPES)
def test_pack_rowmajor_bitexact(cuda, shape, mode):
    N, K = shape
    W = synth.master_weight(3, 1, synth.T_GATE, N, K)
    ref_q, ref_s = O.pack(W, mode)
    q, s = _pack_gpu(W, mode)
    assert np.array_equal(host(q).reshape(ref_q.shape), ref_q)
    assert np.array_equal(host_u16(s).reshape(ref_s.shape), ref_s)


@pytest.mark.parametrize("mode", ["ternary", "absmax"])
@pytest.mark.parametrize("shape", [(1536, 1536), (256, 1536), (3584, 18944)] + EDGE_SHAPES)
def test_pack_tiled_repack_dequant_bitexact(cuda, shape, mode):
    import torch
    from int4_blockwise_gemv_amd import vv
    N, K = shape
    W = synth.master_weight(4, 2, synth.T_DOWN, N, K)
    ref_q, ref_s = O.pack(W, mode)
    want_q, want_s = codes_to_tiled(O.unpack_nibbles(ref_q), ref_s)
    q, s = _pack_gpu(W, mode, tiled=True)
    assert np.array_equal(host(q), want_q)
    assert np.array_equal(host_u16(s), want_s)
    # row-major -> tiled permutation of the GPU's own row-major output
    rq, rs = _pack_gpu(W, mode)
    tq = torch.empty_like(q)
    ts = torch.empty_like(s)
    vv.repack_int4_tiled(rq, rs, N, K, 64, 64, 0, 64 * -(-N // 64), tq, ts)
    torch.cuda.synchronize()
    assert torch.equal(tq, q) and torch.equal(ts, s)
    # dequantised weights are exact in fp32 for both layouts
    ref_w = O.dequant(ref_q, ref_s)
    for lay, (pq, ps) in ((vv.VV_LAYOUT_ROWMAJOR, (rq, rs)), (vv.VV_LAYOUT_TILED, (q, s))):
        out = torch.empty((N, K), dtype=torch.float32, device="cuda")
        vv.dequant_int4(pq, ps, N, K, lay, out)
        torch.cuda.synchronize()
        assert np.array_equal(host(out).astype(np.float64), ref_w)


def test_pack_golden_blocks(cuda):
    from fractions import Fraction
    import os
    gold = os.path.join(os.path.dirname(__file__), "golden")
    for name, mode in (("ternary_hand_block.txt", "ternary"), ("absmax_hand_block.txt", "absmax")):
        d = {}
        for line in open(os.path.join(gold, name)):
            if line.strip() and not line.startswith("#"):
                k, v = line.split(":", 1)
                d[k.strip()] = v.split()
        W = np.array([[float(Fraction(w)) for w in d["W"]]], np.float32)
        q, s = _pack_gpu(W, mode)
        assert [int(b) for b in host(q)] == [int(b, 16) for b in d["bytes"]]
        assert int(host_u16(s)[0]) == int(d["scale_bits"][0], 16)


def test_pack_into_fused_buffer(cuda):
    """Row-range (q|k|v) and 32-row interleaved (gate/up) placement land where the layout note says."""
    import torch
    from int4_blockwise_gemv_amd import vv
    K = 256
    Wa = synth.master_weight(5, 0, synth.T_GATE, 96, K)
    Wb = synth.master_weight(5, 0, synth.T_UP, 96, K)
    rows = 192
    q = torch.zeros(vv.packed_bytes(rows, K, vv.VV_LAYOUT_TILED), dtype=torch.uint8, device="cuda")
    s = torch.zeros(vv.scale_bytes(rows, K, vv.VV_LAYOUT_TILED) // 2, dtype=torch.int16, device="cuda")
    ws = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    vv.pack_int4_tiled(dev(Wa), "ternary", 32, 64, 0, rows, q, s, ws)
    vv.pack_int4_tiled(dev(Wb), "ternary", 32, 64, 32, rows, q, s, ws)
    torch.cuda.synchronize()
    qa, sa = O.pack(Wa, "ternary")
    qb, sb = O.pack(Wb, "ternary")
    ca, cb = O.unpack_nibbles(qa), O.unpack_nibbles(qb)
    inter = np.concatenate([ca[0:32], cb[0:32], ca[32:64], cb[32:64], ca[64:96], cb[64:96]])
    inter_s = np.concatenate([sa[0:32], sb[0:32], sa[32:64], sb[32:64], sa[64:96], sb[64:96]])
    want_q, want_s = codes_to_tiled(inter, inter_s)
    assert np.array_equal(host(q), want_q) and np.array_equal(host_u16(s), want_s)
    # row-range placement: a 64-row block after 128 rows of something else
    q2 = torch.zeros_like(q)
    s2 = torch.zeros_like(s)
    vv.pack_int4_tiled(dev(Wa[:64]), "ternary", 64, 64, 128, rows, q2, s2, ws)
    torch.cuda.synchronize()
    qa2, sa2 = O.pack(Wa[:64], "ternary")
    want_q2, want_s2 = codes_to_tiled(O.unpack_nibbles(qa2), sa2)
    assert np.array_equal(host(q2)[-len(want_q2):], want_q2)
    assert np.array_equal(host_u16(s2)[-len(want_s2):], want_s2)
    assert not host(q2)[:-len(want_q2)].any()


# ---------------------------------------------------------------------------------------------
# GEMV
# ---------------------------------------------------------------------------------------------

def _gemv_gpu(q, s, N, K, x16, bias16=None, out_f16=False):
    import torch
    from int4_blockwise_gemv_amd import vv
    M = x16.shape[0]
    ws = torch.zeros(vv.gemv_workspace(M, N, K), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.float16 if out_f16 else torch.float32, device="cuda")
    xd = dev(x16)
    bd = dev(bias16) if bias16 is not None else None
    vv.gemv_int4(q, s, bd, xd, N, K, y, ws)
    torch.cuda.synchronize()
    return host(y).astype(np.float64)


@pytest.mark.parametrize("mode", ["ternary", "absmax"])
@pytest.mark.parametrize("shape", PROJ_SHAPES)
def test_gemv_projection_shapes(cuda, shape, mode):
    N, K = shape
    W = synth.master_weight(0, 0, synth.T_Q, N, K)
    x = synth.fp16_normal(0, 0, synth.T_X, (1, K))
    ref = O.gemv(*O.pack(W, mode), x)
    q, s = _pack_gpu(W, mode, tiled=True)
    y = _gemv_gpu(q, s, N, K, x)
    err = rel_err(y, ref)
    print(f"gemv {shape} {mode}: max rel err {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("mode", ["ternary", "absmax"])
@pytest.mark.parametrize("shape", [(37888, 3584), (40000, 3616)])
def test_gemv_grids_beyond_one_round(cuda, shape, mode, M):
    """Batch-1 and -2 grids with more workgroups than the chip holds at once (the later ones start
    as the first ones end): the 7B gate|up row count, and a ragged one (rows past a whole tile;
    K = 113 blocks, so a tile's last group holds a single block)."""
    N, K = shape
    W = synth.master_weight(4, 0, synth.T_Q, N, K)
    x = synth.fp16_normal(4, 0, synth.T_X, (M, K))
    ref = O.gemv(*O.pack(W, mode), x)
    q, s = _pack_gpu(W, mode, tiled=True)
    y = _gemv_gpu(q, s, N, K, x)
    err = rel_err(y, ref)
    print(f"gemv {shape} {mode}: max rel err {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 16])
@pytest.mark.parametrize("shape", [(100, 96), (1, 32), (130, 288), (1536, 1536), (256, 8960)])
def test_gemv_batched_ragged_with_bias(cuda, shape, M):
    N, K = shape
    W = synth.master_weight(1, 0, synth.T_K, N, K)
    x = synth.fp16_normal(1, M, synth.T_X, (M, K))
    b = synth.bias(1, 0, synth.T_BK, N)
    ref = O.gemv(*O.pack(W, "absmax"), x, b)
    q, s = _pack_gpu(W, "absmax", tiled=True)
    y = _gemv_gpu(q, s, N, K, x, b)
    assert rel_err(y, ref) <= TOL
    y16 = _gemv_gpu(q, s, N, K, x, b, out_f16=True)
    assert rel_err(y16, ref) <= TOL


def test_gemv_one_hot_columns_exact(cuda):
    """x = e_k returns column k of the dequantised matrix exactly (one product per output)."""
    N, K = 192, 512
    W = synth.master_weight(2, 0, synth.T_O, N, K)
    pq, ps = O.pack(W, "absmax")
    deq = O.dequant(pq, ps)
    q, s = _pack_gpu(W, "absmax", tiled=True)
    ks = [0, 1, 7, 31, 32, 255, 511]
    x = np.zeros((len(ks), K), np.float16)
    for i, k in enumerate(ks):
        x[i, k] = 1
    y = _gemv_gpu(q, s, N, K, x)
    for i, k in enumerate(ks):
        assert np.array_equal(y[i], deq[:, k])


@pytest.mark.parametrize("mode", ["ternary", "absmax"])
@pytest.mark.parametrize("shape", PROJ_SHAPES)
def test_gemv_batch16_projection_shapes(cuda, shape, mode):
    """16 rows (the matrix-core kernel) at every projection shape of both model widths."""
    N, K = shape
    W = synth.master_weight(3, 0, synth.T_Q, N, K)
    x = synth.fp16_normal(3, 16, synth.T_X, (16, K))
    ref = O.gemv(*O.pack(W, mode), x)
    q, s = _pack_gpu(W, mode, tiled=True)
    y = _gemv_gpu(q, s, N, K, x)
    err = rel_err(y, ref)
    print(f"gemv16 {shape} {mode}: max rel err {err:.2e}")
    assert err <= TOL


def test_gemv_deterministic(cuda):
    N, K = 3584, 18944
    W = synth.master_weight(0, 0, synth.T_DOWN, N, K)
    x = synth.fp16_normal(0, 0, synth.T_X, (1, K))
    q, s = _pack_gpu(W, "ternary", tiled=True)
    a = _gemv_gpu(q, s, N, K, x)
    b = _gemv_gpu(q, s, N, K, x)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------------------------
# GEMV on the MatMulNBits row-major bytes (vv_gemv_int4 with VV_LAYOUT_ROWMAJOR)
# ---------------------------------------------------------------------------------------------

def _gemv_rowmajor_gpu(q, s, N, K, x16, bias16=None, out_f16=False):
    import torch
    from int4_blockwise_gemv_amd import vv
    M = x16.shape[0]
    lay = vv.VV_LAYOUT_ROWMAJOR
    ws = torch.zeros(vv.gemv_workspace(M, N, K, lay), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.float16 if out_f16 else torch.float32, device="cuda")
    bd = dev(bias16) if bias16 is not None else None
    vv.gemv_int4(q, s, bd, dev(x16), N, K, y, ws, layout=lay)
    torch.cuda.synchronize()
    return host(y).astype(np.float64)


@pytest.mark.parametrize("mode", ["ternary", "absmax"])
@pytest.mark.parametrize("shape", PROJ_SHAPES)
def test_gemv_rowmajor_projection_shapes(cuda, shape, mode):
    """The row-major kernel on the GPU packer's MatMulNBits output, every projection shape."""
    N, K = shape
    W = synth.master_weight(6, 0, synth.T_V, N, K)
    x = synth.fp16_normal(6, 0, synth.T_X, (1, K))
    ref = O.gemv(*O.pack(W, mode), x)
    q, s = _pack_gpu(W, mode)
    y = _gemv_rowmajor_gpu(q, s, N, K, x)
    err = rel_err(y, ref)
    print(f"row-major gemv {shape} {mode}: max rel err {err:.2e}")
    assert err <= TOL


@pytest.mark.parametrize("M", [1, 2, 3, 5, 16])
@pytest.mark.parametrize("shape", [(100, 96), (1, 32), (130, 2080), (7, 4096), (256, 8960)])
def test_gemv_rowmajor_batched_ragged_with_bias(cuda, shape, M):
    """Ragged rows (not a multiple of the 16 rows of a workgroup), K past one 2048-element chunk
    and not a multiple of it, batches 1..16, bias, fp32 and fp16 outputs."""
    N, K = shape
    W = synth.master_weight(7, 0, synth.T_K, N, K)
    x = synth.fp16_normal(7, M, synth.T_X, (M, K))
    b = synth.bias(7, 0, synth.T_BK, N)
    ref = O.gemv(*O.pack(W, "absmax"), x, b)
    q, s = _pack_gpu(W, "absmax")
    assert rel_err(_gemv_rowmajor_gpu(q, s, N, K, x, b), ref) <= TOL
    assert rel_err(_gemv_rowmajor_gpu(q, s, N, K, x, b, out_f16=True), ref) <= TOL


def test_gemv_rowmajor_one_hot_columns_exact(cuda):
    """x = e_k returns column k of the dequantised matrix exactly: pins the nibble order of the
    row-major bytes (element 2j low nibble, 2j+1 high nibble) in the kernel's pairing."""
    N, K = 70, 2112
    W = synth.master_weight(8, 0, synth.T_O, N, K)
    pq, ps = O.pack(W, "absmax")
    deq = O.dequant(pq, ps)
    q, s = _pack_gpu(W, "absmax")
    ks = [0, 1, 2, 3, 4, 5, 6, 7, 8, 30, 31, 32, 2047, 2048, 2111]
    x = np.zeros((len(ks), K), np.float16)
    for i, k in enumerate(ks):
        x[i, k] = 1
    for r0 in range(0, len(ks), 16):
        y = _gemv_rowmajor_gpu(q, s, N, K, x[r0:r0 + 16])
        for i, k in enumerate(ks[r0:r0 + 16]):
            assert np.array_equal(y[i], deq[:, k]), k


# ---------------------------------------------------------------------------------------------
# degenerate weights: all-zero tensors and blocks, subnormal scales
# ---------------------------------------------------------------------------------------------

def test_pack_all_zero_ternary_tensor(cuda):
    """mean|W| = 0: every code 8, every scale 0 (both layouts); the GEMV then returns the bias."""
    N, K = 96, 160
    W = np.zeros((N, K), np.float32)
    ref_q, ref_s = O.pack(W, "ternary")
    assert (O.unpack_nibbles(ref_q) == 8).all() and (ref_s == 0).all()
    q, s = _pack_gpu(W, "ternary")
    assert np.array_equal(host(q).reshape(ref_q.shape), ref_q)
    assert np.array_equal(host_u16(s).reshape(ref_s.shape), ref_s)
    tq, ts = _pack_gpu(W, "ternary", tiled=True)
    want_q, want_s = codes_to_tiled(O.unpack_nibbles(ref_q), ref_s)
    assert np.array_equal(host(tq), want_q) and np.array_equal(host_u16(ts), want_s)
    x = synth.fp16_normal(9, 0, synth.T_X, (2, K))
    b = synth.bias(9, 0, synth.T_BQ, N)
    assert np.array_equal(_gemv_gpu(tq, ts, N, K, x, b), np.tile(b.astype(np.float64), (2, 1)))
    assert np.array_equal(_gemv_rowmajor_gpu(q, s, N, K, x, b), np.tile(b.astype(np.float64), (2, 1)))


def test_pack_absmax_all_zero_blocks(cuda):
    """General int4 with all-zero blocks (scale 0, codes 8), a whole zero row and a block whose
    only nonzero is a subnormal fp32 (absmax/7 underflows fp16 to 0: codes 8 too)."""
    N, K = 70, 256
    W = synth.master_weight(10, 0, synth.T_UP, N, K).copy()
    W[3, 32:64] = 0.0
    W[5, :] = 0.0
    W[9, 0:32] = 0.0
    W[9, 7] = np.float32(1e-40)
    W[69, 224:256] = 0.0
    ref_q, ref_s = O.pack(W, "absmax")
    assert ref_s[3, 1] == 0 and (ref_s[5] == 0).all() and ref_s[9, 0] == 0
    assert (O.unpack_nibbles(ref_q)[5] == 8).all()
    q, s = _pack_gpu(W, "absmax")
    assert np.array_equal(host(q).reshape(ref_q.shape), ref_q)
    assert np.array_equal(host_u16(s).reshape(ref_s.shape), ref_s)
    tq, ts = _pack_gpu(W, "absmax", tiled=True)
    want_q, want_s = codes_to_tiled(O.unpack_nibbles(ref_q), ref_s)
    assert np.array_equal(host(tq), want_q) and np.array_equal(host_u16(ts), want_s)
    x = synth.fp16_normal(10, 0, synth.T_X, (1, K))
    ref = O.gemv(ref_q, ref_s, x)
    assert rel_err(_gemv_gpu(tq, ts, N, K, x), ref) <= TOL
    assert rel_err(_gemv_rowmajor_gpu(q, s, N, K, x), ref) <= TOL


@pytest.mark.parametrize("M", [1, 16])
def test_gemv_subnormal_scales(cuda, M):
    """fp16 subnormal block scales (bits 0x0001..0x03ff, values down to 2^-24) are used exactly:
    both layouts against the oracle's exact dequantisation."""
    rng = np.random.default_rng(11)
    N, K = 130, 320
    codes = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    sbits = rng.integers(1, 0x400, size=(N, K // 32)).astype(np.uint16)
    sbits[0, 0] = 0x0001
    sbits[1, :] = 0x03FF
    pq = O.pack_nibbles(codes)
    x = synth.fp16_normal(11, M, synth.T_X, (M, K))
    ref = O.gemv(pq, sbits, x)
    assert np.max(np.abs(ref)) > 0
    tq, ts = codes_to_tiled(codes, sbits)
    y = _gemv_gpu(dev(tq), dev(ts), N, K, x)
    assert rel_err(y, ref) <= TOL
    y2 = _gemv_rowmajor_gpu(dev(pq.reshape(-1)), dev(sbits.reshape(-1)), N, K, x)
    assert rel_err(y2, ref) <= TOL
