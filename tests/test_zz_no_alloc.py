"""The allocation-free lm_head + argmax (vv_lm_head_argmax_noalloc) against the workspace entry
point (vv_lm_head_argmax), both through the C ABI: the same kernels, so logits and tokens must
agree bit for bit, on two calls in a row whose second is smaller (the scratch array keeps the first
call's contents), on the vector-ALU (batch 1) and matrix-core (batch 16) paths, and against the
oracle's lm_head and argmax."""
import numpy as np
import pytest

from oracle import vv_oracle as O
from int4_blockwise_gemv_amd import synth
from gpu_util import dev, host, rel_err

pytestmark = pytest.mark.gpu


def _both(W, x):
    import torch
    from int4_blockwise_gemv_amd import vv
    V, H = W.shape
    B = x.shape[0]
    Wd, xd = dev(W), dev(x)
    ws = torch.zeros(vv.lm_workspace(B, V, H), dtype=torch.uint8, device="cuda")
    l_ws = torch.empty((B, V), dtype=torch.float32, device="cuda")
    t_ws = torch.full((B,), -5, dtype=torch.int32, device="cuda")
    vv.lm_head_argmax(Wd, xd, l_ws, t_ws, ws)
    l_na = torch.empty((B, V), dtype=torch.float32, device="cuda")
    t_na = torch.full((B,), -5, dtype=torch.int32, device="cuda")
    vv.lm_head_argmax_noalloc(Wd, xd, l_na, t_na)
    torch.cuda.synchronize()
    return host(l_ws), host(t_ws), host(l_na), host(t_na)


def _check(W, x):
    l_ws, t_ws, l_na, t_na = _both(W, x)
    assert np.array_equal(l_na, l_ws)
    assert np.array_equal(t_na, t_ws)
    ref, _, _ = O.lm_head_argmax(W, x.astype(np.float64))
    assert rel_err(l_na.astype(np.float64), ref) <= 2e-3
    for b in range(ref.shape[0]):
        i, gap = O.argmax_with_gap(ref[b])
        if gap >= 1e-3:
            assert int(t_na[b]) == i


@pytest.mark.parametrize("B", [1, 16])
def test_noalloc_matches_workspace_entry_point_twice(cuda, B):
    """A large call, then a smaller one (fewer rows, a narrower table) on the same scratch."""
    W1 = synth.fp16_normal(7, 0, synth.T_LM, (151936, 1536), std=0.02)
    x1 = synth.fp16_normal(7, 1, synth.T_EMB, (B, 1536)).astype(np.float32)
    _check(W1, x1)
    Bs = max(1, B // 2)
    W2 = synth.fp16_normal(8, 0, synth.T_LM, (40000, 1024), std=0.02)
    x2 = synth.fp16_normal(8, 1, synth.T_EMB, (Bs, 1024)).astype(np.float32)
    _check(W2, x2)


def test_noalloc_rejects_more_keys_than_its_scratch(cuda):
    """16 rows over 3M vocabulary rows of width 256 (the matrix-core plan, ~6000 workgroups) need more
    keys than the 256 KiB scratch holds: the call is rejected on the host before anything runs (the
    buffers are never touched)."""
    import ctypes as C
    import torch
    from int4_blockwise_gemv_amd import vv
    B, V, H = 16, 3 << 20, 256
    assert vv.lm_workspace(B, V, H) > 256 * 1024
    buf = torch.zeros(64, dtype=torch.int32, device="cuda")
    p = C.c_void_p(buf.data_ptr())
    rc = vv.lib().vv_lm_head_argmax_noalloc(p, p, vv.VV_F32, B, V, H, None, p, None)
    assert rc == vv.VV_ERR_RANGE
