"""The C-ABI library loads, exports every symbol include/vv.h declares, and rejects bad
arguments on the host before anything is enqueued (no GPU needed for these paths)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vv.h")

vvmod = pytest.importorskip("int4_blockwise_gemv_amd.vv")


def _lib():
    if not os.path.exists(vvmod.LIB_PATH):
        pytest.skip("libvv.so not built (run __graft_entry__.build())")
    return vvmod.lib()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(vv_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("vv_pack_int4", "vv_gemv_int4", "vv_gqa_decode", "vv_decode_step", "vv_lm_head_argmax",
                     "vv_decode_graph_create", "vv_decode_graph_launch", "vv_decode_graph_destroy"):
        assert required in names


def test_library_exports_every_declared_symbol():
    L = _lib()
    missing = [n for n in _declared_functions() if not hasattr(L, n)]
    assert not missing, missing
    assert set(_declared_functions()) == set(vvmod.exported_symbols())


def test_status_strings_and_version():
    _lib()
    assert vvmod.status_string(0) == "ok"
    assert "workspace" in vvmod.status_string(vvmod.VV_ERR_WORKSPACE)
    assert vvmod.version() >= 100


def test_layout_sizes():
    _lib()
    # 1536 x 1536: 48 blocks per row, 24 tiles
    assert vvmod.packed_bytes(1536, 1536, vvmod.VV_LAYOUT_ROWMAJOR) == 1536 * 48 * 16
    assert vvmod.scale_bytes(1536, 1536, vvmod.VV_LAYOUT_ROWMAJOR) == 1536 * 48 * 2
    assert vvmod.packed_bytes(100, 96, vvmod.VV_LAYOUT_TILED) == 2 * 3 * 64 * 16
    assert vvmod.scale_bytes(100, 96, vvmod.VV_LAYOUT_TILED) == 2 * 1 * 64 * 16
    assert vvmod.packed_bytes(10, 33, vvmod.VV_LAYOUT_TILED) == 0


def _call(fn, *args):
    L = _lib()
    return getattr(L, fn)(*args)


P = C.c_void_p


def test_pack_validation():
    L = _lib()
    dummy = P(64)
    assert L.vv_pack_int4(None, 4, 32, 0, dummy, dummy, dummy, 4096, None) == vvmod.VV_ERR_NULL
    assert L.vv_pack_int4(dummy, 4, 33, 0, dummy, dummy, dummy, 4096, None) == vvmod.VV_ERR_SHAPE
    assert L.vv_pack_int4(dummy, 0, 32, 0, dummy, dummy, dummy, 4096, None) == vvmod.VV_ERR_RANGE
    assert L.vv_pack_int4(dummy, 4, 32, 7, dummy, dummy, dummy, 4096, None) == vvmod.VV_ERR_DTYPE
    assert L.vv_pack_int4(dummy, 4, 32, 0, dummy, dummy, dummy, 16, None) == vvmod.VV_ERR_WORKSPACE
    # destination row out of range: 100 rows in groups of 64 -> rows up to 127 + offset 64 >= 128
    assert L.vv_pack_int4_tiled(dummy, 100, 32, 0, 64, 64, 64, 128, dummy, dummy, dummy, 4096,
                                None) == vvmod.VV_ERR_RANGE
    assert "destination row" in vvmod.last_error()
    assert L.vv_pack_int4_tiled(dummy, 100, 32, 0, 64, 64, 0, 100, dummy, dummy, dummy, 4096,
                                None) == vvmod.VV_ERR_RANGE
    assert L.vv_pack_int4_tiled(dummy, 100, 32, 0, 32, 16, 0, 256, dummy, dummy, dummy, 4096,
                                None) == vvmod.VV_ERR_RANGE
    assert L.vv_repack_int4_tiled(dummy, None, 4, 32, 64, 64, 0, 64, dummy, dummy, None) == vvmod.VV_ERR_NULL
    assert L.vv_dequant_int4(dummy, dummy, 4, 32, 5, dummy, None) == vvmod.VV_ERR_DTYPE


def test_gemv_validation():
    L = _lib()
    d = P(64)
    T, R = vvmod.VV_LAYOUT_TILED, vvmod.VV_LAYOUT_ROWMAJOR
    for lay in (T, R):
        assert L.vv_gemv_int4(None, d, None, d, 1, 64, 64, lay, d, 2, d, 1 << 20, None) == vvmod.VV_ERR_NULL
        assert L.vv_gemv_int4(d, d, None, d, 0, 64, 64, lay, d, 2, d, 1 << 20, None) == vvmod.VV_ERR_RANGE
        assert L.vv_gemv_int4(d, d, None, d, 17, 64, 64, lay, d, 2, d, 1 << 20, None) == vvmod.VV_ERR_RANGE
        assert L.vv_gemv_int4(d, d, None, d, 1, 64, 48, lay, d, 2, d, 1 << 20, None) == vvmod.VV_ERR_SHAPE
        assert L.vv_gemv_int4(d, d, None, d, 1, 64, 64, lay, d, 9, d, 1 << 20, None) == vvmod.VV_ERR_DTYPE
        assert L.vv_gemv_int4(d, d, None, d, 1, 64, 64, lay, d, 2, None, 1 << 20, None) == vvmod.VV_ERR_WORKSPACE
        assert L.vv_gemv_int4(P(65), d, None, d, 1, 64, 64, lay, d, 2, d, 1 << 20, None) == vvmod.VV_ERR_RANGE
        assert vvmod.gemv_workspace(1, 1536, 1536, lay) > 0
    assert L.vv_gemv_int4(d, d, None, d, 1, 64, 64, T, d, 2, d, 4, None) == vvmod.VV_ERR_WORKSPACE
    # unknown layout; row-major scales need only 2-byte alignment, tiled ones 16
    assert L.vv_gemv_int4(d, d, None, d, 1, 64, 64, 5, d, 2, d, 1 << 20, None) == vvmod.VV_ERR_DTYPE
    assert vvmod.gemv_workspace(1, 64, 64, 5) == 0
    assert L.vv_gemv_int4(d, P(66), None, d, 1, 64, 64, T, d, 2, d, 1 << 20, None) == vvmod.VV_ERR_RANGE
    assert L.vv_gemv_int4(d, P(67), None, d, 1, 64, 64, R, d, 2, d, 1 << 20, None) == vvmod.VV_ERR_RANGE


def test_stream_read_validation():
    L = _lib()
    d = P(64)
    assert L.vv_stream_read(None, 32768, d, None) == vvmod.VV_ERR_NULL
    assert L.vv_stream_read(d, 32768, None, None) == vvmod.VV_ERR_NULL
    assert L.vv_stream_read(d, 0, d, None) == vvmod.VV_ERR_RANGE
    assert L.vv_stream_read(d, 32768 + 16, d, None) == vvmod.VV_ERR_RANGE
    assert L.vv_stream_read(P(72), 32768, d, None) == vvmod.VV_ERR_RANGE


def test_gqa_validation():
    L = _lib()
    d = P(64)
    big = 1 << 24
    assert L.vv_gqa_decode(d, 2, d, d, d, 1, 12, 2, 256, 64, 0.1, d, 2, d, big, None) == vvmod.VV_ERR_SHAPE
    assert L.vv_gqa_decode(d, 2, d, d, d, 1, 12, 5, 256, 128, 0.1, d, 2, d, big, None) == vvmod.VV_ERR_SHAPE
    assert L.vv_gqa_decode(d, 2, d, d, d, 1, 18, 2, 256, 128, 0.1, d, 2, d, big, None) == vvmod.VV_ERR_SHAPE
    assert L.vv_gqa_decode(d, 2, d, d, None, 1, 12, 2, 256, 128, 0.1, d, 2, d, big, None) == vvmod.VV_ERR_NULL
    assert L.vv_gqa_decode(d, 3, d, d, d, 1, 12, 2, 256, 128, 0.1, d, 2, d, big, None) == vvmod.VV_ERR_DTYPE
    assert L.vv_gqa_decode(d, 2, d, d, d, 0, 12, 2, 256, 128, 0.1, d, 2, d, big, None) == vvmod.VV_ERR_RANGE
    assert L.vv_gqa_decode(d, 2, d, d, d, 1, 12, 2, 256, 128, 0.1, d, 2, d, 8, None) == vvmod.VV_ERR_WORKSPACE


def test_gqa_split_plan_bounds():
    """The split-KV partials take (8 heads x 132 floats) per split; a sequence never gets more than
    1024 splits (the merge's limit): one KV head at the largest capacity switches to 128-position
    splits even though its workgroup count alone would keep 64."""
    rec = 8 * 132 * 4
    align = lambda n: (n + 255) // 256 * 256
    assert vvmod.gqa_workspace(1, 8, 1, 131072) == align(1024 * rec)          # 128-position splits
    assert vvmod.gqa_workspace(1, 8, 1, 65536) == align(1024 * rec)           # 64-position splits
    assert vvmod.gqa_workspace(1, 8, 4, 4000) == align(4 * 63 * rec)          # 64-position splits
    assert vvmod.gqa_workspace(16, 12, 2, 8192) == align(16 * 2 * 64 * rec)   # > 2048 workgroups: 128


def test_lm_head_validation():
    L = _lib()
    d = P(64)
    big = 1 << 24
    assert L.vv_lm_head_argmax(d, d, 2, 1, 1000, 12, None, d, d, big, None) == vvmod.VV_ERR_SHAPE
    assert L.vv_lm_head_argmax(d, d, 2, 17, 1000, 64, None, d, d, big, None) == vvmod.VV_ERR_RANGE
    assert L.vv_lm_head_argmax(d, d, 2, 1, 1000, 64, None, None, d, big, None) == vvmod.VV_ERR_NULL
    assert L.vv_lm_head_argmax(d, d, 2, 1, 1000, 64, None, d, d, 8, None) == vvmod.VV_ERR_WORKSPACE


def _model_struct(**over):
    vv = vvmod
    layers = (vv.vv_layer * 1)()
    layers[0] = vv.vv_layer(*([64] * 8), None, 64, 64)
    kw = dict(n_layers=1, hidden=256, inter=512, n_q=4, n_kv=2, head_dim=128, vocab=1000, max_batch=4, eps=1e-6,
              rope_theta=1e6, layers=C.cast(layers, C.POINTER(vv.vv_layer)), gf=64, lm_head=64)
    kw.update(over)
    m = vv.vv_model(**kw)
    m._keep = layers
    return m


def _state(ws_bytes, **over):
    kw = dict(batch=1, cap=64, input_embeds=64, pos=64, k_cache=64, v_cache=64, logits=None, token=64, h_trace=None,
              workspace=256, workspace_bytes=ws_bytes, events=None, n_events=0, path=0)
    kw.update(over)
    return vvmod.vv_state(**kw)


def test_decode_step_validation():
    L = _lib()
    m = _model_struct()
    need = vvmod.step_workspace(m, 1, 64)
    assert need > 0
    s = _state(need)
    assert L.vv_decode_step(C.byref(_model_struct(head_dim=64)), C.byref(s), None) == vvmod.VV_ERR_SHAPE
    assert L.vv_decode_step(C.byref(_model_struct(hidden=200)), C.byref(s), None) == vvmod.VV_ERR_SHAPE
    assert L.vv_decode_step(C.byref(_model_struct(n_kv=3)), C.byref(s), None) == vvmod.VV_ERR_SHAPE
    assert L.vv_decode_step(C.byref(m), C.byref(_state(need, batch=5)), None) == vvmod.VV_ERR_RANGE
    assert L.vv_decode_step(C.byref(m), C.byref(_state(need - 1)), None) == vvmod.VV_ERR_WORKSPACE
    assert L.vv_decode_step(C.byref(m), C.byref(_state(need, pos=None)), None) == vvmod.VV_ERR_NULL
    assert L.vv_decode_step(C.byref(_model_struct(lm_head=None)), C.byref(s), None) == vvmod.VV_ERR_NULL
    assert L.vv_decode_step(C.byref(m), C.byref(_state(need, workspace=300)), None) == vvmod.VV_ERR_RANGE
    evs = (C.c_void_p * 4)()
    ev = C.cast(evs, C.POINTER(C.c_void_p))
    lay = vvmod.VV_PATH_LAYERED
    # a start/stop pair per operation: 2 (5 L + 2)
    assert L.vv_decode_step(C.byref(m), C.byref(_state(need, events=ev, n_events=4, path=lay)), None) == \
        vvmod.VV_ERR_RANGE
    # unknown path; the chained path with a batch, a cache or a KV precision it does not serve
    assert L.vv_decode_step(C.byref(m), C.byref(_state(need, path=7)), None) == vvmod.VV_ERR_RANGE
    ch = vvmod.VV_PATH_CHAINED
    need3 = vvmod.step_workspace(m, 3, 64)
    assert L.vv_decode_step(C.byref(m), C.byref(_state(need3, batch=3, path=ch)), None) == vvmod.VV_ERR_UNSUPPORTED
    assert L.vv_decode_step(C.byref(m), C.byref(_state(need, path=ch)), None) == vvmod.VV_ERR_UNSUPPORTED  # 1 split
    st32 = _state(vvmod.step_workspace(m, 1, 128), cap=128, path=ch)   # 2 splits, but fp32 caches
    st32.kv_dtype = vvmod.VV_F32
    assert L.vv_decode_step(C.byref(m), C.byref(st32), None) == vvmod.VV_ERR_UNSUPPORTED
    st = C.c_int32(0)
    assert L.vv_decode_status(None, C.byref(s), C.byref(st), None) == vvmod.VV_ERR_NULL
    assert L.vv_decode_status(C.byref(m), C.byref(s), None, None) == vvmod.VV_ERR_NULL
    h = C.c_void_p()
    evs14 = (C.c_void_p * 14)()   # enough pairs for the one-layer model: 2 (5 + 2)
    assert L.vv_decode_graph_create(C.byref(m), C.byref(_state(need, events=C.cast(evs14, C.POINTER(C.c_void_p)),
                                                              n_events=14)), None, C.byref(h)) == vvmod.VV_ERR_UNSUPPORTED
    assert L.vv_decode_graph_create(C.byref(_model_struct(head_dim=64)), C.byref(s), None,
                                    C.byref(h)) == vvmod.VV_ERR_SHAPE
    assert h.value is None
    assert L.vv_decode_graph_launch(None, None) == vvmod.VV_ERR_NULL
    assert L.vv_decode_graph_destroy(None) == vvmod.VV_OK


def test_lm_head_noalloc_validation():
    """The allocation-free lm_head rejects bad arguments, and inputs needing more argmax keys than its
    256 KiB scratch, on the host (no GPU call is made on these paths)."""
    L = _lib()
    d = P(64)
    assert L.vv_lm_head_argmax_noalloc(None, d, vvmod.VV_F32, 1, 100, 64, None, d, None) == vvmod.VV_ERR_NULL
    assert L.vv_lm_head_argmax_noalloc(d, d, vvmod.VV_F32, 0, 100, 64, None, d, None) == vvmod.VV_ERR_RANGE
    assert L.vv_lm_head_argmax_noalloc(d, d, vvmod.VV_F32, 1, 100, 60, None, d, None) == vvmod.VV_ERR_SHAPE
    assert L.vv_lm_head_argmax_noalloc(d, d, 9, 1, 100, 64, None, d, None) == vvmod.VV_ERR_DTYPE
    assert vvmod.lm_workspace(16, 3 << 20, 256) > 256 * 1024
    assert L.vv_lm_head_argmax_noalloc(d, d, vvmod.VV_F32, 16, 3 << 20, 256, None, d, None) == vvmod.VV_ERR_RANGE


def test_decode_step_event_count_follows_the_launch_plan():
    """The layered plan times one operation per launch: at batch 1 each down projection shares its
    launch with the next layer's q|k|v (prep, q|k|v of layer 0, 4 per layer, lm_head: 4 L + 3 pairs),
    at larger batches 5 L + 2 pairs.  Checked on the rejection of one event too few (host only)."""
    L = _lib()
    vv = vvmod
    layers = (vv.vv_layer * 2)()
    for i in range(2):
        layers[i] = vv.vv_layer(*([64] * 8), None, 64, 64)
    m = _model_struct(n_layers=2, layers=C.cast(layers, C.POINTER(vv.vv_layer)))
    m._keep = layers
    lay = vv.VV_PATH_LAYERED
    for batch, pairs in ((1, 4 * 2 + 3), (2, 5 * 2 + 2)):
        need = vv.step_workspace(m, batch, 64)
        evs = (C.c_void_p * (2 * pairs - 1))()
        st = _state(need, batch=batch, events=C.cast(evs, C.POINTER(C.c_void_p)), n_events=2 * pairs - 1, path=lay)
        assert L.vv_decode_step(C.byref(m), C.byref(st), None) == vv.VV_ERR_RANGE
        assert f"at least {2 * pairs} entries" in L.vv_last_error().decode()
