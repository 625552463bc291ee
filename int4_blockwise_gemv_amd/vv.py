"""Thin ctypes binding of libvv (the C ABI declared in include/vv.h).

Argument marshalling only: every computation runs in the HIP kernels of libvv.so.  torch is
used for device memory (tensor.data_ptr()) and streams (torch.cuda.current_stream()).  Loading
fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libvv.so")

VV_OK = 0
VV_ERR_NULL, VV_ERR_SHAPE, VV_ERR_RANGE, VV_ERR_DTYPE = -1, -2, -3, -4
VV_ERR_WORKSPACE, VV_ERR_UNSUPPORTED, VV_ERR_HIP = -5, -6, -7
VV_Q_TERNARY, VV_Q_ABSMAX = 0, 1
VV_F16, VV_F32 = 1, 2
VV_LAYOUT_ROWMAJOR, VV_LAYOUT_TILED = 0, 1
VV_PATH_AUTO, VV_PATH_LAYERED, VV_PATH_CHAINED = 0, 1, 2
PATH = {"auto": VV_PATH_AUTO, "layered": VV_PATH_LAYERED, "chained": VV_PATH_CHAINED}
MODE = {"ternary": VV_Q_TERNARY, "absmax": VV_Q_ABSMAX}


class VVError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn} -> {status}: {msg}")
        self.status = status


class vv_layer(C.Structure):
    _fields_ = [("qkv_q", C.c_void_p), ("qkv_s", C.c_void_p), ("o_q", C.c_void_p), ("o_s", C.c_void_p),
                ("gu_q", C.c_void_p), ("gu_s", C.c_void_p), ("down_q", C.c_void_p), ("down_s", C.c_void_p),
                ("qkv_bias", C.c_void_p), ("g1", C.c_void_p), ("g2", C.c_void_p)]


class vv_model(C.Structure):
    _fields_ = [("n_layers", C.c_int), ("hidden", C.c_int), ("inter", C.c_int), ("n_q", C.c_int),
                ("n_kv", C.c_int), ("head_dim", C.c_int), ("vocab", C.c_int), ("max_batch", C.c_int),
                ("eps", C.c_float), ("rope_theta", C.c_float), ("layers", C.POINTER(vv_layer)),
                ("gf", C.c_void_p), ("lm_head", C.c_void_p)]


class vv_state(C.Structure):
    _fields_ = [("batch", C.c_int), ("cap", C.c_int), ("input_embeds", C.c_void_p), ("pos", C.c_void_p),
                ("k_cache", C.c_void_p), ("v_cache", C.c_void_p), ("logits", C.c_void_p), ("token", C.c_void_p),
                ("h_trace", C.c_void_p), ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
                ("events", C.POINTER(C.c_void_p)), ("n_events", C.c_int), ("path", C.c_int),
                ("feedback_table", C.c_void_p), ("history", C.c_void_p), ("done", C.c_void_p),
                ("stop_ids", C.c_int32 * 4), ("n_stop", C.c_int), ("kv_dtype", C.c_int)]


_I64, _SZ, _P, _I, _F = C.c_int64, C.c_size_t, C.c_void_p, C.c_int, C.c_float

_SIGS = {
    "vv_packed_bytes": (_SZ, [_I64, _I64, _I]),
    "vv_scale_bytes": (_SZ, [_I64, _I64, _I]),
    "vv_pack_int4_workspace": (_SZ, [_I64, _I64, _I]),
    "vv_pack_int4": (_I, [_P, _I64, _I64, _I, _P, _P, _P, _SZ, _P]),
    "vv_pack_int4_tiled": (_I, [_P, _I64, _I64, _I, _I64, _I64, _I64, _I64, _P, _P, _P, _SZ, _P]),
    "vv_repack_int4_tiled": (_I, [_P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _P, _P, _P]),
    "vv_dequant_int4": (_I, [_P, _P, _I64, _I64, _I, _P, _P]),
    "vv_gemv_int4_workspace": (_SZ, [_I64, _I64, _I64, _I]),
    "vv_gemv_int4": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _I, _P, _SZ, _P]),
    "vv_gqa_decode_workspace": (_SZ, [_I, _I, _I, _I]),
    "vv_gqa_decode": (_I, [_P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _I, _P, _SZ, _P]),
    "vv_lm_head_argmax_workspace": (_SZ, [_I, _I, _I]),
    "vv_lm_head_argmax": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "vv_lm_head_argmax_noalloc": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P]),
    "vv_decode_step_workspace": (_SZ, [C.POINTER(vv_model), _I, _I]),
    "vv_decode_step": (_I, [C.POINTER(vv_model), C.POINTER(vv_state), _P]),
    "vv_decode_path": (_I, [C.POINTER(vv_model), C.POINTER(vv_state)]),
    "vv_decode_status": (_I, [C.POINTER(vv_model), C.POINTER(vv_state), C.POINTER(C.c_int32), _P]),
    "vv_decode_graph_create": (_I, [C.POINTER(vv_model), C.POINTER(vv_state), _P, C.POINTER(_P)]),
    "vv_decode_graph_launch": (_I, [_P, _P]),
    "vv_decode_graph_destroy": (_I, [_P]),
    "vv_prefill_workspace": (_SZ, [C.POINTER(vv_model), _I, _I]),
    "vv_prefill": (_I, [C.POINTER(vv_model), _P, _I, _P, _P, _I, _I, _P, _P, _P, _SZ, _P]),
    "vv_workspace_init": (_I, [_P, _SZ, _P]),
    "vv_stream_read": (_I, [_P, _SZ, _P, _P]),
    "vv_status_string": (C.c_char_p, [_I]),
    "vv_last_error": (C.c_char_p, []),
    "vv_version": (_I, []),
}

_lib = None


def lib():
    """The loaded libvv.so (raises when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libvv.so not found at {LIB_PATH}; build it with "
                               "`python -m int4_blockwise_gemv_amd.build` (there is no fallback path)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGS)


def _check(rc: int, fn: str):
    if rc != VV_OK:
        raise VVError(rc, fn, lib().vv_last_error().decode(errors="replace"))


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(t):
    import torch
    if t.dtype == torch.float16:
        return VV_F16
    if t.dtype == torch.float32:
        return VV_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


# --------------------------------------------------------------------------------------------
# wrappers (tensors are torch CUDA tensors; fp16 data may be float16 or int16/uint16 bit views)
# --------------------------------------------------------------------------------------------

def packed_bytes(rows, K, layout):
    return lib().vv_packed_bytes(rows, K, layout)


def scale_bytes(rows, K, layout):
    return lib().vv_scale_bytes(rows, K, layout)


def pack_workspace(N, K, mode):
    return lib().vv_pack_int4_workspace(N, K, MODE.get(mode, mode))


def pack_int4(W, mode, packed, scales, ws, stream=None):
    N, K = W.shape
    _check(lib().vv_pack_int4(_ptr(W), N, K, MODE.get(mode, mode), _ptr(packed), _ptr(scales), _ptr(ws),
                              0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)), "vv_pack_int4")


def pack_int4_tiled(W, mode, row_group, group_stride, row_offset, dst_rows, packed, scales, ws, stream=None):
    N, K = W.shape
    _check(lib().vv_pack_int4_tiled(_ptr(W), N, K, MODE.get(mode, mode), row_group, group_stride, row_offset, dst_rows,
                                    _ptr(packed), _ptr(scales), _ptr(ws),
                                    0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "vv_pack_int4_tiled")


def repack_int4_tiled(packed, scales, N, K, row_group, group_stride, row_offset, dst_rows, tiled, tiled_scales,
                      stream=None):
    _check(lib().vv_repack_int4_tiled(_ptr(packed), _ptr(scales), N, K, row_group, group_stride, row_offset, dst_rows,
                                      _ptr(tiled), _ptr(tiled_scales), _stream(stream)), "vv_repack_int4_tiled")


def dequant_int4(packed, scales, N, K, layout, out, stream=None):
    _check(lib().vv_dequant_int4(_ptr(packed), _ptr(scales), N, K, layout, _ptr(out), _stream(stream)),
           "vv_dequant_int4")


def gemv_workspace(M, N, K, layout=VV_LAYOUT_TILED):
    return lib().vv_gemv_int4_workspace(M, N, K, layout)


def gemv_int4(packed, scales, bias, x, N, K, y, ws, stream=None, layout=VV_LAYOUT_TILED):
    M = x.shape[0]
    _check(lib().vv_gemv_int4(_ptr(packed), _ptr(scales), _ptr(bias), _ptr(x), M, N, K, layout, _ptr(y),
                              _dtype_code(y), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "vv_gemv_int4")


def gqa_workspace(B, nq, nkv, cap):
    return lib().vv_gqa_decode_workspace(B, nq, nkv, cap)


def gqa_decode(q, k_cache, v_cache, lens, softmax_scale, out, ws, stream=None):
    B, nq, d = q.shape
    _, nkv, cap, _ = k_cache.shape
    _check(lib().vv_gqa_decode(_ptr(q), _dtype_code(q), _ptr(k_cache), _ptr(v_cache), _ptr(lens), B, nq, nkv, cap, d,
                               float(softmax_scale), _ptr(out), _dtype_code(out), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(stream)), "vv_gqa_decode")


def lm_workspace(B, V, H):
    return lib().vv_lm_head_argmax_workspace(B, V, H)


def lm_head_argmax(W, x, logits, token, ws, stream=None):
    V, H = W.shape
    B = x.shape[0]
    _check(lib().vv_lm_head_argmax(_ptr(W), _ptr(x), _dtype_code(x), B, V, H, _ptr(logits), _ptr(token), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream)), "vv_lm_head_argmax")


def lm_head_argmax_noalloc(W, x, logits, token, stream=None):
    """vv_lm_head_argmax without a workspace (the library's scratch array holds the argmax keys)."""
    V, H = W.shape
    B = x.shape[0]
    _check(lib().vv_lm_head_argmax_noalloc(_ptr(W), _ptr(x), _dtype_code(x), B, V, H, _ptr(logits), _ptr(token),
                                           _stream(stream)), "vv_lm_head_argmax_noalloc")


def stream_read(buf, sink, stream=None):
    """One streaming read of the whole tensor `buf` (its byte size a multiple of 32768)."""
    _check(lib().vv_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)),
           "vv_stream_read")


def step_workspace(model: vv_model, batch: int, cap: int) -> int:
    return lib().vv_decode_step_workspace(C.byref(model), batch, cap)


def decode_step(model: vv_model, state: vv_state, stream=None):
    _check(lib().vv_decode_step(C.byref(model), C.byref(state), _stream(stream)), "vv_decode_step")


def decode_path(model: vv_model, state: vv_state) -> str:
    """The launch plan a decode step takes for this model and state ("layered" or "chained")."""
    rc = lib().vv_decode_path(C.byref(model), C.byref(state))
    if rc < 0:
        _check(rc, "vv_decode_path")
    return {VV_PATH_LAYERED: "layered", VV_PATH_CHAINED: "chained"}[rc]


def decode_status(model: vv_model, state: vv_state, stream=None) -> int:
    """Sticky status word of the step (0 = every bounded in-kernel wait was satisfied)."""
    out = C.c_int32(-1)
    _check(lib().vv_decode_status(C.byref(model), C.byref(state), C.byref(out), _stream(stream)), "vv_decode_status")
    return int(out.value)


def prefill_workspace(model: vv_model, S: int, cap: int) -> int:
    return lib().vv_prefill_workspace(C.byref(model), S, cap)


def prefill(model: vv_model, input_embeds, S: int, k_cache, v_cache, cap: int, logits, token, ws, stream=None):
    _check(lib().vv_prefill(C.byref(model), _ptr(input_embeds), S, _ptr(k_cache), _ptr(v_cache), cap,
                            _dtype_code(k_cache), _ptr(logits), _ptr(token), _ptr(ws), ws.numel() * ws.element_size(),
                            _stream(stream)), "vv_prefill")


class DecodeGraph:
    """hipGraph of one decode step (vv_decode_graph_*)."""

    def __init__(self, model: vv_model, state: vv_state, stream=None):
        h = C.c_void_p()
        _check(lib().vv_decode_graph_create(C.byref(model), C.byref(state), _stream(stream), C.byref(h)),
               "vv_decode_graph_create")
        self._h = h

    def launch(self, stream=None):
        _check(lib().vv_decode_graph_launch(self._h, _stream(stream)), "vv_decode_graph_launch")

    def close(self):
        if self._h:
            lib().vv_decode_graph_destroy(self._h)
            self._h = None

    def __del__(self):  # pragma: no cover
        try:
            self.close()
        except Exception:
            pass


def workspace_init(ws, stream=None):
    _check(lib().vv_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "vv_workspace_init")


def status_string(s: int) -> str:
    return lib().vv_status_string(s).decode()


def last_error() -> str:
    return lib().vv_last_error().decode(errors="replace")


def version() -> int:
    return lib().vv_version()
