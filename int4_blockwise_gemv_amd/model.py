"""Device-side model and state for the decode step, built from seeded fp32 masters.

Orchestration only: the masters are uploaded and packed on the GPU by vv_pack_int4_tiled into
the fused layouts the decode step reads (q|k|v rows in one tiled matrix; each gate/up tile holds
32 gate rows and the same 32 up rows), and the ctypes structs of include/vv.h are filled with the
device pointers.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np

from . import synth
from . import vv

TILE = 64


def _cdiv(a, b):
    return (a + b - 1) // b


def _dev_u16(a: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


class TiledMatrix:
    """A tiled int4 buffer holding one or more projections (placed by row groups)."""

    def __init__(self, tiles: int, K: int, device):
        import torch
        self.tiles, self.K = tiles, K
        rows = tiles * TILE
        self.q = torch.empty(vv.packed_bytes(rows, K, vv.VV_LAYOUT_TILED), dtype=torch.uint8, device=device)
        self.s = torch.empty(vv.scale_bytes(rows, K, vv.VV_LAYOUT_TILED) // 2, dtype=torch.int16, device=device)

    def pack(self, W_dev, mode: str, row_offset: int, ws, row_group: int = TILE, group_stride: int = TILE):
        vv.pack_int4_tiled(W_dev, mode, row_group, group_stride, row_offset, self.tiles * TILE, self.q, self.s, ws)


@dataclass
class DeviceLayer:
    qkv: TiledMatrix
    o: TiledMatrix
    gu: TiledMatrix
    down: TiledMatrix
    bias: Optional[object]
    g1: object
    g2: object


class DeviceModel:
    """Packed weights of a decoder on the current CUDA device plus its vv_model struct."""

    def __init__(self, shape, seed: int, layer_ids: Optional[Sequence[int]] = None, with_lm: bool = True,
                 max_batch: int = 1, masters: Optional[Callable[[int], Dict[str, np.ndarray]]] = None,
                 lm: Optional[np.ndarray] = None, gf: Optional[np.ndarray] = None, device="cuda",
                 progress: Optional[Callable[[str], None]] = None):
        import torch
        self.shape = shape
        self.device = device
        self.layer_ids = list(range(shape.layers)) if layer_ids is None else list(layer_ids)
        H, I, d = shape.hidden, shape.inter, shape.head_dim
        nq_rows, nkv_rows = shape.n_q * d, shape.n_kv * d
        nqkv = nq_rows + 2 * nkv_rows
        assert nq_rows % TILE == 0 and nkv_rows % TILE == 0 and H % TILE == 0 and I % TILE == 0
        ws = torch.empty(max(256, vv.pack_workspace(1, 32, shape.mode)), dtype=torch.uint8, device=device)
        self.layers: List[DeviceLayer] = []
        for li in self.layer_ids:
            Ms = masters(li) if masters is not None else synth.layer_masters(shape, seed, li)
            sm = synth.layer_small(shape, seed, li)
            dev = {k: torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(device) for k, v in Ms.items()}
            L = DeviceLayer(qkv=TiledMatrix(nqkv // TILE, H, device), o=TiledMatrix(H // TILE, nq_rows, device),
                            gu=TiledMatrix(2 * (I // TILE), H, device), down=TiledMatrix(H // TILE, I, device),
                            bias=None, g1=_dev_u16(sm["g1"], device), g2=_dev_u16(sm["g2"], device))
            L.qkv.pack(dev["q"], shape.mode, 0, ws)
            L.qkv.pack(dev["k"], shape.mode, nq_rows, ws)
            L.qkv.pack(dev["v"], shape.mode, nq_rows + nkv_rows, ws)
            L.o.pack(dev["o"], shape.mode, 0, ws)
            # each gate/up tile: 32 gate rows (lanes 0-31) then the same 32 up rows (lanes 32-63)
            L.gu.pack(dev["gate"], shape.mode, 0, ws, row_group=32, group_stride=TILE)
            L.gu.pack(dev["up"], shape.mode, 32, ws, row_group=32, group_stride=TILE)
            L.down.pack(dev["down"], shape.mode, 0, ws)
            if shape.qkv_bias:
                L.bias = _dev_u16(np.concatenate([sm["bq"], sm["bk"], sm["bv"]]), device)
            torch.cuda.synchronize()
            del dev
            self.layers.append(L)
            if progress:
                progress(f"layer {li} packed")
        glob = synth.model_globals(shape, seed, 1, with_lm=with_lm and lm is None)
        self.gf = _dev_u16(gf if gf is not None else glob["gf"], device)
        lm_host = lm if lm is not None else glob.get("lm")
        self.lm = _dev_u16(lm_host, device) if lm_host is not None else None
        self.max_batch = max_batch
        self._build_struct()

    def _build_struct(self):
        s = self.shape
        arr = (vv.vv_layer * max(1, len(self.layers)))()
        for i, L in enumerate(self.layers):
            arr[i] = vv.vv_layer(L.qkv.q.data_ptr(), L.qkv.s.data_ptr(), L.o.q.data_ptr(), L.o.s.data_ptr(),
                                 L.gu.q.data_ptr(), L.gu.s.data_ptr(), L.down.q.data_ptr(), L.down.s.data_ptr(),
                                 L.bias.data_ptr() if L.bias is not None else None, L.g1.data_ptr(), L.g2.data_ptr())
        self._layer_arr = arr
        self.struct = vv.vv_model(len(self.layers), s.hidden, s.inter, s.n_q, s.n_kv, s.head_dim, s.vocab,
                                  self.max_batch, s.eps, s.rope_theta, C.cast(arr, C.POINTER(vv.vv_layer)),
                                  self.gf.data_ptr(), self.lm.data_ptr() if self.lm is not None else None)

    def weight_bytes(self) -> int:
        """Algorithmic bytes of the packed int4 weights (nibbles + fp16 scales of the real rows)."""
        s = self.shape
        per = sum(n * k // 2 + n * (k // 32) * 2 for _, n, k in s.proj_shapes())
        return per * len(self.layers)


class DeviceState:
    """KV caches, inputs, outputs and workspace of one decode step."""

    def __init__(self, model: DeviceModel, batch: int, cap: int, device="cuda", trace: bool = False,
                 logits: bool = True, path: str = "auto", kv: str = "f16"):
        import torch
        s = model.shape
        self.model, self.batch, self.cap = model, batch, cap
        L = len(model.layers)
        kv_dtype = {"f16": torch.float16, "f32": torch.float32}[kv]
        self.k = torch.zeros((max(1, L), batch, s.n_kv, cap, s.head_dim), dtype=kv_dtype, device=device)
        self.v = torch.zeros_like(self.k)
        self.emb = torch.zeros((batch, s.hidden), dtype=torch.float16, device=device)
        self.pos = torch.zeros(batch, dtype=torch.int32, device=device)
        self.logits = torch.empty((batch, s.vocab), dtype=torch.float32, device=device) if logits else None
        self.token = torch.zeros(batch, dtype=torch.int32, device=device)
        self.trace = torch.zeros((L + 1, batch, s.hidden), dtype=torch.float32, device=device) if trace else None
        nbytes = vv.step_workspace(model.struct, batch, cap)
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        self.struct = vv.vv_state(batch, cap, self.emb.data_ptr(), self.pos.data_ptr(), self.k.data_ptr(),
                                  self.v.data_ptr(), self.logits.data_ptr() if logits else None,
                                  self.token.data_ptr(), self.trace.data_ptr() if trace else None,
                                  self.ws.data_ptr(), nbytes, None, 0, vv.PATH[path])
        self.struct.kv_dtype = vv.VV_F32 if kv == "f32" else vv.VV_F16

    def enable_feedback(self, stop_ids=(151645, 151643), table=None):
        """Closed-loop greedy decoding: every step gathers the embedding of its argmax token from
        `table` (default: the model's lm_head, the tied fp16 table) as the next input, advances the
        positions and records the tokens in `history` [B][cap] (position-indexed); a stop token
        marks its sequence in `done`."""
        import torch
        assert 0 <= len(stop_ids) <= 4
        tab = table if table is not None else self.model.lm
        self.history = torch.full((self.batch, self.cap), -1, dtype=torch.int32, device=self.emb.device)
        self.done = torch.zeros(self.batch, dtype=torch.int32, device=self.emb.device)
        self._feedback_table = tab
        self.struct.feedback_table = tab.data_ptr()
        self.struct.history = self.history.data_ptr()
        self.struct.done = self.done.data_ptr()
        for i, t in enumerate(stop_ids):
            self.struct.stop_ids[i] = int(t)
        self.struct.n_stop = len(stop_ids)

    def load_cache_layer(self, idx: int, K: np.ndarray, V: np.ndarray):
        import torch
        self.k[idx].copy_(torch.from_numpy(K))
        self.v[idx].copy_(torch.from_numpy(V))

    def prefill(self, embeds, stream=None):
        """decoder_init of sequence 0 (batch-1 states): the prompt embeddings `embeds` (torch fp16
        [S][H] on the device) fill cache positions 0..S-1 of every layer; the last position's
        logits go to logits[0] and its greedy token to token[0].  The next decode step continues
        at pos = S (set by the caller)."""
        import torch
        assert self.batch == 1, "prefill runs one sequence"
        S = int(embeds.shape[0])
        need = vv.prefill_workspace(self.model.struct, S, self.cap)
        if getattr(self, "_pf_ws", None) is None or self._pf_ws.numel() < need:
            self._pf_ws = torch.zeros(need, dtype=torch.uint8, device=self.emb.device)
        vv.prefill(self.model.struct, embeds, S, self.k, self.v, self.cap, self.logits, self.token, self._pf_ws,
                   stream)

    def step(self, stream=None):
        vv.decode_step(self.model.struct, self.struct, stream)

    def path(self) -> str:
        """The launch plan of this state's steps ("layered" or "chained")."""
        return vv.decode_path(self.model.struct, self.struct)

    def status(self, stream=None) -> int:
        return vv.decode_status(self.model.struct, self.struct, stream)

    def graph(self, stream=None) -> vv.DecodeGraph:
        return vv.DecodeGraph(self.model.struct, self.struct, stream)
