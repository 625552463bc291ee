"""Seeded synthetic inputs for the int4 block-32 decode step.

This module only draws random numbers and states workload shapes.  It holds
none of the method's arithmetic (no quantisation, packing, norms, attention or
GEMV): both the HIP path and the fp64 oracle consume the arrays it returns.

Recipe (the same for every consumer):

* every int4-quantised projection starts from an fp32 master
  ``W = float32(standard_normal) * float32(0.02)`` drawn by
  ``numpy.random.default_rng([seed, layer, tensor_id, chunk])`` over fixed
  row chunks (``rows_per_chunk(K)`` rows each), so the values do not depend
  on how many threads draw them;
* RMSNorm weights ``gamma = fp16(1 + 0.1 * N(0,1))``; q/k/v biases
  ``fp16(0.02 * N(0,1))``;
* the KV cache, the input embeddings and the stand-alone GEMV activation are
  ``fp16(N(0,1))``;
* the lm_head table is ``fp16(0.02 * N(0,1))``, row-major ``[V, H]``;
* long-context caches scale K and V by 8 at ``round(0.01 * P)`` positions per
  layer, drawn without replacement;
* ragged batches draw each sequence's past length uniformly from an inclusive
  integer range.

The shapes are those of the VibeVoice Qwen2 decoders (1.5B-shaped: hidden 1536,
28 layers, 12 query / 2 KV heads, head_dim 128, intermediate 8960; 7B-shaped:
hidden 3584, 28 query / 4 KV heads, intermediate 18944), vocabulary 151936.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# tensor ids used in the seed tuple
T_Q, T_K, T_V, T_O, T_GATE, T_UP, T_DOWN = 0, 1, 2, 3, 4, 5, 6
T_G1, T_G2, T_BQ, T_BK, T_BV, T_KC, T_VC = 7, 8, 9, 10, 11, 12, 13
T_GF, T_LM, T_EMB, T_X, T_OUTL, T_LENS, T_QATT = 20, 21, 22, 23, 24, 25, 26
GLOBAL_LAYER = 10_000  # "layer" index used for per-model (not per-layer) tensors

PROJ_NAMES = ("q", "k", "v", "o", "gate", "up", "down")
PROJ_TID = {"q": T_Q, "k": T_K, "v": T_V, "o": T_O, "gate": T_GATE, "up": T_UP, "down": T_DOWN}

_CHUNK_ELEMS = 1 << 20


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def rows_per_chunk(ncols: int) -> int:
    return max(1, _CHUNK_ELEMS // max(1, ncols))


def _normal_rows(seed_key, nrows: int, ncols: int, std: float, out_dtype, threads: Optional[int] = None):
    """fp32 N(0, std) matrix [nrows, ncols], chunked by rows with per-chunk seeds."""
    out = np.empty((nrows, ncols), dtype=out_dtype)
    rpc = rows_per_chunk(ncols)
    nchunks = (nrows + rpc - 1) // rpc
    stdf = np.float32(std)

    def work(c):
        r0 = c * rpc
        r1 = min(nrows, r0 + rpc)
        g = np.random.default_rng(list(seed_key) + [c])
        a = g.standard_normal((r1 - r0, ncols), dtype=np.float32)
        if std != 1.0:
            a *= stdf
        out[r0:r1] = a.astype(out_dtype, copy=False)

    nt = threads or _threads()
    if nchunks == 1 or nt == 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def master_weight(seed: int, layer: int, tid: int, n: int, k: int, std: float = 0.02) -> np.ndarray:
    """fp32 master [n, k] ~ N(0, std)."""
    return _normal_rows((seed, layer, tid), n, k, std, np.float32)


def fp16_normal(seed: int, layer: int, tid: int, shape, std: float = 1.0) -> np.ndarray:
    shape = tuple(int(s) for s in shape)
    ncols = shape[-1]
    nrows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    return _normal_rows((seed, layer, tid), nrows, ncols, std, np.float16).reshape(shape)


def gamma(seed: int, layer: int, tid: int, n: int) -> np.ndarray:
    g = np.random.default_rng([seed, layer, tid, 0]).standard_normal(n, dtype=np.float32)
    return (np.float32(1.0) + np.float32(0.1) * g).astype(np.float16)


def bias(seed: int, layer: int, tid: int, n: int) -> np.ndarray:
    g = np.random.default_rng([seed, layer, tid, 0]).standard_normal(n, dtype=np.float32)
    return (np.float32(0.02) * g).astype(np.float16)


def outlier_positions(seed: int, layer: int, past: int, frac: float = 0.01) -> np.ndarray:
    cnt = int(round(frac * past))
    g = np.random.default_rng([seed, layer, T_OUTL, 0])
    return np.sort(g.choice(past, size=cnt, replace=False))


def ragged_lengths(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    g = np.random.default_rng([seed, GLOBAL_LAYER, T_LENS, 0])
    return g.integers(lo, hi, size=batch, endpoint=True).astype(np.int32)


# ---------------------------------------------------------------------------
# workload shapes
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class ModelShape:
    name: str
    layers: int
    hidden: int
    n_q: int
    n_kv: int
    head_dim: int
    inter: int
    vocab: int
    mode: str = "ternary"          # "ternary" | "absmax"
    qkv_bias: bool = True
    eps: float = 1e-6
    rope_theta: float = 1e6

    @property
    def q_dim(self):
        return self.n_q * self.head_dim

    @property
    def kv_dim(self):
        return self.n_kv * self.head_dim

    def proj_shapes(self):
        """(name, N rows, K cols) of every int4 projection of one layer."""
        H, I = self.hidden, self.inter
        return [("q", self.q_dim, H), ("k", self.kv_dim, H), ("v", self.kv_dim, H),
                ("o", H, self.q_dim), ("gate", I, H), ("up", I, H), ("down", H, I)]


@dataclass(frozen=True)
class Workload:
    name: str
    shape: ModelShape
    batch: int
    past: int                      # P for batch 1 (new token written at index P)
    cap: int                       # cache capacity (positions)
    seeds: tuple = (0,)
    outlier_frac: float = 0.0
    ragged: Optional[tuple] = None  # (lo, hi) inclusive past-length range for batch > 1
    notes: str = ""


QWEN2_1P5B = ModelShape("qwen2-1.5b-shaped", 28, 1536, 12, 2, 128, 8960, 151936)
QWEN2_7B = ModelShape("qwen2-7b-shaped", 28, 3584, 28, 4, 128, 18944, 151936)
QWEN2_7B_ABSMAX = ModelShape("qwen2-7b-shaped-absmax", 28, 3584, 28, 4, 128, 18944, 151936, mode="absmax")
# the Realtime-0.5B decoder shape (20 layers, hidden 896 = 28 blocks per row; Qwen2-0.5B heads and
# intermediate size), for the lock-step CFG pair (batch 2) and single-sequence decoding
QWEN2_0P5B = ModelShape("qwen2-0.5b-shaped", 20, 896, 14, 2, 128, 4864, 151936)

WORKLOADS = {
    "single-layer-1536": Workload("single-layer-1536", QWEN2_1P5B, 1, 256, 256, (0,),
                                  notes="one [1536x1536] ternary GEMV + GQA 12/2 over 256 positions"),
    "decode-1.5b-p4096": Workload("decode-1.5b-p4096", QWEN2_1P5B, 1, 4096, 4097, tuple(range(10))),
    "decode-7b-p4000": Workload("decode-7b-p4000", QWEN2_7B, 1, 4000, 4001, tuple(range(5))),
    "decode-7b-absmax-p16384": Workload("decode-7b-absmax-p16384", QWEN2_7B_ABSMAX, 1, 16384, 16385, (0,),
                                        outlier_frac=0.01),
    "decode-0.5b-cfg-b2": Workload("decode-0.5b-cfg-b2", QWEN2_0P5B, 2, 2048, 2049, (0,),
                                   notes="lock-step classifier-free-guidance pair: 2 sequences at P = 2048"),
    "decode-1.5b-b16-ragged": Workload("decode-1.5b-b16-ragged", QWEN2_1P5B, 16, 0, 8193, (0,),
                                       ragged=(512, 8192)),
}


def past_lengths(w: Workload, seed: int) -> np.ndarray:
    if w.ragged is not None:
        return ragged_lengths(seed, w.batch, *w.ragged)
    return np.full(w.batch, w.past, dtype=np.int32)


# ---------------------------------------------------------------------------
# per-layer / per-model tensor bundles (host numpy)
# ---------------------------------------------------------------------------

def layer_masters(shape: ModelShape, seed: int, layer: int) -> dict:
    """fp32 masters of the seven projections of one layer."""
    return {nm: master_weight(seed, layer, PROJ_TID[nm], n, k) for nm, n, k in shape.proj_shapes()}


def layer_small(shape: ModelShape, seed: int, layer: int) -> dict:
    d = {"g1": gamma(seed, layer, T_G1, shape.hidden), "g2": gamma(seed, layer, T_G2, shape.hidden)}
    if shape.qkv_bias:
        d["bq"] = bias(seed, layer, T_BQ, shape.q_dim)
        d["bk"] = bias(seed, layer, T_BK, shape.kv_dim)
        d["bv"] = bias(seed, layer, T_BV, shape.kv_dim)
    return d


def layer_cache(w: Workload, seed: int, layer: int, lens: np.ndarray):
    """fp16 K and V caches of one layer, [B, n_kv, cap, head_dim]; positions >= len are zero."""
    s = w.shape
    B, cap, d = w.batch, w.cap, s.head_dim
    K = np.zeros((B, s.n_kv, cap, d), np.float16)
    V = np.zeros((B, s.n_kv, cap, d), np.float16)
    maxlen = int(lens.max())
    kf = fp16_normal(seed, layer, T_KC, (B, s.n_kv, maxlen, d))
    vf = fp16_normal(seed, layer, T_VC, (B, s.n_kv, maxlen, d))
    for b in range(B):
        L = int(lens[b])
        K[b, :, :L] = kf[b, :, :L]
        V[b, :, :L] = vf[b, :, :L]
    if w.outlier_frac > 0:
        for b in range(B):
            pos = outlier_positions(seed, layer, int(lens[b]), w.outlier_frac)
            K[b, :, pos] *= np.float16(8)
            V[b, :, pos] *= np.float16(8)
    return K, V


def model_globals(shape: ModelShape, seed: int, batch: int, with_lm: bool = True) -> dict:
    d = {"gf": gamma(seed, GLOBAL_LAYER, T_GF, shape.hidden),
         "emb": fp16_normal(seed, GLOBAL_LAYER, T_EMB, (batch, shape.hidden))}
    if with_lm:
        d["lm"] = fp16_normal(seed, GLOBAL_LAYER, T_LM, (shape.vocab, shape.hidden), std=0.02)
    return d


@dataclass
class TinyShape:
    """Small decoder used by the oracle's own self-consistency tests."""
    layers: int = 2
    hidden: int = 256
    n_q: int = 2
    n_kv: int = 1
    head_dim: int = 128
    inter: int = 512
    vocab: int = 1000
    mode: str = "ternary"
    qkv_bias: bool = True
    eps: float = 1e-6
    rope_theta: float = 1e6
    name: str = "tiny"

    q_dim = property(lambda self: self.n_q * self.head_dim)
    kv_dim = property(lambda self: self.n_kv * self.head_dim)
    proj_shapes = ModelShape.proj_shapes
