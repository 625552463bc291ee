"""Test-side helpers: build oracle models from the seeded generators."""
import numpy as np

from oracle import vv_oracle as O
from int4_blockwise_gemv_amd import synth


def oracle_pack_layer(shape, seed, layer):
    """Oracle-packed projections of one layer: {name: (packed [N,K/32,16], scale_bits [N,K/32])}."""
    masters = synth.layer_masters(shape, seed, layer)
    return {nm: O.pack(W, shape.mode) for nm, W in masters.items()}


def oracle_layer(shape, seed, layer, packs=None):
    packs = packs if packs is not None else oracle_pack_layer(shape, seed, layer)
    sm = synth.layer_small(shape, seed, layer)
    return O.OLayer(q=packs["q"], k=packs["k"], v=packs["v"], o=packs["o"], gate=packs["gate"],
                    up=packs["up"], down=packs["down"], g1=sm["g1"], g2=sm["g2"],
                    bq=sm.get("bq"), bk=sm.get("bk"), bv=sm.get("bv"))


def oracle_model(shape, seed, layer_ids=None, with_lm=True, batch=1, packs=None, glob=None):
    layer_ids = range(shape.layers) if layer_ids is None else layer_ids
    layers = [oracle_layer(shape, seed, li, None if packs is None else packs[li]) for li in layer_ids]
    g = glob if glob is not None else synth.model_globals(shape, seed, batch, with_lm)
    return O.OModel(layers=layers, gf=g["gf"], lm=g.get("lm"), n_q=shape.n_q, n_kv=shape.n_kv,
                    head_dim=shape.head_dim, eps=shape.eps, rope_theta=shape.rope_theta)


def zero_proj(n, k):
    """Packed all-zero projection (codes 8, scale 0)."""
    return O.pack_nibbles(np.full((n, k), 8, np.uint8)), np.zeros((n, k // 32), np.uint16)


def scaled_identity_proj(n, c_bits, scale_bits):
    """n x n projection c * I via codes 15 (q - 8 = 7) on the diagonal and a chosen fp16 scale.

    With scale = c/7 exactly representable, the dequantised matrix is exactly c * I.
    """
    codes = np.full((n, n), 8, np.uint8)
    np.fill_diagonal(codes, c_bits)
    return O.pack_nibbles(codes), np.full((n, n // 32), scale_bits, np.uint16)


def _pack_layer_job(args):
    shape, seed, layer = args
    return layer, oracle_pack_layer(shape, seed, layer)


def oracle_packs_parallel(shape, seed, layer_ids, workers=None):
    """Oracle packing of several layers in worker processes (spawned: they import only numpy, the
    oracle and the seeded generators, never the GPU).  Returns {layer: packs}."""
    import os
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    layer_ids = list(layer_ids)
    if workers is None:
        try:
            ncpu = len(os.sched_getaffinity(0))
        except AttributeError:  # pragma: no cover
            ncpu = os.cpu_count() or 1
        workers = max(1, min(8, ncpu, len(layer_ids)))
    if workers == 1:
        return dict(_pack_layer_job((shape, seed, li)) for li in layer_ids)
    with ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn")) as ex:
        return dict(ex.map(_pack_layer_job, [(shape, seed, li) for li in layer_ids]))
