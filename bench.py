"""Decode-step benchmark (one JSON line on stdout).

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode-7b-p4000] [--seed 0]

One step = one vv_decode_step (28 layers: fused QKV GEMV, attention with KV append, o GEMV,
gate/up GEMV + SiLU, down GEMV, then lm_head + argmax) replayed from a hipGraph on seeded
synthetic weights, KV cache and input already resident in HBM.  The timed region is K
back-to-back replays bracketed by torch.cuda.synchronize().  --path picks the implementation
(auto = layered: one launch per stage; persistent = all layers in one launch).

Also reported:
  roofline     achieved HBM GB/s of the dominant kernel, = its algorithmic bytes per launch / its
               mean duration measured with HIP events on the launch stream during instrumented
               eager steps right after the timed region.  Persistent path: the layer kernel
               (int4 weights + scales + K/V of every layer); layered path: the gate/up GEMV.
               traffic: from committed rocprofv3 counters when they match the kernel source.
  cpu_baseline the fp64 oracle's decode step timed on a bounded sample of the same workload
               (one layer + a vocabulary slice, scaled to a full step).

python bench.py --prefill S [--workload ...] times the prefill (decoder_init) of an S-token prompt
of the workload's model instead and prints its own line (tokens/s; matrix TFLOP/s against the
fp16 matrix-core peak).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def algorithmic_bytes(shape, batch, lens, kv_bytes=2):
    """Bytes one step must read: packed nibbles + fp16 scales + fp16 lm_head + K/V over P+1
    (kv_bytes per element: 2 for fp16 caches, 4 for the fp32-KV variant)."""
    per_layer_w = sum(n * k // 2 + n * (k // 32) * 2 for _, n, k in shape.proj_shapes())
    w = per_layer_w * shape.layers
    kv = sum(int(L) + 1 for L in lens) * shape.n_kv * shape.head_dim * 2 * kv_bytes * shape.layers
    lm = shape.vocab * shape.hidden * 2
    return w, kv, lm


def kernel_source_hash(files=("gemv.hip", "gemv_core.h", "vv_internal.h")):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "int4_blockwise_gemv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_tag, files):
    """HBM bytes per launch from profiles/traffic_<tag>.txt if it was taken on the current source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_tag}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != kernel_source_hash(files):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def build_inputs(wl, seed, path="auto", kv="f16"):
    import torch
    from int4_blockwise_gemv_amd import synth
    from int4_blockwise_gemv_amd.model import DeviceModel, DeviceState
    s = wl.shape
    lens = synth.past_lengths(wl, seed)
    t0 = time.time()
    dm = DeviceModel(s, seed, max_batch=wl.batch, progress=lambda m: None)
    log(f"packed {s.layers} layers + lm_head on the GPU in {time.time() - t0:.1f}s")
    ds = DeviceState(dm, wl.batch, wl.cap, path=path, kv=kv)
    for li in range(s.layers):
        K, V = synth.layer_cache(wl, seed, li, lens)
        if kv == "f32":
            K, V = K.astype(np.float32), V.astype(np.float32)
        ds.load_cache_layer(li, K, V)
    g = synth.model_globals(s, seed, wl.batch, with_lm=False)
    ds.emb.copy_(torch.from_numpy(g["emb"].view(np.int16)).view(torch.float16).cuda())
    ds.pos.copy_(torch.from_numpy(lens).cuda())
    torch.cuda.synchronize()
    log(f"inputs resident ({time.time() - t0:.1f}s total)")
    return dm, ds, lens


def kernel_breakdown(ds, n_layers, steps, persistent):
    """Mean kernel time (ms) per operation of the step over `steps` eager steps.

    Each operation's kernels are launched with hipExtLaunchKernel start/stop events, which
    receive the kernels' own dispatch start and end times (the values rocprofv3 reports), not the
    time the stream reaches a marker."""
    import ctypes as C
    import torch
    if persistent:
        names = ["layers", "lm_head"]
    else:
        names = ["prep"] + ["qkv", "attn", "o", "gateup", "down"] * n_layers + ["lm_head"]
    n_ev = 2 * len(names)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    for e in evs:  # torch creates the HIP event on first record
        e.record()
    torch.cuda.synchronize()
    arr = (C.c_void_p * n_ev)(*[C.c_void_p(e.cuda_event) for e in evs])
    ds.struct.events = C.cast(arr, C.POINTER(C.c_void_p))
    ds.struct.n_events = n_ev
    acc = {k: [] for k in names}
    try:
        for _ in range(steps):
            ds.step()
            torch.cuda.synchronize()
            for i, k in enumerate(names):
                acc[k].append(evs[2 * i].elapsed_time(evs[2 * i + 1]))
    finally:
        ds.struct.events = None
        ds.struct.n_events = 0
    return {k: float(np.mean(v)) for k, v in acc.items()}


def cpu_baseline(wl, seed, budget_s=25.0):
    """The oracle's decode step on a bounded sample: one layer and a slice of the vocabulary."""
    from threadpoolctl import threadpool_info
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle import vv_oracle as O
    from int4_blockwise_gemv_amd import synth
    from helpers import oracle_model
    s = wl.shape
    lens = synth.past_lengths(wl, seed)
    li = 0
    m = oracle_model(s, seed, [li], with_lm=False, batch=wl.batch)
    K, V = synth.layer_cache(wl, seed, li, lens)
    h = synth.model_globals(s, seed, wl.batch, with_lm=False)["emb"].astype(np.float64)
    t0 = time.perf_counter()
    O.layer_step(m.layers[0], m, h, lens, K, V)
    t_layer = time.perf_counter() - t0
    frac_rows = 16384
    lm = synth.fp16_normal(seed, synth.GLOBAL_LAYER, synth.T_LM, (frac_rows, s.hidden), std=0.02)
    f = O.rmsnorm(h, m.gf, m.eps)
    t0 = time.perf_counter()
    O.lm_head_argmax(lm, f)
    t_lm = (time.perf_counter() - t0) * s.vocab / frac_rows
    t_step = t_layer * s.layers + t_lm
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    return {"value": 1.0 / t_step, "unit": "decode steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"1 of {s.layers} layers (layer {li}) + {frac_rows} of {s.vocab} lm_head rows of "
                      f"{wl.name}, seed {seed}, fp64 numpy; scaled to one full step "
                      f"({t_layer:.2f} s/layer, {t_lm:.2f} s lm_head)"}


def prefill_flops(shape, S):
    """Matrix flops of one prefill: every projection over S tokens, causal attention (QK^T and P.V
    over the S (S + 1) / 2 visible pairs), and the lm_head of the last position."""
    proj = sum(2 * S * n * k for _, n, k in shape.proj_shapes()) * shape.layers
    attn = 2 * 2 * shape.n_q * shape.head_dim * (S * (S + 1) // 2) * shape.layers
    lm = 2 * shape.vocab * shape.hidden
    return proj, attn, lm


def prefill_bench(wl, args):
    """Prefill of an S-token prompt of the workload's model (batch 1): K calls timed back to back
    with events on the launch stream, inputs resident.  One JSON line."""
    import torch
    from int4_blockwise_gemv_amd import synth
    from int4_blockwise_gemv_amd.model import DeviceModel, DeviceState
    s, S = wl.shape, args.prefill
    cap = max(S, wl.cap)
    t0 = time.time()
    dm = DeviceModel(s, args.seed, max_batch=1, progress=lambda m: None)
    ds = DeviceState(dm, 1, cap, kv=args.kv)
    emb = synth.fp16_normal(args.seed, synth.GLOBAL_LAYER, synth.T_X, (S, s.hidden))
    x = torch.from_numpy(emb.view(np.int16)).cuda().view(torch.float16)
    torch.cuda.synchronize()
    log(f"packed {s.layers} layers + lm_head, prompt of {S} tokens resident ({time.time() - t0:.1f}s)")
    steps = max(1, min(args.steps, 20))
    warm = max(1, min(args.warmup, 3))
    for _ in range(warm):
        ds.prefill(x)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        ds.prefill(x)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    proj, attn, lm = prefill_flops(s, S)
    tflops = (proj + attn + lm) / (ms * 1e-3) / 1e12
    log(f"prefill of {S} tokens: {ms:.2f} ms ({S / ms * 1e3:.0f} tokens/s, {tflops:.0f} TFLOP/s), "
        f"token {int(ds.token[0])}")
    out = {
        "metric": "prefill tokens/s (decoder_init of one prompt)",
        "value": S / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 weights x fp16 activations, fp32 accumulate (matrix cores)",
        "data": "synthetic (seeded N(0,0.02) fp32 masters ternarised on the GPU, fp16 N(0,1) prompt embeddings)",
        "config": {"workload": f"prefill-{s.name}-s{S}", "layers": s.layers, "hidden": s.hidden, "inter": s.inter,
                   "n_q": s.n_q, "n_kv": s.n_kv, "vocab": s.vocab, "batch": 1, "prompt": S, "quant": s.mode,
                   "kv": args.kv, "seed": args.seed},
        "roofline": {"bound": "mfma", "kernel": "whole prefill (projection GEMMs carry "
                     f"{100 * proj / (proj + attn + lm):.0f}% of the flops)",
                     "achieved": tflops, "peak": 2500.0, "unit": "TFLOP/s", "frac": tflops / 2500.0, "traffic": None,
                     "flops_per_prefill": proj + attn + lm},
        "token": int(ds.token[0]),
        "cpu_baseline": None,
    }
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode-7b-p4000")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", default="auto", choices=["auto", "persistent", "layered"])
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (reference for HBM byte counters)")
    ap.add_argument("--kv", default="f16", choices=["f16", "f32"],
                    help="KV cache precision (f32: the fp32-KV variant, layered path)")
    ap.add_argument("--prefill", type=int, default=0, metavar="S",
                    help="time the prefill (decoder_init) of an S-token prompt instead of the decode step")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this decode step is not sharded across GPUs "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import torch
    from int4_blockwise_gemv_amd import synth
    assert torch.cuda.is_available()
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))
        return
    wl = synth.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    if args.prefill:
        return prefill_bench(wl, args)
    from int4_blockwise_gemv_amd import vv
    dm, ds, lens = build_inputs(wl, args.seed, args.path, args.kv)
    s = wl.shape
    persistent = args.path == "persistent"

    g = ds.graph()
    for _ in range(args.warmup):
        g.launch()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done; timing {args.steps} graph replays")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g.launch()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt * 1e3 / args.steps
    g.close()
    tok = int(ds.token.cpu()[0])
    status = ds.status()
    log(f"{ms * 1e3:.1f} us/step ({1e3 / ms:.1f} steps/s), token {tok}, status {status}")
    if status != 0:
        raise SystemExit("the persistent step reported an in-device wait that gave up")

    wb, kvb, lmb = algorithmic_bytes(s, wl.batch, lens, 4 if args.kv == "f32" else 2)
    total = wb + kvb + lmb
    tag = "7b" if s.hidden == 3584 else "1p5b"
    kb = kernel_breakdown(ds, s.layers, args.steps, persistent)
    log(f"kernel means over {args.steps} eager steps (us): " + ", ".join(f"{k} {v * 1e3:.1f}" for k, v in kb.items()))
    if persistent:
        dom_bytes, dom_ms = wb + kvb, kb["layers"]
        dom_name = "persistent decode-layer kernel (all layers: int4 GEMVs + attention)"
        traffic = read_traffic("persistent_" + tag, ("mega.hip", "gemv_core.h", "vv_internal.h"))
        sum_kern = kb["layers"] + kb["lm_head"]
    else:
        dom_bytes = 2 * s.inter * s.hidden // 2 + 2 * s.inter * (s.hidden // 32) * 2
        dom_ms = kb["gateup"]
        dom_name = "gate/up int4 GEMV (+SiLU*up)"
        traffic = read_traffic("gateup_" + tag, ("gemv.hip", "gemv_core.h", "vv_internal.h"))
        sum_kern = sum(kb[k] for k in ("qkv", "attn", "o", "gateup", "down")) * s.layers + kb["prep"] + kb["lm_head"]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample")
        cpu = cpu_baseline(wl, args.seed)

    out = {
        "metric": "decode steps/s (HBM GB/s, % of 8 TB/s roofline)",
        "value": 1e3 / ms,
        "unit": "decode steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 weights x fp16 activations, fp32 accumulate",
        "data": "synthetic (seeded N(0,0.02) fp32 masters ternarised on the GPU, fp16 N(0,1) KV/inputs)",
        "config": {"workload": wl.name, "layers": s.layers, "hidden": s.hidden, "inter": s.inter,
                   "n_q": s.n_q, "n_kv": s.n_kv, "head_dim": s.head_dim, "vocab": s.vocab, "batch": wl.batch,
                   "past": int(lens.max()), "quant": s.mode, "seed": args.seed,
                   "path": "persistent" if persistent else "layered", "kv": args.kv},
        "hbm": {"algorithmic_bytes_per_step": total, "weights": wb, "kv": kvb, "lm_head": lmb,
                "GB_per_s": total / (ms * 1e-3) / 1e9,
                "frac_of_8TBps": total / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": achieved,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic, "bytes_per_launch": dom_bytes, "mean_launch_us": dom_ms * 1e3},
        "kernels_us": {k: v * 1e3 for k, v in kb.items()},
        "eager_kernel_sum_us": sum_kern * 1e3,
        "token": tok,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
