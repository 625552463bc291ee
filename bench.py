"""Decode-step benchmark (one JSON line on stdout).

python bench.py [--gpus 1] [--steps K] [--warmup W] [--trials T] [--workload decode-7b-p4000]
                [--also decode-1.5b-p4096,...] [--seed 0]

One step = one vv_decode_step (28 layers of fused QKV GEMV, attention with KV append, o GEMV,
gate/up GEMV + SiLU, down GEMV, then lm_head + argmax) replayed from a hipGraph on seeded
synthetic weights, KV cache and input already resident in HBM.  Each trial times K back-to-back
replays bracketed by torch.cuda.synchronize(); `value` and `ms_per_step` are the median of T
trials (min and max are reported beside them).  The headline workload is the 7B-shaped step;
the 1.5B-shaped step (the other shape of the metric), the 7B shape with general int4 weights over
16384 positions with outliers, 16 ragged 1.5B sequences and the 0.5B classifier-free-guidance
pair are measured in the same run and reported under `workloads`.

Also reported, per workload:
  hbm          algorithmic bytes per step (packed int4 nibbles + fp16 scales + fp16 lm_head + K/V
               over P+1 positions) / step time, as a fraction of 8 TB/s, and the gap to 70 %;
  roofline     (headline) the dominant kernel: its algorithmic bytes per launch / its mean
               duration, measured with hipExtLaunchKernel start/stop events (the dispatch's own
               timestamps) on the launch stream during K instrumented eager steps; beside it the
               rocprofv3 average of the same kernel from the committed kernel statistics and the
               HBM traffic from the committed counter summary, each only when it was taken on the
               current kernel source;
  closed_loop  µs per step when every replay is followed by the 4-byte token copy to the host;
  stream_read  the measured streaming-read ceiling of this GPU (vv_stream_read over 4 GiB);
  cpu_baseline the fp64 oracle's decode step timed on a bounded sample of the same workload (one
               layer and a slice of the vocabulary, scaled to one step) on the host's cores.

python bench.py --workload single-layer-1536 times the small workload (one [1536 x 1536] ternary
GEMV and the 12/2-head attention over 256 positions) hot (the same buffers every time) and cold
(rotating over more than 1 GiB of copies).
python bench.py --prefill S times the prefill (decoder_init) of an S-token prompt instead.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
TARGET_FRAC = 0.70
KERNEL_SOURCES = ("gemv.hip", "gemv_core.h", "vv_internal.h", "attn.hip", "step.hip", "lmhead.hip", "chain.hip")


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def algorithmic_bytes(shape, lens, kv_bytes=2):
    """Bytes one step must read: packed nibbles + fp16 scales + fp16 lm_head + K/V over P+1
    (kv_bytes per element: 2 for fp16 caches, 4 for the fp32-KV variant)."""
    per_layer_w = sum(n * k // 2 + n * (k // 32) * 2 for _, n, k in shape.proj_shapes())
    w = per_layer_w * shape.layers
    kv = sum(int(L) + 1 for L in lens) * shape.n_kv * shape.head_dim * 2 * kv_bytes * shape.layers
    lm = shape.vocab * shape.hidden * 2
    return w, kv, lm


def kernel_source_hash(files=KERNEL_SOURCES):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "int4_blockwise_gemv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _summary_fields(path):
    kv = {}
    if os.path.exists(path):
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    return kv


def _current(kv):
    files = tuple(f.strip() for f in kv.get("source_files", "").split(",") if f.strip())
    return bool(files) and kv.get("source_hash") == kernel_source_hash(files)


def read_traffic(tag):
    """HBM bytes per launch from profiles/traffic_<tag>.txt if it was taken on the current source."""
    kv = _summary_fields(os.path.join(ROOT, "profiles", f"traffic_{tag}.txt"))
    if not _current(kv):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_profile_mean(workload, kernel_prefix):
    """Mean duration (µs) of a kernel in profiles/kernels_<workload>.txt, when that summary was taken
    on the current kernel source (its source_hash line), else None."""
    path = os.path.join(ROOT, "profiles", f"kernels_{workload}.txt")
    if not _current(_summary_fields(path)):
        return None
    for line in open(path):
        if line.startswith(kernel_prefix):
            parts = line.split()
            try:
                return float(parts[-4])     # ... calls avg min max pct: avg is the 4th from the end
            except (ValueError, IndexError):
                return None
    return None


def build_inputs(wl, seed, path="auto", kv="f16"):
    import torch
    from int4_blockwise_gemv_amd import synth
    from int4_blockwise_gemv_amd.model import DeviceModel, DeviceState
    s = wl.shape
    lens = synth.past_lengths(wl, seed)
    t0 = time.time()
    dm = DeviceModel(s, seed, max_batch=wl.batch, progress=lambda m: None)
    log(f"{wl.name}: packed {s.layers} layers + lm_head on the GPU in {time.time() - t0:.1f}s")
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
    log(f"{wl.name}: inputs resident ({time.time() - t0:.1f}s total)")
    return dm, ds, lens


# the chained plan splits the MLP launch into [gate/up] and [down | next q|k|v] above this width
CHAIN_SPLIT_MLP_HIDDEN = 2048


def op_names(n_layers, path, hidden=0, batch=1):
    if path == "layered" and batch == 1:   # down and the next layer's q|k|v share a launch
        return (["prep", "qkv"] + ["attn", "o", "gateup", "down_qkv"] * (n_layers - 1)
                + ["attn", "o", "gateup", "down"] + ["lm_head"])
    if path == "chained" and hidden > CHAIN_SPLIT_MLP_HIDDEN:
        return (["prep_qkv"] + ["attn", "chain_mo", "chain_gu", "chain_dq"] * (n_layers - 1)
                + ["attn", "chain_mo", "chain_gu", "chain_d_last"] + ["lm_head"])
    if path == "chained":   # the last layer's MLP launch has no q|k|v segment: timed apart
        return (["prep_qkv"] + ["attn", "chain_mo", "chain"] * (n_layers - 1) + ["attn", "chain_mo", "chain_last"]
                + ["lm_head"])
    return ["prep"] + ["qkv", "attn", "o", "gateup", "down"] * n_layers + ["lm_head"]


def kernel_breakdown(ds, n_layers, steps, path):
    """Mean kernel time (ms) per operation of the step over `steps` eager steps.

    Each operation's kernels are launched with hipExtLaunchKernel start/stop events on the launch
    stream, which receive the kernels' own dispatch start and end times (the values rocprofv3
    reports), not the time the stream reaches a marker."""
    import ctypes as C
    import torch
    names = op_names(n_layers, path, ds.model.shape.hidden, ds.batch)
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


def time_graph(g, steps, warmup, trials):
    """Per-trial ms per step of `steps` back-to-back graph replays (after `warmup` replays)."""
    import torch
    for _ in range(warmup):
        g.launch()
    torch.cuda.synchronize()
    out = []
    for _ in range(trials):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.launch()
        torch.cuda.synchronize()
        out.append((time.perf_counter() - t0) * 1e3 / steps)
    return out


def time_closed_loop(g, ds, steps):
    """ms per step when each replay is followed by the 4-byte token copy to the host (the host
    waits for every token, as a caller that inspects each token would)."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.launch()
        int(ds.token[0].item())
    return (time.perf_counter() - t0) * 1e3 / steps


def stream_ceiling(gib=4, reps=5):
    """GB/s of vv_stream_read over a `gib` GiB buffer (best of `reps`)."""
    import torch
    from int4_blockwise_gemv_amd import vv
    n = gib << 30
    buf = torch.empty(n // 4, dtype=torch.int32, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    vv.stream_read(buf, sink)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        vv.stream_read(buf, sink)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, n / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf
    torch.cuda.empty_cache()
    return best


def cpu_info():
    model = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    return model, cores


def cpu_baseline(wl, seed):
    """The oracle's decode step on a bounded sample: one layer and a slice of the vocabulary, scaled
    to one full step; with all the host's BLAS threads and again with one thread (layer only)."""
    from threadpoolctl import threadpool_info, threadpool_limits
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
    model, cores = cpu_info()
    t0 = time.perf_counter()
    O.layer_step(m.layers[0], m, h, lens, K.copy(), V.copy())
    t_layer = time.perf_counter() - t0
    frac_rows = 16384
    lm = synth.fp16_normal(seed, synth.GLOBAL_LAYER, synth.T_LM, (frac_rows, s.hidden), std=0.02)
    f = O.rmsnorm(h, m.gf, m.eps)
    t0 = time.perf_counter()
    O.lm_head_argmax(lm, f)
    t_lm = (time.perf_counter() - t0) * s.vocab / frac_rows
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    with threadpool_limits(1):
        t0 = time.perf_counter()
        O.layer_step(m.layers[0], m, h, lens, K.copy(), V.copy())
        t_layer1 = time.perf_counter() - t0
    t_step = t_layer * s.layers + t_lm
    return {"value": 1.0 / t_step, "unit": "decode steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"1 of {s.layers} layers (layer {li}) + {frac_rows} of {s.vocab} lm_head rows of "
                      f"{wl.name}, seed {seed}, fp64 numpy; scaled to one full step "
                      f"({t_layer:.2f} s/layer, {t_lm:.2f} s lm_head)",
            "s_per_step": t_step, "host_cores": cores, "cpu_model": model, "blas_threads": int(threads),
            "s_per_layer_1_thread": t_layer1}


def proj_bytes(s, names):
    """Algorithmic bytes (nibbles + fp16 scales) of the named projections of one layer."""
    return sum(n * k // 2 + n * (k // 32) * 2 for nm, n, k in s.proj_shapes() if nm in names)


def eager_sum(kb, L, path):
    if path == "chained" and "chain_gu" in kb:
        return (kb["prep_qkv"] + (kb["attn"] + kb["chain_mo"] + kb["chain_gu"]) * L + kb["chain_dq"] * (L - 1)
                + kb["chain_d_last"] + kb["lm_head"])
    if path == "chained":
        return (kb["prep_qkv"] + (kb["attn"] + kb["chain_mo"]) * L + kb["chain"] * (L - 1) + kb["chain_last"]
                + kb["lm_head"])
    if "down_qkv" in kb:
        return (kb["prep"] + kb["qkv"] + (kb["attn"] + kb["o"] + kb["gateup"]) * L + kb["down_qkv"] * (L - 1)
                + kb["down"] + kb["lm_head"])
    return sum(kb[k] for k in ("qkv", "attn", "o", "gateup", "down")) * L + kb["prep"] + kb["lm_head"]


def measure_decode(wl, args, headline):
    """One workload: graph trials, closed loop, eager kernel breakdown.  Returns its record."""
    import torch
    s = wl.shape
    dm, ds, lens = build_inputs(wl, args.seed, args.path, args.kv)
    g = ds.graph()
    trials = time_graph(g, args.steps, args.warmup, args.trials)
    closed = time_closed_loop(g, ds, max(10, args.steps // 4))
    g.close()
    tok = [int(t) for t in ds.token.cpu()]
    status = ds.status()
    med = float(np.median(trials))
    log(f"{wl.name}: {med * 1e3:.1f} us/step median of {args.trials} trials "
        f"(min {min(trials) * 1e3:.1f}, max {max(trials) * 1e3:.1f}), closed loop {closed * 1e3:.1f} us, "
        f"token {tok[0]}, status {status}")
    if status != 0:
        raise SystemExit("the step reported a bounded in-device wait that gave up")
    wb, kvb, lmb = algorithmic_bytes(s, lens, 4 if args.kv == "f32" else 2)
    total = wb + kvb + lmb
    path = ds.path()
    kb = kernel_breakdown(ds, s.layers, args.steps if headline else max(20, args.steps // 4), path)
    log(f"{wl.name}: kernel means over eager steps (us): " +
        ", ".join(f"{k} {v * 1e3:.1f}" for k, v in kb.items()))
    gbs = total / (med * 1e-3) / 1e9
    target_us = total / (TARGET_FRAC * PEAK_HBM_GBS * 1e9) * 1e6
    rec = {
        "us_per_step": med * 1e3, "us_per_step_min": min(trials) * 1e3, "us_per_step_max": max(trials) * 1e3,
        "trials": args.trials, "steps_per_trial": args.steps, "steps_per_s": 1e3 / med,
        "closed_loop_us_per_step": closed * 1e3,
        "hbm": {"algorithmic_bytes_per_step": total, "weights": wb, "kv": kvb, "lm_head": lmb,
                "GB_per_s": gbs, "frac_of_8TBps": gbs / PEAK_HBM_GBS, "target_frac": TARGET_FRAC,
                "target_us_per_step": target_us, "gap_to_target_us": med * 1e3 - target_us,
                "north_star_bytes_no_lm_head": wb + kvb},
        "kernels_us": {k: v * 1e3 for k, v in kb.items()},
        "eager_kernel_sum_us": eager_sum(kb, s.layers, path) * 1e3,
        "token": tok,
        "config": {"workload": wl.name, "layers": s.layers, "hidden": s.hidden, "inter": s.inter,
                   "n_q": s.n_q, "n_kv": s.n_kv, "head_dim": s.head_dim, "vocab": s.vocab, "batch": wl.batch,
                   "past": int(lens.max()), "quant": s.mode, "seed": args.seed, "path": path, "kv": args.kv},
    }
    if path == "chained" and "chain_gu" in kb:
        # wide models: gate/up in a chained launch of its own
        dom_ms = kb["chain_gu"]
        dom_bytes = proj_bytes(s, ("gate", "up"))
        dom_name = "chained gate/up launch (int4 GEMV + SiLU*up)"
        prof = read_profile_mean(wl.name, "void vv::(anonymous namespace)::k_chain<3>")
        traffic = None
        share = dom_ms * s.layers / med
    elif path == "chained":
        # the chained MLP launch of layers 0..L-2: gate/up, down and the next layer's q|k|v
        dom_ms = kb["chain"]
        dom_bytes = proj_bytes(s, ("gate", "up", "down", "q", "k", "v"))
        dom_name = "chained MLP launch (gate/up | down | next q|k|v int4 GEMVs)"
        prof = read_profile_mean(wl.name, "void vv::(anonymous namespace)::k_chain<2>")
        traffic = read_traffic("chain_7b" if s.hidden == 3584 else "chain_1p5b")
        share = (kb["chain"] * (s.layers - 1) + kb["chain_last"]) / med
    else:
        dom_ms = kb["gateup"]
        dom_bytes = proj_bytes(s, ("gate", "up"))
        dom_name = "gate/up int4 GEMV (+SiLU*up)"
        prof = read_profile_mean(wl.name, "void vv::(anonymous namespace)::k_gemv<1, 2, 8, false, true>")
        traffic = read_traffic("gateup_7b" if s.hidden == 3584 else "gateup_1p5b")
        share = dom_ms * s.layers / med
    rec["roofline"] = {
        "bound": "hbm", "kernel": dom_name,
        "achieved": dom_bytes / (dom_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
        "frac": dom_bytes / (dom_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "traffic": traffic, "bytes_per_launch": dom_bytes, "mean_launch_us": dom_ms * 1e3,
        "rocprof_mean_launch_us": prof, "share_of_step": share,
    }
    del g, ds, dm
    torch.cuda.empty_cache()
    return rec


def single_layer_bench(wl, args):
    """The single-layer workload: one [1536 x 1536] ternary GEMV + GQA 12/2 over 256 positions, hot
    and cold (rotating across > 1 GiB of distinct weight/KV copies, so nothing is cache-resident)."""
    import torch
    from int4_blockwise_gemv_amd import synth, vv
    s = wl.shape
    N = K = s.hidden
    nq, nkv, d, P = s.n_q, s.n_kv, s.head_dim, wl.past
    seed = args.seed
    W = torch.from_numpy(synth.master_weight(seed, 0, synth.T_Q, N, K)).cuda()
    lay = vv.VV_LAYOUT_TILED
    qbytes, sbytes = vv.packed_bytes(N, K, lay), vv.scale_bytes(N, K, lay)
    kv_elems = nkv * P * d
    unit = qbytes + sbytes + 2 * kv_elems * 2
    copies = max(2, -(-(1 << 30) // unit) + 1)
    log(f"single layer: {unit / 1e6:.3f} MB per GEMV + GQA, {copies} copies for the cold run")
    q = torch.empty((copies, qbytes), dtype=torch.uint8, device="cuda")
    sc = torch.empty((copies, sbytes // 2), dtype=torch.int16, device="cuda")
    pws = torch.zeros(max(256, vv.pack_workspace(N, K, "ternary")), dtype=torch.uint8, device="cuda")
    vv.pack_int4_tiled(W, "ternary", 64, 64, 0, N, q[0], sc[0], pws)
    q[1:].copy_(q[0].expand(copies - 1, -1))
    sc[1:].copy_(sc[0].expand(copies - 1, -1))
    Kc, Vc = synth.layer_cache(wl, seed, 0, np.array([P], np.int32))
    kc = torch.from_numpy(Kc.view(np.int16)).cuda().view(torch.float16).reshape(1, -1).repeat(copies, 1)
    vc = torch.from_numpy(Vc.view(np.int16)).cuda().view(torch.float16).reshape(1, -1).repeat(copies, 1)
    x = torch.from_numpy(synth.fp16_normal(seed, 0, synth.T_X, (1, K)).view(np.int16)).cuda().view(torch.float16)
    y = torch.empty((1, N), dtype=torch.float16, device="cuda")
    gws = torch.zeros(vv.gemv_workspace(1, N, K), dtype=torch.uint8, device="cuda")
    lens = torch.full((1,), P, dtype=torch.int32, device="cuda")
    aws = torch.zeros(vv.gqa_workspace(1, nq, nkv, P), dtype=torch.uint8, device="cuda")
    out = torch.empty((1, nq, d), dtype=torch.float16, device="cuda")
    qv = y.view(1, nq, d)

    def one(i):
        vv.gemv_int4(q[i], sc[i], None, x, N, K, y, gws)
        vv.gqa_decode(qv, kc[i].view(1, nkv, P, d), vc[i].view(1, nkv, P, d), lens, nq, nkv, P, 1.0 / d ** 0.5,
                      out, aws)

    def run(idx):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in idx[:20]:
            one(i)
        torch.cuda.synchronize()
        e0.record()
        for i in idx:
            one(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / len(idx)

    n = max(args.steps, copies)
    hot = [run([0] * n) for _ in range(args.trials)]
    cold = [run([i % copies for i in range(n)]) for _ in range(args.trials)]
    hot_us, cold_us = float(np.median(hot)), float(np.median(cold))
    log(f"single layer: hot {hot_us:.2f} us, cold {cold_us:.2f} us per GEMV + GQA")
    cpu = None
    if not args.no_cpu_baseline:
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from oracle import vv_oracle as O
        pq, ps = O.pack(W.cpu().numpy(), "ternary")
        xn = synth.fp16_normal(seed, 0, synth.T_X, (1, K))
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 10.0:
            yo = O.gemv(pq, ps, xn)
            O.gqa_decode(yo.reshape(nq, d), Kc[0], Vc[0], P, 1.0 / d ** 0.5)
            reps += 1
        t = (time.perf_counter() - t0) / reps
        model, cores = cpu_info()
        cpu = {"value": 1.0 / t, "unit": "GEMV+GQA/s", "cores": cores, "kind": "oracle",
               "sample": f"{reps} repetitions of the oracle's GEMV + GQA on the same inputs (fp64 numpy)",
               "cpu_model": model}
    res = {
        "metric": "single-layer GEMV + GQA per second (cold: distinct copies streamed from HBM)",
        "value": 1e6 / cold_us, "unit": "GEMV+GQA/s", "n_gpus": 1, "steps": n, "warmup": 20,
        "ms_per_step": cold_us * 1e-3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int4 weights x fp16 activations, fp32 accumulate", "data": "synthetic (seeded)",
        "config": {"workload": wl.name, "N": N, "K": K, "n_q": nq, "n_kv": nkv, "past": P, "quant": "ternary",
                   "copies": copies},
        "hot_us": hot_us, "cold_us": cold_us, "hot_us_trials": hot, "cold_us_trials": cold,
        "roofline": {"bound": "hbm", "kernel": "GEMV + GQA pair (cold)", "achieved": unit / (cold_us * 1e-6) / 1e9,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": unit / (cold_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                     "traffic": None, "bytes_per_pair": unit},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))


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
    ap.add_argument("--trials", type=int, default=5)
    ap.add_argument("--workload", default="decode-7b-p4000")
    ap.add_argument("--also", default="decode-1.5b-p4096,decode-7b-absmax-p16384,decode-1.5b-b16-ragged,"
                                      "decode-0.5b-cfg-b2",
                    help="comma-separated workloads measured in the same run (reported under `workloads`), "
                         "or 'none'")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-ceiling", action="store_true")
    ap.add_argument("--path", default="auto", choices=["auto", "layered", "chained"])
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times (reference for HBM byte counters)")
    ap.add_argument("--kv", default="f16", choices=["f16", "f32"],
                    help="KV cache precision (f32: the fp32-KV variant)")
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
    if wl.name == "single-layer-1536":
        return single_layer_bench(wl, args)

    head = measure_decode(wl, args, headline=True)
    subs = {}
    for name in [n.strip() for n in args.also.split(",") if n.strip() and n.strip() != "none"]:
        if name != wl.name:
            subs[name] = measure_decode(synth.WORKLOADS[name], args, headline=False)
    ceiling = None
    if not args.no_stream_ceiling:
        ceiling = stream_ceiling()
        log(f"streaming-read ceiling {ceiling:.0f} GB/s")
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample")
        cpu = cpu_baseline(wl, args.seed)

    out = {
        "metric": "decode steps/s (HBM GB/s, % of 8 TB/s roofline)",
        "value": head["steps_per_s"],
        "unit": "decode steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["us_per_step"] * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 weights, fp32 activations (exact int8-digit dot products), fp32 accumulate",
        "data": "synthetic (seeded N(0,0.02) fp32 masters ternarised on the GPU, fp16 N(0,1) KV/inputs)",
        "config": head["config"],
        "trials": {"n": args.trials, "us_per_step_median": head["us_per_step"],
                   "us_per_step_min": head["us_per_step_min"], "us_per_step_max": head["us_per_step_max"]},
        "hbm": head["hbm"],
        "roofline": head["roofline"],
        "closed_loop_us_per_step": head["closed_loop_us_per_step"],
        "stream_read_GB_per_s": ceiling,
        "frac_of_stream_ceiling": (head["hbm"]["GB_per_s"] / ceiling) if ceiling else None,
        "kernels_us": head["kernels_us"],
        "eager_kernel_sum_us": head["eager_kernel_sum_us"],
        "token": head["token"][0],
        "workloads": subs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
