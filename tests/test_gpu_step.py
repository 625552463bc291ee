"""GPU parity of the whole decode step (vv_decode_step) against the oracle's decode step, for every
implementation of the step (vv_state.path), plus graph replay == eager and run-to-run determinism."""
import numpy as np
import pytest

from oracle import vv_oracle as O
from int4_blockwise_gemv_amd import synth
from gpu_util import STEP_PATHS, host, host_u16, rel_err
from helpers import oracle_model

pytestmark = pytest.mark.gpu
TOL = 2e-3


class Case:
    """Seeded inputs of one decode step, on the GPU (packed by the library) and in the oracle."""

    def __init__(self, shape, seed, layer_ids, pos, cap, outlier_frac=0.0, trace=False, with_lm=True,
                 path="auto", kv="f16"):
        import torch
        from int4_blockwise_gemv_amd.model import DeviceModel, DeviceState
        self.shape, self.seed, self.layer_ids = shape, seed, list(layer_ids)
        self.pos = np.asarray(pos, np.int32)
        B = len(self.pos)
        self.w = synth.Workload("case", shape, B, int(self.pos.max()), cap, (seed,), outlier_frac=outlier_frac)
        self.glob = synth.model_globals(shape, seed, B, with_lm)
        self.dm = DeviceModel(shape, seed, self.layer_ids, with_lm=with_lm, max_batch=B, lm=self.glob.get("lm"),
                              gf=self.glob["gf"])
        self.path = path
        self.ds = DeviceState(self.dm, B, cap, trace=trace, logits=with_lm, path=path, kv=kv)
        self.K, self.V = [], []
        for i, li in enumerate(self.layer_ids):
            K, V = synth.layer_cache(self.w, seed, li, self.pos)
            if kv == "f32":   # the fp32-KV variant: the same past values, stored in fp32
                K, V = K.astype(np.float32), V.astype(np.float32)
            self.K.append(K)
            self.V.append(V)
            self.ds.load_cache_layer(i, K, V)
        self.ds.emb.copy_(torch.from_numpy(self.glob["emb"].view(np.int16)).view(torch.float16).cuda())
        self.ds.pos.copy_(torch.from_numpy(self.pos).cuda())
        torch.cuda.synchronize()

    def oracle(self, trace=None):
        m = oracle_model(self.shape, self.seed, self.layer_ids, glob=self.glob)
        Kc = [k.copy() for k in self.K]
        Vc = [v.copy() for v in self.V]
        logits, tok, gap, h = O.decode_step(m, self.glob["emb"], self.pos, Kc, Vc, trace)
        return logits, tok, gap, h, Kc, Vc

    def run(self):
        import torch
        self.ds.step()
        torch.cuda.synchronize()
        assert self.ds.status() == 0, "a bounded in-kernel wait of the step gave up"


def _check_tokens(tok, ref_logits):
    for b in range(ref_logits.shape[0]):
        i, gap = O.argmax_with_gap(ref_logits[b])
        if gap >= 1e-3:
            assert int(tok[b]) == i, (b, int(tok[b]), i, gap)
        else:
            assert int(tok[b]) in set(int(t) for t in np.argsort(ref_logits[b])[-2:])


def _compare(case, ref):
    logits, tok, gap, h, Kc, Vc = ref
    gl = host(case.ds.logits).astype(np.float64)
    for b in range(len(case.pos)):
        e = rel_err(gl[b], logits[b])
        print(f"logits b={b} rel err {e:.2e} (top-2 gap {gap[b]:.2e})")
        assert e <= TOL
    _check_tokens(host(case.ds.token), logits)
    gk = host(case.ds.k).astype(np.float64)
    gv = host(case.ds.v).astype(np.float64)
    for i in range(len(case.layer_ids)):
        for b, p in enumerate(case.pos):
            assert rel_err(gk[i, b, :, p], Kc[i][b, :, p]) <= TOL
            assert rel_err(gv[i, b, :, p], Vc[i][b, :, p]) <= TOL
            # the rest of the cache is untouched
            keep = np.ones(case.w.cap, bool)
            keep[p] = False
            assert np.array_equal(gk[i, b][:, keep], case.K[i][b][:, keep].astype(np.float64))
            assert np.array_equal(gv[i, b][:, keep], case.V[i][b][:, keep].astype(np.float64))


TINY = synth.TinyShape(layers=2, hidden=256, n_q=4, n_kv=2, head_dim=128, inter=512, vocab=1000)


PATHS = STEP_PATHS


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("pos", [[33], [0], [47], [63], [64], [100]])
def test_step_tiny(cuda, pos, path):
    """B = 1 at positions on both sides of the 64-position attention split edges."""
    case = Case(TINY, 0, range(2), pos, 130, path=path)
    case.run()
    _compare(case, case.oracle())


@pytest.mark.parametrize("pos", [[0], [47], [64], [100], [33, 0, 90]])
def test_step_tiny_fp32_kv(cuda, pos):
    """The fp32-KV variant: fp32 caches, k and v appended unrounded."""
    case = Case(TINY, 1, range(2), pos, 130, path="layered", kv="f32")
    case.run()
    _compare(case, case.oracle())


def test_step_1p5b_width_fp32_kv(cuda):
    """The fp32-KV variant at 1.5B width over 4096 past positions (two sampled layers)."""
    case = Case(synth.QWEN2_1P5B, 0, [0, 27], [4096], 4097, path="layered", kv="f32")
    case.run()
    _compare(case, case.oracle())


def test_step_tiny_batched_layered(cuda):
    case = Case(TINY, 0, range(2), [47, 0, 12], 48, path="layered")
    case.run()
    _compare(case, case.oracle())


@pytest.mark.parametrize("B", [8, 16])
def test_step_tiny_batch_matrix_cores(cuda, B):
    """Batches of 5..16 sequences take the matrix-core GEMV; ragged positions."""
    pos = [(7 * b * b + 3 * b) % 90 for b in range(B)]
    case = Case(TINY, 9, range(2), pos, 96, path="layered")
    case.run()
    _compare(case, case.oracle())


def test_step_1p5b_width_batch16_ragged(cuda):
    """Two layers at 1.5B width, 16 sequences of lengths spread over 64..1500 (the batched shape
    at reduced depth and context)."""
    pos = [64 + (97 * b) % 1437 for b in range(16)]
    case = Case(synth.QWEN2_1P5B, 0, [0, 27], pos, 1501, path="layered")
    case.run()
    _compare(case, case.oracle())


@pytest.mark.parametrize("path", PATHS)
def test_step_tiny_absmax_group7(cuda, path):
    shp = synth.TinyShape(layers=3, hidden=384, n_q=7, n_kv=1, head_dim=128, inter=640, vocab=777, mode="absmax")
    pos, cap = ([20, 5], 40) if path == "layered" else ([20], 70)   # the chained path: batch 1, >= 2 splits
    case = Case(shp, 1, range(3), pos, cap, path=path)
    case.run()
    _compare(case, case.oracle())


@pytest.mark.parametrize("path", PATHS)
def test_step_no_rope_no_bias(cuda, path):
    shp = synth.TinyShape(layers=1, hidden=256, n_q=2, n_kv=2, head_dim=128, inter=256, vocab=300, qkv_bias=False,
                          rope_theta=0.0)
    case = Case(shp, 2, range(1), [9], 16 if path == "layered" else 80, path=path)
    case.run()
    _compare(case, case.oracle())


@pytest.mark.parametrize("path", PATHS)
def test_step_tiny_34_layers(cuda, path):
    """34 layers end to end at tiny width: logits, token and every layer's K/V slot against the
    oracle's 34-layer step, and the residual stream after every layer against the oracle's."""
    shp = synth.TinyShape(layers=34, hidden=256, n_q=4, n_kv=2, head_dim=128, inter=256, vocab=500)
    case = Case(shp, 6, range(34), [70], 80, path=path, trace=True)
    case.run()
    tr = {}
    ref = case.oracle(tr)
    _compare(case, ref)
    gtr = host(case.ds.trace).astype(np.float64)
    for li in range(35):
        assert rel_err(gtr[li], tr["h"][li]) <= TOL, li


def test_step_zero_layers(cuda):
    shp = synth.TinyShape(layers=0, hidden=256, n_q=2, n_kv=1, head_dim=128, inter=256, vocab=4000)
    case = Case(shp, 3, [], [0, 0], 4)
    case.run()
    _compare(case, case.oracle())


@pytest.mark.timeout(300)
@pytest.mark.parametrize("path", PATHS)
def test_step_1p5b_width_two_layers(cuda, path):
    """Two layers at full 1.5B width, P = 4096, full 151936-row lm_head."""
    case = Case(synth.QWEN2_1P5B, 0, [0, 27], [4096], 4097, path=path)
    case.run()
    _compare(case, case.oracle())


@pytest.mark.parametrize("seed", range(1, 10))
def test_step_1p5b_width_seeds(cuda, seed):
    """The other seeds of the 1.5B-shaped workload (two sampled layers each, P = 4096)."""
    case = Case(synth.QWEN2_1P5B, seed, [seed, 27 - seed], [4096], 4097, path="auto")
    case.run()
    _compare(case, case.oracle())


@pytest.mark.timeout(300)
@pytest.mark.parametrize("path", PATHS)
def test_step_7b_width_one_layer(cuda, path):
    """One layer at full 7B width, P = 4000, full lm_head."""
    case = Case(synth.QWEN2_7B, 0, [5], [4000], 4001, path=path)
    case.run()
    _compare(case, case.oracle())


@pytest.mark.timeout(300)
@pytest.mark.parametrize("seed", range(1, 5))
def test_step_7b_width_seeds(cuda, seed):
    """The other seeds of the 7B-shaped workload (one sampled layer each, P = 4000)."""
    case = Case(synth.QWEN2_7B, seed, [3 * seed], [4000], 4001, path="auto")
    case.run()
    _compare(case, case.oracle())


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("pos", [[2048, 2048], [2048, 1500], [2048]])
def test_step_0p5b_cfg_pair(cuda, path, pos):
    """The Realtime-0.5B shape (hidden 896, 14/2 heads): the lock-step CFG pair (batch 2) and one
    sequence, two sampled layers, full lm_head (not a multiple of 256 wide: the VALU kernel)."""
    if path == "chained" and len(pos) > 1:
        pytest.skip("the chained path serves batch 1 (the pair takes the layered path)")
    case = Case(synth.QWEN2_0P5B, 0, [0, 19], pos, 2049, path=path)
    case.run()
    _compare(case, case.oracle())


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("pos", [[30, 7], [30]])
def test_graph_replay_equals_eager_and_determinism(cuda, path, pos):
    import torch
    if path == "chained" and len(pos) > 1:
        pytest.skip("the chained path serves batch 1")
    case = Case(TINY, 4, range(2), pos, 40 if path == "layered" else 100, trace=True, path=path)
    case.run()
    ref = [host(case.ds.logits).copy(), host(case.ds.token).copy(), host_u16(case.ds.k).copy(),
           host(case.ds.trace).copy()]
    case.run()
    assert np.array_equal(host(case.ds.logits), ref[0]) and np.array_equal(host(case.ds.trace), ref[3])
    g = case.ds.graph()
    try:
        for r in range(4):
            g.launch()
            torch.cuda.synchronize()
            assert np.array_equal(host(case.ds.logits), ref[0]), r
            assert np.array_equal(host(case.ds.token), ref[1]), r
            assert np.array_equal(host_u16(case.ds.k), ref[2]), r
            assert np.array_equal(host(case.ds.trace), ref[3]), r
            # eager work between replays
            case.run()
            assert np.array_equal(host(case.ds.logits), ref[0])
    finally:
        g.close()


def test_graph_replay_fused_merge(cuda):
    """Batch 1 over fp16 caches with several splits (cap 300: 5 splits) takes the merge inside the o
    projection's launch, whose hand-off words carry the step counter: graph replays interleaved with
    eager steps, a dozen steps in all, give bit-identical results."""
    import torch
    case = Case(TINY, 8, range(2), [250], 300, trace=True, path="layered")
    case.run()
    ref = [host(case.ds.logits).copy(), host(case.ds.token).copy(), host(case.ds.trace).copy()]
    assert case.ds.status() == 0
    g = case.ds.graph()
    try:
        for r in range(6):
            g.launch()
            torch.cuda.synchronize()
            assert np.array_equal(host(case.ds.logits), ref[0]), r
            assert np.array_equal(host(case.ds.token), ref[1]), r
            assert np.array_equal(host(case.ds.trace), ref[2]), r
            case.run()
            assert np.array_equal(host(case.ds.logits), ref[0]), r
    finally:
        g.close()
    assert case.ds.status() == 0
    _compare(case, case.oracle())


# 8 query heads of 128: the o projection takes 4-wave workgroups (K = 1024, four 8-block groups per
# tile) behind 8 merge waves per head pair
WIDE8 = synth.TinyShape(layers=2, hidden=512, n_q=8, n_kv=2, head_dim=128, inter=1024, vocab=1000)


@pytest.mark.parametrize("pos", [[2], [63], [64], [200], [1099]])
def test_step_wide_heads_many_splits(cuda, pos):
    """Batch 1 with 8 query heads over 18 splits (cap 1100; positions in the first split only, at
    split edges and in the last split): the merge in the o projection's launch over up to 18 splits."""
    case = Case(WIDE8, 3, range(2), pos, 1100, path="layered")
    case.run()
    _compare(case, case.oracle())


def test_graph_replay_wide_heads_many_splits(cuda):
    """Graph replays interleaved with eager steps at the 8-head shape over 16 splits: the fused
    merge's hand-off words carry the step counter, so a dozen steps give bit-identical results."""
    import torch
    case = Case(WIDE8, 9, range(2), [777], 1000, trace=True, path="layered")
    case.run()
    ref = [host(case.ds.logits).copy(), host(case.ds.token).copy(), host(case.ds.trace).copy()]
    g = case.ds.graph()
    try:
        for r in range(6):
            g.launch()
            torch.cuda.synchronize()
            assert np.array_equal(host(case.ds.logits), ref[0]), r
            assert np.array_equal(host(case.ds.token), ref[1]), r
            assert np.array_equal(host(case.ds.trace), ref[2]), r
            case.run()
            assert np.array_equal(host(case.ds.logits), ref[0]), r
    finally:
        g.close()
    assert case.ds.status() == 0
    _compare(case, case.oracle())


@pytest.mark.parametrize("path", PATHS)
def test_graph_follows_device_positions(cuda, path):
    """One captured graph serves successive positions: replays at pos, pos+1 == eager steps."""
    import torch
    cap = 16 if path == "layered" else 80
    case = Case(TINY, 5, range(2), [10], cap, path=path)
    g = case.ds.graph()
    try:
        outs = []
        for p in (10, 11):
            case.ds.pos.fill_(p)
            g.launch()
            torch.cuda.synchronize()
            outs.append(host(case.ds.logits).copy())
        # eager from the same starting cache
        case2 = Case(TINY, 5, range(2), [10], cap, path=path)
        for i, p in enumerate((10, 11)):
            case2.ds.pos.fill_(p)
            case2.run()
            assert np.array_equal(host(case2.ds.logits), outs[i])
    finally:
        g.close()


@pytest.mark.parametrize("path", PATHS)
def test_step_kernel_timing_events(path):
    """Timing events: one start/stop pair per operation, each holding its kernels' own times."""
    import ctypes as C
    import torch
    case = Case(TINY, 7, range(2), [33], 40 if path == "layered" else 100, path=path)
    n_ops = 4 * 2 + 3 if path == "layered" else 3 * 2 + 2   # batch 1: down | next q|k|v in one launch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_ops)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    arr = (C.c_void_p * len(evs))(*[C.c_void_p(e.cuda_event) for e in evs])
    case.ds.struct.events = C.cast(arr, C.POINTER(C.c_void_p))
    case.ds.struct.n_events = len(evs)
    try:
        case.run()
    finally:
        case.ds.struct.events = None
        case.ds.struct.n_events = 0
    t = [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(n_ops)]
    assert all(np.isfinite(v) and 0.0 < v < 100.0 for v in t), t
    # operations run in stream order: each starts after the previous one ended
    for i in range(1, n_ops):
        assert evs[2 * i - 1].elapsed_time(evs[2 * i]) >= -1e-3, i
    ref_logits, _, _, _, _, _ = case.oracle()
    logits = host(case.ds.logits)
    assert rel_err(logits, ref_logits) < TOL


@pytest.mark.parametrize("cap", [65, 300, 8192])
def test_chained_graph_replays_interleaved_with_eager(cuda, cap):
    """The chained path's tagged words carry the step counter: graph replays interleaved with eager
    steps give bit-identical results (2, 5 and 128 attention splits: the merge segment's smallest,
    middle and largest plans), and agree with the oracle and with the layered path."""
    import torch
    pos = [cap - 1]
    case = Case(TINY, 10, range(2), pos, cap, trace=True, path="chained")
    case.run()
    ref = [host(case.ds.logits).copy(), host(case.ds.token).copy(), host(case.ds.trace).copy(),
           host_u16(case.ds.k).copy()]
    g = case.ds.graph()
    try:
        for r in range(5):
            g.launch()
            torch.cuda.synchronize()
            assert np.array_equal(host(case.ds.logits), ref[0]), r
            assert np.array_equal(host(case.ds.token), ref[1]), r
            assert np.array_equal(host(case.ds.trace), ref[2]), r
            assert np.array_equal(host_u16(case.ds.k), ref[3]), r
            case.run()
            assert np.array_equal(host(case.ds.logits), ref[0]), r
    finally:
        g.close()
    assert case.ds.status() == 0
    _compare(case, case.oracle())
    lay = Case(TINY, 10, range(2), pos, cap, trace=True, path="layered")
    lay.run()
    assert rel_err(host(case.ds.trace).astype(np.float64), host(lay.ds.trace).astype(np.float64)) <= TOL


def test_chained_path_rejects_what_it_does_not_serve(cuda):
    """Batch 2, a single attention split (cap 64), fp32 caches: VV_ERR_UNSUPPORTED before any launch;
    AUTO takes the layered path for them."""
    from int4_blockwise_gemv_amd import vv
    for pos, cap, kv in (([5, 3], 80, "f16"), ([5], 64, "f16"), ([5], 80, "f32")):
        case = Case(TINY, 0, range(2), pos, cap, path="chained", kv=kv)
        with pytest.raises(vv.VVError) as e:
            case.ds.step()
        assert e.value.status == vv.VV_ERR_UNSUPPORTED
        auto = Case(TINY, 0, range(2), pos, cap, path="auto", kv=kv)
        auto.run()
        _compare(auto, auto.oracle())
