"""GPU parity: quant_dequantize (bit-exact) and quant_gemv (1e-5 * sum|w x|)
against the CPU oracle, through the C ABI.

README "Examples" (backend_check): every device op against the host reference;
(batch_check): a batched pass against the same rows one at a time.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import GEMV_TOL, check_bound, check_rel, dev, host, say
from _golden import q4_k_blocks, q8_0_blocks

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

Q8, Q4 = synth.FMT_Q8_0, synth.FMT_Q4_K


@pytest.fixture(scope="module")
def g():
    import quantized_gguf_q8_amd as g
    return g


# --------------------------------------------------------------------------- #
# dequantize: bit-exact
def test_fp16_scales_all_patterns_bit_exact(g):
    """All 65536 fp16 patterns as Q8_0 scales with q = 1: the device decode keeps
    subnormals (no flush) and matches numpy's binary16 conversion."""
    say("dequant fp16 table")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    blocks = np.zeros((65536, 34), dtype=np.uint8)
    blocks[:, 0:2] = bits.view(np.uint8).reshape(-1, 2)
    blocks[:, 2] = 1
    out = host(g.quant_dequantize(Q8, dev(blocks), 65536, 32))[:, 0]
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(out), nan)
    assert np.array_equal(out[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_dequant_golden_blocks(g):
    say("dequant golden")
    for raw, expect, _ in q8_0_blocks():
        out = host(g.quant_dequantize(Q8, dev(np.frombuffer(raw, np.uint8).copy()), 1, 32))[0]
        assert np.array_equal(out.view(np.uint32), expect.view(np.uint32))
    for raw, expect, _, _ in q4_k_blocks():
        out = host(g.quant_dequantize(Q4, dev(np.frombuffer(raw, np.uint8).copy()), 1, 256))[0]
        assert np.array_equal(out.view(np.uint32), expect.view(np.uint32))


@pytest.mark.parametrize("fmt,n,k", [(Q8, 333, 2048), (Q8, 7, 96), (Q4, 129, 2560), (Q4, 1, 256)])
def test_dequant_random_bit_exact(g, fmt, n, k):
    say(f"dequant fmt={fmt} n={n} k={k}")
    w = synth.quant_matrix(fmt, n, k, seed=0, tensor_id=100 + n)
    if fmt == Q4:   # edge scales: subnormal, zero and large d/dmin
        blk = w.reshape(-1, 144)
        blk[::5, 0:2] = [0x01, 0x00]
        blk[1::7, 2:4] = [0xFF, 0x7B]
        blk[2::11, 0:4] = 0
    ref = oracle.dequant(fmt, w, n, k)
    out = host(g.quant_dequantize(fmt, dev(w), n, k))
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


# --------------------------------------------------------------------------- #
# GEMV
PATHS = {"valu": None, "mfma": "auto"}   # no workspace -> vector units; workspace -> matrix cores


def _gemv_case(g, fmt, n, k, b, seed=0, tid=1, ws=None):
    w = synth.quant_matrix(fmt, n, k, seed=seed, tensor_id=tid)
    x = synth.normal_f32((b, k), seed=seed, tensor_id=tid + 1)
    y = host(g.quant_gemv(fmt, dev(w), n, k, dev(x), ws=ws))
    yr, s = oracle.gemv(fmt, w, n, k, x)
    return y, yr, s, w, x


@pytest.mark.parametrize("fmt,n,k,b", [
    (Q8, 1024, 1024, 1),        # the 1024 x 1024 single-token case
    (Q8, 37, 2304, 1), (Q8, 37, 2304, 3), (Q8, 64, 6144, 8), (Q8, 65, 512, 16),
    (Q8, 5, 224, 1), (Q8, 9, 96, 6),            # K % 256 != 0 path
    (Q4, 70, 2560, 1), (Q4, 70, 2560, 4), (Q4, 33, 9728, 16), (Q4, 1, 256, 2),
    (Q4, 300, 768, 5), (Q4, 17, 11264, 13), (Q8, 4099, 2048, 9), (Q4, 1000, 2560, 2),
])
@pytest.mark.parametrize("path", PATHS)
def test_gemv_parity(g, fmt, n, k, b, path):
    say(f"gemv fmt={fmt} n={n} k={k} b={b} path={path}")
    y, yr, s, _, _ = _gemv_case(g, fmt, n, k, b, tid=n * 7 + b, ws=PATHS[path])
    worst = check_rel(y, yr, s, GEMV_TOL, f"gemv {fmt} {n}x{k} b{b}")
    say(f"  worst err / bound = {worst:.3g}")


@pytest.mark.parametrize("name,n,k", synth.DENSE_1B_LAYER_SET)
@pytest.mark.parametrize("b", [1, 8])
@pytest.mark.parametrize("path", PATHS)
def test_gemv_dense_layer_set_full_size(g, name, n, k, b, path):
    """The ~1B dense decode layer set (Q8_0) at batch 1 and 8, every row."""
    say(f"gemv layer {name} {n}x{k} b={b} path={path}")
    tid = synth.tid(1, n, k)
    w = synth.q8_0_matrix(n, k, seed=0, tensor_id=tid)
    x = synth.normal_f32((b, k), seed=0, tensor_id=tid + 1)
    y = host(g.quant_gemv(Q8, dev(w), n, k, dev(x), ws=PATHS[path]))
    yr, s = oracle.gemv(Q8, w, n, k, x)
    worst = check_rel(y, yr, s, GEMV_TOL, f"{name} b{b}")
    say(f"  worst err / bound = {worst:.3g}")


@pytest.mark.parametrize("name,n,k", synth.Q4K_FFN_PAIR)
@pytest.mark.parametrize("b", [1, 4, 16])
@pytest.mark.parametrize("path", PATHS)
def test_gemv_q4k_ffn_full_size(g, name, n, k, b, path):
    say(f"gemv q4k {name} {n}x{k} b={b} path={path}")
    tid = synth.tid(2, n, k)
    w = synth.q4_k_matrix(n, k, seed=0, tensor_id=tid)
    x = synth.normal_f32((b, k), seed=0, tensor_id=tid + 1)
    y = host(g.quant_gemv(Q4, dev(w), n, k, dev(x), ws=PATHS[path]))
    yr, s = oracle.gemv(Q4, w, n, k, x)
    worst = check_rel(y, yr, s, GEMV_TOL, f"{name} b{b}")
    say(f"  worst err / bound = {worst:.3g}")


@pytest.mark.parametrize("fmt,n,k,b", [
    (Q4, 2560, 9728, 4),        # short and long-K: cut into many K parts
    (Q4, 130, 11264, 16), (Q8, 96, 12288, 8), (Q8, 300, 6144, 3),
])
def test_gemv_split_workspace(g, fmt, n, k, b):
    """The matrix-core path with the larger (split-K) workspace and with the
    minimal one: both within tolerance, and the split result repeatable bit for
    bit."""
    say(f"gemv split ws fmt={fmt} n={n} k={k} b={b}")
    w = synth.quant_matrix(fmt, n, k, seed=9, tensor_id=n + k)
    x = synth.normal_f32((b, k), seed=9, tensor_id=n + k + 1)
    wd, xd = dev(w), dev(x)
    yr, s = oracle.gemv(fmt, w, n, k, x)
    small = torch.zeros(g.quant_gemv_workspace_size(fmt, k, b), dtype=torch.uint8, device="cuda")
    big = torch.zeros(g.quant_gemv_split_workspace_size(fmt, n, k, b), dtype=torch.uint8,
                      device="cuda")
    y1 = host(g.quant_gemv(fmt, wd, n, k, xd, ws=small))
    y2 = host(g.quant_gemv(fmt, wd, n, k, xd, ws=big))
    y3 = host(g.quant_gemv(fmt, wd, n, k, xd, ws=big))
    check_rel(y1, yr, s, GEMV_TOL, "minimal workspace")
    check_rel(y2, yr, s, GEMV_TOL, "split workspace")
    assert np.array_equal(y2, y3)


@pytest.mark.parametrize("fmt,n,k,b", [
    (Q4, 2560, 9728, 16), (Q4, 9728, 2560, 4), (Q8, 1024, 1024, 1), (Q8, 300, 6144, 9),
    (Q4, 33, 20480, 2),      # 20 K parts on 3 row tiles, ragged last tile
    (Q4, 2560, 9728, 1),     # batch 1 on the single launch (large Q4_K)
])
def test_gemv_single_launch_workspace_and_graph_replays(g, fmt, n, k, b):
    """The one-launch matrix-core GEMV of a single matrix: its K parts are added
    in part order by the workgroup that finishes a row tile last, counted in the
    workspace's control block.  A workspace whose control block is zero and
    whose rest is random bytes must not matter, every call must leave the
    control block zero, and replays of a captured call must give the eager bits
    each time."""
    say(f"gemv single launch fmt={fmt} n={n} k={k} b={b}")
    w = synth.quant_matrix(fmt, n, k, seed=12, tensor_id=n + 3 * k)
    x = synth.normal_f32((b, k), seed=12, tensor_id=n + 3 * k + 1)
    wd, xd = dev(w), dev(x)
    yr, s = oracle.gemv(fmt, w, n, k, x)
    nbytes = g.quant_gemv_split_workspace_size(fmt, n, k, b)
    rng = np.random.default_rng(5)
    raw = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    raw[:g.CTRL_BYTES] = 0
    ws = dev(raw)
    y0 = host(g.quant_gemv(fmt, wd, n, k, xd, ws=ws))
    check_rel(y0, yr, s, GEMV_TOL, "garbage workspace")
    assert not host(ws[:g.CTRL_BYTES]).any(), "control block left non-zero"
    y1 = host(g.quant_gemv(fmt, wd, n, k, xd, ws=ws))
    assert np.array_equal(y0, y1)
    yg = torch.full((b, n), float("nan"), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g.quant_gemv(fmt, wd, n, k, xd, y=yg, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.quant_gemv(fmt, wd, n, k, xd, y=yg, ws=ws)
    for rep in range(4):
        yg.fill_(float("nan"))
        graph.replay()
        got = host(yg)
        assert np.array_equal(got, y0), f"replay {rep}"
        # eager work between replays, on the same workspace
        y2 = host(g.quant_gemv(fmt, wd, n, k, xd, ws=ws))
        assert np.array_equal(y2, y0)
    assert not host(ws[:g.CTRL_BYTES]).any(), "control block left non-zero"


# --------------------------------------------------------------------------- #
# fused gate/up with SiLU * up (dense gated feed-forward)
def _swiglu_bound(o):
    """Per-element bound for h = silu(g) * u from the per-product GEMV
    tolerances (first order; |d silu / dg| <= 1.1) plus fp32 rounding."""
    sig = 1.0 / (1.0 + np.exp(-o["g"]))
    return (1.1 * np.abs(o["u"]) * GEMV_TOL * o["sg"] + np.abs(o["g"] * sig) * GEMV_TOL * o["su"]
            + 1e-6 * np.abs(o["h"]))


@pytest.mark.parametrize("fmt,n,k,b", [
    (Q8, 6144, 2048, 1), (Q8, 6144, 2048, 8),          # the ~1B layer set's gate/up
    (Q4, 9728, 2560, 1), (Q4, 9728, 2560, 4), (Q4, 9728, 2560, 16),
    (Q8, 100, 512, 3), (Q4, 77, 768, 1), (Q8, 33, 4096, 16), (Q4, 300, 256, 9),
])
def test_gemv_swiglu(g, fmt, n, k, b):
    say(f"swiglu fmt={fmt} n={n} k={k} b={b}")
    wg = synth.quant_matrix(fmt, n, k, seed=5, tensor_id=3 * n + k)
    wu = synth.quant_matrix(fmt, n, k, seed=5, tensor_id=3 * n + k + 1)
    x = synth.normal_f32((b, k), seed=5, tensor_id=3 * n + k + 2)
    h = host(g.quant_gemv_swiglu(fmt, dev(wg), dev(wu), n, k, dev(x)))
    o = oracle.gated_ffn(fmt, wg, wu, n, k, x)
    worst = check_bound(h, o["h"], _swiglu_bound(o), "swiglu")
    say(f"  worst err / bound = {worst:.3g}")


def test_gemv_swiglu_strided_and_repeatable(g):
    """Row strides of x and h larger than K and N (through the C ABI), and the
    same bits on a second call."""
    import ctypes
    for fmt, n, k, b in ((Q4, 260, 1024, 5), (Q8, 130, 2048, 1)):
        wg = synth.quant_matrix(fmt, n, k, seed=6, tensor_id=n)
        wu = synth.quant_matrix(fmt, n, k, seed=6, tensor_id=n + 1)
        x = synth.normal_f32((b, k), seed=6, tensor_id=n + 2)
        ldx, ldh = k + 64, n + 12
        xp = torch.zeros((b, ldx), dtype=torch.float32, device="cuda")
        xp[:, :k] = dev(x)
        hp = torch.full((b, ldh), 7.0, dtype=torch.float32, device="cuda")
        ws = torch.zeros(max(g.quant_gemv_workspace_size(fmt, k, b), 256), dtype=torch.uint8,
                         device="cuda")
        wgd, wud = dev(wg), dev(wu)
        def call():
            rc = g._lib.quant_gemv_swiglu(fmt, wgd.data_ptr(), wud.data_ptr(), n, k,
                                          xp.data_ptr(), ldx, hp.data_ptr(), ldh, b,
                                          ws.data_ptr(), ws.numel(), None)
            assert rc == 0, rc
            torch.cuda.synchronize()
            return host(hp).copy()
        h1 = call()
        h2 = call()
        assert np.array_equal(h1, h2)
        assert np.all(h1[:, n:] == 7.0)        # the padding columns are not written
        o = oracle.gated_ffn(fmt, wg, wu, n, k, x)
        check_bound(h1[:, :n], o["h"], _swiglu_bound(o), "swiglu strided")


@pytest.mark.parametrize("path", PATHS)
def test_gemv_one_hot_columns_exact(g, path):
    """x = e_c gives the dequantized column c exactly (adds of zero are exact; on
    the matrix cores the power-of-two scaling and the fp16 split are exact too)."""
    say(f"gemv one-hot {path}")
    for fmt, n, k in ((Q8, 96, 2048), (Q4, 96, 2560)):
        w = synth.quant_matrix(fmt, n, k, seed=3, tensor_id=71)
        cols = [0, 31, 32, 255, 256, 1023, k - 1]
        x = np.zeros((len(cols), k), dtype=np.float32)
        for i, c in enumerate(cols):
            x[i, c] = 1.0
        y = host(g.quant_gemv(fmt, dev(w), n, k, dev(x), ws=PATHS[path]))
        dense = oracle.dequant(fmt, w, n, k)
        for i, c in enumerate(cols):
            assert np.array_equal(y[i], dense[:, c])


@pytest.mark.parametrize("path", PATHS)
def test_gemv_batch_equals_single_rows_and_is_deterministic(g, path):
    say(f"gemv batch_check {path}")
    ws = PATHS[path]
    for fmt, n, k in ((Q8, 200, 2048), (Q4, 200, 2560)):
        w = synth.quant_matrix(fmt, n, k, seed=4, tensor_id=72)
        x = synth.normal_f32((16, k), seed=4, tensor_id=73)
        wd, xd = dev(w), dev(x)
        yb = host(g.quant_gemv(fmt, wd, n, k, xd, ws=ws))
        yb2 = host(g.quant_gemv(fmt, wd, n, k, xd, ws=ws))
        assert np.array_equal(yb, yb2)
        yr, s = oracle.gemv(fmt, w, n, k, x)
        for b in range(16):
            y1 = host(g.quant_gemv(fmt, wd, n, k, dev(x[b:b + 1]), ws=ws))
            check_rel(y1, yr[b:b + 1], s[b:b + 1], GEMV_TOL, f"single row {b}")
            check_rel(yb[b:b + 1], yr[b:b + 1], s[b:b + 1], GEMV_TOL, f"batched row {b}")


@pytest.mark.parametrize("path", PATHS)
def test_gemv_integer_case_exact(g, path):
    """d = 1 and small integer activations: every partial sum is an exact integer
    (on the matrix cores an exact multiple of the power-of-two scale)."""
    say(f"gemv integer exact {path}")
    n, k = 130, 4096
    rng = np.random.default_rng(11)
    q = rng.integers(-127, 128, size=(n, k))
    raw = np.zeros((n * k // 32, 34), dtype=np.uint8)
    raw[:, 0:2] = [0x00, 0x3C]
    raw[:, 2:] = q.reshape(-1, 32).astype(np.int8).view(np.uint8)
    x = rng.integers(-8, 9, size=(4, k)).astype(np.float32)
    y = host(g.quant_gemv(Q8, dev(raw.reshape(n, -1)), n, k, dev(x), ws=PATHS[path]))
    ref = (x.astype(np.int64) @ q.T).astype(np.float32)
    assert np.array_equal(y, ref)


def test_gemv_empty_and_errors(g):
    say("gemv edge")
    w = dev(np.zeros(34, dtype=np.uint8))
    y = g.quant_gemv(Q8, w, 0, 32, dev(np.zeros((1, 32), np.float32)))
    assert y.shape == (1, 0)
    with pytest.raises(g.GGQError):
        g.quant_gemv(Q8, dev(np.zeros(17 * 34, np.uint8)), 1, 17 * 32 + 16,
                     dev(np.zeros((1, 17 * 32 + 16), np.float32)))


# --------------------------------------------------------------------------- #
# grouped launches and graph replay
def _group_case(fmt, specs, b, seed=6):
    mats = []
    for i, (n, k) in enumerate(specs):
        w = synth.quant_matrix(fmt, n, k, seed=seed, tensor_id=200 + i)
        x = synth.normal_f32((b, k), seed=seed, tensor_id=300 + i)
        mats.append((w, n, k, x))
    return mats


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("fmt,specs,b", [
    (Q8, [(3072, 2048), (2048, 2048), (6144, 2048), (6144, 2048), (2048, 6144), (4099, 2048)], 1),
    (Q8, [(300, 2048), (77, 6144), (5, 224), (129, 512)], 8),     # includes a K % 256 != 0 member
    (Q4, [(9728, 2560), (2560, 9728), (33, 256)], 4),
    (Q4, [(100, 2560), (1, 9728)], 16),
])
def test_gemv_grouped_parity(g, fmt, specs, b, path):
    say(f"gemv grouped fmt={fmt} b={b} {specs} path={path}")
    mats = _group_case(fmt, specs, b)
    items = [(dev(w), n, k, dev(x), torch.empty((b, n), device="cuda")) for w, n, k, x in mats]
    g.quant_gemv_grouped(fmt, items, ws=PATHS[path])
    first = [host(it[4]) for it in items]
    g.GemvGroup(fmt, items, ws=PATHS[path])()
    for (w, n, k, x), it, y0 in zip(mats, items, first):
        y = host(it[4])
        assert np.array_equal(y, y0)          # deterministic
        yr, s = oracle.gemv(fmt, w, n, k, x)
        check_rel(y, yr, s, GEMV_TOL, f"grouped {n}x{k}")


@pytest.mark.parametrize("b,ws", [(1, None), (8, "auto")])
def test_gemv_layer_set_as_benchmarked(g, b, ws):
    """The exact launches bench.py times: one grouped call over the whole ~1B
    Q8_0 layer set (head included) on the benchmark's seeded inputs, batch 1 on
    the vector units and batch 8 on the matrix cores; every output checked."""
    say(f"gemv bench launch b={b} ws={ws}")
    mats, items = [], []
    for name, n, k in synth.DENSE_1B_LAYER_SET:
        tid = synth.tid(1, n, k)
        w = synth.q8_0_matrix(n, k, seed=0, tensor_id=tid)
        x = synth.normal_f32((b, k), seed=0, tensor_id=tid + b)
        mats.append((name, w, n, k, x))
        items.append((dev(w), n, k, dev(x), torch.empty((b, n), device="cuda")))
    g.GemvGroup(Q8, items, ws=ws)()
    for (name, w, n, k, x), it in zip(mats, items):
        yr, s = oracle.gemv(Q8, w, n, k, x)
        worst = check_rel(host(it[4]), yr, s, GEMV_TOL, f"{name} b{b}")
        say(f"  {name}: worst err / bound = {worst:.3g}")


def test_graph_replays_match_eager(g):
    """Grouped GEMV, GEMM and the MoE layer captured in one HIP graph: every
    replay, with eager work in between, equals the eager result bit for bit."""
    say("graph replay")
    mats = _group_case(Q8, [(2048, 2048), (512, 6144)], 8)
    items = [(dev(w), n, k, dev(x), torch.empty((8, n), device="cuda")) for w, n, k, x in mats]
    grp = g.GemvGroup(Q8, items, ws="auto")
    grp1 = g.GemvGroup(Q8, [(it[0], it[1], it[2], it[3][:1], it[4][:1].clone()) for it in items])
    wq = dev(synth.q4_k_matrix(256, 1024, seed=1, tensor_id=5))
    a = dev(synth.normal_f32((64, 1024), seed=1, tensor_id=6))
    c = torch.empty((64, 256), device="cuda")
    ws = torch.zeros(g.quant_gemm_workspace_size(Q4, 64, 256, 1024), dtype=torch.uint8, device="cuda")
    mo = synth.moe_layer(seed=2, n_tokens=4)
    wr, x = dev(mo["wr"]), dev(mo["x"])
    wg, wu, wd = dev(mo["wg"]), dev(mo["wu"]), dev(mo["wd"])
    e, h, f, k = synth.MOE_EXPERTS, synth.MOE_HIDDEN, synth.MOE_FFN, synth.MOE_TOP_K
    mws = torch.empty(g.moe_workspace_size(e, 4, k, h, f), dtype=torch.uint8, device="cuda")
    ym = torch.empty((4, h), device="cuda")
    idx = torch.empty((4, k), dtype=torch.int32, device="cuda")

    def work():
        grp()
        grp1()
        g.quant_gemm(Q4, wq, 256, 1024, a, c, ws)
        ii, pp, _ = g.moe_route(wr, x, k)
        idx.copy_(ii)
        g.moe_expert_gemv(Q4, wg, wu, wd, e, h, f, x, ii, pp, ym, mws)

    outs = lambda: ([host(it[4]).copy() for it in items] + [host(it[4]).copy() for it in grp1._keep]
                    + [host(c).copy(), host(ym).copy(), host(idx).copy()])
    work()
    ref = outs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        work()
    for rep in range(3):
        for it in items:
            it[4].fill_(float("nan"))
        c.fill_(float("nan"))
        ym.fill_(float("nan"))
        _ = torch.randn(1000, device="cuda").sum()     # eager work between replays
        torch.cuda.synchronize()
        gr.replay()
        got = outs()
        for r_, g_ in zip(ref, got):
            assert np.array_equal(r_, g_), f"replay {rep}"
