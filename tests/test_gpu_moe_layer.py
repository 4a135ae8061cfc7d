"""GPU parity: moe_layer_gemv (router, selection and routed experts in one
call; for one token of at most 256 experts the gate/up stage takes the
selection from the router's logits itself) against
moe_route followed by moe_expert_gemv, bit for bit, and end to end against
the CPU oracle.

README opening paragraph: each token goes to a few experts and only their
weights take part.  The fused routing runs the same arithmetic as the
router and top-k kernels, so logits, indices, probabilities and y must be
identical; the two-call path itself is checked against the oracle in
test_gpu_moe.py.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import GEMV_TOL, check_bound, dev, host, moe_bound, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

Q8, Q4 = synth.FMT_Q8_0, synth.FMT_Q4_K


@pytest.fixture(scope="module")
def g():
    import quantized_gguf_q8_amd as g
    return g


def _layer(seed, fmt, e, h, f, t):
    rng = np.random.default_rng(seed)
    return {
        "wr": (0.05 * rng.standard_normal((e, h))).astype(np.float32),
        "wg": synth.quant_matrix(fmt, e * f, h, seed, 71).reshape(e, f, -1),
        "wu": synth.quant_matrix(fmt, e * f, h, seed, 72).reshape(e, f, -1),
        "wd": synth.quant_matrix(fmt, e * h, f, seed, 73).reshape(e, h, -1),
        "x": synth.normal_f32((t, h), seed, 74),
    }


def _two_calls(g, fmt, d, e, h, f, k):
    idx, probs, logits = g.moe_route(d["wr"], d["x"], k)
    y = g.moe_expert_gemv(fmt, d["wg"], d["wu"], d["wd"], e, h, f, d["x"], idx, probs)
    return [host(v) for v in (y, idx, probs, logits)]


def _same(a, b, what):
    for name, u, v in zip(("y", "idx", "probs", "logits"), a, b):
        assert u.shape == v.shape, (what, name)
        uu = u.view(np.uint32) if u.dtype == np.float32 else u
        vv = v.view(np.uint32) if v.dtype == np.float32 else v
        assert np.array_equal(uu, vv), (what, name)


@pytest.mark.parametrize("fmt,e,h,f,t,k", [
    (Q4, 128, 2048, 768, 1, 8),      # the 35B-A3B-class layer, one token
    (Q8, 128, 2048, 768, 1, 8),
    (Q8, 200, 512, 256, 1, 6),       # 4 logits per lane in the selection, E % 4 != 0
    (Q4, 256, 1024, 512, 1, 8),      # the most experts the gate/up stage selects from
    (Q4, 1024, 256, 256, 1, 32),     # 16 logits per lane, top-32
    (Q4, 5, 1024, 512, 1, 1),        # top-1, two router workgroups (one partly idle)
    (Q4, 16, 512, 2048, 1, 8),       # down stage without the one-token kernel
    (Q4, 128, 2048, 768, 16, 8),     # 16 tokens: router and token split in one launch
    (Q8, 40, 512, 256, 5, 4),        # the same for Q8_0, two token groups of the router
    (Q4, 64, 1024, 512, 31, 4),      # the last token count with the joint launch
    (Q4, 64, 1024, 512, 32, 4),      # the tiled router, then moe_expert_gemv's own split
])
def test_layer_equals_route_then_experts(g, fmt, e, h, f, t, k):
    say(f"moe layer fmt={fmt} e={e} h={h} f={f} t={t} k={k}")
    mo = _layer(5, fmt, e, h, f, t)
    d = {n: dev(v) for n, v in mo.items()}
    ref = _two_calls(g, fmt, d, e, h, f, k)
    ws = torch.zeros(g.moe_layer_workspace_size(e, t, k, h, f), dtype=torch.uint8, device="cuda")
    for rep in range(3):
        got = g.moe_layer_gemv(fmt, d["wr"], d["wg"], d["wu"], d["wd"], e, h, f, d["x"], k, ws=ws)
        _same([host(v) for v in got], ref, f"call {rep}")
        assert int(ws[:g.CTRL_BYTES].count_nonzero()) == 0, "control block not returned to zero"


def test_layer_full_size_against_oracle(g):
    """The 128-expert top-8 Q4_K layer with its own routing, end to end against
    the oracle with the propagated per-product bound."""
    say("moe layer full size vs oracle")
    e, h, f, k = synth.MOE_EXPERTS, synth.MOE_HIDDEN, synth.MOE_FFN, synth.MOE_TOP_K
    mo = synth.moe_layer(seed=0, n_tokens=1)
    y, idx, probs, logits = (host(v) for v in g.moe_layer_gemv(
        Q4, dev(mo["wr"]), dev(mo["wg"]), dev(mo["wu"]), dev(mo["wd"]), e, h, f, dev(mo["x"]), k))
    lref, s = oracle.router_logits(mo["wr"], mo["x"])
    check_bound(logits, lref, GEMV_TOL * s, "router logits")
    assert np.array_equal(oracle.topk(logits, k), idx)
    pref = oracle.route_probs(logits.astype(np.float64), idx)
    check_bound(probs, pref, np.full(pref.shape, 2e-6), "route probs")
    p64 = probs.astype(np.float64)
    yref = oracle.moe(Q4, mo["wg"], mo["wu"], mo["wd"], e, h, f, mo["x"], idx, p64)
    bound = moe_bound(Q4, mo, idx, p64, h, f, GEMV_TOL)
    w = check_bound(y, yref, bound, "moe layer end to end")
    say(f"  worst err / bound = {w:.3g}")


def test_layer_graph_replays(g):
    """Captured in a HIP graph: every replay (with eager work and a sync in
    between) equals the eager call, and the control block stays zero."""
    say("moe layer graph replays")
    e, h, f, k = synth.MOE_EXPERTS, synth.MOE_HIDDEN, synth.MOE_FFN, synth.MOE_TOP_K
    mo = synth.moe_layer(seed=1, n_tokens=1)
    d = {n: dev(v) for n, v in mo.items()}
    ws = torch.zeros(g.moe_layer_workspace_size(e, 1, k, h, f), dtype=torch.uint8, device="cuda")
    out = (torch.empty((1, h), dtype=torch.float32, device="cuda"),
           torch.empty((1, k), dtype=torch.int32, device="cuda"),
           torch.empty((1, k), dtype=torch.float32, device="cuda"),
           torch.empty((1, e), dtype=torch.float32, device="cuda"))
    eager = [host(v) for v in g.moe_layer_gemv(Q4, d["wr"], d["wg"], d["wu"], d["wd"], e, h, f,
                                                 d["x"], k, out=out, ws=ws)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(gr):
            g.moe_layer_gemv(Q4, d["wr"], d["wg"], d["wu"], d["wd"], e, h, f, d["x"], k, out=out,
                             ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        for v in out:
            v.zero_()
        gr.replay()
        torch.cuda.synchronize()
        _same([host(v) for v in out], eager, f"replay {rep}")
        assert int(ws[:g.CTRL_BYTES].count_nonzero()) == 0
        torch.randn(1000, device="cuda").sum().item()   # unrelated eager work between replays
