"""GPU parity: moe_expert_gemm (the routed expert feed-forward at prompt batch,
grouped bf16 products on the matrix cores) against the CPU oracle.

README opening paragraph for the layer; phobos-bench pp<N> for prompt batches.
Each of the three products may be off by the prompt-GEMM tolerance (8e-3 of
sum|a w|); tests.moe_bound propagates that through silu(g)*u, the down
product and the probability-weighted sum.  Full-size layers (128 experts,
top-8, H 2048, F 768) are checked on sampled tokens, which the oracle computes
one by one; small layers on every output.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import GEMM_TOL, check_bound, dev, host, moe_bound, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

Q8, Q4 = synth.FMT_Q8_0, synth.FMT_Q4_K


@pytest.fixture(scope="module")
def g():
    import quantized_gguf_q8_amd as g
    return g


def _small(seed, fmt, e, h, f, t):
    rng = np.random.default_rng(seed)
    return {
        "wr": (0.05 * rng.standard_normal((e, h))).astype(np.float32),
        "wg": synth.quant_matrix(fmt, e * f, h, seed, 71).reshape(e, f, -1),
        "wu": synth.quant_matrix(fmt, e * f, h, seed, 72).reshape(e, f, -1),
        "wd": synth.quant_matrix(fmt, e * h, f, seed, 73).reshape(e, h, -1),
        "x": synth.normal_f32((t, h), seed, 74),
    }


def _run(g, fmt, mo, idx, probs, e, h, f):
    return host(g.moe_expert_gemm(fmt, dev(mo["wg"]), dev(mo["wu"]), dev(mo["wd"]), e, h, f,
                                  dev(mo["x"]), dev(idx), dev(probs)))


def _check_tokens(fmt, mo, idx, probs, h, f, y, tokens, what):
    tokens = [int(t) for t in tokens]
    p64 = probs.astype(np.float64)
    yref = oracle.moe(fmt, mo["wg"], mo["wu"], mo["wd"], mo["wg"].shape[0], h, f,
                      mo["x"][tokens], idx[tokens], p64[tokens])
    bound = moe_bound(fmt, mo, idx, p64, h, f, GEMM_TOL, tokens=tokens)
    return check_bound(y[tokens], yref, bound, what)


@pytest.mark.parametrize("t", [64, 512])
def test_moe_gemm_full_size_sampled(g, t):
    """128-expert, top-8 Q4_K layer routed on the device; 16 sampled tokens."""
    say(f"moe gemm t={t}")
    e, h, f, k = synth.MOE_EXPERTS, synth.MOE_HIDDEN, synth.MOE_FFN, synth.MOE_TOP_K
    mo = synth.moe_layer(seed=2, n_tokens=t)
    idx, probs, _ = g.moe_route(dev(mo["wr"]), dev(mo["x"]), k)
    idx, probs = host(idx), host(probs)
    y = _run(g, Q4, mo, idx, probs, e, h, f)
    assert np.all(np.isfinite(y))
    # the tokens of the busiest expert first, then an even spread
    counts = np.bincount(idx.ravel(), minlength=e)
    busiest = np.nonzero((idx == counts.argmax()).any(axis=1))[0][:4]
    tokens = sorted(set(busiest.tolist()) | set(np.linspace(0, t - 1, 12).astype(int).tolist()))
    w = _check_tokens(Q4, mo, idx, probs, h, f, y, tokens, f"moe gemm t={t}")
    say(f"  experts used {int((counts > 0).sum())}, most pairs {int(counts.max())}, "
        f"worst err / bound {w:.3g}")


@pytest.mark.parametrize("fmt,e,h,f,t,k", [
    (Q4, 6, 512, 256, 5, 3),
    (Q8, 9, 768, 512, 40, 4),
    (Q4, 4, 256, 768, 100, 4),     # ~100 pairs per expert: two tiles each
    (Q8, 1, 256, 256, 300, 1),     # one expert takes every token: five tiles
    (Q4, 130, 256, 256, 40, 32),   # more than 128 experts, top-32
    (Q4, 3, 256, 256, 16, 3),      # exactly 16 pairs per expert, no padding
    (Q8, 2, 256, 512, 64, 2),      # exactly one full tile per expert
    (Q4, 2, 512, 256, 65, 2),      # 65 pairs: a full tile and one row plus padding
    (Q8, 8, 256, 256, 1, 2),       # one token
])
def test_moe_gemm_small_shapes(g, fmt, e, h, f, t, k):
    say(f"moe gemm small fmt={fmt} e={e} h={h} f={f} t={t} k={k}")
    mo = _small(4, fmt, e, h, f, t)
    lref, _ = oracle.router_logits(mo["wr"], mo["x"])
    idx = oracle.topk(lref, k)
    probs = oracle.route_probs(lref, idx).astype(np.float32)
    y = _run(g, fmt, mo, idx, probs, e, h, f)
    w = _check_tokens(fmt, mo, idx, probs, h, f, y, range(t), "moe gemm small")
    say(f"  worst err / bound {w:.3g}")


@pytest.mark.parametrize("fmt", [Q4, Q8])
def test_moe_gemm_repeated_and_out_of_range(g, fmt):
    """Slots that repeat an expert each count once; out-of-range indices count
    with weight 0 (the oracle skips them)."""
    say(f"moe gemm repeated / out of range fmt={fmt}")
    e, h, f, k = 10, 512, 768, 5
    mo = _small(8, fmt, e, h, f, 4)
    idx = np.array([[4, 4, 7, 4, 1], [2, 2, 2, 2, 2], [9, 0, 9, 3, 0], [-1, 5, 10, 5, 99]],
                   dtype=np.int32)
    probs = np.array([[0.3, 0.2, 0.25, 0.15, 0.1]] * 4, dtype=np.float32)
    y = _run(g, fmt, mo, idx, probs, e, h, f)
    _check_tokens(fmt, mo, idx, probs, h, f, y, range(4), "moe gemm repeated")


@pytest.mark.parametrize("fmt", [Q4, Q8])
def test_moe_gemm_out_of_range_poisoned_expert0(g, fmt):
    """Out-of-range slots are grouped with expert 0 yet contribute nothing:
    with expert 0 unselected and its scales NaN, the output stays finite and
    within the bound of the oracle, which leaves those slots out."""
    say(f"moe gemm out of range, expert 0 poisoned fmt={fmt}")
    e, h, f, k = 10, 512, 768, 5
    mo = _small(10, fmt, e, h, f, 4)
    idx = np.array([[4, 4, 7, 4, 1], [2, -2, 2, 2, 2], [9, 11, 9, 3, 5], [-1, 5, 10, 5, 99]],
                   dtype=np.int32)
    probs = np.array([[0.3, 0.2, 0.25, 0.15, 0.1]] * 4, dtype=np.float32)
    blk = 144 if fmt == Q4 else 34
    for key in ("wg", "wu", "wd"):
        mo[key][0].reshape(-1, blk)[:, 0:2] = [0xFF, 0x7F]
    y = _run(g, fmt, mo, idx, probs, e, h, f)
    assert np.all(np.isfinite(y))
    _check_tokens(fmt, mo, idx, probs, h, f, y, range(4), "moe gemm expert 0 poisoned")


def test_moe_gemm_most_pairs(g):
    """T * top_k = 65536 pairs (the largest call), small matrices; sampled tokens."""
    say("moe gemm 65536 pairs")
    e, h, f, k, t = 128, 256, 256, 8, 8192
    mo = _small(9, Q4, e, h, f, t)
    lref, _ = oracle.router_logits(mo["wr"], mo["x"])
    idx = oracle.topk(lref, k)
    probs = oracle.route_probs(lref, idx).astype(np.float32)
    y = _run(g, Q4, mo, idx, probs, e, h, f)
    assert np.all(np.isfinite(y))
    tokens = np.linspace(0, t - 1, 16).astype(int)
    _check_tokens(Q4, mo, idx, probs, h, f, y, tokens, "moe gemm most pairs")


def test_moe_gemm_reads_only_selected_experts(g):
    """NaN scales in every unselected expert leave the output unchanged."""
    say("moe gemm poison")
    e, h, f, k, t = 12, 512, 256, 2, 40
    mo = _small(5, Q4, e, h, f, t)
    idx = (np.arange(t * k, dtype=np.int32) % 5).reshape(t, k) * 2   # experts 0,2,..,8
    probs = np.full((t, k), 0.5, dtype=np.float32)
    y = _run(g, Q4, mo, idx, probs, e, h, f)
    for ex in set(range(e)) - set(idx.ravel().tolist()):
        for key in ("wg", "wu", "wd"):
            mo[key][ex].reshape(-1, 144)[:, 0:2] = [0xFF, 0x7F]
    y2 = _run(g, Q4, mo, idx, probs, e, h, f)
    assert np.array_equal(y, y2)


def test_moe_gemm_deterministic(g):
    """Slots of one expert may be filled in any order; the results may not vary."""
    say("moe gemm determinism")
    e, h, f, k = synth.MOE_EXPERTS, synth.MOE_HIDDEN, synth.MOE_FFN, synth.MOE_TOP_K
    mo = synth.moe_layer(seed=3, n_tokens=256)
    idx, probs, _ = g.moe_route(dev(mo["wr"]), dev(mo["x"]), k)
    idx, probs = host(idx), host(probs)
    y1 = _run(g, Q4, mo, idx, probs, e, h, f)
    y2 = _run(g, Q4, mo, idx, probs, e, h, f)
    assert np.array_equal(y1, y2)


def test_moe_gemm_q8_0_mid_size(g):
    """Q8_0, 64 experts, H 1024, F 512, 256 tokens, top-4 (16 pairs per expert
    on average, up to 2 tiles); 12 sampled tokens."""
    say("moe gemm q8_0 mid size")
    e, h, f, k, t = 64, 1024, 512, 4, 256
    mo = _small(10, Q8, e, h, f, t)
    lref, _ = oracle.router_logits(mo["wr"], mo["x"])
    idx = oracle.topk(lref, k)
    probs = oracle.route_probs(lref, idx).astype(np.float32)
    y = _run(g, Q8, mo, idx, probs, e, h, f)
    tokens = np.linspace(0, t - 1, 12).astype(int)
    _check_tokens(Q8, mo, idx, probs, h, f, y, tokens, "moe gemm q8_0 mid size")


def test_moe_gemm_graph_replays_match_eager(g):
    """Route + moe_expert_gemm captured in a HIP graph: every replay, with eager
    work in between, equals the eager result bit for bit."""
    say("moe gemm graph replay")
    e, h, f, k, t = synth.MOE_EXPERTS, synth.MOE_HIDDEN, synth.MOE_FFN, synth.MOE_TOP_K, 96
    mo = synth.moe_layer(seed=4, n_tokens=t)
    wr, x = dev(mo["wr"]), dev(mo["x"])
    wg, wu, wd = dev(mo["wg"]), dev(mo["wu"]), dev(mo["wd"])
    ws = torch.empty(g.moe_gemm_workspace_size(e, t, k, h, f), dtype=torch.uint8, device="cuda")
    y = torch.empty((t, h), device="cuda")

    def work():
        ii, pp, _ = g.moe_route(wr, x, k)
        g.moe_expert_gemm(Q4, wg, wu, wd, e, h, f, x, ii, pp, y, ws)

    work()
    ref = host(y).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()
    torch.cuda.current_stream().wait_stream(s)
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        work()
    for rep in range(4):
        y.zero_()
        ws.fill_(0xA5)
        gr.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(y), ref), f"replay {rep}"
        work()                                  # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(host(y), ref), f"eager after replay {rep}"

