"""GPU parity: moe_route (logits, exact top-k indices, probabilities) and
moe_expert_gemv (routed expert feed-forward) against the CPU oracle.

README opening paragraph: each token goes to a few experts; only their weights
are used.  Index protocol: (i) device logits within 1e-5 * sum|w x| of the fp64
logits; (ii) the oracle's top-k of the device's own fp32 logits equals the
device's indices exactly, in order; (iii) the device's set equals the fp64
top-k wherever the fp64 gap between rank k and k+1 exceeds twice the logit
tolerance (closer cases are near-ties and are counted, not failed).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import GEMV_TOL, check_bound, check_rel, dev, host, moe_bound, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

Q8, Q4 = synth.FMT_Q8_0, synth.FMT_Q4_K


@pytest.fixture(scope="module")
def g():
    import quantized_gguf_q8_amd as g
    return g


def _route_checks(g, wr, x, k):
    idx, probs, logits = g.moe_route(dev(wr), dev(x), k)
    idx, probs, logits = host(idx), host(probs), host(logits)
    lref, s = oracle.router_logits(wr, x)
    check_rel(logits, lref, s, GEMV_TOL, "router logits")                      # (i)
    assert np.array_equal(oracle.topk(logits, k), idx)                          # (ii)
    ref_idx = oracle.topk(lref, k)
    tol = 2 * GEMV_TOL * s.max(axis=1)
    near = 0
    for t in range(x.shape[0]):                                                 # (iii)
        srt = np.sort(lref[t])[::-1]
        if k < lref.shape[1] and srt[k - 1] - srt[k] <= tol[t]:
            near += 1
            continue
        assert set(idx[t]) == set(ref_idx[t]), t
        gaps = -np.diff(lref[t, ref_idx[t]])
        if np.all(gaps > tol[t]):
            assert np.array_equal(idx[t], ref_idx[t]), t
    # probabilities: the oracle's renormalised softmax of the device's logits
    pref = oracle.route_probs(logits.astype(np.float64), idx)
    check_bound(probs, pref, np.full(pref.shape, 2e-6), "route probs")
    return idx, probs, near


@pytest.mark.parametrize("t", [1, 16, 33, 64, 512])
def test_route_moe_router(g, t):
    """1 and 16 tokens: one wave per expert; from 32 tokens: 16x16 tiles (33:
    a ragged last tile; 512: the prompt batch)."""
    say(f"route t={t}")
    mo = synth.moe_layer(seed=0, n_tokens=t)
    _, _, near = _route_checks(g, mo["wr"], mo["x"], synth.MOE_TOP_K)
    say(f"  near-ties: {near}")


def test_route_ties_and_edges(g):
    say("route ties")
    e, h = 40, 64
    wr = np.zeros((e, h), dtype=np.float32)
    x = synth.normal_f32((3, h), seed=1, tensor_id=5)
    idx, probs, _ = g.moe_route(dev(wr), dev(x), 8)
    assert np.array_equal(host(idx), np.tile(np.arange(8, dtype=np.int32), (3, 1)))
    assert np.array_equal(host(probs), np.full((3, 8), 0.125, np.float32))
    # duplicated router rows give exactly equal logits: lower index first
    wr = synth.normal_f32((e, h), seed=1, tensor_id=6)
    wr[7] = wr[30]
    wr[12] = wr[30]
    _route_checks(g, wr, x, 8)
    idx1, p1, _ = g.moe_route(dev(wr), dev(x), 1)
    assert np.array_equal(host(p1), np.ones((3, 1), np.float32))
    idxe, _, _ = _route_checks(g, wr, x, 32)
    assert all(len(set(r)) == 32 for r in idxe)


@pytest.mark.parametrize("e,k", [(200, 8), (300, 32), (1024, 17)])
def test_route_many_experts(g, e, k):
    """Expert counts past one and four logits per lane, with exact ties from
    duplicated router rows and rounded activations."""
    say(f"route e={e} k={k}")
    h = 64
    wr = synth.normal_f32((e, h), seed=2, tensor_id=7)
    wr[e - 1] = wr[3]
    wr[e // 2] = wr[3]
    wr[e - 2] = 0.0
    x = np.round(synth.normal_f32((5, h), seed=2, tensor_id=8) * 4) / 4
    idx, _, _ = _route_checks(g, wr, x.astype(np.float32), k)
    assert all(len(set(r)) == k for r in idx)


def test_route_tiles_ragged(g):
    """The tiled router with experts and columns that fill no tile or chunk
    evenly (E = 37, H = 300) and 50 tokens."""
    say("route tiles ragged")
    e, h, t = 37, 300, 50
    wr = synth.normal_f32((e, h), seed=3, tensor_id=9, std=0.05)
    x = synth.normal_f32((t, h), seed=3, tensor_id=10)
    _route_checks(g, wr, x, 6)


def _moe_bound(fmt, mo, x, idx, probs, e, h, f):
    """First-order bound for the end-to-end expert layer: per-GEMV 1e-5
    tolerances propagated through silu(g)*u (x is mo["x"])."""
    assert x is mo["x"]
    return moe_bound(fmt, mo, idx, probs, h, f, GEMV_TOL)


def _run_moe(g, fmt, mo, idx, probs, e, h, f):
    x = mo["x"]
    t, k = idx.shape
    ws = torch.empty(g.moe_workspace_size(e, t, k, h, f), dtype=torch.uint8, device="cuda")
    y = host(g.moe_expert_gemv(fmt, dev(mo["wg"]), dev(mo["wu"]), dev(mo["wd"]), e, h, f,
                               dev(x), dev(idx), dev(probs), ws=ws))
    off = g.moe_workspace_h_offset(e, t, k)
    hbuf = host(ws[off:off + t * k * f * 4].view(torch.float32)).reshape(t, k, f)
    return y, hbuf


@pytest.mark.parametrize("t", [1, 16])
def test_moe_layer_full_size(g, t):
    """The 128-expert, top-8 Q4_K layer with its own routing."""
    say(f"moe t={t}")
    e, h, f, k = synth.MOE_EXPERTS, synth.MOE_HIDDEN, synth.MOE_FFN, synth.MOE_TOP_K
    mo = synth.moe_layer(seed=0, n_tokens=t)
    idx, probs, _ = g.moe_route(dev(mo["wr"]), dev(mo["x"]), k)
    idx, probs = host(idx), host(probs)
    y, hbuf = _run_moe(g, Q4, mo, idx, probs, e, h, f)
    p64 = probs.astype(np.float64)
    yref, href = oracle.moe(Q4, mo["wg"], mo["wu"], mo["wd"], e, h, f, mo["x"], idx, p64,
                            want_h=True)
    # stage: hidden state against the oracle's silu(g)*u
    for ti in range(t):
        for s in range(k):
            o = oracle.expert_ffn(Q4, mo["wg"], mo["wu"], mo["wd"], int(idx[ti, s]), h, f,
                                  mo["x"][ti])
            sig = 1.0 / (1.0 + np.exp(-o["g"]))
            hb = (1.1 * np.abs(o["u"]) * GEMV_TOL * o["sg"] + np.abs(o["g"] * sig) * GEMV_TOL * o["su"]
                  + 1e-6 * np.abs(o["h"]))
            check_bound(hbuf[ti, s], o["h"], hb, f"h t{ti} s{s}")
            # stage: down projection + combine fed with the device's own h
    yst = np.zeros((t, h))
    sst = np.zeros((t, h))
    for ti in range(t):
        for s in range(k):
            ex = int(idx[ti, s])
            yy, ss = oracle.matvec_f64(Q4, mo["wd"][ex], h, f, hbuf[ti, s].astype(np.float64))
            yst[ti] += p64[ti, s] * yy
            sst[ti] += p64[ti, s] * ss
    # down product within GEMV_TOL of sum|Wd h| per slot; the fp32 combine
    # (k products p*d and k-1 additions, each rounded once) adds at most
    # k * 2^-24 of sum_s p_s |d_s| <= sum_s p_s sum|Wd h| (1 + GEMV_TOL)
    comb = k * 2.0 ** -24 * (1 + GEMV_TOL)
    w1 = check_rel(y, yst, sst, GEMV_TOL + comb, "down+combine (device h)")
    bound = _moe_bound(Q4, mo, mo["x"], idx, p64, e, h, f)
    w2 = check_bound(y, yref, bound, "moe end to end")
    say(f"  worst down/combine {w1:.3g}, end-to-end {w2:.3g}")


def _small(seed, fmt, e, h, f, t):
    rng = np.random.default_rng(seed)
    mo = {
        "wr": (0.05 * rng.standard_normal((e, h))).astype(np.float32),
        "wg": synth.quant_matrix(fmt, e * f, h, seed, 61).reshape(e, f, -1),
        "wu": synth.quant_matrix(fmt, e * f, h, seed, 62).reshape(e, f, -1),
        "wd": synth.quant_matrix(fmt, e * h, f, seed, 63).reshape(e, h, -1),
        "x": synth.normal_f32((t, h), seed, 64),
    }
    return mo


@pytest.mark.parametrize("fmt,e,h,f,t,k", [
    (Q4, 6, 512, 256, 5, 3), (Q8, 9, 768, 512, 7, 4), (Q4, 4, 256, 768, 33, 4),
    (Q8, 130, 256, 256, 3, 32),
    (Q8, 20, 512, 256, 1, 6),        # one token, Q8_0: the vector-unit stages
    (Q4, 16, 256, 256, 40, 8),       # 320 pairs: lists built by the grouping kernel
    (Q8, 12, 512, 256, 70, 4),       # 280 pairs, Q8_0, experts with > 8 tokens
    # one token whose down projection does not fit the fused one-token
    # down-and-combine kernel (top_k * F floats of h exceed its LDS): the
    # streaming down stage for every slot, then the slot-order combine
    (Q4, 16, 512, 2048, 1, 8),
    (Q8, 16, 512, 2048, 1, 8),
    (Q8, 40, 256, 768, 1, 32),
])
def test_moe_small_shapes(g, fmt, e, h, f, t, k):
    say(f"moe small fmt={fmt} e={e} h={h} f={f} t={t} k={k}")
    mo = _small(3, fmt, e, h, f, t)
    lref, _ = oracle.router_logits(mo["wr"], mo["x"])
    idx = oracle.topk(lref, k)
    probs = oracle.route_probs(lref, idx).astype(np.float32)
    y, _ = _run_moe(g, fmt, mo, idx, probs, e, h, f)
    yref = oracle.moe(fmt, mo["wg"], mo["wu"], mo["wd"], e, h, f, mo["x"], idx,
                      probs.astype(np.float64))
    bound = _moe_bound(fmt, mo, mo["x"], idx, probs.astype(np.float64), e, h, f)
    check_bound(y, yref, bound, "moe small")


@pytest.mark.parametrize("fmt,t", [(Q4, 1), (Q8, 1), (Q4, 3)])
def test_moe_repeated_expert_in_slots(g, fmt, t):
    """A token whose slots name the same expert more than once (not produced by
    moe_route, but valid input): every slot still counts once."""
    say(f"moe repeated expert fmt={fmt} t={t}")
    e, h, f, k = 10, 512, 768, 5
    mo = _small(7, fmt, e, h, f, t)
    idx = np.array([[4, 4, 7, 4, 1], [2, 2, 2, 2, 2], [9, 0, 9, 3, 0]][:t], dtype=np.int32)
    probs = np.array([[0.3, 0.2, 0.25, 0.15, 0.1]] * t, dtype=np.float32)
    y, _ = _run_moe(g, fmt, mo, idx, probs, e, h, f)
    yref = oracle.moe(fmt, mo["wg"], mo["wu"], mo["wd"], e, h, f, mo["x"], idx,
                      probs.astype(np.float64))
    bound = _moe_bound(fmt, mo, mo["x"], idx, probs.astype(np.float64), e, h, f)
    check_bound(y, yref, bound, "moe repeated expert")


@pytest.mark.parametrize("fmt,t", [(Q4, 1), (Q8, 1), (Q4, 3)])
def test_moe_out_of_range_slots(g, fmt, t):
    """Slots naming no expert (negative or >= E) count with weight 0; the
    oracle leaves them out."""
    say(f"moe out-of-range slots fmt={fmt} t={t}")
    e, h, f, k = 10, 512, 768, 5
    mo = _small(8, fmt, e, h, f, t)
    idx = np.array([[-1, 5, 10, 5, 99], [3, -7, 3, 1, 0], [9, 9, 12, 0, 4]][:t], dtype=np.int32)
    probs = np.array([[0.3, 0.2, 0.25, 0.15, 0.1]] * t, dtype=np.float32)
    y, _ = _run_moe(g, fmt, mo, idx, probs, e, h, f)
    yref = oracle.moe(fmt, mo["wg"], mo["wu"], mo["wd"], e, h, f, mo["x"], idx,
                      probs.astype(np.float64))
    bound = _moe_bound(fmt, mo, mo["x"], idx, probs.astype(np.float64), e, h, f)
    check_bound(y, yref, bound, "moe out-of-range slots")


@pytest.mark.parametrize("fmt,t", [(Q4, 1), (Q8, 1), (Q4, 3), (Q8, 17)])
def test_moe_out_of_range_slots_poisoned_expert0(g, fmt, t):
    """Slots naming no expert are grouped with expert 0 but must contribute
    nothing: with expert 0 unselected and its scales NaN, the output is finite
    and within the bound of the oracle, which leaves those slots out."""
    say(f"moe out-of-range slots, expert 0 poisoned fmt={fmt} t={t}")
    e, h, f, k = 10, 512, 768, 5
    mo = _small(9, fmt, e, h, f, t)
    rows = [[-1, 5, 10, 5, 99], [3, -7, 3, 1, 2], [9, 9, 12, 6, 4]]
    idx = np.array([rows[i % 3] for i in range(t)], dtype=np.int32)
    probs = np.array([[0.3, 0.2, 0.25, 0.15, 0.1]] * t, dtype=np.float32)
    blk = 144 if fmt == Q4 else 34
    for key in ("wg", "wu", "wd"):
        mo[key][0].reshape(-1, blk)[:, 0:2] = [0xFF, 0x7F]     # d = NaN
    y, _ = _run_moe(g, fmt, mo, idx, probs, e, h, f)
    assert np.all(np.isfinite(y))
    yref = oracle.moe(fmt, mo["wg"], mo["wu"], mo["wd"], e, h, f, mo["x"], idx,
                      probs.astype(np.float64))
    bound = _moe_bound(fmt, mo, mo["x"], idx, probs.astype(np.float64), e, h, f)
    check_bound(y, yref, bound, "moe out-of-range slots, expert 0 poisoned")


@pytest.mark.parametrize("t", [1, 3])
def test_moe_reads_only_selected_experts(g, t):
    """NaN scales in every unselected expert leave the output unchanged."""
    say(f"moe poison t={t}")
    e, h, f, k = 12, 512, 256, 2
    mo = _small(5, Q4, e, h, f, t)
    lref, _ = oracle.router_logits(mo["wr"], mo["x"])
    idx = oracle.topk(lref, k)
    probs = oracle.route_probs(lref, idx).astype(np.float32)
    y, _ = _run_moe(g, Q4, mo, idx, probs, e, h, f)
    for ex in set(range(e)) - set(idx.ravel().tolist()):
        for key in ("wg", "wu", "wd"):
            mo[key][ex].reshape(-1, 144)[:, 0:2] = [0xFF, 0x7F]
    y2, _ = _run_moe(g, Q4, mo, idx, probs, e, h, f)
    assert np.array_equal(y, y2)


def test_moe_deterministic(g):
    say("moe determinism")
    e, h, f, k = synth.MOE_EXPERTS, synth.MOE_HIDDEN, synth.MOE_FFN, synth.MOE_TOP_K
    mo = synth.moe_layer(seed=1, n_tokens=16)
    idx, probs, _ = g.moe_route(dev(mo["wr"]), dev(mo["x"]), k)
    idx, probs = host(idx), host(probs)
    y1, _ = _run_moe(g, Q4, mo, idx, probs, e, h, f)
    y2, _ = _run_moe(g, Q4, mo, idx, probs, e, h, f)
    assert np.array_equal(y1, y2)
