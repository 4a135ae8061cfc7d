"""Pins of the oracle's products (GEMV, router/top-k, routed MoE, GEMM).

Each check ties the oracle to something other than itself: exact integer
arithmetic, exact rationals, numpy's own routines used as a single step, or an
invariant the method fixes (README "Inference": a batched pass equals single
passes -- the batch_check example; the routed expert layer equals a dense sum
with zero weight on unselected experts).
"""
from fractions import Fraction

import numpy as np
import pytest

import synth

Q8, Q4 = synth.FMT_Q8_0, synth.FMT_Q4_K


def _q8_blocks_with(n, k, d_bits, q):
    raw = np.zeros((n * k // 32, 34), dtype=np.uint8)
    raw[:, 0] = d_bits & 255
    raw[:, 1] = d_bits >> 8
    raw[:, 2:] = q.reshape(-1, 32).astype(np.int8).view(np.uint8)
    return raw.reshape(n, -1)


# --------------------------------------------------------------------------- #
# GEMV
@pytest.mark.parametrize("fmt,k", [(Q8, 1024), (Q4, 768)])
def test_gemv_one_hot_columns_bit_exact(orc, fmt, k):
    n = 48
    w = synth.quant_matrix(fmt, n, k, seed=0, tensor_id=11)
    dense = orc.dequant(fmt, w, n, k)
    cols = [0, 1, 31, 32, 255, 256, k - 1]
    x = np.zeros((len(cols), k), dtype=np.float32)
    for b, c in enumerate(cols):
        x[b, c] = 1.0
    y, s = orc.gemv(fmt, w, n, k, x)
    for b, c in enumerate(cols):
        assert np.array_equal(y[b], dense[:, c].astype(np.float64))
        assert np.array_equal(s[b], np.abs(dense[:, c]).astype(np.float64))


def test_gemv_integer_case_exact(orc):
    """d = 1 makes every weight the int8 quant; small integer activations keep
    every partial sum an exact integer, so the result must equal int64 matmul."""
    n, k = 40, 2048
    g = np.random.default_rng(3)
    q = g.integers(-127, 128, size=(n, k))
    w = _q8_blocks_with(n, k, 0x3C00, q)
    x = g.integers(-8, 9, size=(3, k)).astype(np.float32)
    y, _ = orc.gemv(Q8, w, n, k, x)
    ref = (x.astype(np.int64) @ q.T.astype(np.int64)).astype(np.float64)
    assert np.array_equal(y, ref)


def test_gemv_exact_rationals_small(orc):
    """K <= 256: exact rational dot products from the exact weights; the fp64 sum
    may differ only by its own rounding (K ulps of sum|w x| at most)."""
    n, k = 6, 256
    for fmt in (Q8, Q4):
        w = synth.quant_matrix(fmt, n, k, seed=2, tensor_id=5)
        x = synth.normal_f32((2, k), seed=2, tensor_id=6)
        dense = orc.dequant(fmt, w, n, k)
        y, s = orc.gemv(fmt, w, n, k, x)
        for b in range(2):
            for r in range(n):
                ex = sum(Fraction(float(dense[r, c])) * Fraction(float(x[b, c])) for c in range(k))
                assert abs(Fraction(y[b, r]) - ex) <= Fraction(k * 2.0 ** -52) * Fraction(s[b, r])


def test_gemv_batch_equals_single_passes(orc):
    n, k = 64, 2560
    w = synth.q4_k_matrix(n, k, seed=0, tensor_id=8)
    x = synth.normal_f32((5, k), seed=0, tensor_id=9)
    yb, sb = orc.gemv(Q4, w, n, k, x)
    for b in range(5):
        y1, s1 = orc.gemv(Q4, w, n, k, x[b:b + 1])
        assert np.array_equal(yb[b], y1[0]) and np.array_equal(sb[b], s1[0])


def test_gemv_row_ranges_and_threads_do_not_change_bits(orc):
    n, k = 100, 1024
    w = synth.q8_0_matrix(n, k, seed=0, tensor_id=12)
    x = synth.normal_f32((2, k), seed=0, tensor_id=13)
    y1, _ = orc.gemv(Q8, w, n, k, x, threads=1)
    y7, _ = orc.gemv(Q8, w, n, k, x, threads=7)
    assert np.array_equal(y1, y7)
    yr, _ = orc.gemv(Q8, w, n, k, x, rows=(17, 59))
    assert np.array_equal(yr[:, 17:59], y1[:, 17:59])


def test_gemv_against_numpy_matmul(orc):
    """numpy's fp64 matmul of the exact weights as an independent summation."""
    n, k = 96, 4096
    for fmt in (Q8, Q4):
        w = synth.quant_matrix(fmt, n, k, seed=1, tensor_id=14)
        x = synth.normal_f32((3, k), seed=1, tensor_id=15)
        y, s = orc.gemv(fmt, w, n, k, x)
        ref = x.astype(np.float64) @ orc.dequant(fmt, w, n, k).astype(np.float64).T
        assert np.all(np.abs(y - ref) <= 1e-13 * s)


def test_matvec_f64_plain_and_magnitude_modes(orc):
    """The fp64-input product used for the expert down projection and, with
    absw, for the propagated MoE error bound (sum_c |w[r][c]| v[c]): both modes
    against numpy matmuls of the exact weights and their magnitudes, with a
    signed v so that a mode that forgets the |.| (or applies it to v) fails."""
    n, k = 80, 1536
    rng = np.random.default_rng(11)
    v = rng.standard_normal(k)
    for fmt in (Q8, Q4):
        w = synth.quant_matrix(fmt, n, k, seed=2, tensor_id=16)
        wf = orc.dequant(fmt, w, n, k).astype(np.float64)
        y, s = orc.matvec_f64(fmt, w, n, k, v)
        assert np.all(np.abs(y - wf @ v) <= 1e-13 * s)
        assert np.allclose(s, np.abs(wf) @ np.abs(v), rtol=1e-13, atol=0)
        ya, sa = orc.matvec_f64(fmt, w, n, k, v, absw=True)
        ref = np.abs(wf) @ v
        assert np.all(np.abs(ya - ref) <= 1e-13 * sa)
        assert np.allclose(sa, s, rtol=1e-13, atol=0)
        # a non-negative v makes the magnitude product the sum of magnitudes
        yp, sp = orc.matvec_f64(fmt, w, n, k, np.abs(v), absw=True)
        assert np.allclose(yp, sp, rtol=1e-13, atol=0)
        assert not np.allclose(ya, y)


# --------------------------------------------------------------------------- #
# Router / top-k / routing weights
def test_topk_hand_built_ties(orc):
    l = np.array([[0.5, 2.0, 2.0, -1.0, 3.0, 2.0, 0.5, 3.0]])
    assert orc.topk(l, 4).tolist() == [[4, 7, 1, 2]]
    assert orc.topk(l, 6).tolist() == [[4, 7, 1, 2, 5, 0]]
    assert orc.topk(l.astype(np.float32), 6).tolist() == [[4, 7, 1, 2, 5, 0]]
    assert orc.topk(np.zeros((2, 128)), 8).tolist() == [list(range(8))] * 2


def test_router_zero_weights_give_uniform_choice(orc):
    wr = np.zeros((128, 2048), dtype=np.float32)
    x = synth.normal_f32((3, 2048), seed=0, tensor_id=1)
    l, _ = orc.router_logits(wr, x)
    idx = orc.topk(l, 8)
    assert idx.tolist() == [list(range(8))] * 3
    p = orc.route_probs(l, idx)
    assert np.array_equal(p, np.full((3, 8), 0.125))


def test_router_top1_weight_is_one(orc):
    mo = synth.moe_layer(seed=0, n_tokens=4)
    l, _ = orc.router_logits(mo["wr"], mo["x"])
    idx = orc.topk(l, 1)
    assert np.array_equal(orc.route_probs(l, idx), np.ones((4, 1)))
    assert np.array_equal(idx[:, 0], np.argmax(l, axis=1))


def test_router_permutation_equivariance(orc):
    mo = synth.moe_layer(seed=0, n_tokens=16)
    perm = np.random.default_rng(0).permutation(128)
    l, _ = orc.router_logits(mo["wr"], mo["x"])
    lp, _ = orc.router_logits(mo["wr"][perm], mo["x"])
    idx = orc.topk(l, 8)
    idxp = orc.topk(lp, 8)
    assert np.array_equal(perm[idxp], idx)


def test_router_logits_and_probs_against_numpy(orc):
    mo = synth.moe_layer(seed=0, n_tokens=16)
    l, s = orc.router_logits(mo["wr"], mo["x"])
    ref = mo["x"].astype(np.float64) @ mo["wr"].astype(np.float64).T
    assert np.all(np.abs(l - ref) <= 1e-13 * s)
    idx = orc.topk(l, 8)
    # rank order: non-increasing logits, and nothing outside beats the 8th
    for t in range(16):
        sel = l[t, idx[t]]
        assert np.all(np.diff(sel) <= 0)
        assert np.max(np.delete(l[t], idx[t])) <= sel[-1]
    p = orc.route_probs(l, idx)
    sel = np.take_along_axis(l, idx, axis=1)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    assert np.allclose(p, ex / ex.sum(axis=1, keepdims=True), rtol=1e-14, atol=0)
    assert np.allclose(p.sum(axis=1), 1.0, rtol=1e-15)


# --------------------------------------------------------------------------- #
# Routed MoE
def _small_moe(seed=0, t=3, e=6, h=256, f=256):
    g = np.random.default_rng(seed)
    wr = (0.05 * g.standard_normal((e, h))).astype(np.float32)
    wg = synth.q4_k_matrix(e * f, h, seed, 21).reshape(e, f, -1)
    wu = synth.q4_k_matrix(e * f, h, seed, 22).reshape(e, f, -1)
    wd = synth.q4_k_matrix(e * h, f, seed, 23).reshape(e, h, -1)
    x = synth.normal_f32((t, h), seed, 24)
    return wr, wg, wu, wd, x


def test_moe_routed_equals_dense_sum_bit_exact(orc):
    """Invariant: the routed layer equals the dense sum over all experts, in
    expert-index order, with the unselected experts' weights set to zero."""
    e, h, f, k = 6, 256, 256, 3
    wr, wg, wu, wd, x = _small_moe(e=e, h=h, f=f)
    l, _ = orc.router_logits(wr, x)
    idx = orc.topk(l, k)
    p = orc.route_probs(l, idx)
    y = orc.moe(Q4, wg, wu, wd, e, h, f, x, idx, p)
    for t in range(x.shape[0]):
        gate = np.zeros(e)
        gate[idx[t]] = p[t]
        dense = np.zeros(h)
        for ei in range(e):
            ye = orc.expert_ffn(Q4, wg, wu, wd, ei, h, f, x[t])["y"]
            dense = dense + gate[ei] * ye
        assert np.array_equal(dense, y[t])


def test_moe_all_experts_is_dense_softmax_mixture(orc):
    e, h, f = 4, 256, 256
    wr, wg, wu, wd, x = _small_moe(seed=1, e=e, h=h, f=f, t=2)
    l, _ = orc.router_logits(wr, x)
    idx = orc.topk(l, e)
    p = orc.route_probs(l, idx)
    y = orc.moe(Q4, wg, wu, wd, e, h, f, x, idx, p)
    for t in range(2):
        soft = np.exp(l[t] - l[t].max())
        soft /= soft.sum()
        ref = sum(soft[ei] * orc.expert_ffn(Q4, wg, wu, wd, ei, h, f, x[t])["y"] for ei in range(e))
        assert np.allclose(y[t], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_moe_expert_ffn_against_numpy(orc):
    """One expert's feed-forward from numpy matmuls of the exact weights."""
    e, h, f = 3, 512, 256
    _, wg, wu, wd, x = _small_moe(seed=2, e=e, h=h, f=f, t=1)
    for ei in range(e):
        out = orc.expert_ffn(Q4, wg, wu, wd, ei, h, f, x[0])
        G = orc.dequant(Q4, wg[ei], f, h).astype(np.float64)
        U = orc.dequant(Q4, wu[ei], f, h).astype(np.float64)
        D = orc.dequant(Q4, wd[ei], h, f).astype(np.float64)
        g = G @ x[0].astype(np.float64)
        u = U @ x[0].astype(np.float64)
        hh = g / (1.0 + np.exp(-g)) * u
        yy = D @ hh
        assert np.allclose(out["g"], g, rtol=0, atol=1e-13 * out["sg"].max())
        assert np.allclose(out["h"], hh, rtol=1e-12, atol=1e-12 * np.abs(hh).max())
        assert np.allclose(out["y"], yy, rtol=0, atol=1e-12 * out["sy"].max())


def test_gated_ffn_silu_invariants(orc):
    """Dense gate/up pins that do not restate the formula: with x = e_0 and
    d = 1, row r of each matrix gives its q[0] exactly, so
      * g = 0 gives h = 0 exactly,
      * rows with gate values v and -v and u = 1 differ by exactly v
        (silu(v) - silu(-v) = v, since the logistic function has
        sigma(v) + sigma(-v) = 1),
      * u scales h linearly (u = 3 gives three times the u = 1 value)."""
    n, k = 8, 64
    v = np.array([0, 5, -5, 17, -17, 1, -1, 100], dtype=np.int64)
    qg = np.zeros((n, k), dtype=np.int64)
    qg[:, 0] = v
    qu = np.zeros((n, k), dtype=np.int64)
    qu[:, 0] = [1, 1, 1, 1, 1, 3, 1, 1]
    wg = _q8_blocks_with(n, k, 0x3C00, qg)
    wu = _q8_blocks_with(n, k, 0x3C00, qu)
    x = np.zeros((1, k), dtype=np.float32)
    x[0, 0] = 1.0
    out = orc.gated_ffn(Q8, wg, wu, n, k, x)
    assert np.array_equal(out["g"][0], v.astype(np.float64))
    h = out["h"][0]
    assert h[0] == 0.0
    assert abs((h[1] - h[2]) - 5.0) <= 1e-14 * 5
    assert abs((h[3] - h[4]) - 17.0) <= 1e-14 * 17
    assert abs(h[5] - 3.0 * (h[6] + 1.0)) <= 1e-14   # silu(1) = 1 + silu(-1)
    assert abs(h[7] - 100.0) < 1e-40 + 100.0 * np.exp(-99.0)


def test_gated_ffn_equals_expert_ffn_first_half(orc):
    """The dense gate/up is the routed expert's first half for one expert."""
    _, wg, wu, wd, x = _small_moe(seed=3, e=2, h=512, f=256, t=2)
    for t in range(2):
        out = orc.gated_ffn(Q4, wg[1], wu[1], 256, 512, x[t])
        ref = orc.expert_ffn(Q4, wg, wu, wd, 1, 512, 256, x[t])
        for name in ("g", "u", "sg", "su", "h"):
            assert np.array_equal(out[name][0], ref[name])


def test_moe_reads_only_the_selected_experts(orc):
    """Poisoning every unselected expert's bytes (NaN scales) leaves y unchanged."""
    e, h, f, k = 6, 256, 256, 2
    wr, wg, wu, wd, x = _small_moe(seed=3, e=e, h=h, f=f, t=1)
    l, _ = orc.router_logits(wr, x)
    idx = orc.topk(l, k)
    p = orc.route_probs(l, idx)
    y = orc.moe(Q4, wg, wu, wd, e, h, f, x, idx, p)
    wg2, wu2, wd2 = wg.copy(), wu.copy(), wd.copy()
    for ei in set(range(e)) - set(idx[0].tolist()):
        for arr in (wg2, wu2, wd2):
            blk = arr[ei].reshape(-1, 144)
            blk[:, 0:2] = [0xFF, 0x7F]       # fp16 NaN scale
    y2 = orc.moe(Q4, wg2, wu2, wd2, e, h, f, x, idx, p)
    assert np.array_equal(y, y2)


# --------------------------------------------------------------------------- #
# GEMM
def test_gemm_single_row_equals_gemv(orc):
    n, k = 80, 1024
    for fmt in (Q8, Q4):
        w = synth.quant_matrix(fmt, n, k, seed=4, tensor_id=30)
        a = synth.normal_f32((7, k), seed=4, tensor_id=31)
        c, s = orc.gemm(fmt, w, n, k, a)
        y, sy = orc.gemv(fmt, w, n, k, a)
        assert np.array_equal(c, y) and np.array_equal(s, sy)


def test_gemm_integer_case_exact(orc):
    """Q8_0 with d = 2^-3 and bf16-exact small-integer activations: every partial
    sum is a multiple of 2^-3 below 2^24 in magnitude, so the result is exact."""
    n, k, m = 24, 1024, 9
    g = np.random.default_rng(9)
    q = g.integers(-127, 128, size=(n, k))
    w = _q8_blocks_with(n, k, 0x3000, q)       # fp16 0x3000 = 2^-3
    a = g.integers(-16, 17, size=(m, k)).astype(np.float32)
    c, _ = orc.gemm(Q8, w, n, k, a)
    ref = (a.astype(np.int64) @ q.T.astype(np.int64)).astype(np.float64) / 8.0
    assert np.array_equal(c, ref)


def test_gemm_sampled_columns_match_full(orc):
    n, k, m = 64, 512, 12
    w = synth.q4_k_matrix(n, k, seed=5, tensor_id=32)
    a = synth.normal_f32((m, k), seed=5, tensor_id=33)
    c, s = orc.gemm(Q4, w, n, k, a)
    cols = [0, 5, 63, 17]
    cc, ss = orc.gemm_columns(Q4, w, n, k, a, cols)
    assert np.array_equal(cc, c[:, cols]) and np.array_equal(ss, s[:, cols])
    cr, _ = orc.gemm(Q4, w, n, k, a, rows=(3, 8))
    assert np.array_equal(cr[3:8], c[3:8]) and np.isnan(cr[:3]).all()
