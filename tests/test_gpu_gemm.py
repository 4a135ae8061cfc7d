"""GPU parity: quant_gemm (bf16 operands, fp32 accumulation on the matrix cores)
within 8e-3 * sum|a w| of the fp64 oracle.

phobos-bench pp<N> (README "Command-Line Tools") measures prompt batches; the
full pp512 shapes are checked on sampled rows and columns the way the README's
cluster_correctness example sample-checks a large product against the CPU, and
on every output by a slow test.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import GEMM_TOL, check_rel, dev, host, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

Q8, Q4 = synth.FMT_Q8_0, synth.FMT_Q4_K


@pytest.fixture(scope="module")
def g():
    import quantized_gguf_q8_amd as g
    return g


# The last three split K eight or four ways with step counts that leave the
# last splits short or empty (each split takes a multiple of 4 of the 64-wide
# steps: 68 steps -> 12 x 5 + 8 + 0 + 0; 132 -> 20 x 6 + 12 + 0; 36 -> 12 x 3 + 0).
@pytest.mark.parametrize("fmt,m,n,k", [
    (Q4, 37, 70, 512), (Q8, 130, 200, 1056), (Q8, 1, 64, 64), (Q4, 129, 257, 2560),
    (Q8, 512, 300, 2048), (Q4, 3, 17, 256),
    (Q4, 40, 96, 4352), (Q8, 24, 48, 8448), (Q4, 64, 64, 2304),
])
def test_gemm_parity_full_check(g, fmt, m, n, k):
    say(f"gemm fmt={fmt} m={m} n={n} k={k}")
    w = synth.quant_matrix(fmt, n, k, seed=0, tensor_id=m + n)
    a = synth.normal_f32((m, k), seed=0, tensor_id=m + n + 1)
    c = host(g.quant_gemm(fmt, dev(w), n, k, dev(a)))
    cr, s = oracle.gemm(fmt, w, n, k, a)
    worst = check_rel(c, cr, s, GEMM_TOL, "gemm")
    say(f"  worst err / bound = {worst:.3g}")


@pytest.mark.parametrize("name,fmt,n,k", synth.PP512_GEMMS)
def test_gemm_pp512_sampled(g, name, fmt, n, k):
    """Full-size pp512 products: 48 random rows x all columns and all rows x 192
    random columns, plus the corners."""
    say(f"gemm pp512 {name}")
    m = synth.PP512_M
    tid = synth.tid(4, n, k)
    w = synth.quant_matrix(fmt, n, k, seed=0, tensor_id=tid)
    a = synth.normal_f32((m, k), seed=0, tensor_id=tid + 1)
    c = host(g.quant_gemm(fmt, dev(w), n, k, dev(a)))
    rng = np.random.default_rng(0)
    rows = sorted(set(rng.choice(m, 46, replace=False).tolist()) | {0, m - 1})
    cr, s = oracle.gemm(fmt, w, n, k, a[rows])
    check_rel(c[rows], cr, s, GEMM_TOL, f"{name} rows")
    cols = sorted(set(rng.choice(n, 190, replace=False).tolist()) | {0, n - 1})
    cc, ss = oracle.gemm_columns(fmt, w, n, k, a, cols)
    worst = check_rel(c[:, cols], cc, ss, GEMM_TOL, f"{name} columns")
    say(f"  worst err / bound (columns) = {worst:.3g}")


@pytest.mark.slow
@pytest.mark.parametrize("name,fmt,n,k", synth.PP512_GEMMS)
def test_gemm_pp512_every_output(g, name, fmt, n, k):
    """Full-size pp512 products, every one of the 512 x N outputs against the
    oracle (about 45 G multiply-adds in fp64 per product: ~10 s on 16 threads)."""
    say(f"gemm pp512 every output {name}")
    m = synth.PP512_M
    tid = synth.tid(4, n, k)
    w = synth.quant_matrix(fmt, n, k, seed=0, tensor_id=tid)
    a = synth.normal_f32((m, k), seed=0, tensor_id=tid + 1)
    c = host(g.quant_gemm(fmt, dev(w), n, k, dev(a)))
    cr, s = oracle.gemm(fmt, w, n, k, a)
    assert not np.isnan(cr).any()
    worst = check_rel(c, cr, s, GEMM_TOL, f"{name} all outputs")
    say(f"  worst err / bound = {worst:.3g}")


# 17..128 rows run as the grouped-expert tile over 64-row column tiles (when
# those cover the device): one and two row tiles, ragged last row group and
# ragged last column tile, both formats.
@pytest.mark.parametrize("fmt,m,n,k", [
    (Q4, 17, 12304, 512), (Q8, 64, 12300, 256), (Q4, 65, 6200, 1024), (Q8, 128, 6144, 768),
    (Q4, 100, 6150, 256), (Q8, 33, 12290, 512),
])
def test_gemm_mid_rows_full_check(g, fmt, m, n, k):
    say(f"gemm mid rows fmt={fmt} m={m} n={n} k={k}")
    w = synth.quant_matrix(fmt, n, k, seed=2, tensor_id=m + n)
    a = synth.normal_f32((m, k), seed=2, tensor_id=m + n + 1)
    c = host(g.quant_gemm(fmt, dev(w), n, k, dev(a)))
    cr, s = oracle.gemm(fmt, w, n, k, a)
    worst = check_rel(c, cr, s, GEMM_TOL, "gemm mid rows")
    say(f"  worst err / bound = {worst:.3g}")


@pytest.mark.parametrize("m", [17, 128, 2048])
def test_gemm_prompt_sweep_sampled(g, m):
    """Prompt lengths around pp512 (the GEMV / GEMM crossover just past the
    GEMV's 16 rows, pp128, pp2048) on the Q4_K up projection: sampled rows x
    all columns and all rows x sampled columns."""
    name, fmt, n, k = synth.PP512_GEMMS[0]
    say(f"gemm sweep {name} m={m}")
    tid = synth.tid(4, n, k)
    w = synth.quant_matrix(fmt, n, k, seed=0, tensor_id=tid)
    a = synth.normal_f32((m, k), seed=1, tensor_id=tid + m)
    c = host(g.quant_gemm(fmt, dev(w), n, k, dev(a)))
    rng = np.random.default_rng(m)
    rows = sorted(set(rng.choice(m, min(m, 14), replace=False).tolist()) | {0, m - 1})
    cr, s = oracle.gemm(fmt, w, n, k, a[rows])
    check_rel(c[rows], cr, s, GEMM_TOL, f"m={m} rows")
    cols = sorted(set(rng.choice(n, 62, replace=False).tolist()) | {0, n - 1})
    cc, ss = oracle.gemm_columns(fmt, w, n, k, a, cols)
    worst = check_rel(c[:, cols], cc, ss, GEMM_TOL, f"m={m} columns")
    say(f"  worst err / bound (columns) = {worst:.3g}")


def test_gemm_single_row_matches_gemv_tolerance(g):
    say("gemm M=1 vs oracle gemv")
    for fmt, n, k in ((Q8, 256, 2048), (Q4, 256, 2560)):
        w = synth.quant_matrix(fmt, n, k, seed=2, tensor_id=90)
        a = synth.normal_f32((1, k), seed=2, tensor_id=91)
        c = host(g.quant_gemm(fmt, dev(w), n, k, dev(a)))
        yr, s = oracle.gemv(fmt, w, n, k, a)
        check_rel(c, yr, s, GEMM_TOL, "M=1")


def test_gemm_exact_integer_case(g):
    """bf16-exact operands (Q8_0 d = 2^-3, small-integer activations): every
    product and partial sum is exact in fp32, so the result is exact."""
    say("gemm exact")
    n, k, m = 96, 2048, 40
    rng = np.random.default_rng(9)
    q = rng.integers(-127, 128, size=(n, k))
    raw = np.zeros((n * k // 32, 34), dtype=np.uint8)
    raw[:, 0:2] = [0x00, 0x30]
    raw[:, 2:] = q.reshape(-1, 32).astype(np.int8).view(np.uint8)
    a = rng.integers(-16, 17, size=(m, k)).astype(np.float32)
    c = host(g.quant_gemm(Q8, dev(raw.reshape(n, -1)), n, k, dev(a)))
    ref = ((a.astype(np.int64) @ q.T) / 8.0).astype(np.float32)
    assert np.array_equal(c, ref)


def test_gemm_deterministic(g):
    say("gemm determinism")
    fmt, m, n, k = Q4, 256, 1024, 2560
    w = dev(synth.quant_matrix(fmt, n, k, seed=5, tensor_id=92))
    a = dev(synth.normal_f32((m, k), seed=5, tensor_id=93))
    c1 = host(g.quant_gemm(fmt, w, n, k, a))
    c2 = host(g.quant_gemm(fmt, w, n, k, a))
    assert np.array_equal(c1, c2)
