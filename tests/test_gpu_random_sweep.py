"""GPU parity on seeded random shapes: decode GEMVs (one matrix on every
workspace path, and grouped launches), prompt GEMMs, and MoE layers.

Complements the fixed parametrisations with shapes nobody picked by hand
(also the fused gate/up + SiLU and the prompt-batch MoE):
row counts from 1 to tens of thousands, K from one block to ~12k weights,
batches 1..16, ragged everything.  The GEMV and GEMM checks compare against
the CPU oracle with the per-product bounds of the fixed tests (README
"Inference": decode products; "Command-Line Tools": pp<N> prompt products);
the MoE layers must equal moe_route followed by moe_expert_gemv bit for bit
and leave the control block zero (the two-call path is pinned to the oracle
in test_gpu_moe.py).  Each case prints its parameters before it runs.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import GEMM_TOL, GEMV_TOL, check_bound, check_rel, dev, host, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

Q8, Q4 = synth.FMT_Q8_0, synth.FMT_Q4_K


@pytest.fixture(scope="module")
def g():
    import quantized_gguf_q8_amd as g
    return g


def test_random_gemv_every_path(g):
    rng = np.random.default_rng(2026)
    for case in range(160):
        fmt = Q4 if rng.random() < 0.5 else Q8
        kq = 256 if fmt == Q4 or rng.random() < 0.8 else 32
        k = int(kq * rng.integers(1, 48 if kq == 256 else 200))
        n = int(rng.choice([rng.integers(1, 64), rng.integers(64, 2000), rng.integers(2000, 14000)]))
        b = int(rng.integers(1, 17))
        n = max(1, min(n, int(3e7 // k)))   # keeps the oracle's share to seconds
        mode = ("none", "auto", "split")[case % 3]
        if mode == "none":
            ws = None
        elif mode == "auto":
            ws = "auto"
        else:
            need = max(g.quant_gemv_split_workspace_size(fmt, n, k, b), g.CTRL_BYTES)
            ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        say(f"gemv case {case} fmt={fmt} n={n} k={k} b={b} ws={mode}")
        w = synth.quant_matrix(fmt, n, k, seed=case, tensor_id=case)
        x = synth.normal_f32((b, k), seed=case, tensor_id=case + 1)
        y = host(g.quant_gemv(fmt, dev(w), n, k, dev(x), ws=ws))
        yr, s = oracle.gemv(fmt, w, n, k, x)
        check_rel(y, yr, s, GEMV_TOL, f"gemv case {case}")


def test_random_grouped_gemv(g):
    rng = np.random.default_rng(2027)
    for case in range(40):
        fmt = Q4 if rng.random() < 0.5 else Q8
        b = int(rng.integers(1, 17))
        items, refs = [], []
        for i in range(int(rng.integers(1, 7))):
            k = int(256 * rng.integers(1, 24))
            n = int(rng.integers(1, 4000))
            w = synth.quant_matrix(fmt, n, k, seed=1000 + case, tensor_id=i)
            x = synth.normal_f32((b, k), seed=1000 + case, tensor_id=100 + i)
            items.append((dev(w), n, k, dev(x), torch.empty((b, n), device="cuda")))
            refs.append(oracle.gemv(fmt, w, n, k, x))
        say(f"grouped case {case} fmt={fmt} b={b} shapes={[(it[1], it[2]) for it in items]}")
        g.quant_gemv_grouped(fmt, items, ws="auto" if case % 2 else None)
        for it, (yr, s) in zip(items, refs):
            check_rel(host(it[4]), yr, s, GEMV_TOL, f"grouped case {case}")


def test_random_gemm(g):
    rng = np.random.default_rng(77)
    for case in range(40):
        fmt = Q4 if rng.random() < 0.5 else Q8
        k = int(256 * rng.integers(1, 40)) if fmt == Q4 else int(32 * rng.integers(1, 300))
        m = int(rng.choice([rng.integers(17, 129), rng.integers(129, 1100)]))
        n = int(rng.integers(1, 6000))
        n = max(1, min(n, int(3e8 // (m * k))))
        say(f"gemm case {case} fmt={fmt} m={m} n={n} k={k}")
        w = synth.quant_matrix(fmt, n, k, seed=case, tensor_id=case)
        a = synth.normal_f32((m, k), seed=case, tensor_id=case + 1)
        c = host(g.quant_gemm(fmt, dev(w), n, k, dev(a)))
        cr, s = oracle.gemm(fmt, w, n, k, a)
        check_rel(c, cr, s, GEMM_TOL, f"gemm case {case}")


def test_random_moe_layer(g):
    import test_gpu_moe_layer as ml
    rng = np.random.default_rng(78)
    for case in range(30):
        fmt = Q4 if rng.random() < 0.6 else Q8
        e = int(rng.choice([8, 16, 40, 64, 128, 200, 256]))
        top = int(rng.integers(1, min(e, 9) + 1))
        h = int(256 * rng.integers(1, 9))
        f = int(256 * rng.integers(1, 9))
        t = int(rng.choice([1, 1, 2, 3, 5, 8, 13, 16, 24, 31, 32, 40]))
        say(f"moe case {case} fmt={fmt} e={e} top_k={top} h={h} f={f} t={t}")
        mo = ml._layer(case, fmt, e, h, f, t)
        d = {nm: dev(v) for nm, v in mo.items()}
        ref = ml._two_calls(g, fmt, d, e, h, f, top)
        ws = torch.zeros(g.moe_layer_workspace_size(e, t, top, h, f), dtype=torch.uint8,
                         device="cuda")
        for rep in range(2):
            got = g.moe_layer_gemv(fmt, d["wr"], d["wg"], d["wu"], d["wd"], e, h, f, d["x"],
                                   top, ws=ws)
            ml._same([host(v) for v in got], ref, f"moe case {case} call {rep}")
            assert int(ws[:g.CTRL_BYTES].count_nonzero()) == 0, "control block not returned to zero"


def test_random_swiglu(g):
    from test_gpu_gemv import _swiglu_bound
    rng = np.random.default_rng(79)
    for case in range(24):
        fmt = Q4 if rng.random() < 0.5 else Q8
        k = int(256 * rng.integers(1, 24))
        n = int(rng.integers(1, 7000))
        n = max(1, min(n, int(2e7 // k)))
        b = int(rng.integers(1, 17))
        say(f"swiglu case {case} fmt={fmt} n={n} k={k} b={b}")
        wg = synth.quant_matrix(fmt, n, k, seed=case, tensor_id=3 * case)
        wu = synth.quant_matrix(fmt, n, k, seed=case, tensor_id=3 * case + 1)
        x = synth.normal_f32((b, k), seed=case, tensor_id=3 * case + 2)
        h = host(g.quant_gemv_swiglu(fmt, dev(wg), dev(wu), n, k, dev(x)))
        o = oracle.gated_ffn(fmt, wg, wu, n, k, x)
        check_bound(h, o["h"], _swiglu_bound(o), f"swiglu case {case}")


def test_random_moe_prompt_batch(g):
    import test_gpu_moe_gemm as mg
    rng = np.random.default_rng(80)
    for case in range(16):
        fmt = Q4 if rng.random() < 0.6 else Q8
        e = int(rng.choice([8, 16, 32, 64, 128]))
        top = int(rng.integers(1, min(e, 9) + 1))
        h = int(256 * rng.integers(1, 5))
        f = int(256 * rng.integers(1, 5))
        t = int(rng.integers(17, 301))
        say(f"moe prompt case {case} fmt={fmt} e={e} top_k={top} h={h} f={f} t={t}")
        mo = mg._small(100 + case, fmt, e, h, f, t)
        lref, _ = oracle.router_logits(mo["wr"], mo["x"])
        idx = oracle.topk(lref, top)
        probs = oracle.route_probs(lref, idx).astype(np.float32)
        y = mg._run(g, fmt, mo, idx, probs, e, h, f)
        tokens = np.sort(rng.choice(t, size=min(t, 24), replace=False))
        mg._check_tokens(fmt, mo, idx, probs, h, f, y, tokens, f"moe prompt case {case}")
