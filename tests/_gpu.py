"""Helpers for the GPU parity tests: device transfer and tolerance checks."""
import sys

import numpy as np
import torch

GEMV_TOL = 1e-5   # |y - y_ref| <= 1e-5 * sum |w x|   (fp32 decode GEMV)
GEMM_TOL = 8e-3   # |c - c_ref| <= 8e-3 * sum |a w|   (bf16-operand prompt GEMM)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def check_bound(got: np.ndarray, ref: np.ndarray, bound: np.ndarray, what: str) -> float:
    """Every element within its bound; zero bound demands an exact zero.  Returns
    the worst |err| / bound (0 when all bounds are zero)."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    zero = bound == 0
    assert np.all(err[zero] == 0), f"{what}: nonzero where the exact value is 0"
    ratio = np.zeros_like(err)
    ratio[~zero] = err[~zero] / bound[~zero]
    worst = float(ratio.max()) if ratio.size else 0.0
    nbad = int((ratio > 1).sum())
    assert nbad == 0, f"{what}: {nbad} of {ratio.size} outside the bound (worst {worst:.3g}x)"
    return worst


def check_rel(got, ref, s, tol, what) -> float:
    return check_bound(got, ref, tol * np.asarray(s, dtype=np.float64), what)


def moe_bound(fmt, mo, idx, probs, h, f, tol, tokens=None):
    """Per-element bound on the routed expert layer when each of its three
    products is within tol * sum|a w| of the exact product of its (rounded)
    input: g and u errors dg, du propagate through h = silu(g) * u (|silu'| <=
    1.1) as dh = 1.1|u|dg + |silu(g)|du + 1.1 dg du; the down product then adds
    sum|wd|dh and tol * sum|wd|(|h| + dh); the fp32 activation and the combine
    add 1e-6 of sum|wd h|.  Rows of `tokens` (default: all), in that order."""
    import oracle

    tokens = range(idx.shape[0]) if tokens is None else tokens
    bound = np.zeros((len(tokens), h))
    for i, ti in enumerate(tokens):
        for s in range(idx.shape[1]):
            ex = int(idx[ti, s])
            if not 0 <= ex < mo["wg"].shape[0]:
                continue
            o = oracle.expert_ffn(fmt, mo["wg"], mo["wu"], mo["wd"], ex, h, f, mo["x"][ti])
            sig = 1.0 / (1.0 + np.exp(-o["g"]))
            dg = tol * o["sg"]
            du = tol * o["su"]
            dh = (1.1 * np.abs(o["u"]) * dg + np.abs(o["g"] * sig) * du + 1.1 * dg * du
                  + 1e-6 * np.abs(o["h"]))
            wabs, _ = oracle.matvec_f64(fmt, mo["wd"][ex], h, f, dh, absw=True)
            bound[i] += float(probs[ti, s]) * (tol * o["sy"] + (1 + tol) * wabs + 1e-6 * o["sy"])
    return bound
