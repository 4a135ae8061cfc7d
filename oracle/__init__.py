"""CPU oracle for the fused dequantize-and-multiply path (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  The product library never does, and the oracle
never imports the product library: the two share no code.  The arithmetic lives
in plain C (``ggq_oracle.c``, fp64 accumulation); this module only marshals numpy
arrays into it and splits independent rows across threads (ctypes releases the
GIL during the call, each thread runs the same single-threaded C loop on its own
rows, so results do not depend on the thread count).

Which passage each function follows is stated at the function in the C file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ggq_oracle.c")
_LIB = os.path.join(_HERE, "libggq_oracle.so")

Q8_0 = 8
Q4_K = 12

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no HIP, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        L.ggo_half_to_float.restype = ctypes.c_float
        L.ggo_half_to_float.argtypes = [ctypes.c_uint16]
        L.ggo_q4_k_scale_min.restype = None
        L.ggo_q4_k_scale_min.argtypes = [P, I, P, P]
        L.ggo_dequant.restype = I
        L.ggo_dequant.argtypes = [I, P, I64, I64, I64, I64, P]
        L.ggo_gemv.restype = I
        L.ggo_gemv.argtypes = [I, P, I64, I64, P, I64, I64, I64, I64, P, P, I64]
        L.ggo_matvec_f64.restype = I
        L.ggo_matvec_f64.argtypes = [I, P, I64, I64, P, I, P, P]
        L.ggo_router_logits.restype = None
        L.ggo_router_logits.argtypes = [P, I64, I64, P, I64, P, P]
        L.ggo_topk_f64.restype = None
        L.ggo_topk_f64.argtypes = [P, I64, I64, I, P]
        L.ggo_topk_f32.restype = None
        L.ggo_topk_f32.argtypes = [P, I64, I64, I, P]
        L.ggo_route_probs.restype = None
        L.ggo_route_probs.argtypes = [P, I64, I64, P, I, P]
        L.ggo_expert_ffn.restype = I
        L.ggo_expert_ffn.argtypes = [I, P, P, P, I64, I64, I64, P, P, P, P, P, P, P, P]
        L.ggo_gated_ffn.restype = I
        L.ggo_gated_ffn.argtypes = [I, P, P, I64, I64, P, P, P, P, P, P]
        L.ggo_moe.restype = I
        L.ggo_moe.argtypes = [I, P, P, P, I64, I64, I64, P, I64, I64, P, P, I, P, P]
        L.ggo_gemm.restype = I
        L.ggo_gemm.argtypes = [I, P, I64, I64, P, I64, I64, I64, I64, I64, P, P, I64]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _split(n: int, parts: int):
    parts = max(1, min(parts, n)) if n > 0 else 1
    step = (n + parts - 1) // parts
    return [(i, min(n, i + step)) for i in range(0, n, step)] or [(0, 0)]


def _check(rc):
    if rc != 0:
        raise ValueError(f"oracle call failed (rc={rc})")


# --------------------------------------------------------------------------- #
def half_to_float(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16).ravel()
    f = lib().ggo_half_to_float
    return np.array([f(int(b)) for b in bits], dtype=np.float32)


def q4_k_scale_min(s12: bytes | np.ndarray):
    s = _c(np.frombuffer(bytes(s12), dtype=np.uint8) if isinstance(s12, (bytes, bytearray)) else s12, np.uint8)
    assert s.size == 12
    sc, m = ctypes.c_int(), ctypes.c_int()
    out_sc, out_m = [], []
    for j in range(8):
        lib().ggo_q4_k_scale_min(_p(s), j, ctypes.byref(sc), ctypes.byref(m))
        out_sc.append(sc.value)
        out_m.append(m.value)
    return out_sc, out_m


def dequant(fmt: int, w: np.ndarray, n: int, k: int, threads: int | None = None) -> np.ndarray:
    """Exact fp32 weights [n][k] of a quantized matrix."""
    w = _c(w, np.uint8)
    out = np.empty((n, k), dtype=np.float32)

    def run(rr):
        r0, r1 = rr
        _check(lib().ggo_dequant(fmt, _p(w), n, k, r0, r1, _p(out[r0:r1])))

    with ThreadPoolExecutor(threads or default_threads()) as ex:
        list(ex.map(run, _split(n, threads or default_threads())))
    return out


def gemv(fmt: int, w: np.ndarray, n: int, k: int, x: np.ndarray, threads: int | None = None,
         rows: tuple[int, int] | None = None):
    """y[b][r] (fp64) and s[b][r] = sum |w x| for x [B][k] (fp32), rows [r0, r1)."""
    w = _c(w, np.uint8)
    x = _c(np.atleast_2d(x), np.float32)
    nb = x.shape[0]
    r0, r1 = rows if rows is not None else (0, n)
    y = np.zeros((nb, n), dtype=np.float64)
    s = np.zeros((nb, n), dtype=np.float64)

    def run(rr):
        a, b = rr
        _check(lib().ggo_gemv(fmt, _p(w), n, k, _p(x), k, nb, a, b, _p(y), _p(s), n))

    th = threads or default_threads()
    with ThreadPoolExecutor(th) as ex:
        list(ex.map(run, [(r0 + a, r0 + b) for a, b in _split(r1 - r0, th)]))
    return y, s


def matvec_f64(fmt: int, w: np.ndarray, n: int, k: int, v: np.ndarray, absw: bool = False):
    w = _c(w, np.uint8)
    v = _c(v, np.float64)
    y = np.empty(n, dtype=np.float64)
    s = np.empty(n, dtype=np.float64)
    _check(lib().ggo_matvec_f64(fmt, _p(w), n, k, _p(v), int(absw), _p(y), _p(s)))
    return y, s


def router_logits(wr: np.ndarray, x: np.ndarray):
    wr = _c(wr, np.float32)
    x = _c(np.atleast_2d(x), np.float32)
    e, h = wr.shape
    t = x.shape[0]
    l = np.empty((t, e), dtype=np.float64)
    s = np.empty((t, e), dtype=np.float64)
    lib().ggo_router_logits(_p(wr), e, h, _p(x), t, _p(l), _p(s))
    return l, s


def topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Rank-ordered top-k indices; ties go to the lower index.  fp64 or fp32 input
    is compared in its own precision."""
    lg = np.atleast_2d(logits)
    t, e = lg.shape
    idx = np.empty((t, k), dtype=np.int32)
    if lg.dtype == np.float32:
        lg = _c(lg, np.float32)
        lib().ggo_topk_f32(_p(lg), t, e, k, _p(idx))
    else:
        lg = _c(lg, np.float64)
        lib().ggo_topk_f64(_p(lg), t, e, k, _p(idx))
    return idx


def route_probs(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    lg = _c(np.atleast_2d(logits), np.float64)
    idx = _c(np.atleast_2d(idx), np.int32)
    t, e = lg.shape
    k = idx.shape[1]
    p = np.empty((t, k), dtype=np.float64)
    lib().ggo_route_probs(_p(lg), t, e, _p(idx), k, _p(p))
    return p


def expert_ffn(fmt: int, wg, wu, wd, e: int, hdim: int, f: int, x: np.ndarray):
    """Dict of g, u, sg, su, h [f] and y, sy [hdim] for expert e on one token."""
    wg, wu, wd = (_c(a, np.uint8) for a in (wg, wu, wd))
    x = _c(x, np.float32).ravel()
    out = {n: np.empty(f) for n in ("g", "u", "sg", "su", "h")}
    out["y"] = np.empty(hdim)
    out["sy"] = np.empty(hdim)
    _check(lib().ggo_expert_ffn(fmt, _p(wg), _p(wu), _p(wd), e, hdim, f, _p(x),
                                _p(out["g"]), _p(out["u"]), _p(out["sg"]), _p(out["su"]),
                                _p(out["h"]), _p(out["y"]), _p(out["sy"])))
    return out


def gated_ffn(fmt: int, wg, wu, n: int, k: int, x: np.ndarray):
    """Dense gated feed-forward, gate and up: dict of g, u, sg, su, h, each
    [T][n] fp64, for the activation rows x [T][k]."""
    wg, wu = (_c(a, np.uint8) for a in (wg, wu))
    x = _c(np.atleast_2d(x), np.float32)
    out = {name: np.empty((x.shape[0], n)) for name in ("g", "u", "sg", "su", "h")}
    for t in range(x.shape[0]):
        row = {name: np.empty(n) for name in out}
        _check(lib().ggo_gated_ffn(fmt, _p(wg), _p(wu), n, k, _p(_c(x[t], np.float32)),
                                   _p(row["g"]), _p(row["u"]), _p(row["sg"]), _p(row["su"]),
                                   _p(row["h"])))
        for name in out:
            out[name][t] = row[name]
    return out


def moe(fmt: int, wg, wu, wd, e: int, hdim: int, f: int, x: np.ndarray, idx: np.ndarray,
        probs: np.ndarray, threads: int | None = None, want_h: bool = False):
    """Routed MoE output y [T][hdim] (fp64); optionally h [T][k][f]."""
    wg, wu, wd = (_c(a, np.uint8) for a in (wg, wu, wd))
    x = _c(np.atleast_2d(x), np.float32)
    idx = _c(np.atleast_2d(idx), np.int32)
    probs = _c(np.atleast_2d(probs), np.float64)
    t = x.shape[0]
    k = idx.shape[1]
    y = np.zeros((t, hdim), dtype=np.float64)
    h = np.zeros((t, k, f), dtype=np.float64) if want_h else None

    def run(tt):
        a, b = tt
        _check(lib().ggo_moe(fmt, _p(wg), _p(wu), _p(wd), e, hdim, f, _p(x), a, b,
                             _p(idx), _p(probs), k, _p(y), _p(h)))

    th = threads or default_threads()
    with ThreadPoolExecutor(th) as ex:
        list(ex.map(run, _split(t, th)))
    return (y, h) if want_h else y


def gemm(fmt: int, w: np.ndarray, n: int, k: int, a: np.ndarray, rows=None, cols=None,
         threads: int | None = None):
    """C = A W^T in fp64 with S = |A||W|^T, restricted to the given row range
    (m0, m1) and column range (n0, n1).  Returns full-size arrays (M x N) whose
    entries outside the ranges are NaN."""
    w = _c(w, np.uint8)
    a = _c(a, np.float32)
    m = a.shape[0]
    m0, m1 = rows if rows is not None else (0, m)
    n0, n1 = cols if cols is not None else (0, n)
    c = np.full((m, n), np.nan)
    s = np.full((m, n), np.nan)

    def run(nn):
        a0, a1 = nn
        _check(lib().ggo_gemm(fmt, _p(w), n, k, _p(a), k, m0, m1, a0, a1, _p(c), _p(s), n))

    th = threads or default_threads()
    with ThreadPoolExecutor(th) as ex:
        list(ex.map(run, [(n0 + x, n0 + y) for x, y in _split(n1 - n0, th)]))
    return c, s


def gemm_columns(fmt: int, w: np.ndarray, n: int, k: int, a: np.ndarray, cols, threads=None):
    """C and S for every row of A and the listed columns only: (M, len(cols))."""
    w = _c(w, np.uint8)
    a = _c(a, np.float32)
    m = a.shape[0]
    cols = [int(c) for c in cols]
    outc = np.empty((m, len(cols)))
    outs = np.empty((m, len(cols)))

    def run(j):
        col = cols[j]
        # ldc = 1: entry (mm, col) lands at index mm + col of the output buffer.
        cc = np.empty(m + col)
        ss = np.empty(m + col)
        _check(lib().ggo_gemm(fmt, _p(w), n, k, _p(a), k, 0, m, col, col + 1, _p(cc), _p(ss), 1))
        outc[:, j] = cc[col:col + m]
        outs[:, j] = ss[col:col + m]

    with ThreadPoolExecutor(threads or default_threads()) as ex:
        list(ex.map(run, range(len(cols))))
    return outc, outs
