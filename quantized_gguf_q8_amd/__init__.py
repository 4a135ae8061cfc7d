"""Python binding of libggq (include/ggq.h): products over GGUF block-quantized
weights on MI355X.

This module only marshals arguments: it checks dtypes, devices and shapes of torch
tensors, passes their device pointers and the current HIP stream to the C ABI, and
turns status codes into exceptions.  Every step of the computation runs in the
library's HIP kernels.  If libggq.so has not been built the import fails loudly;
there is no CPU fallback.

Formats (GGUF tensor-type ids): Q8_0 = 8 (34-byte blocks of 32 weights) and
Q4_K = 12 (144-byte super-blocks of 256 weights).  A quantized N x K matrix is a
uint8 tensor of shape [N, row_bytes(fmt, K)] (or any contiguous tensor with that
many bytes).
"""
from __future__ import annotations

import ctypes
import os

import torch

Q8_0 = 8
Q4_K = 12
GEMM_BF16 = 0
# Bytes at the start of every quant_gemv / quant_gemm workspace that must be zero
# before its first use (every call leaves them zero).
CTRL_BYTES = 4096

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libggq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -c 'import __graft_entry__ as g; g.build()')")

# torch is imported first so that its HIP runtime is the one libggq binds to.
_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGS = {
    "ggq_status_string": (ctypes.c_char_p, [_I]),
    "ggq_version": (_I, []),
    "quant_dequantize": (_I, [_I, _P, _I64, _I64, _P, _P]),
    "quant_gemv": (_I, [_I, _P, _I64, _I64, _P, _I64, _P, _I64, _I, _P, _SZ, _P]),
    "quant_gemv_noalloc": (_I, [_I, _P, _I64, _I64, _P, _I64, _P, _I64, _I, _P]),
    "quant_gemv_workspace_size": (_SZ, [_I, _I64, _I]),
    "quant_gemv_split_workspace_size": (_SZ, [_I, _I64, _I64, _I]),
    "quant_gemv_grouped": (_I, [_I, _P, _I, _I, _P, _SZ, _P]),
    "quant_gemv_swiglu": (_I, [_I, _P, _P, _I64, _I64, _P, _I64, _P, _I64, _I, _P, _SZ, _P]),
    "quant_gemm_workspace_size": (_SZ, [_I, _I64, _I64, _I64, _I]),
    "quant_gemm": (_I, [_I, _P, _I64, _I64, _P, _I64, _I64, _P, _I64, _I, _P, _SZ, _P]),
    "moe_route": (_I, [_P, _I64, _I64, _P, _I64, _I, _P, _P, _P, _P]),
    "moe_workspace_size": (_SZ, [_I64, _I64, _I, _I64, _I64]),
    "moe_workspace_h_offset": (_SZ, [_I64, _I64, _I]),
    "moe_expert_gemv": (_I, [_I, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P, _P, _I, _P, _P,
                             _SZ, _P]),
    "moe_layer_workspace_size": (_SZ, [_I64, _I64, _I, _I64, _I64]),
    "moe_layer_gemv": (_I, [_I, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _I, _P, _P, _P, _P,
                            _P, _SZ, _P]),
    "moe_gemm_workspace_size": (_SZ, [_I64, _I64, _I, _I64, _I64]),
    "moe_expert_gemm": (_I, [_I, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P, _P, _I, _P, _P,
                             _SZ, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class GGQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {_lib.ggq_status_string(status).decode()} (status {status})")


def _ck(fn: str, status: int):
    if status != 0:
        raise GGQError(fn, status)


def block_weights(fmt: int) -> int:
    if fmt == Q8_0:
        return 32
    if fmt == Q4_K:
        return 256
    raise ValueError(f"unknown format {fmt}")


def row_bytes(fmt: int, k: int) -> int:
    return k // 32 * 34 if fmt == Q8_0 else k // 256 * 144


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype | None = None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _wbytes(w: torch.Tensor, fmt: int, n: int, k: int, name: str = "w"):
    _dev(w, name, torch.uint8)
    need = n * row_bytes(fmt, k)
    if w.numel() < need:
        raise ValueError(f"{name} holds {w.numel()} bytes, {need} needed")


def version() -> int:
    return _lib.ggq_version()


def quant_dequantize(fmt: int, w: torch.Tensor, n: int, k: int,
                     out: torch.Tensor | None = None) -> torch.Tensor:
    _wbytes(w, fmt, n, k)
    if out is None:
        out = torch.empty((n, k), dtype=torch.float32, device=w.device)
    _dev(out, "out", torch.float32)
    _ck("quant_dequantize", _lib.quant_dequantize(fmt, _ptr(w), n, k, _ptr(out), _stream()))
    return out


def quant_gemv_workspace_size(fmt: int, k: int, batch: int) -> int:
    return _lib.quant_gemv_workspace_size(fmt, k, batch)


def quant_gemv_split_workspace_size(fmt: int, n: int, k: int, batch: int) -> int:
    return _lib.quant_gemv_split_workspace_size(fmt, n, k, batch)


def _ws_arg(ws, need, device):
    """None -> no workspace (vector-unit path); "auto" -> allocate `need` bytes,
    zeroed (the workspace's control block must start at zero); else a uint8
    tensor whose first CTRL_BYTES are zero before its first use."""
    if ws is None:
        return None
    if isinstance(ws, str):
        if ws != "auto":
            raise ValueError("ws must be None, 'auto' or a uint8 device tensor")
        return torch.zeros(max(need, 256), dtype=torch.uint8, device=device)
    _dev(ws, "ws", torch.uint8)
    return ws


def quant_gemv(fmt: int, w: torch.Tensor, n: int, k: int, x: torch.Tensor,
               y: torch.Tensor | None = None, ws=None) -> torch.Tensor:
    """y[b][r] = sum_c w[r][c] x[b][c]; x is [B, K] (B <= 16) or [K].

    ws=None runs the fp32 vector-unit kernel; a workspace (a uint8 tensor of at
    least quant_gemv_workspace_size bytes) lets batch >= 2 use the matrix cores;
    "auto" allocates quant_gemv_split_workspace_size bytes, which also allows K
    to be cut across workgroups."""
    _wbytes(w, fmt, n, k)
    squeeze = x.dim() == 1
    x2 = x.unsqueeze(0) if squeeze else x
    _dev(x2, "x", torch.float32)
    if x2.shape[1] != k:
        raise ValueError(f"x has {x2.shape[1]} columns, K = {k}")
    b = x2.shape[0]
    if y is None:
        y = torch.empty((b, n), dtype=torch.float32, device=w.device)
    _dev(y, "y", torch.float32)
    wst = _ws_arg(ws, quant_gemv_split_workspace_size(fmt, n, k, b), w.device)
    _ck("quant_gemv", _lib.quant_gemv(fmt, _ptr(w), n, k, _ptr(x2), k, _ptr(y), n, b, _ptr(wst),
                                      0 if wst is None else wst.numel(), _stream()))
    return y[0] if squeeze else y


def quant_gemv_noalloc(fmt: int, w: torch.Tensor, n: int, k: int, x: torch.Tensor,
                       y: torch.Tensor) -> torch.Tensor:
    """quant_gemv with the library's fixed device scratch as its workspace: no
    device allocation in the call (y must be given).  Calls on one GPU share
    the scratch; overlapping calls race."""
    _wbytes(w, fmt, n, k)
    squeeze = x.dim() == 1
    x2 = x.unsqueeze(0) if squeeze else x
    _dev(x2, "x", torch.float32)
    if x2.shape[1] != k:
        raise ValueError(f"x has {x2.shape[1]} columns, K = {k}")
    b = x2.shape[0]
    _dev(y, "y", torch.float32)
    if y.numel() < b * n:
        raise ValueError(f"y holds {y.numel()} floats, {b * n} needed")
    _ck("quant_gemv_noalloc", _lib.quant_gemv_noalloc(fmt, _ptr(w), n, k, _ptr(x2), k, _ptr(y),
                                                      n, b, _stream()))
    return y


def quant_gemv_swiglu(fmt: int, wg: torch.Tensor, wu: torch.Tensor, n: int, k: int,
                      x: torch.Tensor, h: torch.Tensor | None = None, ws="auto") -> torch.Tensor:
    """h[b][r] = silu((Wg x)[b][r]) * (Wu x)[b][r] in one pass; x is [B, K] or [K].
    ws: "auto", None (batch 1 only) or a uint8 tensor of quant_gemv_workspace_size."""
    _wbytes(wg, fmt, n, k)
    _wbytes(wu, fmt, n, k)
    squeeze = x.dim() == 1
    x2 = x.unsqueeze(0) if squeeze else x
    _dev(x2, "x", torch.float32)
    if x2.shape[1] != k:
        raise ValueError(f"x has {x2.shape[1]} columns, K = {k}")
    b = x2.shape[0]
    if h is None:
        h = torch.empty((b, n), dtype=torch.float32, device=wg.device)
    _dev(h, "h", torch.float32)
    wst = _ws_arg(ws, quant_gemv_workspace_size(fmt, k, b), wg.device)
    _ck("quant_gemv_swiglu", _lib.quant_gemv_swiglu(fmt, _ptr(wg), _ptr(wu), n, k, _ptr(x2), k,
                                                    _ptr(h), n, b, _ptr(wst),
                                                    0 if wst is None else wst.numel(), _stream()))
    return h[0] if squeeze else h


class GemvDesc(ctypes.Structure):
    """Mirror of ggq_gemv_desc."""
    _fields_ = [("w", _P), ("n", _I64), ("k", _I64), ("x", _P), ("ldx", _I64), ("y", _P),
                ("ldy", _I64)]


MAX_GROUP = 16


class GemvGroup:
    """A grouped call whose arguments are validated and marshalled once; calling
    the object launches it on the current stream.  For decode loops that issue
    the same products every token (and for graph capture).  items: (w, n, k, x, y)
    with x [B, K] and y [B, N]; ws as for quant_gemv."""

    def __init__(self, fmt: int, items, ws=None):
        items = list(items)
        if not 1 <= len(items) <= MAX_GROUP:
            raise ValueError(f"1..{MAX_GROUP} matrices per grouped call")
        self.fmt = fmt
        self._keep = items
        self._arr = (GemvDesc * len(items))()
        self.batch = None
        for i, (w, n, k, x, y) in enumerate(items):
            _wbytes(w, fmt, n, k)
            _dev(x, "x", torch.float32)
            _dev(y, "y", torch.float32)
            if x.dim() != 2 or y.dim() != 2 or x.shape[1] != k or y.shape[1] != n:
                raise ValueError("x must be [B, K] and y [B, N]")
            if self.batch is None:
                self.batch = x.shape[0]
            elif self.batch != x.shape[0] or y.shape[0] != x.shape[0]:
                raise ValueError("every matrix of a group must have the same batch")
            self._arr[i] = GemvDesc(_ptr(w), n, k, _ptr(x), k, _ptr(y), n)
        self._ptr = ctypes.cast(self._arr, _P)
        self.count = len(items)
        self.weight_bytes = sum(n * row_bytes(fmt, k) for _, n, k, _, _ in items)
        need = sum(quant_gemv_split_workspace_size(fmt, n, k, self.batch)
                   for _, n, k, _, _ in items if n)
        self.ws = _ws_arg(ws, need, items[0][0].device)
        self._wsp = _ptr(self.ws)
        self._wsn = 0 if self.ws is None else self.ws.numel()

    def __call__(self):
        _ck("quant_gemv_grouped", _lib.quant_gemv_grouped(self.fmt, self._ptr, self.count,
                                                          self.batch, self._wsp, self._wsn,
                                                          _stream()))


def quant_gemv_grouped(fmt: int, items, ws=None):
    """One launch for several products of the same format and batch; returns the
    list of y tensors."""
    GemvGroup(fmt, items, ws)()
    return [it[4] for it in items]


def quant_gemm_workspace_size(fmt: int, m: int, n: int, k: int, mode: int = GEMM_BF16) -> int:
    return _lib.quant_gemm_workspace_size(fmt, m, n, k, mode)


def quant_gemm(fmt: int, w: torch.Tensor, n: int, k: int, a: torch.Tensor,
               c: torch.Tensor | None = None, ws: torch.Tensor | None = None,
               mode: int = GEMM_BF16) -> torch.Tensor:
    """c[i][r] = sum_c a[i][c] w[r][c] on the matrix cores (bf16 operands, fp32 sums)."""
    _wbytes(w, fmt, n, k)
    _dev(a, "a", torch.float32)
    m = a.shape[0]
    if a.shape[1] != k:
        raise ValueError(f"a has {a.shape[1]} columns, K = {k}")
    if c is None:
        c = torch.empty((m, n), dtype=torch.float32, device=w.device)
    _dev(c, "c", torch.float32)
    need = quant_gemm_workspace_size(fmt, m, n, k, mode)
    if ws is None:
        ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=w.device)
    _dev(ws, "ws", torch.uint8)
    _ck("quant_gemm", _lib.quant_gemm(fmt, _ptr(w), n, k, _ptr(a), k, m, _ptr(c), n, mode,
                                      _ptr(ws), ws.numel(), _stream()))
    return c


def moe_route(wr: torch.Tensor, x: torch.Tensor, top_k: int):
    """Router logits, top-k expert indices (rank order, ties to the lower index)
    and renormalised probabilities.  Returns (idx int32 [T,k], probs [T,k], logits [T,E])."""
    _dev(wr, "wr", torch.float32)
    _dev(x, "x", torch.float32)
    e, h = wr.shape
    t = x.shape[0]
    if x.shape[1] != h:
        raise ValueError("x and wr disagree on the hidden size")
    idx = torch.empty((t, top_k), dtype=torch.int32, device=x.device)
    probs = torch.empty((t, top_k), dtype=torch.float32, device=x.device)
    logits = torch.empty((t, e), dtype=torch.float32, device=x.device)
    _ck("moe_route", _lib.moe_route(_ptr(wr), e, h, _ptr(x), t, top_k, _ptr(idx), _ptr(probs),
                                    _ptr(logits), _stream()))
    return idx, probs, logits


def moe_workspace_size(e: int, t: int, top_k: int, h: int, f: int) -> int:
    return _lib.moe_workspace_size(e, t, top_k, h, f)


def moe_workspace_h_offset(e: int, t: int, top_k: int) -> int:
    return _lib.moe_workspace_h_offset(e, t, top_k)


def moe_expert_gemv(fmt: int, wg: torch.Tensor, wu: torch.Tensor, wd: torch.Tensor, e: int,
                    h: int, f: int, x: torch.Tensor, idx: torch.Tensor, probs: torch.Tensor,
                    y: torch.Tensor | None = None, ws: torch.Tensor | None = None) -> torch.Tensor:
    """Routed expert feed-forward; wg/wu hold E stacked F x H matrices, wd E stacked
    H x F matrices.  Returns y [T, H]."""
    _wbytes(wg, fmt, e * f, h, "wg")
    _wbytes(wu, fmt, e * f, h, "wu")
    _wbytes(wd, fmt, e * h, f, "wd")
    _dev(x, "x", torch.float32)
    _dev(idx, "idx", torch.int32)
    _dev(probs, "probs", torch.float32)
    t, top_k = idx.shape
    if x.shape != (t, h) or probs.shape != (t, top_k):
        raise ValueError("x, idx and probs disagree on T / H / top_k")
    if y is None:
        y = torch.empty((t, h), dtype=torch.float32, device=x.device)
    _dev(y, "y", torch.float32)
    need = moe_workspace_size(e, t, top_k, h, f)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _dev(ws, "ws", torch.uint8)
    _ck("moe_expert_gemv", _lib.moe_expert_gemv(fmt, _ptr(wg), _ptr(wu), _ptr(wd), e, h, f,
                                                _ptr(x), t, _ptr(idx), _ptr(probs), top_k,
                                                _ptr(y), _ptr(ws), ws.numel(), _stream()))
    return y


def moe_layer_workspace_size(e: int, t: int, top_k: int, h: int, f: int) -> int:
    return _lib.moe_layer_workspace_size(e, t, top_k, h, f)


def moe_layer_gemv(fmt: int, wr: torch.Tensor, wg: torch.Tensor, wu: torch.Tensor,
                   wd: torch.Tensor, e: int, h: int, f: int, x: torch.Tensor, top_k: int,
                   out: tuple | None = None, ws: torch.Tensor | None = None):
    """moe_route then moe_expert_gemv (one token: routing in one launch).
    Returns (y [T, H], idx int32 [T, k], probs [T, k], logits [T, E]); `out` may
    give those four tensors to write.  A given `ws` must start with a zero
    control block (torch.zeros); every call leaves it zero."""
    _dev(wr, "wr", torch.float32)
    _wbytes(wg, fmt, e * f, h, "wg")
    _wbytes(wu, fmt, e * f, h, "wu")
    _wbytes(wd, fmt, e * h, f, "wd")
    _dev(x, "x", torch.float32)
    t = x.shape[0]
    if tuple(wr.shape) != (e, h) or x.shape[1] != h:
        raise ValueError("wr, x disagree on E / H")
    if out is None:
        out = (torch.empty((t, h), dtype=torch.float32, device=x.device),
               torch.empty((t, top_k), dtype=torch.int32, device=x.device),
               torch.empty((t, top_k), dtype=torch.float32, device=x.device),
               torch.empty((t, e), dtype=torch.float32, device=x.device))
    y, idx, probs, logits = out
    _dev(y, "y", torch.float32)
    _dev(idx, "idx", torch.int32)
    _dev(probs, "probs", torch.float32)
    _dev(logits, "logits", torch.float32)
    need = moe_layer_workspace_size(e, t, top_k, h, f)
    if ws is None:
        ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=x.device)
    _dev(ws, "ws", torch.uint8)
    _ck("moe_layer_gemv", _lib.moe_layer_gemv(fmt, _ptr(wr), _ptr(wg), _ptr(wu), _ptr(wd), e, h,
                                              f, _ptr(x), t, top_k, _ptr(logits), _ptr(idx),
                                              _ptr(probs), _ptr(y), _ptr(ws), ws.numel(),
                                              _stream()))
    return y, idx, probs, logits


def moe_gemm_workspace_size(e: int, t: int, top_k: int, h: int, f: int) -> int:
    return _lib.moe_gemm_workspace_size(e, t, top_k, h, f)


def moe_expert_gemm(fmt: int, wg: torch.Tensor, wu: torch.Tensor, wd: torch.Tensor, e: int,
                    h: int, f: int, x: torch.Tensor, idx: torch.Tensor, probs: torch.Tensor,
                    y: torch.Tensor | None = None, ws: torch.Tensor | None = None) -> torch.Tensor:
    """moe_expert_gemv's function at prompt batch, on the matrix cores (bf16
    operands, fp32 accumulation; the prompt-GEMM tolerance).  Returns y [T, H]."""
    _wbytes(wg, fmt, e * f, h, "wg")
    _wbytes(wu, fmt, e * f, h, "wu")
    _wbytes(wd, fmt, e * h, f, "wd")
    _dev(x, "x", torch.float32)
    _dev(idx, "idx", torch.int32)
    _dev(probs, "probs", torch.float32)
    t, top_k = idx.shape
    if x.shape != (t, h) or probs.shape != (t, top_k):
        raise ValueError("x, idx and probs disagree on T / H / top_k")
    if y is None:
        y = torch.empty((t, h), dtype=torch.float32, device=x.device)
    _dev(y, "y", torch.float32)
    need = moe_gemm_workspace_size(e, t, top_k, h, f)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _dev(ws, "ws", torch.uint8)
    _ck("moe_expert_gemm", _lib.moe_expert_gemm(fmt, _ptr(wg), _ptr(wu), _ptr(wd), e, h, f,
                                                _ptr(x), t, _ptr(idx), _ptr(probs), top_k,
                                                _ptr(y), _ptr(ws), ws.numel(), _stream()))
    return y
