"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/ggq.h declares, and reject
bad arguments with the documented status before touching HIP.  Fake device
pointers are never dereferenced: every call here fails validation (or is a
documented no-op) on the host.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ggq.h")

OK, ARG, UNSUP, ALIGN, WS = 0, -1, -2, -3, -4


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


@pytest.fixture(scope="module")
def g():
    import quantized_gguf_q8_amd as g
    return g


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("quant_gemv", "quant_gemm", "moe_expert_gemv", "moe_route", "quant_dequantize",
              "quant_gemm_workspace_size", "moe_workspace_size", "moe_workspace_h_offset",
              "quant_gemv_workspace_size", "quant_gemv_split_workspace_size",
              "quant_gemv_swiglu", "moe_expert_gemm", "moe_gemm_workspace_size",
              "ggq_status_string", "ggq_version"):
        assert n in names


def test_library_exports_every_declared_symbol(g):
    lib = ctypes.CDLL(g.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n


def test_status_strings(g):
    for s in (OK, ARG, UNSUP, ALIGN, WS, -5, 12345):
        assert g._lib.ggq_status_string(s)
    assert g._lib.ggq_status_string(ARG) == b"invalid argument"


A16 = 0x10000          # fake, 16-byte (and 256-byte) aligned "device" addresses
B16 = 0x20000
C16 = 0x30000
D16 = 0x40000


def test_gemv_validation(g):
    L = g._lib
    assert L.quant_gemv(99, A16, 4, 32, B16, 32, C16, 4, 1, None, 0, None) == UNSUP
    assert L.quant_gemv(8, A16, 4, 33, B16, 33, C16, 4, 1, None, 0, None) == ARG      # K % 32
    assert L.quant_gemv(12, A16, 4, 512 + 32, B16, 544, C16, 4, 1, None, 0, None) == ARG  # K % 256
    assert L.quant_gemv(8, A16, 4, 32, B16, 32, C16, 4, 0, None, 0, None) == ARG       # batch 0
    assert L.quant_gemv(8, A16, 4, 32, B16, 32, C16, 4, 17, None, 0, None) == ARG      # batch 17
    assert L.quant_gemv(8, A16, 4, 64, B16, 32, C16, 4, 1, None, 0, None) == ARG       # ldx < K
    assert L.quant_gemv(8, A16, 4, 32, B16, 32, C16, 3, 1, None, 0, None) == ARG       # ldy < N
    assert L.quant_gemv(8, None, 4, 32, B16, 32, C16, 4, 1, None, 0, None) == ARG
    assert L.quant_gemv(8, A16, 4, 32, None, 32, C16, 4, 1, None, 0, None) == ARG
    assert L.quant_gemv(8, A16 + 2, 4, 32, B16, 32, C16, 4, 1, None, 0, None) == ALIGN
    assert L.quant_gemv(8, A16, 4, 32, B16 + 4, 32, C16, 4, 1, None, 0, None) == ALIGN
    assert L.quant_gemv(8, A16, 4, 32, B16, 34, C16, 4, 1, None, 0, None) == ALIGN     # ldx % 4
    assert L.quant_gemv(8, A16, 4, 32, B16, 32, C16 + 2, 4, 1, None, 0, None) == ALIGN
    assert L.quant_gemv(8, None, 0, 32, None, 32, None, 0, 1, None, 0, None) == OK     # N == 0 no-op
    assert L.quant_gemv(8, A16, -1, 32, B16, 32, C16, 4, 1, None, 0, None) == ARG


def test_gemv_workspace_validation(g):
    L = g._lib
    need = L.quant_gemv_workspace_size(8, 2048, 8)
    assert need >= 2048 // 32 * 1024
    assert L.quant_gemv_workspace_size(8, 2048, 17) == 0
    assert L.quant_gemv_workspace_size(12, 2000, 4) == 0
    assert L.quant_gemv_workspace_size(12, 2560, 16) > L.quant_gemv_workspace_size(12, 2560, 8)
    assert L.quant_gemv(8, A16, 4, 2048, B16, 2048, C16, 4, 8, D16, need - 1, None) == WS
    assert L.quant_gemv(8, A16, 4, 2048, B16, 2048, C16, 4, 8, D16 + 16, need, None) == ALIGN
    # the split-K workspace adds 16 partial planes of batch x N floats
    S = L.quant_gemv_split_workspace_size
    assert S(12, 2560, 9728, 4) >= L.quant_gemv_workspace_size(12, 9728, 4) + 16 * 4 * 2560 * 4
    assert S(12, 0, 9728, 4) == L.quant_gemv_workspace_size(12, 9728, 4)
    assert S(12, -1, 9728, 4) == 0 and S(12, 2560, 9700, 4) == 0 and S(8, 64, 2048, 17) == 0


def test_gemv_swiglu_validation(g):
    L = g._lib
    f = L.quant_gemv_swiglu
    assert f(5, A16, A16, 4, 2048, B16, 2048, C16, 4, 1, None, 0, None) == UNSUP
    assert f(8, A16, A16, 4, 2080, B16, 2080, C16, 4, 1, None, 0, None) == ARG   # K % 256
    assert f(8, A16, A16, 4, 2048, B16, 2048, C16, 4, 17, None, 0, None) == ARG  # batch
    assert f(8, A16, A16, 4, 2048, B16, 2047, C16, 4, 1, None, 0, None) == ARG   # ldx < K
    assert f(8, A16, A16 + 4, 4, 2048, B16, 2048, C16, 4, 1, None, 0, None) == ALIGN
    need = L.quant_gemv_workspace_size(8, 2048, 4)
    assert f(8, A16, A16, 4, 2048, B16, 2048, C16, 4, 4, None, 0, None) == WS
    assert f(8, A16, A16, 4, 2048, B16, 2048, C16, 4, 4, D16, need - 1, None) == WS
    assert f(8, A16, A16, 4, 2048, B16, 2048, C16, 4, 4, D16 + 16, need, None) == ALIGN
    assert f(8, None, None, 0, 2048, None, 2048, None, 0, 4, None, 0, None) == OK  # N = 0


def test_gemv_grouped_validation(g):
    L = g._lib
    arr = (g.GemvDesc * 3)()
    for i in range(3):
        arr[i] = g.GemvDesc(A16, 4, 2048, B16, 2048, C16, 4)
    p = ctypes.cast(arr, ctypes.c_void_p)
    assert L.quant_gemv_grouped(8, p, 0, 1, None, 0, None) == ARG
    assert L.quant_gemv_grouped(8, p, 17, 1, None, 0, None) == ARG
    assert L.quant_gemv_grouped(8, None, 2, 1, None, 0, None) == ARG
    assert L.quant_gemv_grouped(5, p, 2, 1, None, 0, None) == UNSUP
    arr[1] = g.GemvDesc(A16, 4, 2047, B16, 2048, C16, 4)       # bad K in one member
    assert L.quant_gemv_grouped(8, p, 3, 1, None, 0, None) == ARG
    arr[1] = g.GemvDesc(A16 + 4, 4, 2048, B16, 2048, C16, 4)   # misaligned member
    assert L.quant_gemv_grouped(8, p, 3, 1, None, 0, None) == ALIGN
    arr[1] = g.GemvDesc(A16, 4, 2048, B16, 2048, C16, 4)
    # one control block, then each member's activation fragments
    one = L.quant_gemv_workspace_size(8, 2048, 4)
    need = g.CTRL_BYTES + 3 * (one - g.CTRL_BYTES)
    assert L.quant_gemv_grouped(8, p, 3, 4, D16, need - 1, None) == WS
    for i in range(3):
        arr[i] = g.GemvDesc(None, 0, 2048, None, 2048, None, 0)  # all empty: no-op
    assert L.quant_gemv_grouped(8, p, 3, 4, None, 0, None) == OK


def test_dequant_validation(g):
    L = g._lib
    assert L.quant_dequantize(7, A16, 1, 32, B16, None) == UNSUP
    assert L.quant_dequantize(8, A16, 1, 48, B16, None) == ARG
    assert L.quant_dequantize(12, A16, 1, 128, B16, None) == ARG
    assert L.quant_dequantize(8, A16, 1, 0, B16, None) == ARG
    assert L.quant_dequantize(8, None, 1, 32, B16, None) == ARG
    assert L.quant_dequantize(8, A16 + 8, 1, 32, B16, None) == ALIGN
    assert L.quant_dequantize(12, A16, 0, 256, None, None) == OK


def test_gemm_validation(g):
    L = g._lib
    need = L.quant_gemm_workspace_size(12, 512, 1024, 5120, 0)
    assert need >= 512 * 5120 * 2
    assert L.quant_gemm_workspace_size(12, 512, 1024, 5100, 0) == 0
    assert L.quant_gemm_workspace_size(12, 512, 1024, 5120, 1) == 0
    args = lambda **kw: dict(dict(t=12, w=A16, n=1024, k=5120, a=B16, lda=5120, m=512, c=C16,
                                  ldc=1024, mode=0, ws=D16, wsb=need), **kw)

    def call(d):
        return L.quant_gemm(d["t"], d["w"], d["n"], d["k"], d["a"], d["lda"], d["m"], d["c"],
                            d["ldc"], d["mode"], d["ws"], d["wsb"], None)

    assert call(args(mode=3)) == UNSUP
    assert call(args(t=2)) == UNSUP
    assert call(args(k=5000, lda=5000)) == ARG
    assert call(args(lda=100)) == ARG
    assert call(args(ldc=10)) == ARG
    assert call(args(a=None)) == ARG
    assert call(args(a=B16 + 4)) == ALIGN
    assert call(args(lda=5122)) == ALIGN
    assert call(args(ws=None)) == WS
    assert call(args(wsb=need - 1)) == WS
    assert call(args(ws=D16 + 16)) == ALIGN
    assert call(args(m=0, w=None, a=None, c=None, ws=None)) == OK


def test_route_validation(g):
    L = g._lib
    assert L.moe_route(A16, 128, 2048, B16, 1, 0, C16, D16, D16, None) == ARG
    assert L.moe_route(A16, 128, 2048, B16, 1, 33, C16, D16, D16, None) == ARG
    assert L.moe_route(A16, 4, 2048, B16, 1, 5, C16, D16, D16, None) == ARG
    assert L.moe_route(A16, 2048, 2048, B16, 1, 8, C16, D16, D16, None) == ARG
    assert L.moe_route(A16, 128, 2046, B16, 1, 8, C16, D16, D16, None) == ARG
    assert L.moe_route(A16, 128, (1 << 24) + 4, B16, 1, 8, C16, D16, D16, None) == ARG
    assert L.moe_route(A16, 128, 2048, B16, 1, 8, C16, D16, None, None) == ARG
    assert L.moe_route(A16 + 4, 128, 2048, B16, 1, 8, C16, D16, D16, None) == ALIGN
    assert L.moe_route(None, 128, 2048, None, 0, 8, None, None, None, None) == OK


def test_noalloc_validation(g):
    L = g._lib
    # argument checks are those of quant_gemv, before any device work
    assert L.quant_gemv_noalloc(99, A16, 4, 32, B16, 32, C16, 4, 2, None) == UNSUP
    assert L.quant_gemv_noalloc(8, A16, 4, 33, B16, 33, C16, 4, 2, None) == ARG
    assert L.quant_gemv_noalloc(8, A16, 4, 256, B16, 256, C16, 4, 17, None) == ARG
    assert L.quant_gemv_noalloc(8, A16, 4, 256, B16 + 8, 256, C16, 4, 2, None) == ALIGN
    assert L.quant_gemv_noalloc(8, A16, 0, 256, B16, 256, C16, 0, 2, None) == OK   # N = 0
    # more activation fragments than the fixed scratch holds: refused, nothing launched
    k = 1 << 19
    assert L.quant_gemv_workspace_size(8, k, 16) > (16 << 20)
    assert L.quant_gemv_noalloc(8, A16, 1, k, B16, k, C16, 1, 16, None) == -6
    assert b"scratch" in L.ggq_status_string(-6)


def test_moe_validation(g):
    L = g._lib
    need = L.moe_workspace_size(128, 16, 8, 2048, 768)
    assert need > 16 * 8 * (2048 + 768) * 4
    assert L.moe_workspace_size(0, 16, 8, 2048, 768) == 0
    off = L.moe_workspace_h_offset(128, 16, 8)
    assert off % 256 == 0 and off >= (3 * 128 + 1 + 128) * 4

    def call(t=12, e=128, h=2048, f=768, tt=16, k=8, ws=D16, wsb=need, x=B16):
        return L.moe_expert_gemv(t, A16, A16, A16, e, h, f, x, tt, C16, C16, k, C16, ws, wsb, None)

    # (only failing variants are called: a valid call would launch kernels on fake pointers)
    assert call(t=5) == UNSUP
    assert call(h=2000) == ARG
    assert call(f=100) == ARG
    assert call(k=9, e=8) == ARG
    assert call(x=None) == ARG
    assert call(x=B16 + 8) == ALIGN
    assert call(wsb=need - 1) == WS
    assert call(ws=D16 + 64) == ALIGN
    # 32-bit buffer offsets: h [T*top_k][F] or x [T][H] past 4 GiB is refused
    assert call(tt=8192, k=8, h=256, f=16384) == ARG
    assert call(tt=65536, k=1, h=16384) == ARG


def test_moe_layer_validation(g):
    L = g._lib
    need = L.moe_layer_workspace_size(128, 1, 8, 2048, 768)
    assert need == g.CTRL_BYTES + L.moe_workspace_size(128, 1, 8, 2048, 768)
    assert L.moe_layer_workspace_size(0, 1, 8, 2048, 768) == 0
    assert L.moe_layer_workspace_size(128, 1, 33, 2048, 768) == 0

    def call(t=12, e=128, h=2048, f=768, tt=1, k=8, ws=D16, wsb=need, x=B16, wr=A16, lg=C16):
        return L.moe_layer_gemv(t, wr, A16, A16, A16, e, h, f, x, tt, k, lg, C16, C16, C16, ws,
                                wsb, None)

    # (only failing variants are called: a valid call would launch kernels on fake pointers)
    assert call(t=5) == UNSUP
    assert call(h=2000) == ARG
    assert call(k=9, e=8) == ARG
    assert call(k=33) == ARG
    assert call(e=1025) == ARG
    assert call(wr=None) == ARG
    assert call(lg=None) == ARG
    assert call(wr=A16 + 4) == ALIGN
    assert call(x=B16 + 8) == ALIGN
    assert call(wsb=need - 1) == WS
    assert call(ws=None) == WS
    assert call(ws=D16 + 64) == ALIGN
    assert call(tt=0, wsb=0, ws=None) == OK


def test_moe_gemm_validation(g):
    L = g._lib
    need = L.moe_gemm_workspace_size(128, 512, 8, 2048, 768)
    p = 512 * 8
    slots = p + 15 * 128
    # bf16 x, bf16 h per padded slot, fp32 down outputs per pair, slot list
    assert need >= 512 * 2048 * 2 + slots * 768 * 2 + p * 2048 * 4 + slots * 4
    assert need < 512 * 2048 * 2 + slots * 768 * 2 + p * 2048 * 4 + slots * 4 + 64 * 1024
    assert L.moe_gemm_workspace_size(0, 512, 8, 2048, 768) == 0
    assert L.moe_gemm_workspace_size(128, 65537, 1, 2048, 768) == 0

    def call(t=12, e=128, h=2048, f=768, tt=512, k=8, ws=D16, wsb=need, x=B16):
        return L.moe_expert_gemm(t, A16, A16, A16, e, h, f, x, tt, C16, C16, k, C16, ws, wsb, None)

    # (only failing variants are called: a valid call would launch kernels on fake pointers)
    assert call(t=5) == UNSUP
    assert call(h=2000) == ARG
    assert call(f=100) == ARG
    assert call(k=9, e=8) == ARG
    assert call(e=1025) == ARG
    assert call(tt=8193) == ARG                       # more than 65536 pairs
    assert call(tt=65536, k=1, h=16384) == ARG        # bf16 x past 2 GiB
    assert call(x=None) == ARG
    assert call(x=B16 + 8) == ALIGN
    assert call(wsb=need - 1) == WS
    assert call(ws=None) == WS
    assert call(ws=D16 + 64) == ALIGN
    assert call(tt=0, x=None, ws=None) == OK           # no tokens: nothing to do
