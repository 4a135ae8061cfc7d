"""GPU check of quant_gemv_noalloc (the decode GEMV whose workspace is the
library's fixed device scratch) through the C ABI, against quant_gemv with a
caller workspace of the same size -- same kernels and plan, so the same bits --
and against the oracle at the GEMV tolerance.  Two calls in a row share the
scratch; the second is smaller, so stale contents of the first must not leak
into it (the work counter and the zeroed outputs are reset by the kernels)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from _gpu import GEMV_TOL, check_rel, dev, host, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

Q8, Q4 = synth.FMT_Q8_0, synth.FMT_Q4_K
SCRATCH = 16 << 20


@pytest.fixture(scope="module")
def g():
    import quantized_gguf_q8_amd as g
    return g


def _call_noalloc(g, fmt, w, n, k, x):
    b = x.shape[0]
    y = torch.full((b, n), float("nan"), dtype=torch.float32, device="cuda")
    st = g._lib.quant_gemv_noalloc(fmt, w.data_ptr(), n, k, x.data_ptr(), k, y.data_ptr(), n, b,
                                   torch.cuda.current_stream().cuda_stream)
    assert st == 0, g._lib.ggq_status_string(st)
    return host(y)


def _call_ws(g, fmt, w, n, k, x, ws_bytes):
    b = x.shape[0]
    y = torch.full((b, n), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    st = g._lib.quant_gemv(fmt, w.data_ptr(), n, k, x.data_ptr(), k, y.data_ptr(), n, b,
                           ws.data_ptr(), ws_bytes, torch.cuda.current_stream().cuda_stream)
    assert st == 0, g._lib.ggq_status_string(st)
    return host(y)


def _same_size_ws(g, fmt, n, k, b):
    split = g.quant_gemv_split_workspace_size(fmt, n, k, b)
    return split if split <= SCRATCH else g.quant_gemv_workspace_size(fmt, k, b)


# (fmt, n, k, batch) pairs: the second call of each pair is smaller
CASES = [
    ((Q4, 2560, 9728, 16), (Q4, 300, 1024, 3)),      # K parts (planes fit), then a small call
    ((Q8, 65536, 2048, 8), (Q8, 1000, 512, 2)),      # planes do not fit: whole tiles only
    ((Q4, 9728, 2560, 4), (Q4, 257, 2560, 1)),       # then batch 1 (vector units, no scratch)
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_workspace_call(g, first, second):
    for i, (fmt, n, k, b) in enumerate((first, second)):
        say(f"noalloc call {i}: fmt={fmt} n={n} k={k} batch={b}")
        wh = synth.quant_matrix(fmt, n, k, seed=4, tensor_id=90 + i)
        xh = synth.normal_f32((b, k), seed=4, tensor_id=95 + i)
        w, x = dev(wh), dev(xh)
        y0 = _call_noalloc(g, fmt, w, n, k, x)
        y1 = _call_ws(g, fmt, w, n, k, x, max(256, _same_size_ws(g, fmt, n, k, b)))
        assert np.array_equal(y0, y1), "noalloc differs from the same-size workspace call"
        yr, s = oracle.gemv(fmt, wh, n, k, xh)
        check_rel(y0, yr, s, GEMV_TOL, "noalloc vs oracle")


def test_noalloc_refuses_more_than_its_scratch(g):
    # K = 2^19 Q8_0 columns at batch 16 need 32 MiB of activation fragments
    k = 1 << 19
    assert g.quant_gemv_workspace_size(Q8, k, 16) > SCRATCH
    w = torch.zeros((1, k // 32 * 34), dtype=torch.uint8, device="cuda")
    x = torch.zeros((16, k), dtype=torch.float32, device="cuda")
    y = torch.zeros((16, 1), dtype=torch.float32, device="cuda")
    st = g._lib.quant_gemv_noalloc(Q8, w.data_ptr(), 1, k, x.data_ptr(), k, y.data_ptr(), 1, 16,
                                   torch.cuda.current_stream().cuda_stream)
    assert st == -6 and b"scratch" in g._lib.ggq_status_string(st)
