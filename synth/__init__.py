"""Seeded synthetic inputs shaped like the models the Phobos pages run.

The Phobos README (githubhelp mirror, section "Inference") lists the GGUF models
the engine was tested on (Q8_0 ~1B dense models, a Q4_K_M 4B dense model, a
Q4_K_M 35B mixture of experts).  None of those files exist here, so every test
and benchmark draws seeded synthetic tensors with the same shapes and value
distributions instead.

This module only draws random numbers and writes them into raw byte arrays.  It
holds none of the method's arithmetic: no dequantisation, no dot products, no
unpacking of the packed 6-bit fields.  Both the CPU oracle and the GPU library
consume what it produces; neither imports the other.

Block byte layouts written here (plain reading of the GGUF on-disk format; the
pages name the formats but do not print their bytes):

  Q8_0 (34 bytes / 32 weights):  [0:2] fp16 scale d, [2:34] 32 x int8 q
  Q4_K (144 bytes / 256 weights): [0:2] fp16 d, [2:4] fp16 dmin,
                                  [4:16] 12 bytes of packed 6-bit scales/mins,
                                  [16:144] 128 bytes of 4-bit quants

For Q4_K the 96 bits of the packed field are a bijection onto the sixteen 6-bit
scale/min values, so 12 uniform random bytes give sixteen independent values
uniform on 0..63; likewise 128 uniform random bytes give 256 quants uniform on
0..15.  The generator therefore never needs to know where each bit goes.

Random numbers: numpy's PCG64 seeded with the SeedSequence ``(seed, tensor_id)``,
so every tensor of a workload has its own reproducible stream.
"""
from __future__ import annotations

import numpy as np

Q8_0_BLOCK_BYTES = 34
Q8_0_BLOCK_WEIGHTS = 32
Q4_K_BLOCK_BYTES = 144
Q4_K_BLOCK_WEIGHTS = 256

FMT_Q8_0 = 8    # GGUF tensor-type ids
FMT_Q4_K = 12


def rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tensor_id)])))


def _half_abs_normal(g: np.random.Generator, n: int, scale: float) -> np.ndarray:
    """fp16 bits of scale*|N(0,1)|, drawn in fp64 and rounded to fp16 (RNE)."""
    v = scale * np.abs(g.standard_normal(n))
    return v.astype(np.float16).view(np.uint16)


def q8_0_matrix(n_rows: int, k: int, seed: int = 0, tensor_id: int = 0,
                d_scale: float = 0.01) -> np.ndarray:
    """Random Q8_0 matrix [n_rows][k/32 blocks] as raw bytes, shape (n_rows, k/32*34).

    q uniform on [-127, 127] (-128 never drawn), d = fp16(d_scale*|N(0,1)|).
    """
    assert k % Q8_0_BLOCK_WEIGHTS == 0
    nb = n_rows * (k // Q8_0_BLOCK_WEIGHTS)
    g = rng(seed, tensor_id)
    d = _half_abs_normal(g, nb, d_scale)
    q = g.integers(-127, 128, size=(nb, 32), dtype=np.int16).astype(np.int8)
    out = np.empty((nb, Q8_0_BLOCK_BYTES), dtype=np.uint8)
    out[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    out[:, 2:34] = q.view(np.uint8)
    return out.reshape(n_rows, -1)


def q4_k_matrix(n_rows: int, k: int, seed: int = 0, tensor_id: int = 0,
                d_scale: float = 0.002) -> np.ndarray:
    """Random Q4_K matrix as raw bytes, shape (n_rows, k/256*144).

    d, dmin = fp16(d_scale*|N(0,1)|); packed scale bytes and quant bytes uniform.
    """
    assert k % Q4_K_BLOCK_WEIGHTS == 0
    nb = n_rows * (k // Q4_K_BLOCK_WEIGHTS)
    g = rng(seed, tensor_id)
    d = _half_abs_normal(g, nb, d_scale)
    dmin = _half_abs_normal(g, nb, d_scale)
    out = np.empty((nb, Q4_K_BLOCK_BYTES), dtype=np.uint8)
    out[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    out[:, 2:4] = dmin.view(np.uint8).reshape(nb, 2)
    out[:, 4:144] = g.integers(0, 256, size=(nb, 140), dtype=np.uint8)
    return out.reshape(n_rows, -1)


def quant_matrix(fmt: int, n_rows: int, k: int, seed: int = 0, tensor_id: int = 0) -> np.ndarray:
    if fmt == FMT_Q8_0:
        return q8_0_matrix(n_rows, k, seed, tensor_id)
    if fmt == FMT_Q4_K:
        return q4_k_matrix(n_rows, k, seed, tensor_id)
    raise ValueError(f"unknown format {fmt}")


def row_bytes(fmt: int, k: int) -> int:
    if fmt == FMT_Q8_0:
        return k // Q8_0_BLOCK_WEIGHTS * Q8_0_BLOCK_BYTES
    if fmt == FMT_Q4_K:
        return k // Q4_K_BLOCK_WEIGHTS * Q4_K_BLOCK_BYTES
    raise ValueError(f"unknown format {fmt}")


def normal_f32(shape, seed: int = 0, tensor_id: int = 0, std: float = 1.0) -> np.ndarray:
    """fp32 N(0, std^2) drawn in fp64 then rounded to fp32."""
    g = rng(seed, tensor_id)
    return (std * g.standard_normal(shape)).astype(np.float32)


# ---------------------------------------------------------------------------
# Workloads.  Shapes follow the models named in the Phobos README ("Inference"):
# a ~1B dense Q8_0 transformer, a 4B-class Q4_K dense model and a 35B-A3B-class
# Q4_K mixture of experts; and the llama-bench style pp512 prompt size of the
# phobos-bench tool (README, "Command-Line Tools").  Tensor ids are fixed so the
# same seed always yields the same bytes.
# ---------------------------------------------------------------------------

#: 1B-class dense decode layer set, Q8_0: (name, N rows, K) in forward order.
DENSE_1B_LAYER_SET = (
    ("qkv", 3072, 2048),
    ("o", 2048, 2048),
    ("gate", 6144, 2048),
    ("up", 6144, 2048),
    ("down", 2048, 6144),
    ("head", 65536, 2048),
)

#: 4B-class Q4_K FFN matrices (N, K).
Q4K_FFN_PAIR = (("ffn_up", 9728, 2560), ("ffn_down", 2560, 9728))

#: 35B-A3B-class MoE layer.
MOE_EXPERTS = 128
MOE_TOP_K = 8
MOE_HIDDEN = 2048
MOE_FFN = 768
MOE_ROUTER_STD = 0.02

#: pp512 prompt GEMMs: (name, fmt, N, K), activations M=512 x K.
PP512_M = 512
PP512_GEMMS = (("q4k_up", FMT_Q4_K, 17408, 5120), ("q8_down", FMT_Q8_0, 5120, 17408))


def tid(*parts: int) -> int:
    """Stable tensor id from small integers."""
    v = 0
    for p in parts:
        v = v * 1000003 + int(p)
    return v % (1 << 62)


def moe_layer(seed: int = 0, n_tokens: int = 1, experts: int = MOE_EXPERTS,
              hidden: int = MOE_HIDDEN, ffn: int = MOE_FFN):
    """Router (fp32), stacked Q4_K expert gate/up/down and token activations.

    Returns dict with 'wr' [E][H] f32, 'wg','wu' [E][F][H/256*144] u8,
    'wd' [E][H][F/256*144] u8, 'x' [T][H] f32.
    """
    wr = normal_f32((experts, hidden), seed, tid(3, 0), std=MOE_ROUTER_STD)
    wg = q4_k_matrix(experts * ffn, hidden, seed, tid(3, 1)).reshape(experts, ffn, -1)
    wu = q4_k_matrix(experts * ffn, hidden, seed, tid(3, 2)).reshape(experts, ffn, -1)
    wd = q4_k_matrix(experts * hidden, ffn, seed, tid(3, 3)).reshape(experts, hidden, -1)
    x = normal_f32((n_tokens, hidden), seed, tid(3, 4, n_tokens))
    return {"wr": wr, "wg": wg, "wu": wu, "wd": wd, "x": x}
