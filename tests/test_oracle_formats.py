"""Pins of the oracle's block decoders against facts fixed outside the oracle.

The Phobos README ("Inference") names Q8_0 and Q4_K_M models but prints neither
their bytes nor their arithmetic; the reading pinned here is the GGUF layout
(see tests/golden/*.txt for the byte maps).  Nothing below calls the GPU library.
"""
from fractions import Fraction

import numpy as np
import pytest

import synth
from _golden import q4_k_blocks, q8_0_blocks


# --------------------------------------------------------------------------- #
# fp16 decode: every one of the 65536 bit patterns against numpy's binary16 -> binary32
# conversion (a library routine independent of the oracle's bit decomposition).
def test_half_to_float_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    # Decode through the oracle's Q8_0 path with q = 1: w = d exactly.
    blocks = np.zeros((65536, 34), dtype=np.uint8)
    blocks[:, 0:2] = bits.view(np.uint8).reshape(-1, 2)
    blocks[:, 2] = 1
    w = orc.dequant(orc.Q8_0, blocks, 65536, 32)[:, 0]
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(w), nan)
    assert np.array_equal(w[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    # The scalar entry point agrees on a sample including subnormals and -0.
    sample = [0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0xFBFF, 0x7C00, 0xFC00]
    got = orc.half_to_float(sample)
    assert np.array_equal(got.view(np.uint32), np.array(sample, np.uint16).view(np.float16).astype(np.float32).view(np.uint32))


# --------------------------------------------------------------------------- #
# Q8_0
def test_q8_0_hand_built_blocks(orc):
    for raw, expect, _ in q8_0_blocks():
        w = orc.dequant(orc.Q8_0, np.frombuffer(raw, np.uint8), 1, 32)[0]
        assert np.array_equal(w.view(np.uint32), expect.view(np.uint32)), (raw[:2].hex(), w, expect)


def test_q8_0_brute_force_all_scales_all_quants(orc):
    """Every finite fp16 d times every int8 q, against an integer-exact path:
    d = M * 2^E with integer M, so d*q = (M*q) * 2^E exactly."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    e = (h >> 10) & 31
    h = h[e < 31]                                  # finite patterns: 63488
    nd = h.size
    q = np.arange(-128, 128, dtype=np.int16).astype(np.int8).reshape(8, 32)
    blocks = np.zeros((nd, 8, 34), dtype=np.uint8)
    blocks[:, :, 0:2] = h.view(np.uint8).reshape(nd, 1, 2)
    blocks[:, :, 2:] = q.view(np.uint8)[None]
    w = orc.dequant(orc.Q8_0, blocks.reshape(nd * 8, 34), nd * 8, 32).reshape(nd, 256)

    sign = (h >> 15).astype(np.int64)
    ex = ((h >> 10) & 31).astype(np.int64)
    fr = (h & 1023).astype(np.int64)
    mant = np.where(ex == 0, fr, 1024 + fr)
    expo = np.where(ex == 0, -24, ex - 25)
    qv = q.ravel().astype(np.int64)
    prod = (mant[:, None] * qv[None, :]) * np.where(sign == 1, -1, 1)[:, None]
    ref = np.ldexp(prod.astype(np.float64), expo[:, None]).astype(np.float32)
    # Zero results carry the IEEE sign of d*q: negative iff exactly one factor is negative.
    zero = prod == 0
    neg = (sign[:, None] == 1) ^ (qv[None, :] < 0)
    ref[zero] = np.where(neg[zero], np.float32(-0.0), np.float32(0.0))
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))


# --------------------------------------------------------------------------- #
# Q4_K packed scales: the oracle's shift/mask unpacker against a bit map written as
# a table of (field, bit) -> (byte, bit) from the layout description.
def _bit_map():
    table = {}
    for j in range(4):
        for b in range(6):
            table[("sc", j, b)] = (j, b)            # sc0..3 : bytes 0..3, bits 0..5
            table[("m", j, b)] = (j + 4, b)         # m0..3  : bytes 4..7, bits 0..5
    for j in range(4, 8):
        for b in range(4):
            table[("sc", j, b)] = (j + 4, b)        # low nibble of bytes 8..11
            table[("m", j, b)] = (j + 4, b + 4)     # high nibble of bytes 8..11
        for b in range(4, 6):
            table[("sc", j, b)] = (j - 4, b + 2)    # bits 6,7 of bytes 0..3
            table[("m", j, b)] = (j, b + 2)         # bits 6,7 of bytes 4..7
    return table


def _extract(table, s):
    sc, m = [0] * 8, [0] * 8
    for (field, j, b), (byte, bit) in table.items():
        v = (s[byte] >> bit) & 1
        if field == "sc":
            sc[j] |= v << b
        else:
            m[j] |= v << b
    return sc, m


def test_q4_k_bit_map_is_a_bijection():
    table = _bit_map()
    assert len(table) == 96
    assert len(set(table.values())) == 96
    assert set(table.values()) == {(byte, bit) for byte in range(12) for bit in range(8)}


def test_q4_k_scale_unpack_every_byte_pattern(orc):
    table = _bit_map()
    for background in (0x00, 0xFF):
        for pos in range(12):
            for v in range(256):
                s = [background] * 12
                s[pos] = v
                got = orc.q4_k_scale_min(bytes(s))
                assert got == _extract(table, s), (background, pos, v)


def test_q4_k_hand_built_blocks(orc):
    for raw, expect, sc, m in q4_k_blocks():
        assert orc.q4_k_scale_min(raw[4:16]) == (sc, m)
        w = orc.dequant(orc.Q4_K, np.frombuffer(raw, np.uint8), 1, 256)[0]
        assert np.array_equal(w.view(np.uint32), expect.view(np.uint32)), (w, expect)


def _half_fraction(bits):
    s = bits >> 15
    e = (bits >> 10) & 31
    f = bits & 1023
    v = Fraction(f, 1 << 24) if e == 0 else Fraction(1024 + f) * Fraction(2) ** (e - 25)
    return -v if s else v


def _nearest_f32(fr: Fraction) -> np.float32:
    # Exact value has <= 50 significant bits, so fp64 holds it exactly and the
    # fp64 -> fp32 cast is the only rounding (round to nearest even).
    f64 = float(fr)
    assert Fraction(f64) == fr
    return np.float32(f64)


def test_q4_k_exact_rationals(orc):
    """Random blocks, including subnormal and extreme exponents, against exact
    rational arithmetic with the layout walked independently of the oracle."""
    g = np.random.default_rng(1234)
    nblk = 96
    raw = synth.q4_k_matrix(nblk, 256, seed=7, tensor_id=99).reshape(nblk, 144).copy()
    edge = [0x0001, 0x03FF, 0x0400, 0x7BFF, 0x1C00, 0x3C00, 0x0000, 0x2E66]
    for i in range(nblk):
        if i % 3 == 0:
            for off in (0, 2):
                h = edge[g.integers(len(edge))] if g.random() < 0.5 else int(g.integers(0, 0x7C00))
                raw[i, off] = h & 255
                raw[i, off + 1] = h >> 8
    w = orc.dequant(orc.Q4_K, raw, nblk, 256)
    table = _bit_map()
    for i in range(nblk):
        blk = raw[i]
        d = _half_fraction(int(blk[0]) | int(blk[1]) << 8)
        dm = _half_fraction(int(blk[2]) | int(blk[3]) << 8)
        sc, m = _extract(table, [int(v) for v in blk[4:16]])
        qs = blk[16:]
        for c in range(4):
            for hi in range(2):
                j = 2 * c + hi
                for l in range(32):
                    byte = int(qs[32 * c + l])
                    q = (byte >> 4) if hi else (byte & 15)
                    ref = _nearest_f32(d * sc[j] * q - dm * m[j])
                    got = w[i, 64 * c + 32 * hi + l]
                    assert got.view(np.uint32) == ref.view(np.uint32) or (got == 0 and ref == 0), (i, j, l)


def test_q4_k_reduces_to_plain_nibbles(orc):
    """dmin = 0, every sc = 1, d = 1: the weights are the 4-bit quants themselves."""
    g = np.random.default_rng(5)
    raw = np.zeros((16, 144), dtype=np.uint8)
    raw[:, 0:2] = [0x00, 0x3C]
    raw[:, 4:8] = 1
    raw[:, 12:16] = 1
    raw[:, 16:] = g.integers(0, 256, size=(16, 128), dtype=np.uint8)
    w = orc.dequant(orc.Q4_K, raw, 16, 256)
    for i in range(16):
        qs = raw[i, 16:]
        lo = (qs & 15).astype(np.float32)
        hi = (qs >> 4).astype(np.float32)
        ref = np.concatenate([np.concatenate([lo[32 * c:32 * c + 32], hi[32 * c:32 * c + 32]]) for c in range(4)])
        assert np.array_equal(w[i], ref)


def test_synthetic_distributions(orc):
    """The generator draws what the workloads state: Q8_0 q uniform on [-127,127],
    Q4_K sc/m uniform on 0..63 and q on 0..15; scales are non-negative fp16."""
    q8 = synth.q8_0_matrix(64, 4096, seed=0, tensor_id=1).reshape(-1, 34)
    q = q8[:, 2:].view(np.int8)
    assert q.min() == -127 and q.max() == 127
    d = q8[:, 0:2].copy().view(np.float16).astype(np.float64)
    assert (d >= 0).all() and 0.006 < d.mean() < 0.01
    q4 = synth.q4_k_matrix(256, 2048, seed=0, tensor_id=2).reshape(-1, 144)
    sms = [orc.q4_k_scale_min(bytes(b[4:16])) for b in q4[:512]]
    allv = np.array([v for sc, m in sms for v in sc + m])
    assert allv.min() == 0 and allv.max() == 63 and abs(allv.mean() - 31.5) < 1.5
