"""Reader for the hand-built block fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _values(tokens):
    out = []
    for t in tokens:
        if "*" in t:
            v, n = t.split("*")
            out.extend([_num(v)] * int(n))
        else:
            out.append(_num(t))
    return out


def _num(t):
    if "0x" in t:
        return float.fromhex(t)
    return float(t)


def _blocks(name):
    blocks, cur = [], {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if line.startswith("#"):
                continue
            if not line:
                if cur:
                    blocks.append(cur)
                cur = {}
                continue
            key, rest = line.split(None, 1)
            cur[key] = rest.split()
    if cur:
        blocks.append(cur)
    return blocks


def q8_0_blocks():
    """[(34 raw bytes, 32 expected float32)]"""
    out = []
    for b in _blocks("q8_0_blocks.txt"):
        d = int(b["d"][0], 16)
        q = [int(v) for v in b["q"]]
        raw = bytes([d & 255, d >> 8]) + bytes([v & 255 for v in q])
        out.append((raw, np.array(_values(b["w"]), dtype=np.float32), q))
    return out


def q4_k_blocks():
    """[(144 raw bytes, 256 expected float32, sc list, m list)]"""
    out = []
    for b in _blocks("q4_k_blocks.txt"):
        d = int(b["d"][0], 16)
        dm = int(b["dmin"][0], 16)
        s = bytes(int(v, 16) for v in b["s"])
        rule = b["qs"]
        if rule[0] == "pattern_a":
            qs = bytes(((i % 16) | ((15 - i % 16) << 4)) for i in range(128))
        elif rule[0] == "const":
            qs = bytes([int(rule[1], 16)] * 128)
        elif rule[0] == "index":
            qs = bytes(range(128))
        else:
            raise ValueError(rule)
        raw = bytes([d & 255, d >> 8, dm & 255, dm >> 8]) + s + qs
        assert len(raw) == 144
        w = []
        for j in range(8):
            vals = _values(b[f"w{j}"])
            assert len(vals) == 32, (j, len(vals))
            w.extend(vals)
        out.append((raw, np.array(w, dtype=np.float32),
                    [int(v) for v in b["sc"]], [int(v) for v in b["m"]]))
    return out
