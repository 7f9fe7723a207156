"""Readers for the hand-worked fixtures under tests/golden/ and exact fp32 rounding."""
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def parse_value(tok):
    tok = tok.strip()
    if tok.lstrip("-").startswith("0x"):
        return float.fromhex(tok)
    return float(tok)


def parse_rational(tok):
    """'p/q' or 'p/q*2^e' -> Fraction."""
    e = 0
    if "*2^" in tok:
        tok, es = tok.split("*2^")
        e = int(es)
    return Fraction(tok) * (Fraction(2) ** e)


def fp32_round(q):
    """Round a Fraction to the nearest float32 (ties to even), exactly; subnormals included."""
    q = Fraction(q)
    if q == 0:
        return np.float32(0.0)
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = math.floor(math.log2(q.numerator) - math.log2(q.denominator))
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    e = max(e, -126)                      # subnormal spacing below 2^-126
    ulp = Fraction(2) ** (e - 23)
    n = q / ulp
    lo = math.floor(n)
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return np.float32(sign * float(lo * ulp))


def load_quant_fixtures():
    """List of dicts: name, amax (None = dynamic), g_dec (Fraction), x [1, 16*B] float32,
    scales [1, B] uint8, codes [1, 16*B] uint8 (unpacked nibbles), packed [1, 8*B] uint8
    (the stored bytes, as the fixture file writes them out)."""
    out, cur = [], None
    with open(os.path.join(GOLDEN, "quant_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "tensor":
                kv = dict(p.split("=", 1) for p in parts[2:])
                cur = {"name": parts[1],
                       "amax": None if kv["amax"] == "dynamic" else float(kv["amax"]),
                       "g_dec": parse_rational(kv["g_dec"]), "x": [], "scales": [], "codes": [], "packed": []}
            elif parts[0] == "block":
                kv = dict(p.split("=", 1) for p in parts[1:])
                xs = [parse_value(t) for t in kv["x"].split(",")]
                cs = [int(c, 16) for c in kv["codes"]]
                bs = [int(kv["bytes"][2 * j:2 * j + 2], 16) for j in range(len(kv["bytes"]) // 2)]
                assert len(xs) == 16 and len(cs) == 16 and len(bs) == 8
                cur["x"] += xs
                cur["codes"] += cs
                cur["packed"] += bs
                cur["scales"].append(int(kv["scale"], 16))
            elif parts[0] == "end":
                cur["x"] = np.array([cur["x"]], np.float32)
                cur["codes"] = np.array([cur["codes"]], np.uint8)
                cur["scales"] = np.array([cur["scales"]], np.uint8)
                cur["packed"] = np.array([cur["packed"]], np.uint8)
                out.append(cur)
                cur = None
    return out
