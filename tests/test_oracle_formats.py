"""Pins for oracle/formats.py: code tables and the two RNE encoders.

Each table is checked against a computation that does not share the oracle's
code: exact rationals from the bit fields, and torch's float8_e4m3fn type.
The encoders are checked against torch's fp32 -> float8_e4m3fn cast and
against a brute-force nearest-value search with an explicit tie rule.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from workloads import bf16_to_f32


def frac_e2m1(c):
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return -mag if s else mag


def frac_e4m3(c):
    s, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
    if e == 15 and m == 7:
        return None
    mag = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else Fraction(2) ** (e - 7) * (1 + Fraction(m, 8))
    return -mag if s else mag


def test_e2m1_table_from_bit_fields():
    vals = F.e2m1_value(np.arange(16))
    for c in range(16):
        assert Fraction(float(vals[c])) == frac_e2m1(c)
    # largest magnitude is 6: the divisor the block-scale rule uses
    assert np.max(np.abs(vals)) == 6.0 == F.E2M1_MAX


def test_e4m3_table_from_bit_fields_and_torch():
    vals = F.e4m3_value(np.arange(256))
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for c in range(256):
        fr = frac_e4m3(c)
        if fr is None:
            assert np.isnan(vals[c]) and np.isnan(ref[c])
        else:
            assert Fraction(float(vals[c])) == fr
            assert vals[c] == ref[c] or (vals[c] == 0 and ref[c] == 0)
    assert F.E4M3_POS[-1] == 448.0 and F.E4M3_POS[F.E4M3_MAX_CODE] == 448.0
    assert np.all(np.diff(F.E4M3_POS) > 0)


def test_all_code_pairs_products_exact_and_fp16_representable():
    """All 16 E2M1 codes x 256 E4M3 codes: the oracle's float64 product is the exact
    rational product; every finite product has <= 6 significant bits, lies in
    [2^-10, 2688] when nonzero, and is exactly representable in IEEE fp16."""
    e2 = F.e2m1_value(np.arange(16))
    e4 = F.e4m3_value(np.arange(256))
    for c in range(16):
        for s in range(256):
            fr = frac_e4m3(s)
            if fr is None:
                continue
            v = e2[c] * e4[s]
            assert Fraction(float(v)) == frac_e2m1(c) * fr
            if v != 0:
                a = abs(Fraction(float(v)))
                assert Fraction(1, 1024) <= a <= 2688
                n, d = a.numerator, a.denominator
                assert d & (d - 1) == 0            # dyadic
                assert n.bit_length() - (len(bin(n)) - len(bin(n).rstrip("0"))) <= 6
                assert float(np.float16(v)) == v


def test_e4m3_encode_exhaustive_bf16_vs_torch():
    bits = np.arange(0, 0x7F81, dtype=np.uint32).astype(np.uint16)   # every non-negative finite bf16, and +inf
    s = bf16_to_f32(bits)
    got = F.e4m3_encode(s)
    ref = torch.from_numpy(np.minimum(s, np.float32(448))).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_e4m3_encode_dense_fp32_vs_torch():
    lo, hi = 0, np.float32(480).view(np.uint32)
    pats = np.arange(lo, hi, 401, dtype=np.uint32)
    # plus every midpoint between neighbouring codes and the 4 fp32 values on each side of it
    mids = (F.E4M3_POS[:-1] + F.E4M3_POS[1:]) / 2
    mb = np.float32(mids).view(np.uint32)
    near = (mb[:, None] + np.arange(-4, 5, dtype=np.int64)[None, :]).astype(np.uint32).ravel()
    allp = np.concatenate([pats, near, np.float32(F.E4M3_POS).view(np.uint32)])
    s = allp.view(np.float32)
    got = F.e4m3_encode(s)
    ref = torch.from_numpy(np.minimum(s, np.float32(448))).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("s,code", [
    (1.0625, 0x38), (1.1875, 0x3A), (464.0, 0x7E), (447.0, 0x7E), (1e30, 0x7E), (np.inf, 0x7E),
    (2.0 ** -10, 0x00), (1.5 * 2 ** -10, 0x01), (7.5 * 2 ** -9, 0x08), (0.0, 0x00), (2.0 ** -6, 0x08),
])
def test_e4m3_encode_spot_values(s, code):
    assert int(F.e4m3_encode(np.float32(s))) == code


def brute_e2m1(y):
    """Nearest E2M1 magnitude code by exhaustive search with exact rationals, ties to even code."""
    if y == np.inf or y >= 6:
        return 7
    fy = Fraction(float(y))
    best, bd = None, None
    for c in range(8):
        d = abs(fy - frac_e2m1(c))
        if bd is None or d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    return best


def test_e2m1_encode_boundaries_vs_brute_force():
    thresholds = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]
    ys = []
    for t in thresholds:
        b = int(np.float32(t).view(np.uint32))
        ys += [np.uint32(b + d).view(np.float32) for d in range(-3, 4)]
    ys += [np.float32(v) for v in (0.0, 1e-45, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 7.99, 1e30)]
    ys = np.array(ys, np.float32)
    got = F.e2m1_encode(ys)
    for y, g in zip(ys, got):
        assert g == brute_e2m1(y), y
    assert int(F.e2m1_encode(np.float32(np.inf))) == 7


def test_e2m1_encode_strided_sweep_vs_nearest():
    """Every 251st float32 pattern in [0, 8]: compare with an argmin over exact float64 distances."""
    pats = np.arange(0, np.float32(8).view(np.uint32) + 1, 251, dtype=np.uint32)
    y = pats.view(np.float32)
    got = F.e2m1_encode(y)
    d = np.abs(y.astype(np.float64)[:, None] - F.E2M1_MAG[None, :])
    best = np.argmin(d, axis=1)             # first index wins ties: fix ties explicitly below
    dmin = d[np.arange(len(y)), best]
    tie = np.sum(d == dmin[:, None], axis=1) > 1
    best = np.where(tie & (best % 2 == 1), best + 1, best)
    best = np.where(y >= 6, 7, best)
    assert np.array_equal(got, best.astype(np.uint8))
