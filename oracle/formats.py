"""E2M1 and E4M3FN code tables and round-to-nearest-even encoders (CPU oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring for who may use it.

The Summary page ("Summary of 'Why Gated DeltaNet Survives 4-Bit
Quantization'", Background, item 1) names the two element formats of NVFP4:
4-bit E2M1 values and an 8-bit E4M3 scale per 16-element block.  It does not
spell out their bit layouts; the reading taken here is the OCP
microscaling definitions (the layouts NVIDIA's NVFP4 uses, which the Glonce
article names as the format's owner):

* E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa, no inf/NaN.
  Magnitudes by 3-bit code: 0, 0.5, 1, 1.5, 2, 3, 4, 6.  The largest, 6, is
  the divisor the Summary page uses for the block scale.
* E4M3FN: bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
  exponent 0 is subnormal (m * 2^-9); 0x7F / 0xFF are NaN; no inf; the
  largest finite magnitude is 448 (0x7E).

Encoders round to the nearest representable magnitude, ties to the code with
an even mantissa (the code's least significant bit), and saturate anything
above the largest finite magnitude (including +inf) to it.  They work on
magnitudes; the caller supplies signs.  Midpoint comparisons are done in
float64, where ``2*v`` and the sum of two neighbouring table values are exact
for every float32 ``v`` in range, so the decision is exact.
"""
import numpy as np

# Magnitude of each 3-bit E2M1 code (the definition above, written out).
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0
E4M3_MAX = 448.0
E4M3_MAX_CODE = 0x7E


def e2m1_value(code):
    """Decode 4-bit E2M1 codes (any integer array, values 0..15) to float64."""
    code = np.asarray(code).astype(np.int64)
    mag = E2M1_MAG[code & 7]
    return np.where((code >> 3) & 1, -mag, mag)


def e4m3_value(code):
    """Decode 8-bit E4M3FN codes to float64 from the bit fields; NaN for 0x7F/0xFF."""
    code = np.asarray(code).astype(np.int64)
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 7
    sub = m * 2.0 ** -9
    nrm = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    mag = np.where(e == 0, sub, nrm)
    mag = np.where((code & 0x7F) == 0x7F, np.nan, mag)
    return np.where(s == 1, -mag, mag)


# The 127 non-negative finite E4M3FN magnitudes, ascending, indexed by code.
E4M3_POS = e4m3_value(np.arange(0x7F))


def _nearest_even(v, table):
    """Index of the entry of ascending ``table`` (table[0] == 0) nearest to v >= 0.

    Ties go to the even index; v at or above table[-1] (and +inf) saturates to
    the last index.  For both tables here the index is the magnitude code, and
    an even code is an even mantissa.
    """
    v = np.asarray(v, dtype=np.float64)
    last = len(table) - 1
    hi = np.clip(np.searchsorted(table, v, side="left"), 1, last)
    lo = hi - 1
    twice = 2.0 * v
    mid2 = table[lo] + table[hi]
    idx = np.where(twice < mid2, lo,
                   np.where(twice > mid2, hi, np.where(lo % 2 == 0, lo, hi)))
    idx = np.where(v >= table[last], last, idx)
    idx = np.where(v <= 0.0, 0, idx)
    return idx.astype(np.uint8)


def e2m1_encode(y):
    """3-bit E2M1 magnitude code of float32 magnitudes y >= 0 (RNE, saturating)."""
    y = np.asarray(y, dtype=np.float32)
    assert not np.any(np.isnan(y)) and not np.any(y < 0)
    return _nearest_even(y, E2M1_MAG)


def e4m3_encode(s):
    """7-bit E4M3FN magnitude code of float32 magnitudes s >= 0 (RNE, saturating to 0x7E)."""
    s = np.asarray(s, dtype=np.float32)
    assert not np.any(np.isnan(s)) and not np.any(s < 0)
    return _nearest_even(s, E4M3_POS)
