"""Pins of oracle/kvfp8.py (CPU).

* Encode matches torch's float32 -> float8_e4m3fn cast (round to nearest
  even) of fl(|x| * g_enc) clamped to 448, on dense sweeps and all ties.
* Round trip: every E4M3 value times g_dec decodes exactly when amax is
  448 * 2^j (the scale is a power of two).
* Saturation, signs (including -0.0), amax == 0, and the bf16 decode against
  torch's float32 -> bfloat16 cast.
"""
import numpy as np
import torch

from oracle import kvfp8 as F
from oracle.formats import e4m3_value


def test_encode_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(300000) * 10.0 ** rng.integers(-4, 3, 300000)).astype(np.float32)
    amax = np.float32(7.3)
    codes = F.encode(x, amax)
    g_enc, _ = F.scales(amax)
    y = np.minimum(np.abs(x) * g_enc, np.float32(448)).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes & 0x7F, ref)
    assert np.array_equal(codes >> 7, np.signbit(x).astype(np.uint8))


def test_ties_round_to_even():
    vals = e4m3_value(np.arange(0x7F)).astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)       # exact in float32
    codes = F.encode(mids, np.float32(448))                          # g_enc = 1
    lo = np.arange(0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(codes, expect.astype(np.uint8))


def test_power_of_two_scale_round_trip_is_exact():
    for j in (-6, 0, 3):
        amax = np.float32(448 * 2.0 ** j)
        codes = np.arange(256, dtype=np.uint8)
        codes = codes[(codes & 0x7F) != 0x7F]
        v = F.decode_f32(codes, amax)
        assert np.array_equal(F.encode(v, amax), np.where(v == 0, codes & 0x80, codes))
        assert np.array_equal(v.astype(np.float64), np.where(codes & 0x80, -1, 1) * e4m3_value(codes & 0x7F) * 2.0 ** j)


def test_saturation_signs_and_zero():
    amax = np.float32(2.0)
    c = F.encode(np.array([5.0, -5.0, 2.0, -0.0, 0.0, 1e-30], np.float32), amax)
    assert c.tolist() == [0x7E, 0xFE, 0x7E, 0x80, 0x00, 0x00]
    assert F.encode(np.array([1.0, -1.0], np.float32), 0.0).tolist() == [0x00, 0x80]
    assert np.array_equal(F.decode_f32(np.array([0x00, 0x80], np.uint8), 0.0), np.array([0.0, -0.0], np.float32))


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 256, 5000).astype(np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]
    amax = np.float32(3.1)
    f = F.decode_f32(codes, amax)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.decode_bf16(codes, amax), ref)
