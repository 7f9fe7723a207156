"""Calibrated FP8 (E4M3) KV-cache codec with one scale per tensor (CPU oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring for who may use it.

The pages serve the quantized model with its attention KV cache in FP8, with
calibrated per-tensor scales (paper abstract; Glonce article, "How to use it";
aiany page, "Mechanistic notes").  They do not spell the codec out; the
plain reading, built like the NVFP4 per-tensor scale:

  * E4M3 is the OCP E4M3FN format (largest finite value 448);
  * a calibrated maximum amax of |x| maps onto 448: g_enc = fl(448 / amax),
    g_dec = fl(amax / 448); amax == 0 encodes every element as its sign bit;
  * encode: code = sign(x) << 7 | E4M3 round-to-nearest-even, saturating at
    448, of fl(|x| * g_enc) (|x| above amax saturates);
  * decode to the attention's bf16 input: bf16 RNE of fl(E4M3(code) * g_dec),
    the product taken in binary32.

fl = one IEEE binary32 operation; bf16 inputs widen to binary32 exactly.
"""
import numpy as np

from .formats import e4m3_encode, e4m3_value

FP8_MAX = np.float32(448.0)


def scales(amax):
    amax = np.float32(amax)
    if amax == 0:
        return np.float32(0), np.float32(0)
    return np.float32(FP8_MAX / amax), np.float32(amax / FP8_MAX)


def encode(x, amax):
    """float32 array -> uint8 E4M3FN codes with the calibrated scale."""
    x = np.asarray(x, np.float32)
    g_enc, _ = scales(amax)
    sign = (np.signbit(x).astype(np.uint8) << 7)
    if g_enc == 0:
        return sign
    with np.errstate(over="ignore"):
        y = (np.abs(x) * g_enc).astype(np.float32)
    return sign | e4m3_encode(y).astype(np.uint8)


def decode_f32(codes, amax):
    """Codes -> binary32 fl(E4M3 * g_dec) (sign applied)."""
    codes = np.asarray(codes, np.uint8)
    _, g_dec = scales(amax)
    mag = e4m3_value(codes & 0x7F).astype(np.float32)
    v = (mag * g_dec).astype(np.float32)
    return np.where(codes & 0x80, -v, v).astype(np.float32)


def bf16_bits_of_f32(v):
    """bf16 RNE bit patterns of finite binary32 values."""
    b = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def decode_bf16(codes, amax):
    return bf16_bits_of_f32(decode_f32(codes, amax))
