"""NVFP4 tensor encode / decode, step by step (CPU oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring for who may use it.

What the pages fix (Summary page, Background, item 1): an NVFP4 tensor is
E2M1 element codes, one E4M3 scale per 16-element block derived from the block
maximum divided by 6, and one FP32 scale for the whole tensor.  Everything
else below is a reading, chosen as the plainest one consistent with that
sentence:

* The 16-element blocks run along the last (contraction) axis K of a
  row-major [R, K] tensor -- the only axis on which a block scale can be pulled
  out of a dot product.  K must be a multiple of 16.
* The FP32 per-tensor scale maps the tensor's absolute maximum onto 6 * 448 =
  2688, the largest magnitude an E2M1 value times an E4M3 scale can hold, so
  the block holding the tensor maximum gets the largest E4M3 scale.  The
  decode factor is g_dec = amax / 2688 and the encode factor g_enc =
  2688 / amax.  The maximum is the tensor's own (dynamic) unless the caller
  supplies a calibrated one (static); the abstract and the aiany page
  ("Who it's for") describe calibration-only post-training quantization.
* "Block maximum" is the maximum of |x| over the block; "/6" divides it by
  the largest E2M1 magnitude.

Arithmetic (fl = one IEEE binary32 operation rounded to nearest even; no fused
multiply-add; bf16 inputs are widened to float32 exactly):

  1. amax = max |x| (or the supplied value).
  2. amax == 0: g_dec = 0, every scale code 0x00, every element code is its
     sign bit alone.  Otherwise g_enc = fl(2688 / amax), g_dec =
     fl(amax / 2688).
  3. per block: bmax = max |x|; t = fl(bmax / 6); s = fl(t * g_enc);
     scale code = E4M3 RNE-saturating encode of s, except t == 0 gives 0x00;
     s_dec = the code's value.
  4. per element: s_dec == 0 or x == 0 gives magnitude code 0; otherwise
     rb = fl(g_enc / s_dec) (once per block), y = fl(|x| * rb), magnitude
     code = E2M1 RNE-saturating encode of y.  Element code = sign(x) << 3 |
     magnitude code (the sign of -0.0 is kept).
  5. pack two element codes per byte, the even k in the low nibble; scales
     are [R, K/16] row-major bytes.

The t == 0 and x == 0 rules only matter when g_enc or rb overflows to +inf
(tensors whose maximum is below ~1e-35); for every other input they agree
with plain IEEE arithmetic.  Non-finite inputs are outside the contract.

Decoding (exact): x_hat = (-1)^sign * E2M1(mag) * E4M3(scale) * g_dec,
evaluated in float64; the product of the first two factors has at most six
significant bits, so the float64 result is exact.
"""
import numpy as np

from .formats import e2m1_encode, e2m1_value, e4m3_encode, e4m3_value

BLOCK = 16
G_MAX = np.float32(6.0 * 448.0)  # 2688


def quantize(x, amax=None):
    """Encode a float32 [R, K] tensor to NVFP4.

    Returns (codes uint8 [R, K/2], scales uint8 [R, K/16], g_dec float32,
    amax float32).  ``amax=None`` uses max|x| (dynamic); otherwise the given
    calibrated value (static), which may be smaller than max|x| -- then the
    E4M3 and E2M1 encoders saturate.
    """
    f32 = np.float32
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.ndim == 2 and x.shape[1] % BLOCK == 0
    assert np.all(np.isfinite(x)), "non-finite inputs are outside the contract"
    R, K = x.shape
    if amax is None:
        amax = f32(np.max(np.abs(x))) if x.size else f32(0)
    amax = f32(amax)
    assert np.isfinite(amax) and amax >= 0
    sign = np.signbit(x).astype(np.uint8)
    blocks = np.abs(x).reshape(R, K // BLOCK, BLOCK)

    if amax == 0:
        g_dec = f32(0)
        scode = np.zeros((R, K // BLOCK), np.uint8)
        mag = np.zeros((R, K // BLOCK, BLOCK), np.uint8)
    else:
        with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
            g_enc = G_MAX / amax                       # step 2
            g_dec = amax / G_MAX
            bmax = blocks.max(axis=2)                  # step 3
            t = bmax / f32(6)
            s = t * g_enc
            scode = np.where(t == 0, 0, e4m3_encode(np.where(t == 0, 0, s))).astype(np.uint8)
            s_dec = e4m3_value(scode).astype(np.float32)
            nz = s_dec > 0                             # step 4
            rb = np.where(nz, g_enc / np.where(nz, s_dec, f32(1)), f32(0)).astype(np.float32)
            y = blocks * rb[:, :, None]
            y = np.where(blocks == 0, f32(0), y)
            mag = e2m1_encode(y)
            mag = np.where(nz[:, :, None], mag, 0).astype(np.uint8)
    codes = (sign.reshape(R, K // BLOCK, BLOCK) << 3) | mag
    codes = codes.reshape(R, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)  # step 5
    return packed, scode, f32(g_dec), amax


def unpack_codes(packed):
    """[R, K/2] packed bytes -> [R, K] 4-bit codes (even k from the low nibble)."""
    packed = np.asarray(packed, dtype=np.uint8)
    R, H = packed.shape
    out = np.empty((R, 2 * H), np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def dequantize(packed, scales, g_dec):
    """Decode NVFP4 back to float64 [R, K]: sign * E2M1 * E4M3 * g_dec (exact)."""
    codes = unpack_codes(packed)
    R, K = codes.shape
    sv = e4m3_value(np.asarray(scales, dtype=np.uint8)).reshape(R, K // BLOCK, 1)
    v = e2m1_value(codes).reshape(R, K // BLOCK, BLOCK) * sv
    return v.reshape(R, K) * np.float64(np.float32(g_dec))


def quantize_segments(w, segments):
    """Quantize the rows of a fused weight [N, K] module by module.

    ``segments`` is a list of (n_begin, n_end) covering [0, N) in order; each
    segment is one separately calibrated module with its own amax and FP32
    global scale (the abstract and the Glonce article, "Who it affects":
    per-module calibration).  Returns (codes [N, K/2], scales [N, K/16],
    g_dec float32 [nseg]).
    """
    w = np.asarray(w, dtype=np.float32)
    codes, scales, gs = [], [], []
    pos = 0
    for b, e in segments:
        assert b == pos and e > b
        c, s, g, _ = quantize(w[b:e])
        codes.append(c)
        scales.append(s)
        gs.append(g)
        pos = e
    assert pos == w.shape[0]
    return np.concatenate(codes), np.concatenate(scales), np.array(gs, np.float32)


def dequantize_segments(codes, scales, g_dec, segments):
    """Decode a per-segment-scaled weight to float64 [N, K]."""
    parts = [dequantize(codes[b:e], scales[b:e], g_dec[i]) for i, (b, e) in enumerate(segments)]
    return np.concatenate(parts)
