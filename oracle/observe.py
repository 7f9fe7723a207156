"""Static (calibrated) activation scales, as post-training quantization ships
them (CPU oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring for who may use it.

The pages' recipe is calibration-only post-training quantization (aiany page,
"Who it's for"; paper abstract): an activation's FP32 per-tensor scale can
come from a maximum observed over calibration batches instead of each
tensor's own maximum.  Readings:

  * the observer keeps the running maximum of |x| over the batches it sees;
  * under a static maximum, a block's scale "saturates" when its unrounded
    value s = fl(fl(bmax / 6) * g_enc) exceeds 448 (the E4M3 encode clamps it),
    and an element is "clipped" when y = fl(|x| * fl(g_enc / s_dec)) reaches 7,
    the midpoint between the largest E2M1 magnitude 6 and the next value the
    grid would have (8): below it, rounding alone gives 6.  A normal E4M3
    scale that rounds down lifts a block's largest y to at most 6 * 17/16, so
    clipping happens in saturated blocks and in blocks whose scale is an E4M3
    subnormal (whose rounding can lose up to a third) -- both in the encoder's
    own binary32 steps (oracle/nvfp4.py).
"""
import numpy as np

from .formats import e4m3_encode, e4m3_value
from .nvfp4 import BLOCK, G_MAX


def running_amax(batches, start=0.0):
    """max(start, max |x| over every batch) as float32."""
    m = np.float32(start)
    for x in batches:
        x = np.asarray(x, np.float32)
        if x.size:
            m = max(m, np.float32(np.max(np.abs(x))))
    return np.float32(m)


def saturation_counts(x, amax):
    """(blocks whose scale saturates, elements clipped) of a float32 [R, K]
    tensor encoded with the static maximum amax; amax == 0 encodes every
    element as its sign bit, so nothing saturates."""
    x = np.asarray(x, np.float32)
    R, K = x.shape
    amax = np.float32(amax)
    if amax == 0 or x.size == 0:
        return 0, 0
    g_enc = np.float32(G_MAX / amax)
    xb = np.abs(x).reshape(R, K // BLOCK, BLOCK)
    bmax = xb.max(axis=2)
    t = (bmax / np.float32(6.0)).astype(np.float32)
    with np.errstate(over="ignore"):
        s = (t * g_enc).astype(np.float32)
    sat_blocks = int(np.sum(s > np.float32(448.0)))
    code = np.where(t == 0, 0, e4m3_encode(np.minimum(s, np.float32(448.0))))
    sdec = e4m3_value(code).astype(np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        rb = np.where(sdec != 0, g_enc / np.where(sdec != 0, sdec, 1), 0).astype(np.float32)
        y = (xb * rb[:, :, None]).astype(np.float32)
    clipped = int(np.sum(y >= np.float32(7.0)))
    return sat_blocks, clipped
