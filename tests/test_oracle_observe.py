"""Pins of oracle/observe.py (CPU): hand-worked blocks where g_enc and the
scales are exact, and the equivalence of the saturation tests with what the
encoder emits."""
import numpy as np

from oracle import nvfp4 as Q
from oracle import observe as O


def test_running_amax_is_the_max_over_batches():
    rng = np.random.default_rng(0)
    bs = [rng.standard_normal((4, 32)).astype(np.float32) * (i + 1) for i in range(5)]
    assert O.running_amax(bs) == np.float32(max(np.max(np.abs(b)) for b in bs))
    assert O.running_amax(bs[::-1]) == O.running_amax(bs)
    assert O.running_amax([], 2.5) == np.float32(2.5) and O.running_amax(bs[:1], 1e9) == np.float32(1e9)


def test_hand_worked_blocks():
    # amax = 6: g_enc = 448 exactly.  Block max 6 -> t = 1, s = 448: not saturated.
    # Block max 7.5 -> s = 560 > 448: saturated; the scale clamps to 448, rb = 1, so
    # y = |x|: 6.5 still rounds to 6 (not clipped), -7.0 and 7.5 reach 7 (clipped).
    # A block with max 3 -> s = 224.
    x = np.zeros((1, 48), np.float32)
    x[0, :16] = np.linspace(-6, 6, 16)
    x[0, 16:32] = 1.0
    x[0, 16], x[0, 17], x[0, 18] = 6.5, -7.0, 7.5
    x[0, 32:48] = 3.0
    sat, clip = O.saturation_counts(x, 6.0)
    assert (sat, clip) == (1, 2)
    # dynamic maximum of the same tensor (7): nothing saturates or clips
    assert O.saturation_counts(x, np.max(np.abs(x))) == (0, 0)


def test_clipping_needs_saturation_or_a_subnormal_scale():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((128, 512)) * 10.0 ** rng.integers(-1, 2, (128, 1))).astype(np.float32)
    assert O.saturation_counts(x, np.max(np.abs(x))) == (0, 0)       # normal-range block scales
    x[:64] *= np.float32(1e-5)                                         # these rows get subnormal scales
    sat, clip = O.saturation_counts(x, np.max(np.abs(x)))
    assert sat == 0 and clip > 0


def test_clipped_elements_encode_to_magnitude_6():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    x[5, 7] = 40.0
    amax = np.float32(8.0)
    sat, clip = O.saturation_counts(x, amax)
    assert sat >= 1 and clip >= 1
    codes = Q.unpack_codes(Q.quantize(x, amax)[0]) & 7
    assert codes[5, 7] == 7                         # magnitude code of 6
    assert np.sum(codes == 7) >= clip
