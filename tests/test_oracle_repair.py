"""Pins of the repair comparison (oracle/repair.py), CPU only.

* Power-of-two scaling invariance: NVFP4 encoding of 2^j * W with its own
  maximum gives exactly 2^j times the decoded values of W (while no scale
  leaves the normal E4M3 range), so the per-segment repair has the SAME
  relative error for modules that are power-of-two multiples of one matrix.
* The shared scale matches per-segment exactly for the module holding the
  largest maximum, and is worse for a module far below it, whose E4M3 block
  scales fall into the subnormal range; at the in-projection's 20x ratio the
  two agree closely.
* The mismatch (one module's scale for all) is off by the scale ratio.
"""
import numpy as np

from oracle import nvfp4 as Q
from oracle import repair as R
import workloads as W


def _case(factors, K=256, n=48, M=24, seed=5):
    rng = np.random.default_rng(seed)
    base = (0.02 * rng.standard_normal((n, K))).astype(np.float32)
    w = np.concatenate([(base * np.float32(f)).astype(np.float32) for f in factors])
    segs = [(i * n, (i + 1) * n) for i in range(len(factors))]
    x = W.bf16_to_f32(W.random_act(seed + 1, M, K, "normal"))
    return x, w, segs


def test_per_segment_error_is_scale_invariant():
    x, w, segs = _case([1.0, 2.0 ** -5, 2.0 ** 3])
    res, _, _ = R.relative_errors(x, w, segs, np.arange(x.shape[0]), np.arange(w.shape[0]))
    e = [r["per_segment"] for r in res]
    assert e[0] > 0 and abs(e[1] - e[0]) <= 1e-12 * e[0] and abs(e[2] - e[0]) <= 1e-12 * e[0]


def test_decoded_weights_scale_exactly_by_powers_of_two():
    x, w, segs = _case([1.0, 2.0 ** -5])
    d = R.decoded_weights(w, segs, np.arange(w.shape[0]), "per_segment")
    assert np.array_equal(d[48:], d[:48] * 2.0 ** -5)


def test_shared_scale_equal_for_largest_module_and_worse_far_below_it():
    x, w, segs = _case([1.0, 2.0 ** -18])
    res, _, _ = R.relative_errors(x, w, segs, np.arange(x.shape[0]), np.arange(w.shape[0]))
    assert res[0]["shared"] == res[0]["per_segment"]
    assert res[1]["shared"] > 5 * res[1]["per_segment"]
    # the small module's block scales are E4M3 subnormals (codes < 8) under the shared scale
    sc = Q.quantize(w[48:], np.float32(np.max(np.abs(w))))[1]
    assert np.all(sc < 8)


def test_weight_errors_isolate_the_repair():
    _, w, segs = _case([1.0, 2.0 ** -5, 2.0 ** -16])
    per = R.weight_errors(w, segs, "per_segment")
    sh = R.weight_errors(w, segs, "shared")
    assert abs(per[1] - per[0]) <= 1e-12 * per[0] and abs(per[2] - per[0]) <= 1e-12 * per[0]
    assert sh[0] == per[0] and sh[1] == per[1]       # normal-range block scales: nothing lost
    assert sh[2] > 1.2 * per[2]                      # subnormal block scales lose mantissa bits


def test_shared_scale_is_close_at_a_20x_ratio():
    x, w, segs = _case([1.0, 0.05])
    res, _, _ = R.relative_errors(x, w, segs, np.arange(x.shape[0]), np.arange(w.shape[0]))
    assert res[1]["shared"] < 1.5 * res[1]["per_segment"]


def test_mismatch_is_off_by_the_scale_ratio():
    x, w, segs = _case([1.0, 2.0 ** -3])
    res, ys, ref = R.relative_errors(x, w, segs, np.arange(x.shape[0]), np.arange(w.shape[0]))
    # module 1 decoded with module 0's scale: 8x too large
    y = ys["mismatch"][:, 48:]
    assert abs(np.sqrt(np.mean(y ** 2)) / np.sqrt(np.mean(ref[:, 48:] ** 2)) - 8.0) < 0.2
    assert res[1]["mismatch"] > 5
