"""SwiGLU of a fused gate+up projection, rounded to bf16 (CPU oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring for who may use it.

The pages quantize every linear layer of the model to NVFP4 W4A4, so the
down projection's input -- the SwiGLU of the gate and up projections -- is
quantized on the fly like any other activation (paper abstract; Glonce
article, "How to use it").  The plain reading of that input, as an unfused
pipeline would produce it: the gate+up GEMM yields g and u (FP32), the MLP
forms h = silu(g) * u with silu(z) = z / (1 + e^-z), and h is stored in bf16
(round to nearest even) before it is quantized with the down projection's
activation scale.  A calibrated (static) activation maximum is what lets a
kernel fuse this into the GEMM's epilogue; with a dynamic one the whole h
must exist first.

Here silu and the product are evaluated in float64 and rounded once to bf16;
a float32 implementation of the same formula can differ by one bf16 unit in
the last place where h lies within float32 rounding of a bf16 midpoint.
"""
import numpy as np


def silu(z):
    """z / (1 + e^-z) in float64 (e^-z overflowing to inf gives -0.0 or 0.0)."""
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def bf16_round_bits(v):
    """bf16 bit patterns (uint16) of float64 values: round to float32 first only
    when that is exact-preserving, i.e. round the float64 value to the nearest
    bf16 directly (ties to even), finite inputs only."""
    v = np.asarray(v, np.float64)
    f32 = v.astype(np.float32)
    bits = f32.view(np.uint32).astype(np.uint64)
    # float64 -> float32 can itself round; decide the bf16 rounding on the exact
    # float64 value: candidates are the two bf16 neighbours of f32's truncation.
    lo = (bits & 0xFFFF0000).astype(np.uint32).view(np.float32).astype(np.float64)
    step = np.abs(((bits & 0xFFFF0000) + 0x10000).astype(np.uint32).view(np.float32).astype(np.float64) - lo)
    hi = lo + np.where(v >= 0, step, -step)
    d_lo, d_hi = np.abs(v - lo), np.abs(hi - v)
    lo_bits = (bits >> 16).astype(np.uint32)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo_bits & 1) == 1))
    return np.where(pick_hi, lo_bits + 1, lo_bits).astype(np.uint16)


def swiglu_bf16(g, u):
    """bf16 bits of silu(g) * u, computed in float64 and rounded once."""
    return bf16_round_bits(silu(g) * np.asarray(u, np.float64))
