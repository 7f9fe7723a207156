"""fp64 and exact-integer GEMM on decoded NVFP4 operands (CPU oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring for who may use it.

The linear layer computes out[m, n] = sum_k a_hat[m, k] * w_hat[n, k], with
a_hat the decoded activations and w_hat the decoded weights, where every row
n of a fused weight is decoded with the FP32 global scale of the module
(segment) it belongs to.  That per-segment scale is the pages' repair of the
global-scale mismatch in fused GEMMs (abstract; Glonce article, "Who it
affects" and "Risks and caveats"; aiany page, "Mechanistic notes"); the
mismatch itself is what one gets by decoding every row with a single scale.

Functions:
    gemm_f64    -- the definition: float64 matmul of the decoded operands.
    gemm_bound  -- sum_k |a_hat| |w_hat|, the scale of the accepted error.
    gemm_exact  -- the same sum computed exactly in int64, then scaled once.
    within_tol  -- the elementwise acceptance test |y - ref| <= rtol*bound + atol.
"""
import numpy as np

from .formats import e2m1_value, e4m3_value
from .nvfp4 import BLOCK, unpack_codes

RTOL = 1e-5
ATOL = 1e-6


def gemm_f64(a_hat, w_hat):
    """out = a_hat @ w_hat.T in float64 ([M, K] x [N, K] -> [M, N])."""
    return np.asarray(a_hat, np.float64) @ np.asarray(w_hat, np.float64).T


def gemm_bound(a_hat, w_hat):
    """sum_k |a_hat[m, k]| * |w_hat[n, k]| in float64."""
    return np.abs(np.asarray(a_hat, np.float64)) @ np.abs(np.asarray(w_hat, np.float64)).T


def _int_operand(packed, scales):
    """Integer image of decoded values: E2M1 * E4M3 * 2^10 (exact, |.| <= 2752512)."""
    codes = unpack_codes(packed)
    R, K = codes.shape
    q2 = np.rint(e2m1_value(codes) * 2).astype(np.int64).reshape(R, K // BLOCK, BLOCK)
    s9 = np.rint(e4m3_value(np.asarray(scales, np.uint8)) * 512).astype(np.int64)
    return (q2 * s9[:, :, None]).reshape(R, K)


def gemm_exact(a_codes, a_scales, a_g, w_codes, w_scales, w_g_rows):
    """Exact sum in int64, one float64 scaling at the end.

    Every E2M1 * E4M3 product is an integer multiple of 2^-10 below 2^22 in
    magnitude, so a K <= 2^19 dot product of two such operands fits int64.
    ``w_g_rows`` is the per-row (per-output-column) global decode scale.
    """
    ia = _int_operand(a_codes, a_scales)
    iw = _int_operand(w_codes, w_scales)
    assert ia.shape[1] <= (1 << 19)
    acc = np.zeros((ia.shape[0], iw.shape[0]), np.int64)
    for k0 in range(0, ia.shape[1], 4096):  # int64 matmul in chunks (no BLAS for ints)
        acc += ia[:, k0:k0 + 4096] @ iw[:, k0:k0 + 4096].T
    scale = np.float64(np.float32(a_g)) * np.asarray(w_g_rows, np.float64)[None, :] * 2.0 ** -20
    return acc.astype(np.float64) * scale


def within_tol(y, ref, bound, rtol=RTOL, atol=ATOL):
    """Elementwise acceptance mask |y - ref| <= rtol * bound + atol."""
    return np.abs(np.asarray(y, np.float64) - ref) <= rtol * bound + atol
