"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module only draws random numbers and casts them to bf16 -- it holds
none of the quantizer's or the GEMM's arithmetic, so both the HIP path and
the CPU oracle can consume its outputs without sharing any of the method.

The pages evaluate on a 27B hybrid model and public benchmarks that are not
available here; these tensors stand in for that model's projections, with
the shapes and value distributions of the five workloads below.  Every
generator uses ``numpy.random.default_rng(seed)`` (seed 0 by default) and
draws in a fixed order: outlier channel indices, then activations, then
weights segment by segment.  bf16 values are the round-to-nearest-even cast
of the float32 draws (``torch.Tensor.to(torch.bfloat16)`` on the CPU), kept as
raw uint16 bit patterns.
"""
from dataclasses import dataclass, field

import numpy as np
import torch


def bf16_bits(x):
    """float32 ndarray -> uint16 bf16 bit patterns (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(bits):
    """uint16 bf16 bit patterns -> float32 (exact widening)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    """One linear-layer workload: bf16 activations, fp32 weights, segment table."""
    name: str
    x_bits: np.ndarray            # uint16 [M, K] bf16 patterns
    w: np.ndarray                 # float32 [N, K]
    segments: list                # [(n_begin, n_end), ...] covering [0, N)
    info: dict = field(default_factory=dict)

    @property
    def M(self):
        return self.x_bits.shape[0]

    @property
    def K(self):
        return self.x_bits.shape[1]

    @property
    def N(self):
        return self.w.shape[0]


def _outlier_normal(rng, M, K, n_out, factor):
    idx = rng.choice(K, n_out, replace=False)
    x = rng.standard_normal((M, K), dtype=np.float32)
    x[:, idx] *= np.float32(factor)
    return x, idx


def _weights(rng, sizes, K, factors=None):
    parts, segs, pos = [], [], 0
    for i, n in enumerate(sizes):
        f = 1.0 if factors is None else factors[i]
        parts.append((np.float32(0.02 * f) * rng.standard_normal((n, K), dtype=np.float32)))
        segs.append((pos, pos + n))
        pos += n
    return np.concatenate(parts), segs


def tiny(seed=0):
    """16x256 activations N(0,1) with 2 outlier channels x50; 128x256 weights N(0, 0.02)."""
    rng = np.random.default_rng(seed)
    x, idx = _outlier_normal(rng, 16, 256, 2, 50.0)
    w, segs = _weights(rng, [128], 256)
    return Workload("tiny_m16_k256_n128", bf16_bits(x), w, segs, {"outlier_channels": idx.tolist()})


def decode(seed=0, M=16):
    """Decode skinny GEMM, K=5120, N=12288.

    Activations are Student-t (3 degrees of freedom) with 0.1% of the channels
    (5 of 5120) scaled x100; the M=1 and M=4 cases are the leading rows of the
    M=16 draw, so all three share one weight tensor.
    """
    K, N = 5120, 12288
    rng = np.random.default_rng(seed)
    idx = rng.choice(K, 5, replace=False)
    x = rng.standard_t(3, size=(16, K)).astype(np.float32)
    x[:, idx] *= np.float32(100.0)
    w, segs = _weights(rng, [N], K)
    return Workload(f"decode_m{M}_k5120_n12288", bf16_bits(x[:M]), w, segs,
                    {"outlier_channels": idx.tolist()})


def prefill_gate_up(seed=0, M=8192):
    """Fused gate+up projection: M x 5120 activations, two 17408-row modules."""
    K = 5120
    rng = np.random.default_rng(seed)
    x, idx = _outlier_normal(rng, M, K, 2, 50.0)
    w, segs = _weights(rng, [17408, 17408], K)
    return Workload(f"prefill_gate_up_m{M}_k5120_n34816", bf16_bits(x), w, segs,
                    {"outlier_channels": idx.tolist(), "modules": ["gate", "up"]})


GDN_SEGMENTS = [("q", 2048, 1.0), ("k", 2048, 1.0), ("v", 4096, 0.5),
                ("z", 4096, 2.0), ("beta", 32, 10.0), ("alpha", 32, 0.5)]


def gdn_in_proj(seed=0, M=4096):
    """Fused Gated-DeltaNet input projection: six modules with different scales.

    Module weights are 0.02 * N(0,1) * f with f = (1, 1, 0.5, 2, 10, 0.5), so
    the modules' maxima differ by up to ~20x and each carries its own scale.
    """
    K = 5120
    rng = np.random.default_rng(seed)
    x, idx = _outlier_normal(rng, M, K, 2, 50.0)
    w, segs = _weights(rng, [n for _, n, _ in GDN_SEGMENTS], K, [f for _, _, f in GDN_SEGMENTS])
    return Workload(f"gdn_in_proj_m{M}_k5120_n12352", bf16_bits(x), w, segs,
                    {"outlier_channels": idx.tolist(), "modules": [s for s, _, _ in GDN_SEGMENTS]})


def swiglu_rows(rng, rows, K):
    """bf16(silu(g) * u) for bf16 g, u ~ N(0,1), computed in float32."""
    g = bf16_to_f32(bf16_bits(rng.standard_normal((rows, K), dtype=np.float32)))
    u = bf16_to_f32(bf16_bits(rng.standard_normal((rows, K), dtype=np.float32)))
    with np.errstate(over="ignore"):
        act = (g / (np.float32(1) + np.exp(-g))) * u
    return bf16_bits(act.astype(np.float32))


def decode_down_proj(seed=0, M=16):
    """Down projection at decode: M x 17408 SwiGLU activations, 5120 x 17408 weights.

    The M=1 and M=4 cases are the leading rows of the M=16 draw (g then u),
    then the weights, as in ``down_proj``.
    """
    K, N = 17408, 5120
    rng = np.random.default_rng(seed)
    x = swiglu_rows(rng, 16, K)
    w, segs = _weights(rng, [N], K)
    return Workload(f"decode_down_proj_m{M}_k17408_n5120", x[:M], w, segs)


def down_proj(seed=0, M=32768, chunk=2048):
    """Long-context down projection: M x 17408 SwiGLU activations, 5120 x 17408 weights.

    Rows are drawn in chunks of ``chunk`` (g then u per chunk), then weights.
    """
    K, N = 17408, 5120
    rng = np.random.default_rng(seed)
    x = np.empty((M, K), np.uint16)
    for r0 in range(0, M, chunk):
        x[r0:r0 + chunk] = swiglu_rows(rng, min(chunk, M - r0), K)
    w, segs = _weights(rng, [N], K)
    return Workload(f"down_proj_m{M}_k17408_n5120", x, w, segs)


def random_act(seed, M, K, dist="normal", scale=1.0):
    """Small random bf16 activations for edge-case tests."""
    rng = np.random.default_rng(seed)
    if dist == "normal":
        x = rng.standard_normal((M, K), dtype=np.float32)
    elif dist == "student_t":
        x = rng.standard_t(3, size=(M, K)).astype(np.float32)
    elif dist == "uniform":
        x = rng.uniform(-1, 1, size=(M, K)).astype(np.float32)
    else:
        raise ValueError(dist)
    return bf16_bits(x * np.float32(scale))


def random_weight(seed, N, K, scale=0.02):
    rng = np.random.default_rng(seed)
    return (np.float32(scale) * rng.standard_normal((N, K), dtype=np.float32))
