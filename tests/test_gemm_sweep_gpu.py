"""Seeded randomized parity sweep of nvfp4_gemm with M > 16 in both of its
forms -- the MFMA GEMM and the weight-streaming GEMM over 32- or 64-row blocks (the form is
asserted per case) -- over random M, K (multiples of 16, most of them ragged
against the 128-k tile), N (ragged against the 256-column tile), module splits
and activation distributions, against the oracle (all outputs, or a sample of
rows for the largest cases); and the fused gate+up SwiGLU -> NVFP4 epilogue over
random shapes, bit-identical to the unfused kernels (each checked against the
oracle in its own tests).
"""
import numpy as np
import pytest

import nvfp4_w4a4_block_act_amd as nv
import workloads as W
from gpu_util import assert_within_tol, gpu_pack, oracle_linear_rows, say, to_dev_bf16
from test_swiglu_gpu import _run as swiglu_fused_vs_unfused

pytestmark = pytest.mark.gpu


def _sweep_case(seed, form):
    """A seeded random shape for which nvfp4_gemm takes `form` (1: MFMA GEMM with
    256 x 256 tiles, 2: with 256 x 128 tiles, 0: weight-streaming GEMM over row
    blocks), with 1-5 modules and a ragged k tile."""
    rng = np.random.default_rng(7000 + seed)
    while True:
        if form >= 1:
            M, N = int(rng.integers(300, 1200)), int(rng.integers(2000, 9000))
        else:
            M, N = int(rng.integers(17, 400)), int(rng.integers(1, 1500))
        K = 16 * int(rng.integers(1, 200))
        if nv.nvfp4_gemm_form(M, K, N) == form:
            return rng, M, K, N


@pytest.mark.parametrize("form", [1, 2, 0])
@pytest.mark.parametrize("seed", range(12))
def test_gemm_rows_sweep(seed, form):
    rng, M, K, N = _sweep_case(seed, form)
    nseg = int(rng.integers(1, min(N, 6) + 1))
    cuts = sorted(rng.choice(np.arange(1, N), nseg - 1, replace=False).tolist()) if nseg > 1 else []
    bounds = [0] + cuts + [N]
    segs = list(zip(bounds[:-1], bounds[1:]))
    w = np.concatenate([(0.02 * (1 + i) * rng.standard_normal((e - b, K))).astype(np.float32)
                        for i, (b, e) in enumerate(segs)])
    x_bits = W.random_act(17 * seed + 3, M, K, ("normal", "student_t", "uniform")[seed % 3])
    say(f"[gemm sweep] form={form} seed={seed} M={M} K={K} N={N} nseg={nseg}")
    pw = gpu_pack(w, segs)
    c, s, g = nv.quantize_act(to_dev_bf16(x_bits))
    out = nv.gemm(c, s, g, pw).cpu().numpy().astype(np.float64)
    rows = None if M * N * K <= 300_000_000 else np.sort(rng.choice(M, 48, replace=False))
    ref, bnd = oracle_linear_rows(x_bits, w, segs, rows=rows)
    assert_within_tol(out if rows is None else out[rows], ref, bnd, f"gemm sweep form={form} seed={seed}")


@pytest.mark.parametrize("seed", range(6))
def test_swiglu_fused_sweep(seed):
    rng = np.random.default_rng(8000 + seed)
    M = int(rng.integers(17, 600))
    K = 16 * int(rng.integers(1, 160))
    I = 128 * int(rng.integers(1, 5))
    swiglu_fused_vs_unfused(M, K, I, 500 + seed, (1.0, 0.5)[seed % 2])
