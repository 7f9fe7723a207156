"""Seeded randomized parity sweep of the decode-form linear layer (nvfp4_linear
with 1 <= M <= 16): random token counts, K (multiples of 16, most of them not
multiples of the 128-k tile), output widths, module splits, activation
distributions and dynamic or calibrated activation scales -- 40 cases with
K <= 5120 (one launch, eight waves) and 16 with 5120 < K <= 20496 (one launch
where the rows fit, else quantizer + GEMM; sixteen waves per workgroup on
narrow outputs, eight on outputs of at least 256 workgroups).  Each case must be
bit-identical to nvfp4_quantize_act followed by nvfp4_gemm and within the GEMM
tolerance of the oracle (every output of small cases, a sample of columns of
larger ones); the activation codes and scales must equal the oracle's.
"""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_block_act_amd as nv
import workloads as W
from gpu_util import DEV, assert_within_tol, gpu_pack, oracle_linear_rows, say, to_dev_bf16
from oracle import nvfp4 as Q

pytestmark = pytest.mark.gpu

CASES = 40
LONG_CASES = 16


def case(seed, long_k=False):
    rng = np.random.default_rng((9500 if long_k else 9000) + seed)
    M = int(rng.integers(1, 17))
    if long_k:
        K = 16 * int(rng.integers(321, 1282))                  # 5136 .. 20496
        N = int(rng.integers(12256, 13000)) if seed % 4 == 0 else int(rng.integers(1, 3000))
    else:
        K = 16 * int(rng.integers(1, 321))
        N = int(rng.integers(1, 2049))
    nseg = int(rng.integers(1, min(N, 5) + 1))
    cuts = sorted(rng.choice(np.arange(1, N), nseg - 1, replace=False).tolist()) if nseg > 1 else []
    bounds = [0] + cuts + [N]
    segs = list(zip(bounds[:-1], bounds[1:]))
    w = np.concatenate([np.float32(0.03 * (1 + 2 * i)) * rng.standard_normal((e - b, K), dtype=np.float32)
                        for i, (b, e) in enumerate(segs)])
    dist = ("normal", "student_t", "uniform")[seed % 3]
    x = W.random_act(31 * seed + 7, M, K, dist)
    if seed % 5 == 4:   # a few outlier channels, as in real activations
        xf = W.bf16_to_f32(x)
        xf[:, rng.choice(K, max(1, K // 256), replace=False)] *= np.float32(60.0)
        x = W.bf16_bits(xf)
    amax = None
    if seed % 4 == 3:   # calibrated scale, below the tensor's maximum: saturating blocks
        amax = np.float32(float(np.max(np.abs(W.bf16_to_f32(x)))) * float(rng.uniform(0.3, 1.2)))
    return M, K, N, segs, w, x, amax


@pytest.mark.parametrize("seed", range(CASES))
def test_linear_decode_sweep(seed):
    _check(seed, *case(seed))


@pytest.mark.parametrize("seed", range(LONG_CASES))
def test_linear_long_k_sweep(seed):
    _check(seed, *case(seed, long_k=True))


def _check(seed, M, K, N, segs, w, x_bits, amax):
    say(f"[sweep] seed={seed} M={M} K={K} N={N} nseg={len(segs)} static={amax is not None}")
    pw = gpu_pack(w, segs)
    x = to_dev_bf16(x_bits)
    am = None if amax is None else torch.tensor([amax], dtype=torch.float32, device=DEV)
    out, (c, s, g) = nv.linear(x, pw, am, workspace=nv.Workspace(DEV))
    c2, s2, g2 = nv.quantize_act(x, am)
    ref_gpu = nv.gemm(c2, s2, g2, pw)
    torch.cuda.synchronize()
    assert torch.equal(c, c2) and torch.equal(s, s2) and torch.equal(g, g2)
    assert torch.equal(out, ref_gpu), "one-launch result differs from quantize + gemm"
    oc, os_, og, _ = Q.quantize(W.bf16_to_f32(x_bits), amax)
    assert np.array_equal(c.cpu().numpy(), oc) and np.array_equal(s.cpu().numpy(), os_)
    assert float(g.cpu()[0]) == float(og)
    cols = None if N * K <= 4_000_000 else np.sort(np.random.default_rng(seed).choice(N, 256, replace=False))
    ref, bnd = oracle_linear_rows(x_bits, w, segs, cols=cols, amax=amax)
    y = out.cpu().numpy().astype(np.float64)
    if cols is not None:
        y = y[:, cols]
    assert_within_tol(y, ref, bnd, f"sweep seed={seed}")
