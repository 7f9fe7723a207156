"""GPU parity of nvfp4_linear (quantize + GEMM in one call).  Decode-sized inputs
(M <= 16, K <= 5120) run as one launch in which every GEMM workgroup encodes the
activations itself; its results must be bit-identical to the separate
nvfp4_quantize_act + nvfp4_gemm calls (codes, scales, g_dec and output) and
within tolerance of the oracle.  Larger inputs take the two-kernel route and are
held to the same bar."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_block_act_amd as nv
import workloads as W
from gpu_util import DEV, assert_within_tol, gpu_pack, oracle_linear_rows, say, to_dev_bf16
from oracle import nvfp4 as Q

pytestmark = pytest.mark.gpu


def run_both(x_bits, pw, amax=None, ws=None):
    x = to_dev_bf16(x_bits)
    am = None if amax is None else torch.tensor([amax], dtype=torch.float32, device=DEV)
    ws = ws if ws is not None else nv.Workspace(DEV)
    out, (c, s, g) = nv.linear(x, pw, am, workspace=ws)
    c2, s2, g2 = nv.quantize_act(x, am)
    ref_out = nv.gemm(c2, s2, g2, pw)
    torch.cuda.synchronize()
    assert torch.equal(c, c2) and torch.equal(s, s2) and torch.equal(g, g2)
    assert torch.equal(out, ref_out), "fused result differs from quantize + gemm"
    return out, c.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("M", [1, 4, 16])
def test_linear_decode_full(M):
    d = W.decode(M=M)
    say(f"[linear] decode M={M}")
    pw = gpu_pack(d.w, d.segments)
    ws = nv.Workspace(DEV)
    for rep in range(3):                       # repeated calls give identical results
        out, c, s = run_both(d.x_bits, pw, ws=ws)
    ref, bnd = oracle_linear_rows(d.x_bits, d.w, d.segments)
    assert_within_tol(out.cpu().numpy().astype(np.float64), ref, bnd, f"linear decode M={M}")
    oc, os_, _, _ = Q.quantize(W.bf16_to_f32(d.x_bits))
    assert np.array_equal(c, oc) and np.array_equal(s, os_)


@pytest.mark.parametrize("M,N,K,nseg", [
    (1, 16, 16, 1), (3, 37, 48, 2), (7, 200, 272, 3), (16, 129, 144, 2), (16, 520, 5136, 4), (5, 64, 4112, 1),
    (16, 300, 17408, 2), (2, 40, 160, 1), (8, 100, 5120, 2), (9, 64, 1040, 3), (4, 1000, 5104, 2),
])
def test_linear_ragged(M, N, K, nseg):
    rng = np.random.default_rng(M * 7 + N + K)
    cuts = sorted(rng.choice(np.arange(1, N), nseg - 1, replace=False).tolist()) if nseg > 1 else []
    bounds = [0] + cuts + [N]
    segs = list(zip(bounds[:-1], bounds[1:]))
    w = np.concatenate([(0.02 * (1 + i) * rng.standard_normal((e - b, K))).astype(np.float32)
                        for i, (b, e) in enumerate(segs)])
    x = W.random_act(M + 3 * N, M, K, "student_t")
    say(f"[linear] ragged M={M} N={N} K={K}")
    pw = gpu_pack(w, segs)
    out, _, _ = run_both(x, pw)
    ref, bnd = oracle_linear_rows(x, w, segs)
    assert_within_tol(out.cpu().numpy().astype(np.float64), ref, bnd, f"linear ragged {M}x{K}x{N}")


@pytest.mark.parametrize("M", [1, 2, 4, 5, 8, 9, 16])
def test_linear_static_amax_each_row_bound(M):
    """The one-launch kernel has one instantiation per row bound (1, 4, 8, 16):
    a calibrated amax below the tensor's (saturating blocks) at each of them."""
    rng = np.random.default_rng(100 + M)
    N, K = 96, 1296
    w = (0.05 * rng.standard_normal((N, K))).astype(np.float32)
    segs = [(0, 40), (40, N)]
    x = W.random_act(200 + M, M, K, "student_t")
    amax = np.float32(float(np.max(np.abs(W.bf16_to_f32(x)))) / 3)
    say(f"[linear] static amax M={M}")
    pw = gpu_pack(w, segs)
    out, c, s = run_both(x, pw, amax=amax)
    oc, os_, _, _ = Q.quantize(W.bf16_to_f32(x), amax)
    assert np.array_equal(c, oc) and np.array_equal(s, os_)
    ref, bnd = oracle_linear_rows(x, w, segs, amax=amax)
    assert_within_tol(out.cpu().numpy().astype(np.float64), ref, bnd, f"linear static M={M}")


def test_linear_static_amax_and_prefill_path():
    d = W.tiny()
    pw = gpu_pack(d.w, d.segments)
    amax = float(np.max(np.abs(W.bf16_to_f32(d.x_bits)))) / 4
    out, c, s = run_both(d.x_bits, pw, amax=np.float32(amax))
    oc, os_, _, _ = Q.quantize(W.bf16_to_f32(d.x_bits), np.float32(amax))
    assert np.array_equal(c, oc) and np.array_equal(s, os_)
    # M > 16 goes through the separate kernels
    x = W.random_act(5, 40, 256, "normal")
    out, _, _ = run_both(x, pw)
    ref, bnd = oracle_linear_rows(x, d.w, d.segments)
    assert_within_tol(out.cpu().numpy().astype(np.float64), ref, bnd, "linear prefill path")


@pytest.mark.parametrize("M", [1, 3, 6, 13])
def test_linear_strided_input_and_output(M):
    """Row strides beyond K (input) and N (output), for each row-bound instance of
    the one-launch kernel: the result is bit-identical to quantize + GEMM on
    contiguous tensors, and the output columns outside the slice are untouched."""
    rng = np.random.default_rng(400 + M)
    K, N = 1040, 300
    segs = [(0, 100), (100, N)]
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    pw = gpu_pack(w, segs)
    x_bits = W.random_act(500 + M, M, K, "normal")
    say(f"[strided linear] M={M} K={K} N={N}")
    x = to_dev_bf16(x_bits)
    xwide = torch.zeros((M, K + 48), dtype=torch.bfloat16, device=DEV)
    xwide[:, 16:16 + K] = x
    big = torch.full((M, N + 40), 7.0, dtype=torch.float32, device=DEV)
    out, (c, s, g) = nv.linear(xwide[:, 16:16 + K], pw, out=big[:, 8:8 + N])
    c2, s2, g2 = nv.quantize_act(x)
    ref = nv.gemm(c2, s2, g2, pw)
    torch.cuda.synchronize()
    assert torch.equal(c, c2) and torch.equal(s, s2) and torch.equal(g, g2)
    assert torch.equal(big[:, 8:8 + N], ref)
    assert torch.all(big[:, :8] == 7.0) and torch.all(big[:, 8 + N:] == 7.0)


def test_convenience_layer_on_a_side_stream():
    """quantize_act, gemm and linear enqueued on a side torch stream (their outputs
    and scratch allocated on it) give the default stream's results."""
    d = W.tiny()
    pw = gpu_pack(d.w, d.segments)
    x = to_dev_bf16(d.x_bits)
    ref, (c0, s0, g0) = nv.linear(x, pw)
    ref_g = nv.gemm(c0, s0, g0, pw)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out, _ = nv.linear(x, pw, stream=side)
    c1, s1, g1 = nv.quantize_act(x, stream=side)
    out_g = nv.gemm(c1, s1, g1, pw, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(out_g, ref_g)
    assert torch.equal(c1, c0) and torch.equal(s1, s0) and torch.equal(g1, g0)


@pytest.mark.parametrize("N", [2000, 5000, 8232])
@pytest.mark.parametrize("M", [1, 7, 16])
def test_linear_strips_per_workgroup(M, N):
    """Output widths for which the launchers pick 1, 2 and 3 strips of 16 columns
    per workgroup (125, 313 and 515 strips), with ragged segments and a ragged k
    tile: one launch bit-identical to quantize + GEMM, sampled columns within the
    oracle's tolerance."""
    rng = np.random.default_rng(700 + M + N)
    K = 1040
    segs = [(0, 700), (700, N - 9), (N - 9, N)]
    w = np.concatenate([(0.02 * (1 + i) * rng.standard_normal((e - b, K))).astype(np.float32)
                        for i, (b, e) in enumerate(segs)])
    x_bits = W.random_act(800 + M, M, K, "student_t")
    say(f"[strips] M={M} N={N}")
    pw = gpu_pack(w, segs)
    x = to_dev_bf16(x_bits)
    out, (c, s, g) = nv.linear(x, pw)
    ref_gpu = nv.gemm(*nv.quantize_act(x), pw)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_gpu)
    cols = np.sort(np.unique(np.concatenate([rng.choice(N, 200, replace=False), [0, 699, 700, N - 10, N - 9, N - 1]])))
    ref, bnd = oracle_linear_rows(x_bits, w, segs, cols=cols)
    assert_within_tol(out.cpu().numpy().astype(np.float64)[:, cols], ref, bnd, f"strips M={M} N={N}")


@pytest.mark.parametrize("M,K,N", [(1, 17408, 700), (4, 20480, 700), (3, 10256, 700), (8, 10240, 700),
                                   (6, 5136, 700), (2, 8208, 700), (9, 6144, 700), (5, 17408, 700), (1, 9008, 700),
                                   (1, 17408, 12300), (3, 10256, 12300), (8, 10240, 12300)])
def test_linear_long_k(M, K, N):
    """K beyond 5120: one launch while the wave-local activation tiles fit (up to
    10240 for 8 rows, 20480 for 4), two launches otherwise ((9, 6144), (5, 17408));
    either way bit-identical to quantize + GEMM and within the oracle's tolerance
    on sampled columns.  N = 700 (44 workgroups) runs sixteen waves per workgroup
    (row-bound instances 1, 4 and 8 at five tiles per wave, 1 and 4 at ten);
    N = 12300 (257 workgroups) runs eight (ten and twenty tiles per wave)."""
    rng = np.random.default_rng(900 + M + K + N)
    segs = [(0, 300), (300, N)]
    w = np.concatenate([np.float32(0.02 * (1 + i)) * rng.standard_normal((e - b, K), dtype=np.float32)
                        for i, (b, e) in enumerate(segs)])
    x_bits = W.random_act(1000 + M, M, K, "student_t")
    say(f"[long K] M={M} K={K} N={N}")
    pw = gpu_pack(w, segs)
    x = to_dev_bf16(x_bits)
    out, (c, s, g) = nv.linear(x, pw)
    c2, s2, g2 = nv.quantize_act(x)
    ref_gpu = nv.gemm(c2, s2, g2, pw)
    torch.cuda.synchronize()
    assert torch.equal(c, c2) and torch.equal(s, s2) and torch.equal(g, g2)
    assert torch.equal(out, ref_gpu)
    cols = np.sort(np.unique(np.concatenate([rng.choice(N, 120, replace=False), [0, 299, 300, N - 1]])))
    ref, bnd = oracle_linear_rows(x_bits, w, segs, cols=cols)
    assert_within_tol(out.cpu().numpy().astype(np.float64)[:, cols], ref, bnd, f"long K M={M} K={K} N={N}")
