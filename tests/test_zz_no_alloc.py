"""nvfp4_linear_noalloc (the entry point for callers that cannot allocate) against
nvfp4_linear with a caller workspace, through the C ABI: codes, scales, g_dec and
outputs bit-identical, and the oracle's tolerance on sampled rows; two calls in a
row, the second smaller, both large enough for the two-pass quantizer that uses the
library's scratch, plus a decode-sized call and a call on a side stream."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_block_act_amd as nv
import workloads as W
from gpu_util import DEV, assert_within_tol, gpu_pack, oracle_linear_rows, say, to_dev_bf16

pytestmark = pytest.mark.gpu


def _inputs(M, K, N, seed):
    rng = np.random.default_rng(seed)
    segs = [(0, N // 4), (N // 4, N)]
    w = np.concatenate([(0.02 * (1 + 4 * i) * rng.standard_normal((e - b, K))).astype(np.float32)
                        for i, (b, e) in enumerate(segs)])
    x_bits = W.random_act(seed + 1, M, K, "student_t")
    return x_bits, w, segs


def _call(fn, x, M, K, pw, stream, with_ws):
    N = pw.N
    c = torch.empty((M, K // 2), dtype=torch.uint8, device=DEV)
    s = torch.empty((M, K // 16), dtype=torch.uint8, device=DEV)
    g = torch.empty(1, dtype=torch.float32, device=DEV)
    out = torch.empty((M, N), dtype=torch.float32, device=DEV)
    args = [x, M, K, x.stride(0), None, c, s, g, pw.codes, pw.scales, N, pw.segments, pw.g_dec, out, N]
    if with_ws:
        wsb = nv.nvfp4_linear_workspace_bytes(M, K)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=DEV)
        args += [ws, wsb]
    fn(*args, stream=stream)
    return out, c, s, g


@pytest.mark.parametrize("side_stream", [False, True])
def test_noalloc_equals_linear_twice_second_smaller(side_stream):
    stream = torch.cuda.Stream() if side_stream else torch.cuda.current_stream()
    for M, K, N, seed in [(512, 5120, 2048, 61), (100, 2048, 640, 62), (4, 1024, 512, 63)]:
        say(f"[noalloc] M={M} K={K} N={N} side_stream={side_stream}")
        if M > 16:
            assert nv.nvfp4_linear_workspace_bytes(M, K) > 0      # the two-pass quantizer: the scratch is used
        x_bits, w, segs = _inputs(M, K, N, seed)
        pw = gpu_pack(w, segs)
        x = to_dev_bf16(x_bits)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            a = _call(nv.nvfp4_linear_noalloc, x, M, K, pw, stream.cuda_stream, False)
            b = _call(nv.nvfp4_linear, x, M, K, pw, stream.cuda_stream, True)
        torch.cuda.synchronize()
        for u, v, what in zip(a, b, ("out", "codes", "scales", "g_dec")):
            assert torch.equal(u, v), f"{what} differs from nvfp4_linear"
        rows = np.unique(np.array([0, M // 2, M - 1]))
        ref, bnd = oracle_linear_rows(x_bits, w, segs, rows=rows)
        assert_within_tol(a[0].cpu().numpy().astype(np.float64)[rows], ref, bnd, f"noalloc M={M}")
