"""The linear layer under HIP graph capture, as the benchmark runs it: a graph of
nvfp4_linear calls (one-launch decode form, the two-launch form for K > 5120, and
the large-M form: the two-pass dynamic quantizer -- partial maxima, their
reduction, the encode -- then the GEMM) is replayed several times with the
program's own eager work and synchronizations in between, and every replay must
reproduce the eager result bit for bit."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_block_act_amd as nv
import workloads as W
from gpu_util import DEV, gpu_pack, say, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,N", [(1, 5120, 1024), (16, 5120, 512), (4, 6144, 256), (40, 5120, 1024),
                                   (300, 1024, 512)])
def test_linear_graph_replays_match_eager(M, K, N):
    say(f"[graph] M={M} K={K} N={N}")
    rng = np.random.default_rng(M + K + N)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    pw = gpu_pack(w, [(0, N // 2), (N // 2, N)])
    xs = [to_dev_bf16(W.random_act(100 + i, M, K, "student_t")) for i in range(3)]
    ws = nv.Workspace(DEV)
    outs = [torch.empty((M, N), dtype=torch.float32, device=DEV) for _ in xs]
    acts = [(torch.empty((M, K // 2), dtype=torch.uint8, device=DEV),
             torch.empty((M, K // 16), dtype=torch.uint8, device=DEV),
             torch.empty(1, dtype=torch.float32, device=DEV)) for _ in xs]

    def calls():
        for x, o, a in zip(xs, outs, acts):
            nv.linear(x, pw, None, ws, out=o, act_out=a)

    calls()                                           # eager reference
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    ref_codes = [a[0].clone() for a in acts]
    ref_scales = [a[1].clone() for a in acts]
    ref_g = [a[2].clone() for a in acts]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(4):
        for o, a in zip(outs, acts):                  # eager work between replays
            o.fill_(float("nan"))
            a[0].fill_(0x77)
            a[2].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert torch.equal(o, ref[i]), f"replay {rep}, call {i}: output differs"
            assert torch.equal(acts[i][0], ref_codes[i]), f"replay {rep}, call {i}: codes differ"
            assert torch.equal(acts[i][1], ref_scales[i]), f"replay {rep}, call {i}: scales differ"
            assert torch.equal(acts[i][2], ref_g[i]), f"replay {rep}, call {i}: g_dec differs"
