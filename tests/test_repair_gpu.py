"""GPU side of the repair comparison on the GDN in-projection workload (six
modules, amax ratio ~20): the per-segment epilogue (six FP32 scales) and the
shared-scale re-encode (one segment) both match their oracle variants within
the GEMM tolerance, and their errors against the unquantized product match the
oracle's measurement."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_block_act_amd as nv
import workloads as W
from gpu_util import assert_within_tol, gpu_pack, say, to_dev_bf16
from oracle import gemm as G
from oracle import nvfp4 as Q
from oracle import repair as R

pytestmark = pytest.mark.gpu


def test_per_segment_and_shared_scale_repairs_on_gdn_in_proj():
    d = W.gdn_in_proj(M=512)
    x32 = W.bf16_to_f32(d.x_bits)
    rng = np.random.default_rng(11)
    rows = np.sort(rng.choice(d.M, 48, replace=False))
    cols = np.concatenate([np.sort(rng.choice(np.arange(b, e), min(e - b, 96), replace=False)) for b, e in d.segments])
    x = to_dev_bf16(d.x_bits)
    c, s, g = nv.quantize_act(x)
    outs = {}
    for variant, segs in (("per_segment", d.segments), ("shared", [(0, d.N)])):
        pw = gpu_pack(d.w, segs)
        outs[variant] = nv.gemm(c, s, g, pw).cpu().numpy().astype(np.float64)[rows][:, cols]
    torch.cuda.synchronize()
    res, ys, y_ref = R.relative_errors(x32, d.w, d.segments, rows, cols)
    amax = np.float32(np.max(np.abs(x32)))
    ac, as_, ag, _ = Q.quantize(x32[rows], amax)
    a_hat = Q.dequantize(ac, as_, ag)
    for variant in ("per_segment", "shared"):
        w_hat = R.decoded_weights(d.w, d.segments, cols, variant)
        assert_within_tol(outs[variant], ys[variant], G.gemm_bound(a_hat, w_hat), f"repair {variant}")
    for i, (b, e) in enumerate(d.segments):
        sel = (cols >= b) & (cols < e)
        for variant in ("per_segment", "shared"):
            y = outs[variant][:, sel]
            ref = y_ref[:, sel]
            gpu_err = np.sqrt(np.mean((y - ref) ** 2)) / np.sqrt(np.mean(ref ** 2))
            assert abs(gpu_err - res[i][variant]) <= 1e-4 * res[i][variant] + 1e-9
        say(f"[repair] module {i}: per-segment {res[i]['per_segment']:.5f} shared {res[i]['shared']:.5f} "
            f"mismatch {res[i]['mismatch']:.3g}")
        assert res[i]["shared"] < 1.25 * res[i]["per_segment"]
        ratio = np.max(np.abs(d.w[b:e])) / np.max(np.abs(d.w[d.segments[0][0]:d.segments[0][1]]))
        if abs(np.log(ratio)) > np.log(1.5):          # scales differ: the unrepaired GEMM is far off
            assert res[i]["mismatch"] > 0.3
