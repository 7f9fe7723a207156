"""GPU parity of the static-scale calibration helpers against oracle/observe.py:
the running maximum over batches of different shapes and strides is
bit-identical, the saturation counts equal the oracle's for static maxima below,
at and above the tensor maximum (and zero), and static quantization with the
observed maximum equals the oracle's encode."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_block_act_amd as nv
import workloads as W
from gpu_util import DEV, say, to_dev_bf16
from oracle import nvfp4 as Q
from oracle import observe as O

pytestmark = pytest.mark.gpu


def test_running_amax_over_batches():
    obs = nv.AmaxObserver(DEV)
    xs = []
    for i, (M, K) in enumerate([(16, 5120), (1, 5120), (300, 272), (2048, 512)]):
        bits = W.random_act(40 + i, M, K, "student_t", scale=0.5 + i)
        xs.append(W.bf16_to_f32(bits))
        x = to_dev_bf16(bits)
        if i == 2:                                    # a strided view (ldx > K)
            big = torch.zeros((M, K + 64), dtype=torch.bfloat16, device=DEV)
            big[:, :K] = x
            x = big[:, :K]
        obs.observe(x)
        torch.cuda.synchronize()
        assert obs.amax.item() == float(O.running_amax(xs)), f"batch {i}"


@pytest.mark.parametrize("scale", [0.0, 0.3, 0.9, 1.0, 2.0])
def test_saturation_counts(scale):
    bits = W.random_act(7, 256, 1024, "student_t")
    x32 = W.bf16_to_f32(bits)
    amax = np.float32(np.max(np.abs(x32)) * scale)
    say(f"[calib] stats amax scale {scale}")
    counts = nv.quantize_stats(to_dev_bf16(bits), torch.tensor([amax], device=DEV)).cpu().numpy()
    sat, clip = O.saturation_counts(x32, amax)
    assert counts.tolist() == [sat, clip]
    if 0 < scale < 1:
        assert sat > 0
    if 0 < scale < 0.5:
        assert clip > 0
    if scale >= 1:
        assert sat == 0


def test_static_quantize_with_observed_amax():
    obs = nv.AmaxObserver(DEV)
    cal = [W.random_act(60 + i, 16, 5120, "student_t") for i in range(4)]
    for b in cal:
        obs.observe(to_dev_bf16(b))
    test = W.random_act(99, 16, 5120, "student_t")
    c, s, g = nv.quantize_act(to_dev_bf16(test), obs.amax)
    torch.cuda.synchronize()
    amax = O.running_amax([W.bf16_to_f32(b) for b in cal])
    oc, os_, og, _ = Q.quantize(W.bf16_to_f32(test), amax)
    assert np.array_equal(c.cpu().numpy(), oc) and np.array_equal(s.cpu().numpy(), os_)
    assert g.cpu().numpy().tobytes() == np.float32(og).tobytes()
