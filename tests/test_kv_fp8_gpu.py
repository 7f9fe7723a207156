"""GPU parity of the calibrated FP8 KV-cache codec (bit-exact against
oracle/kvfp8.py): every bf16 bit pattern at two scales, a KV-shaped tensor with
outlier channels and a calibrated maximum below the true one (saturation),
ragged lengths (16-element chunks plus a tail), amax == 0, signed zeros."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_block_act_amd as nv
import workloads as W
from gpu_util import DEV, say
from oracle import kvfp8 as F

pytestmark = pytest.mark.gpu


def _dev_bits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def check(bits, amax, what):
    say(f"[kvfp8] {what} n={bits.size} amax={amax}")
    x = _dev_bits(bits)
    a = torch.tensor([amax], dtype=torch.float32, device=DEV)
    codes = nv.kv_fp8_encode(x, a)
    y = nv.kv_fp8_decode(codes, a)
    torch.cuda.synchronize()
    x32 = W.bf16_to_f32(bits)
    oc = F.encode(x32, np.float32(amax))
    assert np.array_equal(codes.cpu().numpy(), oc), f"{what}: encode mismatches"
    ob = F.decode_bf16(oc, np.float32(amax))
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), ob), f"{what}: decode mismatches"


@pytest.mark.parametrize("amax", [1.0, 3.0e4])
def test_every_finite_bf16(amax):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]                  # drop inf / NaN
    check(bits, amax, "all bf16")


def test_kv_tensor_with_calibrated_saturation():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2048, 1024)).astype(np.float32)
    x[:, rng.choice(1024, 8, replace=False)] *= 20.0          # outlier channels
    bits = W.bf16_bits(x).ravel()
    amax = float(np.max(np.abs(W.bf16_to_f32(bits)))) * 0.7
    check(bits, amax, "kv saturating")


@pytest.mark.parametrize("n", [1, 15, 16, 17, 31, 33, 1000, 12293, (1 << 20) + 7])
def test_ragged_lengths(n):
    rng = np.random.default_rng(n)
    check(W.bf16_bits(rng.standard_normal(n).astype(np.float32)), 2.5, f"ragged {n}")


def test_zero_amax_and_signed_zeros():
    bits = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x0001, 0x8001] * 3, np.uint16)
    check(bits, 0.0, "amax zero")
    check(bits, 1.0, "signed zeros")
