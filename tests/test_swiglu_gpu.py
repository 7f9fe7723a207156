"""GPU parity of the fused gate+up GEMM with the SwiGLU -> NVFP4 epilogue.

* The interleaved gate/up packing holds exactly the oracle's per-module
  encoding of each row (bit-exact), in the documented row order.
* Fused == unfused: nvfp4_gemm_swiglu_quantize gives the same codes, scales
  and g_dec bit for bit as nvfp4_gemm (plain packing) -> nvfp4_swiglu ->
  nvfp4_quantize_act with the same calibrated maximum.
* The unfused h agrees with the oracle's SwiGLU of the oracle's gate/up
  outputs within one bf16 unit in the last place plus the GEMM tolerance
  carried through silu, and the fused codes equal the oracle's encoding of
  that h exactly.
"""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_block_act_amd as nv
import workloads as W
from gpu_util import DEV, say, to_dev_bf16
from oracle import gemm as G
from oracle import nvfp4 as Q
from oracle import swiglu as S

pytestmark = pytest.mark.gpu


def _case(M, K, I, seed, fg=1.0, fu=3.0):
    rng = np.random.default_rng(seed)
    w = np.concatenate([(0.02 * fg * rng.standard_normal((I, K))).astype(np.float32),
                        (0.02 * fu * rng.standard_normal((I, K))).astype(np.float32)])
    x = W.random_act(seed + 1, M, K, "normal")
    return x, w


def _src_rows(I):
    n = np.arange(2 * I)
    return ((n >> 7) & 1) * I + ((n >> 8) << 7) + (n & 127)


def test_gate_up_packing_is_the_interleaved_per_module_encoding():
    I, K = 256, 272
    _, w = _case(4, K, I, 3)
    pw = nv.pack_weight_gate_up(torch.from_numpy(w).to(DEV))
    c, s = nv.weight_to_canonical(pw)
    torch.cuda.synchronize()
    oc, os_, og = Q.quantize_segments(w, [(0, I), (I, 2 * I)])
    src = _src_rows(I)
    assert np.array_equal(c.cpu().numpy(), oc[src]) and np.array_equal(s.cpu().numpy(), os_[src])
    assert pw.g_dec.cpu().numpy().tobytes() == og.tobytes()


def _run(M, K, I, seed, amax_scale=1.0):
    x_bits, w = _case(M, K, I, seed)
    say(f"[swiglu] M={M} K={K} I={I} amax_scale={amax_scale}")
    x = to_dev_bf16(x_bits)
    c, s, g = nv.quantize_act(x)
    wt = torch.from_numpy(w).to(DEV)
    pw = nv.pack_weight(wt, [(0, I), (I, 2 * I)])
    pwi = nv.pack_weight_gate_up(wt)
    gu = nv.gemm(c, s, g, pw)
    h = nv.swiglu(gu)
    amax_h = (h.float().abs().max() * amax_scale).reshape(1).contiguous()
    uc, us, ug = nv.quantize_act(h, amax_h)
    fc, fs, fg = nv.gemm_swiglu_quantize(c, s, g, pwi, amax_h)
    torch.cuda.synchronize()
    assert torch.equal(fc, uc) and torch.equal(fs, us) and torch.equal(fg, ug), "fused != unfused"
    return x_bits, w, gu.cpu().numpy(), h, amax_h, fc, fs


@pytest.mark.parametrize("M,K,I,amax_scale", [(300, 1040, 256, 1.0), (64, 512, 384, 0.5), (17, 5120, 128, 1.0)])
def test_fused_equals_unfused_and_matches_the_oracle(M, K, I, amax_scale):
    x_bits, w, gu, h, amax_h, fc, fs = _run(M, K, I, M + K + I, amax_scale)
    # oracle gate/up outputs and their tolerance
    x32 = W.bf16_to_f32(x_bits)
    ac, as_, ag, _ = Q.quantize(x32, np.float32(np.max(np.abs(x32))))
    a_hat = Q.dequantize(ac, as_, ag)
    w_hat = Q.dequantize_segments(*Q.quantize_segments(w, [(0, I), (I, 2 * I)]), [(0, I), (I, 2 * I)])
    ref = G.gemm_f64(a_hat, w_hat)
    tol = G.RTOL * G.gemm_bound(a_hat, w_hat) + G.ATOL
    assert np.all(np.abs(gu - ref) <= tol)
    g_o, u_o = ref[:, :I], ref[:, I:]
    h_o = S.swiglu_bf16(g_o, u_o)
    hf = (h.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    ho = (h_o.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    sig = 1.0 / (1.0 + np.exp(-g_o))
    dsilu = sig * (1.0 + g_o * (1.0 - sig))
    carried = np.abs(dsilu * u_o) * tol[:, :I] + np.abs(g_o * sig) * tol[:, I:]
    ulp = np.maximum(np.abs(ho), 1e-38) * 2.0 ** -7
    assert np.all(np.abs(hf - ho) <= ulp + 1.01 * carried + 1e-30)
    oc, os_, og, _ = Q.quantize(hf.astype(np.float32), np.float32(amax_h.item()))
    assert np.array_equal(fc.cpu().numpy(), oc) and np.array_equal(fs.cpu().numpy(), os_)
