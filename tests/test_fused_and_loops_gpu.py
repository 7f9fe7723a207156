"""GPU parity at sizes where the kernels' grid-stride loops iterate, and the fused
gate+up -> SwiGLU -> NVFP4 epilogue at the prefill MLP's full size.

* Grid-stride loops: the KV decode (2048 workgroups x 256 threads x 16 elements per
  pass, so n > 2^23 loops), quantize_stats (2048 x 256 threads, one block each,
  so more than 2^19 blocks loop) and the unfused SwiGLU (4096 x 256 threads, one
  element each, so M * I > 2^20 loops), each with a ragged tail.
* The fused epilogue at 8192 x 5120 x (2 x 17408) -- the workgroup numbering that
  interleaves XCDs, several row-panel groups, output columns far past the first
  tile -- is bit-identical to the unfused kernels (both take the MFMA form there),
  and agrees with the oracle on sampled rows and blocks.
* Fused == unfused bit for bit at a mid-size MFMA shape; at a small shape where the
  unfused GEMM takes the weight-streaming form (another fp32 summation order),
  with an activation outlier of 1e4, the fused result is held to the oracle's
  tolerance instead.
"""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_block_act_amd as nv
import workloads as W
from gpu_util import DEV, say, to_dev_bf16
from oracle import gemm as G
from oracle import kvfp8 as F
from oracle import nvfp4 as Q
from oracle import observe as O
from oracle import swiglu as S
from oracle.formats import e4m3_value

pytestmark = pytest.mark.gpu


def test_kv_codec_decode_loops_past_one_grid():
    n = (1 << 24) + (1 << 20) + 9
    rng = np.random.default_rng(41)
    x = rng.standard_normal(n).astype(np.float32)
    x[::997] *= 30.0
    bits = (torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    amax = np.float32(0.8 * np.max(np.abs(x)))                  # calibrated below the maximum: saturates
    say(f"[loops] kv codec n={n}")
    xd = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    a = torch.tensor([amax], dtype=torch.float32, device=DEV)
    codes = nv.kv_fp8_encode(xd, a)
    y = nv.kv_fp8_decode(codes, a)
    torch.cuda.synchronize()
    oc = F.encode(W.bf16_to_f32(bits), amax)
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), F.decode_bf16(oc, amax))


def test_quantize_stats_loops_past_one_grid():
    M, K = 1041, 8192                                            # 533,056 blocks > 2^19
    bits = W.random_act(43, M, K, "student_t")
    x32 = W.bf16_to_f32(bits)
    amax = np.float32(0.05 * np.max(np.abs(x32)))               # many saturated blocks and clipped elements
    say(f"[loops] quantize_stats {M}x{K}")
    cnt = nv.quantize_stats(to_dev_bf16(bits), torch.tensor([amax], dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    sat, clip = O.saturation_counts(x32, amax)
    assert sat > 0 and clip > 0
    assert cnt.cpu().numpy().tolist() == [sat, clip]


def test_swiglu_loops_past_one_grid():
    M, I = 601, 2048                                             # 1,230,848 elements > 2^20
    rng = np.random.default_rng(44)
    gu = (3.0 * rng.standard_normal((M, 2 * I))).astype(np.float32)
    say(f"[loops] swiglu {M}x{I}")
    h = nv.swiglu(torch.from_numpy(gu).to(DEV))
    torch.cuda.synchronize()
    got = h.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.int64)
    want = S.swiglu_bf16(gu[:, :I], gu[:, I:]).astype(np.int64)
    # the kernel evaluates silu in fp32, the oracle in fp64 with one rounding: at
    # most one bf16 unit in the last place apart (same sign), most equal
    same_sign = (got >> 15) == (want >> 15)
    assert np.all(same_sign | ((got & 0x7FFF) == 0) | ((want & 0x7FFF) == 0))
    assert np.all(np.abs((got & 0x7FFF) - (want & 0x7FFF)) <= 1)
    assert np.mean(got == want) > 0.99


def _fused_and_unfused(x_bits, w, I, amax_scale=1.0):
    x = to_dev_bf16(x_bits)
    c, s, g = nv.quantize_act(x)
    wt = torch.from_numpy(w).to(DEV)
    pw = nv.pack_weight(wt, [(0, I), (I, 2 * I)])
    pwi = nv.pack_weight_gate_up(wt)
    del wt
    gu = nv.gemm(c, s, g, pw)
    h = nv.swiglu(gu)
    amax_h = (h.float().abs().max() * amax_scale).reshape(1).contiguous()
    uc, us, ug = nv.quantize_act(h, amax_h)
    fc, fs, fg = nv.gemm_swiglu_quantize(c, s, g, pwi, amax_h)
    torch.cuda.synchronize()
    return gu, h, amax_h, (uc, us, ug), (fc, fs, fg)


def _oracle_gate_up(x_bits, w, I, rows, js):
    """Oracle g and u (fp64) and their tolerances at rows x js, each module encoded
    with its own maximum over the whole module."""
    x32 = W.bf16_to_f32(x_bits)
    ac, as_, ag, _ = Q.quantize(x32[rows], np.float32(np.max(np.abs(x32))))
    a_hat = Q.dequantize(ac, as_, ag)
    outs = []
    for mod in (0, 1):
        wm = w[mod * I:(mod + 1) * I]
        wc, ws, wg, _ = Q.quantize(wm[js], np.float32(np.max(np.abs(wm))))
        w_hat = Q.dequantize(wc, ws, wg)
        outs.append((G.gemm_f64(a_hat, w_hat), G.RTOL * G.gemm_bound(a_hat, w_hat) + G.ATOL))
    return outs


def test_fused_swiglu_full_prefill_shape():
    d = W.prefill_gate_up()
    M, K, I = d.M, d.K, d.N // 2
    assert nv.nvfp4_gemm_form(M, K, 2 * I) == 1
    say(f"[fused] gate+up SwiGLU M={M} K={K} I={I}")
    gu, h, amax_h, (uc, us, ug), (fc, fs, fg) = _fused_and_unfused(d.x_bits, d.w, I)
    assert torch.equal(fc, uc) and torch.equal(fs, us) and torch.equal(fg, ug), "fused != unfused"
    rng = np.random.default_rng(45)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], rng.choice(M, 6, replace=False)]))
    blocks = np.unique(np.concatenate([[0, 7, 8, 31, 32, I // 16 - 1], rng.choice(I // 16, 26, replace=False)]))
    js = (blocks[:, None] * 16 + np.arange(16)).reshape(-1)
    (g_o, g_tol), (u_o, u_tol) = _oracle_gate_up(d.x_bits, d.w, I, rows, js)
    rt = torch.from_numpy(rows).to(DEV)
    jt = torch.from_numpy(js).to(DEV)
    gu_s = gu.index_select(0, rt).cpu().numpy().astype(np.float64)
    assert np.all(np.abs(gu_s[:, js] - g_o) <= g_tol) and np.all(np.abs(gu_s[:, I + js] - u_o) <= u_tol)
    # the GPU's h against the oracle's SwiGLU of the oracle's g, u
    hb = h.index_select(0, rt).index_select(1, jt).view(torch.int16).cpu().numpy().view(np.uint16)
    hf = (hb.astype(np.uint32) << 16).view(np.float32)
    ho = (S.swiglu_bf16(g_o, u_o).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    sig = 1.0 / (1.0 + np.exp(-g_o))
    carried = np.abs(sig * (1.0 + g_o * (1.0 - sig)) * u_o) * g_tol + np.abs(g_o * sig) * u_tol
    assert np.all(np.abs(hf - ho) <= np.maximum(np.abs(ho), 1e-38) * 2.0 ** -7 + 1.01 * carried + 1e-30)
    # the fused codes of those blocks are the oracle's encoding of that h
    oc, os_, og, _ = Q.quantize(hf, np.float32(amax_h.item()))
    fcs = fc.index_select(0, rt).cpu().numpy().reshape(len(rows), I // 16, 8)[:, blocks].reshape(len(rows), -1)
    fss = fs.index_select(0, rt).cpu().numpy()[:, blocks]
    assert np.array_equal(fcs, oc) and np.array_equal(fss, os_)
    assert float(fg.cpu()[0]) == float(og)


@pytest.mark.parametrize("M,K,I,form", [(2048, 512, 1024, 2), (2048, 512, 4096, 1)])
def test_fused_equals_unfused_mid_size_mfma_form(M, K, I, form):
    """Fused == unfused bit for bit where nvfp4_gemm takes an MFMA form: the fused
    kernel runs 256 x 256 tiles; the unfused GEMM runs 256 x 128 tiles at I = 1024
    (128 of them instead of 64) and 256 x 256 at I = 4096 (one full round)."""
    assert nv.nvfp4_gemm_form(M, K, 2 * I) == form
    rng = np.random.default_rng(46)
    w = (0.02 * rng.standard_normal((2 * I, K))).astype(np.float32)
    w[I:] *= 3.0
    x = W.random_act(47, M, K, "student_t")
    say(f"[fused] mid-size M={M} K={K} I={I}")
    _, _, _, u, f = _fused_and_unfused(x, w, I)
    assert all(torch.equal(a, b) for a, b in zip(f, u)), "fused != unfused"


def test_fused_small_shape_with_outlier_within_tolerance():
    """Where nvfp4_gemm takes the weight-streaming form the fused and unfused g, u sum
    in different fp32 orders; with a 1e4 activation outlier the fused encoding is
    checked against the oracle's h: every decoded element within one unit of its
    block's scale (the largest E2M1 rounding error; more only where the element is
    cut to 6) plus bf16 rounding and the GEMM tolerance carried through silu."""
    M, K, I = 48, 512, 256
    assert nv.nvfp4_gemm_form(M, K, 2 * I) == 0
    rng = np.random.default_rng(48)
    w = (0.02 * rng.standard_normal((2 * I, K))).astype(np.float32)
    xf = rng.standard_normal((M, K)).astype(np.float32)
    xf[5, 77] = 1.0e4
    x = torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    say(f"[fused] small shape with outlier M={M} K={K} I={I}")
    _, _, amax_h, _, (fc, fs, fg) = _fused_and_unfused(x, w, I)
    (g_o, g_tol), (u_o, u_tol) = _oracle_gate_up(x, w, I, np.arange(M), np.arange(I))
    ho = S.silu(g_o) * u_o
    h_hat = Q.dequantize(fc.cpu().numpy(), fs.cpu().numpy(), np.float32(fg.item()))
    unit = np.repeat(e4m3_value(fs.cpu().numpy()), 16, axis=1) * np.float64(fg.item())
    sig = 1.0 / (1.0 + np.exp(-g_o))
    carried = np.abs(sig * (1.0 + g_o * (1.0 - sig)) * u_o) * g_tol + np.abs(g_o * sig) * u_tol
    # rounding to the E2M1 grid errs by at most one unit of the block's scale;
    # beyond 6 units (a scale rounded down, or subnormal) the element is cut to 6
    rounding = np.maximum(unit, np.abs(ho) - 6.0 * unit)
    bound = 1.001 * rounding + np.abs(ho) * 2.0 ** -7 + 1.01 * carried + 1e-30
    assert np.all(np.abs(h_hat - ho) <= bound)
    assert np.max(np.abs(ho)) > 100 * np.median(np.abs(ho))    # the outlier reaches h
