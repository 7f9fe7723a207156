"""GPU parity of the weight packer (bit-exact) and of the W4A4 GEMM with the
per-segment epilogue (|gpu - oracle| <= 1e-5 * sum|a||b| + 1e-6 elementwise),
on every workload shape, ragged tails and the mismatch negative control."""
import functools

import numpy as np
import pytest
import torch

import nvfp4_w4a4_block_act_amd as nv
import workloads as W
from gpu_util import (DEV, assert_within_tol, gpu_pack, oracle_linear_rows, say, to_dev_bf16, to_dev_f32)
from oracle import gemm as G
from oracle import nvfp4 as Q

pytestmark = pytest.mark.gpu


def gpu_linear(x_bits, pw):
    x = to_dev_bf16(x_bits)
    c, s, g = nv.quantize_act(x)
    out = nv.gemm(c, s, g, pw)
    torch.cuda.synchronize()
    return out


# ---- packer -------------------------------------------------------------------------
def check_pack(w, segs, what):
    say(f"[pack] {what} N={w.shape[0]} K={w.shape[1]} segs={len(segs)}")
    pw = gpu_pack(w, segs)
    c, s = nv.weight_to_canonical(pw)
    torch.cuda.synchronize()
    oc, os_, og = Q.quantize_segments(w, segs)
    assert np.array_equal(s.cpu().numpy(), os_), f"{what}: scale mismatches"
    assert np.array_equal(c.cpu().numpy(), oc), f"{what}: code mismatches"
    assert pw.g_dec.cpu().numpy().tobytes() == og.tobytes()
    return pw, oc, os_


def test_pack_tiny():
    t = W.tiny()
    check_pack(t.w, t.segments, "tiny")


@pytest.mark.parametrize("N,K,segs", [
    (16, 16, [(0, 16)]), (37, 48, [(0, 5), (5, 37)]), (200, 272, [(0, 64), (64, 96), (96, 200)]),
    (33, 5136, [(0, 1), (1, 33)]),
])
def test_pack_ragged(N, K, segs):
    rng = np.random.default_rng(N + K)
    w = np.concatenate([(0.02 * (i + 1) * rng.standard_normal((e - b, K))).astype(np.float32)
                        for i, (b, e) in enumerate(segs)])
    check_pack(w, segs, "ragged")


@pytest.mark.parametrize("pad", [2, 8])
def test_pack_leading_dimension(pad):
    """Weight rows at a stride of K + pad floats (pad 2: rows not 16-byte aligned, the
    amax pass reads single floats; pad 8: 16-byte pieces) pack like the dense tensor,
    each segment's maximum taken over its rows only (the largest value sits in the pad
    of another segment's rows and must be ignored)."""
    rng = np.random.default_rng(70 + pad)
    N, K = 300, 1040
    segs = [(0, 100), (100, 300)]
    w = np.concatenate([(0.02 * (1 + 5 * i) * rng.standard_normal((e - b, K))).astype(np.float32)
                        for i, (b, e) in enumerate(segs)])
    full = np.zeros((N, K + pad), np.float32)
    full[:, :K] = w
    full[:, K:] = 1.0e3                                   # outside the tensor
    say(f"[pack] leading dimension K + {pad}")
    dev = torch.from_numpy(full).to(DEV)
    pw = nv.pack_weight(dev[:, :K], segs)
    c, s = nv.weight_to_canonical(pw)
    torch.cuda.synchronize()
    oc, os_, og = Q.quantize_segments(w, segs)
    assert np.array_equal(c.cpu().numpy(), oc) and np.array_equal(s.cpu().numpy(), os_)
    assert pw.g_dec.cpu().numpy().tobytes() == og.tobytes()


def test_pack_layout_is_the_documented_tiling():
    """Tiled buffer = canonical codes/scales re-blocked into 16-row x 128-k chunks, strip major;
    inside a chunk the 16 code bytes (2 scale bytes) of row n, k group g sit at slot g * 16 + n."""
    rng = np.random.default_rng(3)
    N, K = 40, 272
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    pw, oc, os_ = check_pack(w, [(0, N)], "layout")
    Np, Kp = 48, 384
    cpad = np.zeros((Np, Kp // 2), np.uint8)
    cpad[:N, :K // 2] = oc
    spad = np.zeros((Np, Kp // 16), np.uint8)
    spad[:N, :K // 16] = os_
    ct = cpad.reshape(Np // 16, 16, Kp // 128, 4, 16).transpose(0, 2, 3, 1, 4).ravel()
    st = spad.reshape(Np // 16, 16, Kp // 128, 4, 2).transpose(0, 2, 3, 1, 4).ravel()
    assert np.array_equal(pw.codes.cpu().numpy(), ct)
    assert np.array_equal(pw.scales.cpu().numpy(), st)


# ---- GEMM -----------------------------------------------------------------------------
def check_linear(x_bits, w, segs, what, rows=None, cols=None):
    say(f"[gemm] {what} M={x_bits.shape[0]} K={x_bits.shape[1]} N={w.shape[0]} segs={len(segs)}")
    pw = gpu_pack(w, segs)
    out = gpu_linear(x_bits, pw)
    ref, bnd = oracle_linear_rows(x_bits, w, segs, rows, cols)
    o = out.cpu().numpy().astype(np.float64)
    if rows is not None:
        o = o[np.asarray(rows)]
    if cols is not None:
        o = o[:, np.asarray(cols)]
    assert_within_tol(o, ref, bnd, what)
    return pw, out


def test_gemm_tiny():
    t = W.tiny()
    check_linear(t.x_bits, t.w, t.segments, "tiny")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_gemm_decode_full(M):
    d = W.decode(M=M)
    check_linear(d.x_bits, d.w, d.segments, f"decode M={M}")


@pytest.mark.parametrize("M,N,K,nseg", [
    (1, 16, 16, 1), (2, 37, 48, 2), (5, 200, 272, 3), (16, 129, 144, 2), (17, 16, 16, 1),
    (17, 130, 144, 3), (33, 300, 5136, 4), (130, 257, 400, 5), (256, 128, 256, 1), (300, 520, 1040, 16),
    (64, 100, 320, 2), (40, 64, 192, 1), (9, 70, 320, 2), (513, 300, 128, 3),
])
def test_gemm_ragged(M, N, K, nseg):
    rng = np.random.default_rng(M * 1000 + N + K)
    cuts = sorted(rng.choice(np.arange(1, N), nseg - 1, replace=False).tolist()) if nseg > 1 else []
    bounds = [0] + cuts + [N]
    segs = list(zip(bounds[:-1], bounds[1:]))
    w = np.concatenate([(0.02 * (1 + 3 * i) * rng.standard_normal((e - b, K))).astype(np.float32)
                        for i, (b, e) in enumerate(segs)])
    x = W.random_act(M + N, M, K, "student_t")
    check_linear(x, w, segs, f"ragged M={M} N={N} K={K}")


@pytest.mark.parametrize("M", [7, 300])
def test_gemm_subnormal_block_scales(M):
    """Blocks 10^0 .. 10^-6 below the tensor maximum get E4M3 subnormal (or zero) scales
    on both operands; their decoded values must still be exact in the GEMM."""
    rng = np.random.default_rng(90 + M)
    K, N = 512, 96
    x = rng.standard_normal((M, K)).astype(np.float32)
    x *= (10.0 ** -rng.integers(0, 7, size=(M, K // 16))).repeat(16, axis=1).astype(np.float32)
    x[0, 0] = 50.0
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    w *= (10.0 ** -rng.integers(0, 7, size=(N, K // 16))).repeat(16, axis=1).astype(np.float32)
    w[0, 0] = 1.0
    from workloads import bf16_bits
    xb = bf16_bits(x)
    sc = Q.quantize(W.bf16_to_f32(xb))[1]
    assert np.any((sc > 0) & (sc < 8)), "no subnormal activation scales"
    check_linear(xb, w, [(0, 40), (40, N)], f"subnormal scales M={M}")


@pytest.mark.parametrize("M,N,K", [(300, 32808, 1040), (520, 65584, 512)])
def test_gemm_ragged_column_split_along_k(M, N, K):
    """Shapes whose whole 256x256 tiles exactly fill their last round of 256
    workgroups (2 x 128 and 3 x 256 tiles): the ragged last column then runs as
    the weight-streaming GEMM over row blocks, with the segment table shifted to
    its columns -- as extra workgroups of the MFMA launch at (520, 65584, 512), as
    a second launch at (300, 32808, 1040), which also has ragged rows and a k
    tail (K % 128 == 16).  The GDN in-projection test covers the merged form with
    four strips per workgroup."""
    assert nv.nvfp4_gemm_form(M, K, N) == 1
    rng = np.random.default_rng(M + N + K)
    segs = [(0, 1000), (1000, N - 20), (N - 20, N)]
    w = np.concatenate([(0.02 * (1 + 2 * i) * rng.standard_normal((e - b, K))).astype(np.float32)
                        for i, (b, e) in enumerate(segs)])
    x = W.random_act(M + K, M, K, "student_t")
    rows = _sample(M, 12, rng, [0, M - 1])
    cols = _sample(N, 300, rng, list(range(N - N % 256, N)) + [0, N - N % 256 - 1])
    check_linear(x, w, segs, f"ragged column split M={M} N={N} K={K}", rows, cols)


@pytest.mark.parametrize("M,N,K", [(4096, 12304, 512), (4096, 12320, 512)])
def test_gemm_ragged_columns_inside_the_mfma_launch(M, N, K):
    """768 whole 256 x 256 tiles fill three rounds, so the 16 / 32 ragged columns run
    as extra workgroups of the MFMA launch (the row-blocked body with one / two strips
    per workgroup).  With the ragged columns as a module of their own, they equal the
    GEMM of that module alone (which runs the same row-blocked body as its own launch)
    bit for bit, and the oracle on sampled rows within tolerance."""
    assert nv.nvfp4_gemm_form(M, K, N) == 1 and nv.nvfp4_gemm_form(M, K, N - 12288) == 0
    rng = np.random.default_rng(N + K)
    segs = [(0, 12288), (12288, N)]
    w = np.concatenate([(0.02 * rng.standard_normal((12288, K))).astype(np.float32),
                        (0.3 * rng.standard_normal((N - 12288, K))).astype(np.float32)])
    x = W.random_act(M + N, M, K, "student_t")
    say(f"[ragged in launch] M={M} N={N} K={K}")
    c, s_, g = nv.quantize_act(to_dev_bf16(x))
    out = nv.gemm(c, s_, g, gpu_pack(w, segs))
    part = nv.gemm(c, s_, g, gpu_pack(np.ascontiguousarray(w[12288:]), [(0, N - 12288)]))
    torch.cuda.synchronize()
    assert torch.equal(out[:, 12288:], part)
    rows = _sample(M, 16, rng, [0, M - 1])
    cols = np.concatenate([np.arange(12288, N), _sample(12288, 40, rng, [0, 12287])])
    ref, bnd = oracle_linear_rows(x, w, segs, rows, cols)
    assert_within_tol(out.cpu().numpy().astype(np.float64)[rows][:, cols], ref, bnd, f"ragged in launch N={N}")


@pytest.mark.parametrize("M,N,K", [(1536, 12300, 512), (512, 12288, 1040), (4096, 5120, 256), (4096, 5120, 48)])
def test_gemm_narrow_mfma_tiles(M, N, K):
    """Shapes whose 256 x 256 tiles would leave a partial last round run the MFMA
    GEMM with 256 x 128 tiles (nvfp4_gemm_form 2): 6 x 97 tiles with the last
    128-column tile holding 12 columns (1536, 12300); a k tail with rows not
    16-byte aligned (512, 12288, 1040); 16 x 40 tiles (4096, 5120), also with
    K = 48, below one k tile.  Sampled rows and columns within the oracle's
    tolerance."""
    assert nv.nvfp4_gemm_form(M, K, N) == 2
    rng = np.random.default_rng(3 * M + N + K)
    segs = [(0, 700), (700, N - 12), (N - 12, N)]
    w = np.concatenate([(0.02 * (1 + 2 * i) * rng.standard_normal((e - b, K), dtype=np.float32))
                        for i, (b, e) in enumerate(segs)])
    x = W.random_act(M + 2 * K, M, K, "student_t")
    rows = _sample(M, 16, rng, [0, 255, 256, M - 1])
    cols = _sample(N, 300, rng, [0, 127, 128, N - N % 128 - 1 if N % 128 else N - 129] + list(range(N - 12, N)))
    check_linear(x, w, segs, f"narrow MFMA tiles M={M} N={N} K={K}", rows, cols)


def test_gemm_narrow_and_wide_mfma_tiles_bit_identical():
    """The two MFMA forms run the same per-wave MFMA sequence on each output: the
    first module's columns of a 2048 x 8192 product (256 x 256 tiles, one full
    round) equal, bit for bit, the 2048 x 2048 product of that module alone
    (256 x 128 tiles), with a k tail (K = 1040)."""
    M, K, N, n1 = 2048, 1040, 8192, 2048
    assert nv.nvfp4_gemm_form(M, K, N) == 1 and nv.nvfp4_gemm_form(M, K, n1) == 2
    rng = np.random.default_rng(77)
    w = np.float32(0.02) * rng.standard_normal((N, K), dtype=np.float32)
    w[n1:] *= np.float32(3.0)
    x = W.random_act(78, M, K, "student_t")
    say(f"[gemm] narrow vs wide M={M} K={K} N={N}/{n1}")
    wide = gpu_linear(x, gpu_pack(w, [(0, n1), (n1, N)]))
    narrow = gpu_linear(x, gpu_pack(w[:n1], [(0, n1)]))
    assert torch.equal(wide[:, :n1], narrow), "256 x 128 tiles differ from 256 x 256 tiles"


def test_gemm_k_zero_and_m_zero():
    w = np.zeros((16, 0), np.float32)
    pw = gpu_pack(w, [(0, 16)])
    x = torch.zeros((3, 0), dtype=torch.bfloat16, device=DEV)
    out, _ = nv.linear(x, pw)
    torch.cuda.synchronize()
    assert out.shape == (3, 16) and torch.all(out == 0)
    d = W.tiny()
    pw = gpu_pack(d.w, d.segments)
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device=DEV)
    out, _ = nv.linear(x, pw)
    assert out.shape == (0, 128)


def test_gemm_output_leading_dimension_and_no_overwrite():
    d = W.tiny()
    pw = gpu_pack(d.w, d.segments)
    x = to_dev_bf16(d.x_bits)
    c, s, g = nv.quantize_act(x)
    big = torch.full((16, 160), 7.0, dtype=torch.float32, device=DEV)
    nv.gemm(c, s, g, pw, out=big[:, 16:144])
    torch.cuda.synchronize()
    ref, bnd = oracle_linear_rows(d.x_bits, d.w, d.segments)
    assert_within_tol(big[:, 16:144].cpu().numpy().astype(np.float64), ref, bnd, "ldo")
    assert torch.all(big[:, :16] == 7.0) and torch.all(big[:, 144:] == 7.0)


def _sample(n, k, rng, must=()):
    pick = set(int(v) for v in must)
    pick |= set(rng.choice(n, min(k, n), replace=False).tolist())
    return np.array(sorted(pick))


def test_gemm_prefill_gate_up_full_size():
    d = W.prefill_gate_up()
    rng = np.random.default_rng(1)
    rows = _sample(d.M, 40, rng, [0, 127, 128, d.M - 1])
    cols = _sample(d.N, 600, rng, [0, 17407, 17408, d.N - 1])
    check_linear(d.x_bits, d.w, d.segments, "prefill gate+up (sampled)", rows, cols)


def test_gemm_gdn_in_proj_full_size_and_negative_control():
    d = W.gdn_in_proj()
    rng = np.random.default_rng(2)
    rows = _sample(d.M, 40, rng, [0, d.M - 1])
    cols = _sample(d.N, 500, rng, list(range(12288, 12352)) + [0, 2047, 2048, 4095, 4096, 8191, 8192])
    pw, out = check_linear(d.x_bits, d.w, d.segments, "gdn in-proj (sampled)", rows, cols)
    # the mismatch: one global scale (the first module's) for every fused module
    g = pw.g_dec.cpu().numpy()
    say(f"[gemm] gdn module scale ratios {np.round(g / g[0], 3).tolist()}")
    assert g.max() / g.min() > 10
    x = to_dev_bf16(d.x_bits)
    c, s, ag = nv.quantize_act(x)
    wrong = nv.gemm(c, s, ag, pw, g_dec=pw.g_dec[:1].repeat(len(d.segments)).contiguous())
    torch.cuda.synchronize()
    ref, bnd = oracle_linear_rows(d.x_bits, d.w, d.segments, rows, cols)
    o = wrong.cpu().numpy().astype(np.float64)[rows][:, cols]
    ok = G.within_tol(o, ref, bnd)
    for i, (b, e) in enumerate(d.segments):
        sel = (cols >= b) & (cols < e)
        frac = float(np.mean(ok[:, sel]))
        say(f"[gemm]   mismatch segment {i}: within tolerance {frac:.3f}")
        if i == 0:
            assert frac == 1.0
        else:
            assert frac < 0.5


@functools.lru_cache(maxsize=1)
def _down_proj():
    return W.down_proj()


def test_gemm_down_proj_full_size():
    d = _down_proj()
    rng = np.random.default_rng(3)
    rows = _sample(d.M, 24, rng, [0, d.M - 1])
    cols = _sample(d.N, 400, rng, [0, d.N - 1])
    check_linear(d.x_bits, d.w, d.segments, "down proj (sampled)", rows, cols)


@pytest.mark.parametrize("calibrated", [False, True])
def test_quantizer_down_proj_activations_full_size(calibrated):
    """The standalone activation quantizer over the full 32768 x 17408 down
    projection input (the two-pass dynamic path the bench times, and a calibrated
    scale at 0.7 of the maximum, which saturates blocks): g_dec exact, codes and
    scales of 64 sampled rows (first and last included) bit-exact against the
    oracle with the same tensor maximum; the row holding the maximum is among
    them."""
    d = _down_proj()
    mag = d.x_bits & 0x7FFF
    at = int(np.argmax(mag))
    amax = float(W.bf16_to_f32(np.array([mag.flat[at]], np.uint16))[0])
    del mag
    if calibrated:
        amax = float(np.float32(amax) * np.float32(0.7))
    say(f"[quantizer full size] calibrated={calibrated} amax={amax}")
    x = to_dev_bf16(d.x_bits)
    am = torch.tensor([amax], dtype=torch.float32, device=DEV) if calibrated else None
    c, s, g = nv.quantize_act(x, am)
    torch.cuda.synchronize()
    del x
    rng = np.random.default_rng(17 + calibrated)
    rows = _sample(d.M, 64, rng, [0, at // d.K, d.M - 1])   # the row holding the maximum
    oc, os_, og, _ = Q.quantize(W.bf16_to_f32(d.x_bits[rows]), np.float32(amax))
    if calibrated:
        assert (os_ == 0x7E).any()   # the maximum's block saturates at E4M3 448
    assert float(g.cpu()[0]) == float(og)
    rows_t = torch.from_numpy(rows).to(DEV)
    assert np.array_equal(c.index_select(0, rows_t).cpu().numpy(), oc)
    assert np.array_equal(s.index_select(0, rows_t).cpu().numpy(), os_)


@pytest.mark.parametrize("M,N,K", [(24, 700, 1040), (32, 200, 5120), (100, 1500, 2064), (70, 100, 1040),
                                   (300, 2000, 512), (24, 5120, 10256), (100, 1500, 11664), (70, 100, 6144),
                                   (128, 5120, 17408), (40, 12300, 10256), (2100, 64, 1040), (2100, 60, 10256)])
def test_gemm_row_blocks_bit_identical_to_16_rows(M, N, K):
    """nvfp4_gemm's weight-streaming form for M > 16 (32-row passes: (24, 700),
    (32, 200), (24, 5120); 64-row: (100, 1500), (300, 2000), (128, 5120); 16-row
    passes for outputs of at most 8 strips: (70, 100), and with all four strips
    in one workgroup over 132 row blocks: (2100, 64), (2100, 60), the latter in
    the sixteen-wave order with a ragged last strip) gives, for every 16-row
    slice of the quantized activations, exactly the M <= 16 kernel's result on
    that slice, and the oracle's within tolerance.  For K > 5120 with fewer M <= 16
    workgroups than CUs the M <= 16 kernel splits the k tiles over sixteen waves,
    and the row blocks replay that order with two accumulator sets per wave of
    eight (1, 2 and 3 strips per workgroup at (100, 1500), (24, 5120) and
    (128, 5120)); the ragged last tile falls to the first set at K = 10256 (tile
    80, wave 0) and to the second at K = 11664 (tile 91, wave 11).  N = 12300
    (257 workgroups at M <= 16) keeps eight waves at K = 10256."""
    assert nv.nvfp4_gemm_form(M, K, N) == 0
    rng = np.random.default_rng(M * 7 + N + K)
    segs = [(0, N // 3), (N // 3, N)]
    w = np.concatenate([(0.02 * (1 + 3 * i) * rng.standard_normal((e - b, K))).astype(np.float32)
                        for i, (b, e) in enumerate(segs)])
    x_bits = W.random_act(M + 2 * K, M, K, "student_t")
    say(f"[row blocks] M={M} N={N} K={K}")
    pw = gpu_pack(w, segs)
    c, s, g = nv.quantize_act(to_dev_bf16(x_bits))
    out = nv.gemm(c, s, g, pw)
    for r0 in range(0, M, 16):
        part = nv.gemm(c[r0:r0 + 16], s[r0:r0 + 16], g, pw)
        assert torch.equal(part, out[r0:r0 + 16]), f"rows {r0}..{r0 + 15} differ from the 16-row kernel"
    torch.cuda.synchronize()
    rows = _sample(M, 24, rng, [0, 15, 16, M - 1])
    ref, bnd = oracle_linear_rows(x_bits, w, segs, rows=rows)
    assert_within_tol(out.cpu().numpy().astype(np.float64)[rows], ref, bnd, f"row blocks M={M} N={N}")
