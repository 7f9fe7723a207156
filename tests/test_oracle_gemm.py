"""Pins for oracle/gemm.py: exact integer path, brute force with rationals, textbook
reduction, the per-segment epilogue and the negative control (the mismatch)."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import gemm as G
from oracle import nvfp4 as Q
from oracle.formats import e2m1_value, e4m3_value
from workloads import bf16_to_f32, random_act, random_weight, tiny


def _encode_case(x_bits, w, segs):
    a_c, a_s, a_g, _ = Q.quantize(bf16_to_f32(x_bits))
    w_c, w_s, w_g = Q.quantize_segments(w, segs)
    a_hat = Q.dequantize(a_c, a_s, a_g)
    w_hat = Q.dequantize_segments(w_c, w_s, w_g, segs)
    rows_g = np.concatenate([np.full(e - b, w_g[i]) for i, (b, e) in enumerate(segs)])
    return a_c, a_s, a_g, w_c, w_s, w_g, rows_g, a_hat, w_hat


def test_exact_int_matches_f64_on_tiny_workload():
    t = tiny()
    a_c, a_s, a_g, w_c, w_s, w_g, rows_g, a_hat, w_hat = _encode_case(t.x_bits, t.w, t.segments)
    ref = G.gemm_f64(a_hat, w_hat)
    ex = G.gemm_exact(a_c, a_s, a_g, w_c, w_s, rows_g)
    bnd = G.gemm_bound(a_hat, w_hat)
    assert np.all(np.abs(ref - ex) <= 1e-12 * bnd)


def test_exact_int_matches_f64_with_segments_and_long_k():
    x = random_act(11, 5, 4096 + 16 * 7, "student_t")
    w = np.concatenate([random_weight(12, 9, 4096 + 112), random_weight(13, 23, 4096 + 112, 0.3)])
    segs = [(0, 9), (9, 32)]
    a_c, a_s, a_g, w_c, w_s, w_g, rows_g, a_hat, w_hat = _encode_case(x, w, segs)
    ref = G.gemm_f64(a_hat, w_hat)
    ex = G.gemm_exact(a_c, a_s, a_g, w_c, w_s, rows_g)
    assert np.all(np.abs(ref - ex) <= 1e-12 * G.gemm_bound(a_hat, w_hat))


def test_brute_force_rationals_tiny():
    """out[m, n] as an exact sum of Fraction products of the codes' values, then
    times the exact global scales; the float64 GEMM must agree to rounding."""
    x = random_act(21, 3, 32, "normal")
    w = random_weight(22, 5, 32)
    segs = [(0, 2), (2, 5)]
    a_c, a_s, a_g, w_c, w_s, w_g, rows_g, a_hat, w_hat = _encode_case(x, w, segs)
    ac, wc = Q.unpack_codes(a_c), Q.unpack_codes(w_c)
    ref = G.gemm_f64(a_hat, w_hat)
    bnd = G.gemm_bound(a_hat, w_hat)
    for m in range(3):
        for n in range(5):
            s = Fraction(0)
            for k in range(32):
                av = Fraction(float(e2m1_value(ac[m, k]))) * Fraction(float(e4m3_value(a_s[m, k // 16])))
                wv = Fraction(float(e2m1_value(wc[n, k]))) * Fraction(float(e4m3_value(w_s[n, k // 16])))
                s += av * wv
            s *= Fraction(float(a_g)) * Fraction(float(rows_g[n]))
            assert abs(float(s) - ref[m, n]) <= 1e-14 * bnd[m, n]


def test_textbook_reduction_unit_scales():
    """All scales 1.0 (code 0x38) and unit globals: the GEMM is a plain product of E2M1 values."""
    rng = np.random.default_rng(31)
    M, N, K = 6, 10, 64
    ac = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    wc = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    pack = lambda c: (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    a_hat = Q.dequantize(pack(ac), np.full((M, K // 16), 0x38, np.uint8), np.float32(1))
    w_hat = Q.dequantize(pack(wc), np.full((N, K // 16), 0x38, np.uint8), np.float32(1))
    lut2 = np.array([0, 1, 2, 3, 4, 6, 8, 12], np.int64)          # 2 * E2M1 magnitude
    ia = np.where(ac >= 8, -1, 1) * lut2[ac & 7]
    iw = np.where(wc >= 8, -1, 1) * lut2[wc & 7]
    assert np.array_equal(G.gemm_f64(a_hat, w_hat), (ia @ iw.T) / 4.0)


def test_single_segment_equals_unsegmented_and_equal_scales():
    x = random_act(41, 4, 128, "normal")
    w = random_weight(42, 24, 128)
    _, _, _, _, _, _, _, a1, w1 = _encode_case(x, w, [(0, 24)])
    c, s, g = Q.quantize_segments(w, [(0, 24)])
    c0, s0, g0, _ = Q.quantize(w)
    assert np.array_equal(c, c0) and np.array_equal(s, s0) and g[0] == g0
    # with equal global scales, splitting into segments changes nothing
    segs = [(0, 8), (8, 24)]
    wc, ws, _ = Q.quantize_segments(np.concatenate([w[:8], w[:8], w[:8]]), [(0, 8), (8, 24)])
    ws_one = Q.quantize(w[:8])
    assert np.array_equal(wc[8:16], ws_one[0]) and np.array_equal(ws[16:24], ws_one[1])


def _gdn_like(seed=51, M=16, K=256):
    """The fused GDN input projection's segment structure, scaled down for the CPU."""
    sizes = [64, 64, 128, 128, 32, 32]
    f = [1.0, 1.0, 0.5, 2.0, 10.0, 0.5]
    rng = np.random.default_rng(seed)
    x = random_act(seed, M, K, "normal")
    parts, segs, pos = [], [], 0
    for n, fi in zip(sizes, f):
        parts.append((0.02 * fi * rng.standard_normal((n, K))).astype(np.float32))
        segs.append((pos, pos + n))
        pos += n
    return x, np.concatenate(parts), segs


def test_negative_control_global_scale_mismatch():
    """Decoding every row of a fused weight with the first module's global scale (the
    mismatch) must fail the tolerance on each segment whose scale differs, while the
    per-segment epilogue passes by construction."""
    x, w, segs = _gdn_like()
    a_c, a_s, a_g, w_c, w_s, w_g, rows_g, a_hat, w_hat = _encode_case(x, w, segs)
    ref = G.gemm_f64(a_hat, w_hat)
    bnd = G.gemm_bound(a_hat, w_hat)
    wrong_rows = np.full_like(rows_g, w_g[0])
    bad = G.gemm_exact(a_c, a_s, a_g, w_c, w_s, wrong_rows)
    good = G.gemm_exact(a_c, a_s, a_g, w_c, w_s, rows_g)
    assert np.all(G.within_tol(good, ref, bnd))
    for i, (b, e) in enumerate(segs):
        ok = G.within_tol(bad[:, b:e], ref[:, b:e], bnd[:, b:e])
        ratio = w_g[i] / w_g[0]
        if i == 0:
            assert np.all(ok)
        else:
            assert abs(ratio - 1) > 1e-3
            assert np.mean(ok) < 0.5, (i, ratio, np.mean(ok))
    assert max(w_g) / min(w_g) > 10            # amax ratios up to ~20x across modules


def test_within_tol_rejects_errors_above_bound():
    x = random_act(61, 4, 64, "normal")
    w = random_weight(62, 8, 64)
    _, _, _, _, _, _, _, a_hat, w_hat = _encode_case(x, w, [(0, 8)])
    ref = G.gemm_f64(a_hat, w_hat)
    bnd = G.gemm_bound(a_hat, w_hat)
    assert np.all(G.within_tol(ref + 0.9e-5 * bnd, ref, bnd))
    assert not np.any(G.within_tol(ref + 1.1e-5 * bnd + 2e-6, ref, bnd))
