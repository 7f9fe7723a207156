"""Pins for oracle/nvfp4.py: hand-worked fixtures, invariants, round trips, special blocks."""
import numpy as np
import pytest

from oracle import nvfp4 as Q
from oracle.formats import e2m1_value, e4m3_value, E4M3_POS
from golden_io import fp32_round, load_quant_fixtures
from workloads import bf16_to_f32, random_act, tiny

FIXTURES = load_quant_fixtures()


@pytest.mark.parametrize("fx", FIXTURES, ids=[f["name"] for f in FIXTURES])
def test_hand_worked_fixtures(fx):
    codes, scales, g_dec, _ = Q.quantize(fx["x"], fx["amax"])
    assert np.array_equal(scales, fx["scales"]), (scales, fx["scales"])
    assert np.array_equal(Q.unpack_codes(codes), fx["codes"]), (Q.unpack_codes(codes), fx["codes"])
    assert g_dec == fp32_round(fx["g_dec"])
    assert np.float32(g_dec).tobytes() == fp32_round(fx["g_dec"]).tobytes()


@pytest.mark.parametrize("fx", FIXTURES, ids=[f["name"] for f in FIXTURES])
def test_hand_worked_packed_bytes(fx):
    """The stored byte order (reading S12 of the format passage: two codes per byte, the
    even element in the low nibble): quantize's packed output equals the fixture's
    literal bytes, not just its unpacked nibbles."""
    codes, _, _, _ = Q.quantize(fx["x"], fx["amax"])
    assert codes.dtype == np.uint8 and codes.shape == fx["packed"].shape
    assert np.array_equal(codes, fx["packed"]), (codes, fx["packed"])


def test_unpack_codes_literal():
    """unpack_codes on literal bytes: 0x21 holds element 0 = 1 (low nibble) and element 1 = 2;
    0xF0 holds 0 then 0xF; 0x8A holds 0xA then 8."""
    got = Q.unpack_codes(np.array([[0x21, 0xF0, 0x8A]], np.uint8))
    assert got.tolist() == [[0x1, 0x2, 0x0, 0xF, 0xA, 0x8]]


def _tensors():
    t = tiny()
    yield "tiny_act", bf16_to_f32(t.x_bits)
    yield "tiny_w", t.w
    yield "student_t", bf16_to_f32(random_act(1, 33, 272, "student_t"))
    yield "uniform", bf16_to_f32(random_act(2, 7, 1024, "uniform", 1e-3))
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    x[:, 5] *= 1000
    x[3, 100:116] = 0
    yield "outliers", x


@pytest.mark.parametrize("name,x", list(_tensors()), ids=lambda v: v if isinstance(v, str) else "")
def test_invariants(name, x):
    codes, scales, g_dec, amax = Q.quantize(x)
    c = Q.unpack_codes(codes)
    R, K = x.shape
    mag = (c & 7).reshape(R, K // 16, 16)
    # scale codes never NaN, never negative
    assert np.all(scales <= 0x7E)
    # blocks with a normal scale (exponent field != 0) reach the largest magnitude 6
    normal = (scales >> 3) != 0
    assert np.all(mag.max(axis=2)[normal] == 7)
    # the block holding the tensor maximum gets the largest scale
    r, k = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert scales[r, k // 16] == 0x7E
    # sign bits follow the input
    assert np.array_equal((c >> 3).astype(bool), np.signbit(x))
    # decode error in normal-scale blocks: at most half the widest E2M1 gap (1,
    # between 4 and 6) times the block's decode scale, plus fp32 rounding slop
    xh = Q.dequantize(codes, scales, g_dec)
    s = e4m3_value(scales).repeat(16, axis=1) * np.float64(g_dec)
    nrm = normal.repeat(16, axis=1)
    assert np.all((np.abs(x - xh) <= s * (1 + 1e-5))[nrm])
    assert amax == np.max(np.abs(x))


def test_sign_symmetry():
    x = bf16_to_f32(random_act(4, 9, 160, "student_t"))
    c1, s1, g1, _ = Q.quantize(x)
    c2, s2, g2, _ = Q.quantize(-x)
    assert np.array_equal(s1, s2) and g1 == g2
    assert np.array_equal(c1 ^ 0x88, c2)


@pytest.mark.parametrize("j", [-20, -3, 0, 5, 30])
def test_power_of_two_scaling_invariance(j):
    x = bf16_to_f32(random_act(5, 12, 96, "normal"))
    c1, s1, g1, _ = Q.quantize(x)
    c2, s2, g2, _ = Q.quantize(x * np.float32(2.0 ** j))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert g2 == np.float32(g1 * np.float32(2.0 ** j))


@pytest.mark.parametrize("j", [-30, -4, 0, 3, 12])
def test_round_trip_of_representable_tensors(j):
    """Tensors built from codes: amax = 2688 * 2^j, every block's largest magnitude 6 and an
    arbitrary E4M3 scale code (normal or subnormal).  Encoding them returns the codes."""
    rng = np.random.default_rng(100 + j)
    R, B = 8, 24
    scales = rng.integers(1, 0x7F, size=(R, B)).astype(np.uint8)
    scales[0, 0] = 0x7E
    mags = rng.integers(0, 8, size=(R, B, 16))
    mags[:, :, 0] = 7
    signs = rng.integers(0, 2, size=(R, B, 16))
    codes = (signs << 3 | mags).astype(np.uint8).reshape(R, B * 16)
    x = (e2m1_value(codes).reshape(R, B, 16) * e4m3_value(scales)[:, :, None] * 2.0 ** j).reshape(R, B * 16)
    x32 = x.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), x)          # exactly representable
    pc, ps, g, amax = Q.quantize(x32)
    assert amax == np.float32(2688 * 2.0 ** j)
    assert np.array_equal(ps, scales)
    assert np.array_equal(Q.unpack_codes(pc), codes)
    assert np.array_equal(Q.dequantize(pc, ps, g), x)


def test_special_blocks():
    x = np.zeros((2, 64), np.float32)
    x[0, 16:32] = 0.7                   # all-equal block with a normal scale
    x[0, 32:48] = -3.0                  # the tensor maximum, all equal
    x[1, 48:64] = 1e-3                  # all-equal small block
    x[1, 0] = -0.0
    codes, scales, g, _ = Q.quantize(x)
    c = Q.unpack_codes(codes)
    assert scales[0, 0] == 0 and np.all(c[0, :16] == 0)
    assert np.all(c[0, 16:32] == 7) and np.all(c[0, 32:48] == 0xF) and scales[0, 2] == 0x7E
    assert (scales[1, 3] >> 3) != 0 and np.all(c[1, 48:64] == 7)
    assert c[1, 0] == 8
    z, zs, zg, _ = Q.quantize(np.zeros((3, 32), np.float32))
    assert zg == 0 and not z.any() and not zs.any()


def test_static_amax_equal_to_max_matches_dynamic():
    x = bf16_to_f32(random_act(6, 10, 64, "student_t"))
    a = Q.quantize(x)
    b = Q.quantize(x, float(np.max(np.abs(x))))
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_static_amax_saturates():
    x = bf16_to_f32(random_act(7, 4, 64, "normal"))
    amax = float(np.max(np.abs(x))) / 8
    codes, scales, _, _ = Q.quantize(x, amax)
    c = Q.unpack_codes(codes)
    big = np.abs(x) > amax
    assert np.all((c & 7)[big] == 7)
    r, k = np.nonzero(big)
    assert np.all(scales[r, k // 16] == 0x7E)


def test_fp32_subnormal_weights_scale_zero():
    """fp32 weights whose block maximum / 6 underflows to 0 get scale 0 and magnitude 0."""
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = np.float32(1e-45)          # smallest fp32 subnormal: t = fl(1e-45 / 6) = 0
    x[0, 16] = np.float32(1.0)
    codes, scales, g, _ = Q.quantize(x)
    assert scales[0, 0] == 0 and Q.unpack_codes(codes)[0, 0] == 0
    assert scales[0, 1] == 0x7E


def test_segments_have_independent_scales():
    rng = np.random.default_rng(8)
    w = np.concatenate([0.02 * rng.standard_normal((32, 64)), 0.4 * rng.standard_normal((16, 64))]).astype(np.float32)
    segs = [(0, 32), (32, 48)]
    c, s, g = Q.quantize_segments(w, segs)
    for i, (b, e) in enumerate(segs):
        c1, s1, g1, _ = Q.quantize(w[b:e])
        assert np.array_equal(c[b:e], c1) and np.array_equal(s[b:e], s1) and g[i] == g1
    assert g[1] > 10 * g[0]
    assert np.array_equal(Q.dequantize_segments(c, s, g, segs)[:32], Q.dequantize(c[:32], s[:32], g[0]))


def test_e4m3_positive_table_used_by_encoder_has_127_codes():
    assert len(E4M3_POS) == 127
