"""Pins of oracle/swiglu.py (CPU): silu's closed forms and identities, and the
bf16 rounding against torch's float32 -> bfloat16 cast (round to nearest
even) on values exactly representable in float32, plus hand-made midpoints."""
import numpy as np
import torch

from oracle import swiglu as S


def test_silu_closed_forms():
    assert S.silu(0.0) == 0.0
    assert abs(S.silu(1.0) - 1.0 / (1.0 + np.exp(-1.0))) < 1e-16
    z = np.linspace(-30, 30, 601)
    # silu(z) - silu(-z) = z and silu(z) -> z, 0 at +-infinity
    assert np.allclose(S.silu(z) - S.silu(-z), z, rtol=0, atol=1e-13)
    assert abs(S.silu(50.0) - 50.0) < 1e-18 * 50 + 1e-12 and abs(S.silu(-50.0)) < 1e-19
    assert S.silu(-1000.0) == 0.0


def test_bf16_rounding_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(200000) * 10.0 ** rng.integers(-6, 6, 200000),
                        [0.0, -0.0, 1.0, -2.5, 3.0e38]]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(S.bf16_round_bits(v.astype(np.float64)), ref)


def test_bf16_rounding_decides_on_the_exact_value():
    one = 1.0
    ulp = 2.0 ** -7                    # bf16 spacing in [1, 2)
    mid = one + ulp / 2                # exact midpoint: ties to even -> 1.0 (0x3F80)
    assert S.bf16_round_bits(mid) == 0x3F80
    assert S.bf16_round_bits(mid + 2.0 ** -40) == 0x3F81     # above the midpoint (not float32-representable)
    assert S.bf16_round_bits(one + 1.5 * ulp) == 0x3F82      # tie between 0x3F81 and 0x3F82 -> even
    assert S.bf16_round_bits(-(mid + 2.0 ** -40)) == 0xBF81


def test_swiglu_bf16_definition():
    g = np.array([0.0, 1.0, -3.0, 20.0], np.float64)
    u = np.array([5.0, 2.0, 0.5, -1.0], np.float64)
    h = S.swiglu_bf16(g, u)
    exp = S.bf16_round_bits(g / (1 + np.exp(-g)) * u)
    assert np.array_equal(h, exp) and h[0] == 0
