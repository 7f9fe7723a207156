"""GPU parity of the activation quantizer: codes, scales and g_dec bit-exact with the oracle."""
import numpy as np
import pytest

from gpu_util import gpu_quantize, say
from golden_io import load_quant_fixtures
from oracle import nvfp4 as Q
from workloads import bf16_bits, bf16_to_f32, random_act, tiny, decode

pytestmark = pytest.mark.gpu


def check(bits, amax=None, what=""):
    say(f"[quant] {what} shape={bits.shape} amax={amax}")
    c, s, g = gpu_quantize(bits, amax)
    oc, os_, og, _ = Q.quantize(bf16_to_f32(bits), amax)
    assert np.array_equal(s, os_), f"{what}: {np.sum(s != os_)} scale mismatches"
    assert np.array_equal(c, oc), f"{what}: {np.sum(c != oc)} code byte mismatches"
    assert np.float32(g).tobytes() == np.float32(og).tobytes(), (g, og)


@pytest.mark.parametrize("fx", load_quant_fixtures(), ids=lambda f: f["name"])
def test_hand_worked_fixtures(fx):
    bits = bf16_bits(fx["x"])
    assert np.array_equal(bf16_to_f32(bits), fx["x"])          # fixture values are bf16-exact
    check(bits, fx["amax"], fx["name"])


def test_tiny_workload():
    check(tiny().x_bits, None, "tiny")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_workload_activations(M):
    check(decode(M=M).x_bits, None, f"decode M={M}")


@pytest.mark.parametrize("M,K,dist", [
    (1, 16, "normal"), (3, 48, "student_t"), (17, 272, "normal"), (100, 5136, "student_t"),
    (257, 1040, "uniform"), (64, 4112, "normal"),       # above the single-launch size: two-pass amax
    (700, 400, "student_t"),
    # 64 partial maxima, reduced inside the encode kernel / 65, reduced by their own kernel
    (1280, 1648, "student_t"), (1293, 1648, "student_t"),
])
def test_ragged_shapes_dynamic(M, K, dist):
    check(random_act(M * 7 + K, M, K, dist), None, f"ragged {M}x{K}")


@pytest.mark.parametrize("frac", [0.125, 1.0, 3.0])
def test_static_amax(frac):
    bits = random_act(5, 33, 320, "student_t")
    amax = float(np.max(np.abs(bf16_to_f32(bits)))) * frac
    check(bits, np.float32(amax), f"static x{frac}")
    big = random_act(6, 300, 1024, "normal")
    check(big, np.float32(2.5), "static large")


def test_every_bf16_block_maximum():
    """Every non-negative finite bf16 value appears as a block maximum.  The values are
    split by binade into tensors of 16 binades each, whose amax is their largest value,
    so every block lands inside the E4M3 range of its tensor's scale: this covers
    bmax / 6, the product with g_enc and the E4M3 rounding for all 32640 inputs."""
    rng = np.random.default_rng(77)
    allmax = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)   # 0 .. largest finite
    for lo in range(0, 0x7F80, 16 * 128):
        maxima = allmax[lo:lo + 16 * 128]
        nb = len(maxima)
        bm = bf16_to_f32(maxima)
        frac = rng.uniform(-1, 1, size=(nb, 15)).astype(np.float32)
        vals = np.concatenate([bm[:, None], frac * bm[:, None]], axis=1)
        perm = rng.permuted(np.tile(np.arange(16), (nb, 1)), axis=1)
        bits = bf16_bits(np.take_along_axis(vals, perm, axis=1))
        bits = bits.reshape(-1, 64 * 16)
        check(bits, None, f"bf16 maxima from 0x{lo:04x}")
    # and one tensor holding all of them (most blocks underflow to scale 0)
    bits = allmax.reshape(-1, 8 * 16)
    check(bits, np.float32(3.0), "all maxima, static 3.0")


def test_every_element_for_every_scale_code():
    """Under g_enc = 1 (amax 2688), a block with maximum 6 * E4M3(c) gets scale code c;
    its other 15 elements sweep every non-negative bf16 value up to that maximum."""
    from oracle.formats import E4M3_POS
    rows = []
    for c in range(1, 0x7F):
        top = np.float32(6 * E4M3_POS[c])
        tb = int(bf16_bits(np.array([top]))[0])
        vals = np.arange(0, tb + 1, dtype=np.uint32).astype(np.uint16)
        vals = np.concatenate([vals, vals[:(-len(vals)) % 15]])
        blk = vals.reshape(-1, 15)
        blk = np.concatenate([np.full((blk.shape[0], 1), tb, np.uint16), blk], axis=1)
        rows.append(blk)
    allb = np.concatenate(rows)
    head = np.zeros((1, 16), np.uint16)
    head[0, 0] = int(bf16_bits(np.array([2688.0], np.float32))[0])
    allb = np.concatenate([head, allb])
    pad = (-allb.shape[0]) % 128
    allb = np.concatenate([allb, np.zeros((pad, 16), np.uint16)]).reshape(-1, 128 * 16)
    check(allb, None, "element sweep per scale code")
    say(f"[quant] element sweep size {allb.size}")


def test_negative_values_and_signed_zero():
    bits = random_act(9, 8, 64, "normal")
    bits[0, :16] = 0x8000          # a block of -0.0
    bits[1, 3] = 0x8000
    check(bits, None, "signed zeros")


def test_all_zero_and_empty():
    check(np.zeros((5, 32), np.uint16), None, "all zero")
    import torch
    import nvfp4_w4a4_block_act_amd as nv
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda:0")
    c, s, g = nv.quantize_act(x)
    torch.cuda.synchronize()
    assert c.numel() == 0 and float(g[0]) == 0.0


def test_leading_dimension():
    import torch
    import nvfp4_w4a4_block_act_amd as nv
    from gpu_util import to_dev_bf16
    bits = random_act(12, 20, 200, "normal")
    full = to_dev_bf16(bits)
    view = full[:, 8:8 + 160]                   # ldx = 200, 16-byte aligned start
    c, s, g = nv.quantize_act(view)
    torch.cuda.synchronize()
    oc, os_, og, _ = Q.quantize(bf16_to_f32(bits[:, 8:168]))
    assert np.array_equal(c.cpu().numpy(), oc) and np.array_equal(s.cpu().numpy(), os_)
    assert np.float32(g.cpu().numpy()[0]) == og


@pytest.mark.parametrize("static", [False, True])
def test_leading_dimension_two_pass(static):
    """A strided view above the single-launch size (the amax pass, its reduction and
    the one-block-per-thread encode all address rows through ldx)."""
    import torch
    import nvfp4_w4a4_block_act_amd as nv
    from gpu_util import to_dev_bf16
    bits = random_act(13, 600, 432, "student_t")
    full = to_dev_bf16(bits)
    view = full[:, 16:16 + 400]                 # ldx = 432, 32-byte aligned start
    sub = bf16_to_f32(bits[:, 16:416])
    amax = np.float32(0.5 * np.max(np.abs(sub))) if static else None
    am = torch.tensor([float(amax)], dtype=torch.float32, device="cuda:0") if static else None
    c, s, g = nv.quantize_act(view, am)
    torch.cuda.synchronize()
    oc, os_, og, _ = Q.quantize(sub, amax)
    assert np.array_equal(c.cpu().numpy(), oc) and np.array_equal(s.cpu().numpy(), os_)
    assert np.float32(g.cpu().numpy()[0]) == og


def test_all_zero_two_pass():
    check(np.zeros((300, 1024), np.uint16), None, "all zero, two-pass")


@pytest.mark.parametrize("static", [False, True])
def test_streamed_tensor_strided(static):
    """A strided view whose bf16 bytes exceed 256 MB (4099 x 32784 inside rows of
    32832; K % 128 != 0), so the maximum and encode passes take their
    non-temporal instances: g_dec exact, and the codes and scales of 48 sampled
    rows (the first, the last and the one holding the maximum among them)
    bit-exact against the oracle with the same tensor maximum (half of it when
    calibrated, which saturates blocks)."""
    import torch
    import nvfp4_w4a4_block_act_amd as nv
    from gpu_util import to_dev_bf16
    M, K, ldx = 4099, 32784, 32832
    assert M * K * 2 > 256 << 20
    bits = random_act(21, M, ldx, "normal")
    view_bits = bits[:, 16:16 + K]
    mag = view_bits & 0x7FFF
    at = int(np.argmax(mag))
    amax = float(bf16_to_f32(np.array([mag.flat[at]], np.uint16))[0])
    del mag
    if static:
        amax = float(np.float32(amax) * np.float32(0.5))
    say(f"[quant streamed] static={static} amax={amax}")
    full = to_dev_bf16(bits)
    am = torch.tensor([amax], dtype=torch.float32, device="cuda:0") if static else None
    c, s, g = nv.quantize_act(full[:, 16:16 + K], am)
    torch.cuda.synchronize()
    del full
    rng = np.random.default_rng(22 + static)
    rows = np.unique(np.concatenate([rng.choice(M, 45, replace=False), [0, M - 1, at // K]]))
    oc, os_, og, _ = Q.quantize(bf16_to_f32(np.ascontiguousarray(view_bits[rows])), np.float32(amax))
    if static:
        assert (os_ == 0x7E).any()
    assert np.float32(g.cpu().numpy()[0]) == og
    rows_t = torch.from_numpy(rows).to("cuda:0")
    assert np.array_equal(c.index_select(0, rows_t).cpu().numpy(), oc)
    assert np.array_equal(s.index_select(0, rows_t).cpu().numpy(), os_)
