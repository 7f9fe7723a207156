"""The device conversion steps, over whole binary32 ranges, against the oracle's
format definitions (Summary page, Background, item 1: E2M1 elements, E4M3 block
scales; readings S1, S2, S6, S7: OCP formats, round to nearest even, saturating).

nvfp4_convert_sweep runs the same device helpers the encoders and the GEMMs use:
op 0 the E2M1 element conversion, op 1 the E4M3 conversion (block scales and the
FP8 KV codec), op 2 the exact E2M1 x E4M3 -> fp16 decode of the GEMMs.

For ops 0 and 1 every binary32 value of a sign-homogeneous range is converted on
the GPU in chunks; the test collects every index where the GPU output changes.
Rounding to the nearest value of an ascending table is a non-decreasing function
of the magnitude, and within one sign binary32 bit patterns order like their
magnitudes, so the oracle is constant on a run of bit patterns as soon as it
takes the same value at the run's first and last pattern.  Checking the oracle
at both ends of every constant run of the GPU output therefore proves the two
functions equal on the whole range.
"""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_block_act_amd as nv
from gpu_util import DEV, say
from oracle.formats import e2m1_encode, e2m1_value, e4m3_encode, e4m3_value

pytestmark = pytest.mark.gpu

CHUNK = 1 << 28
INF = 0x7F800000


def _as_f32(bits):
    return np.asarray(bits, dtype=np.uint64).astype(np.uint32).view(np.float32)


def oracle_e2m1(bits):
    v = _as_f32(bits)
    return ((np.signbit(v).astype(np.uint8) << 3) | e2m1_encode(np.abs(v))).astype(np.uint8)


def oracle_e4m3(bits):
    return e4m3_encode(_as_f32(bits)).astype(np.uint8)


def gpu_runs(op, lo, hi):
    """[(first bit pattern, value)] of every constant run of the GPU output over [lo, hi)."""
    out = torch.empty(CHUNK, dtype=torch.uint8, device=DEV)
    runs, prev = [], None
    for start in range(lo, hi, CHUNK):
        n = min(CHUNK, hi - start)
        nv.nvfp4_convert_sweep(op, start, n, out)
        c = out[:n]
        first = int(c[0])
        if prev is None or first != prev:
            runs.append((start, first))
        idx = torch.nonzero(c[1:] != c[:-1]).flatten()
        assert idx.numel() < 4096, "far more changes than a rounding function has"
        vals = c[idx + 1].tolist() if idx.numel() else []
        runs += [(start + i + 1, v) for i, v in zip(idx.tolist(), vals)]
        prev = int(c[n - 1])
    torch.cuda.synchronize()
    return runs


def check_range(op, lo, hi, oracle, what):
    say(f"[convert] op {op} {what}: bits [{lo:#010x}, {hi:#010x})")
    runs = gpu_runs(op, lo, hi)
    starts = np.array([r[0] for r in runs], np.uint64)
    ends = np.append(starts[1:], np.uint64(hi)) - np.uint64(1)
    vals = np.array([r[1] for r in runs], np.uint8)
    assert np.array_equal(oracle(starts), vals), f"{what}: run starts differ"
    assert np.array_equal(oracle(ends), vals), f"{what}: run ends differ"
    return runs


def test_e2m1_every_nonnegative_binary32():
    """Every binary32 in [0, +inf]: [0, 8] holds every E2M1 decision point; beyond
    it the conversion saturates at 6."""
    runs = check_range(0, 0, INF + 1, oracle_e2m1, "y >= 0")
    assert [v for _, v in runs] == list(range(8))               # 0, .5, 1, 1.5, 2, 3, 4, 6 in order


def test_e2m1_every_negative_binary32():
    runs = check_range(0, 0x80000000, 0x80000000 + INF + 1, oracle_e2m1, "y <= -0")
    assert [v for _, v in runs] == list(range(8, 16))


def test_e4m3_every_nonnegative_binary32():
    """Every binary32 in [0, +inf]: all 127 E4M3FN codes, subnormals included, ties to
    even, 448 and beyond (and +inf) saturating to 0x7E."""
    runs = check_range(1, 0, INF + 1, oracle_e4m3, "s >= 0")
    assert [v for _, v in runs] == list(range(0x7F))


def test_exact_decode_of_every_code_pair():
    """op 2: the GEMMs' fp16 decode of every E2M1 code times every finite E4M3 scale
    code equals the exact product (E2M1 x E4M3 has at most 6 significant bits and lies
    in [2^-10, 2688], so fp16 holds it exactly)."""
    n = 127 * 16
    out = torch.empty(2 * n, dtype=torch.uint8, device=DEV)
    nv.nvfp4_convert_sweep(2, 0, n, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.float16).astype(np.float64)
    i = np.arange(n)
    want = e2m1_value(i & 15) * e4m3_value((i >> 4) & 127)
    assert np.array_equal(got, want)
    # signed zeros: code 8 (-0) decodes to -0.0
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_convert_sweep_rejects_bad_ranges():
    out = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(nv.NVFP4Error) as e:
        nv.nvfp4_convert_sweep(0, 0xFFFFFFF8, 16, out)            # past 2^32
    assert e.value.status == 2
    with pytest.raises(nv.NVFP4Error) as e:
        nv.nvfp4_convert_sweep(3, 0, 16, out)
    assert e.value.status == 1
