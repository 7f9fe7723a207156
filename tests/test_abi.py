"""The C-ABI library loads, exports every symbol its header declares, and rejects
bad arguments on the host (no GPU needed: these calls never reach a launch)."""
import ctypes
import os
import re

import pytest

import nvfp4_w4a4_block_act_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = nv.lib()
    names = declared_functions()
    assert len(names) >= 9, names
    for n in names:
        assert hasattr(lib, n), n
        assert getattr(nv, n, None) is not None, f"binding lacks {n}"


def test_version_and_status_strings():
    """The library reports the header's ABI version (the check build() makes)."""
    with open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "nvfp4.h")) as f:
        want = int(re.search(r"#define NVFP4_ABI_VERSION (\d+)", f.read()).group(1))
    assert want == 3 and nv.nvfp4_abi_version() == want
    for s in range(7):
        assert nv.nvfp4_status_str(s)
    assert nv.nvfp4_status_str(99) == "unknown status"


def test_packed_sizes():
    assert nv.nvfp4_packed_weight_bytes(12288, 5120) == (12288 * 5120 // 2, 12288 * 5120 // 16)
    # N padded to 16, K to 128
    assert nv.nvfp4_packed_weight_bytes(37, 48) == (48 * 128 // 2, 48 * 128 // 16)
    with pytest.raises(nv.NVFP4Error) as e:
        nv.nvfp4_packed_weight_bytes(16, 24)
    assert e.value.status == 2


# fake device addresses: validation must reject before anything dereferences them
A = 1 << 40


def q(x=A, M=4, K=32, ldx=32, amax=None, codes=A + (1 << 20), scales=A + (2 << 20), g=A + (3 << 20),
      ws=None, wsb=0):
    return nv.lib().nvfp4_quantize_act(x, M, K, ldx, amax, codes, scales, g, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), 1), (dict(K=24), 2), (dict(K=32, ldx=16), 2), (dict(g=None), 1), (dict(x=None), 1),
    (dict(codes=None), 1), (dict(x=A + 8), 3), (dict(scales=A + (2 << 20) + 4), 3), (dict(ldx=36), 3),
    (dict(codes=A + 16), 1),                                      # codes overlap x
    (dict(ldx=1 << 31), 2), (dict(ldx=1 << 62), 2),               # leading dimension bound (no overflow)
    (dict(M=4096, K=4096, ldx=4096, codes=A + (64 << 20), scales=A + (80 << 20), g=A + (96 << 20)), 5),
    (dict(amax=A + (3 << 20)), 1),                                # calibrated amax aliases g_dec
    (dict(M=4096, K=4096, ldx=4096, codes=A + (64 << 20), scales=A + (80 << 20), g=A + (96 << 20),
          ws=A + (128 << 20), wsb=4096), 5),                      # partial maxima only, no room for the maximum
    (dict(M=4096, K=4096, ldx=4096, codes=A + (64 << 20), scales=A + (80 << 20), g=A + (96 << 20),
          ws=A + (64 << 20) + 4096, wsb=1 << 20), 1),             # workspace inside the codes
])
def test_quantize_act_validation(kw, status):
    assert q(**kw) == status


def test_quantize_workspace_query():
    assert nv.nvfp4_quantize_act_workspace_bytes(16, 5120) == 0
    assert nv.nvfp4_quantize_act_workspace_bytes(8192, 5120) > 4096
    assert nv.nvfp4_linear_workspace_bytes(8192, 5120) == nv.nvfp4_quantize_act_workspace_bytes(8192, 5120)


def segs(pairs):
    arr = (nv.Segment * max(1, len(pairs)))()
    for i, (b, e) in enumerate(pairs):
        arr[i].n_begin, arr[i].n_end = b, e
    return arr


def g(a=A, sa=A + (1 << 20), ag=A + (2 << 20), M=4, K=32, wc=A + (3 << 20), ws=A + (4 << 20), N=32,
      sg=((0, 32),), wg=A + (5 << 20), out=A + (6 << 20), ldo=32):
    s = segs(list(sg))
    return nv.lib().nvfp4_gemm(a, sa, ag, M, K, wc, ws, N, s, wg, len(sg), out, ldo, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), 1), (dict(N=0, sg=((0, 1),)), 1), (dict(K=8), 2), (dict(ldo=16), 2),
    (dict(sg=((0, 16),)), 4), (dict(sg=((0, 16), (17, 32))), 4), (dict(sg=((0, 16), (16, 16), (16, 32))), 4),
    (dict(sg=tuple((i, i + 1) for i in range(17)), N=17, ldo=17), 4), (dict(sg=()), 4),
    (dict(a=None), 1), (dict(wg=None), 1), (dict(out=A + (6 << 20) + 4), 3), (dict(wc=A + 8), 3),
    (dict(out=A + (3 << 20) + 256), 1),                           # out overlaps the weight codes
    (dict(M=1 << 20, K=8192), 2),                                 # MFMA path: activation codes reach 4 GiB
    (dict(M=32, N=1 << 20, K=8192, sg=((0, 1 << 20),), ldo=1 << 20), 2),   # packed weight codes reach 4 GiB
    (dict(ldo=1 << 31), 2), (dict(ldo=1 << 62), 2),
])
def test_gemm_validation(kw, status):
    assert g(**kw) == status


def test_gemm_empty_m_is_noop():
    assert g(M=0) == 0


def p(w=A, N=32, K=32, ldw=32, sg=((0, 32),), wc=A + (1 << 20), ws=A + (2 << 20), wg=A + (3 << 20),
      work=A + (4 << 20), workb=4096):
    s = segs(list(sg))
    return nv.lib().nvfp4_pack_weight(w, N, K, ldw, s, len(sg), wc, ws, wg, work, workb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(N=0, sg=((0, 1),)), 1), (dict(K=40), 2), (dict(ldw=16), 2), (dict(sg=((0, 31),)), 4),
    (dict(w=A + 4), 3), (dict(workb=0), 5), (dict(work=None), 5), (dict(wc=A + 64), 1), (dict(ldw=1 << 31), 2),
    (dict(wg=A + (4 << 20) + 16), 1),                              # workspace holds w_g_dec
])
def test_pack_validation(kw, status):
    assert p(**kw) == status


def lin(x=A, M=4, K=32, ldx=32, amax=None, ac=A + (1 << 20), as_=A + (2 << 20), ag=A + (3 << 20),
        wc=A + (4 << 20), ws=A + (5 << 20), N=32, sg=((0, 32),), wg=A + (6 << 20), out=A + (7 << 20), ldo=32,
        work=None, workb=0):
    s = segs(list(sg))
    return nv.lib().nvfp4_linear(x, M, K, ldx, amax, ac, as_, ag, wc, ws, N, s, wg, len(sg), out, ldo, work, workb,
                                 None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), 1), (dict(K=24), 2), (dict(ldo=16), 2), (dict(sg=((0, 16),)), 4), (dict(ag=None), 1),
    (dict(x=None), 1), (dict(out=A + 4), 3), (dict(ldx=36), 3), (dict(out=A + (4 << 20) + 128), 1),
    (dict(M=4096, K=4096, ldx=4096, ac=A + (64 << 20), as_=A + (80 << 20), ag=A + (96 << 20), wc=A + (128 << 20),
          ws=A + (160 << 20), wg=A + (192 << 20), out=A + (256 << 20)), 5),
    (dict(M=1 << 20, K=8192, ldx=8192), 2),                      # MFMA path: activation codes reach 4 GiB
    (dict(ldx=1 << 31), 2), (dict(ldo=1 << 62), 2),
])
def test_linear_validation(kw, status):
    assert lin(**kw) == status


def test_linear_validates_everything_before_any_launch():
    """Empty K with a bad output, and a dynamic-mode workspace that overlaps an input,
    are rejected on the host.  (Had anything been launched first, this machine's HIP
    runtime would have turned it into NVFP4_EHIP instead.)"""
    assert lin(x=None, K=0, out=None) == 1
    assert lin(x=None, K=0, out=A + (7 << 20) + 4) == 3
    big = dict(M=4096, K=4096, ldx=4096, ac=A + (64 << 20), as_=A + (80 << 20), ag=A + (96 << 20),
               wc=A + (128 << 20), ws=A + (160 << 20), wg=A + (192 << 20), out=A + (256 << 20))
    wsb = nv.nvfp4_linear_workspace_bytes(4096, 4096)
    assert lin(work=A + 64, workb=wsb, **big) == 1                 # workspace inside x
    assert lin(work=A + (128 << 20), workb=wsb, **big) == 1        # workspace inside the weight codes
    assert lin(work=A + (300 << 20) + 4, workb=wsb, **big) == 3    # misaligned workspace


@pytest.mark.parametrize("call", [
    lambda: q(g=A + (3 << 20) + 4),                                # g_dec_out
    lambda: q(amax=A + (4 << 20) + 8),                             # calibrated amax
    lambda: g(ag=A + (2 << 20) + 4),                               # activation g_dec
    lambda: g(wg=A + (5 << 20) + 8),                               # per-module g_dec
    lambda: nv.lib().nvfp4_quantize_stats(A, 4, 32, 32, A + (1 << 20), A + (2 << 20) + 4, None),   # counts
    lambda: nv.lib().nvfp4_swiglu(A + 4, 4, 64, 128, A + (1 << 20), 64, None),                     # gu
    lambda: nv.lib().nvfp4_swiglu(A, 4, 64, 128, A + (1 << 20) + 2, 64, None),                     # h
    lambda: nv.lib().nvfp4_amax_observe(A, 4, 32, 32, A + (1 << 20) + 4, A + (2 << 20), 4096, None),
    lambda: nv.lib().nvfp4_kv_fp8_encode(A, 64, A + (1 << 20) + 4, A + (2 << 20), None),
])
def test_every_pointer_is_checked_for_alignment(call):
    assert call() == 3


def _no_gpu_here():
    import torch
    return not os.path.exists("/dev/kfd") and not torch.cuda.is_available()


def test_runtime_rejection_maps_to_ehip():
    """On a machine without a GPU the HIP runtime rejects every launch: a call whose
    arguments pass validation returns NVFP4_EHIP (skipped where a GPU exists, since the
    fake addresses must never reach a real launch)."""
    if not _no_gpu_here():
        pytest.skip("a GPU is present; the fake device addresses must not be launched on")
    assert g() == 6
    assert q() == 6
    assert lin() == 6


def gu_pack(w=A, I=128, K=32, ldw=32, wc=A + (1 << 20), ws=A + (2 << 20), wg=A + (3 << 20), work=A + (4 << 20),
            workb=4096):
    return nv.lib().nvfp4_pack_weight_gate_up(w, I, K, ldw, wc, ws, wg, work, workb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(I=0), 1), (dict(I=96), 2), (dict(K=40), 2), (dict(K=0), 2), (dict(ldw=16), 2), (dict(w=A + 4), 3),
    (dict(workb=0), 5), (dict(wg=None), 1), (dict(wc=A + 64), 1), (dict(ldw=1 << 40), 2),
])
def test_pack_gate_up_validation(kw, status):
    assert gu_pack(**kw) == status


def swq(a=A, sa=A + (1 << 20), ag=A + (2 << 20), M=32, K=32, wc=A + (3 << 20), ws=A + (4 << 20), I=128,
        wg=A + (5 << 20), amax=A + (6 << 20), hc=A + (7 << 20), hs=A + (8 << 20), hg=A + (9 << 20)):
    return nv.lib().nvfp4_gemm_swiglu_quantize(a, sa, ag, M, K, wc, ws, I, wg, amax, hc, hs, hg, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), 1), (dict(I=64), 2), (dict(K=8), 2), (dict(amax=None), 1), (dict(hg=None), 1),
    (dict(a=None), 1), (dict(hc=A + 8), 3), (dict(hc=A + (3 << 20) + 256), 1),
    (dict(M=1 << 20, K=8192), 2),                                 # activation codes reach 4 GiB
])
def test_gemm_swiglu_quantize_validation(kw, status):
    assert swq(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), 1), (dict(ldgu=100), 2), (dict(ldh=10), 2), (dict(gu=None), 1), (dict(h=A + 64), 1),
    (dict(M=0), 0), (dict(ldgu=1 << 31), 2), (dict(ldh=1 << 62), 2),
])
def test_swiglu_validation(kw, status):
    a = dict(gu=A, M=4, I=64, ldgu=128, h=A + (1 << 20), ldh=64)
    a.update(kw)
    assert nv.lib().nvfp4_swiglu(a["gu"], a["M"], a["I"], a["ldgu"], a["h"], a["ldh"], None) == status


@pytest.mark.parametrize("fn", ["encode", "decode"])
def test_kv_fp8_validation(fn):
    f = nv.lib().nvfp4_kv_fp8_encode if fn == "encode" else nv.lib().nvfp4_kv_fp8_decode
    assert f(A, -1, A + (1 << 20), A + (2 << 20), None) == 1
    assert f(A, 0, None, None, None) == 0                          # empty: nothing to do
    assert f(None, 16, A + (1 << 20), A + (2 << 20), None) == 1
    assert f(A, 16, None, A + (2 << 20), None) == 1
    assert f(A + 4, 16, A + (1 << 20), A + (2 << 20), None) == 3
    assert f(A, 64, A + (1 << 20), A + 16, None) == 1               # output overlaps input
    assert f(A, 1 << 48, A + (1 << 20), A + (2 << 20), None) == 2   # size bound


def test_observe_and_stats_validation():
    lib = nv.lib()
    wsb = nv.nvfp4_amax_observe_workspace_bytes(4, 32)
    assert wsb > 0
    assert lib.nvfp4_amax_observe(A, 4, 24, 32, A + (1 << 20), A + (2 << 20), wsb, None) == 2
    assert lib.nvfp4_amax_observe(A, 4, 32, 32, None, A + (2 << 20), wsb, None) == 1
    assert lib.nvfp4_amax_observe(A, 4, 32, 32, A + (1 << 20), A + (2 << 20), 0, None) == 5
    assert lib.nvfp4_amax_observe(A + 8, 4, 32, 32, A + (1 << 20), A + (2 << 20), wsb, None) == 3
    assert lib.nvfp4_amax_observe(A, 0, 32, 32, A + (1 << 20), None, 0, None) == 0
    assert lib.nvfp4_amax_observe(A, 4, 32, 1 << 31, A + (1 << 20), A + (2 << 20), wsb, None) == 2
    assert lib.nvfp4_quantize_stats(A, 4, 24, 32, A + (1 << 20), A + (2 << 20), None) == 2
    assert lib.nvfp4_quantize_stats(A, 4, 32, 32, None, A + (2 << 20), None) == 1
    assert lib.nvfp4_quantize_stats(A, 4, 32, 32, A + (1 << 20), A + 64, None) == 1   # counts overlap x
    assert lib.nvfp4_quantize_stats(A, 4, 32, 1 << 62, A + (1 << 20), A + (2 << 20), None) == 2


def test_binding_has_no_cpu_fallback(monkeypatch):
    """With the library path pointing nowhere, the binding raises instead of computing."""
    monkeypatch.setattr(nv, "_LIB", None)
    monkeypatch.setattr(nv, "LIB_PATH", "/nonexistent/libnvfp4_w4a4.so")
    with pytest.raises(ImportError):
        nv.lib()


def test_convenience_layer_stream_must_be_a_torch_stream():
    """The allocating helpers take a torch.cuda.Stream (their tensors are allocated
    on it); a raw handle is refused before anything is touched."""
    for fn, args in [(nv.linear, (None, None)), (nv.quantize_act, (None,)), (nv.gemm, (None, None, None, None)),
                     (nv.pack_weight, (None,))]:
        with pytest.raises(TypeError):
            fn(*args, stream=12345)


def test_gemm_form_query():
    """nvfp4_gemm_form: the skinny GEMM for M <= 16 and wherever too few
    256 x 256 tiles would fill the chip, the MFMA GEMM for the prefill shapes
    (2: its 256 x 128 tiles where 256 x 256 tiles leave a partial last round)."""
    assert nv.nvfp4_gemm_form(-1, 16, 16) == -1
    assert nv.nvfp4_gemm_form(16, 5120, 12288) == 0
    assert nv.nvfp4_gemm_form(17, 5120, 12288) == 0
    assert nv.nvfp4_gemm_form(512, 5120, 12288) == 2         # 192 narrow tiles instead of 96 wide
    assert nv.nvfp4_gemm_form(1024, 5120, 12288) == 1        # 192 wide tiles: one round either way
    assert nv.nvfp4_gemm_form(4096, 5120, 5120) == 2         # 320 wide tiles: a partial second round
    assert nv.nvfp4_gemm_form(8192, 5120, 34816) == 1
    assert nv.nvfp4_gemm_form(4096, 5120, 12352) == 1
    assert nv.nvfp4_gemm_form(32768, 17408, 5120) == 1


def test_read_probe_validation():
    """The read-rate probe: size a multiple of 16 below 2^40, 1..65536 workgroups,
    aligned and disjoint buffers; checked before any launch."""
    f = nv.lib().nvfp4_read_probe
    assert f(A, -16, 256, A + (2 << 20), None) == 1
    assert f(A, 1 << 20, 0, A + (2 << 20), None) == 1
    assert f(A, 1 << 20, 65537, A + (2 << 20), None) == 1
    assert f(A, (1 << 20) + 8, 256, A + (2 << 20), None) == 2
    assert f(A, 1 << 40, 256, A + (2 << 20), None) == 2
    assert f(None, 1 << 20, 256, A + (2 << 20), None) == 1
    assert f(A, 1 << 20, 256, None, None) == 1
    assert f(A + 4, 1 << 20, 256, A + (2 << 20), None) == 3
    assert f(A, 1 << 20, 256, A + (2 << 20) + 4, None) == 3
    assert f(A, 1 << 20, 256, A + 64, None) == 1                   # sink inside the buffer
