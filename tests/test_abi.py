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
    assert nv.nvfp4_abi_version() == 1
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
    (dict(M=4096, K=4096, ldx=4096, codes=A + (64 << 20), scales=A + (80 << 20), g=A + (96 << 20)), 5),
])
def test_quantize_act_validation(kw, status):
    assert q(**kw) == status


def test_quantize_workspace_query():
    assert nv.nvfp4_quantize_act_workspace_bytes(16, 5120) == 0
    assert nv.nvfp4_quantize_act_workspace_bytes(8192, 5120) > 0


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
    (dict(w=A + 4), 3), (dict(workb=0), 5), (dict(work=None), 5), (dict(wc=A + 64), 1),
])
def test_pack_validation(kw, status):
    assert p(**kw) == status


def test_binding_has_no_cpu_fallback(monkeypatch):
    """With the library path pointing nowhere, the binding raises instead of computing."""
    monkeypatch.setattr(nv, "_LIB", None)
    monkeypatch.setattr(nv, "LIB_PATH", "/nonexistent/libnvfp4_w4a4.so")
    with pytest.raises(ImportError):
        nv.lib()
