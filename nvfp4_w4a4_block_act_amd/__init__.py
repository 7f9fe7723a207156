"""Python binding of the gfx950 NVFP4 W4A4 linear-layer library.

Thin ctypes wrappers over the C ABI declared in include/nvfp4.h: the functions
named ``nvfp4_*`` take torch tensors, check nothing the library does not check
itself, pass ``data_ptr()`` values and torch's current HIP stream, and raise
``NVFP4Error`` on a non-OK status.  Every step of the computation runs in the
library's HIP kernels; torch only supplies device memory and the stream.
There is no fallback: if the library is not built, the first call into it
raises ImportError.

Convenience layer (allocation only): ``quantize_act``, ``pack_weight``,
``gemm`` and ``PackedWeight`` allocate outputs with torch and call the C ABI.
Their ``stream`` is a keyword-only ``torch.cuda.Stream`` (default: torch's
current stream); the ``nvfp4_*`` wrappers take a raw hipStream_t handle.
"""
import ctypes
import functools
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4_w4a4.so")

NVFP4_MAX_SEGMENTS = 16
STATUS = {0: "NVFP4_OK", 1: "NVFP4_EINVAL", 2: "NVFP4_ESHAPE", 3: "NVFP4_EALIGN",
          4: "NVFP4_ESEGMENTS", 5: "NVFP4_EWORKSPACE", 6: "NVFP4_EHIP"}


class NVFP4Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib().nvfp4_status_str(status).decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({msg})")


class Segment(ctypes.Structure):
    _fields_ = [("n_begin", ctypes.c_int32), ("n_end", ctypes.c_int32)]


_LIB = None
_i64, _vp, _sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python -m nvfp4_w4a4_block_act_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        lib.nvfp4_abi_version.restype = ctypes.c_int
        lib.nvfp4_status_str.restype = ctypes.c_char_p
        lib.nvfp4_status_str.argtypes = [ctypes.c_int]
        lib.nvfp4_quantize_act_workspace_bytes.restype = _sz
        lib.nvfp4_quantize_act_workspace_bytes.argtypes = [_i64, _i64]
        lib.nvfp4_quantize_act.restype = ctypes.c_int
        lib.nvfp4_quantize_act.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
        lib.nvfp4_packed_weight_bytes.restype = ctypes.c_int
        lib.nvfp4_packed_weight_bytes.argtypes = [_i64, _i64, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]
        lib.nvfp4_pack_weight_workspace_bytes.restype = _sz
        lib.nvfp4_pack_weight_workspace_bytes.argtypes = [_i64, _i64, ctypes.c_int32]
        lib.nvfp4_pack_weight.restype = ctypes.c_int
        lib.nvfp4_pack_weight.argtypes = [_vp, _i64, _i64, _i64, ctypes.POINTER(Segment), ctypes.c_int32,
                                          _vp, _vp, _vp, _vp, _sz, _vp]
        lib.nvfp4_weight_to_canonical.restype = ctypes.c_int
        lib.nvfp4_weight_to_canonical.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp, _vp]
        lib.nvfp4_gemm.restype = ctypes.c_int
        lib.nvfp4_gemm.argtypes = [_vp, _vp, _vp, _i64, _i64, _vp, _vp, _i64, ctypes.POINTER(Segment), _vp,
                                   ctypes.c_int32, _vp, _i64, _vp]
        lib.nvfp4_gemm_form.restype = ctypes.c_int
        lib.nvfp4_gemm_form.argtypes = [_i64, _i64, _i64]
        lib.nvfp4_linear_workspace_bytes.restype = _sz
        lib.nvfp4_linear_workspace_bytes.argtypes = [_i64, _i64]
        lib.nvfp4_linear.restype = ctypes.c_int
        lib.nvfp4_linear.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i64,
                                     ctypes.POINTER(Segment), _vp, ctypes.c_int32, _vp, _i64, _vp, _sz, _vp]
        lib.nvfp4_linear_noalloc.restype = ctypes.c_int
        lib.nvfp4_linear_noalloc.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i64,
                                             ctypes.POINTER(Segment), _vp, ctypes.c_int32, _vp, _i64, _vp]
        lib.nvfp4_pack_weight_gate_up.restype = ctypes.c_int
        lib.nvfp4_pack_weight_gate_up.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp]
        lib.nvfp4_gemm_swiglu_quantize.restype = ctypes.c_int
        lib.nvfp4_gemm_swiglu_quantize.argtypes = [_vp, _vp, _vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _vp,
                                                   _vp, _vp]
        lib.nvfp4_amax_observe_workspace_bytes.restype = _sz
        lib.nvfp4_amax_observe_workspace_bytes.argtypes = [_i64, _i64]
        lib.nvfp4_amax_observe.restype = ctypes.c_int
        lib.nvfp4_amax_observe.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _sz, _vp]
        lib.nvfp4_quantize_stats.restype = ctypes.c_int
        lib.nvfp4_quantize_stats.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp]
        lib.nvfp4_kv_fp8_encode.restype = ctypes.c_int
        lib.nvfp4_kv_fp8_encode.argtypes = [_vp, _i64, _vp, _vp, _vp]
        lib.nvfp4_kv_fp8_decode.restype = ctypes.c_int
        lib.nvfp4_kv_fp8_decode.argtypes = [_vp, _i64, _vp, _vp, _vp]
        lib.nvfp4_swiglu.restype = ctypes.c_int
        lib.nvfp4_swiglu.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp]
        lib.nvfp4_convert_sweep.restype = ctypes.c_int
        lib.nvfp4_convert_sweep.argtypes = [ctypes.c_int32, ctypes.c_uint32, _i64, _vp, _vp]
        lib.nvfp4_read_probe.restype = ctypes.c_int
        lib.nvfp4_read_probe.argtypes = [_vp, _i64, ctypes.c_int32, _vp, _vp]
        _LIB = lib
    return _LIB


def lib():
    """The loaded ctypes library (loads it on first use)."""
    return _lib()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    return torch.cuda.current_stream().cuda_stream


def _check(status, where):
    if status != 0:
        raise NVFP4Error(status, where)


def _segs(segments):
    arr = (Segment * max(1, len(segments)))()
    for i, (b, e) in enumerate(segments):
        arr[i].n_begin, arr[i].n_end = int(b), int(e)
    return arr, len(segments)


# ---- the C ABI, one wrapper per entry point ---------------------------------------
def nvfp4_abi_version():
    return _lib().nvfp4_abi_version()


def nvfp4_status_str(status):
    return _lib().nvfp4_status_str(int(status)).decode()


def nvfp4_quantize_act_workspace_bytes(M, K):
    return _lib().nvfp4_quantize_act_workspace_bytes(int(M), int(K))


def nvfp4_quantize_act(x, M, K, ldx, amax_in, codes, scales, g_dec_out, workspace, workspace_bytes, stream=None):
    _check(_lib().nvfp4_quantize_act(_ptr(x), M, K, ldx, _ptr(amax_in), _ptr(codes), _ptr(scales),
                                     _ptr(g_dec_out), _ptr(workspace), workspace_bytes, _stream(stream)),
           "nvfp4_quantize_act")


def nvfp4_packed_weight_bytes(N, K):
    cb, sb = _sz(0), _sz(0)
    _check(_lib().nvfp4_packed_weight_bytes(int(N), int(K), ctypes.byref(cb), ctypes.byref(sb)),
           "nvfp4_packed_weight_bytes")
    return cb.value, sb.value


def nvfp4_pack_weight_workspace_bytes(N, K, nseg):
    return _lib().nvfp4_pack_weight_workspace_bytes(int(N), int(K), int(nseg))


def nvfp4_pack_weight(w, N, K, ldw, segments, w_codes, w_scales, w_g_dec, workspace, workspace_bytes,
                      stream=None):
    arr, n = _segs(segments)
    _check(_lib().nvfp4_pack_weight(_ptr(w), N, K, ldw, arr, n, _ptr(w_codes), _ptr(w_scales), _ptr(w_g_dec),
                                    _ptr(workspace), workspace_bytes, _stream(stream)), "nvfp4_pack_weight")


def nvfp4_weight_to_canonical(w_codes, w_scales, N, K, codes, scales, stream=None):
    _check(_lib().nvfp4_weight_to_canonical(_ptr(w_codes), _ptr(w_scales), N, K, _ptr(codes), _ptr(scales),
                                            _stream(stream)), "nvfp4_weight_to_canonical")


def nvfp4_gemm(a_codes, a_scales, a_g_dec, M, K, w_codes, w_scales, N, segments, w_g_dec, out, ldo,
               stream=None):
    arr, n = _segs(segments)
    _check(_lib().nvfp4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(a_g_dec), M, K, _ptr(w_codes), _ptr(w_scales),
                             N, arr, _ptr(w_g_dec), n, _ptr(out), ldo, _stream(stream)), "nvfp4_gemm")


def nvfp4_gemm_form(M, K, N):
    return _lib().nvfp4_gemm_form(int(M), int(K), int(N))


def nvfp4_linear_workspace_bytes(M, K):
    return _lib().nvfp4_linear_workspace_bytes(int(M), int(K))


def nvfp4_linear(x, M, K, ldx, amax_in, a_codes, a_scales, a_g_dec, w_codes, w_scales, N, segments, w_g_dec,
                 out, ldo, workspace, workspace_bytes, stream=None):
    arr, n = _segs(segments)
    _check(_lib().nvfp4_linear(_ptr(x), M, K, ldx, _ptr(amax_in), _ptr(a_codes), _ptr(a_scales), _ptr(a_g_dec),
                               _ptr(w_codes), _ptr(w_scales), N, arr, _ptr(w_g_dec), n, _ptr(out), ldo,
                               _ptr(workspace), workspace_bytes, _stream(stream)), "nvfp4_linear")


def nvfp4_linear_noalloc(x, M, K, ldx, amax_in, a_codes, a_scales, a_g_dec, w_codes, w_scales, N, segments,
                         w_g_dec, out, ldo, stream=None):
    arr, n = _segs(segments)
    _check(_lib().nvfp4_linear_noalloc(_ptr(x), M, K, ldx, _ptr(amax_in), _ptr(a_codes), _ptr(a_scales),
                                       _ptr(a_g_dec), _ptr(w_codes), _ptr(w_scales), N, arr, _ptr(w_g_dec), n,
                                       _ptr(out), ldo, _stream(stream)), "nvfp4_linear_noalloc")


def nvfp4_pack_weight_gate_up(w, I, K, ldw, w_codes, w_scales, w_g_dec, workspace, workspace_bytes, stream=None):
    _check(_lib().nvfp4_pack_weight_gate_up(_ptr(w), I, K, ldw, _ptr(w_codes), _ptr(w_scales), _ptr(w_g_dec),
                                            _ptr(workspace), workspace_bytes, _stream(stream)),
           "nvfp4_pack_weight_gate_up")


def nvfp4_gemm_swiglu_quantize(a_codes, a_scales, a_g_dec, M, K, w_codes, w_scales, I, w_g_dec, amax_h,
                               h_codes, h_scales, h_g_dec, stream=None):
    _check(_lib().nvfp4_gemm_swiglu_quantize(_ptr(a_codes), _ptr(a_scales), _ptr(a_g_dec), M, K, _ptr(w_codes),
                                             _ptr(w_scales), I, _ptr(w_g_dec), _ptr(amax_h), _ptr(h_codes),
                                             _ptr(h_scales), _ptr(h_g_dec), _stream(stream)),
           "nvfp4_gemm_swiglu_quantize")


def nvfp4_amax_observe_workspace_bytes(M, K):
    return _lib().nvfp4_amax_observe_workspace_bytes(int(M), int(K))


def nvfp4_amax_observe(x, M, K, ldx, running_amax, workspace, workspace_bytes, stream=None):
    _check(_lib().nvfp4_amax_observe(_ptr(x), M, K, ldx, _ptr(running_amax), _ptr(workspace), workspace_bytes,
                                     _stream(stream)), "nvfp4_amax_observe")


def nvfp4_quantize_stats(x, M, K, ldx, amax_in, counts, stream=None):
    _check(_lib().nvfp4_quantize_stats(_ptr(x), M, K, ldx, _ptr(amax_in), _ptr(counts), _stream(stream)),
           "nvfp4_quantize_stats")


def nvfp4_kv_fp8_encode(x, n, amax, codes, stream=None):
    _check(_lib().nvfp4_kv_fp8_encode(_ptr(x), n, _ptr(amax), _ptr(codes), _stream(stream)), "nvfp4_kv_fp8_encode")


def nvfp4_kv_fp8_decode(codes, n, amax, out, stream=None):
    _check(_lib().nvfp4_kv_fp8_decode(_ptr(codes), n, _ptr(amax), _ptr(out), _stream(stream)), "nvfp4_kv_fp8_decode")


def nvfp4_swiglu(gu, M, I, ldgu, h, ldh, stream=None):
    _check(_lib().nvfp4_swiglu(_ptr(gu), M, I, ldgu, _ptr(h), ldh, _stream(stream)), "nvfp4_swiglu")


def nvfp4_convert_sweep(op, first_bits, n, out, stream=None):
    _check(_lib().nvfp4_convert_sweep(int(op), int(first_bits), int(n), _ptr(out), _stream(stream)),
           "nvfp4_convert_sweep")


def nvfp4_read_probe(buf, nbytes, workgroups, sink, stream=None):
    _check(_lib().nvfp4_read_probe(_ptr(buf), int(nbytes), int(workgroups), _ptr(sink), _stream(stream)),
           "nvfp4_read_probe")


# ---- convenience layer: allocate with torch, call the C ABI --------------------------
def _on_stream(fn):
    """Runs a convenience function on ``stream`` (a torch.cuda.Stream, keyword-only):
    its tensors -- outputs and temporary scratch -- are allocated while that stream
    is current, so torch's caching allocator hands their memory to no other stream
    while the enqueued kernels may still use it; the C ABI gets the raw handle."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, stream=None, **kw)
        if not isinstance(stream, torch.cuda.Stream):
            raise TypeError(f"{fn.__name__}: stream must be a torch.cuda.Stream "
                            "(the nvfp4_* wrappers take raw handles)")
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream.cuda_stream, **kw)
    return wrapper


def _empty(n, dtype, device):
    return torch.empty(max(int(n), 1), dtype=dtype, device=device)


class Workspace:
    """A growable device scratch buffer owned by the caller.

    The kernels write into it, so calls that share one Workspace must be ordered
    (issued on one stream, or synchronized between streams).  Growing it frees the
    old buffer through torch's stream-ordered allocator."""

    def __init__(self, device):
        self.device = device
        self.buf = None

    def get(self, nbytes):
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf, self.buf.numel()


@_on_stream
def quantize_act(x, amax=None, workspace=None, out=None, *, stream=None):
    """bf16 [M, K] cuda tensor -> (codes uint8 [M, K/2], scales uint8 [M, K/16], g_dec float32 [1])."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and (x.stride(1) == 1 or x.shape[1] <= 1)
    M, K = x.shape
    dev = x.device
    if out is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
        g = torch.empty(1, dtype=torch.float32, device=dev)
    else:
        codes, scales, g = out
    need = nvfp4_quantize_act_workspace_bytes(M, K)
    ws = workspace if workspace is not None else Workspace(dev)
    buf, nbytes = ws.get(need)
    nvfp4_quantize_act(x, M, K, max(x.stride(0), K), amax, codes, scales, g, buf, nbytes, stream)
    return codes, scales, g


@dataclass
class PackedWeight:
    codes: torch.Tensor      # uint8, tiled layout
    scales: torch.Tensor     # uint8, tiled layout
    g_dec: torch.Tensor      # float32 [nseg]
    N: int
    K: int
    segments: list

    def nbytes(self):
        return self.codes.numel() + self.scales.numel()


@_on_stream
def pack_weight(w, segments=None, *, stream=None):
    """fp32 [N, K] cuda tensor + [(n_begin, n_end), ...] -> PackedWeight."""
    assert w.dtype == torch.float32 and w.dim() == 2 and (w.stride(1) == 1 or w.shape[1] <= 1)
    N, K = w.shape
    segments = [(0, N)] if segments is None else [tuple(s) for s in segments]
    cb, sb = nvfp4_packed_weight_bytes(N, K)
    codes = _empty(cb, torch.uint8, w.device)
    scales = _empty(sb, torch.uint8, w.device)
    g = torch.empty(len(segments), dtype=torch.float32, device=w.device)
    need = nvfp4_pack_weight_workspace_bytes(N, K, len(segments))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=w.device)
    nvfp4_pack_weight(w, N, K, max(w.stride(0), K), segments, codes, scales, g, ws, need, stream)
    return PackedWeight(codes, scales, g, N, K, segments)


@_on_stream
def weight_to_canonical(pw, *, stream=None):
    codes = torch.empty((pw.N, pw.K // 2), dtype=torch.uint8, device=pw.codes.device)
    scales = torch.empty((pw.N, pw.K // 16), dtype=torch.uint8, device=pw.codes.device)
    nvfp4_weight_to_canonical(pw.codes, pw.scales, pw.N, pw.K, codes, scales, stream)
    return codes, scales


@_on_stream
def gemm(a_codes, a_scales, a_g_dec, pw, out=None, g_dec=None, *, stream=None):
    """NVFP4 activations x packed weight -> fp32 [M, N] (per-segment epilogue).

    ``g_dec`` overrides the weight's per-segment scales (same length)."""
    M = a_codes.shape[0]
    K = pw.K
    assert a_codes.shape[1] * 2 == K
    if out is None:
        out = torch.empty((M, pw.N), dtype=torch.float32, device=a_codes.device)
    wg = pw.g_dec if g_dec is None else g_dec
    nvfp4_gemm(a_codes, a_scales, a_g_dec, M, K, pw.codes, pw.scales, pw.N, pw.segments, wg, out,
               out.stride(0), stream)
    return out


@_on_stream
def linear(x, pw, amax=None, workspace=None, out=None, act_out=None, *, stream=None):
    """The whole W4A4 linear layer via nvfp4_linear: bf16 x [M, K] -> fp32 [M, N].

    Also returns the activation codes, scales and g_dec it produced."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and (x.stride(1) == 1 or x.shape[1] <= 1)
    M, K = x.shape
    assert K == pw.K
    dev = x.device
    if act_out is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
        g = torch.empty(1, dtype=torch.float32, device=dev)
    else:
        codes, scales, g = act_out
    if out is None:
        out = torch.empty((M, pw.N), dtype=torch.float32, device=dev)
    ws = workspace if workspace is not None else Workspace(dev)
    buf, nbytes = ws.get(nvfp4_linear_workspace_bytes(M, K))
    nvfp4_linear(x, M, K, max(x.stride(0), K), amax, codes, scales, g, pw.codes, pw.scales, pw.N, pw.segments,
                 pw.g_dec, out, out.stride(0), buf, nbytes, stream)
    return out, (codes, scales, g)


@_on_stream
def pack_weight_gate_up(w, *, stream=None):
    """fp32 [2I, K] (gate rows, then up rows) -> PackedWeight in the interleaved
    gate/up layout, with the two modules' own scales (segments (0, I), (I, 2I))."""
    assert w.dtype == torch.float32 and w.dim() == 2 and w.is_cuda and w.stride(1) == 1
    N2, K = w.shape
    I = N2 // 2
    cb, sb = nvfp4_packed_weight_bytes(N2, K)
    codes = _empty(cb, torch.uint8, w.device)
    scales = _empty(sb, torch.uint8, w.device)
    g = torch.empty(2, dtype=torch.float32, device=w.device)
    need = nvfp4_pack_weight_workspace_bytes(N2, K, 2)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=w.device)
    nvfp4_pack_weight_gate_up(w, I, K, w.stride(0), codes, scales, g, ws, ws.numel(), stream)
    return PackedWeight(codes, scales, g, N2, K, [(0, I), (I, N2)])


@_on_stream
def gemm_swiglu_quantize(a_codes, a_scales, a_g_dec, pw, amax_h, out=None, *, stream=None):
    """NVFP4 activations x interleaved gate/up weight -> NVFP4 of bf16(silu(g) * u):
    (codes uint8 [M, I/2], scales uint8 [M, I/16], g_dec float32 [1])."""
    M = a_codes.shape[0]
    I = pw.N // 2
    dev = a_codes.device
    if out is None:
        out = (torch.empty((M, I // 2), dtype=torch.uint8, device=dev),
               torch.empty((M, I // 16), dtype=torch.uint8, device=dev),
               torch.empty(1, dtype=torch.float32, device=dev))
    c, s, g = out
    nvfp4_gemm_swiglu_quantize(a_codes, a_scales, a_g_dec, M, pw.K, pw.codes, pw.scales, I, pw.g_dec, amax_h,
                               c, s, g, stream)
    return out


@_on_stream
def swiglu(gu, *, stream=None):
    """fp32 [M, 2I] gate+up output -> bf16 [M, I] = bf16(silu(g) * u)."""
    assert gu.dtype == torch.float32 and gu.dim() == 2 and gu.stride(1) == 1
    M, N2 = gu.shape
    h = torch.empty((M, N2 // 2), dtype=torch.bfloat16, device=gu.device)
    nvfp4_swiglu(gu, M, N2 // 2, gu.stride(0), h, h.stride(0), stream)
    return h


@_on_stream
def kv_fp8_encode(x, amax, out=None, *, stream=None):
    """Contiguous bf16 cuda tensor + device amax [1] -> uint8 E4M3FN codes of the same shape."""
    assert x.dtype == torch.bfloat16 and x.is_contiguous()
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if out is None else out
    nvfp4_kv_fp8_encode(x, x.numel(), amax, codes, stream)
    return codes


@_on_stream
def kv_fp8_decode(codes, amax, out=None, *, stream=None):
    """uint8 E4M3FN codes + device amax [1] -> bf16 tensor of the same shape."""
    assert codes.dtype == torch.uint8 and codes.is_contiguous()
    y = torch.empty(codes.shape, dtype=torch.bfloat16, device=codes.device) if out is None else out
    nvfp4_kv_fp8_decode(codes, codes.numel(), amax, y, stream)
    return y


class AmaxObserver:
    """Running maximum of |x| over calibration batches, kept on the device."""

    def __init__(self, device):
        self.amax = torch.zeros(1, dtype=torch.float32, device=device)
        self.ws = torch.empty(max(nvfp4_amax_observe_workspace_bytes(0, 0), 16), dtype=torch.uint8, device=device)

    @_on_stream
    def observe(self, x, *, stream=None):
        assert x.dtype == torch.bfloat16 and x.dim() == 2 and (x.stride(1) == 1 or x.shape[1] <= 1)
        M, K = x.shape
        nvfp4_amax_observe(x, M, K, max(x.stride(0), K), self.amax, self.ws, self.ws.numel(), stream)
        return self.amax


@_on_stream
def quantize_stats(x, amax, *, stream=None):
    """(saturated-scale blocks, clipped elements) of bf16 x under the static maximum amax [1]."""
    M, K = x.shape
    counts = torch.empty(2, dtype=torch.int32, device=x.device)
    nvfp4_quantize_stats(x, M, K, max(x.stride(0), K), amax, counts, stream)
    return counts
