"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path through
the binding, download results.  Expected values always come from oracle/."""
import sys

import numpy as np
import torch

import nvfp4_w4a4_block_act_amd as nv
from oracle import gemm as G
from oracle import nvfp4 as Q
from workloads import bf16_to_f32

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def to_dev_f32(w):
    return torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(DEV)


def gpu_quantize(bits, amax=None):
    x = to_dev_bf16(bits)
    am = None if amax is None else torch.tensor([amax], dtype=torch.float32, device=DEV)
    c, s, g = nv.quantize_act(x, am)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy(), np.float32(g.cpu().numpy()[0])


def gpu_pack(w, segments):
    pw = nv.pack_weight(to_dev_f32(w), segments)
    torch.cuda.synchronize()
    return pw


def oracle_linear_rows(x_bits, w, segments, rows=None, cols=None, amax=None):
    """Oracle output (fp64) and error bound for output rows x cols of the linear layer.

    The activation scale uses the whole tensor's maximum (or the calibrated
    `amax` when given); each weight row is encoded with its segment's maximum
    over the whole segment."""
    x32 = bf16_to_f32(x_bits)
    if amax is None:
        amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    rows = np.arange(x32.shape[0]) if rows is None else np.asarray(rows)
    cols = np.arange(w.shape[0]) if cols is None else np.asarray(cols)
    ac, as_, ag, _ = Q.quantize(x32[rows], amax)
    a_hat = Q.dequantize(ac, as_, ag)
    w_hat = np.empty((len(cols), w.shape[1]), np.float64)
    for i, (b, e) in enumerate(segments):
        sel = np.nonzero((cols >= b) & (cols < e))[0]
        if len(sel) == 0:
            continue
        seg_amax = np.float32(np.max(np.abs(w[b:e])))
        wc, ws, wg, _ = Q.quantize(w[cols[sel]], seg_amax)
        w_hat[sel] = Q.dequantize(wc, ws, wg)
    return G.gemm_f64(a_hat, w_hat), G.gemm_bound(a_hat, w_hat)


def assert_within_tol(y, ref, bnd, what=""):
    ok = G.within_tol(y, ref, bnd)
    if not np.all(ok):
        idx = np.argwhere(~ok)[:5]
        err = np.abs(y - ref)
        msg = [f"{what}: {np.sum(~ok)} of {ok.size} outside |d| <= 1e-5*bound + 1e-6"]
        for i in idx:
            t = tuple(i)
            msg.append(f"  at {t}: gpu {y[t]!r} oracle {ref[t]!r} |d| {err[t]:.3e} bound {bnd[t]:.3e}")
        raise AssertionError("\n".join(msg))
