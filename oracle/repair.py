"""Two readings of the fused-GEMM global-scale repair, measured (CPU oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring for who may use it.

The pages describe the mismatch -- modules calibrated one by one, each with its
own FP32 global scale, served by kernels that fuse several modules into one
GEMM with a single scale -- and say that correct handling in the fused kernel
repairs it, without fixing how (paper abstract; Glonce article, "Who it
affects" and "Risks and caveats"; aiany page, "Mechanistic notes").  Two plain
readings, both exact functions of the weights:

  per_segment  each module keeps its own codes and FP32 scale; the GEMM
               applies each module's scale to that module's output columns
               (the library's epilogue);
  shared       all fused modules are re-encoded with one FP32 scale, set from
               the largest module maximum, and the GEMM applies that one
               scale (a plain single-segment GEMM).

`mismatch` (each module's codes decoded with the first module's scale) is the
failure both repair.  This module measures, per module, how far each variant
lands from the unquantized product of the bf16 activations and the fp32
weights.
"""
import numpy as np

from . import nvfp4 as Q


def _rel_rms(y, ref):
    den = np.sqrt(np.mean(ref * ref))
    return float(np.sqrt(np.mean((y - ref) ** 2)) / den) if den > 0 else 0.0


def decoded_weights(w, segments, cols, variant):
    """Decoded weight rows `cols` [len(cols), K] (float64) under one variant."""
    w = np.asarray(w, np.float32)
    cols = np.asarray(cols)
    out = np.empty((len(cols), w.shape[1]), np.float64)
    g_first = None
    shared_amax = np.float32(np.max(np.abs(w)))
    for i, (b, e) in enumerate(segments):
        seg_amax = np.float32(np.max(np.abs(w[b:e])))
        g_seg = Q.quantize(np.zeros((1, w.shape[1]), np.float32), seg_amax)[2]
        if i == 0:
            g_first = g_seg
        sel = np.nonzero((cols >= b) & (cols < e))[0]
        if len(sel) == 0:
            continue
        amax = shared_amax if variant == "shared" else seg_amax
        c, s, g, _ = Q.quantize(w[cols[sel]], amax)
        out[sel] = Q.dequantize(c, s, g_first if variant == "mismatch" else g)
    return out


def weight_errors(w, segments, variant):
    """Per module: relative RMS error of the decoded weights under one variant."""
    w = np.asarray(w, np.float32)
    d = decoded_weights(w, segments, np.arange(w.shape[0]), variant)
    return [_rel_rms(d[b:e], w[b:e].astype(np.float64)) for (b, e) in segments]


def relative_errors(x32, w, segments, rows, cols):
    """Per module: relative RMS error of each variant's output against the
    unquantized float64 product, over output rows x cols of that module.

    x32 is the activation tensor (float32 holding bf16 values); its NVFP4
    encoding uses the whole tensor's maximum, as the library does."""
    x32 = np.asarray(x32, np.float32)
    rows, cols = np.asarray(rows), np.asarray(cols)
    amax = np.float32(np.max(np.abs(x32)))
    ac, as_, ag, _ = Q.quantize(x32[rows], amax)
    a_hat = Q.dequantize(ac, as_, ag)
    y_ref = x32[rows].astype(np.float64) @ np.asarray(w, np.float64)[cols].T
    ys = {v: a_hat @ decoded_weights(w, segments, cols, v).T for v in ("per_segment", "shared", "mismatch")}
    res = []
    for (b, e) in segments:
        sel = (cols >= b) & (cols < e)
        res.append({v: _rel_rms(ys[v][:, sel], y_ref[:, sel]) for v in ys} if np.any(sel) else None)
    return res, ys, y_ref
