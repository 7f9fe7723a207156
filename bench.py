#!/usr/bin/env python3
"""Benchmark of the NVFP4 W4A4 linear layer on one MI355X.

Default workload: the decode skinny GEMM -- M in {1, 4, 16} tokens, K = 5120,
N = 12288, weights N(0, 0.02) pre-packed, bf16 Student-t(3) activations with
0.1% of channels x100 quantized on the fly.  One step = the whole hot path for
the three token counts: activation quantization (dynamic per-tensor scale) +
W4A4 GEMM + per-segment epilogue, three times, each one nvfp4_linear call
(a single fused launch at these sizes).  The packed weight is kept in
16 device copies (566 MB, more than the 256 MB MALL) and each step uses the
next copy, so every call streams its weights from HBM.  The 16 steps that use
the 16 copies in turn are captured in one HIP graph, replayed once per 16
timed steps (remainders replay single-step graphs); inputs are resident in HBM
before the timed region starts.

The same run then measures the prefill half of the metric (``config.prefill``):
the gate+up (8192 x 5120 x 2 x 17408), GDN in-projection (4096 x 5120 x 12352)
and down-projection (32768 x 17408 x 5120) GEMMs -- quantize + GEMM + epilogue
per step, the GEMM kernel alone timed with event pairs, each with its roofline
against the fp16 matrix-core peak and an oracle baseline -- and the standalone
activation quantizer over the down projection's input (GB/s against HBM).

Prints one JSON line (see the keys below).  ``--config`` selects another
workload on its own (decode_down_proj, prefill_gate_up, gdn_in_proj,
down_proj, down_proj_quantize, tiny, ...); ``--no-prefill`` skips the prefill
legs.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X published HBM3E bandwidth
F16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X published dense fp16/bf16 matrix peak


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=480)
    ap.add_argument("--warmup", type=int, default=48)
    ap.add_argument("--config", default="decode",
                    choices=["decode", "decode_down_proj", "prefill_gate_up", "gdn_in_proj", "down_proj",
                             "down_proj_quantize", "tiny",
                             "copy_calibration", "gdn_repair_compare", "gate_up_swiglu", "kv_fp8", "static_calibration",
                             "read_probe"])
    ap.add_argument("--copies", type=int, default=16, help="device copies of the packed weight (decode)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-prefill", action="store_true", help="decode only (no prefill legs in the default run)")
    ap.add_argument("--no-gpu-state", action="store_true",
                    help="skip the amd-smi / rocm-smi power and clock snapshot (e.g. under a profiler)")
    ap.add_argument("--prefill-steps", type=int, default=20, help="timed steps of each prefill leg")
    ap.add_argument("--prefill-cpu-seconds", type=float, default=5.0,
                    help="target CPU time of each prefill leg's oracle sample")
    return ap.parse_args()


def main():
    args = parse()
    global GPU_STATE
    GPU_STATE = not args.no_gpu_state
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(how the layer would shard is a design, not code); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("bench.py needs --steps >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    import torch
    import nvfp4_w4a4_block_act_amd as nv
    import workloads as W
    torch.cuda.init()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    if args.config == "decode":
        res = bench_decode(args, torch, nv, W, dev)
    elif args.config == "decode_down_proj":
        res = bench_decode(args, torch, nv, W, dev, W.decode_down_proj(M=16))
    elif args.config == "copy_calibration":
        res = bench_copy(args, torch, dev)
    elif args.config == "read_probe":
        res = bench_read_probe(args, torch, nv, dev)
    elif args.config == "gdn_repair_compare":
        res = bench_repair(args, torch, nv, W, dev)
    elif args.config == "gate_up_swiglu":
        res = bench_swiglu(args, torch, nv, W, dev)
    elif args.config == "kv_fp8":
        res = bench_kv_fp8(args, torch, nv, W, dev)
    elif args.config == "static_calibration":
        res = bench_calibration(args, torch, nv, W, dev)
    elif args.config == "down_proj_quantize":
        res = bench_quantize(args, torch, nv, W, dev)
    else:
        res = bench_gemm(args, torch, nv, W, dev)
    print(json.dumps(res), flush=True)


# ---------------------------------------------------------------------------------------
PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
PKG_CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "nvfp4_w4a4_block_act_amd", "csrc")


def source_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(PKG_CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(summary, files):
    """HBM bytes per launch recorded by the rocprofv3 counter runs in profiles/<summary>
    (FETCH_SIZE + WRITE_SIZE, each scaled by the copy-kernel calibration), or None when
    the summary is missing or was taken on kernel sources other than the current ones."""
    path = os.path.join(PROFILES, summary)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_sha256") != source_digest(files):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def bench_copy(args, torch, dev):
    """A plain device-to-device copy of known size: the calibration run for the
    FETCH_SIZE / WRITE_SIZE counters (one read and one write of 512 MiB per launch)."""
    n = 512 << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    sec, wall = time_region(torch, lambda i: dst.copy_(src), args.steps, args.warmup)
    return {"metric": "device copy GB/s (counter calibration)", "value": round(2 * n * args.steps / sec / 1e9, 1),
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(sec / args.steps * 1e3, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "u8", "data": "synthetic",
            "config": {"workload": "copy_512MiB", "bytes_read_per_launch": n, "bytes_written_per_launch": n}}


def bench_read_probe(args, torch, nv, dev):
    """The read rate of a bare stream (nvfp4_read_probe: non-temporal 16-byte loads,
    one contiguous share per workgroup) for the sizes the HBM-bound kernels stream:
    the decode GEMMs' packed weights (K = 5120, N = 12288 and K = 17408, N = 5120;
    16 rotating copies, so no launch finds its bytes in the 256 MB last-level cache)
    and the bf16 input of the 32768 x 17408 activation quantizer (larger than that
    cache, one buffer), each over 256 / 512 / 1024 workgroups.  Per-launch time from
    HIP event pairs around graphs of back-to-back launches on the launch stream."""
    sizes = [("decode_weight_k5120_n12288", 12288 * 5120 * 9 // 16, 16),
             ("decode_weight_k17408_n5120", 5120 * 17408 * 9 // 16, 16),
             ("activation_bf16_m32768_k17408", 32768 * 17408 * 2, 1)]
    grids = (256, 512, 1024)
    sink = torch.zeros(max(grids), dtype=torch.int32, device=dev)
    rows = []
    for name, nbytes, copies in sizes:
        bufs = [torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device=dev)
                for _ in range(copies)]
        per_graph = 16
        for wg in grids:
            g = torch.cuda.CUDAGraph()
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                for r in range(per_graph):
                    nv.nvfp4_read_probe(bufs[r % copies], nbytes, wg, sink)
            mean, med, p10, p90 = kernel_time_pairs(torch, lambda i: g.replay(), max(8, args.steps // per_graph))
            mean, med = mean / per_graph, med / per_graph
            rows.append({"stream": name, "bytes": nbytes, "workgroups": wg, "mean_us": round(mean * 1e6, 3),
                         "median_us": round(med * 1e6, 3), "GBps": round(nbytes / mean / 1e9, 1),
                         "frac_of_hbm_peak": round(nbytes / mean / 1e9 / HBM_PEAK_GBS, 4)})
            del g
        del bufs
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    head = rows[0]
    return {"metric": "HBM read rate of a bare stream (read-rate probe), GB/s", "value": head["GBps"], "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": 0, "ms_per_step": round(head["mean_us"] / 1e3, 6),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
            "config": {"workload": "read_probe_decode_weight_k5120_n12288_256wg", "probes": rows}}


def bench_repair(args, torch, nv, W, dev):
    """The two readings of the mismatch repair on the GDN in-projection (six modules,
    amax ratio ~20): the per-segment epilogue (six FP32 scales, the library's default)
    against re-encoding all modules with one shared scale (a single-segment GEMM).
    Times both GEMMs and reports, per module, the relative RMS error of each output
    against the unquantized float64 product over a sample of rows and columns."""
    d = W.gdn_in_proj()
    M, K, N = d.M, d.K, d.N
    x = to_dev_bf16(torch, d.x_bits, dev)
    c, s, g = nv.quantize_act(x)
    w = torch.from_numpy(d.w).to(dev)
    variants = {"per_segment": nv.pack_weight(w, d.segments), "shared": nv.pack_weight(w, [(0, N)])}
    del w
    out = torch.empty((M, N), dtype=torch.float32, device=dev)
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(M, 64, replace=False))
    cols = np.concatenate([np.sort(rng.choice(np.arange(b, e), min(e - b, 128), replace=False))
                           for b, e in d.segments])
    x32 = (d.x_bits.astype(np.uint32) << 16).view(np.float32)[rows].astype(np.float64)
    y_ref = x32 @ d.w[cols].astype(np.float64).T
    steps = max(1, args.steps)
    res = {"metric": "NVFP4 W4A4 fused-GEMM repair comparison: per-segment epilogue vs shared-scale re-encode",
           "value": None, "unit": "ms", "n_gpus": 1, "steps": steps, "warmup": min(args.warmup, 5),
           "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
           "config": {"workload": d.name, "M": M, "K": K, "N": N,
                      "segments": [[int(b), int(e)] for b, e in d.segments]}}
    for name, pw in variants.items():
        sec, _ = time_region(torch, lambda i, pw=pw: nv.gemm(c, s, g, pw, out=out), steps, min(args.warmup, 5))
        y = out.cpu().numpy().astype(np.float64)[rows][:, cols]
        errs = []
        for b, e in d.segments:
            sel = (cols >= b) & (cols < e)
            ref = y_ref[:, sel]
            errs.append(round(float(np.sqrt(np.mean((y[:, sel] - ref) ** 2)) / np.sqrt(np.mean(ref ** 2))), 6))
        res["config"][name] = {"gemm_ms": round(sec / steps * 1e3, 4), "rel_rms_error_per_module": errs}
    res["value"] = res["config"]["per_segment"]["gemm_ms"]
    res["ms_per_step"] = res["value"]
    return res


def bench_swiglu(args, torch, nv, W, dev):
    """Gate+up projection of the prefill MLP (M = 8192, K = 5120, I = 17408) up to the
    down projection's NVFP4 input, two ways: unfused (GEMM to fp32, SwiGLU to bf16,
    activation quantizer with a calibrated maximum) and fused (the GEMM's epilogue emits
    the NVFP4 codes directly).  The calibrated maximum is that of this batch's h, taken
    from one unfused run before timing.  TFLOP/s counts the GEMM's 2 M N K."""
    d = W.prefill_gate_up()
    M, K, N = d.M, d.K, d.N
    I = N // 2
    x = to_dev_bf16(torch, d.x_bits, dev)
    c, s, g = nv.quantize_act(x)
    w = torch.from_numpy(d.w).to(dev)
    pw = nv.pack_weight(w, d.segments)
    pwi = nv.pack_weight_gate_up(w)
    del w
    gu = torch.empty((M, N), dtype=torch.float32, device=dev)
    h = torch.empty((M, I), dtype=torch.bfloat16, device=dev)
    hq = (torch.empty((M, I // 2), dtype=torch.uint8, device=dev), torch.empty((M, I // 16), dtype=torch.uint8,
          device=dev), torch.empty(1, dtype=torch.float32, device=dev))
    fq = (torch.empty_like(hq[0]), torch.empty_like(hq[1]), torch.empty_like(hq[2]))
    nv.gemm(c, s, g, pw, out=gu)
    nv.nvfp4_swiglu(gu, M, I, gu.stride(0), h, h.stride(0))
    amax_h = h.float().abs().max().reshape(1).contiguous()
    ws = nv.Workspace(dev)

    def unfused(i):
        nv.gemm(c, s, g, pw, out=gu)
        nv.nvfp4_swiglu(gu, M, I, gu.stride(0), h, h.stride(0))
        nv.quantize_act(h, amax_h, ws, out=hq)

    def fused(i):
        nv.gemm_swiglu_quantize(c, s, g, pwi, amax_h, out=fq)

    steps = max(1, args.steps)
    t_un, _ = time_region(torch, unfused, steps, min(args.warmup, 5))
    t_fu, _ = time_region(torch, fused, steps, min(args.warmup, 5))
    same = bool(torch.equal(fq[0], hq[0]) and torch.equal(fq[1], hq[1]) and torch.equal(fq[2], hq[2]))
    flops = 2.0 * M * N * K
    value = flops * steps / t_fu / 1e12
    return {"metric": "NVFP4 W4A4 gate+up GEMM with fused SwiGLU -> NVFP4 epilogue TFLOP/s, % of MI355X fp16 MFMA roofline",
            "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": min(args.warmup, 5),
            "ms_per_step": round(t_fu / steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f16", "data": "synthetic",
            "config": {"workload": "gate_up_swiglu_m8192_k5120_i17408", "M": M, "K": K, "I": I,
                       "unfused_ms": round(t_un / steps * 1e3, 4), "fused_ms": round(t_fu / steps * 1e3, 4),
                       "fused_equals_unfused": same,
                       "hbm_bytes_avoided": M * N * 4 * 2 + M * I * 2 * 2},
            "roofline": {"bound": "mfma", "achieved": round(value, 2), "peak": F16_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(value / F16_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                         "kernel": "gemm_mfma_kernel (SwiGLU epilogue)"}}


def bench_kv_fp8(args, torch, nv, W, dev):
    """FP8 KV-cache codec on one layer's keys and values for a 32768-token context with
    8 KV heads of 128 (2 x 32768 x 1024 bf16, 128 MB), N(0, 1) with 8 outlier channels
    x20; amax calibrated on a different draw of the same distribution.  One step =
    encode K and V, then decode both; GB/s counts bf16 read + fp8 written (encode) and
    fp8 read + bf16 written (decode)."""
    rng = np.random.default_rng(0)
    T, C = 32768, 1024
    outl = rng.choice(C, 8, replace=False)

    def draw():
        x = rng.standard_normal((T, C)).astype(np.float32)
        x[:, outl] *= 20.0
        return torch.from_numpy(x).to(dev).to(torch.bfloat16)

    kv = [draw(), draw()]
    cal = draw()
    amax = cal.float().abs().max().reshape(1).contiguous()
    del cal
    codes = [torch.empty((T, C), dtype=torch.uint8, device=dev) for _ in kv]
    outs = [torch.empty((T, C), dtype=torch.bfloat16, device=dev) for _ in kv]

    def step(i):
        for x, c in zip(kv, codes):
            nv.kv_fp8_encode(x, amax, out=c)
        for c, y in zip(codes, outs):
            nv.kv_fp8_decode(c, amax, out=y)

    steps = max(1, args.steps)
    sec, _ = time_region(torch, step, steps, min(args.warmup, 5))
    n = 2 * T * C
    step_bytes = 2 * (n * 3)
    enc_t = kernel_time_pairs(torch, lambda i: nv.kv_fp8_encode(kv[0], amax, out=codes[0]), 50)[0]
    dec_t = kernel_time_pairs(torch, lambda i: nv.kv_fp8_decode(codes[0], amax, out=outs[0]), 50)[0]
    per = T * C * 3
    sat = float((codes[0] & 0x7F).eq(0x7E).float().mean().item())
    value = step_bytes * steps / sec / 1e9
    achieved = per / ((enc_t + dec_t) / 2) / 1e9
    return {"metric": "FP8 KV-cache codec GB/s (encode + decode), % of MI355X HBM roofline", "value": round(value, 1),
            "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": min(args.warmup, 5),
            "ms_per_step": round(sec / steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "fp8", "data": "synthetic",
            "config": {"workload": "kv_fp8_t32768_c1024_k_and_v", "encode_us": round(enc_t * 1e6, 2),
                       "decode_us": round(dec_t * 1e6, 2), "saturated_fraction": sat},
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                         "kernel": "kv_fp8_encode_kernel / kv_fp8_decode_kernel"}}


def bench_calibration(args, torch, nv, W, dev):
    """Static activation scales as calibration-only PTQ ships them, on the decode
    linear layer (K = 5120, N = 12288): observe the running maximum over 16
    calibration batches of 16 tokens (Student-t(3) activations with outlier
    channels, the decode distribution), then on 16 held-out batches compare the
    static scale with the dynamic one: saturated block scales, clipped elements, and
    the layer output's relative RMS error against the unquantized float64 product
    (512 sampled output columns).  Times the observer and the static linear call."""
    d = W.decode(M=16)
    K, N = d.K, d.N
    w = torch.from_numpy(d.w).to(dev)
    pw = nv.pack_weight(w, d.segments)
    del w
    obs = nv.AmaxObserver(dev)
    cal = [to_dev_bf16(torch, W.random_act(1000 + i, 16, K, "student_t"), dev) for i in range(16)]
    for x in cal:
        obs.observe(x)
    amax = obs.amax.clone()
    rng = np.random.default_rng(0)
    cols = np.sort(rng.choice(N, 512, replace=False))
    wsub = d.w[cols].astype(np.float64)
    sat = clip = blocks = elems = 0
    err = {"static": [], "dynamic": []}
    for i in range(16):
        bits = W.random_act(5000 + i, 16, K, "student_t")
        x = to_dev_bf16(torch, bits, dev)
        cnt = nv.quantize_stats(x, amax).cpu().numpy()
        sat, clip = sat + int(cnt[0]), clip + int(cnt[1])
        blocks, elems = blocks + 16 * K // 16, elems + 16 * K
        ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64) @ wsub.T
        for name, a in (("static", amax), ("dynamic", None)):
            y = nv.linear(x, pw, a)[0].cpu().numpy().astype(np.float64)[:, cols]
            err[name].append(float(np.sqrt(np.mean((y - ref) ** 2)) / np.sqrt(np.mean(ref ** 2))))
    x0 = cal[0]
    t_obs = kernel_time_pairs(torch, lambda i: obs.observe(x0), 50)[0]
    out = torch.empty((16, N), dtype=torch.float32, device=dev)
    t_lin = kernel_time_pairs(torch, lambda i: nv.linear(x0, pw, amax, out=out), 50)[0]
    return {"metric": "NVFP4 static activation scale: calibration observer and held-out saturation / error",
            "value": round(float(np.mean(err["static"])), 6), "unit": "relative RMS error (static scale)",
            "n_gpus": 1, "steps": 16, "warmup": 0, "ms_per_step": round(t_lin * 1e3, 5), "higher_is_better": False,
            "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
            "config": {"workload": "decode_static_calibration_m16_k5120_n12288", "calibration_batches": 16,
                       "heldout_batches": 16, "calibrated_amax": float(amax.item()),
                       "saturated_block_fraction": sat / blocks, "clipped_element_fraction": clip / elems,
                       "rel_rms_error_static": round(float(np.mean(err["static"])), 6),
                       "rel_rms_error_dynamic": round(float(np.mean(err["dynamic"])), 6),
                       "observer_us": round(t_obs * 1e6, 2), "static_linear_us": round(t_lin * 1e6, 2)}}


def to_dev_bf16(torch, bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def time_region(torch, fn, steps, warmup):
    """Warm up, then time exactly `steps` calls of fn between synchronizations.
    fn(i) is called with i >= 1 for warmup calls and i = 0 .. steps-1 when timed."""
    for i in range(warmup):
        fn(i + 1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / 1e3, wall


def kernel_time_pairs(torch, launch, n, warmup=5):
    """Per-launch durations from HIP event pairs recorded around each launch on the launch
    stream (torch's current stream, which the library launches on).  Returns seconds:
    (mean, median, p10, p90)."""
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(evs):
        a.record()
        launch(i)
        b.record()
    torch.cuda.synchronize()
    d = np.array([a.elapsed_time(b) for a, b in evs]) / 1e3
    return float(np.mean(d)), float(np.median(d)), float(np.percentile(d, 10)), float(np.percentile(d, 90))


def copy_bandwidth(torch, dev, nbytes=512 << 20, reps=20):
    """Device-to-device copy GB/s (read + write), context for the HBM roofline."""
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    sec, _ = time_region(torch, lambda i: dst.copy_(src), reps, 3)
    del src, dst
    return 2 * nbytes * reps / sec / 1e9


def cpu_threads():
    try:
        return len(os.sched_getaffinity(0))
    except Exception:
        return os.cpu_count()


def host_info():
    """The host the CPU baseline ran on: CPU model, logical CPUs, the ones this
    process may use, RAM and the BLAS numpy calls (vendor, threads)."""
    info = {"cpu_model": None, "os_cpu_count": os.cpu_count(), "affinity": cpu_threads(), "ram_gb": None,
            "blas": None}
    try:
        with open("/proc/cpuinfo") as f:
            info["cpu_model"] = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
        with open("/proc/meminfo") as f:
            kb = next(int(l.split()[1]) for l in f if l.startswith("MemTotal"))
        info["ram_gb"] = round(kb / 2**20, 1)
    except Exception:
        pass
    try:
        import threadpoolctl
        info["blas"] = [{k: d.get(k) for k in ("internal_api", "version", "num_threads")}
                        for d in threadpoolctl.threadpool_info() if d.get("user_api") == "blas"]
    except Exception:
        pass
    return info


def oracle_threads():
    """Threads the oracle uses at most: its fp64 matmuls run on the BLAS thread
    pool; its elementwise numpy steps on one thread."""
    try:
        import threadpoolctl
        n = [d.get("num_threads") for d in threadpoolctl.threadpool_info() if d.get("user_api") == "blas"]
        if n and n[0]:
            return int(n[0])
    except Exception:
        pass
    return cpu_threads()


GPU_STATE = True


def gpu_state():
    """GPU power and clocks as amd-smi (else rocm-smi) reports them when called; None
    where neither tool answers or --no-gpu-state is given.  amd-smi's readings trail
    the load by about a second, so a snapshot taken right after a timed region
    reflects that region."""
    if not GPU_STATE:
        return None
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "--power", "--clock", "--json"], capture_output=True,
                           text=True, timeout=20)
        card = json.loads(r.stdout)["gpu_data"][0]
        clk = [v["clk"]["value"] for k, v in card["clock"].items()
               if k.startswith("gfx") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
        out = {"source": "amd-smi", "socket_power_W": card["power"]["socket_power"]["value"]}
        if clk:
            out.update({"gfx_clk_MHz_mean": round(sum(clk) / len(clk), 1), "gfx_clk_MHz_max": max(clk)})
        return out
    except Exception:
        pass
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--json"], capture_output=True,
                           text=True, timeout=20)
        card = next(iter(json.loads(r.stdout).values()))
        keep = {k: v for k, v in card.items() if "sclk" in k.lower() or "mclk" in k.lower()
                or "power" in k.lower()}
        return dict(keep, source="rocm-smi") if keep else None
    except Exception:
        return None


# ---------------------------------------------------------------------------------------
DECODE_COUNTERS = "linear_decode_kernel_decode_k5120_n12288_counters.md"
DECODE_SOURCES = ("gemm_skinny.hip", "rows_body.hpp", "quant_device.hpp", "common.hpp", "launch.hpp")
QUANT_COUNTERS = "quantize_act_kernel_down_proj_activation_m32768_k17408.md"
QUANT_SOURCES = ("quantize.hip", "quant_device.hpp", "common.hpp", "launch.hpp")
# the MFMA GEMM's counter summaries (FETCH_SIZE / WRITE_SIZE per launch), by prefill workload
MFMA_COUNTERS = {"prefill_gate_up": "gemm_mfma_kernel_prefill_gate_up_m8192_k5120_n34816.md",
                 "gdn_in_proj": "gemm_mfma_kernel_gdn_in_proj_m4096_k5120_n12352.md",
                 "down_proj": "gemm_mfma_kernel_down_proj_m32768_k17408_n5120.md"}
MFMA_SOURCES = ("gemm_mfma.hip", "rows_body.hpp", "quant_device.hpp", "common.hpp", "launch.hpp")


def one_launch_rows(K):
    """Rows up to which nvfp4_linear runs as one launch for this K (its documented bounds)."""
    return 16 if K <= 5120 else 8 if K <= 10240 else 4 if K <= 20480 else 0


def bench_decode(args, torch, nv, W, dev, d16=None):
    """The decode linear layer at M = 1, 4, 16 (the default: K = 5120, N = 12288;
    ``--config decode_down_proj``: K = 17408, N = 5120, where M = 16 runs as the
    quantizer then the GEMM)."""
    Ms = (1, 4, 16)
    headline = d16 is None
    if headline:
        d16 = W.decode(M=16)
    K, N = d16.K, d16.N
    workload = (f"decode_skinny_gemm_m1_m4_m16_k{K}_n{N}" if headline else f"decode_down_proj_m1_m4_m16_k{K}_n{N}")
    one_launch = {M: M <= one_launch_rows(K) for M in Ms}
    w = torch.from_numpy(d16.w).to(dev)
    pw0 = nv.pack_weight(w, d16.segments)
    del w
    copies = [pw0] + [nv.PackedWeight(pw0.codes.clone(), pw0.scales.clone(), pw0.g_dec.clone(), N, K,
                                      pw0.segments) for _ in range(args.copies - 1)]
    xs = {M: to_dev_bf16(torch, d16.x_bits[:M], dev) for M in Ms}
    acts = {M: (torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
                torch.empty((M, K // 16), dtype=torch.uint8, device=dev),
                torch.empty(1, dtype=torch.float32, device=dev)) for M in Ms}
    outs = {M: torch.empty((M, N), dtype=torch.float32, device=dev) for M in Ms}
    ws = nv.Workspace(dev)
    torch.cuda.synchronize()

    def step_eager(r):
        # one nvfp4_linear call per token count: a single launch (activation
        # quantization + GEMM + epilogue) where the rows fit the one-launch
        # layer, else the quantizer then the GEMM
        # every call streams a different weight copy, so no call finds its
        # weights in the 256 MB last-level cache (16 copies = 566 MB)
        for i, M in enumerate(Ms):
            nv.linear(xs[M], copies[(len(Ms) * r + i) % len(copies)], None, ws, out=outs[M], act_out=acts[M])

    nc = len(copies)
    if args.no_graph:
        sec, wall = time_region(torch, step_eager, args.steps, args.warmup)
    else:
        # one graph of exactly the timed steps and one of the warmup steps (weight
        # copies in rotation), so the timed region is a single replay: the host's
        # submission of separate replays does not show up as idle GPU time
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for r in range(nc):                # run the path once on a side stream before capture
                step_eager(r)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()

        def capture(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for r in range(n):
                    step_eager(r)
            return g

        timed_graph = capture(args.steps)
        warm_graph = capture(args.warmup) if args.warmup > 0 else None
        torch.cuda.synchronize()
        sec, wall = time_region(torch, lambda i: (timed_graph if i == 0 else warm_graph).replay(), 1,
                                1 if warm_graph is not None else 0)
    # algorithmic bytes of one step: packed weight + bf16 activations + fp32 outputs, per call
    wbytes = pw0.nbytes()
    step_bytes = sum(wbytes + 2 * M * K + 4 * M * N for M in Ms)
    value = step_bytes * args.steps / sec / 1e9

    # dominant kernel: the one-launch decode linear (linear_decode_kernel), one per
    # call.  Per M, a graph of nc back-to-back calls (one per weight copy) is
    # replayed with a HIP event pair around each replay on the launch stream;
    # per-launch duration = event time / nc.  Algorithmic bytes per launch =
    # weight codes+scales + bf16 activations + activation codes+scales written +
    # fp32 output.  The same is measured for two other forms of the call:
    # the GEMM alone on pre-quantized activations, and the quantizer followed by
    # the GEMM (two launches).
    def per_launch(call):
        if args.no_graph:
            launch = lambda i: [call(r) for r in range(nc)]
        else:
            gg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gg):
                for r in range(nc):
                    call(r)
            launch = lambda i, gg=gg: gg.replay()
        return [v / nc for v in kernel_time_pairs(torch, launch, max(8, args.steps // nc))]

    kern, forms = {}, {}
    for M in Ms:
        mean, med, p10, p90 = per_launch(
            lambda r, M=M: nv.linear(xs[M], copies[r], None, ws, out=outs[M], act_out=acts[M]))
        kb = wbytes + 2 * M * K + M * K * 9 // 16 + 4 * M * N
        kern[M] = {"mean_us": mean * 1e6, "median_us": med * 1e6, "p10_us": p10 * 1e6, "p90_us": p90 * 1e6,
                   "bytes": kb, "GBps": kb / mean / 1e9}
        c, sc, g = acts[M]
        gemv = per_launch(lambda r, M=M, c=c, sc=sc, g=g: nv.gemm(c, sc, g, copies[r], out=outs[M]))
        qg = per_launch(lambda r, M=M: nv.gemm(*nv.quantize_act(xs[M], None, ws, out=acts[M]), copies[r],
                                               out=outs[M]))
        gb = wbytes + M * K * 9 // 16 + 4 * M * N
        forms[M] = {"gemm_only_us": round(gemv[0] * 1e6, 3), "gemm_only_GBps": round(gb / gemv[0] / 1e9, 1),
                    "quantize_then_gemm_us": round(qg[0] * 1e6, 3),
                    "quantize_then_gemm_GBps": round(kb / qg[0] / 1e9, 1),
                    "one_launch_us": round(mean * 1e6, 3)}
    tot_b = sum(k["bytes"] for k in kern.values())
    tot_t = sum(k["mean_us"] for k in kern.values()) * 1e-6
    achieved = tot_b / tot_t / 1e9
    copy_gbs = copy_bandwidth(torch, dev)

    res = {
        "metric": "NVFP4 W4A4 decode linear GB/s (quantize + GEMM + epilogue), % of MI355X HBM roofline",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(sec / args.steps * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16",
        "dtype_note": "NVFP4 operands decoded exactly to fp16, fp16 MFMA products, fp32 accumulation",
        "data": "synthetic",
        "config": {"workload": workload, "M": list(Ms), "K": K, "N": N,
                   "segments": 1, "weight_copies": len(copies), "graphs": not args.no_graph,
                   "one_launch": {str(M): one_launch[M] for M in Ms},
                   "step_bytes": step_bytes, "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
                   "linear_kernel": {str(M): {k: round(v, 3) if isinstance(v, float) else v for k, v in kern[M].items()}
                                   for M in Ms},
                   "call_forms": {str(M): forms[M] for M in Ms},
                   "device_copy_GBps": round(copy_gbs, 1), "gpu_state_after_run": gpu_state()},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(DECODE_COUNTERS, DECODE_SOURCES) if headline else None,
                     "traffic_unit": "bytes per launch (mean over the three token counts)",
                     "algorithmic_bytes_per_launch": round(tot_b / len(Ms), 1),
                     "kernel": "linear_decode_kernel" if all(one_launch.values()) else
                               "linear_decode_kernel (one-launch rows); quantize_act_small_kernel + gemm_skinny_kernel "
                               "per call for the others",
                     "per_launch_bytes": {str(M): kern[M]["bytes"] for M in Ms}},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode(d16, Ms, args.cpu_seconds, step_bytes)
    if headline and not args.no_prefill:
        del copies, pw0, xs, acts, outs, ws
        if not args.no_graph:
            del timed_graph, warm_graph
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        res["config"]["prefill"] = prefill_legs(args, torch, nv, W, dev)
    return res


# ---- the oracle on the host: its row-independent steps over a thread pool ----------
def _row_chunks(rows, threads):
    return [c for c in np.array_split(np.arange(rows), max(1, min(threads, rows))) if len(c)]


def oracle_quantize(x32, amax, pool, threads):
    """oracle.nvfp4.quantize of a float32 [R, K] tensor with the given tensor maximum,
    row chunks on the pool (rows are independent once the maximum is fixed)."""
    from oracle import nvfp4 as Q
    parts = list(pool.map(lambda r: Q.quantize(x32[r], amax), _row_chunks(x32.shape[0], threads)))
    return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]), parts[0][2])


def oracle_dequantize(c, s, g, pool, threads):
    from oracle import nvfp4 as Q
    parts = list(pool.map(lambda r: Q.dequantize(c[r], s[r], g), _row_chunks(c.shape[0], threads)))
    return np.concatenate(parts)


def oracle_amax(x32, pool, threads):
    return np.float32(max(pool.map(lambda r: np.max(np.abs(x32[r])), _row_chunks(x32.shape[0], threads))))


def cpu_kind(threads):
    return (f"oracle (numpy; its encode/decode steps on {threads} threads over row chunks, "
            f"fp64 GEMMs on the BLAS threads)")


def cpu_baseline_decode(d16, Ms, target_s, step_bytes):
    """The oracle on the host: per call, quantize + decode the activations and run the fp64
    GEMM against the decoded weights (the weight decode is part of every oracle step).
    Sample: a slice of the weight's output columns (weights are encoded outside the
    timed part, like the GPU's pre-packed weights)."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import gemm as G
    from oracle import nvfp4 as Q
    from workloads import bf16_to_f32
    N, K = d16.N, d16.K
    cols = 1536
    threads = cpu_threads()
    wc, ws, wg, _ = Q.quantize(d16.w[:cols], np.float32(np.max(np.abs(d16.w))))
    t_all, reps = 0.0, 0
    with ThreadPoolExecutor(threads) as pool:
        while t_all < target_s and reps < 1000:
            t0 = time.perf_counter()
            w_hat = oracle_dequantize(wc, ws, wg, pool, threads)
            for M in Ms:
                x32 = bf16_to_f32(d16.x_bits[:M])
                c, s, g = oracle_quantize(x32, oracle_amax(x32, pool, threads), pool, threads)
                G.gemm_f64(oracle_dequantize(c, s, g, pool, threads), w_hat)
            t_all += time.perf_counter() - t0
            reps += 1
    per_step = t_all / reps * (N / cols)
    return {"value": round(step_bytes / per_step / 1e9, 4), "unit": "GB/s", "cores": max(threads, oracle_threads()),
            "kind": "oracle", "host": host_info(),
            "sample": f"{reps} oracle steps over {cols} of {N} output columns (token counts {list(Ms)}), "
                      f"scaled by {N / cols:.1f} to the full step; {t_all:.1f} s of CPU time; {cpu_kind(threads)}"}


# ---------------------------------------------------------------------------------------
GEMM_CONFIGS = {
    "tiny": lambda W: W.tiny(),
    "prefill_gate_up": lambda W: W.prefill_gate_up(),
    "gdn_in_proj": lambda W: W.gdn_in_proj(),
    "down_proj": lambda W: W.down_proj(),
}
GEMM_METRIC = "NVFP4 W4A4 prefill GEMM TFLOP/s (quantize + GEMM + epilogue), % of MI355X fp16 MFMA roofline"


def gemm_leg(args, torch, nv, dev, d, steps, warmup, cpu_seconds, x=None, counters=None):
    """One prefill workload: quantize (dynamic scale) + GEMM + per-module epilogue per
    step, timed over `steps` steps; the GEMM call alone timed with an event pair around
    each launch on its stream.  TFLOP/s counts 2 M N K.  `traffic` is the GEMM launch's
    HBM bytes from the counter summary `counters` in profiles/ (null when absent or
    taken on other sources); its algorithmic bytes are the activation and weight codes
    and scales read once and the fp32 output written once."""
    M, K, N = d.M, d.K, d.N
    pw = nv.pack_weight(torch.from_numpy(d.w).to(dev), d.segments)
    if x is None:
        x = to_dev_bf16(torch, d.x_bits, dev)
    c = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    s = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    g = torch.empty(1, dtype=torch.float32, device=dev)
    out = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws = nv.Workspace(dev)
    torch.cuda.synchronize()

    def step(i):
        nv.quantize_act(x, None, ws, out=(c, s, g))
        nv.gemm(c, s, g, pw, out=out)

    sec, _ = time_region(torch, step, steps, warmup)
    flops = 2.0 * M * N * K
    mean, med, p10, p90 = kernel_time_pairs(torch, lambda i: nv.gemm(c, s, g, pw, out=out), max(8, steps), 2)
    achieved = flops / mean / 1e12
    leg = {"workload": d.name, "M": M, "K": K, "N": N, "segments": len(d.segments),
           "gemm_form": {0: "weight_streaming", 1: "mfma", 2: "mfma_256x128"}[nv.nvfp4_gemm_form(M, K, N)],
           "steps": steps, "step_ms": round(sec / steps * 1e3, 4),
           "step_TFLOPs": round(flops * steps / sec / 1e12, 2),
           "gemm_kernel_mean_ms": round(mean * 1e3, 4), "gemm_kernel_median_ms": round(med * 1e3, 4),
           "gemm_kernel_p10_ms": round(p10 * 1e3, 4), "gemm_kernel_p90_ms": round(p90 * 1e3, 4),
           "gpu_state_after_run": gpu_state(),
           "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": F16_MFMA_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(achieved / F16_MFMA_PEAK_TFLOPS, 4),
                        "traffic": measured_traffic(counters, MFMA_SOURCES) if counters else None,
                        "traffic_unit": "HBM bytes per GEMM launch",
                        "algorithmic_bytes_per_launch": (M + N) * K * 9 // 16 + 4 * M * N,
                        "kernel": "gemm_mfma_kernel" if nv.nvfp4_gemm_form(M, K, N) >= 1 else "gemm_rows_kernel"}}
    if cpu_seconds > 0:
        leg["cpu_baseline"] = cpu_baseline_gemm(d, cpu_seconds, flops)
    del pw, c, s, g, out, ws
    return leg


def bench_gemm(args, torch, nv, W, dev):
    d = GEMM_CONFIGS[args.config](W)
    steps = max(1, args.steps)
    leg = gemm_leg(args, torch, nv, dev, d, steps, min(args.warmup, 5),
                   0 if args.no_cpu_baseline else args.cpu_seconds, counters=MFMA_COUNTERS.get(args.config))
    res = {"metric": GEMM_METRIC, "value": leg["step_TFLOPs"], "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
           "warmup": min(args.warmup, 5), "ms_per_step": leg["step_ms"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f16",
           "dtype_note": "NVFP4 operands decoded exactly to fp16, fp16 MFMA products, fp32 accumulation",
           "data": "synthetic",
           "config": {k: v for k, v in leg.items() if k not in ("roofline", "cpu_baseline")},
           "roofline": leg["roofline"]}
    if "cpu_baseline" in leg:
        res["cpu_baseline"] = leg["cpu_baseline"]
    return res


def cpu_baseline_gemm(d, target_s, flops):
    """The oracle on the host for one quantize + GEMM step of a prefill workload:
    quantize and decode a row sample of the activations (with the whole tensor's
    maximum), fp64 GEMM against a column sample of the decoded weight, scaled to the
    full M x N."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import gemm as G
    from oracle import nvfp4 as Q
    from workloads import bf16_to_f32
    rows, cols = min(d.M, 512), min(d.N, 4096)
    threads = cpu_threads()
    wc, ws, wg, _ = Q.quantize(d.w[:cols], np.float32(np.max(np.abs(d.w[:cols]))))
    t_all, reps = 0.0, 0
    with ThreadPoolExecutor(threads) as pool:
        w_hat = oracle_dequantize(wc, ws, wg, pool, threads)
        while t_all < target_s and reps < 1000:
            t0 = time.perf_counter()
            x32 = bf16_to_f32(d.x_bits[:rows])
            c, s, g = oracle_quantize(x32, oracle_amax(x32, pool, threads), pool, threads)
            G.gemm_f64(oracle_dequantize(c, s, g, pool, threads), w_hat)
            t_all += time.perf_counter() - t0
            reps += 1
    per_step = t_all / reps * (d.M / rows) * (d.N / cols)
    return {"value": round(flops / per_step / 1e12, 6), "unit": "TFLOP/s", "cores": max(threads, oracle_threads()),
            "kind": "oracle", "host": host_info(),
            "sample": f"{reps} oracle steps over {rows} of {d.M} rows and {cols} of {d.N} output columns, "
                      f"scaled by {d.M * d.N / (rows * cols):.1f} to the full step; {t_all:.1f} s of CPU time; "
                      f"{cpu_kind(threads)}"}


def quantize_leg(args, torch, nv, dev, x, x_bits, steps, cpu_seconds):
    """The standalone activation quantizer over one tensor: dynamic scale (amax pass,
    its reduction, the encode) as the leg's rate, the static (calibrated) mode too."""
    M, K = x.shape
    c = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    s = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    g = torch.empty(1, dtype=torch.float32, device=dev)
    ws = nv.Workspace(dev)
    torch.cuda.synchronize()
    sec, _ = time_region(torch, lambda i: nv.quantize_act(x, None, ws, out=(c, s, g)), steps, 3)
    nbytes = M * K * (2 + 2 + 9 / 16)      # amax pass reads x, encode pass reads x and writes codes+scales
    value = nbytes * steps / sec / 1e9
    amax = (g * 2688.0).contiguous()       # static mode with a calibrated maximum (here the tensor's own)
    sec_s, _ = time_region(torch, lambda i: nv.quantize_act(x, amax, ws, out=(c, s, g)), steps, 3)
    static_bytes = M * K * (2 + 9 / 16)
    leg = {"workload": f"down_proj_activation_quantize_m{M}_k{K}", "M": M, "K": K, "steps": steps,
           "dynamic_ms": round(sec / steps * 1e3, 4), "dynamic_GBps": round(value, 1),
           "algorithmic_bytes_dynamic": int(nbytes), "algorithmic_bytes_static": int(static_bytes),
           "static_ms": round(sec_s / steps * 1e3, 4),
           "static_GBps": round(static_bytes * steps / sec_s / 1e9, 1),
           "roofline": {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(value / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic(QUANT_COUNTERS, QUANT_SOURCES),
                        "traffic_unit": "bytes per dynamic-mode call (amax pass, its reduction and the encode)",
                        "algorithmic_bytes_per_call": int(nbytes),
                        "kernel": "amax_partial_kernel + amax_finalize_kernel + quantize_act_kernel"}}
    if cpu_seconds > 0:
        leg["cpu_baseline"] = cpu_baseline_quantize(x_bits, cpu_seconds, nbytes)
    del c, s, g, ws, amax
    return leg


def cpu_baseline_quantize(x_bits, target_s, nbytes):
    """The oracle's quantize of a row sample (with the whole tensor's maximum, and the
    maximum pass over the sample itself), scaled to the full tensor."""
    from concurrent.futures import ThreadPoolExecutor
    from workloads import bf16_to_f32
    M = x_bits.shape[0]
    rows = min(M, 256)
    threads = cpu_threads()
    amax = np.float32(np.max(np.abs(bf16_to_f32(x_bits[:rows]))))
    t_all, reps = 0.0, 0
    with ThreadPoolExecutor(threads) as pool:
        while t_all < target_s and reps < 1000:
            t0 = time.perf_counter()
            x32 = bf16_to_f32(x_bits[:rows])
            oracle_amax(x32, pool, threads)
            oracle_quantize(x32, amax, pool, threads)
            t_all += time.perf_counter() - t0
            reps += 1
    per_call = t_all / reps * (M / rows)
    return {"value": round(nbytes / per_call / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "host": host_info(),
            "sample": f"{reps} oracle quantize calls over {rows} of {M} rows, scaled by {M / rows:.1f}; "
                      f"{t_all:.1f} s of CPU time; {cpu_kind(threads)}"}


def bench_quantize(args, torch, nv, W, dev):
    d = W.down_proj()
    x = to_dev_bf16(torch, d.x_bits, dev)
    leg = quantize_leg(args, torch, nv, dev, x, d.x_bits, args.steps, 0 if args.no_cpu_baseline else args.cpu_seconds)
    res = {"metric": "NVFP4 activation quantize GB/s (dynamic scale), % of MI355X HBM roofline",
           "value": leg["dynamic_GBps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": 3,
           "ms_per_step": leg["dynamic_ms"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32", "data": "synthetic",
           "config": {k: v for k, v in leg.items() if k not in ("roofline", "cpu_baseline")},
           "roofline": leg["roofline"]}
    if "cpu_baseline" in leg:
        res["cpu_baseline"] = leg["cpu_baseline"]
    return res


def prefill_legs(args, torch, nv, W, dev):
    """The prefill half of the metric, in the same run as the decode headline: the
    gate+up (8192 x 5120 x 2 x 17408), GDN in-projection (4096 x 5120 x 12352, six
    modules) and down projection (32768 x 17408 x 5120) GEMMs, each quantize + GEMM
    per step, and the standalone quantizer over the down projection's input."""
    cpu_s = 0 if args.no_cpu_baseline else args.prefill_cpu_seconds
    legs = {}
    for name in ("prefill_gate_up", "gdn_in_proj", "down_proj"):
        print(f"[bench] prefill leg {name}", file=sys.stderr, flush=True)
        d = GEMM_CONFIGS[name](W)
        x = to_dev_bf16(torch, d.x_bits, dev)
        legs[name] = gemm_leg(args, torch, nv, dev, d, args.prefill_steps, 3, cpu_s, x=x,
                              counters=MFMA_COUNTERS[name])
        if name == "down_proj":
            print("[bench] prefill leg down_proj_quantize", file=sys.stderr, flush=True)
            legs["down_proj_quantize"] = quantize_leg(args, torch, nv, dev, x, d.x_bits, args.prefill_steps, cpu_s)
        del d, x
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return legs


if __name__ == "__main__":
    main()
