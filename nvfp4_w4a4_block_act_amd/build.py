"""Build the gfx950 HIP library libnvfp4_w4a4.so in-tree with hipcc.

Usage: python -m nvfp4_w4a4_block_act_amd.build   (or build() from Python).
Always recompiles.  Every .hip file is compiled for gfx950 only, with FP
contraction off (the encoder must round each binary32 operation on its own)
and the packed-fp32 instructions disabled.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libnvfp4_w4a4.so")
ARCH = "gfx950"

HIP_SOURCES = ["quantize.hip", "gemm_skinny.hip", "gemm_mfma.hip", "kv_fp8.hip", "stream_probe.hip"]
HOST_SOURCES = ["api.cpp", "dispatch.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function"]
DEVICE = [f"--offload-arch={ARCH}", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the NVFP4 library)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if p.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False):
    hipcc = _hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(objdir, src + ".o")
        jobs.append([hipcc, *COMMON, *DEVICE, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(objdir, src + ".o")
        jobs.append([hipcc, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out:
                print(out)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
