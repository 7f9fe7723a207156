"""CPU oracle for the NVFP4 W4A4 linear layer -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct reference that the HIP path
is checked against.  Only the test suite, the smoke check in
``__graft_entry__.smoke`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (the C-ABI library and its Python binding) never
imports, links or calls anything here, and nothing here imports the product.

Sources (the pages this follows; no page prints code or worked values):

* Summary page "Summary of 'Why Gated DeltaNet Survives 4-Bit Quantization'",
  section "Background", item 1: the NVFP4 format -- E2M1 element values, one
  E4M3 scale per block of 16 elements derived from the block maximum divided
  by 6, and one FP32 scale per tensor.
* The paper abstract (chatpaper / ai-news-brief pages) and the Glonce article,
  sections "Who it affects" and "How to use it", plus the aiany page,
  "Mechanistic notes": modules calibrated one by one carry their own global
  scale; a GEMM that fuses several modules must apply each module's own scale
  to its output columns (the global-scale-mismatch repair).

Modules:
    formats -- E2M1 / E4M3FN code tables, round-to-nearest-even encoders.
    nvfp4   -- tensor quantize (encode), dequantize (decode), per-segment
               weight quantize.
    gemm    -- fp64 GEMM on decoded operands, exact int64 GEMM, error bound.

Parity status: every function is pinned by the CPU tests in
``tests/test_oracle_*.py`` (brute force over all code pairs, library casts,
closed forms, hand-worked fixtures under ``tests/golden/``).  What stays
unpinned is agreement with the pages' own NVIDIA implementation at rounding
ties and in the op order of the scale computation: the pages fix neither, so
the readings documented in ``nvfp4.quantize`` define them ("parity unpinned"
for those two points only).
"""
from . import formats, nvfp4, gemm  # noqa: F401
