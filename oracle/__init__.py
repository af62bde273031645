"""CPU oracle for the FP8 block-scaled GEMM path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, header,
table or helper with the HIP library under ``fp8_block_scaled_gemm_amd/``.

What it computes, and where the pages say so (pages are the five DeepGEMM
news/blog pages; each function cites the page title and section it follows):

* ``e4m3``  - the FP8 E4M3 number format (4 exponent bits, 3 mantissa bits),
  named in the ai.abqq.net DeepGEMM summary, section 3 "core functions and
  features".  Decode is the format definition; encode is round-to-nearest-even
  with saturation at the largest finite value (448).
* ``quant`` - DeepSeek-V3 style fine-grained scaling (机器之心 DeepGEMM report,
  opening section; CSDN "DeepGEMM: concise, efficient ..." article, "what is
  DeepGEMM"): one fp32 scale per 1x128 activation group and per 128x128 weight
  block, scale = amax / 448.
* ``bf16``  - exact widening of bf16 activations to fp32 (for the bf16-input quantizer).
* ``gemm``  - the three GEMM forms the pages list (normal, contiguous-grouped,
  masked-grouped: 机器之心 report, "quick start"; ai.abqq.net summary, section 3;
  3loumao explainer, section 03): dequantise exactly and multiply in fp64.
* ``train`` - the backward GEMMs of a linear layer (the pages say the library serves V3/R1
  training; the layouts are readings): per-channel token groups, transposed block scales and
  the GEMM whose two operands both carry per-row group scales.

Every function here is pinned by ``tests/test_oracle_*.py`` against facts that
do not come from this package (the format definition, torch's independent
float8_e4m3fn codec, exact rational arithmetic, closed forms, invariants).
"""

from . import bf16, e4m3, quant, gemm, train  # noqa: F401
