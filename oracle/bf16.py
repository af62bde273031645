"""bfloat16 inputs for the CPU oracle.  TEST INFRASTRUCTURE ONLY.

bf16 is the upper half of an IEEE fp32 word: 1 sign bit, 8 exponent bits, 7 mantissa bits.
Widening a bf16 value to fp32 is therefore exact (append 16 zero bits), so an activation
quantizer fed bf16 data computes exactly what the fp32 quantizer computes on the widened
values.  Activations often arrive in bf16 on the DeepSeek-V3 path the pages describe
(bf16 output of the GEMM itself: 机器之心 DeepGEMM report, "quick start"), which is why the
bf16-input quantizer exists.
"""

import numpy as np


def decode(bits):
    """bf16 bit patterns (any integer array) -> float32 values, exactly (NaN payloads kept)."""
    b = np.asarray(bits).astype(np.uint32) & np.uint32(0xFFFF)
    return (b << np.uint32(16)).view(np.float32)
