"""FP8 E4M3 codec (OCP "E4M3FN" variant) for the CPU oracle.  TEST INFRASTRUCTURE ONLY.

The pages fix only the field widths: E4M3 has a 4-bit exponent and a 3-bit
mantissa (ai.abqq.net DeepGEMM summary, section 3 "core functions and
features").  The variant is the one whose largest finite value is 448, which is
what the amax/448 scale rule of the fine-grained scaling implies (reading O4):

* code = s eeee mmm, exponent bias 7;
* e in 1..15: value (-1)^s * (1 + m/8) * 2^(e-7), except e=15, m=7 which is NaN
  (0x7F, 0xFF); so the largest finite magnitude is 1.75 * 2^8 = 448 (0x7E);
* e = 0: subnormal (-1)^s * (m/8) * 2^-6, smallest positive 2^-9 (0x01);
* no infinities.

Encoding (reading O3/O7 and the rounding rule "round to nearest, ties to even,
saturating"): finite |v| >= 448 gives the signed 448 code; otherwise v is
rounded to the nearest multiple of the quantum 2^(e-3) of its binade (the
subnormal binade shares the quantum of the first normal binade, 2^-9), ties to
even; the sign bit is kept, so negatives that round to zero give 0x80.
"""

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6          # 2^-6 is the smallest normal magnitude
_MANT_BITS = 3


def decode(codes):
    """Decode E4M3 codes (any integer array) to float64 values; NaN codes give NaN."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.ldexp(1.0, (e - 7).astype(np.int64))
    subnormal = (m / 8.0) * np.ldexp(1.0, _MIN_NORMAL_EXP)
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def encode(values):
    """Encode finite float values to E4M3 codes (uint8): RNE, saturating at 448, sign kept.

    Inputs are converted to float64 first; a float32 input is therefore encoded
    exactly as its own value (no intermediate rounding).  Non-finite inputs are
    outside the contract (reading O8) and raise.
    """
    v = np.asarray(values, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("E4M3 encode: non-finite input is outside the contract")
    neg = np.signbit(v)
    a = np.abs(v)

    # Binade exponent e = floor(log2 a), clamped to the subnormal binade.
    _, ex = np.frexp(a)                       # a = f * 2^ex with f in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, _MIN_NORMAL_EXP)
    quantum = np.ldexp(1.0, e - _MANT_BITS)   # spacing of E4M3 values in that binade
    r = np.rint(a / quantum) * quantum        # exact: division by a power of two; rint = ties-to-even

    # Pack the rounded magnitude r (0 <= r <= 448 whenever a < 448).
    _, rex = np.frexp(r)
    r_e = rex.astype(np.int64) - 1            # floor(log2 r) for r > 0
    is_normal = r >= np.ldexp(1.0, _MIN_NORMAL_EXP)
    exp_field = np.where(is_normal, r_e + 7, 0)
    mant_normal = np.rint((r / np.ldexp(1.0, np.where(is_normal, r_e, 0)) - 1.0) * 8.0)
    mant_sub = np.rint(r / np.ldexp(1.0, _MIN_NORMAL_EXP - _MANT_BITS))
    mant = np.where(is_normal, mant_normal, mant_sub).astype(np.int64)
    code = (exp_field << 3) | mant

    code = np.where(a >= E4M3_MAX, 0x7E, code)  # saturate
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


def all_finite_codes():
    """The 254 non-NaN codes, as uint8 (0x00..0x7E and 0x80..0xFE)."""
    c = np.arange(256, dtype=np.int64)
    keep = (c & 0x7F) != 0x7F
    return c[keep].astype(np.uint8)
