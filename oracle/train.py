"""Training-side layouts for the CPU oracle: the backward GEMMs of a linear layer.
TEST INFRASTRUCTURE ONLY.

The pages say the library serves DeepSeek-V3/R1 training as well as inference, and name "MoE
training forward" as a use of the contiguous layout (机器之心 DeepGEMM report, opening
section; 3loumao explainer, section 03 "how DeepSeek innovated"; ai.abqq.net summary, section 3
"application scenarios").  They say nothing about the backward pass.  The readings taken here
(listed again in the design notes):

* O22 the backward passes of Y = X W^T (X: M x K tokens, W: N x K) keep the fine-grained recipe,
  with the scale groups along each GEMM's own contraction dimension:
    - dgrad  dX = dY W: the contraction runs over N.  dY is quantized like any activation
      (1 x 128 groups along N).  W enters as W^T (K x N); a 128 x 128 block is square, so the
      block quantization of W^T is exactly the transpose of W's codes and scales.
    - wgrad  dW = dY^T X: the contraction runs over the M tokens.  Both dY and X are
      quantized in groups of 128 consecutive tokens per column ("per-channel groups"), and
      stored transposed so that the group dimension is contiguous: dY^T (N x M), X^T (K x M).
      Both operands of that GEMM then carry one scale per row per 128-token group.
* O23 the wgrad output is bf16 like every other GEMM output here, and the promotion multiplies
  the partial of each 128-token block by fl32(s_row_a * s_row_b).
* O24 a token count M that is not a multiple of 128 leaves a last group of M mod 128 tokens,
  quantized as if zero-padded to 128 (as reading O14 does for K).

Every quantization decision below is the one the forward quantizers make (reading O2/O3: the
scale amax/448 in fp32, an IEEE fp32 division, E4M3 round-to-nearest-even with saturation);
only the grouping differs.
"""

import numpy as np

from . import bf16, e4m3, gemm, quant

GROUP = 128
_F448 = np.float32(448.0)


def quantize_per_channel_group(x):
    """Quantize x (M, K) float32 in groups of 128 consecutive rows of one column (O22, O24).

    Returns (qt, st): qt uint8 (K, M), the codes of x transposed (qt[k, m] encodes x[m, k]);
    st float32 (K, ceil(M/128)), st[k, mb] the scale of column k over rows
    [128*mb, min(128*mb + 128, M)).  This is the per-row-group layout of an activation
    operand, for the matrix x^T.
    """
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    mb = -(-m // GROUP)
    qt = np.empty((k, m), dtype=np.uint8)
    st = np.empty((k, mb), dtype=np.float32)
    for b in range(mb):
        rows = x[b * GROUP:min(m, (b + 1) * GROUP)]        # (r, K): the group of every column
        amax = np.max(np.abs(rows), axis=0)                  # per column, exact
        s = np.where(amax == 0, np.float32(1.0), amax / _F448).astype(np.float32)
        y = (rows / s[None, :]).astype(np.float32)           # IEEE fp32 division
        qt[:, b * GROUP:b * GROUP + rows.shape[0]] = e4m3.encode(y).T
        st[:, b] = s
    return qt, st


def quantize_per_channel_group_bf16(bits):
    """The per-channel-group quantizer on bf16 input (bits as uint16, (M, K)), widened exactly."""
    return quantize_per_channel_group(bf16.decode(bits))


def transpose_blocks(q, s):
    """W^T's block quantization from W's (O22): codes (N, K) -> (K, N), block scales
    (ceil(N/128), ceil(K/128)) -> (ceil(K/128), ceil(N/128))."""
    return np.ascontiguousarray(np.asarray(q).T), np.ascontiguousarray(np.asarray(s).T)


def gemm_nt_row_scaled(qa, sa, qb, sb):
    """D = A' B'^T (M, N) fp64 where both operands carry one scale per row per 128-wide group of
    the contraction dimension: qa (M, K), sa (M, ceil(K/128)), qb (N, K), sb (N, ceil(K/128)).

        D[m, n] = sum_kb sa[m, kb] * sb[n, kb] * sum_{k in kb} dec(qa[m, k]) * dec(qb[n, k])
    """
    return gemm.dequantize_rows(qa, sa) @ gemm.dequantize_rows(qb, sb).T


def linear_forward(x, w):
    """Y = X W^T through the library's recipe: X per-token groups, W 128x128 blocks."""
    qa, sa = quant.quantize_per_token_group(x)
    qb, sb = quant.quantize_per_block(w)
    return gemm.gemm_nt(qa, sa, qb, sb)


def linear_dgrad(dy, w):
    """dX = dY W (O22): dY per-token groups along N, W^T from W's block quantization."""
    qa, sa = quant.quantize_per_token_group(dy)
    qwt, swt = transpose_blocks(*quant.quantize_per_block(w))
    return gemm.gemm_nt(qa, sa, qwt, swt)


def linear_wgrad(dy, x):
    """dW = dY^T X (O22): both operands in per-channel groups of 128 tokens, transposed."""
    qa, sa = quantize_per_channel_group(dy)
    qb, sb = quantize_per_channel_group(x)
    return gemm_nt_row_scaled(qa, sa, qb, sb)


def linear_wgrad_k_grouped(dy, x, group_tokens):
    """MoE weight gradients over the contiguous layout (the layout the pages name for MoE training
    forward): expert e's tokens are rows [start_e, start_e + T_e) of dY (M, N) and X (M, K), with
    start_e the sum of the earlier counts; dW_e = dY_e^T X_e, returned as (G, N, K) fp64, zero for an
    expert with no tokens.  Every T_e is a multiple of 128 (the layout's alignment), so no 128-token
    group straddles two experts: quantizing the whole matrices per channel gives each expert's
    operands exactly (reading O22)."""
    dy = np.asarray(dy, dtype=np.float32)
    x = np.asarray(x, dtype=np.float32)
    n, k = dy.shape[1], x.shape[1]
    out = np.zeros((len(group_tokens), n, k))
    start = 0
    for e, t in enumerate(group_tokens):
        assert t % GROUP == 0, "expert token counts must be multiples of 128"
        if t:
            out[e] = linear_wgrad(dy[start:start + t], x[start:start + t])
        start += t
    return out
