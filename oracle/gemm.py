"""FP8 block-scaled GEMMs for the CPU oracle: dequantise exactly, multiply in fp64.
TEST INFRASTRUCTURE ONLY.

The three forms are the ones the pages list: a normal GEMM, a grouped GEMM
over a contiguous layout (all experts' rows joined into one block) and a
grouped GEMM over a masked layout (per-expert buffers, only marked rows
computed) - 机器之心 DeepGEMM report, "quick start"; ai.abqq.net summary,
section 3; 3loumao explainer, section 03 "how DeepSeek innovated".

The product is the plain definition the two-level accumulation approximates:

    D[m, n] = sum_kb sa[m, kb] * sb[n // 128, kb] * sum_{k in kb} dec(qa[m, k]) * dec(qb[n, k])

written here as D = A' B'^T with A' = dec(qa) * sa and B' = dec(qb) * sb,
both exact in fp64 (an E4M3 value has a 4-bit significand, a fp32 scale a
24-bit one).  The result stays fp64; it is not rounded to bf16.  The promotion
order on the GPU (per 128-deep K block) is a rounding-order choice that this
definition does not fix; the tolerance covers it.
"""

import numpy as np

from . import e4m3

GROUP = 128


def dequantize_rows(q, s):
    """A' = dec(q) * s with q (R, K) codes and s (R, ceil(K/128)) per-row group scales, fp64.
    A ragged last group (K mod 128 elements, reading O14) uses its own scale like the others."""
    q = np.asarray(q)
    r, k = q.shape
    kb = -(-k // GROUP)
    vals = np.zeros((r, kb * GROUP))
    vals[:, :k] = e4m3.decode(q)
    vals = vals.reshape(r, kb, GROUP)
    return (vals * np.asarray(s, dtype=np.float64)[:, :, None]).reshape(r, kb * GROUP)[:, :k]


def dequantize_blocks(q, s):
    """B' = dec(q) * s with q (N, K) codes and s (ceil(N/128), ceil(K/128)) block scales, fp64."""
    q = np.asarray(q)
    n, k = q.shape
    row_scales = np.repeat(np.asarray(s, dtype=np.float64), GROUP, axis=0)[:n]
    return dequantize_rows(q, row_scales)


def gemm_nt(qa, sa, qb, sb):
    """Normal GEMM D = A' B'^T (M, N) fp64; qa (M, K), sa (M, K/128), qb (N, K), sb (ceil(N/128), K/128)."""
    return dequantize_rows(qa, sa) @ dequantize_blocks(qb, sb).T


def gemm_grouped_contiguous(qa, sa, qb, sb, m_indices):
    """Contiguous-grouped GEMM: row r of D uses expert m_indices[r]'s weights.

    qa (M_total, K), sa (M_total, K/128), qb (G, N, K), sb (G, ceil(N/128), K/128),
    m_indices int (M_total,).  Rows whose index is outside [0, G) are left NaN
    (the GPU leaves them unwritten).
    """
    m_indices = np.asarray(m_indices)
    a = dequantize_rows(qa, sa)
    g_count, n, _ = np.asarray(qb).shape
    out = np.full((a.shape[0], n), np.nan)
    for g in range(g_count):
        rows = np.nonzero(m_indices == g)[0]
        if rows.size:
            out[rows] = a[rows] @ dequantize_blocks(qb[g], sb[g]).T
    return out


def gemm_grouped_masked(qa, sa, qb, sb, masked_m):
    """Masked-grouped GEMM: for each expert g only rows r < masked_m[g] are computed.

    qa (G, M_max, K), sa (G, M_max, K/128), qb (G, N, K), sb (G, ceil(N/128), K/128).
    Returns (G, M_max, N) fp64 with NaN in the rows that must stay unwritten.
    masked_m is clamped to [0, M_max] (reading O13).
    """
    qa = np.asarray(qa)
    g_count, m_max, _ = qa.shape
    n = np.asarray(qb).shape[1]
    out = np.full((g_count, m_max, n), np.nan)
    for g in range(g_count):
        rows = int(min(max(int(masked_m[g]), 0), m_max))
        if rows:
            out[g, :rows] = gemm_nt(qa[g, :rows], sa[g, :rows], qb[g], sb[g])
    return out
