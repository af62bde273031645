"""Fine-grained FP8 quantizers for the CPU oracle.  TEST INFRASTRUCTURE ONLY.

The pages name the technique only: DeepGEMM uses the fine-grained scaling
proposed with DeepSeek-V3 (机器之心 DeepGEMM report, opening section; CSDN
"DeepGEMM: concise, efficient ..." article, "what is DeepGEMM"), with E4M3 data
(ai.abqq.net summary, section 3).  The readings taken where the pages are
silent (listed again in the design notes):

* O1 granularity: activations get one scale per row per 128-wide K group
  (1x128); weights one scale per 128x128 block, partial blocks at the N edge
  included;
* O2 scale: s = fl32(amax / 448), amax = max |x| over the group (exact);
* O3 quantized value: q = E4M3_rne_sat(fl32(x / s)), an IEEE fp32 division;
* O5 all-zero group: s = 1.0 and every code 0x00 (or 0x80 for -0.0);
* O14 ragged K (K not a multiple of 128): the last group holds K mod 128 elements and
  takes its amax over them (quantized as if zero-padded to 128).

All arithmetic that decides a code is done in IEEE fp32 here (numpy float32
division is correctly rounded), exactly as the GPU path must do it.
"""

import numpy as np

from . import bf16, e4m3

GROUP = 128
_F448 = np.float32(448.0)


def _scale_from_amax(amax):
    amax = np.asarray(amax, dtype=np.float32)
    safe = np.where(amax == 0, np.float32(1.0), amax)
    s = (safe / _F448).astype(np.float32)
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def _pad_k(x):
    """Reading O14 (ragged K): a K that is not a multiple of 128 leaves a last group of K mod 128
    elements; it is quantized as if padded with zeros to 128, which leaves its amax (and so its
    scale) that of the elements present.  Returns the zero-padded array."""
    k = x.shape[-1]
    kp = -(-k // GROUP) * GROUP
    if kp == k:
        return x
    pad = [(0, 0)] * (x.ndim - 1) + [(0, kp - k)]
    return np.pad(x, pad)


def quantize_per_token_group(x):
    """Quantize activations x (M, K) float32 with one scale per (row, 128-wide K group).

    Returns (q, sa): q uint8 (M, K) E4M3 codes, sa float32 (M, ceil(K/128)) with
    sa[m, kb] the scale of row m, columns [128*kb, min(128*kb + 128, K)).
    """
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    xp = _pad_k(x)
    g = xp.reshape(m, xp.shape[1] // GROUP, GROUP)
    amax = np.max(np.abs(g), axis=2)
    s = _scale_from_amax(amax)
    y = (g / s[:, :, None]).astype(np.float32)           # IEEE fp32 division
    q = e4m3.encode(y).reshape(m, xp.shape[1])[:, :k]
    return q, s


def quantize_per_token_group_bf16(bits):
    """The per-token-group quantizer on bf16 activations (bits as uint16, (M, K)): the values
    are widened to fp32 exactly (oracle.bf16.decode) and quantized as above."""
    return quantize_per_token_group(bf16.decode(bits))


def quantize_per_block(w):
    """Quantize weights w (N, K) float32 with one scale per 128x128 block.

    Returns (q, sb): q uint8 (N, K), sb float32 (ceil(N/128), ceil(K/128)).  A partial
    last block (N not a multiple of 128, or K: reading O14) takes its amax over the elements
    present.
    """
    w = np.asarray(w, dtype=np.float32)
    n, k_in = w.shape
    w = _pad_k(w)
    k = w.shape[1]
    nb = -(-n // GROUP)
    kb = k // GROUP
    q = np.empty((n, k), dtype=np.uint8)
    sb = np.empty((nb, kb), dtype=np.float32)
    for i in range(nb):
        rows = w[i * GROUP:min(n, (i + 1) * GROUP)]
        blk = rows.reshape(rows.shape[0], kb, GROUP)
        amax = np.max(np.abs(blk), axis=(0, 2))
        s = _scale_from_amax(amax)
        sb[i] = s
        y = (blk / s[None, :, None]).astype(np.float32)
        q[i * GROUP:i * GROUP + rows.shape[0]] = e4m3.encode(y).reshape(rows.shape[0], k)
    return q[:, :k_in].copy(), sb


def quantize_per_block_grouped(w):
    """Per-block quantization of grouped weights w (G, N, K): each group on its own."""
    w = np.asarray(w, dtype=np.float32)
    qs, ss = zip(*(quantize_per_block(w[g]) for g in range(w.shape[0])))
    return np.stack(qs), np.stack(ss)
