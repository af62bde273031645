"""Seeded synthetic inputs for the FP8 block-scaled GEMM workloads.

This module only draws random numbers and builds index structures; it holds
none of the method's arithmetic (no quantization, no GEMM).  It is the one
module that both the HIP path's tests/bench and the CPU oracle's checks feed
from.  Only numpy is imported at module level; ``DeviceGen`` draws the same
distributions with torch's seeded generator on a device, for inputs of many GB.

Workloads (the pages benchmark the GEMM shapes of DeepSeek-V3/R1 inference, prefill and
decode, with no tensor parallelism - 机器之心 DeepGEMM report, "performance"; that shape set is
not a public dataset, so these seeded, V3-shaped synthetic workloads stand in for it):

* ``small``        M=128, N=512, K=512; A, B ~ N(0, 1).
* ``dense_v3``     M in {64, 128, 4096} x (N, K) in six V3 projection shapes;
                   A ~ N(0, 1) with 1% of rows scaled by 100; B ~ N(0, 0.02^2).
* ``contiguous``   G in {4, 8} experts, ~8192 rows each (uniform +-25%), every
                   group padded to a multiple of 128 and joined into one A with an
                   int32 expert index per row; per-expert B of (N, K) in
                   {(4096, 7168), (7168, 2048)}.
* ``masked``       G=32 experts, 256-row buffers, valid rows per expert uniform
                   in [0, 256]; (N, K) in {(4096, 7168), (7168, 2048)}.
* ``large_dense``  M=16384, N=7168, K=16384.
* ``zipf``         G=64 experts, 32768 routed rows, sizes ~ Zipf(s=1.1), padded
                   to 128; (N, K) = (2048, 7168).
"""

import numpy as np

ALIGN_M = 128  # row alignment of each group in the contiguous layout

DENSE_V3_NK = [(2112, 7168), (24576, 1536), (32768, 512),
               (7168, 16384), (4096, 7168), (7168, 2048)]
DENSE_V3_M = [64, 128, 4096]
GROUPED_NK = [(4096, 7168), (7168, 2048)]


def rng_for(name, *extra):
    """A numpy Generator seeded from a workload name and integers (stable across runs)."""
    seed = [sum(ord(c) * (i + 1) for i, c in enumerate(name))] + [int(e) for e in extra]
    return np.random.default_rng(seed)


def normal(rng, shape, std=1.0):
    """float32 N(0, std^2) samples."""
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def activations_with_outliers(rng, m, k, frac=0.01, factor=100.0):
    """A ~ N(0,1) with max(1, round(frac*m)) rows (drawn without replacement) multiplied by factor."""
    a = normal(rng, (m, k))
    n_out = max(1, int(round(frac * m)))
    rows = rng.choice(m, size=n_out, replace=False)
    a[rows] *= np.float32(factor)
    return a


def to_bf16_bits(x):
    """float32 -> bf16 bit patterns (uint16), round to nearest even: how a bf16 activation
    tensor of these values would hold them (input data for the bf16-input quantizer)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def pad_to(x, align=ALIGN_M):
    return -(-int(x) // align) * align


def uniform_group_sizes(rng, groups, mean_rows=8192, spread=0.25):
    """Rows per expert: round(mean_rows * U(1-spread, 1+spread))."""
    return np.rint(mean_rows * rng.uniform(1 - spread, 1 + spread, size=groups)).astype(np.int64)


def zipf_group_sizes(rng, groups=64, total_rows=32768, s=1.1):
    """Finite Zipf over ranks 1..groups (p_i ~ i^-s); counts ~ Multinomial(total_rows, p);
    ranks mapped to experts by a seeded permutation."""
    p = np.arange(1, groups + 1, dtype=np.float64) ** (-s)
    p /= p.sum()
    counts = rng.multinomial(total_rows, p)
    perm = rng.permutation(groups)
    sizes = np.empty(groups, dtype=np.int64)
    sizes[perm] = counts
    return sizes


def contiguous_layout(sizes, align=ALIGN_M):
    """Padded contiguous layout for per-expert row counts.

    Returns (m_indices int32 (M_total,), starts, valid): expert g owns rows
    [starts[g], starts[g] + pad(sizes[g])); its first sizes[g] rows are valid and the
    padding rows carry the same expert index.
    """
    padded = np.array([pad_to(s, align) for s in sizes], dtype=np.int64)
    starts = np.concatenate([[0], np.cumsum(padded)[:-1]]).astype(np.int64)
    m_indices = np.repeat(np.arange(len(sizes), dtype=np.int32), padded)
    valid = np.zeros(int(padded.sum()), dtype=bool)
    for g, (st, sz) in enumerate(zip(starts, sizes)):
        valid[st:st + sz] = True
    return m_indices, starts, valid


def contiguous_activations(rng, sizes, k, align=ALIGN_M, outliers=True):
    """A for the contiguous layout: valid rows random, padding rows zero."""
    m_indices, starts, valid = contiguous_layout(sizes, align)
    a = np.zeros((m_indices.shape[0], k), dtype=np.float32)
    nvalid = int(valid.sum())
    a[valid] = activations_with_outliers(rng, nvalid, k) if outliers else normal(rng, (nvalid, k))
    return a, m_indices, valid


def masked_counts(rng, groups=32, m_max=256):
    """Valid rows per expert, uniform integers in [0, m_max]."""
    return rng.integers(0, m_max + 1, size=groups).astype(np.int32)


def masked_activations(rng, groups, m_max, k):
    """A (G, M_max, K): every row random, including rows past masked_m (they must be ignored)."""
    a = activations_with_outliers(rng, groups * m_max, k)
    return a.reshape(groups, m_max, k)


def grouped_weights(rng, groups, n, k, std=0.02):
    return normal(rng, (groups, n, k), std)


def dense_v3_shapes():
    """The 18 (M, N, K) shapes of the V3-shaped dense workload, decode shapes first."""
    return [(m, n, k) for m in DENSE_V3_M for (n, k) in DENSE_V3_NK]


class DeviceGen:
    """The same recipes drawn on a torch device with a seeded torch generator (for workloads whose
    fp32 inputs are GBs: the full-size tests copy only the rows the oracle checks to the host)."""

    def __init__(self, torch, dev, seed):
        self.t = torch
        self.dev = dev
        self.g = torch.Generator(device=dev)
        self.g.manual_seed(int(seed))

    def normal(self, shape, std=1.0):
        return self.t.randn(shape, generator=self.g, device=self.dev, dtype=self.t.float32) * std

    def activations(self, m, k, frac=0.01, factor=100.0):
        """N(0,1) with max(1, round(frac*m)) rows, drawn without replacement, multiplied by factor."""
        a = self.normal((m, k))
        n_out = max(1, int(round(frac * m)))
        rows = self.t.randperm(m, generator=self.g, device=self.dev)[:n_out]
        a[rows] *= factor
        return a
