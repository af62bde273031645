"""GEMM parity at the workloads' full sizes.

Every workload the benchmark times runs here at its real shape, through the same entry points and
launch configuration (default workspace, so the same tile plan and K split):

- the 18 DeepSeek-V3 dense shapes: the 12 decode shapes (M = 64, 128) checked in full, the six
  M = 4096 shapes on a row sample;
- contiguous MoE, G in {4, 8}, and Zipf MoE, 64 experts: row samples;
- masked MoE, 32 x 256: every valid row of every expert checked in full;
- the 16384 x 7168 x 16384 prefill: a row sample.

A row sample holds both rows at every M-tile boundary of the plan the GEMM runs (the tile height
read from its configuration name), the first and last row, and 1024 further rows drawn by a
seeded generator; for the grouped layouts also every non-empty expert's first and last valid row
and its first and last padding row.  The counts are asserted.

Inputs are drawn on the device by ``inputs.DeviceGen`` (seeded). The oracle receives, copied to
the host, only the fp32 rows and weight matrices that the checked outputs depend on, and
quantizes them itself. An output row depends only on its own activation row and on its group's
weights. So the GPU's quantized bytes and scales for exactly those rows and weights are compared
with the oracle's bit for bit first. After that, the GPU GEMM (which runs on the library's own
quantization) and the oracle GEMM see identical operands for every checked output.

Acceptance as everywhere: |gpu - ref| <= 8e-3 |ref| + 1e-3 rms(ref) elementwise, relative
Frobenius <= 2e-3. Masked rows past masked_m keep the sentinel in every group, checked over the
whole output.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_gemm_amd as dg
from fp8_block_scaled_gemm_amd import inputs
import oracle
from gpu_util import BF16_NAN, _pool, bits32, check_gemm, device, oracle_quant_blocks, oracle_quant_rows, say

pytestmark = pytest.mark.gpu


N_SEEDED = 1024   # seeded rows of a row sample, beyond the fixed ones


def tile_height(config):
    """Rows of one M-tile of a GEMM plan, from its configuration name "BNxBM/...": BM."""
    return int(config.split("/")[0].split("x")[1])


def boundary_rows(m, bm):
    """The first and last row, and both rows at every boundary between two M-tiles of bm rows."""
    rows = {0, m - 1}
    for t in range(bm, m, bm):
        rows |= {t - 1, t}
    return rows


def sample_rows(m, bm, seed, n_random=N_SEEDED, pool=None):
    """Every M-tile boundary row (both sides) plus n_random further rows of `pool` (default: all
    rows) drawn by a seeded generator; asserts the counts."""
    fixed = boundary_rows(m, bm)
    pool = np.arange(m) if pool is None else np.asarray(pool)
    rest = np.setdiff1d(pool, np.fromiter(fixed, dtype=np.int64))
    rnd = np.random.default_rng(seed).choice(rest, size=min(n_random, rest.size), replace=False)
    rows = np.array(sorted(fixed | set(rnd.tolist())), dtype=np.int64)
    assert fixed <= set(rows.tolist()) and rows.size >= min(m, len(fixed) + min(n_random, rest.size))
    return rows


def oracle_gemm_rows(qa, sa, qb, sb, chunk=1024):
    """Oracle D for a few activation rows x all N columns, 128-aligned column blocks in threads."""
    n = qb.shape[0]
    starts = list(range(0, n, chunk))
    parts = list(_pool().map(
        lambda c: oracle.gemm.gemm_nt(qa, sa, qb[c:c + chunk], sb[c // 128:(min(c + chunk, n) + 127) // 128]),
        starts))
    return np.concatenate(parts, axis=1)


def gpu_bytes(t):
    return t.view(torch.uint8).cpu().numpy()


def idx(rows, t):
    return torch.as_tensor(rows, dtype=torch.long, device=t.device)


def check_act_rows(a_dev, qa_dev, sa_dev, rows):
    """Oracle quantization of the sampled fp32 rows of a_dev; the GPU's bytes and scales for them
    must match."""
    r = idx(rows, a_dev)
    qa_s, sa_s = oracle_quant_rows(a_dev[r].cpu().numpy())
    assert np.array_equal(gpu_bytes(qa_dev[r]), qa_s), "activation bytes differ on sampled rows"
    assert np.array_equal(bits32(sa_dev[:, r].T.contiguous().cpu().numpy()), bits32(sa_s)), \
        "activation scales differ on sampled rows"
    return qa_s, sa_s


def check_weights(w_dev, qb_dev, sb_dev):
    """Oracle quantization of one (N, K) weight matrix; the GPU's bytes and scales must match."""
    qb, sb = oracle_quant_blocks(w_dev.cpu().numpy())
    assert np.array_equal(gpu_bytes(qb_dev), qb), "weight bytes differ"
    assert np.array_equal(bits32(sb_dev.cpu().numpy()), bits32(sb)), "weight scales differ"
    return qb, sb


def dense_rows(m, n, k, seed):
    """All rows of a decode-size GEMM (M <= 128), else the row sample of its plan."""
    config = dg.dg_gemm_config_name(0, m, n, k)
    if m <= 128:
        return np.arange(m, dtype=np.int64), config
    return sample_rows(m, tile_height(config), seed), config


@pytest.mark.parametrize("n,k", inputs.DENSE_V3_NK)
def test_dense_v3_full_size(n, k):
    """The three M of one (N, K) of the DeepSeek-V3 dense set at full size: M = 64 and 128 checked
    in full, M = 4096 on its row sample."""
    dev = device()
    gen = inputs.DeviceGen(torch, dev, 7000 + n + k)
    w = gen.normal((n, k), 0.02)
    say("full dense weights", n, k)
    qb_d, sb_d = dg.dg_quantize_per_block(w)
    qb, sb = check_weights(w, qb_d, sb_d)
    for m in inputs.DENSE_V3_M:
        rows, config = dense_rows(m, n, k, m + n + k)
        say("full dense gemm", m, n, k, config, f"{rows.size} rows checked")
        a = gen.activations(m, k)
        qa_d, sa_d = dg.dg_quantize_per_token_group(a)
        d = dg.dg_gemm_fp8_nt(qa_d, sa_d, qb_d, sb_d)
        torch.cuda.synchronize()
        if m <= 128:
            assert rows.size == m
        else:
            assert rows.size >= N_SEEDED + 2 * (-(-m // tile_height(config)) - 1)
        qa_s, sa_s = check_act_rows(a, qa_d, sa_d, rows)
        check_gemm(d[idx(rows, d)], oracle_gemm_rows(qa_s, sa_s, qb, sb), f"dense {m}x{n}x{k}")


def test_large_dense_full_size():
    """M=16384, N=7168, K=16384 prefill, on its row sample."""
    m, n, k = 16384, 7168, 16384
    dev = device()
    gen = inputs.DeviceGen(torch, dev, 5150)
    w = gen.normal((n, k), 0.02)
    rows, config = dense_rows(m, n, k, 99)
    say("full large dense", m, n, k, config, f"{rows.size} rows checked")
    assert rows.size >= N_SEEDED + 2 * (-(-m // tile_height(config)) - 1)
    qb_d, sb_d = dg.dg_quantize_per_block(w)
    qb, sb = check_weights(w, qb_d, sb_d)
    a = gen.activations(m, k)
    qa_d, sa_d = dg.dg_quantize_per_token_group(a)
    d = dg.dg_gemm_fp8_nt(qa_d, sa_d, qb_d, sb_d)
    torch.cuda.synchronize()
    qa_s, sa_s = check_act_rows(a, qa_d, sa_d, rows)
    check_gemm(d[idx(rows, d)], oracle_gemm_rows(qa_s, sa_s, qb, sb), "large dense")


def contiguous_case(name, sizes, n, k, seed):
    """Row sample of a contiguous-layout GEMM: every M-tile boundary of its plan, every non-empty
    expert's first and last valid row and first and last padding row, and 1024 seeded valid rows;
    checked expert by expert (padding rows must be exactly zero)."""
    dev = device()
    g = len(sizes)
    m_idx_np, starts, valid_np = inputs.contiguous_layout(sizes)
    m_total = m_idx_np.shape[0]
    gen = inputs.DeviceGen(torch, dev, seed)
    w = gen.normal((g, n, k), 0.02)
    a = gen.activations(m_total, k) * torch.from_numpy(valid_np).to(dev).float()[:, None]
    config = dg.dg_gemm_config_name(1, m_total, n, k, g)
    say(f"full {name}", g, m_total, n, k, config)
    qb_d, sb_d = dg.dg_quantize_per_block(w)
    qa_d, sa_d = dg.dg_quantize_per_token_group(a)
    d = dg.dg_gemm_fp8_grouped_contiguous(qa_d, sa_d, qb_d, sb_d, torch.from_numpy(m_idx_np).to(dev))
    torch.cuda.synchronize()
    rows = set(sample_rows(m_total, tile_height(config), seed, pool=np.nonzero(valid_np)[0]).tolist())
    ends = set()
    for e in range(g):
        st, sz, pad = int(starts[e]), int(sizes[e]), inputs.pad_to(sizes[e])
        if sz > 0:
            ends |= {st, st + sz - 1}
        if pad > sz:
            ends |= {st + sz, st + pad - 1}
    rows = np.array(sorted(rows | ends), dtype=np.int64)
    assert ends <= set(rows.tolist()) and rows.size >= N_SEEDED + len(ends)
    say(f"full {name}: {rows.size} rows checked")
    owner = m_idx_np[rows]
    for e in range(g):
        r_e = rows[owner == e]
        if r_e.size == 0:
            continue
        qb, sb = check_weights(w[e], qb_d[e], sb_d[e])
        qa_s, sa_s = check_act_rows(a, qa_d, sa_d, r_e)
        ref = oracle_gemm_rows(qa_s, sa_s, qb, sb)
        got = d[idx(r_e, d)].float().cpu().numpy()
        is_pad = ~valid_np[r_e]
        assert np.all(got[is_pad] == 0.0) and np.all(ref[is_pad] == 0.0), f"{name}: padding rows not zero"
        if (~is_pad).any():
            check_gemm(got[~is_pad], ref[~is_pad], f"{name} expert {e}")


@pytest.mark.parametrize("g", [4, 8])
@pytest.mark.parametrize("n,k", inputs.GROUPED_NK)
def test_contiguous_full_size(g, n, k):
    """G experts of ~8192 rows (+-25%) padded to 128, per-expert (N, K), on the row sample."""
    sizes = inputs.uniform_group_sizes(inputs.rng_for("contiguous", g), g)
    contiguous_case(f"contiguous G={g}", sizes, n, k, 8100 + g + n)


def test_zipf_full_size():
    """64 experts, 32768 routed rows with Zipf(1.1) sizes, (N, K) = (2048, 7168)."""
    sizes = inputs.zipf_group_sizes(inputs.rng_for("zipf"))
    contiguous_case("zipf", sizes, 2048, 7168, 8300)


@pytest.mark.parametrize("n,k", inputs.GROUPED_NK)
def test_masked_full_size(n, k):
    """32 experts x 256-row buffers, masked_m ~ U{0..256}: every valid row of every expert against
    the oracle, and the sentinel kept in every row past masked_m of every expert."""
    dev = device()
    g, m_max = 32, 256
    masked_np = inputs.masked_counts(inputs.rng_for("masked"))
    gen = inputs.DeviceGen(torch, dev, 8500 + n)
    w = gen.normal((g, n, k), 0.02)
    a = gen.activations(g * m_max, k).reshape(g, m_max, k)
    say("full masked", g, m_max, n, k, dg.dg_gemm_config_name(2, m_max, n, k, g))
    qb_d, sb_d = dg.dg_quantize_per_block(w)
    qa_d, sa_d = dg.dg_quantize_per_token_group(a)
    sentinel = int(np.uint16(BF16_NAN).view(np.int16))
    d = torch.full((g, m_max, n), sentinel, dtype=torch.int16, device=dev).view(torch.bfloat16)
    masked = torch.from_numpy(masked_np.astype(np.int32)).to(dev)
    dg.dg_gemm_fp8_grouped_masked(qa_d, sa_d, qb_d, sb_d, masked, d=d)
    torch.cuda.synchronize()
    # untouched rows, every expert (on the device: compare the bit patterns with the sentinel)
    bits = d.view(torch.int16)
    row_ids = torch.arange(m_max, device=dev)[None, :, None]
    past = row_ids >= masked.clamp(0, m_max)[:, None, None]
    assert bool(torch.all(bits[past.expand_as(bits)] == sentinel)), "masked rows were written"
    written = bits[(~past).expand_as(bits)]
    assert not bool(torch.any(written == sentinel)), "a valid row was left unwritten"
    # every valid row of every expert against the oracle
    checked = 0
    for e in range(g):
        mv = int(masked_np[e])
        if mv == 0:
            continue
        rows = np.arange(mv, dtype=np.int64)
        qb, sb = check_weights(w[e], qb_d[e], sb_d[e])
        qa_s, sa_s = check_act_rows(a[e], qa_d[e], sa_d[e], rows)
        check_gemm(d[e][:mv], oracle_gemm_rows(qa_s, sa_s, qb, sb), f"masked expert {e}")
        checked += mv
    assert checked == int(np.sum(masked_np))
