"""GEMM parity at the workloads' full sizes, on sampled output rows.

Every workload the benchmark times runs here at its real shape, through the same entry points and
launch configuration (default workspace, so the same tile plan and K split):

- the 18 DeepSeek-V3 dense shapes;
- contiguous MoE, G in {4, 8};
- masked MoE, 32 x 256;
- the 16384 x 7168 x 16384 prefill;
- Zipf MoE, 64 experts.

Inputs are drawn on the device by ``inputs.DeviceGen`` (seeded). The oracle receives, copied to
the host, only the fp32 rows and weight matrices that the sampled outputs depend on, and
quantizes them itself. An output row depends only on its own activation row and on its group's
weights. So the GPU's quantized bytes and scales for exactly those rows and weights are compared
with the oracle's bit for bit first. After that, the GPU GEMM (which runs on the library's own
quantization) and the oracle GEMM see identical operands for every sampled output.

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
from gpu_util import BF16_NAN, _pool, bits32, check_gemm, device, oracle_quant_blocks, say

pytestmark = pytest.mark.gpu


def sample_rows(m, seed, n_random=20):
    """Rows at the first tile boundaries (64- and 128-row tiles, both sides), the last rows and
    seeded random rows."""
    fixed = {0, 1, 63, 64, 127, 128, 191, 192, 255, 256, m - 2, m - 1}
    rng = np.random.default_rng(seed)
    rnd = set(rng.choice(m, size=min(n_random, m), replace=False).tolist())
    return np.array(sorted(r for r in fixed | rnd if 0 <= r < m), dtype=np.int64)


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
    qa_s, sa_s = oracle.quant.quantize_per_token_group(a_dev[r].cpu().numpy())
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


@pytest.mark.parametrize("n,k", inputs.DENSE_V3_NK)
def test_dense_v3_full_size(n, k):
    """The three M of one (N, K) of the DeepSeek-V3 dense set, full size, sampled rows."""
    dev = device()
    gen = inputs.DeviceGen(torch, dev, 7000 + n + k)
    w = gen.normal((n, k), 0.02)
    say("full dense weights", n, k)
    qb_d, sb_d = dg.dg_quantize_per_block(w)
    qb, sb = check_weights(w, qb_d, sb_d)
    for m in inputs.DENSE_V3_M:
        say("full dense gemm", m, n, k, dg.dg_gemm_config_name(0, m, n, k))
        a = gen.activations(m, k)
        qa_d, sa_d = dg.dg_quantize_per_token_group(a)
        d = dg.dg_gemm_fp8_nt(qa_d, sa_d, qb_d, sb_d)
        torch.cuda.synchronize()
        rows = sample_rows(m, m + n + k)
        qa_s, sa_s = check_act_rows(a, qa_d, sa_d, rows)
        check_gemm(d[idx(rows, d)], oracle_gemm_rows(qa_s, sa_s, qb, sb), f"dense {m}x{n}x{k}")


def test_large_dense_full_size():
    """M=16384, N=7168, K=16384 prefill, sampled rows."""
    m, n, k = 16384, 7168, 16384
    dev = device()
    gen = inputs.DeviceGen(torch, dev, 5150)
    w = gen.normal((n, k), 0.02)
    say("full large dense", m, n, k, dg.dg_gemm_config_name(0, m, n, k))
    qb_d, sb_d = dg.dg_quantize_per_block(w)
    qb, sb = check_weights(w, qb_d, sb_d)
    a = gen.activations(m, k)
    qa_d, sa_d = dg.dg_quantize_per_token_group(a)
    d = dg.dg_gemm_fp8_nt(qa_d, sa_d, qb_d, sb_d)
    torch.cuda.synchronize()
    rows = sample_rows(m, 99)
    qa_s, sa_s = check_act_rows(a, qa_d, sa_d, rows)
    check_gemm(d[idx(rows, d)], oracle_gemm_rows(qa_s, sa_s, qb, sb), "large dense")


def contiguous_case(name, sizes, n, k, seed, n_experts=3):
    dev = device()
    g = len(sizes)
    m_idx_np, starts, valid_np = inputs.contiguous_layout(sizes)
    m_total = m_idx_np.shape[0]
    gen = inputs.DeviceGen(torch, dev, seed)
    w = gen.normal((g, n, k), 0.02)
    a = gen.activations(m_total, k) * torch.from_numpy(valid_np).to(dev).float()[:, None]
    say(f"full {name}", g, m_total, n, k, dg.dg_gemm_config_name(1, m_total, n, k, g))
    qb_d, sb_d = dg.dg_quantize_per_block(w)
    qa_d, sa_d = dg.dg_quantize_per_token_group(a)
    d = dg.dg_gemm_fp8_grouped_contiguous(qa_d, sa_d, qb_d, sb_d, torch.from_numpy(m_idx_np).to(dev))
    torch.cuda.synchronize()
    # sampled experts: the largest, the smallest non-empty and one in between
    order = [e for e in np.argsort(sizes) if sizes[e] > 0]
    experts = sorted({int(order[-1]), int(order[0]), int(order[len(order) // 2])})[:n_experts]
    rng = np.random.default_rng(seed)
    for e in experts:
        st, sz = int(starts[e]), int(sizes[e])
        pad = inputs.pad_to(sz)
        rows = {st, st + sz - 1} | set((st + rng.choice(sz, size=min(8, sz), replace=False)).tolist())
        if pad > sz:
            rows |= {st + sz, st + pad - 1}   # padding rows: exactly zero
        rows = np.array(sorted(rows), dtype=np.int64)
        qb, sb = check_weights(w[e], qb_d[e], sb_d[e])
        qa_s, sa_s = check_act_rows(a, qa_d, sa_d, rows)
        ref = oracle_gemm_rows(qa_s, sa_s, qb, sb)
        got = d[idx(rows, d)].float().cpu().numpy()
        is_pad = ~valid_np[rows]
        assert np.all(got[is_pad] == 0.0) and np.all(ref[is_pad] == 0.0), f"{name}: padding rows not zero"
        check_gemm(got[~is_pad], ref[~is_pad], f"{name} expert {e}")


@pytest.mark.parametrize("g", [4, 8])
@pytest.mark.parametrize("n,k", inputs.GROUPED_NK)
def test_contiguous_full_size(g, n, k):
    """G experts of ~8192 rows (+-25%) padded to 128, per-expert (N, K); sampled experts and rows."""
    sizes = inputs.uniform_group_sizes(inputs.rng_for("contiguous", g), g)
    contiguous_case(f"contiguous G={g}", sizes, n, k, 8100 + g + n)


def test_zipf_full_size():
    """64 experts, 32768 routed rows with Zipf(1.1) sizes, (N, K) = (2048, 7168)."""
    sizes = inputs.zipf_group_sizes(inputs.rng_for("zipf"))
    contiguous_case("zipf", sizes, 2048, 7168, 8300)


@pytest.mark.parametrize("n,k", inputs.GROUPED_NK)
def test_masked_full_size(n, k):
    """32 experts x 256-row buffers, masked_m ~ U{0..256}: sampled experts and rows against the
    oracle, and the sentinel kept in every row past masked_m of every expert."""
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
    nonempty = [e for e in range(g) if masked_np[e] > 0]
    experts = sorted({nonempty[0], nonempty[len(nonempty) // 2], nonempty[-1]})
    rng = np.random.default_rng(n)
    for e in experts:
        mv = int(masked_np[e])
        rows = np.array(sorted({0, mv - 1} | set(rng.choice(mv, size=min(6, mv), replace=False).tolist())))
        qb, sb = check_weights(w[e], qb_d[e], sb_d[e])
        qa_s, sa_s = check_act_rows(a[e], qa_d[e], sa_d[e], rows)
        check_gemm(d[e][idx(rows, d)], oracle_gemm_rows(qa_s, sa_s, qb, sb), f"masked expert {e}")
