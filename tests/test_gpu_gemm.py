"""GPU GEMMs (normal, contiguous-grouped, masked-grouped) against the fp64 CPU oracle.

Both sides get the same E4M3 bytes and fp32 scales (made by the oracle quantizer), so only the
GEMM is under test.  Acceptance: |gpu - ref| <= 8e-3 |ref| + 1e-3 rms(ref) elementwise, relative
Frobenius error <= 2e-3, masked rows untouched.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_gemm_amd as dg
from fp8_block_scaled_gemm_amd import inputs
import oracle
import oracle_pins
from gpu_util import BF16_NAN, bf16_bits, check_gemm, device, sa_to_dev, say, to_dev

pytestmark = pytest.mark.gpu


def quantized_operands(name, m, n, k, a_outliers=True, b_std=0.02):
    rng = inputs.rng_for(name, m, n, k)
    a = inputs.activations_with_outliers(rng, m, k) if a_outliers and m >= 2 else inputs.normal(rng, (m, k))
    b = inputs.normal(rng, (n, k), b_std)
    qa, sa = oracle.quant.quantize_per_token_group(a)
    qb, sb = oracle.quant.quantize_per_block(b)
    return qa, sa, qb, sb


def run_dense(qa, sa, qb, sb, workspace=True, ld_extra=0):
    m = qa.shape[0]
    ld = dg.dg_get_scale_ld(m) + ld_extra
    d = dg.dg_gemm_fp8_nt(to_dev(qa), sa_to_dev(sa, ld), to_dev(qb), to_dev(sb), use_workspace=workspace)
    torch.cuda.synchronize()
    return d


def test_small_config():
    """M=128, N=512, K=512, A and B ~ N(0, 1)."""
    say("gemm small 128x512x512")
    rng = inputs.rng_for("small")
    a = inputs.normal(rng, (128, 512))
    b = inputs.normal(rng, (512, 512))
    qa, sa = oracle.quant.quantize_per_token_group(a)
    qb, sb = oracle.quant.quantize_per_block(b)
    check_gemm(run_dense(qa, sa, qb, sb), oracle.gemm.gemm_nt(qa, sa, qb, sb), "small")


@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (77, 200, 384), (130, 260, 256), (257, 1000, 640),
                                   (64, 130, 512), (200, 2112, 1024), (129, 127, 128), (33, 4096, 768)])
def test_ragged_shapes(m, n, k):
    say("gemm ragged", m, n, k)
    qa, sa, qb, sb = quantized_operands("ragged", m, n, k)
    ref = oracle.gemm.gemm_nt(qa, sa, qb, sb)
    check_gemm(run_dense(qa, sa, qb, sb, ld_extra=4), ref, f"ragged {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(4608, 4096, 6144), (4096, 6144, 6144), (4096, 5120, 6144)])
def test_split_last_round(m, n, k):
    """More tiles than the persistent grid holds, with a partial last round and a long K: the whole
    tiles of the full rounds run unsplit and the last round's tiles are split in K (split1+tailN).
    Against the oracle, bit-identical on a repeat, and within tolerance of the unsplit
    (no-workspace) plan."""
    name = dg.dg_gemm_config_name(0, m, n, k)
    say("gemm split last round", m, n, k, name)
    if dg.dg_get_num_cus() == 256:   # 256x192: 24 x 16 = 384 tiles (tail 128); 256x256: 16 x 24 = 384
        assert "+tail" in name, name  # (tail 128); 256x128: 32 x 20 = 640 (tail 128)
    qa, sa, qb, sb = quantized_operands("tail", m, n, k)
    ref = oracle.gemm.gemm_nt(qa, sa, qb, sb)
    d1, d2 = run_dense(qa, sa, qb, sb), run_dense(qa, sa, qb, sb)
    assert np.array_equal(bf16_bits(d1), bf16_bits(d2))
    check_gemm(d1, ref, f"split last round {m}x{n}x{k}")
    check_gemm(run_dense(qa, sa, qb, sb, workspace=False), ref, f"unsplit {m}x{n}x{k}")


def test_split_k_deterministic():
    """Small M with a long K takes the split-K path; repeated calls are bit-identical and the
    no-workspace path agrees within tolerance."""
    say("gemm split-k 64x512x4096")
    m, n, k = 64, 512, 4096
    assert dg.dg_gemm_workspace_size(m, n, k) > 0
    qa, sa, qb, sb = quantized_operands("splitk", m, n, k)
    ref = oracle.gemm.gemm_nt(qa, sa, qb, sb)
    d1 = run_dense(qa, sa, qb, sb)
    d2 = run_dense(qa, sa, qb, sb)
    assert np.array_equal(bf16_bits(d1), bf16_bits(d2))
    check_gemm(d1, ref, "split-k")
    check_gemm(run_dense(qa, sa, qb, sb, workspace=False), ref, "no split")


def test_split_k_shared_workspace_sequence():
    """Split-K calls with different tile counts and splits, one after another on one workspace:
    each call's partials must never disturb the next call's arrival counters (regression: a
    workspace reused by a GEMM with more output tiles than the previous one)."""
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=device())
    shapes = [(64, 512, 4096), (64, 2112, 4096), (64, 4608, 8192), (128, 640, 4096), (64, 512, 4096)]
    for (m, n, k) in shapes:
        say("gemm split-k sequence", m, n, k, dg.dg_gemm_config_name(0, m, n, k))
        assert 0 < dg.dg_gemm_workspace_size(m, n, k) <= ws.numel()
        qa, sa, qb, sb = quantized_operands("splitseq", m, n, k)
        d = dg.dg_gemm_fp8_nt(to_dev(qa), sa_to_dev(sa), to_dev(qb), to_dev(sb), workspace=ws)
        torch.cuda.synchronize()
        check_gemm(d, oracle.gemm.gemm_nt(qa, sa, qb, sb), f"split sequence {m}x{n}x{k}")
    assert int(ws[:64 << 10].count_nonzero()) == 0, "arrival counters not left at zero"


def test_closed_form_all_448():
    say("gemm all-448")
    a = np.full((96, 512), 448.0, np.float32)
    b = np.full((136, 512), 448.0, np.float32)
    qa, sa = oracle.quant.quantize_per_token_group(a)
    qb, sb = oracle.quant.quantize_per_block(b)
    d = run_dense(qa, sa, qb, sb).float().cpu().numpy()
    assert np.all(d == 448.0 * 448.0 * 512)


def test_closed_form_hadamard():
    say("gemm hadamard")
    h = (448.0 * oracle_pins.hadamard(128)).astype(np.float32)
    qa, sa = oracle.quant.quantize_per_token_group(h)
    qb, sb = oracle.quant.quantize_per_block(h)
    d = run_dense(qa, sa, qb, sb).float().cpu().numpy()
    assert np.array_equal(d, 448.0 * 448.0 * 128 * np.eye(128))


def _rounding_cases(count):
    """fp32 bit patterns for the bf16 rounding test: ties to even in both directions, just below and
    above ties, large values that round to infinity, subnormals, both signs; then random patterns."""
    base = []
    for hi in (0x3F80, 0x3F81, 0x4049, 0x404A, 0x7F7F, 0x7F7E, 0x0001, 0x0040, 0x00FF, 0x0080, 0x3400):
        for lo in (0x8000, 0x7FFF, 0x8001, 0x0000, 0xFFFF, 0x4000, 0xC000):
            base.append((hi << 16) | lo)
    base += [0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x00008000, 0x00018000, 0x00000001, 0x007FFFFF]
    rng = np.random.default_rng(11)
    rand = rng.integers(0, 1 << 31, size=count, dtype=np.int64)
    rand = rand[((rand >> 23) & 0xFF) != 0xFF]   # finite patterns only
    pos = np.array(base + list(rand), dtype=np.int64)[: count // 2]
    bits = np.concatenate([pos, pos | (1 << 31)])[:count]   # and the negatives
    return bits.astype(np.uint32)


def test_bf16_output_rounding():
    """Closed form for the epilogue's fp32 -> bf16 rounding: A and B one-hot (one +-1.0 per row, same K
    column for row i of A and row i of B, block scales 1), so output (i, i) is exactly the activation
    scale sa[i] (+-), which is chosen to hit round-to-nearest-even ties, near-ties, overflow and
    subnormals; every diagonal element must equal torch's CPU bf16 conversion of that fp32 value,
    every other element is 0."""
    m = n = 256
    k = 256
    say("gemm bf16 rounding", m, n, k, dg.dg_gemm_config_name(0, m, n, k))
    bits = _rounding_cases(m)
    vals = bits.view(np.float32)
    qa = np.zeros((m, k), np.uint8)
    qb = np.zeros((n, k), np.uint8)
    idx = np.arange(m)
    qa[idx, idx % 128] = 0x38            # E4M3 1.0 (the sign goes into the scale)
    qb[idx, idx % 128] = 0x38
    sa = np.ones((m, k // 128), np.float32)
    sa[:, 0] = vals                      # K group 0 holds the only nonzero product of row i
    sb = np.ones((n // 128, k // 128), np.float32)
    d = run_dense(qa, sa, qb, sb)
    got = bf16_bits(d)
    want = torch.from_numpy(vals.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    diag = got[idx, idx]
    bad = np.nonzero(diag != want)[0]
    assert bad.size == 0, [(hex(int(bits[i])), hex(int(diag[i])), hex(int(want[i]))) for i in bad[:5]]
    off = got.copy()
    off[idx, idx] = 0
    same_col = (idx[:, None] % 128 == idx[None, :] % 128) & (idx[:, None] != idx[None, :])
    # rows i and i +- 128 share a K column: those entries carry row i's value as well
    assert np.array_equal(off[same_col], np.broadcast_to(want[:, None], (m, n))[same_col])
    assert np.all(off[~same_col] == 0)


def test_kblock_rebalance_bit_identical():
    """Scaling K block kb of A by 2^j and of B by 2^-j leaves the output bit-identical."""
    say("gemm k-block rebalance")
    qa, sa, qb, sb = quantized_operands("rebalance", 96, 384, 512)
    d0 = run_dense(qa, sa, qb, sb)
    sa2, sb2 = sa.copy(), sb.copy()
    sa2[:, 2] *= np.float32(2.0 ** 6)
    sb2[:, 2] *= np.float32(2.0 ** -6)
    d1 = run_dense(qa, sa2, qb, sb2)
    assert np.array_equal(bf16_bits(d0), bf16_bits(d1))


def test_row_scale_and_permutation():
    say("gemm row scale / permutation")
    qa, sa, qb, sb = quantized_operands("perm", 160, 256, 384)
    d0 = run_dense(qa, sa, qb, sb).float().cpu().numpy()
    sa2 = sa.copy()
    sa2[5] *= np.float32(4.0)
    d1 = run_dense(qa, sa2, qb, sb).float().cpu().numpy()
    assert np.array_equal(d1[5], 4.0 * d0[5]) and np.array_equal(d1[6:], d0[6:])
    p = np.random.default_rng(1).permutation(160)
    d2 = run_dense(qa[p], sa[p], qb, sb).float().cpu().numpy()
    assert np.array_equal(d2, d0[p])


def test_contiguous_small():
    """Three experts with ragged sizes padded to 128; padding rows give exact zeros; a block
    whose index is -1 is skipped and left untouched."""
    say("gemm contiguous small")
    rng = inputs.rng_for("contig_small")
    n, k = 384, 512
    sizes = np.array([100, 300, 1], dtype=np.int64)
    a, m_idx, valid = inputs.contiguous_activations(rng, sizes, k)
    b = inputs.grouped_weights(rng, 3, n, k)
    qa, sa = oracle.quant.quantize_per_token_group(a)
    qb, sb = oracle.quant.quantize_per_block_grouped(b)
    m_idx = m_idx.copy()
    m_idx = np.concatenate([m_idx, np.full(128, -1, np.int32)])      # an unmapped trailing block
    qa = np.concatenate([qa, np.zeros((128, k), np.uint8)])
    sa = np.concatenate([sa, np.ones((128, k // 128), np.float32)])
    m_total = qa.shape[0]
    d = torch.full((m_total, n), 0, dtype=torch.int16, device=device()).fill_(-1).view(torch.bfloat16)
    dg.dg_gemm_fp8_grouped_contiguous(to_dev(qa), sa_to_dev(sa), to_dev(qb), to_dev(sb), to_dev(m_idx), d=d)
    torch.cuda.synchronize()
    ref = oracle.gemm.gemm_grouped_contiguous(qa, sa, qb, sb, m_idx)
    mapped = m_idx >= 0
    check_gemm(d[torch.from_numpy(mapped).to(device())], ref[mapped], "contiguous")
    bits = bf16_bits(d)
    assert np.all(bits[~mapped] == BF16_NAN)
    pad = mapped & ~np.concatenate([valid, np.zeros(128, bool)])
    assert np.all(d.float().cpu().numpy()[pad] == 0.0)


def test_contiguous_g1_equals_dense():
    say("gemm contiguous G=1 vs dense")
    qa, sa, qb, sb = quantized_operands("contig_g1", 256, 320, 384)
    d0 = run_dense(qa, sa, qb, sb)
    d1 = dg.dg_gemm_fp8_grouped_contiguous(to_dev(qa), sa_to_dev(sa), to_dev(qb[None]), to_dev(sb[None]),
                                           to_dev(np.zeros(256, np.int32)))
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(d0), bf16_bits(d1))


def masked_case(name, g, m_max, n, k, masked):
    rng = inputs.rng_for(name, g, m_max, n, k)
    a = inputs.masked_activations(rng, g, m_max, k)
    b = inputs.grouped_weights(rng, g, n, k)
    qa, sa = oracle.quant.quantize_per_token_group(a.reshape(g * m_max, k))
    qa = qa.reshape(g, m_max, k)
    kb = -(-k // 128)
    sa = sa.reshape(g, m_max, kb)
    qb, sb = oracle.quant.quantize_per_block_grouped(b)
    ld = dg.dg_get_scale_ld(m_max)
    sa_dev = np.zeros((g, kb, ld), np.float32)
    sa_dev[:, :, :m_max] = sa.transpose(0, 2, 1)
    d = torch.full((g, m_max, n), -1, dtype=torch.int16, device=device()).view(torch.bfloat16)
    masked = np.asarray(masked, np.int32)
    dg.dg_gemm_fp8_grouped_masked(to_dev(qa), to_dev(sa_dev), to_dev(qb), to_dev(sb), to_dev(masked), d=d)
    torch.cuda.synchronize()
    ref = oracle.gemm.gemm_grouped_masked(qa, sa, qb, sb, masked)
    bits = bf16_bits(d)
    for e in range(g):
        rows = int(min(max(masked[e], 0), m_max))
        assert np.all(bits[e, rows:] == BF16_NAN), f"group {e}: rows past masked_m were written"
        if rows:
            check_gemm(d[e, :rows], ref[e, :rows], f"masked group {e}")
    return d


def test_masked_small():
    say("gemm masked small")
    masked_case("masked_small", 6, 256, 384, 512, [0, 1, 100, 256, 300, -5])


def test_masked_decode_split():
    """Small m_max with a long K takes the split-K path in the masked layout."""
    say("gemm masked split-k")
    masked_case("masked_split", 4, 64, 256, 2048, [64, 7, 0, 33])


def test_gemm_errors():
    say("gemm errors")
    a = torch.zeros((4, 100), dtype=torch.uint8, device=device())
    b = torch.zeros((8, 100), dtype=torch.uint8, device=device())
    sa = torch.zeros((1, 4), dtype=torch.float32, device=device())
    sb = torch.zeros((1, 1), dtype=torch.float32, device=device())
    with pytest.raises(dg.DGError, match="INVALID_ARG"):
        dg.dg_gemm_fp8_nt(a, sa, b, sb)


# ---- ragged K (K % 128 != 0, K % 16 == 0): the last K group is partial --------------------------

@pytest.mark.parametrize("m,n,k", [(1, 32, 16), (64, 200, 144), (64, 512, 4112), (130, 260, 400),
                                   (300, 1000, 1040), (33, 4096, 784), (257, 640, 2064)])
def test_ragged_k(m, n, k):
    """Dense GEMM with a partial last K group, across the decode (split and unsplit) and large
    tile configurations; the absent K positions must contribute nothing."""
    say("gemm ragged k", m, n, k, dg.dg_gemm_config_name(0, m, n, k))
    qa, sa, qb, sb = quantized_operands("ragged_k", m, n, k)
    check_gemm(run_dense(qa, sa, qb, sb, ld_extra=4), oracle.gemm.gemm_nt(qa, sa, qb, sb), f"ragged k {m}x{n}x{k}")


def test_ragged_k_grouped():
    """Contiguous and masked layouts with a partial last K group."""
    say("gemm ragged k grouped")
    masked_case("masked_ragged_k", 3, 128, 256, 400, [128, 5, 70])
    rng = inputs.rng_for("contig_ragged_k")
    n, k = 256, 272
    sizes = np.array([129, 40], dtype=np.int64)
    a, m_idx, valid = inputs.contiguous_activations(rng, sizes, k)
    b = inputs.grouped_weights(rng, 2, n, k)
    qa, sa = oracle.quant.quantize_per_token_group(a)
    qb, sb = oracle.quant.quantize_per_block_grouped(b)
    d = dg.dg_gemm_fp8_grouped_contiguous(to_dev(qa), sa_to_dev(sa), to_dev(qb), to_dev(sb), to_dev(m_idx))
    torch.cuda.synchronize()
    check_gemm(d, oracle.gemm.gemm_grouped_contiguous(qa, sa, qb, sb, m_idx), "contiguous ragged k")


def test_ragged_k_from_gpu_quantizers():
    """End to end on a partial last K group: the GPU quantizers' bytes equal the oracle's, and the
    GEMM of them matches the oracle GEMM."""
    say("gemm ragged k end to end")
    m, n, k = 96, 384, 656
    rng = inputs.rng_for("ragged_k_e2e")
    a = inputs.activations_with_outliers(rng, m, k)
    b = inputs.normal(rng, (n, k), 0.02)
    qa_d, sa_d = dg.dg_quantize_per_token_group(to_dev(a))
    qb_d, sb_d = dg.dg_quantize_per_block(to_dev(b))
    d = dg.dg_gemm_fp8_nt(qa_d, sa_d, qb_d, sb_d)
    torch.cuda.synchronize()
    qa, sa = oracle.quant.quantize_per_token_group(a)
    qb, sb = oracle.quant.quantize_per_block(b)
    assert np.array_equal(qa_d.cpu().numpy(), qa) and np.array_equal(qb_d.cpu().numpy(), qb)
    assert np.array_equal(sa_d.cpu().numpy()[:, :m].T.view(np.uint32), sa.view(np.uint32))
    assert np.array_equal(sb_d.cpu().numpy().view(np.uint32), sb.view(np.uint32))
    check_gemm(d, oracle.gemm.gemm_nt(qa, sa, qb, sb), "ragged k end to end")


# ---- CU cap (dg_set_num_cus): the persistent grid leaves CUs free for other kernels -------------

@pytest.mark.parametrize("cap", [1, 7, 64, 200])
def test_cu_cap(cap):
    """Every form stays correct with the grid capped to `cap` CUs (plans and K splits change
    with the cap); a capped call whose plan equals the uncapped one is bit-identical to it."""
    say("gemm cu cap", cap)
    full = dg.dg_get_num_cus()
    # (520, 1003, 1024): large tiles with the direct-store epilogue (N % 8 != 0), several per
    # workgroup under the small caps
    cases = [(64, 512, 4096), (300, 1000, 1024), (128, 256, 2048), (520, 1003, 1024)]
    try:
        for (m, n, k) in cases:
            qa, sa, qb, sb = quantized_operands("cucap", m, n, k)
            name_full = dg.dg_gemm_config_name(0, m, n, k)
            d_full = run_dense(qa, sa, qb, sb)
            dg.dg_set_num_cus(cap)
            assert dg.dg_get_num_cus() == min(cap, full)
            name_cap = dg.dg_gemm_config_name(0, m, n, k)
            d_cap = run_dense(qa, sa, qb, sb)
            dg.dg_set_num_cus(full)
            check_gemm(d_cap, oracle.gemm.gemm_nt(qa, sa, qb, sb), f"cap {cap} {m}x{n}x{k} ({name_cap})")
            if name_cap == name_full:
                assert np.array_equal(bf16_bits(d_cap), bf16_bits(d_full))
        dg.dg_set_num_cus(cap)
        masked_case("masked_cap", 4, 64, 256, 2048, [64, 7, 0, 33])
        test_contiguous_small()
    finally:
        dg.dg_set_num_cus(full)


# ---- the 256x192 and 256x256 tiles (two-slot pipelined main loop): K block counts 1, 2, odd,
# partial; edges -------------------------------------------------------------------------------

def _cap_for(prefix, layout, m, n, k, groups=1):
    """The largest CU cap under which the planner gives this shape a configuration starting with
    `prefix` (the cap changes how many rounds each tile size needs), or None."""
    full = dg.dg_get_num_cus()
    try:
        for cap in range(full, 0, -1):
            dg.dg_set_num_cus(cap)
            if dg.dg_gemm_config_name(layout, m, n, k, groups).startswith(prefix):
                return cap
    finally:
        dg.dg_set_num_cus(full)
    return None


_WIDE_SHAPES = [(300, 500, 16), (300, 500, 128), (300, 500, 256), (300, 500, 384), (300, 500, 400),
                (520, 1000, 1280), (257, 193, 2064), (777, 2000, 3200)]
_SQUARE_SHAPES = [(500, 500, 16), (500, 500, 128), (500, 500, 256), (500, 500, 384), (500, 500, 400),
                  (512, 1000, 1280), (450, 300, 2064), (1000, 2000, 3200)]


@pytest.mark.parametrize("tile,m,n,k", [("256x192",) + s for s in _WIDE_SHAPES] +
                                       [("256x256",) + s for s in _SQUARE_SHAPES])
def test_wide_tile_k_blocks_and_edges(tile, m, n, k):
    """The 256x192 and 256x256 tiles on shapes the planner gives them under a CU cap: one K block
    (whole and partial), two, an odd count, a partial last group, and M / N edges inside a tile."""
    cap = _cap_for(tile, 0, m, n, k)
    assert cap is not None, (tile, m, n, k)
    full = dg.dg_get_num_cus()
    qa, sa, qb, sb = quantized_operands("wide", m, n, k)
    try:
        dg.dg_set_num_cus(cap)
        name = dg.dg_gemm_config_name(0, m, n, k)
        say("gemm wide tile", m, n, k, "cap", cap, name)
        d1 = run_dense(qa, sa, qb, sb, ld_extra=4)
        d2 = run_dense(qa, sa, qb, sb, ld_extra=4)
    finally:
        dg.dg_set_num_cus(full)
    assert name.startswith(tile), name
    assert np.array_equal(bf16_bits(d1), bf16_bits(d2))
    check_gemm(d1, oracle.gemm.gemm_nt(qa, sa, qb, sb), f"wide {m}x{n}x{k} ({name})")


@pytest.mark.parametrize("tile,m_max", [("256x192", 384), ("256x256", 512)])
def test_wide_tile_masked(tile, m_max):
    """The masked layout on the 256x192 and 256x256 tiles (groups partly or wholly empty)."""
    g, n, k = 3, 500, 1024
    cap = _cap_for(tile, 2, m_max, n, k, g)
    assert cap is not None, tile
    full = dg.dg_get_num_cus()
    try:
        dg.dg_set_num_cus(cap)
        say("gemm wide tile masked", g, m_max, n, k, "cap", cap, dg.dg_gemm_config_name(2, m_max, n, k, g))
        masked_case("masked_wide", g, m_max, n, k, [m_max, 200, 0])
    finally:
        dg.dg_set_num_cus(full)


def test_plan_override_results():
    """Plans forced with DG_PLAN (the planner's alternatives) give results within the GEMM
    tolerance of the oracle: a few-row tile and split the planner did not pick, and a large tile."""
    import os
    cases = [((64, 2112, 1024), "tile=64x128,splits=3"), ((300, 1000, 1024), "tile=256x256,splits=2")]
    for (m, n, k), plan in cases:
        qa, sa, qb, sb = quantized_operands("override", m, n, k)
        old = os.environ.get("DG_PLAN")
        os.environ["DG_PLAN"] = plan
        try:
            name = dg.dg_gemm_config_name(0, m, n, k)
            say("gemm forced plan", m, n, k, plan, name)
            d = run_dense(qa, sa, qb, sb)
        finally:
            if old is None:
                os.environ.pop("DG_PLAN", None)
            else:
                os.environ["DG_PLAN"] = old
        assert name.split("/")[0] == plan.split(",")[0][len("tile="):], name
        check_gemm(d, oracle.gemm.gemm_nt(qa, sa, qb, sb), f"forced {plan} {m}x{n}x{k}")


# 128-row expert blocks of the two-pass contiguous cases: 256-row tiles (0,0) whole, (0,1), (-1,2),
# (2,3) and (2,-1) split between two experts or an expert and an unmapped block, (-1,-1) unmapped,
# and a last tile of one block.
_TWO_PASS_BLOCKS = [0, 0, 0, 1, -1, 2, 2, 3, 2, -1, -1, -1, 3]


@pytest.mark.parametrize("n,k,cap", [(500, 1040, None), (512, 1040, None), (384, 128, None), (500, 1040, 3),
                                     (512, 1040, 2)])
def test_contiguous_square_tiles(n, k, cap):
    """The contiguous form on 256x256 tiles (forced with DG_PLAN): tiles whose 128-row halves name
    two experts run once per half and store only that half; unmapped halves and tiles are left
    untouched; a tile of one block ends the rows.  N edges on both epilogue paths (N % 8 != 0 and
    == 0), a partial last K group; with a CU cap, one workgroup runs several tiles and passes in
    a row.  The same rows agree with the 256x128 plan bit for bit."""
    import os
    g = 4
    m_idx = np.repeat(np.array(_TWO_PASS_BLOCKS, np.int32), 128)
    m_total = m_idx.shape[0]
    rng = inputs.rng_for("contig_square", n, k)
    a = inputs.activations_with_outliers(rng, m_total, k)
    b = inputs.grouped_weights(rng, g, n, k)
    qa, sa = oracle.quant.quantize_per_token_group(a)
    qb, sb = oracle.quant.quantize_per_block_grouped(b)
    ref = oracle.gemm.gemm_grouped_contiguous(qa, sa, qb, sb, np.where(m_idx < 0, 0, m_idx))
    mapped = m_idx >= 0
    outs = {}
    old = os.environ.get("DG_PLAN")
    full = dg.dg_get_num_cus()
    try:
        if cap is not None:
            dg.dg_set_num_cus(cap)
        for tile in ("256x256", "256x128"):
            os.environ["DG_PLAN"] = "tile=" + tile
            name = dg.dg_gemm_config_name(1, m_total, n, k, g)
            say("gemm contiguous two-pass", m_total, n, k, name, "cap", cap)
            assert name.startswith(tile + "/"), name
            d = torch.full((m_total, n), -1, dtype=torch.int16, device=device()).view(torch.bfloat16)
            dg.dg_gemm_fp8_grouped_contiguous(to_dev(qa), sa_to_dev(sa), to_dev(qb), to_dev(sb), to_dev(m_idx), d=d)
            torch.cuda.synchronize()
            outs[tile] = d
    finally:
        dg.dg_set_num_cus(full)
        if old is None:
            os.environ.pop("DG_PLAN", None)
        else:
            os.environ["DG_PLAN"] = old
    d = outs["256x256"]
    bits = bf16_bits(d)
    assert np.all(bits[~mapped] == BF16_NAN), "rows of unmapped blocks were written"
    check_gemm(d[torch.from_numpy(mapped).to(device())], ref[mapped], f"contiguous 256x256 n={n} k={k}")
    assert np.array_equal(bits, bf16_bits(outs["256x128"]))


def test_contiguous_square_planner_choice():
    """Large experts: the planner itself gives the contiguous form 256x256 tiles (under a CU cap
    that makes them save rounds), one expert boundary inside a tile."""
    g, n, k = 2, 1024, 256
    m_idx = np.repeat(np.array([0] * 33 + [1] * 31, np.int32), 128)
    m_total = m_idx.shape[0]
    cap = _cap_for("256x256", 1, m_total, n, k, g)
    assert cap is not None
    rng = inputs.rng_for("contig_square_plan", n, k)
    a = inputs.activations_with_outliers(rng, m_total, k)
    b = inputs.grouped_weights(rng, g, n, k)
    qa, sa = oracle.quant.quantize_per_token_group(a)
    qb, sb = oracle.quant.quantize_per_block_grouped(b)
    full = dg.dg_get_num_cus()
    try:
        dg.dg_set_num_cus(cap)
        name = dg.dg_gemm_config_name(1, m_total, n, k, g)
        say("gemm contiguous planner 256x256", m_total, n, k, "cap", cap, name)
        d = dg.dg_gemm_fp8_grouped_contiguous(to_dev(qa), sa_to_dev(sa), to_dev(qb), to_dev(sb), to_dev(m_idx))
        torch.cuda.synchronize()
    finally:
        dg.dg_set_num_cus(full)
    assert name.startswith("256x256/"), name
    check_gemm(d, oracle.gemm.gemm_grouped_contiguous(qa, sa, qb, sb, m_idx), "contiguous planner 256x256")
