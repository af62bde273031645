"""Normal GEMM with the per-token-group activation quantization inside the GEMM launch
(dg_gemm_fp8_nt_act_quant / _bf16) against the fp64 CPU oracle, and against the two launches it
replaces.

The oracle side quantizes x with the oracle quantizer and multiplies with the oracle GEMM
(acceptance as for every GEMM: |gpu - ref| <= 8e-3 |ref| + 1e-3 rms(ref), relative Frobenius
<= 2e-3).  Against dg_quantize_per_token_group + dg_gemm_fp8_nt the result must be bit-identical:
the same bytes and scales feed the same tile plan.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_gemm_amd as dg
from fp8_block_scaled_gemm_amd import inputs
import oracle
from gpu_util import (bf16_bits, check_gemm, cu_masked_stream, device, oracle_quant_blocks, oracle_quant_rows,
                      say, to_dev)

pytestmark = pytest.mark.gpu

DG_ERR_WORKSPACE = -3


def operands(name, m, n, k, bf16=False):
    """x (numpy fp32; bf16-representable when bf16), its device tensor, and the block-quantized
    weights (oracle bytes and scales, on the device and on the host)."""
    rng = inputs.rng_for(name, m, n, k)
    x = inputs.activations_with_outliers(rng, m, k) if m >= 2 else inputs.normal(rng, (m, k))
    if bf16:
        bits = inputs.to_bf16_bits(x)
        x = oracle.bf16.decode(bits).astype(np.float32)
        xd = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device()).view(torch.bfloat16)
    else:
        xd = to_dev(x)
    w = inputs.normal(rng, (n, k), 0.02)
    qb, sb = oracle_quant_blocks(w) if n * k >= 1 << 24 else oracle.quant.quantize_per_block(w)
    return x, xd, qb, sb


def oracle_ref(x, qb, sb):
    qa, sa = oracle_quant_rows(x) if x.shape[0] >= 512 else oracle.quant.quantize_per_token_group(x)
    return oracle.gemm.gemm_nt(qa, sa, qb, sb)


def two_step(xd, b, sb):
    """The two launches the fused entry point replaces (with a workspace, so the same plan)."""
    q, sa = dg.dg_quantize_per_token_group(xd)
    return dg.dg_gemm_fp8_nt(q, sa, b, sb)


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (77, 200, 384), (64, 2112, 1024), (128, 640, 4096),
                                   (130, 260, 400), (257, 1000, 640), (33, 4096, 768), (1024, 2048, 1024)])
def test_matches_oracle(m, n, k, bf16):
    """Ragged M, N and K (K = 400: a partial last K group), decode-sized M with split K, and a
    large-tile shape; fp32 and bf16 activations."""
    say("act-quant gemm vs oracle", m, n, k, "bf16" if bf16 else "fp32", dg.dg_gemm_config_name(0, m, n, k))
    x, xd, qb, sb = operands("actq", m, n, k, bf16)
    b, sbd = to_dev(qb), to_dev(sb)
    d = dg.dg_gemm_fp8_nt_act_quant(xd, b, sbd)
    torch.cuda.synchronize()
    check_gemm(d, oracle_ref(x, qb, sb), f"act-quant {m}x{n}x{k}")
    assert np.array_equal(bf16_bits(d), bf16_bits(two_step(xd, b, sbd)))


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("m,n,k", [(64, 2112, 7168), (64, 24576, 1536), (128, 7168, 16384), (128, 4096, 7168),
                                   (4096, 7168, 2048), (4608, 4096, 6144)])
def test_full_size_bit_identical_to_two_steps(m, n, k, bf16):
    """DeepSeek-V3 decode and prefill shapes (and a split-last-round shape): bit-identical to
    quantize + GEMM, with sampled outputs against the oracle (rows and columns at random, the
    edges included)."""
    say("act-quant gemm full size", m, n, k, "bf16" if bf16 else "fp32", dg.dg_gemm_config_name(0, m, n, k))
    x, xd, qb, sb = operands("actq_full", m, n, k, bf16)
    b, sbd = to_dev(qb), to_dev(sb)
    d = dg.dg_gemm_fp8_nt_act_quant(xd, b, sbd)
    ref2 = two_step(xd, b, sbd)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(d), bf16_bits(ref2))
    rng = np.random.default_rng(m * 7 + n)
    rows = np.unique(np.concatenate([[0, m - 1], rng.integers(0, m, 6)]))
    cols = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 24)]))
    qa, sa = oracle.quant.quantize_per_token_group(x[rows])
    # sampled weight rows, each with the scales of its 128-row block
    ref = oracle.gemm.dequantize_rows(qa, sa) @ oracle.gemm.dequantize_rows(qb[cols], np.asarray(sb)[cols // 128]).T
    check_gemm(d.cpu()[rows][:, cols], ref, f"act-quant sampled {m}x{n}x{k}")


def test_work_queue_with_a_small_grid():
    """With the GEMM capped to 2 CUs the grid has a few workgroups and the quantization step has
    hundreds of chunks: each workgroup takes many chunks in turn.  Bit-identical to the two
    launches under the same cap, and within tolerance of the oracle."""
    m, n, k = 512, 384, 2048
    x, xd, qb, sb = operands("actq_queue", m, n, k)
    b, sbd = to_dev(qb), to_dev(sb)
    old = dg.dg_get_num_cus()
    dg.dg_set_num_cus(2)
    try:
        say("act-quant gemm, 2 CUs", m, n, k, dg.dg_gemm_config_name(0, m, n, k))
        d = dg.dg_gemm_fp8_nt_act_quant(xd, b, sbd)
        ref2 = two_step(xd, b, sbd)
        torch.cuda.synchronize()
    finally:
        dg.dg_set_num_cus(old)
    assert np.array_equal(bf16_bits(d), bf16_bits(ref2))
    check_gemm(d, oracle_ref(x, qb, sb), "act-quant 2 CUs")


@pytest.mark.parametrize("m,n,k", [(64, 4096, 7168), (512, 2048, 7168)])
def test_full_grid_on_a_cu_masked_stream(m, n, k):
    """The grid is planned for every CU, but the stream may only use 16 of them: most workgroups
    start only after others have finished.  Chunks are taken only by running workgroups, so the
    wait still ends; the result is the two launches' and the counters are left zero."""
    x, xd, qb, sb = operands("actq_cumask", m, n, k)
    b, sbd = to_dev(qb), to_dev(sb)
    ws = torch.zeros(dg.dg_gemm_fp8_nt_act_quant_workspace_size(m, n, k), dtype=torch.uint8, device=device())
    say("act-quant gemm on 16 CUs", m, n, k, dg.dg_gemm_config_name(0, m, n, k))
    torch.cuda.synchronize()
    s = cu_masked_stream(0, 16)
    with torch.cuda.stream(s):
        d = dg.dg_gemm_fp8_nt_act_quant(xd, b, sbd, workspace=ws)
    s.synchronize()
    ref2 = two_step(xd, b, sbd)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(d), bf16_bits(ref2))
    assert int(ws[:64 << 10].count_nonzero()) == 0


def test_shared_workspace_sequence_leaves_counters_zero():
    """Calls of different shapes, dtypes and plans one after another on one workspace, mixed with
    the normal GEMM on the same workspace: every result is bit-identical to the two launches and
    the counter prefix is zero after each call."""
    ws = torch.zeros(96 << 20, dtype=torch.uint8, device=device())
    shapes = [(64, 512, 4096, False), (300, 1000, 640, True), (64, 4608, 7168, False), (1, 16, 128, True),
              (2048, 1024, 1024, False), (64, 512, 4096, True)]
    for (m, n, k, bf16) in shapes:
        need = dg.dg_gemm_fp8_nt_act_quant_workspace_size(m, n, k)
        say("act-quant gemm sequence", m, n, k, need, dg.dg_gemm_config_name(0, m, n, k))
        assert 0 < need <= ws.numel()
        x, xd, qb, sb = operands("actq_seq", m, n, k, bf16)
        b, sbd = to_dev(qb), to_dev(sb)
        d = dg.dg_gemm_fp8_nt_act_quant(xd, b, sbd, workspace=ws)
        q, sa = dg.dg_quantize_per_token_group(xd)
        ref2 = dg.dg_gemm_fp8_nt(q, sa, b, sbd, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(d), bf16_bits(ref2)), (m, n, k)
        assert int(ws[:64 << 10].count_nonzero()) == 0, "counters not left at zero"


def test_workspace_errors_and_empty():
    """A workspace smaller than required is an error raised before any launch; empty shapes are
    no-ops."""
    say("act-quant gemm workspace errors")
    m, n, k = 64, 256, 512
    x, xd, qb, sb = operands("actq_err", m, n, k)
    b, sbd = to_dev(qb), to_dev(sb)
    need = dg.dg_gemm_fp8_nt_act_quant_workspace_size(m, n, k)
    assert need >= (64 << 10) + m * k + (k // 128) * dg.dg_get_scale_ld(m) * 4
    small = torch.zeros(need - 16, dtype=torch.uint8, device=device())
    with pytest.raises(dg.DGError) as e:
        dg.dg_gemm_fp8_nt_act_quant(xd, b, sbd, workspace=small)
    assert e.value.status == DG_ERR_WORKSPACE
    d = torch.empty((0, n), dtype=torch.bfloat16, device=device())
    dg.dg_gemm_fp8_nt_act_quant(torch.empty((0, k), device=device()), b, sbd, d=d)
    torch.cuda.synchronize()


def test_zero_and_extreme_rows():
    """Rows of zeros (scale 1), a row of huge values, and a row of tiny values: the fused
    quantization gives the two launches' result bit for bit."""
    say("act-quant gemm special rows")
    m, n, k = 8, 256, 512
    rng = inputs.rng_for("actq_special")
    x = inputs.normal(rng, (m, k))
    x[1] = 0.0
    x[2, :] = np.float32(1.0e36) * np.sign(x[2])
    x[3] *= np.float32(1e-30)
    x[4, 128:256] = 0.0
    w = inputs.normal(rng, (n, k), 0.02)
    qb, sb = oracle.quant.quantize_per_block(w)
    xd, b, sbd = to_dev(x), to_dev(qb), to_dev(sb)
    d = dg.dg_gemm_fp8_nt_act_quant(xd, b, sbd)
    ref2 = two_step(xd, b, sbd)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(d), bf16_bits(ref2))
    qa, sa = oracle.quant.quantize_per_token_group(x)
    ref = oracle.gemm.gemm_nt(qa, sa, qb, sb)
    finite = np.all(np.isfinite(ref), axis=1)
    check_gemm(d.cpu()[torch.from_numpy(finite)], ref[finite], "special rows")
