"""GPU training-side layouts against the CPU oracle: the per-channel-group quantizer and the block
transpose bit-exact, the row-scaled GEMM and a linear layer's forward / dgrad / wgrad within the
GEMM acceptance (|gpu - ref| <= 8e-3 |ref| + 1e-3 rms(ref), relative Frobenius <= 2e-3)."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_gemm_amd as dg
from fp8_block_scaled_gemm_amd import inputs
import oracle
from gpu_util import bits32, check_gemm, device, sa_to_dev, say, to_dev

pytestmark = pytest.mark.gpu


def run_channel_group(x_dev, ld_extra=0):
    """GPU per-channel quantization of x_dev (M, K) -> (qt (K, M) numpy, st (K, MB) numpy)."""
    m, k = x_dev.shape[-2:]
    ld = dg.dg_get_scale_ld(k) + ld_extra
    st = torch.full(x_dev.shape[:-2] + (max(-(-m // 128), 1), ld), float("nan"), dtype=torch.float32,
                    device=device())
    qt, st = dg.dg_quantize_per_channel_group(x_dev, st=st)
    torch.cuda.synchronize()
    st_np = st.cpu().numpy()
    if ld > k:   # entries past the columns stay untouched
        assert np.all(np.isnan(st_np[..., k:]))
    return qt.cpu().numpy(), np.swapaxes(st_np[..., :k], -1, -2).copy()


def assert_channel_exact(x, qt, st):
    qo, so = oracle.train.quantize_per_channel_group(x)
    assert np.array_equal(bits32(st), bits32(so)), np.argwhere(bits32(st) != bits32(so))[:5]
    bad = np.argwhere(qt != qo)
    assert bad.size == 0, [(tuple(i), hex(qt[tuple(i)]), hex(qo[tuple(i)])) for i in bad[:5]]


@pytest.mark.parametrize("m,k,ld_extra", [(128, 64, 0), (16, 4, 0), (256, 200, 4), (272, 1000, 0),
                                          (4096, 512, 8), (144, 7168, 0)])
def test_channel_group_bit_exact(m, k, ld_extra):
    say("quant channel group", m, k)
    rng = inputs.rng_for("quant_ch", m, k)
    # columns of very different magnitudes, a few outlier tokens, one all-zero column
    x = inputs.activations_with_outliers(rng, m, k) * np.exp2(rng.uniform(-8, 8, size=(1, k))).astype(np.float32)
    x[:, k // 2] = 0.0
    qt, st = run_channel_group(to_dev(x), ld_extra)
    assert_channel_exact(x, qt, st)


@pytest.mark.parametrize("m,k", [(128, 64), (272, 1000), (2048, 2112)])
def test_channel_group_bf16_bit_exact(m, k):
    say("quant channel group bf16", m, k)
    rng = inputs.rng_for("quant_ch_bf16", m, k)
    xt = torch.from_numpy(inputs.activations_with_outliers(rng, m, k)).to(torch.bfloat16)
    qt, st = run_channel_group(xt.to(device()))
    bits = xt.view(torch.int16).numpy().view(np.uint16)
    qo, so = oracle.train.quantize_per_channel_group_bf16(bits)
    assert np.array_equal(qt, qo) and np.array_equal(bits32(st), bits32(so))


def test_channel_group_batched():
    say("quant channel group batched 3x144x96")
    rng = inputs.rng_for("quant_ch_batched")
    x = inputs.normal(rng, (3, 144, 96))
    qt, st = run_channel_group(to_dev(x))
    for g in range(3):
        assert_channel_exact(x[g], qt[g], st[g])


@pytest.mark.parametrize("shape", [(256, 384), (272, 144), (2, 128, 256), (7168, 2048), (16, 16)])
def test_transpose_blocks_bit_exact(shape):
    say("transpose blocks", shape)
    rng = inputs.rng_for("transpose", *shape)
    w = inputs.normal(rng, shape, 0.02)
    q, s = dg.dg_quantize_per_block(to_dev(w))
    qt, st = dg.dg_transpose_blocks(q, s)
    torch.cuda.synchronize()
    ws = w.reshape((-1,) + shape[-2:])
    for g in range(ws.shape[0]):
        qo, so = oracle.train.transpose_blocks(*oracle.quant.quantize_per_block(ws[g]))
        qg = qt.cpu().numpy().reshape((-1,) + qo.shape)[g]
        sg = st.cpu().numpy().reshape((-1,) + so.shape)[g]
        assert np.array_equal(qg, qo) and np.array_equal(bits32(sg), bits32(so))


def row_scaled_operands(name, m, n, k):
    rng = inputs.rng_for(name, m, n, k)
    codes = oracle.e4m3.all_finite_codes()
    kb = -(-k // 128)
    qa = rng.choice(codes, size=(m, k)).astype(np.uint8)
    qb = rng.choice(codes, size=(n, k)).astype(np.uint8)
    sa = np.exp2(rng.uniform(-10, -4, size=(m, kb))).astype(np.float32)
    sb = np.exp2(rng.uniform(-10, -4, size=(n, kb))).astype(np.float32)
    return qa, sa, qb, sb


def run_row_scaled(qa, sa, qb, sb, ld_extra=0, workspace=True):
    m, n = qa.shape[0], qb.shape[0]
    d = dg.dg_gemm_fp8_nt_row_scaled(to_dev(qa), sa_to_dev(sa, dg.dg_get_scale_ld(m) + ld_extra), to_dev(qb),
                                     sa_to_dev(sb, dg.dg_get_scale_ld(n) + ld_extra), use_workspace=workspace)
    torch.cuda.synchronize()
    return d


@pytest.mark.parametrize("m,n,k", [(256, 256, 256), (200, 130, 384), (4096, 512, 1024), (64, 7168, 2048),
                                   (128, 4096, 7168), (300, 520, 272), (1, 16, 128), (1000, 2000, 1536)])
def test_row_scaled_gemm(m, n, k):
    say("row-scaled gemm", m, n, k, dg.dg_gemm_config_name(3, m, n, k))
    qa, sa, qb, sb = row_scaled_operands("rowscaled", m, n, k)
    ref = oracle.train.gemm_nt_row_scaled(qa, sa, qb, sb)
    check_gemm(run_row_scaled(qa, sa, qb, sb, ld_extra=4), ref, f"row-scaled {m}x{n}x{k}")


def test_row_scaled_split_last_round():
    """The row-scaled kernel with a split last round: 16 x 20 = 320 tiles of 256x128 on 256 CUs, the
    64 last-round tiles split in K (48 K blocks, two pieces).  Against the oracle, bit-identical on
    a repeat, and the unsplit path agrees within tolerance."""
    m, n, k = 2048, 5120, 6144
    name = dg.dg_gemm_config_name(3, m, n, k)
    say("row-scaled split last round", m, n, k, name)
    if dg.dg_get_num_cus() == 256:
        assert "+tail" in name, name
    qa, sa, qb, sb = row_scaled_operands("rowscaled_tail", m, n, k)
    ref = oracle.train.gemm_nt_row_scaled(qa, sa, qb, sb)
    d1, d2 = run_row_scaled(qa, sa, qb, sb), run_row_scaled(qa, sa, qb, sb)
    assert torch.equal(d1.view(torch.int16), d2.view(torch.int16))
    check_gemm(d1, ref, "row-scaled split last round")
    check_gemm(run_row_scaled(qa, sa, qb, sb, workspace=False), ref, "row-scaled unsplit")


def test_row_scaled_split_k_deterministic():
    """A split-K plan (few rows, long K): repeated calls bit-identical; the unsplit path agrees."""
    m, n, k = 64, 1024, 8192
    say("row-scaled split-k", m, n, k, dg.dg_gemm_config_name(3, m, n, k))
    qa, sa, qb, sb = row_scaled_operands("rowscaled_split", m, n, k)
    ref = oracle.train.gemm_nt_row_scaled(qa, sa, qb, sb)
    d1, d2 = run_row_scaled(qa, sa, qb, sb), run_row_scaled(qa, sa, qb, sb)
    assert torch.equal(d1.view(torch.int16), d2.view(torch.int16))
    check_gemm(d1, ref, "row-scaled split")
    check_gemm(run_row_scaled(qa, sa, qb, sb, workspace=False), ref, "row-scaled unsplit")


def test_row_scaled_equals_block_scaled_for_blockwise_rows():
    """Row scales constant over each 128-row block of B: the row-scaled kernel and the block-scaled
    kernel compute the same products (bit-identical when both take the same tile plan)."""
    m, n, k = 4096, 1024, 1024
    say("row-scaled vs block-scaled", m, n, k, dg.dg_gemm_config_name(0, m, n, k), dg.dg_gemm_config_name(3, m, n, k))
    qa, sa, qb, _ = row_scaled_operands("rowscaled_block", m, n, k)
    sb_blocks = np.exp2(np.random.default_rng(5).uniform(-10, -4, size=(n // 128, k // 128))).astype(np.float32)
    sb_rows = np.repeat(sb_blocks, 128, axis=0)
    d_row = run_row_scaled(qa, sa, qb, sb_rows)
    d_blk = dg.dg_gemm_fp8_nt(to_dev(qa), sa_to_dev(sa), to_dev(qb), to_dev(sb_blocks))
    torch.cuda.synchronize()
    ref = oracle.gemm.gemm_nt(qa, sa, qb, sb_blocks)
    check_gemm(d_row, ref, "row-scaled")
    check_gemm(d_blk, ref, "block-scaled")
    if dg.dg_gemm_config_name(0, m, n, k) == dg.dg_gemm_config_name(3, m, n, k):
        assert torch.equal(d_row.view(torch.int16), d_blk.view(torch.int16))


@pytest.mark.parametrize("m,n,k", [(512, 384, 256), (272, 256, 400), (2048, 1024, 768)])
def test_linear_layer_forward_dgrad_wgrad(m, n, k):
    """Y = X W^T, dX = dY W, dW = dY^T X through the library only (quantizers, transpose, GEMMs)
    against the oracle's compositions on the same fp32 inputs."""
    say("linear layer", m, n, k)
    rng = inputs.rng_for("linear", m, n, k)
    x = inputs.activations_with_outliers(rng, m, k)
    w = inputs.normal(rng, (n, k), 0.02)
    dy = inputs.normal(rng, (m, n), 1e-2)
    xd, wd, dyd = to_dev(x), to_dev(w), to_dev(dy)
    # forward
    qx, sx = dg.dg_quantize_per_token_group(xd)
    qw, sw = dg.dg_quantize_per_block(wd)
    y = dg.dg_gemm_fp8_nt(qx, sx, qw, sw)
    # dgrad: dY per-token groups along N, W^T from W's blocks
    qdy, sdy = dg.dg_quantize_per_token_group(dyd)
    qwt, swt = dg.dg_transpose_blocks(qw, sw)
    dx = dg.dg_gemm_fp8_nt(qdy, sdy, qwt, swt)
    # wgrad: both operands in per-channel groups of 128 tokens
    qdyt, sdyt = dg.dg_quantize_per_channel_group(dyd)
    qxt, sxt = dg.dg_quantize_per_channel_group(xd)
    dw = dg.dg_gemm_fp8_nt_row_scaled(qdyt, sdyt, qxt, sxt)
    torch.cuda.synchronize()
    check_gemm(y, oracle.train.linear_forward(x, w), "forward")
    check_gemm(dx, oracle.train.linear_dgrad(dy, w), "dgrad")
    check_gemm(dw, oracle.train.linear_wgrad(dy, x), "wgrad")


def test_wgrad_full_size_sampled_rows():
    """dW = dY^T X for 4096 tokens, N = 7168, K = 2048 (a DeepSeek-V3 projection), sampled rows of dW:
    the GPU's quantized bytes and scales of the sampled rows and of X^T are checked bit-exact first,
    then the GEMM rows against the oracle on those operands."""
    m, n, k = 4096, 7168, 2048
    say("wgrad full size", m, n, k, dg.dg_gemm_config_name(3, n, k, m))
    dev = device()
    gen = inputs.DeviceGen(torch, dev, 9100)
    x = gen.activations(m, k)
    dy = gen.normal((m, n), 1e-2)
    qdyt, sdyt = dg.dg_quantize_per_channel_group(dy)
    qxt, sxt = dg.dg_quantize_per_channel_group(x)
    dw = dg.dg_gemm_fp8_nt_row_scaled(qdyt, sdyt, qxt, sxt)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 1, 127, 128, 255, 256, n - 2, n - 1} |
                           set(np.random.default_rng(3).choice(n, size=12, replace=False).tolist())))
    ridx = torch.as_tensor(rows, device=dev)
    # oracle operands of the sampled dW rows (columns of dY) and of X^T, checked against the GPU's
    qa_o, sa_o = oracle.train.quantize_per_channel_group(dy[:, ridx].cpu().numpy())
    qb_o, sb_o = oracle.train.quantize_per_channel_group(x.cpu().numpy())
    assert np.array_equal(qdyt[ridx].cpu().numpy(), qa_o)
    assert np.array_equal(bits32(sdyt[:, ridx].T.contiguous().cpu().numpy()), bits32(sa_o))
    assert np.array_equal(qxt.cpu().numpy(), qb_o)
    assert np.array_equal(bits32(sxt[:, :k].T.contiguous().cpu().numpy()), bits32(sb_o))
    check_gemm(dw[ridx], oracle.train.gemm_nt_row_scaled(qa_o, sa_o, qb_o, sb_o), "wgrad sampled rows")


@pytest.mark.parametrize("tokens,n,k", [([256, 0, 128, 640], 256, 384), ([512] * 3 + [384, 640, 128, 0, 768], 512, 1024),
                                        ([128], 136, 200)])
def test_moe_wgrad_k_grouped(tokens, n, k):
    """dW_e = dY_e^T X_e per expert over the contiguous layout through the library (per-channel
    quantization of the whole dY and X, then the k-grouped row-scaled GEMM) against the oracle; an
    expert with no tokens gets zeros (the output is pre-filled with NaN)."""
    t = sum(tokens)
    say("moe wgrad k-grouped", tokens, n, k)
    rng = inputs.rng_for("moe_wgrad", t, n, k)
    x = inputs.activations_with_outliers(rng, t, k)
    dy = inputs.normal(rng, (t, n), 1e-2)
    qdyt, sdyt = dg.dg_quantize_per_channel_group(to_dev(dy))
    qxt, sxt = dg.dg_quantize_per_channel_group(to_dev(x))
    d = torch.full((len(tokens), n, k), float("nan"), dtype=torch.bfloat16, device=device())
    dg.dg_gemm_fp8_k_grouped_row_scaled(qdyt, sdyt, qxt, sxt, tokens, d=d)
    torch.cuda.synchronize()
    ref = oracle.train.linear_wgrad_k_grouped(dy, x, tokens)
    for e, te in enumerate(tokens):
        if te == 0:
            assert bool(torch.all(d[e] == 0)), f"empty expert {e} not zeroed"
        else:
            check_gemm(d[e], ref[e], f"expert {e} ({te} tokens)")


def test_moe_dgrad_contiguous():
    """dX = dY W_e per token over the contiguous layout: the contiguous-grouped GEMM on the experts'
    transposed weight blocks (dg_transpose_blocks of the (G, N, K) block quantization)."""
    g, n, k = 4, 384, 256
    sizes = [200, 0, 77, 300]
    m_idx, starts, valid = inputs.contiguous_layout(sizes)
    m_total = m_idx.shape[0]
    say("moe dgrad contiguous", sizes, n, k)
    rng = inputs.rng_for("moe_dgrad", n, k)
    w = inputs.normal(rng, (g, n, k), 0.02)
    dy = inputs.normal(rng, (m_total, n), 1e-2) * valid[:, None].astype(np.float32)
    qw, sw = dg.dg_quantize_per_block(to_dev(w))
    qwt, swt = dg.dg_transpose_blocks(qw, sw)
    qdy, sdy = dg.dg_quantize_per_token_group(to_dev(dy))
    dx = dg.dg_gemm_fp8_grouped_contiguous(qdy, sdy, qwt, swt, torch.from_numpy(m_idx).to(device()))
    torch.cuda.synchronize()
    qa, sa = oracle.quant.quantize_per_token_group(dy)
    tq = [oracle.train.transpose_blocks(*oracle.quant.quantize_per_block(w[e])) for e in range(g)]
    ref = oracle.gemm.gemm_grouped_contiguous(qa, sa, np.stack([q for q, _ in tq]), np.stack([s for _, s in tq]), m_idx)
    rows = np.nonzero(m_idx >= 0)[0]
    check_gemm(dx[torch.as_tensor(rows, device=device())], ref[rows], "moe dgrad")
