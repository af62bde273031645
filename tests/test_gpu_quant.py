"""GPU quantizers against the CPU oracle: bytes and scales must be bit-exact."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import fp8_block_scaled_gemm_amd as dg
from fp8_block_scaled_gemm_amd import inputs
import oracle
import oracle_pins
from gpu_util import bits32, device, oracle_quant_blocks, oracle_quant_rows, say, sa_from_dev, to_dev

pytestmark = pytest.mark.gpu


def run_token_group(x, ld_extra=0):
    m, k = x.shape
    xd = to_dev(x)
    ld = dg.dg_get_scale_ld(m) + ld_extra
    sa = torch.full((-(-k // 128), ld), float("nan"), dtype=torch.float32, device=device())
    q, sa = dg.dg_quantize_per_token_group(xd, sa=sa)
    torch.cuda.synchronize()
    sa_np = sa.cpu().numpy()
    if ld > m:   # entries past the rows stay untouched
        assert np.all(np.isnan(sa_np[:, m:]))
    return q.cpu().numpy(), sa_np[:, :m].T.copy()


def assert_token_group_exact(x, ld_extra=0):
    q, s = run_token_group(x, ld_extra)
    qo, so = oracle.quant.quantize_per_token_group(x)
    assert np.array_equal(bits32(s), bits32(so)), np.argwhere(bits32(s) != bits32(so))[:5]
    bad = np.argwhere(q != qo)
    assert bad.size == 0, [(tuple(i), float(x[tuple(i)]), hex(q[tuple(i)]), hex(qo[tuple(i)])) for i in bad[:5]]


@pytest.mark.parametrize("m,k,ld_extra", [(128, 512, 0), (1, 128, 0), (3, 384, 4), (77, 256, 0),
                                          (130, 1024, 8), (1000, 640, 0)])
def test_token_group_bit_exact(m, k, ld_extra):
    say("quant token group", m, k)
    rng = inputs.rng_for("quant_tok", m, k)
    x = inputs.activations_with_outliers(rng, m, k) if m > 2 else inputs.normal(rng, (m, k))
    assert_token_group_exact(x, ld_extra)


def test_token_group_special_values():
    say("quant token group special values")
    x = np.zeros((8, 256), np.float32)
    x[1, 7] = np.float32(-0.0)                    # all-zero groups keep the sign of zero
    x[2, 3] = np.float32(3.7)                     # one-hot
    x[3, 200] = np.float32(-1e-3)
    x[4, :] = np.float32(448.0)                   # exactly representable, s = 1
    x[5, :128] = np.float32(1e-30)                # tiny but normal amax
    x[5, 128:] = np.linspace(-1e4, 1e4, 128, dtype=np.float32)
    x[6, :128] = np.float32(-2.0 ** -11)
    x[6, 0] = np.float32(1.0)                     # small negatives round to -0 (0x80)
    x[7, :] = np.float32(2.0 ** 20) * np.sign(np.arange(256) - 127.5).astype(np.float32)
    assert_token_group_exact(x)


def _near_tie_rows(seed=5, rows=16):
    """Rows whose entries sit within a few ulps of x = tie * s (tie = midpoint of two E4M3 codes)."""
    rng = np.random.default_rng(seed)
    pos = [float(v) for v, _ in oracle_pins._POS]
    out = []
    for _ in range(rows):
        amax = np.float32(np.exp2(rng.uniform(-3, 6)) * rng.uniform(1, 2))
        s = oracle_pins.rn32(Fraction(float(amax)) / 448)
        xs = [amax]
        for i in rng.choice(len(pos) - 1, size=14, replace=False):
            c = oracle_pins.rn32(Fraction(pos[i] + pos[i + 1]) / 2 * Fraction(float(s)))
            for _ in range(4):
                c = np.nextafter(c, np.float32(-np.inf))
            for _ in range(9):
                if abs(float(c)) <= float(amax):
                    xs.append(c if rng.random() < 0.5 else -c)
                c = np.nextafter(c, np.float32(np.inf))
        out.append((xs + [np.float32(0)] * 128)[:128])
    return np.array(out, dtype=np.float32)


def test_token_group_near_ties():
    say("quant token group near ties")
    assert_token_group_exact(_near_tie_rows())


def conversion_class_values():
    """fp32 values covering every rounding class of fp32 -> E4M3 for |v| <= 448: every exponent
    from 2^-24 to 2^8, all top-7 mantissa bits (3 kept + guard + 3 more), sticky patterns of the
    low 16 bits, both signs."""
    exps = np.arange(127 - 24, 127 + 9, dtype=np.uint32)
    hi = np.arange(128, dtype=np.uint32) << 16
    lo = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    bits = (exps[:, None, None] << 23) | hi[None, :, None] | lo[None, None, :]
    v = bits.reshape(-1).view(np.float32)
    v = v[np.abs(v) <= 448]
    return np.concatenate([v, -v, np.float32([0.0, -0.0])])


def test_conversion_classes_exhaustive():
    """With 448 in every group, s = 1 exactly and x / s = x: the group quantizer then converts the
    test values themselves, so this covers the fp32 -> E4M3 rounding of every class."""
    say("quant conversion classes")
    v = conversion_class_values()
    per = 127
    n_rows = -(-v.size // per)
    vals = np.zeros(n_rows * per, np.float32)
    vals[:v.size] = v
    x = np.concatenate([np.full((n_rows, 1), 448.0, np.float32), vals.reshape(n_rows, per)], axis=1)
    q, s = run_token_group(x)
    assert np.all(s == 1.0)
    want = oracle.e4m3.encode(x)
    bad = np.argwhere(q != want)
    assert bad.size == 0, [(float(x[tuple(i)]), hex(q[tuple(i)]), hex(want[tuple(i)])) for i in bad[:8]]


def test_token_group_power_of_two_invariance():
    say("quant pow2 invariance")
    rng = inputs.rng_for("quant_pow2")
    x = inputs.normal(rng, (64, 512))
    q0, s0 = run_token_group(x)
    for j in (-9, 5):
        q, s = run_token_group((x * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(q, q0) and np.array_equal(s, (s0 * np.float32(2.0 ** j)).astype(np.float32))


def run_block(w):
    wd = to_dev(w)
    q, sb = dg.dg_quantize_per_block(wd)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sb.cpu().numpy()


@pytest.mark.parametrize("shape", [(512, 512), (200, 256), (2112, 384), (1, 128), (3, 200, 256), (2, 128, 128)])
def test_block_bit_exact(shape):
    say("quant block", shape)
    rng = inputs.rng_for("quant_blk", *shape)
    w = inputs.normal(rng, shape, 0.02)
    w.reshape(-1)[:: 997] *= np.float32(50.0)   # a few large entries in some blocks
    q, sb = run_block(w)
    if w.ndim == 3:
        qo, so = oracle.quant.quantize_per_block_grouped(w)
    else:
        qo, so = oracle.quant.quantize_per_block(w)
    assert np.array_equal(bits32(sb), bits32(so))
    assert np.array_equal(q, qo), np.argwhere(q != qo)[:5]


@pytest.mark.parametrize("m,k", [(4096, 7168), (128, 16384)])
def test_token_group_v3_sizes(m, k):
    """Full V3 activation sizes: every group bit-exact."""
    say("quant token group full size", m, k)
    rng = inputs.rng_for("quant_tok_v3", m, k)
    x = inputs.activations_with_outliers(rng, m, k)
    q, s = run_token_group(x)
    qo, so = oracle_quant_rows(x)
    assert np.array_equal(bits32(s), bits32(so))
    assert np.array_equal(q, qo)


@pytest.mark.parametrize("n,k", [(2112, 7168), (7168, 2048)])
def test_block_v3_sizes(n, k):
    say("quant block full size", n, k)
    rng = inputs.rng_for("quant_blk_v3", n, k)
    w = inputs.normal(rng, (n, k), 0.02)
    q, sb = run_block(w)
    qo, so = oracle_quant_blocks(w)
    assert np.array_equal(bits32(sb), bits32(so))
    assert np.array_equal(q, qo)


def test_quant_errors():
    say("quant errors")
    x = torch.zeros((4, 100), dtype=torch.float32, device=device())
    with pytest.raises(dg.DGError, match="INVALID_ARG"):
        dg.dg_quantize_per_token_group(x)
    q, sa = dg.dg_quantize_per_token_group(torch.zeros((0, 128), dtype=torch.float32, device=device()))
    assert q.shape == (0, 128)


def test_token_group_batched():
    """(G, M, K) input: per-group MN-major scales (G, K/128, ld_sa), bytes per group."""
    say("quant token group batched")
    rng = inputs.rng_for("quant_batched")
    x = inputs.normal(rng, (3, 77, 256))
    x[1] *= np.float32(30.0)
    ld = dg.dg_get_scale_ld(77) + 4
    sa = torch.full((3, 2, ld), float("nan"), dtype=torch.float32, device=device())
    q, sa = dg.dg_quantize_per_token_group(to_dev(x), sa=sa)
    torch.cuda.synchronize()
    q, sa = q.cpu().numpy(), sa.cpu().numpy()
    assert np.all(np.isnan(sa[:, :, 77:]))
    for g in range(3):
        qo, so = oracle.quant.quantize_per_token_group(x[g])
        assert np.array_equal(q[g], qo)
        assert np.array_equal(bits32(sa[g, :, :77].T), bits32(so))


def run_token_group_bf16(bits, ld_extra=0):
    """bf16 bits (M, K) or (G, M, K) -> GPU (q, sa) via the bf16 entry point."""
    xd = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device()).view(torch.bfloat16)
    m, k = bits.shape[-2:]
    ld = dg.dg_get_scale_ld(m) + ld_extra
    lead = bits.shape[:-2]
    sa = torch.full(lead + (-(-k // 128), ld), float("nan"), dtype=torch.float32, device=device())
    q, sa = dg.dg_quantize_per_token_group(xd, sa=sa)
    torch.cuda.synchronize()
    sa_np = sa.cpu().numpy()
    if ld > m:
        assert np.all(np.isnan(sa_np[..., m:]))
    return q.cpu().numpy(), sa_np[..., :m]


@pytest.mark.parametrize("m,k,ld_extra", [(128, 512, 0), (1, 128, 0), (77, 384, 4), (1000, 640, 0),
                                          (4096, 7168, 0)])
def test_token_group_bf16_bit_exact(m, k, ld_extra):
    """bf16 activations (N(0,1) with 1% outlier rows, rounded to bf16): bit-exact against the
    oracle on the same bf16 values."""
    say("quant token group bf16", m, k)
    rng = inputs.rng_for("quant_bf16", m, k)
    bits = inputs.to_bf16_bits(inputs.activations_with_outliers(rng, m, k) if m > 1 else inputs.normal(rng, (m, k)))
    q, s = run_token_group_bf16(bits, ld_extra)
    qo, so = oracle_quant_rows(oracle.bf16.decode(bits)) if m >= 512 else \
        oracle.quant.quantize_per_token_group_bf16(bits)
    assert np.array_equal(bits32(s.T), bits32(so))
    assert np.array_equal(q, qo)


def test_token_group_bf16_special_values():
    """Extreme bf16 inputs: the largest finite value, the smallest subnormal, signed zeros,
    groups of one magnitude, an all-zero group."""
    say("quant token group bf16 special values")
    rng = np.random.default_rng(41)
    bits = rng.integers(0, 1 << 16, size=(6, 512)).astype(np.uint16)
    bits &= np.uint16(0x7F7F) | np.uint16(0x8000)            # finite patterns only (exponent < 255)
    bits[0, :128] = 0x7F7F                                    # max finite
    bits[0, 128:256] = 0xFF7F                                 # -max finite
    bits[1, :] = 0x0001                                       # smallest subnormal everywhere
    bits[2, :128] = 0x8000                                    # -0.0 group
    bits[2, 128:256] = 0x0000                                 # +0.0 group
    bits[3, 5] = 0x7F7F                                       # one huge value among random ones
    q, s = run_token_group_bf16(bits)
    qo, so = oracle.quant.quantize_per_token_group_bf16(bits)
    assert np.array_equal(bits32(s.T), bits32(so))
    assert np.array_equal(q, qo)


def test_token_group_bf16_batched_matches_fp32():
    """(G, M, K) bf16 input gives the bytes and scales of the fp32 entry point on the widened values."""
    say("quant token group bf16 batched")
    rng = inputs.rng_for("quant_bf16_batched")
    bits = inputs.to_bf16_bits(inputs.normal(rng, (3, 40, 384)) * np.float32(7.0))
    q16, s16 = run_token_group_bf16(bits, ld_extra=4)
    widened = oracle.bf16.decode(bits)
    q32, s32 = dg.dg_quantize_per_token_group(to_dev(widened))
    torch.cuda.synchronize()
    assert np.array_equal(q16, q32.cpu().numpy())
    assert np.array_equal(bits32(s16), bits32(s32.cpu().numpy()[..., :40]))


@pytest.mark.parametrize("m,k", [(3, 16), (77, 144), (130, 400), (8, 7184), (512, 2064)])
def test_token_group_ragged_k(m, k):
    """K % 128 != 0: the last group holds K mod 128 elements; its scale is their amax / 448."""
    say("quant token group ragged k", m, k)
    rng = inputs.rng_for("quant_ragged_k", m, k)
    x = inputs.activations_with_outliers(rng, m, k) if m > 1 else inputs.normal(rng, (m, k))
    x[:, -16:] *= np.float32(300.0)   # outliers inside the partial group
    assert_token_group_exact(x)
    bits = inputs.to_bf16_bits(x)
    q, s = run_token_group_bf16(bits)
    qo, so = oracle.quant.quantize_per_token_group_bf16(bits)
    assert np.array_equal(bits32(s.T), bits32(so)) and np.array_equal(q, qo)


@pytest.mark.parametrize("shape", [(130, 16), (256, 144), (2, 200, 400), (129, 2064)])
def test_block_ragged_k(shape):
    """K % 128 != 0: the last 128 x (K mod 128) block takes its amax over the columns present."""
    say("quant block ragged k", shape)
    rng = inputs.rng_for("quant_blk_ragged", *shape)
    w = inputs.normal(rng, shape, 0.02)
    w[..., -16:] *= np.float32(40.0)
    q, sb = run_block(w)
    qo, so = oracle.quant.quantize_per_block_grouped(w) if w.ndim == 3 else oracle.quant.quantize_per_block(w)
    assert np.array_equal(bits32(sb), bits32(so))
    assert np.array_equal(q, qo)
