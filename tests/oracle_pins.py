"""Pins for the CPU oracle: checks against facts that do not come from the oracle.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
something the format definition, an independent library, exact rational
arithmetic, a closed form or an invariant fixes.  They look the oracle's
functions up at call time, so ``test_oracle_mutants.py`` can plant a mistake
in the oracle and show that some pin catches it.
"""

import os
from fractions import Fraction

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# --------------------------------------------------------------------------
# Independent helpers (brute force; none of them calls the oracle)
# --------------------------------------------------------------------------


def _e4m3_value_table():
    """Exact Fraction value of each non-NaN code, from the bit fields (brute force)."""
    table = {}
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 0xF, c & 7
        if e == 15 and m == 7:
            continue
        mag = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        table[c] = -mag if s else mag
    return table


_TABLE = _e4m3_value_table()
_POS = sorted((v, c) for c, v in _TABLE.items() if c < 0x80)   # 0x00..0x7E, increasing


def brute_encode(v):
    """Nearest E4M3 code to the exact value of float v by exhaustive search; ties to the even code;
    magnitudes at or above 448 saturate; the sign bit is kept."""
    fv = Fraction(float(v))
    neg = np.signbit(v)
    a = abs(fv)
    if a >= 448:
        code = 0x7E
    else:
        best = None
        for val, c in _POS:
            d = abs(val - a)
            if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
                best = (d, c)
        code = best[1]
    return code | (0x80 if neg else 0)


def rn32(fr):
    """Round a Fraction to the nearest float32, ties to even (exhaustive over neighbours)."""
    guess = np.float32(float(fr))
    cands = {guess, np.nextafter(guess, np.float32(np.inf)), np.nextafter(guess, np.float32(-np.inf))}
    best = None
    for c in cands:
        d = abs(Fraction(float(c)) - fr)
        even = (np.array(c, dtype=np.float32).view(np.uint32) & 1) == 0
        if best is None or d < best[0] or (d == best[0] and even):
            best = (d, c)
    return np.float32(best[1])


def brute_quantize_group(x):
    """One group, scalar loop: amax, s = RN32(amax/448) (1.0 for amax = 0), q_i = enc(RN32(x_i/s))."""
    xs = [np.float32(v) for v in x]
    amax = max(abs(Fraction(float(v))) for v in xs)
    s = np.float32(1.0) if amax == 0 else rn32(amax / 448)
    q = [brute_encode(rn32(Fraction(float(v)) / Fraction(float(s)))) if v != 0 else (0x80 if np.signbit(v) else 0)
         for v in xs]
    return np.array(q, dtype=np.uint8), s


def read_named_codes():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_named_codes.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, value = line.split()[:2]
            rows.append((int(code, 16), float(value)))
    return rows


def hadamard(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


# --------------------------------------------------------------------------
# E4M3 codec pins
# --------------------------------------------------------------------------


def pin_e4m3_named_codes():
    for code, value in read_named_codes():
        got = float(oracle.e4m3.decode(np.array([code]))[0])
        if np.isnan(value):
            assert np.isnan(got), hex(code)
            continue
        assert got == value and np.signbit(got) == np.signbit(value), (hex(code), got, value)
        assert int(oracle.e4m3.encode(np.array([value]))[0]) == code, hex(code)


def pin_e4m3_decode_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3.decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def pin_e4m3_roundtrip():
    codes = oracle.e4m3.all_finite_codes()
    assert codes.size == 254
    back = oracle.e4m3.encode(oracle.e4m3.decode(codes))
    assert np.array_equal(back, codes)


def pin_e4m3_encode_vs_torch(n=200_000, seed=7):
    rng = np.random.default_rng(seed)
    # log-uniform magnitudes over the whole E4M3 range and beyond, both signs, fp32
    mags = np.exp2(rng.uniform(-14, 9.5, size=n)).astype(np.float32)
    vals = (mags * np.where(rng.random(n) < 0.5, -1, 1)).astype(np.float32)
    # exact midpoints between neighbouring codes, and their fp32 neighbours
    pos = np.array([float(v) for v, _ in _POS])
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    vals = np.concatenate([vals, near, -near, np.float32([0.0, -0.0, 448, 449, 463.9, 464, 465, 1e30, -1e30])])
    clamped = np.clip(vals, -448, 448)   # torch's cast does not saturate
    ref = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3.encode(vals)
    bad = np.nonzero(ref != got)[0]
    assert bad.size == 0, [(float(vals[i]), hex(ref[i]), hex(got[i])) for i in bad[:5]]


def pin_e4m3_ties_and_saturation():
    enc = oracle.e4m3.encode
    for (v0, c0), (v1, c1) in zip(_POS[:-1], _POS[1:]):
        mid = (v0 + v1) / 2
        want = c0 if (c0 & 1) == 0 else c1
        assert int(enc(np.array([float(mid)]))[0]) == want, (float(mid), hex(want))
        assert int(enc(np.array([-float(mid)]))[0]) == want | 0x80
    for v in (448.0, 449.0, 463.99, 464.0, 465.0, 1e30):
        assert int(enc(np.array([v]))[0]) == 0x7E
        assert int(enc(np.array([-v]))[0]) == 0xFE
    assert int(enc(np.array([-0.0]))[0]) == 0x80
    assert int(enc(np.array([-(2.0 ** -11)]))[0]) == 0x80
    assert int(enc(np.array([2.0 ** -10]))[0]) == 0x00        # tie between 0 and 2^-9 -> even (0)
    assert int(enc(np.array([3 * 2.0 ** -11]))[0]) == 0x01    # 0.75 * 2^-9: nearest is 2^-9
    assert int(enc(np.array([3 * 2.0 ** -10]))[0]) == 0x02    # tie between 2^-9 and 2^-8 -> even


def pin_e4m3_brute_force_sample(n=3000, seed=11):
    rng = np.random.default_rng(seed)
    vals = (np.exp2(rng.uniform(-12, 9.2, size=n)) * np.where(rng.random(n) < 0.5, -1, 1)).astype(np.float32)
    got = oracle.e4m3.encode(vals)
    for v, g in zip(vals, got):
        assert int(g) == brute_encode(v), (float(v), hex(int(g)))


# --------------------------------------------------------------------------
# Quantizer pins
# --------------------------------------------------------------------------


def pin_quant_brute_force(seed=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((3, 256)).astype(np.float32)
    x[1, :128] *= np.float32(100.0)
    x[2, 5] = np.float32(-0.0)
    q, sa = oracle.quant.quantize_per_token_group(x)
    assert q.shape == (3, 256) and sa.shape == (3, 2)
    for m in range(3):
        for kb in range(2):
            bq, bs = brute_quantize_group(x[m, 128 * kb:128 * kb + 128])
            assert sa[m, kb] == bs, (m, kb)
            assert np.array_equal(q[m, 128 * kb:128 * kb + 128], bq), (m, kb)


def pin_quant_near_ties(seed=5):
    """Inputs placed within a few fp32 ulps of x = tie * s, where the rounding of x/s decides the code."""
    rng = np.random.default_rng(seed)
    pos = [float(v) for v, _ in _POS]
    for trial in range(6):
        amax = np.float32(np.exp2(rng.uniform(-3, 6)) * rng.uniform(1, 2))
        s = rn32(Fraction(float(amax)) / 448)
        mids = rng.choice(len(pos) - 1, size=12, replace=False)
        xs = [amax]
        for i in mids:
            t = Fraction(pos[i] + pos[i + 1]) / 2 * Fraction(float(s))
            c = rn32(t)
            for _ in range(4):
                c = np.nextafter(c, np.float32(-np.inf))
            for _ in range(9):
                if abs(float(c)) <= float(amax):
                    xs.append(c)
                c = np.nextafter(c, np.float32(np.inf))
        xs = (xs + [np.float32(0)] * 128)[:128]
        x = np.array(xs, dtype=np.float32)[None, :]
        q, sa = oracle.quant.quantize_per_token_group(x)
        bq, bs = brute_quantize_group(x[0])
        assert sa[0, 0] == bs
        assert np.array_equal(q[0], bq), np.nonzero(q[0] != bq)


def pin_quant_one_hot():
    for c, j in ((3.7, 0), (-1e-3, 77), (2.5e4, 127)):
        x = np.zeros((1, 128), np.float32)
        x[0, j] = np.float32(c)
        q, sa = oracle.quant.quantize_per_token_group(x)
        assert sa[0, 0] == np.float32(abs(np.float32(c))) / np.float32(448)
        want = np.zeros(128, np.uint8)
        want[j] = 0x7E if c > 0 else 0xFE
        assert np.array_equal(q[0], want)


def pin_quant_representable(seed=9):
    """amax = 448 * 2^j with E4M3-representable entries: s = 2^j exactly and q recovers the codes."""
    rng = np.random.default_rng(seed)
    codes = np.array([c for c in _TABLE if c != 0x80], dtype=np.uint8)   # -0 has no Fraction sign
    for j in (-5, 0, 3):
        c = rng.choice(codes, size=(2, 128))
        c[:, 0] = 0x7E
        x = (np.array([[float(_TABLE[int(v)]) for v in row] for row in c]) * 2.0 ** j).astype(np.float32)
        q, sa = oracle.quant.quantize_per_token_group(x)
        assert np.all(sa == np.float32(2.0 ** j))
        assert np.array_equal(q, c.astype(np.uint8))
        qb, sb = oracle.quant.quantize_per_block(x)
        assert sb[0, 0] == np.float32(2.0 ** j) and np.array_equal(qb, c.astype(np.uint8))


def pin_quant_pow2_invariance(seed=13):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((4, 384)).astype(np.float32)
    q0, s0 = oracle.quant.quantize_per_token_group(x)
    w = rng.standard_normal((200, 256)).astype(np.float32) * np.float32(0.02)
    qw0, sw0 = oracle.quant.quantize_per_block(w)
    for j in (-7, 1, 9):
        q, s = oracle.quant.quantize_per_token_group((x * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(q, q0) and np.array_equal(s, (s0 * np.float32(2.0 ** j)).astype(np.float32))
        qw, sw = oracle.quant.quantize_per_block((w * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(qw, qw0) and np.array_equal(sw, (sw0 * np.float32(2.0 ** j)).astype(np.float32))


def pin_quant_zero_group():
    x = np.zeros((2, 256), np.float32)
    x[1, 130] = np.float32(-0.0)
    x[0, 200] = np.float32(1.0)
    q, sa = oracle.quant.quantize_per_token_group(x)
    assert sa[0, 0] == 1.0 and sa[1, 0] == 1.0 and sa[1, 1] == 1.0
    assert sa[0, 1] == np.float32(1.0) / np.float32(448)
    assert q[1, 130] == 0x80 and np.count_nonzero(q) == 2 and q[0, 200] == 0x7E


def pin_quant_block_edges(seed=17):
    """Per-block scales: block (i, kb) depends only on its own 128x128 elements; the partial last
    block's amax covers only the rows present; compare each block with the brute-force loop."""
    rng = np.random.default_rng(seed)
    n, k = 200, 256
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[150, 3] = np.float32(5.0)            # big value in the partial block only
    q, sb = oracle.quant.quantize_per_block(w)
    assert sb.shape == (2, 2)
    for i in range(2):
        for kb in range(2):
            blk = w[128 * i:min(n, 128 * i + 128), 128 * kb:128 * kb + 128]
            amax = np.max(np.abs(blk))
            assert sb[i, kb] == rn32(Fraction(float(amax)) / 448)
    blk = w[128:200, 0:128]
    for r in (0, 22, 71):                  # brute-force a few rows of the partial block
        row = blk[r]
        s = sb[1, 0]
        want = [brute_encode(rn32(Fraction(float(v)) / Fraction(float(s)))) for v in row]
        assert np.array_equal(q[128 + r, :128], np.array(want, np.uint8))
    w2 = w.copy()
    w2[0:128, 128:] *= np.float32(3.0)
    q2, sb2 = oracle.quant.quantize_per_block(w2)
    assert sb2[1, 1] == sb[1, 1] and sb2[0, 0] == sb[0, 0] and sb2[1, 0] == sb[1, 0]
    assert np.array_equal(q2[128:], q[128:]) and np.array_equal(q2[:128, :128], q[:128, :128])


def pin_quant_block_grouped(seed=19):
    """Grouped weights (G, N, K): every group's blocks take their scale from that group's own
    elements only.  Three groups of magnitudes 1e-3, 1 and 1e3 (so a scale shared across groups, or
    one group's blocks reused for another, is off by orders of magnitude), N = 200 (a partial
    72-row block).  Each block scale is checked against the exact amax / 448 rounded to fp32,
    sampled rows of every block against the scalar brute-force encoder, and a power-of-two change
    of one group must move that group's scales only."""
    rng = np.random.default_rng(seed)
    g, n, k = 3, 200, 256
    mags = [1e-3, 1.0, 1e3]
    w = np.stack([(rng.standard_normal((n, k)) * mags[e]).astype(np.float32) for e in range(g)])
    w[2, 190, 200] = np.float32(-4.5e3)   # the partial block of the last group holds its largest value
    q, sb = oracle.quant.quantize_per_block_grouped(w)
    assert q.shape == (g, n, k) and q.dtype == np.uint8
    assert sb.shape == (g, 2, 2) and sb.dtype == np.float32
    for e in range(g):
        for i in range(2):
            for kb in range(2):
                blk = w[e, 128 * i:min(n, 128 * i + 128), 128 * kb:128 * kb + 128]
                assert sb[e, i, kb] == rn32(Fraction(float(np.max(np.abs(blk)))) / 448), (e, i, kb)
        for r in (0, 127, 128, 199):      # first and last row of each 128-row block
            for kb in range(2):
                s = sb[e, r // 128, kb]
                cols = range(128 * kb, 128 * kb + 128, 5)
                want = [brute_encode(rn32(Fraction(float(w[e, r, c])) / Fraction(float(s)))) for c in cols]
                assert np.array_equal(q[e, r, list(cols)], np.array(want, np.uint8)), (e, r, kb)
    w2 = w.copy()
    w2[1] *= np.float32(2.0 ** 5)
    q2, sb2 = oracle.quant.quantize_per_block_grouped(w2)
    assert np.array_equal(q2, q)
    assert np.array_equal(sb2[1], (sb[1] * np.float32(32.0)).astype(np.float32))
    assert np.array_equal(sb2[0], sb[0]) and np.array_equal(sb2[2], sb[2])


# --------------------------------------------------------------------------
# GEMM pins
# --------------------------------------------------------------------------


def _random_operands(rng, m, n, k, g=None):
    codes = oracle.e4m3.all_finite_codes()
    kb = -(-k // 128)
    qa = rng.choice(codes, size=(m, k)).astype(np.uint8)
    sa = np.exp2(rng.uniform(-8, 2, size=(m, kb))).astype(np.float32)
    shape_b = (n, k) if g is None else (g, n, k)
    qb = rng.choice(codes, size=shape_b).astype(np.uint8)
    nb = -(-n // 128)
    shape_sb = (nb, kb) if g is None else (g, nb, kb)
    sb = np.exp2(rng.uniform(-12, -2, size=shape_sb)).astype(np.float32)
    return qa, sa, qb, sb


def exact_gemm(qa, sa, qb, sb):
    """Exact rational D with Fractions (brute force, tiny shapes only)."""
    m, k = qa.shape
    n = qb.shape[0]
    out = [[Fraction(0)] * n for _ in range(m)]
    mag = [[Fraction(0)] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            tot = Fraction(0)
            tot_abs = Fraction(0)
            for kb in range(-(-k // 128)):
                scale = Fraction(float(sa[i, kb])) * Fraction(float(sb[j // 128, kb]))
                for kk in range(128 * kb, min(128 * kb + 128, k)):
                    t = _TABLE[int(qa[i, kk])] * _TABLE[int(qb[j, kk])] * scale
                    tot += t
                    tot_abs += abs(t)
            out[i][j] = tot
            mag[i][j] = tot_abs
    return out, mag


def pin_gemm_exact_rational(seed=21):
    rng = np.random.default_rng(seed)
    m, n, k = 3, 130, 256          # N spans two scale blocks, the second partial
    qa, sa, qb, sb = _random_operands(rng, m, n, k)
    got = oracle.gemm.gemm_nt(qa, sa, qb, sb)
    assert got.shape == (m, n)
    ex, mag = exact_gemm(qa, sa, qb, sb)
    for i in range(m):
        for j in range(n):
            # fp64 sum of k exact products: |err| <= k * 2^-53 * sum |terms| (+ the final rounding)
            bound = Fraction(k + 1) * Fraction(2) ** -53 * mag[i][j]
            assert abs(Fraction(float(got[i, j])) - ex[i][j]) <= bound, (i, j, float(ex[i][j]), got[i, j])



def pin_gemm_all_448():
    a = np.full((4, 512), 448.0, np.float32)
    b = np.full((136, 512), 448.0, np.float32)
    qa, sa = oracle.quant.quantize_per_token_group(a)
    qb, sb = oracle.quant.quantize_per_block(b)
    d = oracle.gemm.gemm_nt(qa, sa, qb, sb)
    assert np.all(d == 448.0 * 448.0 * 512) and 448 * 448 * 512 == 102_760_448


def pin_gemm_hadamard():
    h = (448.0 * hadamard(128)).astype(np.float32)
    qa, sa = oracle.quant.quantize_per_token_group(h)
    qb, sb = oracle.quant.quantize_per_block(h)
    d = oracle.gemm.gemm_nt(qa, sa, qb, sb)
    assert np.array_equal(d, 448.0 * 448.0 * 128 * np.eye(128))


def pin_gemm_one_hot():
    k = 384
    qa = np.zeros((5, k), np.uint8)
    qb = np.zeros((7, k), np.uint8)
    sa = np.ones((5, 3), np.float32)
    sb = np.ones((1, 3), np.float32)
    qa[2, 200] = 0x3C          # 1.5
    qb[6, 200] = 0xC0          # -2
    sa[2, 1] = np.float32(0.25)
    sb[0, 1] = np.float32(3.0)
    d = oracle.gemm.gemm_nt(qa, sa, qb, sb)
    want = np.zeros((5, 7))
    want[2, 6] = 1.5 * -2.0 * 0.25 * 3.0
    assert np.array_equal(d, want)


def pin_gemm_invariants(seed=23):
    rng = np.random.default_rng(seed)
    qa, sa, qb, sb = _random_operands(rng, 6, 260, 384)
    d = oracle.gemm.gemm_nt(qa, sa, qb, sb)
    # K-block rebalancing by a power of two: bit-identical
    sa2, sb2 = sa.copy(), sb.copy()
    sa2[:, 1] *= np.float32(2.0 ** 5)
    sb2[:, 1] *= np.float32(2.0 ** -5)
    assert np.array_equal(oracle.gemm.gemm_nt(qa, sa2, qb, sb2), d)
    # row scaling: D row scales exactly
    sa3 = sa.copy()
    sa3[4] *= np.float32(8.0)
    d3 = oracle.gemm.gemm_nt(qa, sa3, qb, sb)
    assert np.array_equal(d3[4], 8.0 * d[4]) and np.array_equal(d3[:4], d[:4])
    # permuting A rows permutes D rows; permuting B rows inside a block permutes D columns
    p = rng.permutation(6)
    np.testing.assert_allclose(oracle.gemm.gemm_nt(qa[p], sa[p], qb, sb), d[p], rtol=1e-14, atol=0)
    pb = np.concatenate([rng.permutation(128), 128 + rng.permutation(128), [256, 257, 258, 259]])
    np.testing.assert_allclose(oracle.gemm.gemm_nt(qa, sa, qb[pb], sb), d[:, pb], rtol=1e-14, atol=0)
    # sign flips
    np.testing.assert_array_equal(oracle.gemm.gemm_nt(qa ^ np.uint8(0x80), sa, qb, sb), -d)


def pin_gemm_grouped(seed=29):
    rng = np.random.default_rng(seed)
    g, n, k = 3, 144, 256
    sizes = [128, 256, 128]
    m_total = sum(sizes)
    qa, sa, qb, sb = _random_operands(rng, m_total, n, k, g=g)
    m_idx = np.repeat(np.arange(g, dtype=np.int32), sizes)
    d = oracle.gemm.gemm_grouped_contiguous(qa, sa, qb, sb, m_idx)
    start = 0
    for e, sz in enumerate(sizes):
        np.testing.assert_array_equal(d[start:start + sz],
                                      oracle.gemm.gemm_nt(qa[start:start + sz], sa[start:start + sz], qb[e], sb[e]))
        start += sz
    # G = 1 contiguous is the dense GEMM
    d1 = oracle.gemm.gemm_grouped_contiguous(qa, sa, qb[:1], sb[:1], np.zeros(m_total, np.int32))
    np.testing.assert_array_equal(d1, oracle.gemm.gemm_nt(qa, sa, qb[0], sb[0]))
    # masked: rows < masked_m equal per-group dense; rows past it NaN; full mask = batched dense
    m_max = 128
    qam = qa[:g * m_max].reshape(g, m_max, k)
    sam = sa[:g * m_max].reshape(g, m_max, k // 128)
    masked = np.array([0, 77, 128], np.int32)
    dm = oracle.gemm.gemm_grouped_masked(qam, sam, qb, sb, masked)
    assert np.all(np.isnan(dm[0])) and np.all(np.isnan(dm[1, 77:]))
    full = oracle.gemm.gemm_nt(qam[1], sam[1], qb[1], sb[1])
    np.testing.assert_array_equal(dm[1, :77], full[:77])
    np.testing.assert_array_equal(dm[2], oracle.gemm.gemm_nt(qam[2], sam[2], qb[2], sb[2]))
    dfull = oracle.gemm.gemm_grouped_masked(qam, sam, qb, sb, np.full(g, 999, np.int32))   # clamped
    for e in range(g):
        np.testing.assert_array_equal(dfull[e], oracle.gemm.gemm_nt(qam[e], sam[e], qb[e], sb[e]))


def pin_bf16_decode_vs_torch():
    """All 65536 bf16 patterns widen to the same fp32 bits as torch's bfloat16 -> float32 cast."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    got = oracle.bf16.decode(bits)
    finite = np.isfinite(ref)
    assert np.array_equal(ref[finite].view(np.uint32), got[finite].view(np.uint32))
    assert np.array_equal(np.isnan(ref), np.isnan(got)) and np.array_equal(np.isinf(ref), np.isinf(got))


def pin_bf16_named_values():
    """Values fixed by the bf16 format definition (sign, 8-bit exponent bias 127, 7-bit mantissa)."""
    named = {0x3F80: 1.0, 0xC000: -2.0, 0x3FC0: 1.5, 0x0000: 0.0, 0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127,
             0x0080: 2.0 ** -126, 0x0001: 2.0 ** -133, 0x4049: 3.140625}
    for b, v in named.items():
        assert float(oracle.bf16.decode(np.array([b]))[0]) == v, hex(b)
    assert np.signbit(oracle.bf16.decode(np.array([0x8000]))[0])


def pin_quant_bf16_matches_widened(seed=31):
    """The bf16 quantizer equals the fp32 quantizer on the exactly widened values (bit for bit),
    and on bf16 data that is exactly representable its scale follows the one-hot closed form."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((8, 256)) * 3).astype(np.float32)
    bits = (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)      # truncation: still valid bf16 data
    widened = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    q1, s1 = oracle.quant.quantize_per_token_group_bf16(bits)
    q2, s2 = oracle.quant.quantize_per_token_group(widened)
    assert np.array_equal(q1, q2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    one = np.zeros((1, 128), np.uint16)
    one[0, 5] = 0xC2E0                                                  # -112.0
    q, s = oracle.quant.quantize_per_token_group_bf16(one)
    assert s[0, 0] == np.float32(112.0) / np.float32(448.0) and q[0, 5] == 0xFE and q[0].sum() == 0xFE


def pin_quant_ragged_k(seed=37):
    """K not a multiple of 128 (reading O14): every group, the last one partial, against the scalar
    brute force on exactly the elements present; weights too (a 128 x partial block)."""
    rng = np.random.default_rng(seed)
    for k in (16, 144, 400):
        x = (rng.standard_normal((3, k)) * 5).astype(np.float32)
        x[2, -16:] *= np.float32(1000.0)                # the partial group holds the row's outliers
        q, sa = oracle.quant.quantize_per_token_group(x)
        kb = -(-k // 128)
        assert q.shape == (3, k) and sa.shape == (3, kb)
        for m in range(3):
            for g in range(kb):
                bq, bs = brute_quantize_group(x[m, 128 * g:min(128 * g + 128, k)])
                assert sa[m, g] == bs and np.array_equal(q[m, 128 * g:128 * g + len(bq)], bq), (k, m, g)
        w = (rng.standard_normal((130, k)) * 0.1).astype(np.float32)
        qw, sw = oracle.quant.quantize_per_block(w)
        assert qw.shape == (130, k) and sw.shape == (2, kb)
        last = w[128:, 128 * (kb - 1):]
        bq, bs = brute_quantize_group(last.reshape(-1))
        assert sw[1, kb - 1] == bs and np.array_equal(qw[128:, 128 * (kb - 1):].reshape(-1), bq)


def pin_gemm_ragged_k_exact(seed=43):
    """Ragged K: the fp64 oracle against exact rational arithmetic over the K elements present."""
    rng = np.random.default_rng(seed)
    m, n, k = 2, 131, 272          # K = 2 full groups + 16; N spans a partial block
    qa, sa, qb, sb = _random_operands(rng, m, n, k)
    got = oracle.gemm.gemm_nt(qa, sa, qb, sb)
    ex, mag = exact_gemm(qa, sa, qb, sb)
    for i in range(m):
        for j in range(n):
            bound = Fraction(k + 1) * Fraction(2) ** -53 * mag[i][j]
            assert abs(Fraction(float(got[i, j])) - ex[i][j]) <= bound, (i, j)


# --------------------------------------------------------------------------
# Training-side layouts (per-channel token groups, transposed blocks, row-scaled GEMM)
# --------------------------------------------------------------------------


def pin_channel_quant_brute_force(seed=47):
    """Every 128-token group of every column, by the scalar brute-force group quantizer; M ragged
    (200 = 128 + 72), columns of very different magnitudes, one all-zero column."""
    rng = np.random.default_rng(seed)
    m, k = 200, 5
    x = (rng.standard_normal((m, k)) * np.array([1e-3, 1.0, 37.0, 0.0, 5e2])).astype(np.float32)
    x[3, 1] = np.float32(-0.0)
    qt, st = oracle.train.quantize_per_channel_group(x)
    assert qt.shape == (k, m) and st.shape == (k, 2)
    for col in range(k):
        for b, (r0, r1) in enumerate(((0, 128), (128, m))):
            q_ref, s_ref = brute_quantize_group(x[r0:r1, col])
            assert st[col, b] == s_ref, (col, b)
            assert np.array_equal(qt[col, r0:r1], q_ref), (col, b)


def pin_channel_quant_is_token_quant_of_transpose(seed=53):
    """Grouping 128 tokens of a column is grouping 128 elements of a row of x^T: the per-channel
    quantizer must agree with the (separately pinned) per-token-group quantizer on x^T."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((272, 48)) * np.exp2(rng.uniform(-6, 6, size=(1, 48)))).astype(np.float32)
    qt, st = oracle.train.quantize_per_channel_group(x)
    q_ref, s_ref = oracle.quant.quantize_per_token_group(np.ascontiguousarray(x.T))
    assert np.array_equal(qt, q_ref) and np.array_equal(st.view(np.uint32), s_ref.view(np.uint32))


def pin_channel_quant_bf16_widening(seed=59):
    """The bf16 variant quantizes torch's exact bf16 -> fp32 widening of its input."""
    rng = np.random.default_rng(seed)
    xt = torch.from_numpy(rng.standard_normal((144, 12)).astype(np.float32)).to(torch.bfloat16)
    bits = xt.view(torch.int16).numpy().view(np.uint16)
    got = oracle.train.quantize_per_channel_group_bf16(bits)
    ref = oracle.train.quantize_per_channel_group(xt.float().numpy())
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


def pin_block_quant_commutes_with_transpose(seed=61):
    """A 128 x 128 block is square: quantizing W^T block-wise gives W's codes and block scales
    transposed, partial edge blocks included (N = 200, K = 272)."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((200, 272)) * np.exp2(rng.uniform(-4, 4, size=(200, 1)))).astype(np.float32)
    qt_ref, st_ref = oracle.quant.quantize_per_block(np.ascontiguousarray(w.T))
    qt, st = oracle.train.transpose_blocks(*oracle.quant.quantize_per_block(w))
    assert qt.shape == (272, 200) and st.shape == (3, 2)
    assert np.array_equal(qt, qt_ref) and np.array_equal(st, st_ref)


def exact_gemm_row_scaled(qa, sa, qb, sb):
    """Exact rational D with per-row group scales on both operands (brute force, tiny shapes)."""
    m, k = qa.shape
    n = qb.shape[0]
    out, mag = [[Fraction(0)] * n for _ in range(m)], [[Fraction(0)] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            tot = tot_abs = Fraction(0)
            for kb in range(-(-k // 128)):
                scale = Fraction(float(sa[i, kb])) * Fraction(float(sb[j, kb]))
                for kk in range(128 * kb, min(128 * kb + 128, k)):
                    t = _TABLE[int(qa[i, kk])] * _TABLE[int(qb[j, kk])] * scale
                    tot += t
                    tot_abs += abs(t)
            out[i][j], mag[i][j] = tot, tot_abs
    return out, mag


def pin_row_scaled_gemm_exact(seed=67):
    """The both-sides row-scaled GEMM against exact rational arithmetic (K ragged, 2.1 groups)."""
    rng = np.random.default_rng(seed)
    m, n, k = 3, 5, 272
    codes = oracle.e4m3.all_finite_codes()
    qa = rng.choice(codes, size=(m, k)).astype(np.uint8)
    qb = rng.choice(codes, size=(n, k)).astype(np.uint8)
    sa = np.exp2(rng.uniform(-8, 2, size=(m, 3))).astype(np.float32)
    sb = np.exp2(rng.uniform(-12, -2, size=(n, 3))).astype(np.float32)
    got = oracle.train.gemm_nt_row_scaled(qa, sa, qb, sb)
    ex, mag = exact_gemm_row_scaled(qa, sa, qb, sb)
    for i in range(m):
        for j in range(n):
            bound = Fraction(k + 1) * Fraction(2) ** -53 * mag[i][j]
            assert abs(Fraction(float(got[i, j])) - ex[i][j]) <= bound, (i, j)


def pin_row_scaled_reduces_to_block_scaled(seed=71):
    """Per-row scales that are constant over each 128-row block give the block-scaled GEMM."""
    rng = np.random.default_rng(seed)
    qa, sa, qb, sb = _random_operands(rng, 4, 200, 384)
    sb_rows = np.repeat(sb, 128, axis=0)[:200]
    got = oracle.train.gemm_nt_row_scaled(qa, sa, qb, sb_rows)
    ref = oracle.gemm.gemm_nt(qa, sa, qb, sb)
    assert np.array_equal(got, ref)


def _exactly_quantizable(rng, rows, cols):
    """Values whose every 128-group, along rows and along columns (and every 128 x 128 block),
    contains +-448 and otherwise powers of two in [2^-4, 2^8] or 0: every scale is exactly 1 and
    every value an exact E4M3 code, so quantization is the identity (and sums stay exact in fp64)."""
    v = np.exp2(rng.integers(-4, 9, size=(rows, cols))).astype(np.float32)
    v *= rng.choice(np.array([-1.0, 0.0, 1.0], dtype=np.float32), size=(rows, cols))
    r, c = np.indices((rows, cols))
    v[(r % 128) == (c % 128)] = np.float32(448.0)
    return v


def pin_linear_layer_identities(seed=73):
    """On exactly quantizable operands the forward, dgrad and wgrad compositions must return the
    exact products X W^T, dY W and dY^T X: a transposed operand or scale, or a wrong grouping,
    breaks at least one of them."""
    rng = np.random.default_rng(seed)
    m, n, k = 256, 384, 256
    x = _exactly_quantizable(rng, m, k)
    w = _exactly_quantizable(rng, n, k)
    dy = _exactly_quantizable(rng, m, n)
    x64, w64, dy64 = x.astype(np.float64), w.astype(np.float64), dy.astype(np.float64)
    assert np.array_equal(oracle.train.linear_forward(x, w), x64 @ w64.T)
    assert np.array_equal(oracle.train.linear_dgrad(dy, w), dy64 @ w64)
    assert np.array_equal(oracle.train.linear_wgrad(dy, x), dy64.T @ x64)


def pin_k_grouped_wgrad_exact(seed=79):
    """MoE wgrad over the contiguous layout on exactly quantizable operands: each expert's dW_e must
    equal the exact product of its own token rows (an empty expert gives zeros), so a shifted,
    swapped or dropped segment fails."""
    rng = np.random.default_rng(seed)
    tokens = [256, 0, 128, 384]
    m, n, k = sum(tokens), 136, 128
    x = _exactly_quantizable(rng, m, k)
    dy = _exactly_quantizable(rng, m, n)
    got = oracle.train.linear_wgrad_k_grouped(dy, x, tokens)
    assert got.shape == (4, n, k)
    start = 0
    for e, t in enumerate(tokens):
        ref = dy[start:start + t].astype(np.float64).T @ x[start:start + t].astype(np.float64)
        assert np.array_equal(got[e], ref), e
        start += t


def pin_k_grouped_wgrad_sums_to_dense(seed=83):
    """The experts' weight gradients sum to the dense weight gradient over all tokens (128-aligned
    segments: the per-channel groups of the whole matrix are the experts' groups)."""
    rng = np.random.default_rng(seed)
    tokens = [128, 384, 256]
    m = sum(tokens)
    x = (rng.standard_normal((m, 96)) * np.exp2(rng.uniform(-3, 3, size=(m, 1)))).astype(np.float32)
    dy = rng.standard_normal((m, 80)).astype(np.float32)
    per_expert = oracle.train.linear_wgrad_k_grouped(dy, x, tokens)
    dense = oracle.train.linear_wgrad(dy, x)
    assert np.allclose(per_expert.sum(axis=0), dense, rtol=1e-12, atol=1e-12 * np.abs(dense).max())


ALL_PINS = [
    pin_e4m3_named_codes, pin_e4m3_decode_vs_torch, pin_e4m3_roundtrip, pin_e4m3_encode_vs_torch,
    pin_e4m3_ties_and_saturation, pin_e4m3_brute_force_sample,
    pin_quant_brute_force, pin_quant_near_ties, pin_quant_one_hot, pin_quant_representable,
    pin_quant_pow2_invariance, pin_quant_zero_group, pin_quant_block_edges, pin_quant_block_grouped,
    pin_gemm_exact_rational, pin_gemm_all_448, pin_gemm_hadamard, pin_gemm_one_hot,
    pin_gemm_invariants, pin_gemm_grouped,
    pin_bf16_decode_vs_torch, pin_bf16_named_values, pin_quant_bf16_matches_widened,
    pin_quant_ragged_k, pin_gemm_ragged_k_exact,
    pin_channel_quant_brute_force, pin_channel_quant_is_token_quant_of_transpose, pin_channel_quant_bf16_widening,
    pin_block_quant_commutes_with_transpose, pin_row_scaled_gemm_exact, pin_row_scaled_reduces_to_block_scaled,
    pin_linear_layer_identities, pin_k_grouped_wgrad_exact, pin_k_grouped_wgrad_sums_to_dense,
]
