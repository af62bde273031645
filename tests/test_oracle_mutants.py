"""Plant plausible mistakes in the CPU oracle (on the CPU only) and show that the pins catch each.

If a mutant survives every pin, the pins are too weak to trust the oracle.
"""

import numpy as np
import pytest

import oracle
import oracle_pins

E = oracle.e4m3
Q = oracle.quant
G = oracle.gemm
B = oracle.bf16
T = oracle.train

_orig_encode = E.encode
_orig_decode = E.decode


def _encode_half_away(values):
    v = np.asarray(values, dtype=np.float64)
    neg = np.signbit(v)
    a = np.abs(v)
    _, ex = np.frexp(a)
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    quantum = np.ldexp(1.0, e - 3)
    r = np.floor(a / quantum + 0.5) * quantum            # ties away from zero
    return _orig_encode(np.where(neg, -r, r))


def _encode_no_saturation(values):
    v = np.asarray(values, dtype=np.float64)
    out = _orig_encode(v)
    return np.where(np.abs(v) > 448, out | 0x7F, out).astype(np.uint8)


def _encode_drops_negative_zero(values):
    out = _orig_encode(values)
    return np.where(out == 0x80, 0, out).astype(np.uint8)


def _decode_bias8(codes):
    return _orig_decode(codes) / 2.0


def _quant_tok_divisor(div):
    def f(x):
        x = np.asarray(x, dtype=np.float32)
        m, k = x.shape
        g = x.reshape(m, k // 128, 128)
        amax = np.max(np.abs(g), axis=2)
        s = np.where(amax == 0, np.float32(1), amax / np.float32(div)).astype(np.float32)
        return E.encode((g / s[:, :, None]).astype(np.float32)).reshape(m, k), s
    return f


def _quant_tok_reciprocal(x):
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    g = x.reshape(m, k // 128, 128)
    amax = np.max(np.abs(g), axis=2)
    s = np.where(amax == 0, np.float32(1), amax / np.float32(448)).astype(np.float32)
    r = (np.float32(1) / s).astype(np.float32)
    return E.encode((g * r[:, :, None]).astype(np.float32)).reshape(m, k), s


def _quant_tok_fp64_division(x):
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    g = x.reshape(m, k // 128, 128)
    amax = np.max(np.abs(g), axis=2)
    s = np.where(amax == 0, np.float32(1), amax / np.float32(448)).astype(np.float32)
    return E.encode(g.astype(np.float64) / s[:, :, None].astype(np.float64)).reshape(m, k), s


_orig_block = Q.quantize_per_block


def _quant_block_whole_panel(w):
    """amax over the full N panel of each K block instead of 128x128."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    q, sb = _orig_block(w)
    amax = np.max(np.abs(w.reshape(n, k // 128, 128)), axis=(0, 2))
    s = np.where(amax == 0, 1, amax / np.float32(448)).astype(np.float32)
    sb = np.broadcast_to(s, sb.shape).copy()
    q = E.encode((w.reshape(n, k // 128, 128) / s[None, :, None]).astype(np.float32)).reshape(n, k)
    return q, sb


_orig_block_grouped = Q.quantize_per_block_grouped


def _block_grouped_reuses_group0(w):
    """Every group quantized with group 0's blocks."""
    w = np.asarray(w, dtype=np.float32)
    q0, s0 = _orig_block(w[0])
    return np.stack([q0] * w.shape[0]), np.stack([s0] * w.shape[0])


def _block_grouped_shared_scale(w):
    """One scale per (N block, K block) taken over all groups together."""
    w = np.asarray(w, dtype=np.float32)
    g, n, k = w.shape
    amax = np.zeros((-(-n // 128), k // 128), np.float32)
    for e in range(g):
        for i in range(amax.shape[0]):
            blk = w[e, 128 * i:128 * i + 128].reshape(-1, k // 128, 128)
            amax[i] = np.maximum(amax[i], np.max(np.abs(blk), axis=(0, 2)))
    s = np.where(amax == 0, np.float32(1), amax / np.float32(448)).astype(np.float32)
    rows = np.repeat(s, 128, axis=0)[:n]                          # (n, k/128)
    q = np.stack([E.encode((w[e].reshape(n, k // 128, 128) / rows[:, :, None]).astype(np.float32)).reshape(n, k)
                  for e in range(g)])
    return q, np.stack([s] * g)


def _block_grouped_swaps_outputs(w):
    q, s = _orig_block_grouped(w)
    return s, q


def _gemm_no_sb(qa, sa, qb, sb):
    return G.dequantize_rows(qa, sa) @ E.decode(qb).T


def _gemm_sb_mod(qa, sa, qb, sb):
    n = qb.shape[0]
    rows = np.asarray(sb, np.float64)[np.arange(n) % sb.shape[0]]
    return G.dequantize_rows(qa, sa) @ G.dequantize_rows(qb, rows).T


def _gemm_sa_reversed_kb(qa, sa, qb, sb):
    return G.dequantize_rows(qa, np.asarray(sa)[:, ::-1]) @ G.dequantize_blocks(qb, sb).T


_orig_contig = G.gemm_grouped_contiguous
_orig_masked = G.gemm_grouped_masked


def _contig_off_by_one(qa, sa, qb, sb, m_indices):
    return _orig_contig(qa, sa, qb, sb, (np.asarray(m_indices) + 1) % np.asarray(qb).shape[0])


def _masked_no_clamp_computes_all(qa, sa, qb, sb, masked_m):
    return _orig_masked(qa, sa, qb, sb, np.full(len(masked_m), np.asarray(qa).shape[1]))


_orig_bf16_decode = B.decode


def _bf16_decode_drops_sign(bits):
    return np.abs(_orig_bf16_decode(bits))


def _bf16_decode_shift8(bits):
    b = np.asarray(bits).astype(np.uint32) & np.uint32(0xFFFF)
    return (b << np.uint32(8)).view(np.float32)


def _gemm_drops_k_tail(qa, sa, qb, sb):
    """Ragged K handled by dropping the partial last group."""
    k = np.asarray(qa).shape[1]
    kf = k // 128 * 128
    if kf == k:
        return _orig_gemm_nt(qa, sa, qb, sb)
    return _orig_gemm_nt(np.asarray(qa)[:, :kf], np.asarray(sa)[:, :kf // 128], np.asarray(qb)[:, :kf],
                         np.asarray(sb)[:, :kf // 128])


def _quant_tail_scale_from_full_window(x):
    """Ragged K: the last group's scale taken over 128 elements wrapped from the row start."""
    x = np.asarray(x, dtype=np.float32)
    k = x.shape[1]
    if k % 128 == 0:
        return _orig_tok(x)
    wrapped = np.concatenate([x, x[:, :128 - k % 128]], axis=1)
    q, s = _orig_tok(wrapped)
    return q[:, :k], s


_orig_channel = T.quantize_per_channel_group
_orig_wgrad = T.linear_wgrad
_orig_kgrouped = T.linear_wgrad_k_grouped

def _channel_quant_whole_column(x):
    """Per-channel quantizer with one scale over the whole column instead of per 128 tokens."""
    x = np.asarray(x, dtype=np.float32)
    m, k = x.shape
    amax = np.max(np.abs(x), axis=0)
    s = np.where(amax == 0, np.float32(1), amax / np.float32(448)).astype(np.float32)
    q = E.encode((x / s[None, :]).astype(np.float32)).T.copy()
    return q, np.repeat(s[:, None], -(-m // 128), axis=1)


def _channel_quant_not_transposed(x):
    """Per-channel scales right, codes left in x's own (M, K) layout read as (K, M)."""
    qt, st = _orig_channel(x)
    return qt.T.copy().reshape(qt.shape), st


def _transpose_blocks_keeps_scales(q, s):
    return np.ascontiguousarray(np.asarray(q).T), np.asarray(s)


def _row_scaled_uses_block_index(qa, sa, qb, sb):
    sb_block = np.asarray(sb)[::128]
    return G.dequantize_rows(qa, sa) @ G.dequantize_rows(qb, np.repeat(sb_block, 128, axis=0)[:qb.shape[0]]).T


def _wgrad_swapped(dy, x):
    return _orig_wgrad(x, dy)


def _k_grouped_experts_reversed(dy, x, group_tokens):
    return _orig_kgrouped(dy, x, group_tokens)[::-1].copy()


def _k_grouped_segment_shifted(dy, x, group_tokens):
    """Every expert's segment starts 128 tokens late (wrapping): the classic off-by-one-group slip."""
    shift = 128
    return _orig_kgrouped(np.roll(dy, -shift, axis=0), np.roll(x, -shift, axis=0), group_tokens)


_orig_gemm_nt = G.gemm_nt
_orig_tok = Q.quantize_per_token_group

MUTANTS = {
    "encode_ties_away": (E, "encode", _encode_half_away),
    "encode_no_saturation": (E, "encode", _encode_no_saturation),
    "encode_drops_negative_zero": (E, "encode", _encode_drops_negative_zero),
    "decode_bias8": (E, "decode", _decode_bias8),
    "quant_scale_amax_over_240": (Q, "quantize_per_token_group", _quant_tok_divisor(240)),
    "quant_reciprocal_multiply": (Q, "quantize_per_token_group", _quant_tok_reciprocal),
    "quant_fp64_division": (Q, "quantize_per_token_group", _quant_tok_fp64_division),
    "quant_block_whole_panel": (Q, "quantize_per_block", _quant_block_whole_panel),
    "block_grouped_reuses_group0": (Q, "quantize_per_block_grouped", _block_grouped_reuses_group0),
    "block_grouped_shared_scale": (Q, "quantize_per_block_grouped", _block_grouped_shared_scale),
    "block_grouped_swaps_outputs": (Q, "quantize_per_block_grouped", _block_grouped_swaps_outputs),
    "gemm_drops_weight_scale": (G, "gemm_nt", _gemm_no_sb),
    "gemm_weight_scale_index_mod": (G, "gemm_nt", _gemm_sb_mod),
    "gemm_act_scale_kb_reversed": (G, "gemm_nt", _gemm_sa_reversed_kb),
    "contiguous_expert_off_by_one": (G, "gemm_grouped_contiguous", _contig_off_by_one),
    "masked_writes_all_rows": (G, "gemm_grouped_masked", _masked_no_clamp_computes_all),
    "bf16_decode_drops_sign": (B, "decode", _bf16_decode_drops_sign),
    "bf16_decode_shift8": (B, "decode", _bf16_decode_shift8),
    "gemm_drops_ragged_k_tail": (G, "gemm_nt", _gemm_drops_k_tail),
    "quant_ragged_tail_wrapped_scale": (Q, "quantize_per_token_group", _quant_tail_scale_from_full_window),
    "channel_quant_whole_column": (T, "quantize_per_channel_group", _channel_quant_whole_column),
    "channel_quant_not_transposed": (T, "quantize_per_channel_group", _channel_quant_not_transposed),
    "transpose_blocks_keeps_scales": (T, "transpose_blocks", _transpose_blocks_keeps_scales),
    "row_scaled_gemm_block_index": (T, "gemm_nt_row_scaled", _row_scaled_uses_block_index),
    "wgrad_operands_swapped": (T, "linear_wgrad", _wgrad_swapped),
    "k_grouped_experts_reversed": (T, "linear_wgrad_k_grouped", _k_grouped_experts_reversed),
    "k_grouped_segment_shifted": (T, "linear_wgrad_k_grouped", _k_grouped_segment_shifted),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    module, attr, fn = MUTANTS[name]
    monkeypatch.setattr(module, attr, fn)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} survived every pin"
