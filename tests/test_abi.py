"""The C ABI library loads on a host without a GPU, exports every symbol the header declares,
and rejects invalid arguments synchronously (these checks run before any HIP call)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")
LIB = os.path.join(ROOT, "fp8_block_scaled_gemm_amd", "libdg.so")

DG_OK, DG_ERR_INVALID_ARG = 0, -1


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libdg.so is not built: run `python -m fp8_block_scaled_gemm_amd._build`")
    import fp8_block_scaled_gemm_amd as dg
    return dg.lib()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("dg_gemm_fp8_nt", "dg_gemm_fp8_grouped_contiguous", "dg_gemm_fp8_grouped_masked",
                     "dg_quantize_per_token_group", "dg_quantize_per_block"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), name
    # and the binding wraps every one of them with the same name
    import fp8_block_scaled_gemm_amd as dg
    for name in names:
        if name not in ("dg_status_string", "dg_last_error_message"):
            assert callable(getattr(dg, name)), name


def test_pure_utilities(lib):
    assert lib.dg_get_m_alignment_for_contiguous_layout() == 128
    assert [lib.dg_get_scale_ld(m) for m in (0, 1, 4, 5, 127, 128, 129)] == [0, 4, 4, 8, 128, 128, 132]
    assert lib.dg_status_string(DG_OK) == b"DG_OK"
    assert lib.dg_status_string(DG_ERR_INVALID_ARG) == b"DG_ERR_INVALID_ARG"
    assert lib.dg_set_num_cus(0) == DG_ERR_INVALID_ARG
    assert b"n must be" in lib.dg_last_error_message()
    assert lib.dg_gemm_workspace_size(64, 512, 100, 1) == 0   # k % 16 != 0: invalid, never split


def _p(v):
    return ctypes.c_void_p(v)


def test_argument_validation(lib):
    fake = _p(0x1000)          # aligned, never dereferenced: validation fails first
    mis = _p(0x1004)
    # quantizers
    assert lib.dg_quantize_per_token_group(fake, 1, 4, 100, fake, fake, 4, None) == DG_ERR_INVALID_ARG
    assert lib.dg_quantize_per_token_group(fake, 1, 5, 128, fake, fake, 4, None) == DG_ERR_INVALID_ARG  # ld_sa < m
    assert lib.dg_quantize_per_token_group(fake, 1, 4, 128, fake, fake, 6, None) == DG_ERR_INVALID_ARG  # ld_sa % 4
    assert lib.dg_quantize_per_token_group(None, 1, 4, 128, fake, fake, 4, None) == DG_ERR_INVALID_ARG
    assert lib.dg_quantize_per_token_group(mis, 1, 4, 128, fake, fake, 4, None) == DG_ERR_INVALID_ARG
    assert lib.dg_quantize_per_token_group(None, 1, 0, 128, None, None, 0, None) == DG_OK       # empty
    assert lib.dg_quantize_per_token_group(None, 0, 4, 128, None, None, 4, None) == DG_OK
    assert lib.dg_quantize_per_token_group_bf16(fake, 1, 4, 100, fake, fake, 4, None) == DG_ERR_INVALID_ARG
    assert lib.dg_quantize_per_token_group_bf16(fake, 1, 5, 128, fake, fake, 4, None) == DG_ERR_INVALID_ARG
    assert lib.dg_quantize_per_token_group_bf16(mis, 1, 4, 128, fake, fake, 4, None) == DG_ERR_INVALID_ARG
    assert lib.dg_quantize_per_token_group_bf16(None, 1, 0, 128, None, None, 0, None) == DG_OK
    assert lib.dg_quantize_per_block(fake, 1, 10, 130, fake, fake, None) == DG_ERR_INVALID_ARG
    assert lib.dg_quantize_per_block(None, 1, 10, 128, fake, fake, None) == DG_ERR_INVALID_ARG
    assert lib.dg_quantize_per_block(None, 0, 10, 128, None, None, None) == DG_OK
    # dense GEMM
    args = lambda m, n, k, ld, a=fake, d=fake: (a, fake, ld, fake, fake, d, m, n, k, None, 0, None)
    assert lib.dg_gemm_fp8_nt(*args(4, 8, 100, 4)) == DG_ERR_INVALID_ARG        # k % 16 != 0
    assert lib.dg_gemm_fp8_nt(*args(4, 8, 0, 4)) == DG_ERR_INVALID_ARG
    assert lib.dg_gemm_fp8_nt(*args(8, 8, 128, 4)) == DG_ERR_INVALID_ARG          # ld_sa < m
    assert lib.dg_gemm_fp8_nt(*args(-1, 8, 128, 4)) == DG_ERR_INVALID_ARG
    assert lib.dg_gemm_fp8_nt(*args(4, 8, 128, 4, a=None)) == DG_ERR_INVALID_ARG
    assert lib.dg_gemm_fp8_nt(*args(4, 8, 128, 4, d=mis)) == DG_ERR_INVALID_ARG
    assert lib.dg_gemm_fp8_nt(*args(0, 8, 128, 0, a=None, d=None)) == DG_OK       # empty: no-op
    assert b"gemm" in lib.dg_last_error_message() or True
    # dense GEMM with the activation quantization in the launch: the workspace is required
    for fn in (lib.dg_gemm_fp8_nt_act_quant, lib.dg_gemm_fp8_nt_act_quant_bf16):
        fargs = lambda m, n, k, x=fake, ws=fake, d=fake: (x, fake, fake, d, m, n, k, ws, 1 << 20, None)
        assert fn(*fargs(4, 8, 100)) == DG_ERR_INVALID_ARG          # k % 16 != 0
        assert fn(*fargs(4, 8, 0)) == DG_ERR_INVALID_ARG
        assert fn(*fargs(-1, 8, 128)) == DG_ERR_INVALID_ARG
        assert fn(*fargs(4, 8, 128, x=None)) == DG_ERR_INVALID_ARG
        assert fn(*fargs(4, 8, 128, ws=None)) == DG_ERR_INVALID_ARG
        assert b"null pointer" in lib.dg_last_error_message()
        assert fn(*fargs(4, 8, 128, x=mis)) == DG_ERR_INVALID_ARG
        assert fn(*fargs(4, 8, 128, ws=mis)) == DG_ERR_INVALID_ARG
        assert fn(*fargs(0, 8, 128, x=None, ws=None, d=None)) == DG_OK   # empty: no-op
        assert fn(*fargs(4, 0, 128, x=None, ws=None, d=None)) == DG_OK
    assert lib.dg_gemm_fp8_nt_act_quant_workspace_size(4, 8, 100) == 0
    assert lib.dg_gemm_fp8_nt_act_quant_workspace_size(0, 8, 128) == 0
    # contiguous: m_total must be 128-aligned, m_indices required
    assert lib.dg_gemm_fp8_grouped_contiguous(fake, fake, 100, fake, fake, fake, 2, fake, 100, 8, 128,
                                              None) == DG_ERR_INVALID_ARG
    assert lib.dg_gemm_fp8_grouped_contiguous(fake, fake, 128, fake, fake, None, 2, fake, 128, 8, 128,
                                              None) == DG_ERR_INVALID_ARG
    assert lib.dg_gemm_fp8_grouped_contiguous(None, None, 0, None, None, None, 0, None, 0, 8, 128,
                                              None) == DG_OK
    # masked: masked_m required, group cap
    assert lib.dg_gemm_fp8_grouped_masked(fake, fake, 256, fake, fake, fake, None, 4, 256, 8, 128, None, 0,
                                          None) == DG_ERR_INVALID_ARG
    assert lib.dg_gemm_fp8_grouped_masked(fake, fake, 256, fake, fake, fake, fake, 2000, 256, 8, 128, None, 0,
                                          None) == DG_ERR_INVALID_ARG
    assert lib.dg_gemm_fp8_grouped_masked(fake, fake, 200, fake, fake, fake, fake, 4, 256, 8, 128, None, 0,
                                          None) == DG_ERR_INVALID_ARG     # ld_sa < m_max


def test_training_layout_argument_validation(lib):
    fake, fake2 = _p(0x1000), _p(0x2000)   # aligned, never dereferenced: validation fails first
    mis = _p(0x1004)
    for fn in (lib.dg_quantize_per_channel_group, lib.dg_quantize_per_channel_group_bf16):
        assert fn(fake, 1, 100, 8, fake, fake, 8, None) == DG_ERR_INVALID_ARG    # m % 16 != 0
        assert fn(fake, 1, 128, 6, fake, fake, 8, None) == DG_ERR_INVALID_ARG    # k % 4 != 0
        assert fn(fake, 1, 128, 8, fake, fake, 4, None) == DG_ERR_INVALID_ARG    # ld_st < k
        assert fn(fake, 1, 128, 8, fake, fake, 10, None) == DG_ERR_INVALID_ARG   # ld_st % 4 != 0
        assert fn(None, 1, 128, 8, fake, fake, 8, None) == DG_ERR_INVALID_ARG
        assert fn(mis, 1, 128, 8, fake, fake, 8, None) == DG_ERR_INVALID_ARG
        assert fn(None, 1, 0, 8, None, None, 8, None) == DG_OK                   # empty: no-op
        assert fn(None, 0, 128, 8, None, None, 8, None) == DG_OK
    assert lib.dg_transpose_blocks(fake, fake, 1, 100, 128, fake2, fake, None) == DG_ERR_INVALID_ARG   # rows % 16
    assert lib.dg_transpose_blocks(fake, fake, 1, 128, 120, fake2, fake, None) == DG_ERR_INVALID_ARG   # cols % 16
    assert lib.dg_transpose_blocks(fake, fake, 1, 128, 128, fake, fake, None) == DG_ERR_INVALID_ARG    # in place
    assert lib.dg_transpose_blocks(mis, fake, 1, 128, 128, fake2, fake, None) == DG_ERR_INVALID_ARG
    assert lib.dg_transpose_blocks(None, fake, 1, 128, 128, fake2, fake, None) == DG_ERR_INVALID_ARG
    assert lib.dg_transpose_blocks(None, None, 1, 0, 128, None, None, None) == DG_OK
    rs = lambda m, n, k, ld_sa, ld_sb, a=fake: (a, fake, ld_sa, fake, fake, ld_sb, fake, m, n, k, None, 0, None)
    assert lib.dg_gemm_fp8_nt_row_scaled(*rs(4, 8, 128, 4, 4)) == DG_ERR_INVALID_ARG     # ld_sb < n
    assert lib.dg_gemm_fp8_nt_row_scaled(*rs(4, 8, 128, 4, 10)) == DG_ERR_INVALID_ARG    # ld_sb % 4 != 0
    assert lib.dg_gemm_fp8_nt_row_scaled(*rs(4, 8, 100, 4, 8)) == DG_ERR_INVALID_ARG     # k % 16 != 0
    assert lib.dg_gemm_fp8_nt_row_scaled(*rs(8, 8, 128, 4, 8)) == DG_ERR_INVALID_ARG     # ld_sa < m
    assert lib.dg_gemm_fp8_nt_row_scaled(*rs(4, 8, 128, 4, 8, a=None)) == DG_ERR_INVALID_ARG
    assert lib.dg_gemm_fp8_nt_row_scaled(*rs(0, 8, 128, 0, 8, a=None)) == DG_OK           # empty: no-op


def test_k_grouped_argument_validation(lib):
    fake = _p(0x1000)
    counts = lambda *c: (ctypes.c_int64 * len(c))(*c)
    kg = lambda cnt, g, total, ld_sa=8, ld_sb=8, m=8, n=8: (fake, fake, ld_sa, fake, fake, ld_sb, fake, cnt, g, m, n,
                                                             total, None, 0, None)
    assert lib.dg_gemm_fp8_k_grouped_row_scaled(*kg(counts(128, 100), 2, 228)) == DG_ERR_INVALID_ARG   # 100 % 128
    assert lib.dg_gemm_fp8_k_grouped_row_scaled(*kg(counts(128, 256), 2, 256)) == DG_ERR_INVALID_ARG   # sum != total
    assert lib.dg_gemm_fp8_k_grouped_row_scaled(*kg(counts(128, -128), 2, 0)) == DG_ERR_INVALID_ARG    # negative
    assert lib.dg_gemm_fp8_k_grouped_row_scaled(*kg(None, 2, 256)) == DG_ERR_INVALID_ARG               # no counts
    assert lib.dg_gemm_fp8_k_grouped_row_scaled(*kg(counts(128), 1, 128, ld_sa=4)) == DG_ERR_INVALID_ARG  # ld_sa < m
    assert lib.dg_gemm_fp8_k_grouped_row_scaled(*kg(counts(128), 1, 128, m=3, n=5, ld_sa=4)) == DG_ERR_INVALID_ARG  # m*n % 8
    assert lib.dg_gemm_fp8_k_grouped_row_scaled(*kg(None, 0, 0)) == DG_OK                                # no groups
