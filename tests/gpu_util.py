"""Helpers shared by the GPU tests: device transfer of operands, the acceptance check and a
thread-parallel driver for the (row-independent) CPU oracle quantizers."""

import concurrent.futures as cf
import os
import sys

import numpy as np
import pytest
import torch

import oracle

# Acceptance (elementwise and Frobenius), as stated for this method's parity:
#   |gpu - ref| <= 8e-3 * |ref| + 1e-3 * rms(ref)  and  ||gpu - ref||_F / ||ref||_F <= 2e-3
REL_TOL = 8e-3
RMS_TOL = 1e-3
FROB_TOL = 2e-3

BF16_NAN = 0xFFFF   # sentinel pre-filled into outputs that must stay unwritten


def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch.device("cuda", 0)


def say(*msg):
    """Name the case on stdout (flushed) before a GPU step, so a crash still says what ran."""
    print("[case]", *msg, flush=True)
    sys.stdout.flush()


def to_dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device())


def sa_to_dev(sa_rows, ld=None, fill=0.0):
    """Oracle activation scales (rows, KB) -> device (KB, ld) MN-major."""
    rows, kb = sa_rows.shape
    ld = ld or max(4, -(-rows // 4) * 4)
    out = np.full((kb, ld), fill, dtype=np.float32)
    out[:, :rows] = sa_rows.T
    return to_dev(out)


def sa_from_dev(sa_dev, rows):
    return sa_dev.cpu().numpy()[:, :rows].T.copy()


def bits32(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def check_gemm(got, ref, what=""):
    """Acceptance check of a bf16 GEMM output (torch, any device) against the fp64 oracle."""
    g = got.float().cpu().numpy().astype(np.float64) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = np.abs(g - ref)
    bound = REL_TOL * np.abs(ref) + RMS_TOL * rms
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{what}: {len(bad)} elements outside tolerance; first {bad[:3].tolist()} "
                           f"got {g[tuple(bad[0])]} ref {ref[tuple(bad[0])]}")
    nref = float(np.linalg.norm(ref))
    frob = float(np.linalg.norm(g - ref)) / nref if nref > 0 else float(np.linalg.norm(g))
    assert frob <= FROB_TOL, f"{what}: relative Frobenius error {frob:.3e} > {FROB_TOL}"
    return frob


def bf16_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        _POOL = cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4))
    return _POOL


def oracle_quant_rows(x, chunk=512):
    """Oracle per-token-group quantization, run on row chunks in threads (numpy releases the GIL)."""
    parts = list(_pool().map(oracle.quant.quantize_per_token_group,
                             [x[i:i + chunk] for i in range(0, x.shape[0], chunk)]))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def oracle_quant_blocks(w, chunk=512):
    """Oracle per-block quantization of (N, K) or (G, N, K), 128-row-aligned chunks in threads."""
    if w.ndim == 3:
        res = [oracle_quant_blocks(w[g], chunk) for g in range(w.shape[0])]
        return np.stack([r[0] for r in res]), np.stack([r[1] for r in res])
    assert chunk % 128 == 0
    parts = list(_pool().map(oracle.quant.quantize_per_block,
                             [w[i:i + chunk] for i in range(0, w.shape[0], chunk)]))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def cu_masked_stream(first, count):
    """A HIP stream whose kernels may only run on CUs [first, first + count)
    (hipExtStreamCreateWithCUMask, default priority), wrapped for torch."""
    import ctypes
    total = torch.cuda.get_device_properties(0).multi_processor_count
    hip = ctypes.CDLL("libamdhip64.so")
    words = (total + 31) // 32
    mask = [0] * words
    for cu in range(first, min(first + count, total)):
        mask[cu // 32] |= 1 << (cu % 32)
    arr = (ctypes.c_uint32 * words)(*mask)
    handle = ctypes.c_void_p()
    err = hip.hipExtStreamCreateWithCUMask(ctypes.byref(handle), ctypes.c_uint32(words), arr)
    if err != 0:
        pytest.fail(f"hipExtStreamCreateWithCUMask failed ({err})")
    return torch.cuda.ExternalStream(handle.value, device=device())
