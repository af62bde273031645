"""Python binding of libdg.so, the gfx950 FP8 block-scaled GEMM library.

Argument marshalling only: every step of the path runs in the HIP kernels of
libdg.so, called through its C ABI (``include/dg.h``).  PyTorch supplies
device memory and the current stream; nothing here computes.  If the library
is not built, every call raises - there is no fallback.

Functions carry the C names:

* ``dg_quantize_per_token_group(x)``  -> (q uint8 (M, K), sa float32 (ceil(K/128), ld_sa)); fp32 or
  bf16 x (the bf16 entry point is ``dg_quantize_per_token_group_bf16``)
* ``dg_quantize_per_block(w)``        -> (q uint8 like w, sb float32 ([G,] ceil(N/128), ceil(K/128)))
* ``dg_gemm_fp8_nt(a, sa, b, sb)``    -> d bf16 (M, N)
* ``dg_gemm_fp8_nt_act_quant(x, b, sb)`` -> d bf16 (M, N) from unquantized fp32 or bf16 x, its
  per-token-group quantization done inside the GEMM launch
* ``dg_gemm_fp8_grouped_contiguous(a, sa, b, sb, m_indices)``  -> d bf16 (M_total, N)
* ``dg_gemm_fp8_grouped_masked(a, sa, b, sb, masked_m)``       -> d bf16 (G, M_max, N)
* training-side layouts: ``dg_quantize_per_channel_group(x)`` -> (qt uint8 (K, M), st float32
  (ceil(M/128), ld_st)) in groups of 128 tokens per column, transposed (fp32 or bf16 x);
  ``dg_transpose_blocks(q, s)`` -> the block quantization of the transposed matrix;
  ``dg_gemm_fp8_nt_row_scaled(a, sa, b, sb)`` -> d bf16 (M, N) with per-row scales on both operands;
  ``dg_gemm_fp8_k_grouped_row_scaled(a, sa, b, sb, group_tokens)`` -> d bf16 (G, M, N), the MoE weight
  gradients over the contiguous layout
* utilities ``dg_get_num_cus``, ``dg_set_num_cus``,
  ``dg_get_m_alignment_for_contiguous_layout``, ``dg_get_scale_ld``,
  ``dg_gemm_workspace_size``.

Activation scales use the K-group-major layout of the library: ``sa[kb, row]``
(for the masked form ``sa[g, kb, row]``), row stride ``ld_sa = sa.shape[-1]``.
"""

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdg.so")

_lib = None
_lock = threading.Lock()

_c_int64 = ctypes.c_int64
_vp = ctypes.c_void_p

_SIGNATURES = {
    "dg_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "dg_last_error_message": (ctypes.c_char_p, []),
    "dg_quantize_per_token_group": (ctypes.c_int, [_vp, _c_int64, _c_int64, _c_int64, _vp, _vp, _c_int64, _vp]),
    "dg_quantize_per_token_group_bf16": (ctypes.c_int, [_vp, _c_int64, _c_int64, _c_int64, _vp, _vp, _c_int64,
                                                        _vp]),
    "dg_quantize_per_block": (ctypes.c_int, [_vp, _c_int64, _c_int64, _c_int64, _vp, _vp, _vp]),
    "dg_gemm_fp8_nt": (ctypes.c_int, [_vp, _vp, _c_int64, _vp, _vp, _vp, _c_int64, _c_int64, _c_int64,
                                      _vp, ctypes.c_size_t, _vp]),
    "dg_gemm_fp8_nt_no_alloc": (ctypes.c_int, [_vp, _vp, _c_int64, _vp, _vp, _vp, _c_int64, _c_int64, _c_int64,
                                               _vp]),
    "dg_gemm_fp8_nt_act_quant": (ctypes.c_int, [_vp, _vp, _vp, _vp, _c_int64, _c_int64, _c_int64, _vp,
                                                ctypes.c_size_t, _vp]),
    "dg_gemm_fp8_nt_act_quant_bf16": (ctypes.c_int, [_vp, _vp, _vp, _vp, _c_int64, _c_int64, _c_int64, _vp,
                                                     ctypes.c_size_t, _vp]),
    "dg_gemm_fp8_nt_act_quant_workspace_size": (ctypes.c_size_t, [_c_int64, _c_int64, _c_int64]),
    "dg_gemm_fp8_grouped_contiguous": (ctypes.c_int, [_vp, _vp, _c_int64, _vp, _vp, _vp, _c_int64, _vp,
                                                      _c_int64, _c_int64, _c_int64, _vp]),
    "dg_gemm_fp8_grouped_masked": (ctypes.c_int, [_vp, _vp, _c_int64, _vp, _vp, _vp, _vp, _c_int64,
                                                  _c_int64, _c_int64, _c_int64, _vp, ctypes.c_size_t, _vp]),
    "dg_gemm_fp8_nt_row_scaled": (ctypes.c_int, [_vp, _vp, _c_int64, _vp, _vp, _c_int64, _vp, _c_int64, _c_int64,
                                                 _c_int64, _vp, ctypes.c_size_t, _vp]),
    "dg_gemm_fp8_k_grouped_row_scaled": (ctypes.c_int, [_vp, _vp, _c_int64, _vp, _vp, _c_int64, _vp, _vp,
                                                        _c_int64, _c_int64, _c_int64, _c_int64, _vp, ctypes.c_size_t,
                                                        _vp]),
    "dg_quantize_per_channel_group": (ctypes.c_int, [_vp, _c_int64, _c_int64, _c_int64, _vp, _vp, _c_int64, _vp]),
    "dg_quantize_per_channel_group_bf16": (ctypes.c_int, [_vp, _c_int64, _c_int64, _c_int64, _vp, _vp, _c_int64,
                                                          _vp]),
    "dg_transpose_blocks": (ctypes.c_int, [_vp, _vp, _c_int64, _c_int64, _c_int64, _vp, _vp, _vp]),
    "dg_get_num_cus": (ctypes.c_int, []),
    "dg_set_num_cus": (ctypes.c_int, [ctypes.c_int]),
    "dg_get_m_alignment_for_contiguous_layout": (ctypes.c_int, []),
    "dg_get_scale_ld": (_c_int64, [_c_int64]),
    "dg_gemm_workspace_size": (ctypes.c_size_t, [_c_int64, _c_int64, _c_int64, _c_int64]),
    "dg_gemm_config_name": (ctypes.c_char_p, [ctypes.c_int, _c_int64, _c_int64, _c_int64, _c_int64]),
    "dg_get_debug_status": (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(_c_int64), ctypes.c_int]),
}

DG_DIAG_MIXED_BLOCK = 1
DG_DIAG_EXPERT_RANGE = 2
DG_DIAG_FQ_TIMEOUT = 4


def lib():
    """Load libdg.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(f"libdg.so is not built ({LIB_PATH}); run "
                                       "`python -m fp8_block_scaled_gemm_amd._build` first")
                handle = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in _SIGNATURES.items():
                    fn = getattr(handle, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = handle
    return _lib


class DGError(RuntimeError):
    def __init__(self, fn, status):
        L = lib()
        super().__init__(f"{fn}: {L.dg_status_string(status).decode()} "
                         f"({L.dg_last_error_message().decode()})")
        self.status = status


def _check(fn, status):
    if status != 0:
        raise DGError(fn, status)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _bytes(t):
    """View an FP8 tensor (uint8 or float8_e4m3fn) as uint8."""
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def _dev(*ts):
    for t in ts:
        _require(t.is_cuda and t.is_contiguous(), "tensors must be contiguous CUDA (HIP) tensors")
    return ts[0].device


# ---------------------------------------------------------------------------
# utilities
# ---------------------------------------------------------------------------

def dg_get_num_cus():
    r = lib().dg_get_num_cus()
    _check("dg_get_num_cus", r if r < 0 else 0)
    return r


def dg_set_num_cus(n):
    _check("dg_set_num_cus", lib().dg_set_num_cus(int(n)))


def dg_get_m_alignment_for_contiguous_layout():
    return lib().dg_get_m_alignment_for_contiguous_layout()


def dg_get_scale_ld(rows):
    return lib().dg_get_scale_ld(int(rows))


def dg_gemm_workspace_size(m, n, k, num_groups=1):
    return lib().dg_gemm_workspace_size(int(m), int(n), int(k), int(num_groups))


def dg_gemm_config_name(layout, m, n, k, num_groups=1):
    """Tile configuration / K split the GEMM picks (layout 0 normal, 1 contiguous, 2 masked,
    3 row-scaled normal)."""
    return lib().dg_gemm_config_name(int(layout), int(m), int(n), int(k), int(num_groups)).decode()


def dg_get_debug_status(clear=True):
    """(flags, block): the sticky device diagnostics (DG_DIAG_* bits) of the current device and the
    first 128-row block a contiguous-layout check found wrong (-1 if none).  Synchronises."""
    flags, block = ctypes.c_uint32(0), _c_int64(-1)
    _check("dg_get_debug_status", lib().dg_get_debug_status(ctypes.byref(flags), ctypes.byref(block), int(clear)))
    return int(flags.value), int(block.value)


_ws_cache = {}
_ws_retired = []


def default_workspace(device, nbytes):
    """A zero-filled workspace for the current stream of `device`, grown on demand (the kernels
    leave its counters zeroed).  Calls that share a workspace must be ordered on one stream, so
    every (device, stream) pair gets its own.  A buffer that a larger request supersedes is kept
    alive until the process ends, never freed: a graph captured with it, or a kernel still queued
    on it, may use it later.  Inside graph capture there is no default workspace (a buffer made
    there would be zero-filled only when the graph runs): pass one created before the capture."""
    if nbytes == 0:
        return None
    dev = torch.device(device)
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    stream = torch.cuda.current_stream(dev)
    if torch.cuda.is_current_stream_capturing():
        raise ValueError("no default workspace during graph capture: pass workspace= (a zero-filled uint8 "
                         "tensor of dg_gemm_workspace_size(...) bytes created before the capture)")
    key = (dev.index, stream.cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            _ws_retired.append(ws)
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _ws_cache[key] = ws
    return ws


# ---------------------------------------------------------------------------
# quantizers
# ---------------------------------------------------------------------------

def dg_quantize_per_token_group(x, q=None, sa=None):
    """x float32 or bfloat16 (M, K) -> (q uint8 (M, K), sa float32 (K/128, ld_sa)); or x (G, M, K)
    -> (q (G, M, K), sa (G, K/128, ld_sa)) for the per-expert masked layout.  Runs on x's stream.
    bfloat16 input goes to dg_quantize_per_token_group_bf16 (same result as the widened fp32)."""
    _require(x.dtype in (torch.float32, torch.bfloat16) and x.dim() in (2, 3),
             "x must be float32 or bfloat16, (M, K) or (G, M, K)")
    grouped = x.dim() == 3
    g, m, k = (x.shape if grouped else (1,) + tuple(x.shape))
    kb = -(-k // 128)   # a last K group of k % 128 elements is partial
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if sa is None:
        sa = torch.empty(((g,) if grouped else ()) + (max(kb, 1), dg_get_scale_ld(m)),
                         dtype=torch.float32, device=x.device)
    q = _bytes(q)
    _dev(x, q, sa)
    name = "dg_quantize_per_token_group" + ("_bf16" if x.dtype == torch.bfloat16 else "")
    _check(name, getattr(lib(), name)(_ptr(x), g, m, k, _ptr(q), _ptr(sa), sa.shape[-1], _stream(x)))
    return q, sa


def dg_quantize_per_token_group_bf16(x, q=None, sa=None):
    """bfloat16 x (M, K) or (G, M, K) -> (q, sa): dg_quantize_per_token_group_bf16."""
    _require(x.dtype == torch.bfloat16, "x must be bfloat16")
    return dg_quantize_per_token_group(x, q=q, sa=sa)


def dg_quantize_per_block(w, q=None, sb=None):
    """w float32 (N, K) or (G, N, K) -> (q uint8, sb float32 ([G,] ceil(N/128), K/128))."""
    _require(w.dtype == torch.float32 and w.dim() in (2, 3), "w must be float32 (N, K) or (G, N, K)")
    grouped = w.dim() == 3
    g, n, k = (w.shape if grouped else (1,) + tuple(w.shape))
    nb, kb = -(-n // 128), max(-(-k // 128), 1)
    if q is None:
        q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    if sb is None:
        sb = torch.empty(((g,) if grouped else ()) + (nb, kb), dtype=torch.float32, device=w.device)
    q = _bytes(q)
    _dev(w, q, sb)
    _check("dg_quantize_per_block",
           lib().dg_quantize_per_block(_ptr(w), g, n, k, _ptr(q), _ptr(sb), _stream(w)))
    return q, sb


def dg_quantize_per_channel_group(x, qt=None, st=None):
    """x float32 or bfloat16 (M, K) -> (qt uint8 (K, M), st float32 (ceil(M/128), ld_st)): groups of 128
    consecutive tokens of one column, codes transposed (qt[col, tok] encodes x[tok, col]), scales in
    the activation-scale layout of x^T.  x (G, M, K) -> (qt (G, K, M), st (G, ceil(M/128), ld_st))."""
    _require(x.dtype in (torch.float32, torch.bfloat16) and x.dim() in (2, 3),
             "x must be float32 or bfloat16, (M, K) or (G, M, K)")
    grouped = x.dim() == 3
    g, m, k = (x.shape if grouped else (1,) + tuple(x.shape))
    mb = max(-(-m // 128), 1)
    if qt is None:
        qt = torch.empty(((g,) if grouped else ()) + (k, m), dtype=torch.uint8, device=x.device)
    if st is None:
        st = torch.empty(((g,) if grouped else ()) + (mb, dg_get_scale_ld(k)), dtype=torch.float32, device=x.device)
    qt = _bytes(qt)
    _dev(x, qt, st)
    name = "dg_quantize_per_channel_group" + ("_bf16" if x.dtype == torch.bfloat16 else "")
    _check(name, getattr(lib(), name)(_ptr(x), g, m, k, _ptr(qt), _ptr(st), st.shape[-1], _stream(x)))
    return qt, st


def dg_quantize_per_channel_group_bf16(x, qt=None, st=None):
    """bfloat16 x (M, K) or (G, M, K) -> (qt, st): dg_quantize_per_channel_group_bf16."""
    _require(x.dtype == torch.bfloat16, "x must be bfloat16")
    return dg_quantize_per_channel_group(x, qt=qt, st=st)


def dg_transpose_blocks(q, s, qt=None, st=None):
    """Block-quantized (q uint8 ([G,] R, C), s ([G,] ceil(R/128), ceil(C/128))) -> the same for the
    transposed matrix: (qt ([G,] C, R), st ([G,] ceil(C/128), ceil(R/128)))."""
    q = _bytes(q)
    _require(q.dim() in (2, 3) and s.dim() == q.dim() and s.dtype == torch.float32, "q (R, C) or (G, R, C), s float32")
    grouped = q.dim() == 3
    g, r, c = (q.shape if grouped else (1,) + tuple(q.shape))
    lead = (g,) if grouped else ()
    if qt is None:
        qt = torch.empty(lead + (c, r), dtype=torch.uint8, device=q.device)
    if st is None:
        st = torch.empty(lead + (s.shape[-1], s.shape[-2]), dtype=torch.float32, device=q.device)
    qt = _bytes(qt)
    _dev(q, s, qt, st)
    _check("dg_transpose_blocks", lib().dg_transpose_blocks(_ptr(q), _ptr(s), g, r, c, _ptr(qt), _ptr(st), _stream(q)))
    return qt, st


# ---------------------------------------------------------------------------
# GEMMs
# ---------------------------------------------------------------------------

def dg_gemm_fp8_nt(a, sa, b, sb, d=None, workspace=None, use_workspace=True):
    """D (M, N) bf16 = A (M, K) * B (N, K)^T with fine-grained scales and promoted accumulation."""
    a, b = _bytes(a), _bytes(b)
    m, k = a.shape
    n = b.shape[0]
    if d is None:
        d = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    _dev(a, sa, b, sb, d)
    if workspace is None and use_workspace:
        workspace = default_workspace(a.device, dg_gemm_workspace_size(m, n, k, 1))
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("dg_gemm_fp8_nt",
           lib().dg_gemm_fp8_nt(_ptr(a), _ptr(sa), sa.shape[-1], _ptr(b), _ptr(sb), _ptr(d), m, n, k,
                                _ptr(workspace), ws_bytes, _stream(a)))
    return d


def dg_gemm_fp8_nt_no_alloc(a, sa, b, sb, d):
    """dg_gemm_fp8_nt with the split-K scratch held by the library (no workspace argument; the
    output d (M, N) bf16 must be given: this call allocates nothing)."""
    a, b = _bytes(a), _bytes(b)
    m, k = a.shape
    n = b.shape[0]
    _dev(a, sa, b, sb, d)
    _require(d.dtype == torch.bfloat16 and tuple(d.shape) == (m, n), "d must be bfloat16 (M, N)")
    _check("dg_gemm_fp8_nt_no_alloc",
           lib().dg_gemm_fp8_nt_no_alloc(_ptr(a), _ptr(sa), sa.shape[-1], _ptr(b), _ptr(sb), _ptr(d), m, n, k,
                                         _stream(a)))
    return d


def dg_gemm_fp8_nt_act_quant_workspace_size(m, n, k):
    return int(lib().dg_gemm_fp8_nt_act_quant_workspace_size(int(m), int(n), int(k)))


def dg_gemm_fp8_nt_act_quant(x, b, sb, d=None, workspace=None):
    """D (M, N) bf16 = A (M, K) * B (N, K)^T where (A, sa) is the per-token-group quantization of
    x (float32 or bfloat16 (M, K)), done inside the GEMM launch.  The workspace is required (by
    default a zero-filled one per device); the result is bit-identical to
    dg_quantize_per_token_group(x) followed by dg_gemm_fp8_nt."""
    _require(x.dtype in (torch.float32, torch.bfloat16) and x.dim() == 2, "x must be float32 or bfloat16 (M, K)")
    b = _bytes(b)
    m, k = x.shape
    n = b.shape[0]
    if d is None:
        d = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    _dev(x, b, sb, d)
    if workspace is None:
        workspace = default_workspace(x.device, dg_gemm_fp8_nt_act_quant_workspace_size(m, n, k))
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    name = "dg_gemm_fp8_nt_act_quant" + ("_bf16" if x.dtype == torch.bfloat16 else "")
    _check(name, getattr(lib(), name)(_ptr(x), _ptr(b), _ptr(sb), _ptr(d), m, n, k, _ptr(workspace), ws_bytes,
                                      _stream(x)))
    return d


def dg_gemm_fp8_nt_act_quant_bf16(x, b, sb, d=None, workspace=None):
    """bfloat16 x (M, K): dg_gemm_fp8_nt_act_quant_bf16."""
    _require(x.dtype == torch.bfloat16, "x must be bfloat16")
    return dg_gemm_fp8_nt_act_quant(x, b, sb, d=d, workspace=workspace)


def dg_gemm_fp8_nt_row_scaled(a, sa, b, sb, d=None, workspace=None, use_workspace=True):
    """D (M, N) bf16 = A (M, K) * B (N, K)^T where both operands carry per-row group scales:
    sa (ceil(K/128), ld_sa >= M), sb (ceil(K/128), ld_sb >= N) - e.g. the weight gradient
    dW = dY^T X from dg_quantize_per_channel_group(dY) and dg_quantize_per_channel_group(X)."""
    a, b = _bytes(a), _bytes(b)
    m, k = a.shape
    n = b.shape[0]
    if d is None:
        d = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    _dev(a, sa, b, sb, d)
    if workspace is None and use_workspace:
        workspace = default_workspace(a.device, dg_gemm_workspace_size(m, n, k, 1))
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("dg_gemm_fp8_nt_row_scaled",
           lib().dg_gemm_fp8_nt_row_scaled(_ptr(a), _ptr(sa), sa.shape[-1], _ptr(b), _ptr(sb), sb.shape[-1], _ptr(d),
                                           m, n, k, _ptr(workspace), ws_bytes, _stream(a)))
    return d


def dg_gemm_fp8_k_grouped_row_scaled(a, sa, b, sb, group_tokens, d=None, workspace=None, use_workspace=True):
    """MoE weight gradients: a (M, T) and b (N, T) per-channel-quantized over T tokens in the contiguous
    layout, group_tokens (host sequence of G counts, multiples of 128) -> d bf16 (G, M, N) with
    d[g] = a[:, seg_g] * b[:, seg_g]^T (zeros for an empty expert)."""
    a, b = _bytes(a), _bytes(b)
    m, t = a.shape
    n = b.shape[0]
    counts = [int(c) for c in group_tokens]
    g = len(counts)
    if d is None:
        d = torch.empty((g, m, n), dtype=torch.bfloat16, device=a.device)
    _dev(a, sa, b, sb, d)
    if workspace is None and use_workspace:
        workspace = default_workspace(a.device, max([dg_gemm_workspace_size(m, n, c, 1) for c in counts if c] or [0]))
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    arr = (ctypes.c_int64 * max(g, 1))(*counts)
    _check("dg_gemm_fp8_k_grouped_row_scaled",
           lib().dg_gemm_fp8_k_grouped_row_scaled(_ptr(a), _ptr(sa), sa.shape[-1], _ptr(b), _ptr(sb), sb.shape[-1],
                                                  _ptr(d), arr, g, m, n, t, _ptr(workspace), ws_bytes, _stream(a)))
    return d


def dg_gemm_fp8_grouped_contiguous(a, sa, b, sb, m_indices, d=None):
    """D (M_total, N): row r uses expert m_indices[r] of B (G, N, K)."""
    a, b = _bytes(a), _bytes(b)
    m, k = a.shape
    g, n, _ = b.shape
    if d is None:
        d = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    _require(m_indices.dtype == torch.int32, "m_indices must be int32")
    _dev(a, sa, b, sb, m_indices, d)
    _check("dg_gemm_fp8_grouped_contiguous",
           lib().dg_gemm_fp8_grouped_contiguous(_ptr(a), _ptr(sa), sa.shape[-1], _ptr(b), _ptr(sb),
                                                _ptr(m_indices), g, _ptr(d), m, n, k, _stream(a)))
    return d


def dg_gemm_fp8_grouped_masked(a, sa, b, sb, masked_m, d=None, workspace=None, use_workspace=True):
    """D (G, M_max, N): expert g computes only its first masked_m[g] rows; the rest stay untouched."""
    a, b = _bytes(a), _bytes(b)
    g, m_max, k = a.shape
    n = b.shape[1]
    if d is None:
        d = torch.empty((g, m_max, n), dtype=torch.bfloat16, device=a.device)
    _require(masked_m.dtype == torch.int32, "masked_m must be int32")
    _dev(a, sa, b, sb, masked_m, d)
    if workspace is None and use_workspace:
        workspace = default_workspace(a.device, dg_gemm_workspace_size(m_max, n, k, g))
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("dg_gemm_fp8_grouped_masked",
           lib().dg_gemm_fp8_grouped_masked(_ptr(a), _ptr(sa), sa.shape[-1], _ptr(b), _ptr(sb), _ptr(d),
                                            _ptr(masked_m), g, m_max, n, k, _ptr(workspace), ws_bytes,
                                            _stream(a)))
    return d
