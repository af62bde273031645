"""Boundary conventions on the GPU: the DG_DEBUG checks and plan log, the device diagnostics
word, the bounded wait's give-up report, and the binding's per-stream default workspaces (two
streams' split-K GEMMs run concurrently; a captured graph keeps a workspace that a later, larger
call supersedes)."""

import os

import numpy as np
import pytest
import torch

import fp8_block_scaled_gemm_amd as dg
from fp8_block_scaled_gemm_amd import inputs
import oracle
from gpu_util import bf16_bits, check_gemm, device, sa_to_dev, say, to_dev

pytestmark = pytest.mark.gpu

FQ_SYNC_WORD = (64 * 1024) // 4 - 16   # the in-launch quantization's counters in the counter prefix


class _env:
    """Set environment variables for the duration of a block (the library reads them per call)."""

    def __init__(self, **kv):
        self.kv, self.old = kv, {}

    def __enter__(self):
        for k, v in self.kv.items():
            self.old[k] = os.environ.get(k)
            os.environ[k] = v

    def __exit__(self, *exc):
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _contiguous_operands(g, n, k, m_total):
    rng = inputs.rng_for("boundary_contig", g, n, k, m_total)
    a = inputs.activations_with_outliers(rng, m_total, k)
    b = inputs.normal(rng, (g, n, k), 0.02)
    qa, sa = oracle.quant.quantize_per_token_group(a)
    qb, sb = oracle.quant.quantize_per_block_grouped(b)
    return to_dev(qa), sa_to_dev(sa), to_dev(qb), to_dev(sb), (qa, sa, qb, sb)


def test_debug_contiguous_checks(capfd):
    """DG_DEBUG=1: a 128-row block naming two experts, and a block whose expert is out of range,
    are reported through the diagnostics word (the call itself returns DG_OK and faults nothing);
    a valid layout, a whole -1 block and runs without DG_DEBUG report nothing; the plan is logged."""
    g, n, k, m_total = 3, 256, 256, 512
    say("debug contiguous checks", g, n, k, m_total)
    qa, sa, qb, sb, host = _contiguous_operands(g, n, k, m_total)
    dg.dg_get_debug_status(clear=True)
    valid = np.repeat(np.array([0, 1, -1, 2], np.int32), 128)
    mixed = valid.copy()
    mixed[128 + 72] = 2                      # block 1 names experts 1 and 2
    out_of_range = valid.copy()
    out_of_range[384:512] = 7                # block 3: expert 7 of 3

    def run(m_idx):
        d = torch.full((m_total, n), float("nan"), dtype=torch.bfloat16, device=device())
        dg.dg_gemm_fp8_grouped_contiguous(qa, sa, qb, sb, to_dev(m_idx), d=d)
        return d, dg.dg_get_debug_status(clear=True)

    # without DG_DEBUG nothing is checked or logged
    with _env(DG_DEBUG="0"):
        _, st = run(mixed)
    assert st == (0, -1), st
    capfd.readouterr()
    with _env(DG_DEBUG="1"):
        d, st = run(valid)
        assert st == (0, -1), st
        err = capfd.readouterr().err
        assert "[dg] gemm contiguous m=512 n=256 k=256" in err, err
        # the valid layout's rows are right, and the -1 block is left unwritten
        qa_h, sa_h, qb_h, sb_h = host
        ref = oracle.gemm.gemm_grouped_contiguous(qa_h, sa_h, qb_h, sb_h, np.where(valid < 0, 0, valid))
        rows = np.nonzero(valid >= 0)[0]
        check_gemm(d.float().cpu().numpy()[rows], ref[rows], "debug valid layout")
        assert np.all(bf16_bits(d)[256:384] == bf16_bits(torch.tensor(float("nan"), dtype=torch.bfloat16)))
        _, st = run(mixed)
        assert st == (dg.DG_DIAG_MIXED_BLOCK, 1), st
        _, st = run(out_of_range)
        assert st == (dg.DG_DIAG_EXPERT_RANGE, 3), st
    # the flags were cleared by the last read
    assert dg.dg_get_debug_status(clear=False) == (0, -1)


def test_act_quant_wait_gives_up_and_reports():
    """The in-launch quantization's wait is bounded: a workspace whose chunk counter is not zero
    on entry (a misuse) makes every workgroup give up after the bound, which DG_FQ_MAX_POLLS lowers
    for this test, and the give-up is reported (DG_DIAG_FQ_TIMEOUT).  The kernel still resets its
    counters on exit, so the next call on the same workspace is right again."""
    m, n, k = 64, 512, 1024
    say("act-quant wait give-up", m, n, k)
    dev = device()
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    x = torch.randn((m, k), generator=gen, device=dev)
    qb, sb = dg.dg_quantize_per_block(torch.randn((n, k), generator=gen, device=dev) * 0.02)
    ws = torch.zeros(dg.dg_gemm_fp8_nt_act_quant_workspace_size(m, n, k), dtype=torch.uint8, device=dev)
    ws.view(torch.int32)[FQ_SYNC_WORD] = 1 << 30   # every chunk looks taken: none is ever finished
    dg.dg_get_debug_status(clear=True)
    with _env(DG_FQ_MAX_POLLS="64"):
        dg.dg_gemm_fp8_nt_act_quant(x, qb, sb, workspace=ws)
        flags, _ = dg.dg_get_debug_status(clear=True)
    assert flags & dg.DG_DIAG_FQ_TIMEOUT, flags
    assert int(ws[:64 << 10].count_nonzero()) == 0   # counters reset on exit
    d = dg.dg_gemm_fp8_nt_act_quant(x, qb, sb, workspace=ws)
    qa, sa = dg.dg_quantize_per_token_group(x)
    ref = dg.dg_gemm_fp8_nt(qa, sa, qb, sb, workspace=torch.zeros(dg.dg_gemm_workspace_size(m, n, k) or 1,
                                                                  dtype=torch.uint8, device=dev))
    flags, _ = dg.dg_get_debug_status(clear=True)
    assert flags == 0, flags
    assert np.array_equal(bf16_bits(d), bf16_bits(ref))


def _dense_problem(seed, m, n, k):
    dev = device()
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    qa, sa = dg.dg_quantize_per_token_group(torch.randn((m, k), generator=gen, device=dev))
    qb, sb = dg.dg_quantize_per_block(torch.randn((n, k), generator=gen, device=dev) * 0.02)
    return qa, sa, qb, sb


def test_two_streams_split_k_default_workspaces():
    """Split-K GEMMs on two streams at once, each with the binding's default workspace: every
    stream gets its own, and the outputs equal serial runs bit for bit."""
    shapes = [(64, 2112, 7168), (128, 4096, 7168)]
    for m, n, k in shapes:
        assert not dg.dg_gemm_config_name(0, m, n, k).endswith("/split1"), "the case must split K"
    say("two streams, split-K", shapes, [dg.dg_gemm_config_name(0, *s) for s in shapes])
    probs = [_dense_problem(11 + i, *s) for i, s in enumerate(shapes)]
    torch.cuda.synchronize()
    ref = []
    for (m, n, k), (qa, sa, qb, sb) in zip(shapes, probs):
        ws = torch.zeros(dg.dg_gemm_workspace_size(m, n, k), dtype=torch.uint8, device=device())
        ref.append(dg.dg_gemm_fp8_nt(qa, sa, qb, sb, workspace=ws))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[], []]
    wss = []
    for i, st in enumerate(streams):
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            wss.append(dg.default_workspace(device(), dg.dg_gemm_workspace_size(*shapes[i])))
    assert wss[0].data_ptr() != wss[1].data_ptr()
    for _ in range(6):
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                qa, sa, qb, sb = probs[i]
                outs[i].append(dg.dg_gemm_fp8_nt(qa, sa, qb, sb))
    torch.cuda.synchronize()
    for i in range(2):
        for d in outs[i]:
            assert np.array_equal(bf16_bits(d), bf16_bits(ref[i])), (i, shapes[i])


def test_graph_keeps_superseded_default_workspace():
    """A graph captured with a workspace taken from the default cache keeps working after a larger
    eager call has superseded that workspace (it is kept alive, not freed and reused), and the
    default workspace refuses to be created inside a capture."""
    dev = device()
    small, large = (64, 2112, 4096), (128, 7168, 16384)
    assert dg.dg_gemm_workspace_size(*large) > dg.dg_gemm_workspace_size(*small) > 0
    say("graph with a superseded default workspace", small, large)
    dg._ws_cache.clear()
    qa, sa, qb, sb = _dense_problem(21, *small)
    ws = dg.default_workspace(dev, dg.dg_gemm_workspace_size(*small))
    d = torch.empty((small[0], small[1]), dtype=torch.bfloat16, device=dev)
    dg.dg_gemm_fp8_nt(qa, sa, qb, sb, d=d, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    refused = []
    with torch.cuda.graph(graph):
        try:
            dg.default_workspace(dev, 1 << 10)
        except ValueError as e:
            refused.append(str(e))
        dg.dg_gemm_fp8_nt(qa, sa, qb, sb, d=d, workspace=ws)
    torch.cuda.synchronize()
    assert refused, "default_workspace must refuse during capture"
    # a larger call on the same (device, stream) supersedes the cached buffer
    qa2, sa2, qb2, sb2 = _dense_problem(22, *large)
    dg.dg_gemm_fp8_nt(qa2, sa2, qb2, sb2)
    assert dg.default_workspace(dev, 1).data_ptr() != ws.data_ptr()
    ptr = ws.data_ptr()
    del ws
    # fresh allocations of the same size must not land on the superseded buffer, which stays alive
    junk = [torch.full((dg.dg_gemm_workspace_size(*small),), 0x5A, dtype=torch.uint8, device=dev) for _ in range(4)]
    assert all(j.data_ptr() != ptr for j in junk)
    ref = dg.dg_gemm_fp8_nt(qa, sa, qb, sb,
                            workspace=torch.zeros(dg.dg_gemm_workspace_size(*small), dtype=torch.uint8, device=dev))
    for _ in range(3):
        d.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(d), bf16_bits(ref))
    del junk
