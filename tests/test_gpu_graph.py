"""The path captured in a HIP graph: replays must give the eager results bit for bit.

The split-K arrival counters and the counters of the in-launch activation quantization are
reset by the kernels themselves (no memset node), so a captured step can be replayed any number
of times.  Each replay gets new inputs (copied into the captured buffers), with eager work of
the same library on other buffers and workspaces between the replays.
"""

import numpy as np
import pytest
import torch

import fp8_block_scaled_gemm_amd as dg
from gpu_util import bf16_bits, device, say

pytestmark = pytest.mark.gpu


def step(bufs, out, ws):
    """One pass of the path over the buffers: quantizers, a split-K normal GEMM, a large-tile
    normal GEMM, a split masked GEMM, and the GEMM with the quantization in its launch."""
    qb, sb = dg.dg_quantize_per_block(bufs["w"], q=out["qb"], sb=out["sb"])
    qa, sa = dg.dg_quantize_per_token_group(bufs["x"], q=out["qa"], sa=out["sa"])
    dg.dg_gemm_fp8_nt(qa, sa, qb, sb, d=out["d_dec"], workspace=ws["dec"])
    qa2, sa2 = dg.dg_quantize_per_token_group(bufs["x2"], q=out["qa2"], sa=out["sa2"])
    dg.dg_gemm_fp8_nt(qa2, sa2, qb, sb, d=out["d_big"], workspace=ws["big"])
    qm, sm = dg.dg_quantize_per_token_group(bufs["xm"], q=out["qm"], sa=out["sm"])
    qbm, sbm = dg.dg_quantize_per_block(bufs["wm"], q=out["qbm"], sb=out["sbm"])
    dg.dg_gemm_fp8_grouped_masked(qm, sm, qbm, sbm, bufs["masked_m"], d=out["d_mask"], workspace=ws["mask"])
    dg.dg_gemm_fp8_nt_act_quant(bufs["x"], qb, sb, d=out["d_fq"], workspace=ws["fq"])


def make_out(dev, m, m2, n, k, g, mm, nm):
    ld, ld2, ldm = dg.dg_get_scale_ld(m), dg.dg_get_scale_ld(m2), dg.dg_get_scale_ld(mm)
    e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
    return {"qb": e((n, k), torch.uint8), "sb": e((-(-n // 128), k // 128), torch.float32),
            "qa": e((m, k), torch.uint8), "sa": e((k // 128, ld), torch.float32),
            "qa2": e((m2, k), torch.uint8), "sa2": e((k // 128, ld2), torch.float32),
            "qm": e((g, mm, k), torch.uint8), "sm": e((g, k // 128, ldm), torch.float32),
            "qbm": e((g, nm, k), torch.uint8), "sbm": e((g, -(-nm // 128), k // 128), torch.float32),
            "d_dec": e((m, n), torch.bfloat16), "d_big": e((m2, n), torch.bfloat16),
            "d_mask": torch.full((g, mm, nm), float("nan"), dtype=torch.bfloat16, device=dev),
            "d_fq": e((m, n), torch.bfloat16)}


def make_ws(dev, m, m2, n, k, g, mm, nm):
    z = lambda nbytes: torch.zeros(max(nbytes, 1 << 16), dtype=torch.uint8, device=dev)
    return {"dec": z(dg.dg_gemm_workspace_size(m, n, k)), "big": z(dg.dg_gemm_workspace_size(m2, n, k)),
            "mask": z(dg.dg_gemm_workspace_size(mm, nm, k, g)),
            "fq": z(dg.dg_gemm_fp8_nt_act_quant_workspace_size(m, n, k))}


def test_graph_replays_match_eager():
    dev = device()
    m, m2, n, k = 64, 1024, 2112, 4096
    g, mm, nm = 4, 96, 768
    say("graph capture of the path", dict(m=m, m2=m2, n=n, k=k, g=g, mm=mm, nm=nm),
        dg.dg_gemm_config_name(0, m, n, k), dg.dg_gemm_config_name(2, mm, nm, k, g),
        dg.dg_gemm_config_name(0, m2, n, k))
    gen = torch.Generator(device=dev)

    def inputs(seed):
        gen.manual_seed(seed)
        r = lambda shape, std: torch.randn(shape, generator=gen, device=dev) * std
        return {"w": r((n, k), 0.02), "x": r((m, k), 1.0), "x2": r((m2, k), 1.0), "xm": r((g, mm, k), 1.0),
                "wm": r((g, nm, k), 0.02),
                "masked_m": torch.tensor([mm, 0, 37, 70], dtype=torch.int32, device=dev)}

    bufs = inputs(0)
    out, ws = make_out(dev, m, m2, n, k, g, mm, nm), make_ws(dev, m, m2, n, k, g, mm, nm)
    step(bufs, out, ws)   # warm-up (and the first use of every workspace) before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(bufs, out, ws)
    torch.cuda.synchronize()

    for seed in (1, 2, 3, 4):
        new = inputs(seed)
        for key in bufs:
            bufs[key].copy_(new[key])
        out["d_mask"].fill_(float("nan"))   # rows >= masked_m must stay as the caller left them
        graph.replay()
        torch.cuda.synchronize()
        # the eager reference: separate outputs and workspaces, on the same inputs
        ref_out, ref_ws = make_out(dev, m, m2, n, k, g, mm, nm), make_ws(dev, m, m2, n, k, g, mm, nm)
        step(new, ref_out, ref_ws)
        torch.cuda.synchronize()
        for key in ("qb", "sb", "qa", "sa", "d_dec", "d_big", "d_fq"):
            a, b = out[key], ref_out[key]
            if a.dtype == torch.bfloat16:
                assert np.array_equal(bf16_bits(a), bf16_bits(b)), (seed, key)
            else:
                assert torch.equal(a[..., :m] if key == "sa" else a, b[..., :m] if key == "sa" else b), (seed, key)
        got_mask, ref_mask = bf16_bits(out["d_mask"]), bf16_bits(ref_out["d_mask"])
        assert np.array_equal(got_mask, ref_mask), seed   # written rows equal, unwritten rows both NaN
        for gi, mv in enumerate(new["masked_m"].tolist()):
            assert np.all(got_mask[gi, mv:] == bf16_bits(torch.tensor(float("nan"), dtype=torch.bfloat16))), gi
        # the fused GEMM equals the two-launch GEMM of the same step
        assert np.array_equal(bf16_bits(out["d_fq"]), bf16_bits(out["d_dec"])), seed
        for key in ("dec", "big", "mask", "fq"):
            assert int(ws[key][:64 << 10].count_nonzero()) == 0, (seed, key)
