"""Benchmark of the FP8 block-scaled GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all|dense_v3|small|contiguous|masked|
                     large_dense|zipf|train_v3|train_moe|overlap] [--no-flush] [--no-rotate]
                     [--no-cpu-baseline] [--cpu-seconds S] [--eager]
    python bench.py --copy-calibration      # counter calibration: one plain 1 GiB device copy
    python bench.py --plan-sweep [--out F]  # every few-row plan of the M = 64 / 128 shapes, timed

By default every configuration of the benchmark set runs (small, dense_v3, contiguous,
masked, large_dense, zipf); dense_v3 - the DeepSeek-V3 dense shapes at M in {64, 128, 4096} -
gives the headline fields, and every configuration gets its own entry under "configs".

One step is one pass of the whole hot path over one batch of synthetic input:
weight quantization (128x128 blocks) of every weight matrix of the workload,
then, per GEMM shape, activation quantization (1x128 groups) followed by the
FP8 GEMM with promoted accumulation - every kernel of the library, in the order
a forward pass runs them.  Inputs are resident in HBM before timing.

Timing, two passes per workload:
  * the step: captured once as a HIP graph; the timed region is K graph replays on one
    stream, bracketed by device synchronisation.  This gives `value` and `ms_per_step`.
  * per launch: for each kernel of the step, an untimed 512 MB write first evicts the
    256 MB last-level cache (MALL), then one HIP event pair on the launch stream brackets R
    launches over R distinct copies of the weights (R copies > 768 MB, so no launch reads
    weights another left in the cache); duration = time / R, median over K steps.  This is
    the cold-weight duration a forward pass sees, and it amortises the event pair's own
    few microseconds over R launches.  --no-flush / --no-rotate switch either off.  A short
    device spin (--spin-ms, 0.2 ms) opens each timing pass so the host's enqueue stays ahead;
    a long one leaves the device nearly idle, and the MFMA-bound launches after it run slower
    (16384 x 7168 x 16384: 1633 us after 0.2 ms, 1707 after 2 ms, 1873 after 20 ms), which a
    loop of back-to-back kernels never sees.

Prints ONE JSON line: the workload's GEMM FP8 TFLOP/s over the whole step, plus
per-shape GEMM TFLOP/s and HBM GB/s, the roofline of the dominant GEMM kernel
(with the HBM traffic that rocprofv3 counters measured for it, when the committed
counter summary matches the kernel source) and the CPU oracle's throughput on a
bounded sample of the same workload.

The train_v3 workload is a linear layer's training step per DeepSeek-V3 (N, K) at 4096 tokens:
forward, dgrad (dY W through the transposed weight blocks) and wgrad (dY^T X from per-channel
token groups, the row-scaled GEMM), with every quantizer and the transpose inside the step.

Workloads: DeepSeek-V3/R1 inference shapes (prefill and decode, no tensor
parallelism - the pages' own benchmark set, 机器之心 DeepGEMM report,
"performance") are not a public dataset; seeded synthetic inputs of those
shapes stand in for them.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 TFLOPS + HBM GB/s per GEMM shape on 1 MI355X (roofline fraction)"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    choices=["all", "dense_v3", "small", "contiguous", "masked", "large_dense", "zipf", "train_v3",
                             "train_moe", "overlap"],
                    help="all (default): every configuration of the benchmark set, dense_v3 as the headline")
    ap.add_argument("--no-flush", action="store_true", help="no 512 MB write ahead of each timed GEMM")
    ap.add_argument("--no-rotate", action="store_true", help="time each GEMM once per step, on its own weights")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU work of the oracle sample")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--num-cus", type=int, default=0,
                    help="cap the GEMMs' persistent grid to this many CUs (dg_set_num_cus; 0 = all)")
    ap.add_argument("--act-dtype", default="fp32", choices=["fp32", "bf16"],
                    help="activation input type of the dense workloads (bf16: the bf16-input quantizer)")
    ap.add_argument("--act-quant", default="separate", choices=["separate", "fused", "auto"],
                    help="dense workloads: activation quantization as its own launch (separate), inside the "
                         "GEMM launch (fused: dg_gemm_fp8_nt_act_quant), or inside it for M <= 128 only (auto)")
    ap.add_argument("--spin-ms", type=float, default=0.2,
                    help="device spin before each per-kernel timing pass (gives the host's enqueue a head start; "
                         "kept short: a long idle spin slows the MFMA-bound launches after it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--plan-sweep", action="store_true",
                    help="only time every few-row plan (tile x K split) of the M = 64 / 128 DeepSeek-V3 shapes")
    ap.add_argument("--out", default="", help="--plan-sweep: also write the markdown table here")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# GPU-side seeded input generation (fp8_block_scaled_gemm_amd.inputs.DeviceGen: the same recipes,
# drawn on the device so that multi-GB workloads are ready in seconds)
# ---------------------------------------------------------------------------

def Gen(torch, dev, seed):
    from fp8_block_scaled_gemm_amd.inputs import DeviceGen
    return DeviceGen(torch, dev, seed)


# ---------------------------------------------------------------------------
# ops of one step
# ---------------------------------------------------------------------------

class Op:
    """One launch of the step.  A GEMM op may name its weight tensor (`weights`) and a function
    launching it on any tensor of that shape (`make`): the per-kernel timing then runs it over
    rotated copies of the weights, so that no launch finds its weights in the 256 MB MALL."""

    def __init__(self, kind, label, launch, flops=0.0, nbytes=0.0, config="", weights=None, make=None):
        self.kind, self.label, self.launch = kind, label, launch
        self.flops, self.nbytes, self.config = float(flops), float(nbytes), config
        self.weights, self.make = weights, make
        self.copies = None
        self.rot = 1      # launches per timed event pair (weight copies)
        self.times = []   # ms per launch, one entry per timed step


def dense_gemm_bytes(m, n, k):
    """Algorithmic HBM bytes of one dense GEMM: A + its scales, B + its scales, bf16 D."""
    kb = -(-k // 128)
    return m * k + 4 * m * kb + n * k + 4 * (-(-n // 128)) * kb + 2 * m * n


def contiguous_gemm_bytes(m_total, n, k, groups):
    """Algorithmic HBM bytes of one contiguous-grouped GEMM: the padded rows of A + their scales,
    every expert's B + its scales, the padded rows of bf16 D, and the int32 expert index per row."""
    kb = -(-k // 128)
    return (m_total * k + 4 * m_total * kb + groups * (n * k + 4 * (-(-n // 128)) * kb)
            + 2 * m_total * n + 4 * m_total)


def masked_gemm_bytes(masked_m, m_max, n, k):
    """Algorithmic HBM bytes of one masked-grouped GEMM: B + its scales of every expert with rows,
    each valid row's A (k bytes), its scales (k/32 bytes) and its bf16 D row, and the counts."""
    masked_m = np.asarray(masked_m)
    rows = int(np.sum(np.clip(masked_m, 0, m_max)))
    active = int(np.sum(masked_m > 0))
    kb = -(-k // 128)
    return active * (n * k + 4 * (-(-n // 128)) * kb) + rows * (k + 4 * kb + 2 * n) + 4 * len(masked_m)


def quant_bytes(elems, k, in_bytes=4):
    """input read (fp32 or bf16) + E4M3 write + one fp32 scale per 128 elements."""
    return in_bytes * elems + elems + 4 * elems // 128


def fused_gemm_bytes(m, n, k, in_bytes):
    """Algorithmic HBM bytes of the GEMM that quantizes its activations in the launch: the
    unquantized activations, B + its scales, bf16 D."""
    return in_bytes * m * k + n * k + 4 * (-(-n // 128)) * (k // 128) + 2 * m * n


def kernel_config(config):
    """Kernel instance of a GEMM configuration name: the tile (the K split is a launch parameter
    of the same kernel), and whether the activation quantization runs in the launch."""
    return config.split("/split")[0] + (" +act-quant" if config.endswith("+act-quant") else "")


def build_dense(torch, dg, dev, shapes, name, act_dtype="fp32", act_quant="separate"):
    """Ops for a list of dense (M, N, K) shapes sharing weights per (N, K).  act_dtype "bf16": the
    activations arrive in bf16 and go through the bf16-input quantizer.  act_quant: "separate" =
    a quantizer launch then the GEMM; "fused" = dg_gemm_fp8_nt_act_quant (quantization inside the
    GEMM launch) for every shape; "auto" = fused for M <= 128, separate otherwise."""
    gen = Gen(torch, dev, 1234)
    ops = []
    weights = {}
    for (m, n, k) in shapes:
        if (n, k) not in weights:
            w32 = gen.normal((n, k), 0.02)
            qb = torch.empty((n, k), dtype=torch.uint8, device=dev)
            sb = torch.empty((-(-n // 128), k // 128), dtype=torch.float32, device=dev)
            weights[(n, k)] = (w32, qb, sb)
            ops.append(Op("wquant", f"wq {n}x{k}",
                          (lambda w32=w32, qb=qb, sb=sb: dg.dg_quantize_per_block(w32, q=qb, sb=sb)),
                          nbytes=quant_bytes(n * k, k)))
    in_bytes = 2 if act_dtype == "bf16" else 4
    for (m, n, k) in shapes:
        w32, qb, sb = weights[(n, k)]
        a32 = gen.activations(m, k)
        if act_dtype == "bf16":
            a32 = a32.to(torch.bfloat16)
        if act_quant == "fused" or (act_quant == "auto" and m <= 128):
            d = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            ws = dg.default_workspace(dev, dg.dg_gemm_fp8_nt_act_quant_workspace_size(m, n, k))
            ops.append(Op("gemm", f"{m}x{n}x{k}",
                          (lambda a32=a32, qb=qb, sb=sb, d=d, ws=ws: dg.dg_gemm_fp8_nt_act_quant(a32, qb, sb, d=d,
                                                                                                  workspace=ws)),
                          flops=2.0 * m * n * k, nbytes=fused_gemm_bytes(m, n, k, in_bytes),
                          config=dg.dg_gemm_config_name(0, m, n, k, 1) + " +act-quant"))
            continue
        qa = torch.empty((m, k), dtype=torch.uint8, device=dev)
        sa = torch.empty((k // 128, dg.dg_get_scale_ld(m)), dtype=torch.float32, device=dev)
        d = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        ws = dg.default_workspace(dev, dg.dg_gemm_workspace_size(m, n, k, 1))
        ops.append(Op("aquant", f"aq {m}x{k}",
                      (lambda a32=a32, qa=qa, sa=sa: dg.dg_quantize_per_token_group(a32, q=qa, sa=sa)),
                      nbytes=quant_bytes(m * k, k, in_bytes)))
        make = (lambda w, qa=qa, sa=sa, sb=sb, d=d, ws=ws: dg.dg_gemm_fp8_nt(qa, sa, w, sb, d=d, workspace=ws))
        ops.append(Op("gemm", f"{m}x{n}x{k}", (lambda make=make, qb=qb: make(qb)),
                      flops=2.0 * m * n * k, nbytes=dense_gemm_bytes(m, n, k),
                      config=dg.dg_gemm_config_name(0, m, n, k, 1), weights=qb, make=make))
    return ops


def rowscaled_gemm_bytes(m, n, k):
    """Algorithmic HBM bytes of one row-scaled GEMM: A + per-row scales, B + per-row scales, bf16 D."""
    kb = -(-k // 128)
    return m * k + 4 * m * kb + n * k + 4 * n * kb + 2 * m * n


def build_train(torch, dg, dev, m, nk_list):
    """A linear layer's training step per (N, K) at m tokens: forward Y = X W^T, dgrad dX = dY W (dY in
    per-token groups, W^T from W's transposed blocks), wgrad dW = dY^T X (both in per-channel token
    groups, row-scaled GEMM).  Every quantizer and the block transpose run inside the step."""
    gen = Gen(torch, dev, 4321)
    ops = []
    u8, f32 = torch.uint8, torch.float32
    for (n, k) in nk_list:
        w32 = gen.normal((n, k), 0.02)
        x32 = gen.activations(m, k)
        dy32 = gen.normal((m, n), 1e-2)
        qw = torch.empty((n, k), dtype=u8, device=dev)
        sw = torch.empty((-(-n // 128), -(-k // 128)), dtype=f32, device=dev)
        qwt = torch.empty((k, n), dtype=u8, device=dev)
        swt = torch.empty((-(-k // 128), -(-n // 128)), dtype=f32, device=dev)
        qx = torch.empty((m, k), dtype=u8, device=dev)
        sx = torch.empty((-(-k // 128), dg.dg_get_scale_ld(m)), dtype=f32, device=dev)
        qdy = torch.empty((m, n), dtype=u8, device=dev)
        sdy = torch.empty((-(-n // 128), dg.dg_get_scale_ld(m)), dtype=f32, device=dev)
        qdyt = torch.empty((n, m), dtype=u8, device=dev)
        sdyt = torch.empty((-(-m // 128), dg.dg_get_scale_ld(n)), dtype=f32, device=dev)
        qxt = torch.empty((k, m), dtype=u8, device=dev)
        sxt = torch.empty((-(-m // 128), dg.dg_get_scale_ld(k)), dtype=f32, device=dev)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        dx = torch.empty((m, k), dtype=torch.bfloat16, device=dev)
        dw = torch.empty((n, k), dtype=torch.bfloat16, device=dev)
        ws = dg.default_workspace(dev, max(dg.dg_gemm_workspace_size(m, n, k, 1), dg.dg_gemm_workspace_size(m, k, n, 1),
                                           dg.dg_gemm_workspace_size(n, k, m, 1)))
        ops.append(Op("wquant", f"wq {n}x{k}", lambda w32=w32, qw=qw, sw=sw: dg.dg_quantize_per_block(w32, q=qw, sb=sw),
                      nbytes=quant_bytes(n * k, k)))
        ops.append(Op("transpose", f"wT {n}x{k}",
                      lambda qw=qw, sw=sw, qwt=qwt, swt=swt: dg.dg_transpose_blocks(qw, sw, qt=qwt, st=swt),
                      nbytes=2 * n * k))
        ops.append(Op("aquant", f"aq X {m}x{k}", lambda x32=x32, qx=qx, sx=sx: dg.dg_quantize_per_token_group(x32, q=qx, sa=sx),
                      nbytes=quant_bytes(m * k, k)))
        ops.append(Op("gemm", f"fwd {m}x{n}x{k}",
                      lambda qx=qx, sx=sx, qw=qw, sw=sw, y=y, ws=ws: dg.dg_gemm_fp8_nt(qx, sx, qw, sw, d=y, workspace=ws),
                      flops=2.0 * m * n * k, nbytes=dense_gemm_bytes(m, n, k), config=dg.dg_gemm_config_name(0, m, n, k, 1)))
        ops.append(Op("aquant", f"aq dY {m}x{n}", lambda dy32=dy32, qdy=qdy, sdy=sdy: dg.dg_quantize_per_token_group(dy32, q=qdy, sa=sdy),
                      nbytes=quant_bytes(m * n, n)))
        ops.append(Op("gemm", f"dgrad {m}x{k}x{n}",
                      lambda qdy=qdy, sdy=sdy, qwt=qwt, swt=swt, dx=dx, ws=ws: dg.dg_gemm_fp8_nt(qdy, sdy, qwt, swt, d=dx, workspace=ws),
                      flops=2.0 * m * n * k, nbytes=dense_gemm_bytes(m, k, n), config=dg.dg_gemm_config_name(0, m, k, n, 1)))
        ops.append(Op("cquant", f"cq dY {m}x{n}",
                      lambda dy32=dy32, qdyt=qdyt, sdyt=sdyt: dg.dg_quantize_per_channel_group(dy32, qt=qdyt, st=sdyt),
                      nbytes=quant_bytes(m * n, m)))
        ops.append(Op("cquant", f"cq X {m}x{k}",
                      lambda x32=x32, qxt=qxt, sxt=sxt: dg.dg_quantize_per_channel_group(x32, qt=qxt, st=sxt),
                      nbytes=quant_bytes(m * k, m)))
        ops.append(Op("gemm", f"wgrad {n}x{k}x{m}",
                      lambda qdyt=qdyt, sdyt=sdyt, qxt=qxt, sxt=sxt, dw=dw, ws=ws: dg.dg_gemm_fp8_nt_row_scaled(
                          qdyt, sdyt, qxt, sxt, d=dw, workspace=ws),
                      flops=2.0 * m * n * k, nbytes=rowscaled_gemm_bytes(n, k, m),
                      config="rowscaled " + dg.dg_gemm_config_name(3, n, k, m, 1)))
    return ops


def build_contiguous(torch, dg, dev, cases):
    """cases: list of (label, sizes (np int array), n, k)."""
    from fp8_block_scaled_gemm_amd import inputs
    gen = Gen(torch, dev, 4321)
    ops = []
    for label, sizes, n, k in cases:
        g = len(sizes)
        m_idx_np, starts, valid_np = inputs.contiguous_layout(sizes)
        m_total = m_idx_np.shape[0]
        w32 = gen.normal((g, n, k), 0.02)
        qb = torch.empty((g, n, k), dtype=torch.uint8, device=dev)
        sb = torch.empty((g, -(-n // 128), k // 128), dtype=torch.float32, device=dev)
        a32 = gen.activations(m_total, k) * torch.from_numpy(valid_np).to(dev).float()[:, None]
        qa = torch.empty((m_total, k), dtype=torch.uint8, device=dev)
        sa = torch.empty((k // 128, dg.dg_get_scale_ld(m_total)), dtype=torch.float32, device=dev)
        d = torch.empty((m_total, n), dtype=torch.bfloat16, device=dev)
        m_idx = torch.from_numpy(m_idx_np).to(dev)
        rows = int(np.sum(sizes))
        ops.append(Op("wquant", f"wq {g}x{n}x{k}",
                      (lambda w32=w32, qb=qb, sb=sb: dg.dg_quantize_per_block(w32, q=qb, sb=sb)),
                      nbytes=quant_bytes(g * n * k, k)))
        ops.append(Op("aquant", f"aq {m_total}x{k}",
                      (lambda a32=a32, qa=qa, sa=sa: dg.dg_quantize_per_token_group(a32, q=qa, sa=sa)),
                      nbytes=quant_bytes(m_total * k, k)))
        nbytes = contiguous_gemm_bytes(m_total, n, k, g)
        make = (lambda w, qa=qa, sa=sa, sb=sb, m_idx=m_idx, d=d:
                dg.dg_gemm_fp8_grouped_contiguous(qa, sa, w, sb, m_idx, d=d))
        ops.append(Op("gemm", f"{label} G={g} rows={rows} (padded {m_total}) N={n} K={k}",
                      (lambda make=make, qb=qb: make(qb)),
                      flops=2.0 * rows * n * k, nbytes=nbytes,
                      config=dg.dg_gemm_config_name(1, m_total, n, k, g), weights=qb, make=make))
    return ops


def build_train_moe(torch, dg, dev, cases):
    """MoE layer training step over the contiguous layout, per case (sizes, n, k): forward (contiguous
    GEMM), dgrad (contiguous GEMM on the experts' transposed weight blocks) and wgrad (per-channel
    quantization of the whole dY and X, then the k-grouped row-scaled GEMM per expert)."""
    from fp8_block_scaled_gemm_amd import inputs
    gen = Gen(torch, dev, 5678)
    ops = []
    u8, f32 = torch.uint8, torch.float32
    for sizes, n, k in cases:
        g = len(sizes)
        m_idx_np, starts, valid_np = inputs.contiguous_layout(sizes)
        m_total = m_idx_np.shape[0]
        padded = [int(c) for c in np.diff(np.append(starts, m_total))]
        rows = int(np.sum(sizes))
        valid = torch.from_numpy(valid_np).to(dev).float()[:, None]
        w32 = gen.normal((g, n, k), 0.02)
        x32 = gen.activations(m_total, k) * valid
        dy32 = gen.normal((m_total, n), 1e-2) * valid
        m_idx = torch.from_numpy(m_idx_np).to(dev)
        qw = torch.empty((g, n, k), dtype=u8, device=dev)
        sw = torch.empty((g, -(-n // 128), -(-k // 128)), dtype=f32, device=dev)
        qwt = torch.empty((g, k, n), dtype=u8, device=dev)
        swt = torch.empty((g, -(-k // 128), -(-n // 128)), dtype=f32, device=dev)
        qx = torch.empty((m_total, k), dtype=u8, device=dev)
        sx = torch.empty((-(-k // 128), dg.dg_get_scale_ld(m_total)), dtype=f32, device=dev)
        qdy = torch.empty((m_total, n), dtype=u8, device=dev)
        sdy = torch.empty((-(-n // 128), dg.dg_get_scale_ld(m_total)), dtype=f32, device=dev)
        qdyt = torch.empty((n, m_total), dtype=u8, device=dev)
        sdyt = torch.empty((m_total // 128, dg.dg_get_scale_ld(n)), dtype=f32, device=dev)
        qxt = torch.empty((k, m_total), dtype=u8, device=dev)
        sxt = torch.empty((m_total // 128, dg.dg_get_scale_ld(k)), dtype=f32, device=dev)
        y = torch.empty((m_total, n), dtype=torch.bfloat16, device=dev)
        dx = torch.empty((m_total, k), dtype=torch.bfloat16, device=dev)
        dw = torch.empty((g, n, k), dtype=torch.bfloat16, device=dev)
        ws = dg.default_workspace(dev, max([dg.dg_gemm_workspace_size(n, k, c, 1) for c in padded if c] or [0]))
        tag = f"G={g} rows={rows} N={n} K={k}"
        ops.append(Op("wquant", f"wq {g}x{n}x{k}", lambda w32=w32, qw=qw, sw=sw: dg.dg_quantize_per_block(w32, q=qw, sb=sw),
                      nbytes=quant_bytes(g * n * k, k)))
        ops.append(Op("transpose", f"wT {g}x{n}x{k}",
                      lambda qw=qw, sw=sw, qwt=qwt, swt=swt: dg.dg_transpose_blocks(qw, sw, qt=qwt, st=swt),
                      nbytes=2 * g * n * k))
        ops.append(Op("aquant", f"aq X {m_total}x{k}", lambda x32=x32, qx=qx, sx=sx: dg.dg_quantize_per_token_group(x32, q=qx, sa=sx),
                      nbytes=quant_bytes(m_total * k, k)))
        ops.append(Op("gemm", f"fwd {tag}",
                      lambda qx=qx, sx=sx, qw=qw, sw=sw, m_idx=m_idx, y=y: dg.dg_gemm_fp8_grouped_contiguous(qx, sx, qw, sw, m_idx, d=y),
                      flops=2.0 * rows * n * k,
                      nbytes=m_total * k + g * n * k + 2 * m_total * n + 4 * m_total * (k // 128) + 4 * m_total,
                      config=dg.dg_gemm_config_name(1, m_total, n, k, g)))
        ops.append(Op("aquant", f"aq dY {m_total}x{n}", lambda dy32=dy32, qdy=qdy, sdy=sdy: dg.dg_quantize_per_token_group(dy32, q=qdy, sa=sdy),
                      nbytes=quant_bytes(m_total * n, n)))
        ops.append(Op("gemm", f"dgrad {tag}",
                      lambda qdy=qdy, sdy=sdy, qwt=qwt, swt=swt, m_idx=m_idx, dx=dx: dg.dg_gemm_fp8_grouped_contiguous(
                          qdy, sdy, qwt, swt, m_idx, d=dx),
                      flops=2.0 * rows * n * k,
                      nbytes=m_total * n + g * n * k + 2 * m_total * k + 4 * m_total * (n // 128) + 4 * m_total,
                      config=dg.dg_gemm_config_name(1, m_total, k, n, g)))
        ops.append(Op("cquant", f"cq dY {m_total}x{n}",
                      lambda dy32=dy32, qdyt=qdyt, sdyt=sdyt: dg.dg_quantize_per_channel_group(dy32, qt=qdyt, st=sdyt),
                      nbytes=quant_bytes(m_total * n, m_total)))
        ops.append(Op("cquant", f"cq X {m_total}x{k}",
                      lambda x32=x32, qxt=qxt, sxt=sxt: dg.dg_quantize_per_channel_group(x32, qt=qxt, st=sxt),
                      nbytes=quant_bytes(m_total * k, m_total)))
        ops.append(Op("gemm", f"wgrad {tag}",
                      lambda qdyt=qdyt, sdyt=sdyt, qxt=qxt, sxt=sxt, dw=dw, ws=ws, padded=padded:
                      dg.dg_gemm_fp8_k_grouped_row_scaled(qdyt, sdyt, qxt, sxt, padded, d=dw, workspace=ws),
                      flops=2.0 * rows * n * k,
                      nbytes=(n + k) * m_total + 4 * (n + k) * (m_total // 128) + 2 * g * n * k,
                      config="kgrouped " + dg.dg_gemm_config_name(3, n, k, max(padded), 1)))
    return ops


def build_masked(torch, dg, dev, cases):
    """cases: list of (masked_m np int32 array, m_max, n, k)."""
    gen = Gen(torch, dev, 999)
    ops = []
    for masked_np, m_max, n, k in cases:
        g = len(masked_np)
        w32 = gen.normal((g, n, k), 0.02)
        qb = torch.empty((g, n, k), dtype=torch.uint8, device=dev)
        sb = torch.empty((g, -(-n // 128), k // 128), dtype=torch.float32, device=dev)
        a32 = gen.activations(g * m_max, k).reshape(g, m_max, k)
        qa = torch.empty((g, m_max, k), dtype=torch.uint8, device=dev)
        sa = torch.empty((g, k // 128, dg.dg_get_scale_ld(m_max)), dtype=torch.float32, device=dev)
        d = torch.empty((g, m_max, n), dtype=torch.bfloat16, device=dev)
        masked = torch.from_numpy(masked_np.astype(np.int32)).to(dev)
        ws = dg.default_workspace(dev, dg.dg_gemm_workspace_size(m_max, n, k, g))
        rows = int(np.sum(np.clip(masked_np, 0, m_max)))
        ops.append(Op("wquant", f"wq {g}x{n}x{k}",
                      (lambda w32=w32, qb=qb, sb=sb: dg.dg_quantize_per_block(w32, q=qb, sb=sb)),
                      nbytes=quant_bytes(g * n * k, k)))
        ops.append(Op("aquant", f"aq {g}x{m_max}x{k}",
                      (lambda a32=a32, qa=qa, sa=sa: dg.dg_quantize_per_token_group(a32, q=qa, sa=sa)),
                      nbytes=quant_bytes(g * m_max * k, k)))
        nbytes = masked_gemm_bytes(masked_np, m_max, n, k)
        make = (lambda w, qa=qa, sa=sa, sb=sb, d=d, masked=masked, ws=ws:
                dg.dg_gemm_fp8_grouped_masked(qa, sa, w, sb, masked, d=d, workspace=ws))
        ops.append(Op("gemm", f"masked G={g} rows={rows} M_max={m_max} N={n} K={k}",
                      (lambda make=make, qb=qb: make(qb)),
                      flops=2.0 * rows * n * k, nbytes=nbytes,
                      config=dg.dg_gemm_config_name(2, m_max, n, k, g), weights=qb, make=make))
    return ops


def build_workload(name, torch, dg, dev, act_dtype="fp32", act_quant="separate"):
    from fp8_block_scaled_gemm_amd import inputs
    if act_dtype != "fp32" and name not in ("dense_v3", "small", "large_dense"):
        raise SystemExit(f"bench.py: --act-dtype {act_dtype} applies to the dense workloads only")
    if act_quant != "separate" and name not in ("dense_v3", "small", "large_dense"):
        raise SystemExit(f"bench.py: --act-quant {act_quant} applies to the dense workloads only")
    if name == "dense_v3":
        # decode shapes first, then prefill, then the second decode size: the weights read by the two
        # decode passes are separated by > 1 GB of traffic, so neither pass is served by the 256 MB MALL
        order = [64, 4096, 128]
        shapes = [(m, n, k) for m in order for (n, k) in inputs.DENSE_V3_NK]
        desc = ("DeepSeek-V3 dense GEMMs: M in {64,128,4096} x (N,K) in {(2112,7168),(24576,1536),"
                "(32768,512),(7168,16384),(4096,7168),(7168,2048)}; A~N(0,1) with 1% rows x100, B~N(0,0.02^2)")
        return build_dense(torch, dg, dev, shapes, name, act_dtype, act_quant), desc
    if name == "train_v3":
        return (build_train(torch, dg, dev, 4096, inputs.DENSE_V3_NK),
                "linear-layer training step at 4096 tokens for each DeepSeek-V3 (N,K) in {(2112,7168),(24576,1536),"
                "(32768,512),(7168,16384),(4096,7168),(7168,2048)}: forward X W^T, dgrad dY W, wgrad dY^T X; "
                "X~N(0,1) with 1% rows x100, W~N(0,0.02^2), dY~N(0,0.01^2)")
    if name == "train_moe":
        sizes = inputs.uniform_group_sizes(inputs.rng_for("contiguous", 8), 8)
        return (build_train_moe(torch, dg, dev, [(sizes, n, k) for (n, k) in inputs.GROUPED_NK]),
                "MoE layer training step over the contiguous layout: G=8, ~8192 tokens/expert (+-25%) padded to 128, "
                "(N,K) in {(4096,7168),(7168,2048)}: forward, dgrad (transposed expert blocks), wgrad (k-grouped)")
    if name == "small":
        return build_dense(torch, dg, dev, [(128, 512, 512)], name, act_dtype, act_quant), "M=128, N=512, K=512"
    if name == "large_dense":
        return (build_dense(torch, dg, dev, [(16384, 7168, 16384)], name, act_dtype, act_quant),
                "dense prefill M=16384, N=7168, K=16384")
    if name == "contiguous":
        cases = []
        for g in (4, 8):
            sizes = inputs.uniform_group_sizes(inputs.rng_for("contiguous", g), g)
            for (n, k) in inputs.GROUPED_NK:
                cases.append(("contiguous", sizes, n, k))
        return (build_contiguous(torch, dg, dev, cases),
                "contiguous-grouped MoE: G in {4,8}, ~8192 rows/expert (+-25%) padded to 128, (N,K) in "
                "{(4096,7168),(7168,2048)}")
    if name == "zipf":
        sizes = inputs.zipf_group_sizes(inputs.rng_for("zipf"))
        return (build_contiguous(torch, dg, dev, [("zipf", sizes, 2048, 7168)]),
                "contiguous-grouped MoE: G=64, 32768 routed rows, Zipf(1.1) sizes padded to 128, N=2048, K=7168")
    if name == "masked":
        masked = inputs.masked_counts(inputs.rng_for("masked"))
        cases = [(masked, 256, n, k) for (n, k) in inputs.GROUPED_NK]
        return (build_masked(torch, dg, dev, cases),
                "masked-grouped MoE decode: G=32, 256-row buffers, masked_m ~ U{0..256}, (N,K) in "
                "{(4096,7168),(7168,2048)}")
    raise ValueError(name)


# ---------------------------------------------------------------------------
# CPU oracle baseline on a bounded sample
# ---------------------------------------------------------------------------

def cpu_baseline(workload, seconds):
    import oracle
    from fp8_block_scaled_gemm_amd import inputs
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    # sample: for each (N, K) of the dense V3 set, 128 activation rows x `rows_b` weight rows through
    # the whole oracle path (quantize A rows, quantize B rows, fp64 GEMM); rows_b scaled to the budget
    nk = (inputs.DENSE_V3_NK if workload in ("dense_v3", "train_v3") else
          inputs.GROUPED_NK if workload == "train_moe" else [(512, 512)])
    train = workload in ("train_v3", "train_moe")
    rng = inputs.rng_for("cpu_sample")

    def run(rows_b):
        flops, t, per_shape = 0.0, 0.0, []
        for (n, k) in nk:
            a = inputs.activations_with_outliers(rng, 128, k)
            b = inputs.normal(rng, (min(rows_b, n), k), 0.02)
            t0 = time.perf_counter()
            if train:   # forward, dgrad and wgrad of the sampled slice through the oracle
                dy = inputs.normal(rng, (a.shape[0], b.shape[0]), 1e-2)
                t0 = time.perf_counter()
                oracle.train.linear_forward(a, b)
                oracle.train.linear_dgrad(dy, b)
                oracle.train.linear_wgrad(dy, a)
                flops += 3 * 2.0 * a.shape[0] * b.shape[0] * k
            else:
                qa, sa = oracle.quant.quantize_per_token_group(a)
                qb, sb = oracle.quant.quantize_per_block(b)
                oracle.gemm.gemm_nt(qa, sa, qb, sb)
                flops += 2.0 * a.shape[0] * b.shape[0] * k
            per_shape.append(time.perf_counter() - t0)
            t += per_shape[-1]
        return flops, t, per_shape

    # calibration: each shape's time at 128 and 384 weight rows, as a fixed part (the activation
    # rows) plus a part per weight row
    _, _, c1 = run(128)
    _, _, c3 = run(384)
    per_row = [max((b - a) / 256, 1e-9) for a, b in zip(c1, c3)]
    fixed = [max(a - 128 * r, 0.0) for a, r in zip(c1, per_row)]
    max_n = max(n for (n, _) in nk)

    def predicted(rows):                  # the sample rows of a shape are capped at its N
        return sum(f + r * min(rows, n) for f, r, (n, _) in zip(fixed, per_row, nk))

    rows_b = 128
    while rows_b < max_n and predicted(rows_b + 128) <= seconds:
        rows_b += 128
    f, t, _ = run(rows_b)
    return {"value": f / t / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": ((f"oracle forward + dgrad + wgrad of 128 tokens x {rows_b} weight rows for each (N,K) "
                        if train else
                        f"oracle quantize + fp64 GEMM of 128 activation rows x {rows_b} weight rows for each (N,K) ")
                       + f"of the workload ({f / 1e9:.2f} GFLOP in {t:.1f} s; quantization single-threaded numpy, "
                       f"GEMM on {blas_threads} BLAS threads)"),
            "seconds": t}


# ---------------------------------------------------------------------------

def cu_masked_stream(torch, first, count, total):
    """A HIP stream whose kernels may only run on CUs [first, first + count) (hipExtStreamCreateWithCUMask;
    default priority), wrapped for torch."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    words = (total + 31) // 32
    mask = [0] * words
    for cu in range(first, first + count):
        mask[cu // 32] |= 1 << (cu % 32)
    arr = (ctypes.c_uint32 * words)(*mask)
    handle = ctypes.c_void_p()
    err = hip.hipExtStreamCreateWithCUMask(ctypes.byref(handle), ctypes.c_uint32(words), arr)
    if err != 0:
        raise RuntimeError(f"hipExtStreamCreateWithCUMask failed ({err})")
    return torch.cuda.ExternalStream(handle.value, device=torch.device("cuda", 0))


def overlap_bench(args, torch, dg, dev):
    """Comm-overlap mode (the CU cap beside a communication kernel, on one GPU): the prefill GEMM
    4096 x 7168 x 16384 runs on a stream masked to the first C CUs with its persistent grid capped
    to C (dg_set_num_cus), while a device copy standing in for an all-to-all runs on a stream
    masked to the remaining CUs.  Times each alone and both together."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    c = args.num_cus if args.num_cus > 0 else cus - 32
    dg.dg_set_num_cus(c)
    m, n, k = 4096, 7168, 16384
    gen = Gen(torch, dev, 77)
    qa, sa = dg.dg_quantize_per_token_group(gen.activations(m, k))
    qb, sb = dg.dg_quantize_per_block(gen.normal((n, k), 0.02))
    d = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    s_gemm = cu_masked_stream(torch, 0, c, cus)
    s_comm = cu_masked_stream(torch, c, cus - c, cus)
    reps = max(args.steps, 5)

    def run(gemm, comm):
        torch.cuda.synchronize()
        e = {}
        for name, st, on, fn in (("gemm", s_gemm, gemm, lambda: dg.dg_gemm_fp8_nt(qa, sa, qb, sb, d=d)),
                                 ("comm", s_comm, comm, lambda: dst.copy_(src))):
            if not on:
                continue
            with torch.cuda.stream(st):
                e[name] = [torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
                fn()   # warm
                e[name][0].record()
                for _ in range(reps):
                    fn()
                e[name][1].record()
        torch.cuda.synchronize()
        return {kk: v[0].elapsed_time(v[1]) / reps for kk, v in e.items()}

    run(True, True)
    alone_g = run(True, False)["gemm"]
    alone_c = run(False, True)["comm"]
    both = run(True, True)
    flops = 2.0 * m * n * k
    copy_bytes = 2.0 * src.numel()
    out = {"metric": METRIC, "value": round(flops / (both["gemm"] * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
           "n_gpus": 1, "steps": reps, "warmup": 1, "ms_per_step": round(both["gemm"], 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
           "config": {"workload": "overlap", "gemm": f"{m}x{n}x{k}", "gemm_cus": c, "comm_cus": cus - c,
                      "gemm_config": dg.dg_gemm_config_name(0, m, n, k),
                      "comm_stand_in": "512 MiB device copy (read + write) on a CU-masked stream"},
           "overlap": {"gemm_alone_ms": round(alone_g, 4), "gemm_with_comm_ms": round(both["gemm"], 4),
                       "gemm_alone_tflops": round(flops / (alone_g * 1e-3) / 1e12, 1),
                       "comm_alone_gbps": round(copy_bytes / (alone_c * 1e-3) / 1e9, 1),
                       "comm_with_gemm_gbps": round(copy_bytes / (both["comm"] * 1e-3) / 1e9, 1)},
           "roofline": None, "cpu_baseline": None}
    print(json.dumps(out), flush=True)


def source_digest():
    """sha256 of the GEMM kernel source: traffic counters are only valid for the kernel they measured."""
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm.hip", "gemm_common.hpp", "common.hpp"):
        with open(os.path.join(ROOT, "fp8_block_scaled_gemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel, launches_bytes):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary, scaled by the
    copy-kernel calibration; None if there is none for this workload/kernel or the source changed."""
    path = os.path.join(ROOT, "profiles", "traffic_counters.json")
    try:
        with open(path) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    rec = data.get(workload, {}).get(kernel)
    if not rec or rec.get("source_sha") != source_digest():
        return None
    return {"bytes_per_launch": rec["hbm_bytes_per_launch"], "algorithmic_bytes_per_launch": launches_bytes,
            "ratio": round(rec["hbm_bytes_per_launch"] / launches_bytes, 3), "source": "profiles/traffic_counters.json"}


def copy_calibration(torch, dev, nbytes=1 << 30, reps=5):
    """A plain device copy of known size, profiled with the FETCH_SIZE / WRITE_SIZE counters to scale
    them to bytes (one launch reads and writes nbytes)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": reps}), flush=True)


def plan_sweep(args, torch, dg, dev):
    """Every few-row plan the planner weighs (64x64 and 64x128 tiles x K splits 1..16, forced with
    DG_PLAN) on the twelve M = 64 / 128 DeepSeek-V3 shapes, timed like bench.py's per-launch pass
    (R launches over rotated weight copies after a 512 MB write, median of 5), next to the plan the
    planner picks.  Writes a markdown table (the evidence behind the few-row planner's model)."""
    from fp8_block_scaled_gemm_amd import inputs
    gen = Gen(torch, dev, 99)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    ws = torch.zeros(256 << 20, dtype=torch.uint8, device=dev)
    lines = ["| shape | planner's plan | us | GB/s | best plan | us | GB/s | planner / best |",
             "|---|---|---|---|---|---|---|---|"]
    detail = []
    old_plan = os.environ.pop("DG_PLAN", None)
    for m in (64, 128):
        for (n, k) in inputs.DENSE_V3_NK:
            qa, sa = dg.dg_quantize_per_token_group(gen.activations(m, k))
            qb, sb = dg.dg_quantize_per_block(gen.normal((n, k), 0.02))
            r = max(1, min(MAX_ROT, -(-ROT_BYTES // (n * k))))
            copies = [qb] + [qb.clone() for _ in range(r - 1)]
            d = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            wbytes = dense_gemm_bytes(m, n, k)

            def timed():
                for w in copies:
                    dg.dg_gemm_fp8_nt(qa, sa, w, sb, d=d, workspace=ws)
                torch.cuda.synchronize()
                ts = []
                for rep in range(5):
                    flush.fill_(rep)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for w in copies:
                        dg.dg_gemm_fp8_nt(qa, sa, w, sb, d=d, workspace=ws)
                    e1.record()
                    torch.cuda.synchronize()
                    ts.append(e0.elapsed_time(e1) * 1e3 / r)
                return float(np.median(ts))

            default = dg.dg_gemm_config_name(0, m, n, k)
            t_default = timed()
            results = {default: t_default}
            for tile in ("64x64", "64x128"):
                for sp in (1, 2, 3, 4, 6, 8, 12, 16):
                    os.environ["DG_PLAN"] = f"tile={tile},splits={sp}"
                    name = dg.dg_gemm_config_name(0, m, n, k)
                    if name not in results:
                        results[name] = timed()
            os.environ.pop("DG_PLAN", None)
            best = min(results, key=results.get)
            shape = f"{m}x{n}x{k}"
            print(f"[bench] plan sweep {shape}: planner {default} {t_default:.1f} us, best {best} "
                  f"{results[best]:.1f} us", file=sys.stderr, flush=True)
            lines.append(f"| {shape} | {default} | {t_default:.1f} | {wbytes / t_default / 1e3:.0f} | {best} | "
                         f"{results[best]:.1f} | {wbytes / results[best] / 1e3:.0f} | {t_default / results[best]:.2f} |")
            detail.append(f"| {shape} | " + ", ".join(f"{nm.split('/')[0]} s{nm.split('split')[1]}: {t:.1f}"
                                                   for nm, t in sorted(results.items())) + " |")
            del copies
    if old_plan is not None:
        os.environ["DG_PLAN"] = old_plan
    out = ["# Few-row plans: every tile x K split the planner weighs, against its choice", "",
           "Command:", "", "```", "python3 bench.py --plan-sweep --out profiles/decode_plan_sweep.md", "```", "",
           "Per launch, R launches over rotated weight copies (> 768 MB) after an untimed 512 MB write, "
           "median of 5; GB/s = algorithmic bytes (A, B, their scales, bf16 D) / time.  Plans forced with "
           "DG_PLAN.", ""] + lines + ["", "All plans (us):", "", "| shape | tile, split: us |", "|---|---|"] + detail
    text = "\n".join(out) + "\n"
    if args.out:
        with open(args.out, "w") as fh:
            fh.write(text)
    print(text)


DEFAULT_SET = ["small", "dense_v3", "contiguous", "masked", "large_dense", "zipf"]
HEADLINE = "dense_v3"
ROT_BYTES = 768 << 20     # weight copies a GEMM's timed launches rotate over: > 3x the 256 MB MALL
MAX_ROT = 32
FLUSH_BYTES = 512 << 20   # untimed write ahead of every timed GEMM: the MALL holds none of its operands


def kernel_of(config):
    """Kernel instance of a GEMM configuration name (the K split is a launch parameter of the same
    kernel): '256x192/8waves/split1' -> 'gemm_fp8_kernel 256x192/8waves'."""
    return "gemm_fp8_kernel " + kernel_config(config)


def rooflines(workload, ops):
    """Per GEMM kernel instance of the step: its roofline against the bound its work sets (MFMA when
    the flops take longer at peak than the bytes, else HBM), from the per-launch durations."""
    by_k = {}
    for op in ops:
        if op.kind == "gemm":
            by_k.setdefault(kernel_of(op.config), []).append(op)
    out = {}
    for kern, kops in by_k.items():
        # every timed launch counts once (a GEMM timed over R weight copies is R launches), so the
        # average launch duration is the one a kernel trace of the same run reports
        t = sum(sum(o.times) * o.rot for o in kops) * 1e-3
        launches = sum(len(o.times) * o.rot for o in kops)
        f = sum(o.flops * len(o.times) * o.rot for o in kops)
        b = sum(o.nbytes * len(o.times) * o.rot for o in kops)
        mfma = f / (PEAK_FP8_TFLOPS * 1e12) >= b / (PEAK_HBM_GBS * 1e9)
        if mfma:
            achieved, peak, unit = f / t / 1e12, PEAK_FP8_TFLOPS, "TFLOP/s"
        else:
            achieved, peak, unit = b / t / 1e9, PEAK_HBM_GBS, "GB/s"
        traffic = measured_traffic(workload, kern, b / launches)
        out[kern] = {"bound": "mfma" if mfma else "hbm", "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4),
                     "traffic": traffic["bytes_per_launch"] if traffic else None, "traffic_detail": traffic,
                     "kernel": kern, "launches": launches, "avg_launch_us": round(t / launches * 1e6, 2),
                     "algorithmic_bytes_per_launch": round(b / launches), "flops_per_launch": round(f / launches),
                     "device_us_per_step": round(sum(sum(o.times) for o in kops) * 1e-3 / max(1, len(kops[0].times)) * 1e6, 1),
                     "shapes": sorted({o.label for o in kops})}
    return out


def run_workload(name, args, torch, dg, dev, stream, flush_buf):
    """Build one workload, time its step (graph replays) and every launch (cold MALL), summarize."""
    ops, desc = build_workload(name, torch, dg, dev, args.act_dtype, args.act_quant)
    torch.cuda.synchronize()
    print(f"[bench] workload {name}: {len(ops)} ops per step", file=sys.stderr, flush=True)

    def step():
        for op in ops:
            op.launch()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: K steps, each one replay of the step captured as a HIP graph (no host launch
    # gaps between the kernels); wall clock bracketed by device synchronisation ------------------------
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        graph.replay()
        torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        ev0.record()
        for _ in range(args.steps):
            if graph is not None:
                graph.replay()
            else:
                step()
        ev1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    gpu_ms_per_step = ev0.elapsed_time(ev1) / args.steps
    print(f"[bench] {name}: timed {args.steps} steps: {ms_per_step:.3f} ms/step (device {gpu_ms_per_step:.3f})",
          file=sys.stderr, flush=True)
    del graph

    # ---- per-launch durations, cold MALL.  A GEMM runs R times back to back over R copies of its
    # weights (R x weight bytes > 768 MB, so no launch finds its weights in the MALL) between one HIP
    # event pair on the stream, after an untimed 512 MB write; its duration is the pair's time / R.
    # Other launches (quantizers) take one event pair each.  A short bounded spin kernel at the
    # start of every step gives the host's enqueue a head start (a long one idles the device, and
    # the MFMA-bound launches right after it run slower). -------------------------------------------
    for op in ops:
        if op.weights is not None and not args.no_rotate:
            wbytes = op.weights.numel() * op.weights.element_size()
            r = max(1, min(MAX_ROT, -(-ROT_BYTES // max(wbytes, 1))))
            op.copies = [op.weights] + [op.weights.clone() for _ in range(r - 1)]
            op.rot = r
    torch.cuda.synchronize()
    cal0, cal1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        torch.cuda._sleep(1_000_000)
        cal0.record()
        torch.cuda._sleep(10_000_000)
        cal1.record()
    torch.cuda.synchronize()
    cycles_per_ms = 10_000_000 / max(cal0.elapsed_time(cal1), 1e-3)
    spin_cycles = int(args.spin_ms * cycles_per_ms)
    n = len(ops)
    with torch.cuda.stream(stream):
        for _ in range(args.steps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
            torch.cuda._sleep(spin_cycles)
            for i, op in enumerate(ops):
                if op.kind == "gemm" and flush_buf is not None:
                    flush_buf.fill_(1)
                ev[2 * i].record()
                if op.copies:
                    for w in op.copies:
                        op.make(w)
                else:
                    op.launch()
                ev[2 * i + 1].record()
            torch.cuda.synchronize()
            for i, op in enumerate(ops):
                op.times.append(ev[2 * i].elapsed_time(ev[2 * i + 1]) / (len(op.copies) if op.copies else 1))
    print(f"[bench] {name}: per-launch timing done", file=sys.stderr, flush=True)
    for op in ops:
        op.copies = None

    gemm_flops = sum(op.flops for op in ops if op.kind == "gemm")
    shapes = []
    for op in ops:
        if op.kind != "gemm":
            continue
        t = float(np.median(op.times)) * 1e-3
        tf, gb = op.flops / t / 1e12, op.nbytes / t / 1e9
        shapes.append({"shape": op.label, "config": op.config, "us": round(t * 1e6, 2),
                       "tflops": round(tf, 1), "gbps": round(gb, 1),
                       "mfma_frac": round(tf / PEAK_FP8_TFLOPS, 4), "hbm_frac": round(gb / PEAK_HBM_GBS, 4),
                       "roofline_frac": round(max(op.flops / (PEAK_FP8_TFLOPS * 1e12),
                                                  op.nbytes / (PEAK_HBM_GBS * 1e9)) / t, 4),
                       "rotations": op.rot})
    kernels = rooflines(name, ops)
    dominant = max(kernels.values(), key=lambda r: r["avg_launch_us"] * r["launches"])
    quant = {}
    for kind in ("wquant", "aquant", "cquant", "transpose"):
        ks = [op for op in ops if op.kind == kind]
        if ks:
            t = sum(float(np.median(o.times)) for o in ks) * 1e-3
            b = sum(o.nbytes for o in ks)
            quant[kind] = {"us": round(t * 1e6, 1), "gbps": round(b / t / 1e9, 1),
                           "hbm_frac": round(b / t / 1e9 / PEAK_HBM_GBS, 4)}
    gemm_only_ms = sum(float(np.median(o.times)) for o in ops if o.kind == "gemm")
    summary = {"workload": name, "description": desc,
               "value": round(gemm_flops / (ms_per_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
               "ms_per_step": round(ms_per_step, 4), "device_ms_per_step": round(gpu_ms_per_step, 4),
               "gemms": len(shapes), "gemm_only_ms": round(gemm_only_ms, 4),
               "gemm_only_tflops": round(gemm_flops / (gemm_only_ms * 1e-3) / 1e12, 1),
               "timing": "eager" if args.eager else "hip graph replay per step",
               "roofline": dominant, "kernels": kernels, "quant": quant, "shapes": shapes}
    del ops
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return summary


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (got --gpus {args.gpus}); the path has no "
              "multi-GPU mode - see the sharding notes of the design document", file=sys.stderr)
        sys.exit(2)
    import torch
    import fp8_block_scaled_gemm_amd as dg

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    if args.copy_calibration:
        copy_calibration(torch, dev)
        return
    if args.plan_sweep:
        dg.lib()
        plan_sweep(args, torch, dg, dev)
        return
    dg.lib()
    if args.num_cus > 0:
        dg.dg_set_num_cus(args.num_cus)
    if args.workload == "overlap":
        overlap_bench(args, torch, dg, dev)
        return
    names = DEFAULT_SET if args.workload == "all" else [args.workload]
    stream = torch.cuda.Stream()
    flush_buf = None if args.no_flush else torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    results = {}
    for name in names:
        results[name] = run_workload(name, args, torch, dg, dev, stream, flush_buf)
    head = results[HEADLINE] if HEADLINE in results else results[names[0]]

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(head["workload"], args.cpu_seconds)

    config = {"workload": head["workload"], "description": head["description"], "gemms": head["gemms"],
              "activation_input": args.act_dtype, "activation_quantization": args.act_quant,
              "step": ("per (N,K): weight quantization + transpose; forward (quantize X, GEMM), dgrad "
                       "(quantize dY, GEMM with W^T), wgrad (per-channel quantize dY and X, row-scaled GEMM)"
                       if head["workload"] == "train_v3" else
                       "per (N,K): expert weight quantization + transpose; forward (quantize X, contiguous GEMM), "
                       "dgrad (quantize dY, contiguous GEMM with W_e^T), wgrad (per-channel quantize dY and X, "
                       "k-grouped row-scaled GEMM)" if head["workload"] == "train_moe" else
                       "weight quantization (all weights) + per shape: activation quantization, FP8 GEMM"),
              "timing": head["timing"], "device_ms_per_step": head["device_ms_per_step"],
              "gemm_only_tflops": head["gemm_only_tflops"], "gemm_only_ms": head["gemm_only_ms"],
              "per_launch_timing": ("median over steps; each GEMM after an untimed 512 MB write, launched over "
                                    "rotated weight copies (> 768 MB) between one event pair, time / copies"),
              "also_timed": [n for n in names if n != head["workload"]]}
    out = {"metric": METRIC, "value": head["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
           "config": config, "roofline": head["roofline"], "cpu_baseline": cpu, "quant": head["quant"],
           "shapes": head["shapes"],
           "configs": {n: {k: v for k, v in r.items() if k != "description"} for n, r in results.items()}}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
