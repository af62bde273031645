"""The normal GEMM that allocates nothing (dg_gemm_fp8_nt_no_alloc): its split-K counters and
partials live in the library's own per-device scratch.  Its output must equal dg_gemm_fp8_nt's
with a workspace (the same plan and K split, so bit for bit) and the oracle's within the GEMM
tolerance, over consecutive calls on the shared scratch, the second with a smaller input."""

import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import fp8_block_scaled_gemm_amd as dg
from fp8_block_scaled_gemm_amd import inputs
import oracle
from gpu_util import bf16_bits, check_gemm, device, sa_to_dev, say, to_dev

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DG_ERR_HIP, DG_ERR_WORKSPACE = -4, -3


def _operands(m, n, k):
    rng = inputs.rng_for("no_alloc", m, n, k)
    a = inputs.activations_with_outliers(rng, m, k)
    b = inputs.normal(rng, (n, k), 0.02)
    qa, sa = oracle.quant.quantize_per_token_group(a)
    qb, sb = oracle.quant.quantize_per_block(b)
    return (qa, sa, qb, sb), (to_dev(qa), sa_to_dev(sa), to_dev(qb), to_dev(sb))


@pytest.mark.gpu
def test_no_alloc_matches_workspace_entry_point():
    shapes = [(128, 4096, 7168), (64, 512, 7168), (128, 4096, 7168)]   # larger, smaller, the first again
    for m, n, k in shapes:
        assert not dg.dg_gemm_config_name(0, m, n, k).endswith("/split1"), "each case must use the split-K scratch"
    for i, (m, n, k) in enumerate(shapes):
        say("no-alloc gemm", i, m, n, k, dg.dg_gemm_config_name(0, m, n, k))
        host, (qa, sa, qb, sb) = _operands(m, n, k)
        d = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=device())
        dg.dg_gemm_fp8_nt_no_alloc(qa, sa, qb, sb, d)
        ws = torch.zeros(dg.dg_gemm_workspace_size(m, n, k), dtype=torch.uint8, device=device())
        ref = dg.dg_gemm_fp8_nt(qa, sa, qb, sb, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(d), bf16_bits(ref)), (i, m, n, k)
        check_gemm(d, oracle.gemm.gemm_nt(*host), f"no-alloc {m}x{n}x{k}")


_REJECT = r"""
import sys
sys.path.insert(0, {root!r})
import fp8_block_scaled_gemm_amd as dg
L = dg.lib()
assert L.dg_set_num_cus(1024) == 0
p = 1 << 20   # aligned stand-in addresses: the calls return before anything touches them
print(L.dg_gemm_fp8_nt_no_alloc(p, p, 4096, p, p, p, 4096, 4096, 16384, None),
      L.dg_gemm_workspace_size(4096, 4096, 16384, 1))
"""


def test_no_alloc_rejects_plans_beyond_the_scratch():
    """A plan that needs more split-K scratch than the library holds is refused before any launch
    (planned for a 1024-CU cap on a host without a GPU: 4096 x 4096 x 16384 splits every tile)."""
    r = subprocess.run([sys.executable, "-c", _REJECT.format(root=ROOT)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    status, need = (int(v) for v in r.stdout.split())
    assert need > (64 << 20)
    assert status == DG_ERR_WORKSPACE
