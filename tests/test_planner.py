"""The GEMM planner on the host: tile configuration, K split and workspace size per shape.

With no GPU visible, a CU cap set with dg_set_num_cus stands in for the device's CU count and
the occupancy comes from each configuration's LDS, so the plans below are those the library
makes on a 256-CU MI355X (the GPU tests and bench.py report the same names there).  The queries
run in a subprocess: the cap is process-wide.
"""

import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "fp8_block_scaled_gemm_amd", "libdg.so")

_QUERY = r"""
import json, sys
sys.path.insert(0, {root!r})
import fp8_block_scaled_gemm_amd as dg
L = dg.lib()
assert L.dg_set_num_cus({cus}) == 0
out = []
for (layout, m, n, k, g) in json.loads(sys.argv[1]):
    out.append([layout, m, n, k, g, L.dg_gemm_config_name(layout, m, n, k, g).decode(),
                L.dg_gemm_workspace_size(m, n, k, g),
                L.dg_gemm_fp8_nt_act_quant_workspace_size(m, n, k) if layout == 0 else 0])
print(json.dumps(out))
"""


def plans(cases, cus=256, plan_override=None):
    if not os.path.exists(LIB):
        pytest.fail("libdg.so is not built: run `python -m fp8_block_scaled_gemm_amd._build`")
    env = dict(os.environ)
    env.pop("DG_PLAN", None)
    if plan_override is not None:
        env["DG_PLAN"] = plan_override
    r = subprocess.run([sys.executable, "-c", _QUERY.format(root=ROOT, cus=cus), json.dumps(cases)],
                       capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stderr[-2000:]
    return {tuple(row[:5]): tuple(row[5:]) for row in json.loads(r.stdout.strip().splitlines()[-1])}


NAME = re.compile(r"^(\d+)x(\d+)/(\d+)waves/split(\d+)(?:\+tail(\d+))?$")

# DeepSeek-V3 dense shapes (M, N, K) and the plan of each on 256 CUs
V3_PLANS = {
    (64, 2112, 7168): "64x64/4waves/split8", (64, 24576, 1536): "64x64/4waves/split1",
    (64, 32768, 512): "64x64/4waves/split1", (64, 7168, 16384): "64x64/4waves/split4",
    (64, 4096, 7168): "64x64/4waves/split6", (64, 7168, 2048): "64x64/4waves/split4",
    (128, 2112, 7168): "64x64/4waves/split6", (128, 24576, 1536): "64x128/4waves/split1",
    (128, 32768, 512): "64x128/4waves/split1", (128, 7168, 16384): "64x128/4waves/split4",
    (128, 4096, 7168): "64x128/4waves/split6", (128, 7168, 2048): "64x128/4waves/split4",
    (4096, 2112, 7168): "256x192/8waves/split1", (4096, 24576, 1536): "256x256/8waves/split1",
    (4096, 32768, 512): "256x256/8waves/split1", (4096, 7168, 16384): "256x256/8waves/split1",
    (4096, 4096, 7168): "256x256/8waves/split1", (4096, 7168, 2048): "256x256/8waves/split1",
}


def test_v3_dense_plans_on_256_cus():
    got = plans([[0, m, n, k, 1] for (m, n, k) in V3_PLANS])
    for (m, n, k), want in V3_PLANS.items():
        name, ws, ws_fq = got[(0, m, n, k, 1)]
        assert name == want, ((m, n, k), name, want)
        splits = NAME.match(name)
        split_plan = int(splits.group(4)) > 1 or splits.group(5) is not None
        if split_plan:
            assert ws > 0, (m, n, k, ws)
        # the in-launch quantization's workspace: counters, E4M3 activations, scales, partials
        ld = -(-m // 4) * 4
        assert ws_fq >= 64 * 1024 + m * k + (k // 128) * ld * 4 + (max(ws - 64 * 1024, 0) if split_plan else 0)


def test_split_last_round_plans():
    """Shapes with a partial last round of the persistent grid and a long K split only that round
    (the GPU tests assert the same names at 256 CUs)."""
    got = plans([[0, 4608, 4096, 6144, 1], [0, 4096, 6144, 6144, 1], [0, 4096, 5120, 6144, 1],
                 [3, 2048, 5120, 6144, 1], [0, 4096, 7168, 1024, 1]])
    assert got[(0, 4608, 4096, 6144, 1)][0] == "256x192/8waves/split1+tail2"
    assert got[(0, 4096, 6144, 6144, 1)][0] == "256x256/8waves/split1+tail2"
    assert got[(0, 4096, 5120, 6144, 1)][0] == "256x128/8waves/split1+tail2"
    assert got[(3, 2048, 5120, 6144, 1)][0] == "256x128/8waves/split1+tail2"
    assert "+tail" not in got[(0, 4096, 7168, 1024, 1)][0]   # pieces would be < 24 K blocks


def test_plan_invariants_over_shapes():
    ms = [1, 17, 64, 65, 128, 129, 256, 1000, 4096, 8192]
    nks = [(128, 128), (512, 7168), (2112, 7168), (7168, 2048), (4096, 512), (24576, 1536), (300, 16400)]
    cases = [[layout, m, n, k, 1] for layout in (0, 3) for m in ms for (n, k) in nks]
    cases += [[1, 128 * g * 4, n, k, g] for g in (1, 4, 8) for (n, k) in nks]
    cases += [[2, m, n, k, g] for g in (1, 8, 32) for m in (32, 256) for (n, k) in nks]
    for cus in (256, 80, 7):
        got = plans(cases, cus)
        for (layout, m, n, k, g), (name, ws, _) in got.items():
            mt = NAME.match(name)
            assert mt, (layout, m, n, k, g, name)
            bn, bm, waves, splits = (int(mt.group(i)) for i in range(1, 5))
            tail = mt.group(5)
            assert (bn, bm, waves) in {(64, 64, 4), (64, 128, 4), (256, 128, 8), (256, 192, 8), (256, 256, 8)}, name
            assert 1 <= splits <= 16 and (tail is None or splits == 1)
            if tail is not None:
                assert 2 <= int(tail) <= 16
            if layout == 1:   # the contiguous form never splits K (no workspace argument)
                assert splits == 1 and tail is None, name
            if layout == 3:   # per-row B scales run on the three-stage 256x128 tile only
                assert (bn, bm) not in {(256, 192), (256, 256)}, name
            if layout == 1:   # a contiguous tile spans one or two whole 128-row expert blocks
                assert bm in (128, 256), name
            if layout == 0 and m <= 128:   # few rows: the 64-row weight tiles
                assert bn == 64, (m, name)
            if layout in (0, 3) and m > 128:
                assert bn == 256, (m, name)
            if layout in (0, 2) and (splits > 1 or tail is not None):
                assert ws > 0, (layout, m, n, k, g, name)   # a split plan has its workspace size
            kb = -(-k // 128)
            assert splits <= kb and int(tail or 1) <= kb


def test_plan_override():
    """DG_PLAN replaces the planner's tile and K split where they are valid for the form and size,
    the workspace query follows the overridden plan, and anything else leaves the plan alone."""
    cases = [[0, 64, 2112, 7168, 1], [0, 4096, 2112, 7168, 1], [1, 4096, 2112, 7168, 4], [3, 4096, 2112, 7168, 1],
             [2, 128, 4096, 7168, 8]]
    base = plans(cases)
    got = plans(cases, plan_override="tile=64x128,splits=3")
    assert got[(0, 64, 2112, 7168, 1)][0] == "64x128/4waves/split3"
    # 56 K blocks in 3 splits of 19: a split tile needs 64 x 128 x 4 bytes per split
    assert got[(0, 64, 2112, 7168, 1)][1] == 64 * 1024 + 33 * 3 * 64 * 128 * 4
    assert got[(0, 4096, 2112, 7168, 1)][0] == base[(0, 4096, 2112, 7168, 1)][0].split("/split")[0] + "/split3"
    assert got[(1, 4096, 2112, 7168, 4)][0] == base[(1, 4096, 2112, 7168, 4)][0]   # contiguous: no split
    assert got[(2, 128, 4096, 7168, 8)][0] == "64x128/4waves/split3"
    got = plans(cases, plan_override="tile=256x256")
    assert got[(0, 4096, 2112, 7168, 1)][0].startswith("256x256/8waves/")
    assert got[(1, 4096, 2112, 7168, 4)][0].startswith("256x256/")
    assert got[(3, 4096, 2112, 7168, 1)][0].startswith("256x128/")   # row-scaled: 256x128 only
    got = plans(cases, plan_override="tile=256x192")
    assert got[(1, 4096, 2112, 7168, 4)] == base[(1, 4096, 2112, 7168, 4)]   # contiguous: no 192-row tile
    assert got[(0, 64, 2112, 7168, 1)] == base[(0, 64, 2112, 7168, 1)]   # not a few-row tile
    for junk in ("tile=100x7", "splits=0", "nonsense", "tile=64x64,splits=99"):
        got = plans(cases, plan_override=junk)
        for key, val in got.items():
            if junk.endswith("99") and key[0] != 1 and key[1] <= 128:
                kb = -(-key[3] // 128)   # capped at 16 splits, none of them empty
                assert val[0] == f"64x64/4waves/split{-(-kb // -(-kb // 16))}", (junk, key, val)
            elif junk.endswith("99"):
                pass
            else:
                assert val == base[key], (junk, key, val)


def test_contiguous_tile_choice():
    """The contiguous form takes 256x256 tiles where its experts are large (few expert boundaries
    per 256-row block, each costing one extra tile pass) and keeps 256x128 for many small experts:
    the MoE workloads G = 4 and 8 with ~8192 rows per expert, and 64 Zipf-sized experts."""
    cases = [[1, 31360, 4096, 7168, 4], [1, 31360, 7168, 2048, 4], [1, 62976, 4096, 7168, 8],
             [1, 62976, 7168, 2048, 8], [1, 36608, 2048, 7168, 64], [1, 4096, 4096, 7168, 32]]
    got = plans(cases)
    for c in cases[:4]:
        assert got[tuple(c)][0] == "256x256/8waves/split1", (c, got[tuple(c)])
    for c in cases[4:]:
        assert got[tuple(c)][0] == "256x128/8waves/split1", (c, got[tuple(c)])
