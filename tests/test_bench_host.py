"""bench.py's host arithmetic, without a GPU: the algorithmic bytes of each GEMM form (counted by
hand for one DeepSeek-V3 decode shape), the kernel-instance names, the roofline aggregation over
timed launches (every launch of a GEMM timed over R weight copies counts R times; the bound is
the one the work sets at the published peaks), and the rule that a counter record is used only
for the kernel source it was measured on."""

import numpy as np
import pytest

import bench


def test_dense_bytes_hand_computed():
    # 64 x 2112 x 7168: A 64*7168, A scales 4*64*56, B 2112*7168, B scales 4*17*56, D 2*64*2112
    assert bench.dense_gemm_bytes(64, 2112, 7168) == 458752 + 14336 + 15138816 + 3808 + 270336
    assert abs(bench.dense_gemm_bytes(64, 2112, 7168) / 1e6 - 15.9) < 0.05
    # a partial last K group still carries a scale
    assert bench.dense_gemm_bytes(1, 1, 130) == 130 + 8 + 130 + 8 + 2


def test_grouped_bytes():
    # one expert, every row valid: the contiguous and masked forms move what the dense one does,
    # plus the int32 index per row (contiguous) or the group count (masked)
    m, n, k = 256, 384, 512
    dense = bench.dense_gemm_bytes(m, n, k)
    assert bench.contiguous_gemm_bytes(m, n, k, 1) == dense + 4 * m
    assert bench.masked_gemm_bytes([m], m, n, k) == dense + 4
    # empty experts move no weights; counts past m_max are clamped, negative ones are zero
    one = bench.masked_gemm_bytes([100], 256, n, k)
    assert bench.masked_gemm_bytes([100, 0, -3], 256, n, k) == one + 8
    assert bench.masked_gemm_bytes([300], 256, n, k) == bench.masked_gemm_bytes([256], 256, n, k)
    # G experts' weights are all read once
    assert (bench.contiguous_gemm_bytes(512, n, k, 4) - bench.contiguous_gemm_bytes(512, n, k, 1)
            == 3 * (n * k + 4 * 3 * 4))


def test_kernel_names():
    assert bench.kernel_config("256x192/8waves/split1+tail2") == "256x192/8waves"
    assert bench.kernel_config("64x64/4waves/split8") == "64x64/4waves"
    assert bench.kernel_config("64x64/4waves/split8+act-quant") == "64x64/4waves +act-quant"
    assert bench.kernel_of("256x256/8waves/split1") == "gemm_fp8_kernel 256x256/8waves"


def _op(label, config, flops, nbytes, times_ms, rot):
    op = bench.Op("gemm", label, None, flops=flops, nbytes=nbytes, config=config)
    op.times = list(times_ms)
    op.rot = rot
    return op


def test_rooflines_weight_every_launch(monkeypatch):
    monkeypatch.setattr(bench, "measured_traffic", lambda *a: None)
    # two shapes on one kernel instance: 2 steps each, the second timed over 3 weight copies
    a = _op("a", "256x256/8waves/split1", 2e12, 1e9, [1.0, 1.0], 1)     # 1 ms per launch
    b = _op("b", "256x256/8waves/split1", 1e12, 5e8, [0.5, 0.5], 3)     # 0.5 ms per launch
    r = bench.rooflines("w", [a, b])["gemm_fp8_kernel 256x256/8waves"]
    launches = 2 * 1 + 2 * 3
    t = (2 * 1.0 + 3 * 2 * 0.5) * 1e-3
    flops = 2 * 2e12 + 3 * 2 * 1e12
    assert r["launches"] == launches and r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["avg_launch_us"] == pytest.approx(t / launches * 1e6, rel=1e-6)
    assert r["achieved"] == pytest.approx(flops / t / 1e12, rel=1e-4)
    assert r["frac"] == pytest.approx(r["achieved"] / bench.PEAK_FP8_TFLOPS, rel=1e-3)
    assert r["flops_per_launch"] == round(flops / launches)
    assert r["traffic"] is None


def test_rooflines_hbm_bound(monkeypatch):
    monkeypatch.setattr(bench, "measured_traffic", lambda *a: None)
    # 1 GFLOP over 100 MB: 0.2 us at the MFMA peak, 12.5 us at the HBM peak -> HBM-bound
    op = _op("d", "64x64/4waves/split4", 1e9, 1e8, [0.025, 0.025, 0.025], 8)
    r = bench.rooflines("w", [op])["gemm_fp8_kernel 64x64/4waves"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(1e8 / 25e-6 / 1e9, rel=1e-4)
    assert r["frac"] == pytest.approx(0.5, rel=1e-3)


def test_traffic_needs_the_measured_source(monkeypatch, tmp_path):
    # a counter record is used only for the kernel source it was measured on
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    rec = {"w": {"gemm_fp8_kernel 256x256/8waves": {"source_sha": "abc", "hbm_bytes_per_launch": 300}}}
    (tmp_path / "profiles" / "traffic_counters.json").write_text(__import__("json").dumps(rec))
    monkeypatch.setattr(bench, "source_digest", lambda: "abc")
    got = bench.measured_traffic("w", "gemm_fp8_kernel 256x256/8waves", 200)
    assert got["bytes_per_launch"] == 300 and got["ratio"] == 1.5
    monkeypatch.setattr(bench, "source_digest", lambda: "changed")
    assert bench.measured_traffic("w", "gemm_fp8_kernel 256x256/8waves", 200) is None
    assert bench.measured_traffic("other", "gemm_fp8_kernel 256x256/8waves", 200) is None
