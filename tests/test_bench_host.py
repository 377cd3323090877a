"""Host-side logic of bench.py: kernel-to-stage mapping, algorithmic work per
stage, roofline bound selection and the counter-summary lookup."""
import json
import os

import pytest

import bench


def test_kernel_stage_mapping():
    assert bench.kernel_stage("moe::plan_kernel(int const*, int)") == "plan"
    assert bench.kernel_stage("void moe::gemm_bf16_kernel<256, true>(unsigned short const*)") == "gate_up"
    assert bench.kernel_stage("void moe::gemm_bf16_kernel<128, false>(x)") == "down"
    assert bench.kernel_stage("void moe::gemm_fp8_kernel<4, 256, true>(x)") == "gate_up"
    assert bench.kernel_stage("void moe::gemm_fp8_kernel<4, 128, false>(x)") == "down"
    assert bench.kernel_stage("void moe::decode_kernel<1, 3, 2, false>(x)") == "decode"
    assert bench.kernel_stage("moe::combine_kernel(x)") == "combine"
    assert bench.kernel_stage("void moe::gemm_mx_kernel<256, true, 2>(unsigned char const*)") == "gate_up"
    assert bench.kernel_stage("void moe::gemm_mx_kernel<256, false, 2>(x)") == "down"
    assert bench.kernel_stage("void moe::gemm_mx_wide_kernel<true>(x)") == "gate_up"
    assert bench.kernel_stage("void moe::gemm_mx_wide_kernel<false>(x)") == "down"
    assert bench.kernel_stage("void moe::route_kernel<2>(moe::RouteArgs)") == "router"
    assert bench.kernel_stage("void moe::route_plan_kernel<1>(moe::RouteArgs)") == "route_plan"
    assert bench.kernel_stage("__amd_rocclr_copyBuffer") is None


def test_stage_work_matches_the_layer_formula():
    # DeepSeek-OCR-2 decode, T=1: 6 touched experts x (2FH + HF) bf16 weights
    T, H, F, k = 1, 1280, 896, 6
    b, f = bench.stage_work("decode", "bf16", T, H, F, k, touched=6, valid=6)
    # weights, the token row, the output row and the routing (ids + weights)
    assert b == 6 * 3 * F * H * 2 + T * H * 2 + T * H * 2 + T * k * 8
    assert f == 2 * 6 * 3 * F * H
    gu = bench.stage_work("gate_up", "bf16", 2048, H, F, k, touched=64, valid=2048 * 6)
    dn = bench.stage_work("down", "bf16", 2048, H, F, k, touched=64, valid=2048 * 6)
    assert gu[1] + dn[1] == bench.algorithmic_flops(2048 * 6, H, F)
    total = bench.algorithmic_bytes("bf16", 2048, H, F, k, 64)
    assert total == 64 * 3 * F * H * 2 + 2048 * H * 2 + 2048 * H * 2 + 2048 * k * 8
    # fp8: one byte per weight plus an fp32 scale per 128-wide block
    b8, _ = bench.stage_work("down", "fp8", 128, 7168, 2048, 8, touched=128, valid=1024)
    assert b8 == pytest.approx(128 * 7168 * 2048 * (1 + 4 / 128))
    # mxfp4: half a byte per weight plus one E8M0 byte per 32
    b4, f4 = bench.stage_work("gate_up", "mxfp4", 128, 7168, 2048, 8, touched=128, valid=1024)
    assert b4 == pytest.approx(128 * 2 * 2048 * 7168 * (0.5 + 1 / 32) + 128 * 7168 * (1 + 1 / 32))
    assert f4 == 2 * 1024 * 2 * 2048 * 7168


def test_roofline_bound_follows_arithmetic_intensity():
    # below the bf16 ridge (2500 TFLOP/s / 8 TB/s = 312.5 flop/B): HBM bound
    r = bench.roofline_for("down", "bf16", "bf16", bytes_=1e9, flops=100e9, ms=1.0)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["achieved"] == pytest.approx(1000.0)
    assert r["frac"] == pytest.approx(1000.0 / 8000.0, rel=1e-3)
    r = bench.roofline_for("gate_up", "fp8", "fp8", bytes_=1e9, flops=1e12, ms=1.0)
    assert r["bound"] == "mfma" and r["peak"] == 5000.0 and r["achieved"] == pytest.approx(1000.0)


def test_committed_traffic_requires_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    os.makedirs(tmp_path / "include")
    os.makedirs(tmp_path / "mixture_experts_routed_amd" / "csrc")
    (tmp_path / "include" / "a.h").write_text("x")
    digest = bench.source_digest()
    doc = {"source_sha256": digest, "stages": {"down": {"hbm_bytes": 1234}}}
    (tmp_path / "profiles" / "hbm_w.json").write_text(json.dumps(doc))
    assert bench.committed_traffic("w", "down") == 1234
    assert bench.committed_traffic("w", "gate_up") is None
    (tmp_path / "include" / "a.h").write_text("y")   # sources changed since
    assert bench.committed_traffic("w", "down") is None


def test_gpus_other_than_one_exit_with_a_message(capsys, monkeypatch):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as ex:
        bench.main()
    assert ex.value.code == 2
    assert "one GPU" in capsys.readouterr().out
