"""Host logic of bench.py: the algorithmic byte count and the reading of the
committed HBM-traffic and VALU counter summaries (no GPU needed)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_conv_alg_bytes_four_step(monkeypatch):
    # two orders, each reads z^n and x^n and writes z^{n+1} and reads one half spectrum
    # per channel, complex fp32 (8 bytes per bin): 704.6 MB per order at L = 64k, D = 768
    B, L, D, N = 1, 65536, 768, 2
    assert bench.conv_alg_bytes(B, L, D, N, 2, False) == 2 * (3 * B * L * D * 2 + 8 * D * (L + 1))
    assert abs(bench.conv_alg_bytes(B, L, D, N, 2, False) / 2 - 704.6e6) < 0.1e6
    assert bench.conv_alg_bytes(B, L, D, N, 4, False) == 2 * (3 * B * L * D * 4 + 8 * D * (L + 1))
    # as stored: the bf16 copy the row passes of bf16 workloads read, unless the knob keeps fp32
    monkeypatch.delenv("HYENA_SPECTRUM_FP32", raising=False)
    assert bench.four_step_spectrum_bytes(2) == 4.0 and bench.four_step_spectrum_bytes(4) == 8.0
    assert bench.conv_alg_bytes(B, L, D, N, 2, False, bench.four_step_spectrum_bytes(2)) == \
        2 * (3 * B * L * D * 2 + 4 * D * (L + 1))
    monkeypatch.setenv("HYENA_SPECTRUM_FP32", "1")
    assert bench.four_step_spectrum_bytes(2) == 8.0


def test_cpu_baseline_reports_workers_and_model():
    # a tiny causal workload through the pooled oracle: the report names the
    # process count and the CPU model
    from synth import make_1d
    inp = make_1d(3, 1, 256, 64, N=2, K=8)
    r = bench.cpu_baseline(inp, 128, 2)
    assert r["cores"] == 2 and r["kind"] == "oracle" and r["value"] > 0
    assert isinstance(r["cpu_model"], str) and r["cpu_model"]
    assert "2 processes" in r["sample"]


def test_conv_alg_bytes_lds_regime():
    B, L, D, N = 8, 2048, 768, 2
    want = (N + 1) * B * L * D * 2 + B * L * D * 2 + N * 8 * D * (L + 1)
    assert bench.conv_alg_bytes(B, L, D, N, 2, True) == want


def test_traffic_summary_with_current_sources(tmp_path):
    p = tmp_path / "t.txt"
    p.write_text(f"text\n@conv_stage_bytes_per_step: 1.5e9\n@conv_source_sha256: {bench.conv_source_hash()}\n")
    assert bench.measured_traffic("w", str(p)) == 1.5e9


def test_traffic_summary_is_void_after_a_kernel_change(tmp_path):
    p = tmp_path / "t.txt"
    p.write_text("@conv_stage_bytes_per_step: 1.5e9\n@conv_source_sha256: 0000\n")
    assert bench.measured_traffic("w", str(p)) is None
    assert bench.measured_traffic("no_such_workload") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_valu_summary_with_current_sources(tmp_path):
    p = tmp_path / "v.txt"
    p.write_text("@conv_valu_instr_per_step: 2.5e8\n@conv_valu_flops_per_step: 1.6e10\n"
                 f"@conv_source_sha256: {bench.conv_source_hash()}\n")
    assert bench.measured_valu("w", str(p)) == (2.5e8, 1.6e10)


def test_valu_summary_is_void_after_a_kernel_change(tmp_path):
    p = tmp_path / "v.txt"
    p.write_text("@conv_valu_instr_per_step: 2.5e8\n@conv_valu_flops_per_step: 1.6e10\n@conv_source_sha256: 0\n")
    assert bench.measured_valu("w", str(p)) is None
    assert bench.measured_valu("no_such_workload") is None


def test_nd_alg_bytes_by_boundary():
    B, G, C, N = 2, 64, 128, 2
    V = G ** 3
    assert bench.nd_conv_alg_bytes(B, G, G, G, C, N) == N * (3 * B * C * V * 4 + 8 * C * 128 * 128 * 65)
    assert bench.nd_conv_alg_bytes(B, G, G, G, C, N, True) == N * (3 * B * C * V * 4 + 8 * C * 64 * 64 * 33)


def test_nd_alg_bytes_2d_fused():
    # 2D grid: v and x^1, x^2 read once, z^3 written once, two half spectra 128 x 65
    B, Y, C, N = 8, 64, 384, 2
    V = Y * Y
    want = 4 * B * C * V * 4 + N * 8 * C * 128 * 65
    assert bench.nd_conv_alg_bytes(B, 1, Y, Y, C, N) == want
