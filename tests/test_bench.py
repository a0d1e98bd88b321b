"""CPU tests of bench.py's contract: the one-GPU limit and the recorded-traffic lookup."""
import subprocess
import sys
from pathlib import Path

import bench

ROOT = Path(__file__).resolve().parent.parent


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=60)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr
    assert res.stdout == ""


def test_defaults_fit_the_contract():
    a = bench.parse_args([])
    assert (a.gpus, a.steps, a.warmup, a.workload) == (1, 50, 20, "t16384_d128")


def test_recorded_traffic_needs_the_current_source(tmp_path, monkeypatch):
    """A counter summary is used only when it names the current kernel source."""
    monkeypatch.setattr(bench, "PROFILES", tmp_path)
    summary = bench.traffic_summary("t16384_d128")
    assert summary.parent == tmp_path
    assert bench.recorded_traffic("t16384_d128") == (None, None)
    summary.write_text("    kernel_source_sha256_16: 0000000000000000\n"
                       "    hbm_bytes_per_launch: 1.5e8\n")
    assert bench.recorded_traffic("t16384_d128") == (None, None)
    summary.write_text(f"    kernel_source_sha256_16: {bench.source_digest()}\n"
                       "    hbm_bytes_per_launch: 1.5e8\n    mfma_busy_pct: 80.5\n")
    traffic, extra = bench.recorded_traffic("t16384_d128")
    assert traffic == 1.5e8 and extra == {"mfma_busy_pct": 80.5}
    assert bench.recorded_traffic("t4096_outliers") == (None, None)


def test_every_forward_workload_is_benchmarked():
    from attention_flashattention_fwd_amd import inputs
    lines = {bench.HEADLINE, *bench.SECONDARY}
    assert set(inputs.WORKLOADS) | set(inputs.KV_WORKLOADS) == lines


def test_markers_work_without_a_profiler():
    m = bench.Markers()
    m.push("test range")
    m.pop()


def test_source_digest_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int a; // note\n/* block */ int b;\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCE", src)
    d1 = bench.source_digest()
    src.write_text("int a;   // another note\nint b;\n")
    assert bench.source_digest() == d1
    src.write_text("int a; int c;\n")
    assert bench.source_digest() != d1
