"""bench.py's contract: one JSON line with the fields the measurement needs,
one GPU only, and a traffic figure only while the counters match the kernel
source they were taken on."""
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    src = tmp_path / "attend.hip"
    shutil.copy(bench.ATTEND_SRC, src)
    rec = json.load(open(bench.TRAFFIC_FILE))
    rec["attend_hip_sha256_16"] = bench.source_hash(str(src))
    prof = tmp_path / "traffic.json"
    prof.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ATTEND_SRC", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(prof))
    assert bench.measured_traffic() == rec["hbm_bytes_per_launch"]
    # commentary and blank lines do not change the kernel
    src.write_text(src.read_text() + "\n// a note\n\n")
    assert bench.measured_traffic() == rec["hbm_bytes_per_launch"]
    # code does
    src.write_text(src.read_text() + "static int unused_after_profiling;\n")
    assert bench.measured_traffic() is None


@pytest.mark.gpu
def test_bench_json_line():
    """A short run on the smallest workload: every field the measurement
    reports, with the right types and consistent values."""
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", "c1",
                        "--steps", "3", "--warmup", "1", "--no-flexprefill"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "stages_ms", "step_ms", "speedup_vs_dense"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "ms" and d["higher_is_better"] is False and d["dtype"] == "bf16"
    assert d["value"] == d["ms_per_step"] and d["value"] > 0
    assert d["config"]["workload"].startswith("c1")
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["traffic"] is None                     # counters exist for h128 only
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "ms" and cb["cores"] >= 1 and cb["value"] > 0
    assert cb["pairs_match_gpu"] is True
    st = d["stages_ms"]
    assert set(st) == {"route", "select", "v_relayout", "attend"}
    assert sum(st.values()) <= d["value"] * 1.05
    assert d["step_ms"]["p10"] <= d["step_ms"]["median"] <= d["step_ms"]["p90"]


def test_stratified_blocks():
    for nb, per in ((1024, 64), (4096, 64), (64, 64), (10, 64)):
        b = bench.stratified_blocks(nb, per, seed=3)
        assert len(b) == min(nb, per) and len(set(b.tolist())) == len(b)
        assert b[0] == 0 and b[-1] == nb - 1 and list(b) == sorted(b)


def test_diagonal_pairs_count_three_quarters():
    assert bench.pair_flop(10, 0) == 10 * bench.PAIR_FLOP
    assert bench.pair_flop(10, 4) == 6 * bench.PAIR_FLOP + 3 * bench.PAIR_FLOP
