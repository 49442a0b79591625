"""Host-side logic of the benchmark (no GPU): the counter summaries it turns
rocprofv3 --pmc files into, the traffic lookup keyed by kernel-source hashes,
and the one-GPU refusal."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
CALIB = "void at::native::vectorized_elementwise_kernel<4, at::native::CUDAFunctorOnSelf_add<float> >(int, float*)"
STEP1 = "void oasis::(anonymous namespace)::attn_score_kernel<128, 2, 1, 2>(unsigned short const*, int)"
SCORE = "void oasis::(anonymous namespace)::score_mfma_kernel<128, 1>(unsigned short const*, int)"


def _write(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            r = {f: 0 for f in FIELDS}
            r.update(Kernel_Name=name, Counter_Name=counter, Counter_Value=value, Dispatch_Id=i)
            w.writerow(r)


def test_traffic_summary_scales_by_the_calibration_copy(tmp_path):
    gib_kib = bench.CALIB_ELEMS * 4 / 1024
    fetch, write, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.txt"
    # the calibration add reads 1 GiB and writes 1 GiB; FETCH_SIZE reads half (factor 2)
    _write(fetch, "FETCH_SIZE", [(CALIB, gib_kib / 2), (STEP1, 1000.0), (STEP1, 1200.0), (SCORE, 300.0)])
    _write(write, "WRITE_SIZE", [(CALIB, gib_kib), (STEP1, 50.0), (STEP1, 70.0), (SCORE, 4.0)])
    bench.traffic_summary(str(fetch), str(write), str(out), "test")
    lines = open(out).read().splitlines()
    assert any(ln.startswith("calibration") and "fetch_factor 2.0000" in ln and "write_factor 1.0000" in ln
               for ln in lines)
    # mean over dispatches, scaled: (1100 * 2 + 60 * 1) KiB
    step = [ln for ln in lines if ln.startswith("op attend_and_score ")][0].split()
    assert float(step[5]) == pytest.approx((1100 * 2 + 60) * 1024)
    assert step[3] == bench.op_source_hash("attend_and_score")
    score = [ln for ln in lines if ln.startswith("op lookahead_score ")][0].split()
    assert float(score[5]) == pytest.approx((300 * 2 + 4) * 1024)


def test_traffic_summary_needs_the_calibration_kernel(tmp_path):
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    _write(fetch, "FETCH_SIZE", [(STEP1, 1000.0)])
    _write(write, "WRITE_SIZE", [(STEP1, 50.0)])
    with pytest.raises(SystemExit):
        bench.traffic_summary(str(fetch), str(write), str(tmp_path / "t.txt"), "test")


def test_load_traffic_drops_ops_whose_sources_changed(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    good = bench.op_source_hash("lookahead_score")
    (prof / "traffic_w.txt").write_text(
        f"op lookahead_score source {good} hbm_bytes 123\n"
        f"op attend_and_score source 0000000000000000 hbm_bytes 456\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_traffic("w") == {"lookahead_score": 123.0}
    assert bench.load_traffic("absent") == {}


def test_source_hash_covers_code_not_comments(tmp_path, monkeypatch):
    """Measured traffic stays valid across comment and whitespace edits of an
    op's sources and is dropped when their code changes."""
    src = tmp_path / "score.hip"
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    monkeypatch.setitem(bench.OP_SOURCES, "lookahead_score", ["score.hip"])
    src.write_text("// header\nint f(int x) {\n  return x + 1;  // one\n}\n")
    h0 = bench.op_source_hash("lookahead_score")
    src.write_text("/* a longer\n   header */\nint f(int x)   {\n\n  return x + 1;\n}\n")
    assert bench.op_source_hash("lookahead_score") == h0
    src.write_text("// header\nint f(int x) {\n  return x + 2;  // one\n}\n")
    assert bench.op_source_hash("lookahead_score") != h0


def test_counter_summary_means_per_kernel_and_counter(tmp_path):
    a, b, out = tmp_path / "a.csv", tmp_path / "b.csv", tmp_path / "c.txt"
    _write(a, "MfmaUtil", [(STEP1, 4.0), (STEP1, 6.0), (SCORE, 2.0)])
    _write(b, "OccupancyPercent", [(STEP1, 10.0), (SCORE, 20.0), (SCORE, 30.0)])
    bench.counter_summary([str(a), str(b)], str(out), "test")
    rows = {ln.split()[0]: ln.split()[1:] for ln in open(out).read().splitlines() if not ln.startswith("#")}
    assert rows["kernel"] == ["MfmaUtil(calls)", "OccupancyPercent(calls)"]
    assert rows["attn_score_kernel<128,2,1,2>"] == ["5(2)", "10(1)"]
    assert rows["score_mfma_kernel<128,1>"] == ["2(1)", "25(2)"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr
