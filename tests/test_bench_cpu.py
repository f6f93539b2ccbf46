"""CPU checks of bench.py's measurement plumbing (no GPU).

- code_lines keeps exactly the code of a C/C++ source: comment and blank-line edits do
  not change the kernel-source hash that a traffic figure is tied to, code edits do;
- summarize_profile scales FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what they read
  for the copy probe of known size.  With a copy of B bytes whose counters report B / 2
  KiB fetched (128-byte requests counted as 64 bytes) and B KiB written, the scales are
  2 and 1, and the GEMM's mean per dispatch is scaled the same way;
- measured_traffic returns the figure only while its source hash is the current one;
- the default warm-up runs at least the minimum count of steps and keeps going until
  the minimum time has passed; an explicit count runs exactly that many;
- bench.py measures one GPU: --gpus 2 exits with status 2 and says so.
"""
import csv
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_lines_ignores_comments_only():
    a = "int a = 1;  // one\n/* block\n   comment */\nint b = 2;\n\n   // only a comment\n"
    b = "int a = 1;\n\nint b = 2;   /* trailing */\n"
    assert bench.code_lines(a) == bench.code_lines(b) == ["int a = 1;", "int b = 2;"]
    assert bench.code_lines("int a = 3;") != bench.code_lines(a)[:1]


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="", encoding="utf-8") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def test_summarize_profile_scales_by_the_copy_probe(tmp_path):
    raw, prof = tmp_path / "raw", tmp_path / "prof"
    copy_mib = 4
    known = copy_mib << 20
    gemm = "void mosaic::gather_gemm_bf16_defer_kernel<1, 1, 16, true, false, true>(...)"
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float>>(...)"
    _write_csv(str(raw / "trace" / "trace_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs", "Percentage"],
               [[gemm, 4, 12e6, 3e6, 2.9e6, 3.1e6, 99.0], [copy, 3, 1e6, 3.3e5, 3.2e5, 3.4e5, 1.0]])
    _write_csv(str(raw / "fetch" / "fetch_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"],
               [[gemm, "FETCH_SIZE", 1000], [gemm, "FETCH_SIZE", 3000]] +
               [[copy, "FETCH_SIZE", known / 1024 / 2]] * 3)
    _write_csv(str(raw / "write" / "write_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"],
               [[gemm, "WRITE_SIZE", 500], [gemm, "WRITE_SIZE", 500]] + [[copy, "WRITE_SIZE", known / 1024]] * 3)
    (raw / "commands.txt").write_text("rocprofv3 --kernel-trace --stats -- python3 bench.py\n")
    # the traced run's own result line: its source hash and algorithmic bytes are what the
    # summary keeps (not the hash of the sources present when it is summarised)
    (raw / "trace.log").write_text("[bench] noise\n" + json.dumps(
        {"roofline": {"kernel_source_hash": bench.kernel_source_hash(),
                      "algorithmic_bytes_per_launch": 1000 * 1024}}) + "\n")
    os.makedirs(prof)
    bench.summarize_profile(str(raw), "wl", copy_mib, "logits", prof_dir=str(prof))

    t = json.loads((prof / "traffic_gather_gemm_wl.json").read_text())
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    assert t["fetch_bytes_per_launch"] == 2000 * 1024 * 2
    assert t["write_bytes_per_launch"] == 500 * 1024
    assert t["bytes_per_launch"] == 2000 * 1024 * 2 + 500 * 1024
    assert t["kernel_source_hash"] == bench.kernel_source_hash()
    md = (prof / "gather_gemm_wl_rocprof.md").read_text()
    assert "rocprofv3 --kernel-trace --stats" in md and "| 4 | 12.000 | 3000.0 |" in md
    assert "L2-miss / algorithmic = 4.50" in md     # (2000 * 2 + 500) KiB over 1000 KiB

    assert bench.measured_traffic("wl", "logits", prof_dir=str(prof)) == t["bytes_per_launch"]
    t["kernel_source_hash"] = "0" * 16
    (prof / "traffic_gather_gemm_wl.json").write_text(json.dumps(t))
    assert bench.measured_traffic("wl", "logits", prof_dir=str(prof)) is None
    assert bench.measured_traffic("absent", "logits", prof_dir=str(prof)) is None

    # output of a run on other sources keeps that run's hash, so it never matches these
    (raw / "trace.log").write_text(json.dumps({"roofline": {"kernel_source_hash": "f" * 16}}) + "\n")
    bench.summarize_profile(str(raw), "wl", copy_mib, "logits", prof_dir=str(prof))
    assert bench.measured_traffic("wl", "logits", prof_dir=str(prof)) is None


def test_source_hash_follows_the_paths_kernels():
    # the fp8 path's figures hang on the FP8 kernels' source, the others' on the bf16 kernels'
    assert bench.kernel_source_hash("argmax_lse") == bench.kernel_source_hash("logits")
    assert bench.kernel_source_hash("dense_select") == bench.kernel_source_hash("logits")
    assert bench.kernel_source_hash("fp8") != bench.kernel_source_hash("logits")


def test_no_traffic_without_both_counters(tmp_path):
    raw, prof = tmp_path / "raw", tmp_path / "prof"
    _write_csv(str(raw / "fetch" / "fetch_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"],
               [["gather_gemm_lowm_kernel", "FETCH_SIZE", 10]])
    os.makedirs(prof)
    bench.summarize_profile(str(raw), "wl", 4, "logits", prof_dir=str(prof))
    assert not (prof / "traffic_gather_gemm_wl.json").exists()
    assert (prof / "gather_gemm_wl_rocprof.md").exists()


class _FakeClock:
    """Wall clock that advances by a fixed time per step."""

    def __init__(self, step_s):
        self.t, self.step_s = 0.0, step_s

    def __call__(self):
        return self.t

    def step(self):
        self.t += self.step_s


def test_warm_up_by_time_and_by_count():
    # 1-ms steps: 0.15 s of work needs 150 steps
    clk = _FakeClock(0.001)
    syncs = []
    n = bench.warm_up(clk.step, None, min_steps=3, min_seconds=0.15, sync=lambda: syncs.append(1), clock=clk)
    assert n == 150 and len(syncs) == 150
    # 100-ms steps: the minimum count decides
    clk = _FakeClock(0.1)
    assert bench.warm_up(clk.step, None, min_steps=3, min_seconds=0.15, clock=clk) == 3
    # an explicit count runs exactly that many, including none
    clk = _FakeClock(0.001)
    assert bench.warm_up(clk.step, 5, clock=clk) == 5 and abs(clk.t - 0.005) < 1e-12
    assert bench.warm_up(clk.step, 0, clock=clk) == 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
