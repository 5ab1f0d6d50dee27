"""Host-side parts of bench.py that need no GPU: the one-GPU contract, the launch-curve
line fit, and the counter-summary lookup keyed to the kernel source."""

import hashlib
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_launch_line_fit_recovers_a_known_line():
    # a rate of R GB/s moves R * 1e3 bytes per microsecond
    fixed, rate = 14.0, 6000.0
    pts = [{"k": k, "kv_bytes": k * 2 ** 20, "us": fixed + k * 2 ** 20 / (rate * 1e3)}
           for k in (0, 8, 64, 128, 256, 1024)]
    f, g = bench.fit_launch_line(pts, 64)
    assert abs(f - fixed) < 1e-9 and abs(g - rate) < 1e-6


def test_launch_line_fit_ignores_points_below_k_min():
    pts = [{"k": 0, "kv_bytes": 0, "us": 100.0},            # far off the line
           {"k": 64, "kv_bytes": 64, "us": 10.0 + 64e-3},
           {"k": 128, "kv_bytes": 128, "us": 10.0 + 128e-3}]
    f, g = bench.fit_launch_line(pts, 64)
    assert abs(f - 10.0) < 1e-9 and abs(g - 1.0) < 1e-9


def test_launch_line_fit_without_positive_slope_has_no_rate():
    pts = [{"k": 64, "kv_bytes": 64, "us": 5.0}, {"k": 128, "kv_bytes": 128, "us": 5.0}]
    f, g = bench.fit_launch_line(pts, 64)
    assert f == 5.0 and g is None


def test_counter_fields_follow_the_kernel_source(tmp_path, monkeypatch):
    src = tmp_path / "attn.hip"
    src.write_text("kernel source\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    summary = tmp_path / "attn_kernel_{workload}_counters.txt"
    (tmp_path / "attn_kernel_w_counters.txt").write_text(
        f"# comment: ignored\nsource_sha256: {sha}\ntraffic_bytes_per_launch: 123\n")
    monkeypatch.setattr(bench, "ATTN_SRC", str(src))
    monkeypatch.setattr(bench, "COUNTERS", str(summary))
    assert bench.counter_field("w", "traffic_bytes_per_launch") == 123.0
    assert bench.counter_field("w", "missing_field") is None
    assert bench.counter_field("other", "traffic_bytes_per_launch") is None
    src.write_text("changed kernel source\n")   # counters now belong to another source
    assert bench.counter_field("w", "traffic_bytes_per_launch") is None


def test_all_bytes_counts_each_buffer_once():
    # the c0 shape (1 seq, 8/2 heads, d 64, fp32, bs 32, T 4, ctx 2048, k 16), by hand:
    # algorithmic 557056 (512 tokens x 2 heads x 64 x K,V x 4 B + 64 x 2 x 64 x 4 B reps);
    # per layer: Q in + O out 16384, draft K/V 4096, table 256, indices read 136;
    # selecting layer: indices written 136, first-draft Q 2048, table 256, scores 1024;
    # split partials (S + 1) x 2 units x 16 rows x 66 floats x 4 B, written and read
    from block_sparse_speculative_amd import synth
    from block_sparse_speculative_amd import workload as WL
    w = synth.WORKLOADS["tiny"]
    assert WL.algorithmic_bytes(w, [2048], 1) == 557056
    assert WL.all_bytes(w, [2048], 1, 16, 1) == 557056 + 16384 + 4096 + 256 + 136 + 3464
    assert WL.all_bytes(w, [2048], 1, 16, 3) == 581392 + 2 * 4 * 2 * 16 * 66 * 4
