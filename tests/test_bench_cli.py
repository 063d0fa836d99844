"""bench.py's command line and line handling on the host (no GPU)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    cp = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                        text=True, timeout=120)
    assert cp.returncode == 2
    assert "one GPU" in cp.stderr
    assert cp.stdout.strip() == ""


def test_other_workload_summary_keeps_the_figures():
    import bench
    line = json.dumps({"metric": bench.METRIC, "value": 5799.1, "unit": "GB/s", "steps": 3, "warmup": 1,
                       "ms_per_step": 11.85, "dtype": "bf16",
                       "config": {"workload": "long: 32 layers", "us_per_step": 11850.0, "tail_waste_slots": 0},
                       "roofline": {"achieved": 5915.0, "frac": 0.7394, "avg_us": 359.4}})
    row = bench.summarize_line(line)
    assert row == {"value": 5799.1, "unit": "GB/s", "us_per_step": 11850.0, "steps": 3, "warmup": 1, "dtype": "bf16",
                   "roofline_achieved": 5915.0, "roofline_frac": 0.7394, "kernel_avg_us": 359.4,
                   "tail_waste_slots": 0, "config": "long: 32 layers"}


def test_other_workloads_cover_every_bench_workload():
    import bench
    names = [n for n, _ in bench.OTHER_WORKLOADS]
    assert names == ["gqa8b-fp8", "gqa8b-int8", "sweep_b8", "sweep_b16", "sweep_b32", "fork-shared", "long"]
    for _, extra in bench.OTHER_WORKLOADS:
        assert "--no-others" not in extra  # added by the runner itself
