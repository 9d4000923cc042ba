"""bench.py's command-line contract on the host: one GPU only, and the
counter-summary helper reads rocprofv3 CSVs per dispatch (CPU-only)."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, cwd=ROOT, env=e,
                          timeout=120)


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = _run("--gpus", n)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_a_rank_of_a_multi_process_launch_is_refused():
    r = _run("--gpus", "1", env={"WORLD_SIZE": "2"})
    assert r.returncode == 2 and "one GPU" in r.stderr


def _write_counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_counter_helper_sums_per_dispatch(tmp_path):
    """rocprofv3 writes one row per counter instance; the helper sums the rows
    of each dispatch of the matching kernels and counts the dispatches."""
    sys.path.insert(0, ROOT)
    try:
        import bench
    finally:
        sys.path.pop(0)
    p = str(tmp_path / "c.csv")
    _write_counter_csv(p, [
        {"Dispatch_Id": 1, "Kernel_Name": "moe::ffn_decode_bf16<1>", "Counter_Name": "FETCH_SIZE", "Counter_Value": 10},
        {"Dispatch_Id": 1, "Kernel_Name": "moe::ffn_decode_bf16<1>", "Counter_Name": "FETCH_SIZE", "Counter_Value": 5},
        {"Dispatch_Id": 2, "Kernel_Name": "moe::ffn_decode_bf16<2>", "Counter_Name": "FETCH_SIZE", "Counter_Value": 7},
        {"Dispatch_Id": 3, "Kernel_Name": "moe::gate_kernel", "Counter_Name": "FETCH_SIZE", "Counter_Value": 100},
        {"Dispatch_Id": 2, "Kernel_Name": "moe::ffn_decode_bf16<2>", "Counter_Name": "WRITE_SIZE", "Counter_Value": 3},
    ])
    total, n = bench._counter_per_dispatch(p, "FETCH_SIZE", "ffn_")
    assert (total, n) == (22.0, 2)
    total, n = bench._counter_per_dispatch(p, "WRITE_SIZE", "ffn_")
    assert (total, n) == (3.0, 1)
    assert bench._counter_per_dispatch(p, "FETCH_SIZE", "nothing") == (0, 0)
