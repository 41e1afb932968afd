"""The benchmark's accounting on the CPU: the frozen operation model it reads, the kernel names
it reports, and its refusal of more than one GPU (no device is touched)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_operation_model_totals():
    # the method's own work per forward + backward state-step and what each kernel issues
    assert bench.method_slots() == 30.25
    assert bench.op_slots("fwd") == 16.5
    assert bench.op_slots("bwd") == 29.25
    recompute = bench._slots(lambda v: v["credit"] == "recompute")
    assert recompute == 15.5
    assert bench.method_slots() + recompute == bench.op_slots("fwd") + bench.op_slots("bwd")
    assert abs(bench.PEAK_TOPS - 256 * 4 * 16 * 2.4e9 / 1e12) < 1e-9
    # the step roofline: 1.30e12 state-steps/s; >= 50% of it means <= 105.7 ms at workload 3
    ceiling = bench.PEAK_TOPS * 1e12 / bench.method_slots()
    assert abs(ceiling - 1.2999e12) < 1e9
    assert abs(65536 * 256 * 4096 / (0.5 * ceiling) * 1e3 - 105.7) < 0.1


def test_kernel_names():
    assert bench.kernel_names(12, 2) == ("k_sparse_fwd", "k_sparse_bwd")
    assert bench.kernel_names(8, 2) == ("k_sparse_fwd", "k_sparse_bwd")
    assert bench.kernel_names(16, 2) == ("k_sparse_fwd_wide", "k_sparse_bwd_wide")
    assert bench.kernel_names(15, 2) == ("k_sparse_fwd", "k_sparse_bwd_wide")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
