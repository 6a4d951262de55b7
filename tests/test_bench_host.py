"""Host-side checks of bench.py's arithmetic and protocol helpers (no GPU):
the algorithmic work and bytes the roofline divides by, the bound each
workload is priced against, the device warm-up helper, and the refusal of
more than one GPU."""

import os
import subprocess
import sys
from types import SimpleNamespace

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _shape(B, L, H, P, io, tv):
    return SimpleNamespace(B=B, L=L, H=H, P=P, io=io, time_varying=tv)


def test_algorithmic_counts_of_the_metric_workload():
    # B = 16, L = 16384, H = 128, P = 256, bf16: 8 P H flops per token
    # (4 P H for the drive, 4 P H for the readout), u in and y out in bf16,
    # the parameters once (lambda, B~ and C~ as complex64, D and log Delta)
    w = _shape(16, 16384, 128, 256, "bf16", False)
    tokens = 16 * 16384
    assert bench.algorithmic_flops(w) == 8 * 256 * 128 * tokens == 68_719_476_736
    params = 8 * 256 + 2 * 8 * 256 * 128 + 4 * 128 + 4 * 256
    assert bench.algorithmic_bytes(w) == tokens * 128 * 2 * 2 + params == 134_745_600


def test_time_varying_bytes_include_the_intervals():
    w = _shape(16, 16000, 96, 128, "f32", True)
    tokens = 16 * 16000
    params = 8 * 128 + 2 * 8 * 128 * 96 + 4 * 96 + 4 * 128
    assert bench.algorithmic_bytes(w) == tokens * 96 * 2 * 4 + tokens * 128 * 4 + params


def test_roofline_bound_per_workload():
    # the metric workload does 512 flop per byte: above the bf16 ridge
    # (2.5 PF/s / 8 TB/s = 312), so it is priced against the matrix cores;
    # the time-varying float32 workload is priced against HBM
    r3 = bench.roofline_fracs(_shape(16, 16384, 128, 256, "bf16", False), 0.0687, 0.110, {})
    assert r3["bound"] == "mfma"
    assert abs(r3["k_scan_mfma_frac"] - 68.719476736e9 / 68.7e-6 / 2.5e15) < 1e-3
    r4 = bench.roofline_fracs(_shape(16, 16000, 96, 128, "f32", True), 0.115, 0.197, {})
    assert r4["bound"] == "hbm"


def test_keep_busy_runs_whole_batches_for_the_time_given():
    calls, syncs = [], []
    fake_torch = SimpleNamespace(cuda=SimpleNamespace(synchronize=lambda: syncs.append(1)))
    n = bench.keep_busy(calls.append, fake_torch, 0.02, batch=7)
    assert n == len(calls) and n > 0 and n % 7 == 0
    assert calls == list(range(n)) and len(syncs) == n // 7
    assert bench.keep_busy(calls.append, fake_torch, 0.0) == 0


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, cwd=ROOT, timeout=300)
    assert out.returncode == 2 and "one GPU" in out.stderr
