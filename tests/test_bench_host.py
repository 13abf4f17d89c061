"""Host-side logic of bench.py that runs without a GPU: the clock record's window selection and the refusal
of more than one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def sampler_with(windows):
    s = bench.ClockSampler.__new__(bench.ClockSampler)   # no amdsmi: the windows are given
    s.period_s, s.windows, s.error = 0.02, list(windows), None
    return s


def test_clock_record_keeps_only_windows_inside_the_busy_span():
    """A refresh first seen at t averages the second before it: it counts only when t - 1.05 s is not before
    the busy span's start and t is not after its end."""
    s = sampler_with([(10.5, [100] * 8),                 # averages idle time before the steps started
                      (11.2, [2000, 2100] + [2050] * 6),  # inside
                      (12.2, [1990] + [2010] * 7),        # inside
                      (13.5, [150] * 8)])                 # after the timed region
    r = s.record(busy_from=10.0, busy_to=13.0)
    assert r["windows"] == 2 and r["xcds"] == 8
    assert r["MHz_min_xcd"] == 1990 and r["MHz_max_xcd"] == 2100
    assert r["MHz_mean"] == pytest.approx((2000 + 2100 + 6 * 2050 + 1990 + 7 * 2010) / 16, abs=0.05)


def test_clock_record_without_windows_says_why():
    s = sampler_with([])
    s.error = "AmdSmiLibraryException: driver not loaded"
    r = s.record(0.0, 1.0)
    assert r["windows"] == 0 and "MHz_mean" not in r and "driver" in r["error"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_sampler_start_and_stop_do_not_block():
    """start() and stop() return promptly whether or not amdsmi finds a driver (without one, as on a host
    with no GPU, the record carries the reason)."""
    import time

    s = bench.ClockSampler()
    t0 = time.perf_counter()
    s.start()
    time.sleep(0.05)
    s.stop()
    assert time.perf_counter() - t0 < 5.0
    r = s.record(0.0, 1e18)
    assert isinstance(r["windows"], int)
    assert "error" not in r or (isinstance(r["error"], str) and r["error"])


def test_also_rejects_unknown_or_repeated_workloads():
    """--also names other workloads; an unknown name, or the headline itself, is refused before any GPU
    work."""
    for also in ("nosuch", "moe"):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--also", also], capture_output=True,
                           text=True, timeout=120)
        assert r.returncode == 2 and "--also" in r.stderr and r.stdout == ""
