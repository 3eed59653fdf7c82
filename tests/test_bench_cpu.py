"""Host logic of bench.py, on the CPU: the one-GPU guard exits before any GPU
work, the committed HBM traffic record is used only while the kernel source
it was measured on is unchanged, and the warm-up runs for its GPU time."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("argv, env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, capture_output=True, text=True,
                       env=dict(os.environ, **env), timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_records_are_used_only_on_their_source():
    # a committed counter record counts only while the kernel source it was
    # measured on is unchanged; otherwise the bench reports traffic as null
    recs = json.load(open(bench.TRAFFIC_FILE))
    assert recs
    for key, rec in recs.items():
        t = bench.measured_traffic(key)
        if rec["source_sha"] != bench.source_sha(rec["source"]):
            assert t is None, key
        else:
            assert t is not None and t["total_bytes"] == rec["fetch_bytes"] + rec["write_bytes"]
            assert t["total_bytes"] > 0 and rec["algorithmic_bytes"] > 0


def test_stale_or_missing_traffic_record_reads_as_none(tmp_path, monkeypatch):
    recs = json.load(open(bench.TRAFFIC_FILE))
    key = sorted(recs)[0]
    stale = dict(recs)
    stale[key] = dict(recs[key], source_sha="0" * 16)
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(stale))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.measured_traffic(key) is None
    assert bench.measured_traffic("no_such_kernel") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.json"))
    assert bench.measured_traffic(key) is None


def test_copy_calibration_uses_the_three_large_copies_only():
    # readings (KiB per dispatch) of one counter run: three 1 GiB copies and
    # a small copy made by the runtime; the small one must not dilute the scale
    assert abs(bench.copy_scale([524308.4, 524299.5, 524299.5, 6.6]) - 2.0) < 1e-3
    assert bench.copy_scale([1048576.0, 1048576.0, 1048576.0, 8.0]) == 1.0
    with pytest.raises(ValueError):
        bench.copy_scale([524308.4, 6.6])


def test_cpu_model_is_a_string_or_none():
    m = bench.cpu_model()
    assert m is None or (isinstance(m, str) and m)


class _FakeClockTorch:
    """Stands in for torch in bench.warm(): every launch advances a GPU clock
    by a fixed time, and events read that clock."""

    def __init__(self, us_per_call):
        self.now_ms = 0.0
        self.us = us_per_call
        outer = self

        class Event:
            def __init__(self, enable_timing=False):
                self.t = None

            def record(self):
                self.t = outer.now_ms

            def synchronize(self):
                pass

            def elapsed_time(self, other):
                return other.t - self.t

        class _Cuda:
            pass

        self.cuda = _Cuda()
        self.cuda.Event = Event

    def launch(self, k):
        self.now_ms += self.us / 1000.0


@pytest.mark.parametrize("us, calls", [(500.0, 60), (31.0, 968), (1e4, 4)])
def test_warm_up_runs_for_at_least_its_gpu_time(us, calls):
    # warm() keeps calling the section's launches until 30 ms of GPU time
    # have passed, checking every 4 calls
    t = _FakeClockTorch(us)
    n = bench.warm(t, t.launch)
    assert n == calls
    assert t.now_ms >= 30.0


def test_warm_up_stops_at_its_call_limit():
    t = _FakeClockTorch(0.001)
    assert bench.warm(t, t.launch, max_calls=100) == 100


def test_trial_statistics_are_order_statistics():
    # 20 trials of 5 calls: median and spread come from the sorted per-call times
    t = _FakeClockTorch(100.0)
    calls = [0]

    def f():
        calls[0] += 1
        t.now_ms += 0.1 * (1 + calls[0] % 3)     # 0.1, 0.2 or 0.3 ms per call

    r = bench.trials(t, f, n_trials=20, per=5)
    assert calls[0] == 100 and r["trials"] == 20 and r["calls_per_trial"] == 5
    assert r["min_ms"] <= r["p10_ms"] <= r["median_ms"] <= r["p90_ms"] <= r["max_ms"]
    assert abs(r["median_ms"] - 0.2) < 0.03


def test_warm_up_honours_its_minimum_call_count():
    t = _FakeClockTorch(1e4)          # 10 ms per call: 30 ms is reached after 4 calls
    assert bench.warm(t, t.launch, min_calls=10) == 12
