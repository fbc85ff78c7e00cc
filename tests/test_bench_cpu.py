"""Host logic of bench.py, on the CPU: the single-GPU refusal, the clock-settle loop and
the rule that keeps the recorded HBM traffic only while the kernel source is unchanged."""
import json
import os
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


class _FakeClock:
    """Stands in for torch.cuda: launches advance a clock by a per-launch duration that
    falls as the 'GPU' warms up, events read the clock."""

    def __init__(self, durations):
        self.durations = list(durations)
        self.t = 0.0
        self.launches = 0
        clock = self

        class _Event:
            def __init__(self, enable_timing=True):
                self.at = None

            def record(self):
                self.at = clock.t

            def elapsed_time(self, other):
                return other.at - self.at

        class _Cuda:
            Event = _Event

            @staticmethod
            def synchronize():
                pass

        self.cuda = _Cuda

    def launch(self, _i):
        d = self.durations[min(self.launches, len(self.durations) - 1)]
        self.launches += 1
        self.t += d


def test_settle_runs_until_the_launch_time_stops_falling():
    # 0.6 ms at first, falling linearly to 0.5 ms over 40 launches, then flat.
    durs = [0.6 - 0.1 * min(i, 40) / 40 for i in range(400)]
    fake = _FakeClock(durs)
    n, first, last = bench.settle(fake.launch, fake, max_s=5.0)
    assert first == pytest.approx(0.6)
    assert last == pytest.approx(0.5, rel=1e-6)
    assert n == fake.launches and n > 40   # it ran past the ramp


def test_settle_stops_at_its_time_limit():
    # Never settles (keeps falling by 5 % per launch); the wall-clock limit ends it.
    fake = _FakeClock([1.0 * 0.95 ** i for i in range(100000)])
    n, _first, _last = bench.settle(fake.launch, fake, max_s=0.05)
    assert n >= 1


def test_traffic_is_kept_only_for_the_recorded_source(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel v1\n")
    rec = tmp_path / "traffic.json"
    rec.write_text(json.dumps({"source_sha256": bench.source_sha(str(src)), "hbm_bytes_per_launch": 123.0}))
    monkeypatch.setattr(bench, "ATTN_KERNEL_SRC", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.load_traffic(1.0) == 123.0
    src.write_text("// kernel v2\n")
    assert bench.load_traffic(1.0) is None

