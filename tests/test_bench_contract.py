"""Host-side parts of bench.py that need no GPU: the one-GPU guard, the traffic figure
(used only while the kernel sources match the recorded digest) and the clock summary."""
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def write_traffic(path, gemm_digest, gemv_digest):
    with open(path, "w") as f:
        f.write("# comment: 1\n")
        f.write(f"gemm_source_sha256: {gemm_digest}\n")
        f.write("gemm_hbm_bytes_per_dispatch: 3288000000\n")
        f.write(f"gemv_source_sha256: {gemv_digest}\n")
        f.write("gemv_hbm_bytes_per_dispatch: 67316000\n")


def test_traffic_only_for_matching_sources(tmp_path, monkeypatch):
    p = tmp_path / "hbm_traffic.txt"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.read_traffic() == {}  # no file
    write_traffic(p, bench.source_digest(bench.GEMM_SRC), bench.source_digest(bench.GEMV_SRC))
    assert bench.read_traffic() == {"gemm": 3288000000.0, "gemv": 67316000.0}
    write_traffic(p, "0" * 16, bench.source_digest(bench.GEMV_SRC))  # GEMM sources changed
    assert bench.read_traffic() == {"gemv": 67316000.0}


def test_source_digest_depends_on_content_and_order(tmp_path):
    a, b = tmp_path / "a", tmp_path / "b"
    a.write_bytes(b"one")
    b.write_bytes(b"two")
    d = bench.source_digest([str(a), str(b)])
    assert len(d) == 16 and d != bench.source_digest([str(b), str(a)])
    b.write_bytes(b"three")
    assert d != bench.source_digest([str(a), str(b)])


def make_probe(samples, why=None):
    p = bench.ClockProbe.__new__(bench.ClockProbe)
    p.handle, p.why, p.samples, p.inited, p.seconds = None, why, list(samples), False, 2.5
    return p


def test_clock_summary_scales_the_peak():
    s = make_probe([2400.0, 1200.0, 1200.0]).summary(78.65, 157.3)
    assert s["gfxclk_mhz"] == 1200.0 and s["samples"] == 3
    assert s["peak_at_clock"] == pytest.approx(78.65)
    assert s["frac_at_clock"] == pytest.approx(1.0)
    assert s["gfxclk_mhz_min"] == 1200.0 and s["gfxclk_mhz_max"] == 2400.0


def test_clock_summary_without_a_rate_has_no_fraction():
    s = make_probe([1900.0, 1900.0]).summary(None, 2500.0)
    assert s["gfxclk_mhz"] == 1900.0 and "frac_at_clock" not in s
    assert s["peak_at_clock"] == pytest.approx(2500.0 * 1900 / 2400, abs=0.01)  # rounded to 0.01


def test_clock_summary_without_samples_says_why():
    assert make_probe([], why="amdsmi: no device") .summary(1.0, 157.3) == \
        {"gfxclk_mhz": None, "why": "amdsmi: no device"}
    assert make_probe([]).summary(1.0, 157.3)["gfxclk_mhz"] is None


def test_clock_measure_keeps_the_second_half(monkeypatch):
    """Readings taken in the first half of the run are dropped (the driver's cached
    metrics may predate the load)."""
    p = make_probe([])
    p.handle = object()
    reads = iter([100.0, 100.0, 2000.0, 2000.0, 2000.0, 2000.0])
    p.read = lambda: next(reads)
    t = iter([0.0, 0.1, 0.2, 0.3, 0.5, 0.7, 0.9, 1.0])
    monkeypatch.setattr(bench.time, "perf_counter", lambda: next(t))
    monkeypatch.setattr(bench.time, "sleep", lambda s: None)

    class Ev:
        n = 0

        def record(self, stream):
            pass

        def query(self):
            Ev.n += 1
            return Ev.n > 6

    fake_torch = types.SimpleNamespace(cuda=types.SimpleNamespace(Event=Ev))
    launches = []
    p.measure(fake_torch, None, lambda: launches.append(1), 1.0, 0.25)
    assert len(launches) == 4
    assert p.samples == [2000.0, 2000.0, 2000.0] and p.seconds == 1.0
