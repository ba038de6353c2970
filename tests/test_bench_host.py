"""Host-side helpers of bench.py (no GPU).

The bench line's roofline.traffic comes from the committed HBM-traffic
summary only while the permute kernel's source still hashes to the value
recorded there.  These tests check that the hash finds the kernel in the
source (a rewrite of the kernel's surroundings once made the lookup fail and
the whole run abort), that a stale or foreign record yields no traffic
figure, and that the timing summary reports the distribution it claims.
"""
import importlib.util
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_permute_source_hash_finds_the_kernel(bench):
    h = bench.permute_source_sha256()
    assert h is not None and len(h) == 64


def test_recorded_traffic_only_for_the_matching_source(bench, tmp_path, monkeypatch):
    rec = tmp_path / "traffic.md"
    rec.write_text(f"kernel_source_sha256: {bench.permute_source_sha256()}\n"
                   "traffic_bytes_per_launch: 1234567\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.recorded_traffic(2) == 1234567.0
    assert bench.recorded_traffic(3) is None          # another workload
    rec.write_text("kernel_source_sha256: " + "0" * 64 + "\ntraffic_bytes_per_launch: 1234567\n")
    assert bench.recorded_traffic(2) is None          # stale: the kernel changed since
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.recorded_traffic(2) is None


def test_dist_us_summary(bench):
    ms = np.array([1.0, 2.0, 3.0, 4.0]) * 1e-3
    d = bench.dist_us(ms)
    assert d["n"] == 4 and d["max"] == pytest.approx(4.0) and d["median"] == pytest.approx(2.5)
    assert d["mean"] == pytest.approx(2.5) and 3.9 <= d["p99"] <= 4.0
    assert bench.dist_us(ms, per=2)["max"] == pytest.approx(2.0)
