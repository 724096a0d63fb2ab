"""Host logic of bench.py (CPU only): the one-GPU contract, the lookup of the
committed traffic figures, and the parser of the driver's clock report."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "--gpus 2 is not supported" in r.stderr
    assert r.stdout == ""


def test_traffic_lookup(bench, tmp_path, monkeypatch):
    sha = bench.kernel_source_sha256()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_w.json").write_text(json.dumps(
        {"workload": "w", "source_sha256": sha, "kernels": {"k": {"bytes": 1234.4}}}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda: sha)
    assert bench.measured_traffic("w", "k") == 1234
    # another partial dtype than the profiled run's, another kernel, another workload
    assert bench.measured_traffic("w", "k", "bf16") is None
    assert bench.measured_traffic("w", "other") is None
    assert bench.measured_traffic("none", "k") is None
    # kernels changed since the profile was taken
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda: "0" * 64)
    assert bench.measured_traffic("w", "k") is None


def test_committed_traffic_is_read_when_current(bench):
    """When the committed traffic profiles were taken with the current kernel
    sources, the bench reads them (above the algorithmic bytes); after a kernel
    change they are stale and the bench reports null, which this skips."""
    stale = []
    for w in ("7b_tp8", "7b_tp8_bwd", "7b_tp8_bwd_fp8", "7b_tp8_attn"):
        with open(os.path.join(ROOT, "profiles", f"traffic_{w}.json")) as fh:
            t = json.load(fh)
        if t["source_sha256"] != bench.kernel_source_sha256():
            stale.append(w)
    if stale:
        pytest.skip(f"traffic profiles predate the current kernel sources: {stale}")
    assert bench.measured_traffic("7b_tp8", "row_partial") > 184549376


@pytest.mark.parametrize("text,mhz", [
    ("0: 500Mhz\n1: 2400Mhz *\n", 2400.0),
    ("S: 94Mhz *\n0: 500Mhz\n1: 2400Mhz\n", 94.0),
    ("0: 500Mhz\n1: 2400Mhz\n", None),
])
def test_clock_line_parser(bench, tmp_path, text, mhz):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text(text)
    c = bench.ClockSampler()
    c.path = str(f)
    assert c._read() == mhz


def test_clock_sampler_without_a_source_reports_nothing(bench):
    c = bench.ClockSampler()
    c.path = None
    with c:
        pass
    assert c.summary() is None
