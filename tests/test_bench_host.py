"""Host logic of bench.py: stored traffic counters apply only to the kernel
sources and workload they were taken on."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _write(tmp_path, **over):
    c = {"workload": "c2", "kernel_sources_sha256": bench.kernel_sources_sha256(),
         "fetch_kib": 1000.0, "write_kib": 500.0,
         "copy_1gib_fetch_kib": float(1 << 19), "copy_1gib_write_kib": float(1 << 20)}
    c.update(over)
    p = tmp_path / "counters.json"
    p.write_text(json.dumps(c))
    return str(p)


def test_traffic_scaled_by_copy_calibration(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "COUNTERS", _write(tmp_path))
    # fetch counter reads half of a copy's bytes -> x2; write counter exact -> x1
    assert bench.counter_traffic("c2") == (2 * 1000 + 500) * 1024


def test_traffic_null_on_other_sources_or_workload(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "COUNTERS", _write(tmp_path, kernel_sources_sha256="0" * 64))
    assert bench.counter_traffic("c2") is None
    monkeypatch.setattr(bench, "COUNTERS", _write(tmp_path))
    assert bench.counter_traffic("c3") is None
    monkeypatch.setattr(bench, "COUNTERS", str(tmp_path / "absent.json"))
    assert bench.counter_traffic("c2") is None


def test_hash_ignores_comments_only():
    src = "int a; // note\n/* block */ int b;\n"
    assert bench.normalize_source(src) == bench.normalize_source("int a;\nint b; // other\n")
    assert bench.normalize_source(src) != bench.normalize_source("int a; int c;")
    assert len(bench.kernel_sources_sha256()) == 64


def test_multi_gpu_refused():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_device_info_fields(monkeypatch):
    """device_info() runs on its own (bench imports torch inside main) and
    reports name, architecture and compute units of device 0."""
    import torch

    class Props:
        name = "AMD Instinct MI355X"
        gcnArchName = "gfx950:sramecc+:xnack-"
        multi_processor_count = 256

    monkeypatch.setattr(torch.cuda, "get_device_properties", lambda i: Props())
    d = bench.device_info()
    assert d["name"] == Props.name and d["arch"] == Props.gcnArchName and d["compute_units"] == 256
    assert "max_engine_clock_mhz" in d and "2.4 GHz" in d["peak_basis"]


def test_engine_clock_from_sysfs_levels(tmp_path, monkeypatch):
    """The highest level of an AMD card's pp_dpm_sclk; other vendors ignored."""
    import glob as _glob
    amd = tmp_path / "card1" / "device"
    amd.mkdir(parents=True)
    (amd / "vendor").write_text("0x1002\n")
    (amd / "pp_dpm_sclk").write_text("0: 500Mhz\n1: 1800Mhz *\n2: 2400Mhz\n")
    other = tmp_path / "card0" / "device"
    other.mkdir(parents=True)
    (other / "vendor").write_text("0x1a03\n")
    (other / "pp_dpm_sclk").write_text("0: 9999Mhz\n")
    real = _glob.glob
    monkeypatch.setattr(_glob, "glob", lambda pat: sorted(real(str(tmp_path / "card*" / "device" / "pp_dpm_sclk"))))
    assert bench.max_engine_clock_mhz() == 2400
