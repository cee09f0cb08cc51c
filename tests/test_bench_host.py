"""Host-side pieces of bench.py.  CPU only: nothing here touches a GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from linear_attention_recurrent_gdn_amd import inputs as I  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)


def test_practical_read_without_the_probe_is_none(monkeypatch, tmp_path):
    from linear_attention_recurrent_gdn_amd import _build

    monkeypatch.setattr(_build, "PROBE", str(tmp_path / "missing"))
    assert bench.practical_read(56397824) is None


def test_practical_read_takes_the_best_grid(monkeypatch, tmp_path):
    # a stand-in probe that prints the probe's JSON lines for two grid sizes
    from linear_attention_recurrent_gdn_amd import _build

    fake = tmp_path / "probe.py"
    fake.write_text(
        "import sys, json\n"
        "n = int(sys.argv[1])\n"
        "print(json.dumps({'bytes': n, 'grid': 1024, 'us': 10.0, 'TBps': n / 10.0e6}))\n"
        "print(json.dumps({'bytes': n, 'grid': 2048, 'us': 8.0, 'TBps': n / 8.0e6}))\n")
    launcher = tmp_path / "probe"
    launcher.write_text(f"#!/bin/sh\nexec {sys.executable} {fake} \"$@\"\n")
    launcher.chmod(0o755)
    monkeypatch.setattr(_build, "PROBE", str(launcher))
    r = bench.practical_read(64_000_000)
    assert r["grid"] == 2048 and r["us"] == 8.0
    assert r["GBps"] == pytest.approx(64_000_000 / 8.0e6 * 1e3)


@pytest.mark.parametrize("name", ["gdn_decode", "kda_decode", "gdn_serving", "hybrid_stack"])
def test_decode_bytes_grow_by_one_entry_per_token(name):
    wl = I.WORKLOADS[name]
    step = [bench.decode_bytes(wl, j + 1) - bench.decode_bytes(wl, j) for j in range(wl.window - 1)]
    assert len(set(step)) == 1 and step[0] > 0
