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


@pytest.mark.parametrize("name,layers", [("gdn_decode", 1), ("kda_decode", 1), ("gdn_serving", 1),
                                         ("hybrid_stack", 36), ("tiny_gdn", 1)])
def test_staggered_schedule_reaches_offsets_and_spreads_flushes(name, layers):
    # the set-up phase ends with every (layer, sequence) at its offset; after
    # it, every window of W consecutive steps flushes every unit exactly once,
    # and any K consecutive steps flush K/W of the units, within one group
    import numpy as np

    wl = I.WORKLOADS[name]
    sch = bench.Schedule(wl, layers)
    W = wl.window
    for t in range(W):
        sch.step(setup_token=t)
    assert (sch.fill == sch.offsets).all()
    flushed = []
    for t in range(3 * W):
        calls = sch.step()
        assert all(forced is None for _, forced, _ in calls)  # after set-up only full windows flush
        flushed.append(sum(n_due for _, _, n_due in calls))
    flushed = np.array(flushed)
    for t in range(0, 2 * W):
        assert flushed[t:t + W].sum() == layers * wl.n_seq  # each sequence of each layer once per window
    groups = layers if layers > 1 else (W if wl.stagger else bench.stagger_groups(wl))
    per_group = layers * wl.n_seq // groups if layers == 1 else wl.n_seq
    for K in (5, 20, 64):
        for t in range(0, W):
            share = flushed[t:t + K].sum()
            assert abs(share - K * layers * wl.n_seq / W) <= per_group, (K, t, share)


def test_stagger_groups_leave_a_unit_per_cu():
    for name in ("gdn_decode", "kda_decode"):
        wl = I.WORKLOADS[name]
        G = bench.stagger_groups(wl)
        assert G > 1 and wl.n_units // G >= 256 and wl.window % G == 0


@pytest.mark.parametrize("name", ["gdn_decode", "kda_decode", "gdn_serving"])
def test_stagger_layouts_same_offsets_different_sequences(name):
    # both layouts give every offset to the same number of sequences; "blocks"
    # gives it to a run of consecutive sequences, the offsets falling along
    # the sequence index (so the fills do along the dispatch order, with one
    # wrap), "interleaved" to sequences s = g mod G
    import numpy as np

    wl = I.WORKLOADS[name]
    blocks = bench.window_offsets(wl, 1, "blocks")[0]
    inter = bench.window_offsets(wl, 1, "interleaved")[0]
    assert sorted(blocks.tolist()) == sorted(inter.tolist())
    G = wl.window if wl.stagger else bench.stagger_groups(wl)
    run = wl.n_seq // G
    assert (np.diff(blocks) <= 0).all()
    assert all(len(set(blocks[i:i + run].tolist())) == 1 for i in range(0, wl.n_seq, run))
    assert inter[0] == 0 and inter[1] == wl.window // G


def test_stack_offsets_ignore_layout():
    import numpy as np

    wl = I.WORKLOADS["hybrid_stack"]
    a = bench.window_offsets(wl, wl.layers, "blocks")
    b = bench.window_offsets(wl, wl.layers, "interleaved")
    assert (a == b).all() and (a[:, 0] == (np.arange(wl.layers) * wl.window) // wl.layers).all()
