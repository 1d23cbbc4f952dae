"""Host logic of bench.py (CPU): the one-GPU guard, the layer count that
keeps a timed step cold, the traffic record's source check, and the phase
breakdown's arithmetic on synthetic timestamps."""

import json
import os
import subprocess
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    for args, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                           text=True, timeout=120, env=dict(os.environ, **env), cwd=ROOT)
        assert r.returncode == 2, (args, env, r.stderr[-400:])
        assert "one GPU" in r.stderr and r.stdout == ""


def test_layers_for_keeps_a_step_above_one_gib():
    assert bench.layers_for(1) == 256          # capped
    assert bench.layers_for(1 << 30) == 4      # at least four layers
    assert bench.layers_for(32792580) == 33    # the kv_len-8000 layer: 33 x 32.8 MB >= 1 GiB
    for b in (4_100_000, 12_290_000, 98_300_000):
        n = bench.layers_for(b)
        assert n * b >= (1 << 30) or n == 256


def test_traffic_record_needs_the_current_source(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    rec = {"workload": "W", "source_digest": "abc", "hbm_bytes_per_launch": 123}
    (tmp_path / "profiles" / "decode_kernel_d256_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "abc")
    assert bench.measured_traffic("W") == 123
    assert bench.measured_traffic("other workload") is None
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "changed")
    assert bench.measured_traffic("W") is None
    (tmp_path / "profiles" / "decode_kernel_d256_traffic.json").write_text("not json")
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "abc")
    assert bench.measured_traffic("W") is None


def test_phase_breakdown_arithmetic():
    """One launch of four active splits of one unit; split 3 arrives last and
    merges, split 2 is a helper.  Ticks are 10 ns (100 MHz)."""
    t = np.zeros((4, 16), dtype=np.int64)
    start = np.array([1000, 1010, 1020, 1030])
    for w in range(4):
        t[w, 0] = start[w]
        for k in range(1, 7):
            t[w, k] = start[w] + 100 * k
        t[w, 14] = w  # arrival rank
        role = 1 if w == 3 else (2 if w == 2 else 3)
        t[w, 15] = w | (0 << 16) | (4 << 32) | (role << 48)
    for w in (2, 3):
        t[w, 7] = start[w] + 700
        t[w, 8] = start[w] + 900
        t[w, 13] = 1
    b = bench.phase_breakdown(torch.from_numpy(t.reshape(-1)).view(4, 16), 1, 4)
    close = lambda a, e: abs(a - e) < 1e-9  # noqa: E731
    assert close(b["last start"], 0.3)
    for k, name in enumerate(bench.PHASES, start=1):
        assert close(b[name + " (median)"], k + 0.15) and close(b[name + " (last)"], k + 0.3)
    assert close(b["merge begins (median)"], 7.25) and close(b["merge ends (last)"], 9.3)
    assert close(b["last arrival's merge and claims"], 2.0) and close(b["helper merge"], 2.0)
    assert close(b["helper start after last arrival"], 7.2 - 6.3)
    assert close(b["helpers end (last)"], 9.2) and close(b["last arrivals end (last)"], 9.3)
    assert b["merging workgroups"] == 2 and b["active workgroups"] == 4 and b["slices per last arrival"] == 1
