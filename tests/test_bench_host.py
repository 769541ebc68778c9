"""Host-side figures that bench.py reports (no GPU): the executed-FLOP count
of the kernel's wave-tiles, checked by brute force over every row's visible
keys, and the algorithmic byte count's parts."""
from __future__ import annotations

import numpy as np
import pytest

import bench
from workloads import make_case, make_custom_case


def _brute_tiles(case, rows_wg=256, kbk=64):
    """Number of (wave, key tile) pairs that hold at least one key some row of
    the wave may see, counted one row and one key at a time."""
    G = case["num_qo_heads"] // case["num_kv_heads"]
    gw = min(G, 16)
    tq = rows_wg // gw
    W = case["window_left"]
    n = 0
    for q_len, kv_len in zip(case["q_lens"], case["kv_lens"]):
        prefix = kv_len - q_len
        for t0 in range(0, q_len, tq):
            ntok = min(tq, q_len - t0)
            for w in range(rows_wg // 32):
                tiles = set()
                for r in range(w * 32, w * 32 + 32):
                    tok = r // gw
                    if tok >= ntok:
                        continue
                    pos = prefix + t0 + tok
                    for k in range(kv_len):
                        if k <= pos and (W < 0 or pos - k <= W):
                            tiles.add(k // kbk)
                n += len(tiles)
    return n


@pytest.mark.parametrize("spec", [
    dict(num_qo_heads=8, num_kv_heads=2, q_lens=(70, 1, 33), prefix_lens=(5, 40, 0)),
    dict(num_qo_heads=32, num_kv_heads=2, q_lens=(130, 17), prefix_lens=(0, 200), window_left=40),
    dict(num_qo_heads=4, num_kv_heads=4, q_lens=(300, 0, 9), prefix_lens=(64, 10, 0), window_left=0),
    dict(num_qo_heads=24, num_kv_heads=1, q_lens=(90,), prefix_lens=(7,)),
])
def test_executed_flops_matches_brute_force(spec):
    case = make_custom_case(batch=len(spec["q_lens"]), head_dim=64, page_size=16, seed=3, **spec)
    G = case["num_qo_heads"] // case["num_kv_heads"]
    n_hg = -(-G // min(G, 16))
    want = _brute_tiles(case) * case["num_kv_heads"] * n_hg * 4.0 * 32 * 64 * case["head_dim"]
    assert bench.executed_flops(case) == want


@pytest.mark.parametrize("name", ["tiny", "chunked", "swa_sinks"])
def test_executed_at_least_causal(name):
    case = make_case(name)
    causal = 4.0 * case["head_dim"] * case["num_qo_heads"] * bench.causal_pairs(case)
    assert bench.executed_flops(case) >= causal > 0


def _fake_clock_run(monkeypatch, smi_values, dpm_values, seconds=0.3):
    """sampled_clock against scripted readouts: the firmware's per-XCD clock
    (None: not readable) and the driver's DPM level, with launches that do
    nothing and a synchronize that returns at once."""
    import sys
    import types

    smi = iter(smi_values)
    dpm = iter(dpm_values)
    last = {"smi": None, "dpm": None}

    def smi_now():
        try:
            last["smi"] = next(smi)
        except StopIteration:
            pass
        return last["smi"]

    def dpm_now():
        try:
            last["dpm"] = next(dpm)
        except StopIteration:
            pass
        return last["dpm"]

    fake_torch = types.SimpleNamespace(cuda=types.SimpleNamespace(synchronize=lambda *a: None))
    monkeypatch.setitem(sys.modules, "torch", fake_torch)
    monkeypatch.setattr(bench, "_smi_gfxclk_now", smi_now)
    monkeypatch.setattr(bench, "_sysfs_sclk_now", dpm_now)
    return bench.sampled_clock(lambda: None, seconds)


def test_clock_sample_prefers_firmware_clock_and_drops_the_ramp(monkeypatch):
    # the firmware's figure lags: idle readings first, then the loaded clock;
    # the first 40 % of the window and readings below 500 MHz are dropped
    smi = [2100.0] + [95.0] * 10 + [2094.0] * 1000
    r = _fake_clock_run(monkeypatch, smi, [2109] * 1000)
    assert r is not None
    assert r["source"].startswith("amdsmi")
    assert r["median_mhz"] == pytest.approx(2094.0)
    assert r["min_mhz"] >= 500
    assert r["dpm_level_median_mhz"] == pytest.approx(2109.0)


def test_clock_sample_falls_back_to_the_dpm_level(monkeypatch):
    r = _fake_clock_run(monkeypatch, [None] * 1000, [2372] * 1000)
    assert r is not None
    assert r["source"].startswith("sysfs pp_dpm_sclk")
    assert r["median_mhz"] == pytest.approx(2372.0)


def test_clock_sample_without_any_readout(monkeypatch):
    assert _fake_clock_run(monkeypatch, [None] * 1000, [None] * 1000) is None
