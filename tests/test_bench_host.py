"""Host-side pieces of bench.py that need no GPU: the CPU baselines of the
float64 oracle and the JSON encoding of the line."""

import json
import math

import bench


def test_json_float_keeps_the_line_strict_json():
    assert bench._json_float(1.5e-6) == 1.5e-6
    for v in (math.inf, -math.inf, math.nan):
        enc = json.dumps({"r": bench._json_float(v)}, allow_nan=False)
        assert json.loads(enc)["r"] in ("inf", "-inf", "nan")


def test_cpu_baseline_repeats_the_sample(monkeypatch):
    monkeypatch.setattr(bench, "CPU_SECONDS", 0.05)
    r = bench.cpu_baseline(1, 3)
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["value"] > 0
    assert r["seconds"] >= 0.05 and "runs" in r["sample"]


def test_cpu_detail_single_core_and_batch_split():
    d = bench.cpu_detail(2, 2)
    assert d["cores_available"] >= 1
    for leg in ("single_core", "batch_split"):
        for what in ("sequential", "solve"):
            assert d[leg][what]["seconds"] > 0 and d[leg][what]["state_updates_per_s"] > 0
    assert 1 <= d["batch_split"]["workers"] <= 16
