"""The bench line's contract, on a one-layer slice of the 7B workload, run in
this process: one JSON line with the required fields, consistent with each
other (value = blocks / step time, roofline fraction = achieved / peak)."""
import json
import sys

import pytest

from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def test_bench_line_fields(capsys, monkeypatch):
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py", "--layers", "1", "--steps", "2", "--warmup", "1",
                                      "--no-cpu-baseline", "--no-train-step"])
    bench.main()
    lines = [l for l in capsys.readouterr().out.strip().splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["vs_baseline"] is None
    assert d["config"]["workload"] == "llama7b_all_linear" and d["config"]["tensors"] == 7
    blocks = d["config"]["blocks"]
    assert abs(d["value"] - blocks / (d["ms_per_step"] * 1e-3)) <= 1e-3 * d["value"]
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert 0.0 < r["frac"] < 1.0 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert r["traffic"] is None or r["traffic"] > 0
    assert 0.0 < d["step_hbm_frac"] < 1.0
