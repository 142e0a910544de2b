"""The JSON line bench.py prints, on the smallest workload, in this process:
every field the driver reads, with the relations between them."""
import json
import math
import sys

import pytest

pytestmark = pytest.mark.gpu


def test_bench_line_contract(monkeypatch, capsys):
    import bench
    print("[gpu] bench contract c1", flush=True, file=sys.stderr)
    monkeypatch.setattr(sys, "argv", ["bench.py", "--config", "c1", "--steps", "3", "--warmup", "1", "--no-extra",
                                      "--cpu-planes", "8"])
    bench.main()
    lines = [l for l in capsys.readouterr().out.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert d["metric"] == bench.METRIC and d["unit"] == "voxels/s" and d["n_gpus"] == 1
    assert d["steps"] == 3 and d["warmup"] == 1 and d["higher_is_better"] is True
    assert d["scaling"] in ("weak", "strong") and d["vs_baseline"] is None and d["data"] == "synthetic"
    assert d["dtype"] == "f32" and d["config"]["workload"].startswith("c1")
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert math.isclose(d["value"], 64 ** 3 / (d["ms_per_step"] * 1e-3), rel_tol=1e-6)
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0 and "traffic" in r
    assert math.isclose(r["frac"], r["achieved"] / r["peak"], rel_tol=1e-12)
    assert math.isclose(r["achieved"], r["bytes_per_voxel"] * r["voxels_per_launch"] / (r["ms_per_launch"] * 1e-3)
                        / 1e9, rel_tol=1e-9)
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["unit"] == "voxels/s" and c["sample"]
