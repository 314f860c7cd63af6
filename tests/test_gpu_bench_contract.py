"""bench.py's output contract on the GPU: one JSON line with the keys, types and objects the benchmark
promises (run on the small four-rank configuration, rank 0, so it takes seconds)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_contract_line():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "3",
                          "--warmup", "1"], capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [line for line in res.stdout.splitlines() if line.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "params/s" and d["higher_is_better"] is True and d["scaling"] == "weak"
    assert d["vs_baseline"] is None and d["data"] == "synthetic" and d["dtype"] == "f32"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["value"] == pytest.approx(d["config"]["shard_numel"] / (d["ms_per_step"] * 1e-3), rel=1e-9)
    assert d["config"]["workload"].startswith("tiny") and "model" not in d["config"]
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] > 0 and r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-12)
    assert "traffic" in r  # bytes per update call for the workload the counters were taken on, else null
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] == 1 and c["value"] > 0 and c["unit"] == "params/s" and c["sample"]
