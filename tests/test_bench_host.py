"""Host-side parts of bench.py (CPU only): the one-GPU guard, the committed HBM-traffic record and its
source check, and the oracle baseline leg on a small shard."""
import importlib.util
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


@pytest.mark.parametrize("name", ["llama-13b", "gpt2-1.5b"])
def test_traffic_record_is_consistent(name):
    """The committed counter records: per-call bytes of the update on a rank shard (the benchmark's default,
    Llama-13B, and GPT-2), scaled by the copy calibration, next to the 28 B/param algorithmic count."""
    sys.path.insert(0, ROOT)
    from synth.workloads import WORKLOADS

    rec = json.load(open(os.path.join(ROOT, "profiles", f"traffic_adamw_tiled_kernel_{name}.json")))
    w = WORKLOADS[name]
    assert rec["workload"] == name and rec["kernel"] == "adamw_tiled_kernel"
    s = -(-sum(w.numels) // w.world)
    assert rec["shard_numel"] == s and rec["algorithmic_bytes"] == 28 * s
    assert rec["launches_per_call"] == -(-s // 2**25)
    scaled = (rec["fetch_kib_raw_per_call"] * rec["fetch_scale"] + rec["write_kib_raw_per_call"] * rec["write_scale"])
    assert scaled * 1024 == pytest.approx(rec["bytes_per_call"], rel=1e-12)
    assert 1.0 <= rec["bytes_per_call"] / rec["algorithmic_bytes"] < 1.01
    assert os.path.exists(os.path.join(ROOT, rec["summary"]))


def test_traffic_is_null_once_the_source_changes(tmp_path):
    bench = _bench()
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic_adamw_tiled_kernel_gpt2-1.5b.json")))
    got = bench.measured_traffic("adamw_tiled_kernel", "gpt2-1.5b")
    assert got is None or got == rec["bytes_per_call"]
    assert bench.measured_traffic("adamw_tiled_kernel", "no-such-workload") is None
    # the same record beside a source that differs by one byte
    (tmp_path / "profiles").mkdir()
    shutil.copy(os.path.join(ROOT, "profiles", "traffic_adamw_tiled_kernel_gpt2-1.5b.json"), tmp_path / "profiles")
    src_dir = tmp_path / "mixed_precision_adam_amd" / "csrc"
    src_dir.mkdir(parents=True)
    text = open(os.path.join(ROOT, "mixed_precision_adam_amd", "csrc", "zero_shard.hip"), "rb").read()
    (src_dir / "zero_shard.hip").write_bytes(text + b"\n")
    bench.ROOT = str(tmp_path)
    assert bench.measured_traffic("adamw_tiled_kernel", "gpt2-1.5b") is None
    (src_dir / "zero_shard.hip").write_bytes(text)
    assert bench.measured_traffic("adamw_tiled_kernel", "gpt2-1.5b") == got


def test_cpu_baseline_leg_on_a_small_shard():
    sys.path.insert(0, ROOT)
    from synth.workloads import WORKLOADS

    bench = _bench()
    out = bench.cpu_baseline(WORKLOADS["tiny"], 0, 1)
    assert out["kind"] == "oracle" and out["cores"] == 1 and out["unit"] == "params/s"
    assert out["value"] > 0 and "whole rank's shard (250001 params" in out["sample"]
