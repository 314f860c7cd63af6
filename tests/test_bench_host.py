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


def _args(**kw):
    import argparse

    base = dict(workload="llama-13b", grad_format="workload", prepend=0)
    base.update(kw)
    return argparse.Namespace(**base)


def test_workload_overrides():
    """--grad-format swaps the gradient format (fp16 brings a 65536 loss scale, bf16 none, and neither keeps
    the injected infinities); --prepend puts an extra tensor in front and renames the workload, so no
    counter record of the original list applies to it."""
    sys.path.insert(0, ROOT)
    import synth

    bench = _bench()
    w = bench.workload(_args())
    assert w.name == "llama-13b" and w.grad_kind == synth.FP16 and w.loss_scale == 65536.0 and w.inject
    w = bench.workload(_args(grad_format="bf16"))
    assert w.grad_kind == synth.BF16 and w.loss_scale == 1.0 and not w.inject and w.name == "llama-13b"
    w = bench.workload(_args(workload="gpt2-1.5b", grad_format="fp16"))
    assert w.grad_kind == synth.FP16 and w.loss_scale == 65536.0
    w0 = bench.workload(_args(workload="gpt2-1.5b"))
    w = bench.workload(_args(workload="gpt2-1.5b", prepend=3))
    assert w.name == "gpt2-1.5b+3" and w.numels == [3] + list(w0.numels)
    assert bench.measured_traffic("adamw_tiled_kernel", w.name) is None


def _counter_csv(path, rows, counter):
    path.mkdir(parents=True)
    lines = ['"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"']
    for i, (name, value) in enumerate(rows):
        lines.append(f'{i},"{name}","{counter}",{value}')
    (path / "run_counter_collection.csv").write_text("\n".join(lines) + "\n")


def test_traffic_record_from_counter_runs(tmp_path, monkeypatch):
    """--traffic-record: per-call sums over the update's launches, each counter scaled by what it read for
    the 1 GiB copies (small uploads through the same copy kernel are left out), written with the source's
    SHA-256; a dispatch count that is not a whole number of calls is refused."""
    bench = _bench()
    s = 194_701_400  # GPT-2 rank shard: 6 launches per call
    upd = "void (anonymous namespace)::adamw_tiled_kernel<0, 0>(unsigned short const*)"
    copy = "__amd_rocclr_copyBuffer"
    _counter_csv(tmp_path / "f", [(upd, 100.0)] * 12 + [("other", 5.0)], "FETCH_SIZE")
    _counter_csv(tmp_path / "w", [(upd, 300.0)] * 12, "WRITE_SIZE")
    _counter_csv(tmp_path / "cf", [(copy, 1.0), (copy, 524288.0), (copy, 524288.0)], "FETCH_SIZE")
    _counter_csv(tmp_path / "cw", [(copy, 2.0), (copy, 1048576.0)], "WRITE_SIZE")
    (tmp_path / "profiles").mkdir()
    src_dir = tmp_path / "mixed_precision_adam_amd" / "csrc"
    src_dir.mkdir(parents=True)
    text = open(os.path.join(ROOT, "mixed_precision_adam_amd", "csrc", "zero_shard.hip"), "rb").read()
    (src_dir / "zero_shard.hip").write_bytes(text)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    args = _args(workload="gpt2-1.5b", traffic_record=[str(tmp_path / d) for d in ("f", "w", "cf", "cw")])
    bench.traffic_record(args)
    rec = json.load(open(tmp_path / "profiles" / "traffic_adamw_tiled_kernel_gpt2-1.5b.json"))
    assert rec["shard_numel"] == s and rec["launches_per_call"] == 6 and rec["calls_counted"] == 2
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["fetch_kib_raw_per_call"] == 600.0 and rec["write_kib_raw_per_call"] == 1800.0
    assert rec["bytes_per_call"] == (600.0 * 2.0 + 1800.0) * 1024 and rec["algorithmic_bytes"] == 28 * s
    assert bench.measured_traffic("adamw_tiled_kernel", "gpt2-1.5b") == rec["bytes_per_call"]
    _counter_csv(tmp_path / "f7", [(upd, 100.0)] * 7, "FETCH_SIZE")
    args.traffic_record[0] = str(tmp_path / "f7")
    with pytest.raises(SystemExit):
        bench.traffic_record(args)
