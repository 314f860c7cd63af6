#!/usr/bin/env python3
"""Benchmark: one data-parallel rank's ZeRO step on one MI355X.

A step is the whole hot path on one rank's shard: shard layout (host),
flatten of the per-tensor 16-bit gradients into the rank's contiguous shard
fused with the fp64 gradient square-norm and the non-finite flag, the decision
(clip coefficient, loss scale, skip) on one GPU thread (`--decision host`:
on the host after a 16-byte readback), and the fused AdamW update of the fp32
master/m/v shard with the bf16 parameter writeback.  Nothing in a default
step waits on the host.

Default workload: the largest shard that fits one GPU, Llama-13B's tensor list
(40 layers, d=5120, SwiGLU ffn 13824, vocab 32000), N = 4 data-parallel
ranks, rank 0's shard of 3,253,966,080 parameters (52 GB of model state),
synthetic fp16 gradients ~N(0, 1e-3) stored multiplied by a dynamic loss
scale of 65536 and unscaled inside the update, already resident in HBM.
`--workload gpt2-1.5b | llama-7b | 1t-zero3` selects the other shard shapes.

Prints one JSON line.  Per-kernel durations come from HIP events recorded on
the stream the kernels run on; the roofline entry is for the fused AdamW
kernel (28 algorithmic bytes per parameter: read grad 2 + master/m/v 12,
write master/m/v 12 + param 2).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "params updated/sec and HBM GB/s (% of peak) for sharded fused AdamW step, 1 GPU"
HBM_PEAK_GBS = 8000.0
ADAM_BYTES_PER_PARAM = 28
FLATTEN_BYTES_PER_PARAM = 4
NORM_BYTES_PER_PARAM = 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama-13b")
    ap.add_argument("--prepend", type=int, default=0,
                    help="put a tensor of this many elements in front of the workload's list: an odd count "
                         "shifts every later tensor against the shard's 16-byte lines (the flatten's phase-shifted "
                         "path)")
    ap.add_argument("--grad-format", choices=("workload", "bf16", "fp16"), default="workload",
                    help="override the workload's gradient format (fp16 then takes a 65536 loss scale, bf16 none): "
                         "separates the format's cost from the shard's size")
    ap.add_argument("--state", choices=("tiled", "arrays"), default="tiled",
                    help="optimizer-state layout: tiled master/m/v (default) or three separate arrays")
    ap.add_argument("--unfused", action="store_true", help="flatten and square-norm as two passes")
    ap.add_argument("--decision", choices=("device", "host"), default="device",
                    help="decision on the GPU (no host round trip, default) or on the host after a 16-byte readback")
    ap.add_argument("--bucket", type=int, default=0,
                    help="constant bucket capacity in shard elements (0: one pass over the whole shard)")
    ap.add_argument("--produce", action="store_true",
                    help="produce the rank's gradients inside every timed step (the synthetic generator stands in "
                         "for backward): before the step, or bucket by bucket on a producer stream with --bucket")
    ap.add_argument("--source-sets", type=int, default=2,
                    help="identical copies of the source gradients, used in turn by successive steps, so that a "
                         "step's gradients come from HBM rather than from the Infinity Cache left by the last step "
                         "(one-pass paths; the bucketed path uses one)")
    ap.add_argument("--producer", choices=("separate", "same"), default="separate",
                    help="with --produce: generate gradients on their own stream (default) or on the compute stream")
    ap.add_argument("--event-every", type=int, default=1,
                    help="bracket the kernels of every k-th timed step with HIP events (each record costs a few us "
                         "of GPU time: nothing next to a large shard's step, 1%% of the GPT-2 shard's)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--cpu-sample", type=int, default=0, help="elements of the shard the oracle times (0: all)")
    ap.add_argument("--cpu-steps", type=int, default=4, help="steps the oracle times")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="only run plain device copies of this many bytes (for HBM counter scaling)")
    ap.add_argument("--rmw-calibration", action="store_true",
                    help="only time the update's access pattern without its arithmetic (zero_calibrate_tiled_rmw) "
                         "next to the update itself, on the workload's shard size")
    ap.add_argument("--reps", type=int, default=20, help="repetitions per kernel in --rmw-calibration")
    ap.add_argument("--traffic-record", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="only write profiles/traffic_adamw_tiled_kernel_<workload>.json from four rocprofv3 --pmc "
                         "output directories: FETCH_SIZE and WRITE_SIZE of this benchmark's command, and of "
                         "--copy-calibration 1073741824 (the scale of each counter)")
    return ap.parse_args()


def _counter_rows(d: str):
    """(kernel name, counter value) of every dispatch in a rocprofv3 --pmc csv output directory."""
    import csv
    import glob

    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one counter_collection.csv under {d}, found {files}")
    with open(files[0]) as f:
        return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in csv.DictReader(f)]


def traffic_record(args) -> None:
    """Per-call HBM bytes of the tiled update from counter runs, each counter scaled by what it reads for a
    plain 1 GiB device copy (the runtime's copy kernel; the average is over the 1 GiB copies only, not the
    runtime's small uploads through the same kernel).  Tied to the SHA-256 of the kernel source."""
    import hashlib

    import mixed_precision_adam_amd as Z

    w = workload(args)
    lay, _ = Z.zero_shard_layout(w.numels, w.world, w.ranks[0])
    n = lay.shard_numel
    lpc = -(-n // (1 << 25))  # launches per update call
    fetch, write, cfetch, cwrite = (_counter_rows(d) for d in args.traffic_record)
    copy_kib = (1 << 30) / 1024

    def copy_scale(rows):
        vals = [v for k, v in rows if "copyBuffer" in k]
        big = [v for v in vals if v > max(vals) / 2]
        return copy_kib / (sum(big) / len(big))

    fs, ws = copy_scale(cfetch), copy_scale(cwrite)
    f = [v for k, v in fetch if "adamw_tiled_kernel" in k]
    wr = [v for k, v in write if "adamw_tiled_kernel" in k]
    if not f or len(f) % lpc or len(wr) % lpc:
        raise SystemExit(f"{len(f)} / {len(wr)} update dispatches is not a whole number of {lpc}-launch calls")
    fk, wk = sum(f) / (len(f) // lpc), sum(wr) / (len(wr) // lpc)
    src = os.path.join(ROOT, "mixed_precision_adam_amd", "csrc", "zero_shard.hip")
    rec = {"kernel": "adamw_tiled_kernel", "workload": w.name, "shard_numel": n, "launches_per_call": lpc,
           "calls_counted": len(f) // lpc, "fetch_kib_raw_per_call": fk, "write_kib_raw_per_call": wk,
           "fetch_scale": fs, "write_scale": ws, "bytes_per_call": (fk * fs + wk * ws) * 1024,
           "algorithmic_bytes": ADAM_BYTES_PER_PARAM * n,
           "source_sha256": hashlib.sha256(open(src, "rb").read()).hexdigest(),
           "source": "mixed_precision_adam_amd/csrc/zero_shard.hip",
           "summary": f"profiles/hbm_traffic_{w.name}.md"}
    out = os.path.join(ROOT, "profiles", f"traffic_adamw_tiled_kernel_{w.name}.json")
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


def workload(args):
    """The named workload, with its gradient format overridden by --grad-format."""
    import dataclasses

    import synth
    from synth.workloads import WORKLOADS

    w = WORKLOADS[args.workload]
    if args.prepend:
        w = dataclasses.replace(w, numels=[args.prepend] + list(w.numels), name=f"{w.name}+{args.prepend}")
    if args.grad_format == "bf16" and w.grad_kind != synth.BF16:
        w = dataclasses.replace(w, grad_kind=synth.BF16, loss_scale=1.0, inject={})
    elif args.grad_format == "fp16" and w.grad_kind != synth.FP16:
        w = dataclasses.replace(w, grad_kind=synth.FP16, loss_scale=65536.0, inject={})
    return w


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def rmw_calibration(args) -> None:
    """The update's ceiling on one shard: zero_calibrate_tiled_rmw (the tiled update's exact loads and stores,
    the arithmetic replaced by an XOR with 0) and the update itself, alternating on the same buffers of the
    workload's shard size, each timed with HIP events over `reps` back-to-back calls on torch's stream.
    Prints both rates at the update's 28 bytes per element and their ratio."""
    import torch

    import mixed_precision_adam_amd as Z
    import synth

    w = workload(args)
    dev = torch.device("cuda:0")
    lay, _ = Z.zero_shard_layout(w.numels, w.world, w.ranks[0])
    n = lay.shard_numel
    dt16 = torch.bfloat16 if w.grad_kind == synth.BF16 else torch.float16
    gdt = Z.ZERO_BF16 if w.grad_kind == synth.BF16 else Z.ZERO_FP16
    grad = torch.zeros(n, dtype=dt16, device=dev)
    synth.fill_tensor(w.grad_field(1), lay.shard_offset, grad[:lay.shard_valid])
    state = torch.zeros(Z.zero_state_tiled_numel(n), dtype=torch.float32, device=dev)
    master = torch.zeros(n, dtype=torch.float32, device=dev)
    synth.fill_tensor(w.master_field(), lay.shard_offset, master[:lay.shard_valid])
    zeros = torch.zeros(n, dtype=torch.float32, device=dev)
    Z.zero_state_tile(master, zeros, zeros, state, n)
    del master, zeros
    param = torch.zeros(n, dtype=torch.bfloat16, device=dev)
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
              grad_scale=1.0 / w.loss_scale, step=1)

    def calib():
        Z.zero_calibrate_tiled_rmw(grad, state, param, n, 0)

    def update():
        Z.zero_adamw_step_tiled(grad, gdt, state, param, n, **hp)

    def timed(f) -> float:
        f()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.reps):
            f()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e-3 / args.reps

    rounds = []
    for _ in range(3):  # alternate, so slow drift of the box affects both alike
        rounds.append((timed(calib), timed(update)))
    c = sorted(r[0] for r in rounds)[1]
    u = sorted(r[1] for r in rounds)[1]
    launches = -(-n // (1 << 25))
    print(json.dumps({"rmw_calibration": w.name, "grad_format": "bf16" if gdt == Z.ZERO_BF16 else "fp16",
                      "shard_numel": n, "launches_per_call": launches, "reps": args.reps,
                      "rmw_ms": c * 1e3, "rmw_gbs": ADAM_BYTES_PER_PARAM * n / c / 1e9,
                      "update_ms": u * 1e3, "update_gbs": ADAM_BYTES_PER_PARAM * n / u / 1e9,
                      "update_over_rmw": c / u, "rounds_ms": [[a * 1e3, b * 1e3] for a, b in rounds]}))


def copy_calibration(nbytes: int, reps: int = 10) -> None:
    """Plain device-to-device copies of nbytes: the reference for the HBM counters' scale, and two copy rates
    the streaming kernels are compared with (read + write bytes per second, timed with HIP events on torch's
    stream, which every copy here runs on): torch's copy_ (the runtime's copy kernel), and the library's
    flatten over a single contiguous tensor, which is a plain 16-byte-vector copy kernel."""
    import torch

    import mixed_precision_adam_amd as Z

    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    n = nbytes // 2  # 16-bit elements
    _, segs = Z.zero_shard_layout([n], 1, 0)
    table = torch.frombuffer(bytearray(Z.zero_flatten_plan(segs, [a.data_ptr()])), dtype=torch.uint8).to("cuda")

    def timed(copy) -> float:
        copy()  # warm-up
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            copy()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e-3 / reps

    sec = timed(lambda: b.copy_(a))
    b.zero_()  # so that the check below sees what the flatten wrote
    sec_fl = timed(lambda: Z.zero_flatten_grads(table, len(segs), Z.ZERO_BF16, b, n))
    if not torch.equal(a, b):
        raise RuntimeError("flatten copy mismatch")
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps, "ms_per_copy": sec * 1e3,
                      "copy_gbs": 2 * nbytes / sec / 1e9, "ms_per_flatten_copy": sec_fl * 1e3,
                      "flatten_copy_gbs": 2 * nbytes / sec_fl / 1e9}))


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per update call of `kernel` (all of its launches) from the committed counter record, or None
    when there is no record for this kernel and workload or the kernel source has changed since the
    counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(ROOT, "mixed_precision_adam_amd", "csrc", "zero_shard.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if rec.get("source_sha256") != sha:
        return None
    return rec.get("bytes_per_call")


def cpu_baseline(w, sample: int, steps: int) -> dict:
    """The oracle (single-threaded C), untuned, on the first `sample` elements of the rank's shard (default:
    all of it up to 2^28 elements): `steps` whole steps (flatten unless the gradients are generated in the
    shard, square-norm, decision, AdamW), timed with a monotonic clock."""
    import numpy as np

    import oracle
    import synth

    rank = w.ranks[0]
    lay = oracle.layout(w.numels, w.world, rank)
    sample = min(sample if sample > 0 else 1 << 28, lay.shard_valid)
    odt = oracle.BF16 if w.grad_kind == synth.BF16 else oracle.FP16
    lo, hi = lay.shard_offset, lay.shard_offset + sample
    numels, tensors = [], []
    start = 0
    gf = w.grad_field(1)
    for n in w.numels:  # the tensors' parts that fall in the sample, as their own tensor list
        a, b = max(start, lo), min(start + n, hi)
        if b > a:
            numels.append(b - a)
            tensors.append(synth.fill_host(gf, a, b - a))
        start += n
    master = synth.fill_host(w.master_field(), lo, sample)
    m = np.zeros(sample, np.float32)
    v = np.zeros(sample, np.float32)
    q = np.zeros(sample, np.uint16)
    allowed = sorted(os.sched_getaffinity(0))
    os.sched_setaffinity(0, {allowed[0]})  # the single-threaded oracle on one host core, as timed
    try:
        t0 = time.perf_counter()
        for t in range(1, steps + 1):
            shard = tensors[0] if w.flat_shard_only else oracle.flatten(tensors, numels, 1, 0)
            sq, flag = oracle.sqnorm(shard, odt)
            dec = oracle.step_decision([sq], [flag], w.clip, w.loss_scale, 0, 2**31 - 1)
            oracle.adamw_step(shard, odt, master, m, v, q, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                              weight_decay=w.weight_decay, grad_scale=dec["grad_scale"], step=t)
        dt = time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, allowed)
    return {"value": sample * steps / dt, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"{'whole' if sample == lay.shard_valid else f'first {sample} params of the'} rank's shard "
                      f"({sample} params, {len(numels)} tensor pieces), {steps} full steps "
                      f"({'' if w.flat_shard_only else 'flatten + '}fp64 sqnorm + decision + AdamW) on the same "
                      f"gradients, {dt:.2f} s pinned to host core {allowed[0]}"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one rank's step on one GPU; --gpus {args.gpus} is not supported: the library "
              "has no collectives, and how the step shards over GPUs is described, not implemented", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.rmw_calibration:
        rmw_calibration(args)
        return
    if args.traffic_record:
        traffic_record(args)
        return

    import torch

    import mixed_precision_adam_amd as Z
    import synth
    from mixed_precision_adam_amd.driver import (AdamWConfig, BucketPipeline, DeviceDecision, RankShard,
                                                 ScalerState, wait_spin)

    w = workload(args)
    # Gradients generated straight into the shard (the 1T ZeRO-3 shard): no per-tensor sources, no flatten;
    # the step is square-norm -> decision -> update.
    flat = w.flat_shard_only
    if flat:
        assert not (args.bucket or args.produce or args.unfused) and args.decision == "device", \
            "a shard-only workload runs the one-pass device path"
    dev = torch.device("cuda:0")
    rank = w.ranks[0]
    torch.cuda.set_device(dev)

    # --- inputs resident in HBM: the rank's landing tensors, master init, zero m/v
    lay, segs = Z.zero_shard_layout(w.numels, w.world, rank)
    starts = [0]
    for n in w.numels:
        starts.append(starts[-1] + n)
    landing = sorted({s.tensor for s in segs})
    dt16 = torch.bfloat16 if w.grad_kind == synth.BF16 else torch.float16
    sources = [None] * len(w.numels)
    gf = w.grad_field(1)
    if flat:
        landing = []
    for t in landing:
        sources[t] = torch.empty(w.numels[t], dtype=dt16, device=dev)
        synth.fill_tensor(gf, starts[t], sources[t])
    gdt = Z.ZERO_BF16 if w.grad_kind == synth.BF16 else Z.ZERO_FP16
    sh = RankShard(w.numels, w.world, rank, gdt, dev, sources=None if flat else sources,
                   tiled=args.state == "tiled", fused=not (args.unfused or flat))
    if flat:
        sh.grad[lay.shard_valid:].zero_()
        synth.fill_tensor(gf, lay.shard_offset, sh.grad[:lay.shard_valid])
    # Further copies of the sources (same values) with their own flatten tables, used in turn.
    n_sets = 1 if (flat or args.bucket) else max(1, args.source_sets)
    source_sets, tables = [sources], [sh.seg_table]
    for _ in range(1, n_sets):
        copy = [x.clone() if x is not None else None for x in sources]
        blob = Z.zero_flatten_plan(sh.segments, [x if x is not None else 0 for x in copy])
        source_sets.append(copy)
        tables.append(torch.frombuffer(bytearray(blob), dtype=torch.uint8).to(dev))
    master0 = torch.zeros(lay.shard_numel, dtype=torch.float32, device=dev)
    synth.fill_tensor(w.master_field(), lay.shard_offset, master0[:lay.shard_valid])
    sh.load_master(master0)
    del master0
    cfg = AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                      max_norm=w.clip)
    growth = 2**31 - 1 if w.grad_kind == synth.BF16 else 1000
    scaler = ScalerState(scale=w.loss_scale, growth_interval=growth)
    ddec = DeviceDecision([sh], cfg, loss_scale=w.loss_scale, growth_interval=growth) if args.decision == "device" \
        else None
    prod_stream = None
    if args.produce:
        assert args.decision == "device", "--produce needs the device decision"
        prod_stream = torch.cuda.Stream() if args.producer == "separate" else torch.cuda.current_stream()
    landing_set = set(landing)

    current = [0]  # the source set the step in flight uses
    piece_tables = {}  # (source set, tensors) -> device piece table, built once (in the warm-up steps)

    def produce(idx, st):
        """Writes the gradients of source tensors `idx` (those that land in the shard) on stream `st`: one
        generator launch for all of them."""
        key = (current[0], tuple(t for t in idx if t in landing_set))
        if not key[1]:
            return
        if key not in piece_tables:
            srcs = source_sets[current[0]]
            pieces = [(srcs[t].data_ptr(), starts[t], w.numels[t]) for t in key[1]]
            blob = synth.piece_table(pieces)
            piece_tables[key] = (torch.frombuffer(bytearray(blob), dtype=torch.uint8).to(dev), len(pieces),
                                 max(w.numels[t] for t in key[1]))
            torch.cuda.synchronize()  # the table is in place before any stream reads it
        table, n_pieces, max_n = piece_tables[key]
        synth.fill_device_many(gf, table.data_ptr(), n_pieces, max_n, st.cuda_stream)

    pipe = None
    if args.bucket:
        assert ddec is not None and sh.fused, "the bucketed step uses the fused flatten and the device decision"
        pipe = BucketPipeline(sh, sources, args.bucket, cfg, loss_scale=w.loss_scale, growth_interval=growth)
        ddec = None
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    ev = {k: [] for k in ("flatten", "sqnorm", "adamw")}
    numels_c = (ctypes.c_int64 * len(w.numels))(*w.numels)
    lay_out = Z.zero_layout()
    nseg = ctypes.c_int32(0)
    seg_buf = (Z.zero_segment * len(segs))()
    lib = Z.library()
    # events for the timed steps are created up front, outside the timed region; they bracket the flatten
    # and the update of every k-th step (a record costs a few microseconds of GPU time)
    pool = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]

    count = [0]

    def step(e=None):
        if w.lr_min is not None:  # the workload's cosine schedule, cycled over its step count
            count[0] += 1
            cfg.lr = Z.zero_cosine_lr((count[0] - 1) % w.steps + 1, w.steps, w.lr, w.lr_min)
        # a1: layout (host) -- recomputed every step as part of the path
        rc = lib.zero_shard_layout(ctypes.cast(numels_c, ctypes.c_void_p), len(w.numels), w.world, rank,
                                   ctypes.byref(lay_out), ctypes.cast(seg_buf, ctypes.c_void_p), len(segs),
                                   ctypes.byref(nseg))
        assert rc == 0 and nseg.value == len(segs)
        current[0] = (current[0] + 1) % n_sets
        sh.seg_table = tables[current[0]]
        if pipe is not None:                           # fixed-capacity buckets, last bucket first
            if args.produce:                           # backward stand-in on the producer stream
                pipe.launch_production(produce, prod_stream, stream)
            if e:
                e[0].record(stream)
            pipe.reduce_all(stream, wait=args.produce)  # a2 + a3, bucket by bucket
            if e:
                e[1].record(stream)
            pipe.decide(stream)                        # a4 over the bucket partials
            if e:
                e[4].record(stream)
            sh.adamw_dev(pipe.state, stream)           # a5
            if e:
                e[5].record(stream)
                ev["flatten"].append((e[0], e[1]))
                ev["adamw"].append((e[4], e[5]))
            return None
        if ddec is not None:                           # everything on the GPU, nothing waits on the host
            if args.produce:                           # backward stand-in, all before the step
                produce(landing, stream)
            if e:
                e[0].record(stream)
            if not flat:
                sh.flatten(stream)                     # a2 + a3 (fused)
            if flat or not sh.fused:
                sh.sqnorm(stream)                      # a3
            if e:
                e[1].record(stream)
            Z.zero_step_decision_dev(ddec.sq_base, ddec.flag_base, 1, cfg.max_norm, ddec.state, lr=cfg.lr,
                                     beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.eps,
                                     weight_decay=cfg.weight_decay, stream=stream)   # a4
            if e:
                e[4].record(stream)
            sh.adamw_dev(ddec.state, stream)           # a5
            if e:
                e[5].record(stream)
                ev["flatten"].append((e[0], e[1]))
                ev["adamw"].append((e[4], e[5]))
            return None
        if e:
            e[0].record(stream)
        sh.flatten(stream)                             # a2 (+ a3 when fused)
        if e:
            e[1].record(stream)
            e[2].record(stream)
        if not sh.fused:
            sh.sqnorm(stream)                          # a3
        if e:
            e[3].record(stream)
        sh.readback(stream)                            # 16 bytes to the host
        wait_spin(stream)
        sq, fl = sh.norm_result()                      # a4: host decision
        dec = Z.zero_step_decision([sq], [fl], cfg.max_norm, scaler.scale, scaler.good_steps,
                                   scaler.growth_interval)
        scaler.scale, scaler.good_steps = dec["loss_scale"], dec["good_steps"]
        if not dec["skip"]:
            scaler.adam_step += 1
            if e:
                e[4].record(stream)
            sh.adamw(cfg, dec["grad_scale"], scaler.adam_step, stream)   # a5
            if e:
                e[5].record(stream)
        if e:
            ev["flatten"].append((e[0], e[1]))
            ev["sqnorm"].append((e[2], e[3]))
            if not dec["skip"]:
                ev["adamw"].append((e[4], e[5]))
        return dec

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps, synchronized on both sides (one process: no barrier needed)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        sample = k % args.event_every == args.event_every - 1 or (args.steps < args.event_every and k == args.steps - 1)
        dec = step(pool[k] if sample else None)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    if ddec is not None or pipe is not None:
        st = (ddec or pipe).read()
        dec = {"global_norm": st["global_norm"], "grad_scale": st["grad_scale"], "skip": st["skip"]}

    def avg_ms(pairs):
        return sum(a.elapsed_time(b) for a, b in pairs) / max(len(pairs), 1)

    S = lay.shard_numel
    ms = {k: avg_ms(v) for k, v in ev.items()}
    adam_gbs = ADAM_BYTES_PER_PARAM * S / (ms["adamw"] * 1e-3) / 1e9
    ms_per_step = elapsed / args.steps * 1e3
    params_per_s = S * args.steps / elapsed
    if flat:
        step_bpp = ADAM_BYTES_PER_PARAM + NORM_BYTES_PER_PARAM
    else:
        step_bpp = ADAM_BYTES_PER_PARAM + FLATTEN_BYTES_PER_PARAM + (0 if sh.fused else NORM_BYTES_PER_PARAM)
    result = {
        "metric": METRIC,
        "value": params_per_s,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: rank {rank} of N={w.world}, shard {S} params "
                        f"(psi={lay.psi}, {len(segs)} tensor pieces), {'bf16' if gdt == 0 else 'fp16'} grads"
                        + (", gradients generated inside each step" if args.produce else "")
                        + (", gradients generated in the shard (no flatten)" if flat else "")
                        + (", cosine lr" if w.lr_min is not None else "")
                        + (f", flattened in buckets of {args.bucket}" if args.bucket else ""),
            "psi": lay.psi, "world": w.world, "rank": rank, "shard_numel": S, "segments": len(segs),
        },
        "roofline": {
            "kernel": "adamw_tiled_kernel" if sh.tiled else "adamw_vec_kernel",
            "bound": "hbm",
            "achieved": adam_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": adam_gbs / HBM_PEAK_GBS,
            "traffic": measured_traffic("adamw_tiled_kernel" if sh.tiled else "adamw_vec_kernel", w.name)
            if args.grad_format == "workload" else None,
            "bytes_per_param": ADAM_BYTES_PER_PARAM,
            "per": "update call: the shard in launches of at most 2^25 elements, timed together",
        },
        "breakdown": {
            "adamw_ms": ms["adamw"],
            "adamw_params_per_s": S / (ms["adamw"] * 1e-3),
            "state_layout": args.state,
            "decision": args.decision,
            "bucket_numel": args.bucket or None,
            "gradients_produced_in_step": args.produce,
            "source_sets": n_sets,
            "producer_stream": args.producer if args.produce else None,
            "buckets": len(pipe.windows) if pipe is not None else None,
            "flatten_norm_fused": sh.fused,
            "flatten_ms": None if flat else ms["flatten"],
            "flatten_gbs": None if flat else FLATTEN_BYTES_PER_PARAM * S / (ms["flatten"] * 1e-3) / 1e9,
            "sqnorm_ms": ms["flatten"] if flat else (ms["sqnorm"] if ev["sqnorm"] else None),
            "sqnorm_gbs": NORM_BYTES_PER_PARAM * S / (ms["flatten" if flat else "sqnorm"] * 1e-3) / 1e9
            if flat or (ev["sqnorm"] and not sh.fused) else None,
            "step_bytes_per_param": step_bpp,
            "step_gbs_algorithmic": step_bpp * params_per_s / 1e9,
            "last_global_norm": dec["global_norm"],
            "last_grad_scale": dec["grad_scale"],
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_sample, args.cpu_steps)
        result["cpu_baseline"]["host_cores_available"] = os.cpu_count()
        result["cpu_baseline"]["cpu_model"] = cpu_model()
    print(json.dumps(result))


if __name__ == "__main__":
    main()
