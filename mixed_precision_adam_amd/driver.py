"""Host-side sequencing of one rank's ZeRO step over the C ABI.

Holds the device buffers of a simulated data-parallel rank (PyTorch
allocations) and calls the library entry points in the order of the step:
flatten -> square-norm -> (simulated all-reduce + decision) -> AdamW.  Three
ways of sequencing it: ``rank_step`` (decision on the host after a 16-byte
readback), ``DeviceDecision`` (decision on the GPU, nothing waits on the
host) and ``BucketPipeline`` (flatten + norm partials in constant-capacity
buckets as gradients arrive on a producer stream).  No arithmetic of the
method happens here: every step is a library call.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import (ZERO_BF16, ZERO_FP16, ZERO_STATE_TILE, read_step_state, zero_adamw_step, zero_adamw_step_dev,
               zero_adamw_step_tiled, zero_adamw_step_tiled_dev, zero_bucket_segments, zero_flatten_grads,
               zero_flatten_grads_partials, zero_flatten_grads_sqnorm, zero_flatten_partials_count,
               zero_flatten_plan, zero_grad_sqnorm, zero_grad_sqnorm_workspace_bytes, zero_shard_layout,
               zero_sqnorm_reduce, zero_state_tile, zero_state_tiled_numel, zero_state_untile, zero_step_decision,
               zero_step_decision_dev, zero_step_state_init)

_TORCH16 = {ZERO_BF16: torch.bfloat16, ZERO_FP16: torch.float16}


@dataclass
class AdamWConfig:
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    max_norm: float = 1.0


@dataclass
class ScalerState:
    """Dynamic loss scale (1.0 and no growth for bf16 training)."""
    scale: float = 1.0
    good_steps: int = 0
    growth_interval: int = 2**31 - 1
    adam_step: int = 0  # Adam t of the last applied update


class RankShard:
    """One simulated rank: the flat 16-bit grad shard, the fp32 master/m/v state (three arrays, or one
    tiled array when ``tiled``), the 16-bit param shard (bf16, or fp16 with ``param_dtype=ZERO_FP16``) and
    the norm scratch."""

    def __init__(self, numels, world: int, rank: int, grad_dtype: int, device="cuda", sources=None,
                 tiled: bool = False, fused: bool = False, param_dtype: int = ZERO_BF16):
        self.layout, self.segments = zero_shard_layout(numels, world, rank)
        self.grad_dtype = grad_dtype
        self.device = torch.device(device)
        self.tiled = tiled
        self.fused = fused  # flatten and square-norm in one pass
        n = self.layout.shard_numel
        self.n = n
        self.grad = torch.empty(n, dtype=_TORCH16[grad_dtype], device=self.device)
        if tiled:
            self.state = torch.zeros(zero_state_tiled_numel(n), dtype=torch.float32, device=self.device)
        else:
            self.master = torch.zeros(n, dtype=torch.float32, device=self.device)
            self.m = torch.zeros(n, dtype=torch.float32, device=self.device)
            self.v = torch.zeros(n, dtype=torch.float32, device=self.device)
        self.param_dtype = param_dtype
        self.param = torch.zeros(n, dtype=_TORCH16[param_dtype], device=self.device)
        self.ws_bytes = zero_grad_sqnorm_workspace_bytes(n)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        # square-norm (double) and non-finite flag (int32) side by side: one 16-byte readback per step
        self.norm_dev = torch.zeros(2, dtype=torch.float64, device=self.device)
        self.sq_dev = self.norm_dev.data_ptr()
        self.flag_dev = self.norm_dev.data_ptr() + 8
        self.norm_host = torch.zeros(2, dtype=torch.float64).pin_memory()
        self._norm_np = self.norm_host.numpy()
        self.seg_table = None
        self.n_segs = 0
        if sources is not None:
            self.set_sources(sources)

    # -- state access (initialisation and checks) -------------------------------------------------

    def load_master(self, master: torch.Tensor) -> None:
        """Sets the fp32 master shard (device tensor of n floats); m and v start at zero."""
        if self.tiled:
            zeros = torch.zeros(self.n, dtype=torch.float32, device=self.device)
            zero_state_tile(master, zeros, zeros, self.state, self.n)
        else:
            self.master.copy_(master)
            self.m.zero_()
            self.v.zero_()

    def state_views(self, lo: int = 0, hi: int | None = None):
        """(master, m, v) device tensors for shard elements [lo, hi).  With the tiled layout lo and hi must
        be tile-aligned (hi may be n)."""
        hi = self.n if hi is None else hi
        if not self.tiled:
            return self.master[lo:hi], self.m[lo:hi], self.v[lo:hi]
        t = ZERO_STATE_TILE
        assert lo % t == 0 and (hi % t == 0 or hi == self.n)
        tiles = self.state.view(-1, 3, t)[lo // t: (hi + t - 1) // t]
        cnt = hi - lo
        return tuple(tiles[:, k, :].reshape(-1)[:cnt] for k in range(3))

    def read_state(self):
        """Whole (master, m, v) as separate device tensors (untiling when needed)."""
        if not self.tiled:
            return self.master, self.m, self.v
        out = [torch.empty(self.n, dtype=torch.float32, device=self.device) for _ in range(3)]
        zero_state_untile(self.state, *out, self.n)
        return tuple(out)

    # -- the step ------------------------------------------------------------------------------

    def set_sources(self, sources) -> None:
        """sources[t]: device tensor (or address) of tensor t's gradient; only tensors that land in the
        shard need one."""
        ptrs = [sources[t] if sources[t] is not None else 0 for t in range(len(sources))]
        table = zero_flatten_plan(self.segments, ptrs)
        self.n_segs = len(self.segments)
        host = torch.frombuffer(bytearray(table), dtype=torch.uint8) if table else torch.zeros(32, dtype=torch.uint8)
        self.seg_table = host.to(self.device)
        self._sources = sources  # keep the tensors alive

    def flatten(self, stream=None) -> None:
        if self.fused:
            zero_flatten_grads_sqnorm(self.seg_table, self.n_segs, self.grad_dtype, self.grad, self.n, self.ws,
                                      self.ws_bytes, self.sq_dev, self.flag_dev, stream)
        else:
            zero_flatten_grads(self.seg_table, self.n_segs, self.grad_dtype, self.grad, self.n, stream)

    def sqnorm(self, stream=None) -> None:
        """Square-norm and non-finite flag of the shard as it stands (a separate pass)."""
        zero_grad_sqnorm(self.grad, self.grad_dtype, self.n, self.ws, self.ws_bytes, self.sq_dev, self.flag_dev,
                         stream)

    def readback(self, stream=None) -> None:
        """Queue the 16-byte copy of the square-norm and flag to pinned host memory on `stream` (the stream
        the norm ran on, so the copy is ordered after it and a wait on that stream covers both)."""
        stream = stream or torch.cuda.current_stream()
        with torch.cuda.stream(stream):
            self.norm_host.copy_(self.norm_dev, non_blocking=True)

    def norm_result(self):
        """Host copies of the last sqnorm; call after the stream has been synchronized."""
        return float(self._norm_np[0]), int(self._norm_np[1:2].view(np.int32)[0])

    def adamw_dev(self, step_state, stream=None) -> None:
        """The update with its scalars taken from a device-resident zero_step_state."""
        if self.tiled:
            zero_adamw_step_tiled_dev(self.grad, self.grad_dtype, self.state, self.param, self.n, step_state, stream,
                                      param_dtype=self.param_dtype)
        else:
            zero_adamw_step_dev(self.grad, self.grad_dtype, self.master, self.m, self.v, self.param, self.n,
                                step_state, stream, param_dtype=self.param_dtype)

    def adamw(self, cfg: AdamWConfig, grad_scale: float, step: int, stream=None) -> None:
        kw = dict(lr=cfg.lr, beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.eps, weight_decay=cfg.weight_decay,
                  grad_scale=grad_scale, step=step, stream=stream, param_dtype=self.param_dtype)
        if self.tiled:
            zero_adamw_step_tiled(self.grad, self.grad_dtype, self.state, self.param, self.n, **kw)
        else:
            zero_adamw_step(self.grad, self.grad_dtype, self.master, self.m, self.v, self.param, self.n, **kw)


class DeviceDecision:
    """Device-resident decision for a set of simulated ranks: their square-norms and flags land side by side
    in one device buffer, one GPU thread takes the decision, and the update kernels read it from device
    memory.  A step then needs no host round trip (and can be captured in a HIP graph)."""

    def __init__(self, shards, cfg: AdamWConfig, loss_scale: float = 1.0, growth_interval: int = 2**31 - 1):
        n = len(shards)
        dev = shards[0].device
        self.shards = shards
        self.cfg = cfg
        self.norms = torch.zeros(n + (n + 1) // 2, dtype=torch.float64, device=dev)  # n doubles, then n int32
        self.sq_base = self.norms.data_ptr()
        self.flag_base = self.sq_base + 8 * n
        for r, sh in enumerate(shards):
            sh.sq_dev = self.sq_base + 8 * r
            sh.flag_dev = self.flag_base + 4 * r
        self.state = torch.zeros(16, dtype=torch.float64, device=dev)  # 128 bytes >= sizeof(zero_step_state)
        zero_step_state_init(self.state, loss_scale, growth_interval)

    def step(self, flatten: bool = True, stream=None) -> None:
        """Enqueues one whole step; nothing waits on the host."""
        stream = stream or torch.cuda.current_stream()
        for sh in self.shards:
            if flatten:
                sh.flatten(stream)
            if not (flatten and sh.fused):
                sh.sqnorm(stream)
        c = self.cfg
        zero_step_decision_dev(self.sq_base, self.flag_base, len(self.shards), c.max_norm, self.state, lr=c.lr,
                               beta1=c.beta1, beta2=c.beta2, eps=c.eps, weight_decay=c.weight_decay, stream=stream)
        for sh in self.shards:
            sh.adamw_dev(self.state, stream)

    def read(self) -> dict:
        """The decided state (synchronizes)."""
        return read_step_state(self.state)


class BucketPipeline:
    """Constant-capacity buckets for one rank's shard: as backward produces gradients (last tensors first),
    each bucket of at most `bucket_numel` shard elements is flattened on the compute stream as soon as its
    source tensors are ready, overlapping with the production of the next bucket, and leaves its partial
    square-sums and flags in its own slice of one partials buffer.  One reduction folds them all (window
    order), the device decision follows, and the update runs over the whole shard (clipping needs the global
    norm first).  The bucket capacity is fixed: it does not grow with the model."""

    def __init__(self, shard: "RankShard", sources, bucket_numel: int, cfg: AdamWConfig, loss_scale: float = 1.0,
                 growth_interval: int = 2**31 - 1):
        assert bucket_numel > 0 and bucket_numel % 8 == 0, "whole 16-byte vectors per bucket"
        self.sh = shard
        self.cfg = cfg
        self.sources = sources
        n = shard.n
        self.windows = [(a, min(n, a + bucket_numel)) for a in range(0, n, bucket_numel)] or [(0, 0)]
        dev = shard.device
        counts = [zero_flatten_partials_count(b - a) for a, b in self.windows]
        self.part_first = np.cumsum([0] + counts).tolist()  # window k owns partials [first[k], first[k+1])
        total = max(self.part_first[-1], 1)
        self.part_sum = torch.zeros(total, dtype=torch.float64, device=dev)
        self.part_flag = torch.zeros(total, dtype=torch.int32, device=dev)
        self.norms = torch.zeros(2, dtype=torch.float64, device=dev)  # the rank's square-norm, then its flag
        self.tables, self.counts, self.tensors = [], [], []
        for a, b in self.windows:
            segs = zero_bucket_segments(shard.segments, a, b - a)
            ptrs = [sources[t] if sources[t] is not None else 0 for t in range(len(sources))]
            blob = zero_flatten_plan(segs, ptrs)
            table = torch.frombuffer(bytearray(blob), dtype=torch.uint8) if blob else torch.zeros(32, dtype=torch.uint8)
            self.tables.append(table.to(dev))
            self.counts.append(len(segs))
            self.tensors.append(sorted({sg.tensor for sg in segs}))
        self.state = torch.zeros(16, dtype=torch.float64, device=dev)
        zero_step_state_init(self.state, loss_scale, growth_interval)
        self.events = [torch.cuda.Event() for _ in self.windows]

    def step(self, produce=None, producer=None, stream=None) -> None:
        """One step.  `produce(tensor_indices, stream)` writes those source tensors' gradients (stands in for
        backward); it runs on `producer` in backward order, one bucket at a time, each followed by an event
        the compute stream waits for.  Without `produce` the sources are taken as ready."""
        stream = stream or torch.cuda.current_stream()
        if produce is not None:
            self.launch_production(produce, producer, stream)
        self.reduce_all(stream, wait=produce is not None)
        self.decide(stream)
        self.sh.adamw_dev(self.state, stream)

    def launch_production(self, produce, producer, stream) -> None:
        """Queues gradient production on `producer`, last bucket first, with one event per bucket."""
        producer.wait_stream(stream)  # the previous step has finished reading the sources
        done = set()
        for k in range(len(self.windows) - 1, -1, -1):
            need = [t for t in self.tensors[k] if t not in done]
            produce(need, producer)
            done.update(need)
            self.events[k].record(producer)

    def reduce_all(self, stream=None, wait: bool = False) -> None:
        """Flatten + norm partials of every bucket, last first; with `wait` each waits for its event."""
        for k in range(len(self.windows) - 1, -1, -1):
            if wait:
                stream.wait_event(self.events[k])
            self.reduce_bucket(k, stream)

    def reduce_bucket(self, k: int, stream=None) -> None:
        """Flatten of bucket k, leaving its partial square-sums and flags in its slice of the partials."""
        sh = self.sh
        a, b = self.windows[k]
        f = self.part_first[k]
        zero_flatten_grads_partials(self.tables[k], self.counts[k], sh.grad_dtype, sh.grad.data_ptr() +
                                    a * sh.grad.element_size(), b - a, self.part_sum.data_ptr() + 8 * f,
                                    self.part_flag.data_ptr() + 4 * f, stream)

    def decide(self, stream=None) -> None:
        """Folds every bucket's partials (window order), then the device decision."""
        c = self.cfg
        sq, fl = self.norms.data_ptr(), self.norms.data_ptr() + 8
        zero_sqnorm_reduce(self.part_sum, self.part_flag, self.part_first[-1], sq, fl, stream)
        zero_step_decision_dev(sq, fl, 1, c.max_norm, self.state, lr=c.lr, beta1=c.beta1, beta2=c.beta2, eps=c.eps,
                               weight_decay=c.weight_decay, stream=stream)

    def read(self) -> dict:
        return read_step_state(self.state)


def wait_spin(stream) -> None:
    """Waits for the work queued on `stream` by polling an event: the decision that follows sits on the
    critical path between the norm and the update, and polling wakes within microseconds of completion."""
    done = torch.cuda.Event()
    done.record(stream)
    while not done.query():
        pass


def rank_norms(shards, cfg: AdamWConfig, scaler: ScalerState, flatten: bool = True, stream=None) -> dict:
    """First half of a step over the simulated ranks: flatten (and square-norm), the 16-byte readback, the
    simulated all-reduce and the decision.  Updates the loss-scale state; returns the decision."""
    stream = stream or torch.cuda.current_stream()
    for sh in shards:
        if flatten:
            sh.flatten(stream)
        if not (flatten and sh.fused):
            sh.sqnorm(stream)
        sh.readback(stream)
    wait_spin(stream)
    sq, fl = zip(*(sh.norm_result() for sh in shards))
    dec = zero_step_decision(sq, fl, cfg.max_norm, scaler.scale, scaler.good_steps, scaler.growth_interval)
    scaler.scale, scaler.good_steps = dec["loss_scale"], dec["good_steps"]
    dec["rank_sqnorms"] = list(sq)
    dec["rank_flags"] = list(fl)
    return dec


def rank_update(shards, cfg: AdamWConfig, scaler: ScalerState, dec: dict, stream=None) -> None:
    """Second half: the AdamW update of every simulated rank with the decision's factor (nothing on skip)."""
    if dec["skip"]:
        return
    stream = stream or torch.cuda.current_stream()
    scaler.adam_step += 1
    for sh in shards:
        sh.adamw(cfg, dec["grad_scale"], scaler.adam_step, stream)


def rank_step(shards, cfg: AdamWConfig, scaler: ScalerState, flatten: bool = True, stream=None) -> dict:
    """One training step over the simulated ranks; returns the decision (grad_scale, skip, norm, ...)."""
    dec = rank_norms(shards, cfg, scaler, flatten, stream)
    rank_update(shards, cfg, scaler, dec, stream)
    return dec
