"""Host-side sequencing of one rank's ZeRO step over the C ABI.

Holds the device buffers of a simulated data-parallel rank (PyTorch
allocations) and calls the library entry points in the order of the step:
flatten -> square-norm -> (simulated all-reduce + decision) -> AdamW.  No
arithmetic of the method happens here; the decision is the library's
``zero_step_decision``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import (ZERO_BF16, ZERO_FP16, zero_adamw_step, zero_flatten_grads, zero_flatten_plan,
               zero_grad_sqnorm, zero_grad_sqnorm_workspace_bytes, zero_shard_layout, zero_step_decision)

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
    """One simulated rank: the flat 16-bit grad shard, fp32 master/m/v, bf16 param and norm scratch."""

    def __init__(self, numels, world: int, rank: int, grad_dtype: int, device="cuda", sources=None):
        self.layout, self.segments = zero_shard_layout(numels, world, rank)
        self.grad_dtype = grad_dtype
        self.device = torch.device(device)
        n = self.layout.shard_numel
        self.n = n
        self.grad = torch.empty(n, dtype=_TORCH16[grad_dtype], device=self.device)
        self.master = torch.zeros(n, dtype=torch.float32, device=self.device)
        self.m = torch.zeros(n, dtype=torch.float32, device=self.device)
        self.v = torch.zeros(n, dtype=torch.float32, device=self.device)
        self.param = torch.zeros(n, dtype=torch.bfloat16, device=self.device)
        self.ws_bytes = zero_grad_sqnorm_workspace_bytes(n)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.sq_dev = torch.zeros(1, dtype=torch.float64, device=self.device)
        self.flag_dev = torch.zeros(1, dtype=torch.int32, device=self.device)
        self.sq_host = torch.zeros(1, dtype=torch.float64).pin_memory()
        self.flag_host = torch.zeros(1, dtype=torch.int32).pin_memory()
        self.seg_table = None
        self.n_segs = 0
        if sources is not None:
            self.set_sources(sources)

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
        zero_flatten_grads(self.seg_table, self.n_segs, self.grad_dtype, self.grad, self.n, stream)

    def sqnorm(self, stream=None) -> None:
        zero_grad_sqnorm(self.grad, self.grad_dtype, self.n, self.ws, self.ws_bytes, self.sq_dev, self.flag_dev,
                         stream)
        self.sq_host.copy_(self.sq_dev, non_blocking=True)
        self.flag_host.copy_(self.flag_dev, non_blocking=True)

    def norm_result(self):
        """Host copies of the last sqnorm; call after the stream has been synchronized."""
        return float(self.sq_host[0]), int(self.flag_host[0])

    def adamw(self, cfg: AdamWConfig, grad_scale: float, step: int, stream=None) -> None:
        zero_adamw_step(self.grad, self.grad_dtype, self.master, self.m, self.v, self.param, self.n, lr=cfg.lr,
                        beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.eps, weight_decay=cfg.weight_decay,
                        grad_scale=grad_scale, step=step, stream=stream)


def rank_step(shards, cfg: AdamWConfig, scaler: ScalerState, flatten: bool = True, stream=None) -> dict:
    """One training step over the simulated ranks; returns the decision (grad_scale, skip, norm, ...)."""
    for sh in shards:
        if flatten:
            sh.flatten(stream)
        sh.sqnorm(stream)
    (stream or torch.cuda.current_stream()).synchronize()
    sq, fl = zip(*(sh.norm_result() for sh in shards))
    dec = zero_step_decision(sq, fl, cfg.max_norm, scaler.scale, scaler.good_steps, scaler.growth_interval)
    scaler.scale, scaler.good_steps = dec["loss_scale"], dec["good_steps"]
    if not dec["skip"]:
        scaler.adam_step += 1
        for sh in shards:
            sh.adamw(cfg, dec["grad_scale"], scaler.adam_step, stream)
    dec["rank_sqnorms"] = list(sq)
    dec["rank_flags"] = list(fl)
    return dec
