"""Synthetic workloads: model-shaped tensor lists and per-config input recipes.

The pages size their examples by model (GPT-2 1.5B, 7B and 13B models, a 1T
model over 1024 ranks) but ship no weights or gradients; these recipes stand in
for them.  Tensor lists follow the public architectures (row-major weights,
tensors in module order); values come from the counter-based generator in
``synth`` so any slice can be regenerated.  No method arithmetic here.
"""
from __future__ import annotations

from dataclasses import dataclass, field as dc_field

from . import BF16, F32, FP16, STREAM_GRAD, STREAM_MASTER, Field
from . import field as make_field


def gpt2_tensors(d: int = 1600, layers: int = 48, vocab: int = 50257, ctx: int = 1024, ffn: int = 6400):
    """GPT-2 1.5B: token and position embeddings, 48 pre-LN blocks, final LN; tied LM head."""
    names, numels = ["wte", "wpe"], [vocab * d, ctx * d]
    for i in range(layers):
        for n, k in (("ln1.w", d), ("ln1.b", d), ("qkv.w", d * 3 * d), ("qkv.b", 3 * d), ("proj.w", d * d),
                     ("proj.b", d), ("ln2.w", d), ("ln2.b", d), ("fc.w", d * ffn), ("fc.b", ffn),
                     ("fc2.w", ffn * d), ("fc2.b", d)):
            names.append(f"h{i}.{n}")
            numels.append(k)
    names += ["lnf.w", "lnf.b"]
    numels += [d, d]
    return names, numels


def llama_tensors(d: int, ffn: int, layers: int, vocab: int = 32000):
    """Llama: embedding, RMSNorm + q/k/v/o + RMSNorm + SwiGLU gate/up/down per layer, final norm, untied head."""
    names, numels = ["embed"], [vocab * d]
    for i in range(layers):
        for n, k in (("attn_norm", d), ("q", d * d), ("k", d * d), ("v", d * d), ("o", d * d), ("ffn_norm", d),
                     ("gate", d * ffn), ("up", d * ffn), ("down", ffn * d)):
            names.append(f"l{i}.{n}")
            numels.append(k)
    names += ["norm", "lm_head"]
    numels += [d, vocab * d]
    return names, numels


@dataclass
class Workload:
    """One configuration: tensors, DP world size, simulated ranks and input recipe."""

    name: str
    cid: int
    numels: list
    world: int
    ranks: list               # ranks simulated on the one GPU
    steps: int
    grad_kind: int            # BF16 or FP16
    grad_sigma: float
    loss_scale: float = 1.0   # initial (dynamic) loss scale; grads are stored multiplied by it
    outlier_per_million: int = 0
    outlier_sigma: float = 0.0
    lr: float = 1e-4
    lr_min: float | None = None  # cosine schedule from lr down to lr_min over `steps`
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    clip: float = 1.0
    master_sigma: float = 0.02
    # step -> (value, fraction of the rank's shard) of a single injected non-finite gradient
    inject: dict = dc_field(default_factory=dict)
    flat_shard_only: bool = False  # grads generated straight into the shard (no per-tensor source)

    @property
    def seed(self) -> int:
        return 0x5EED0000 + self.cid

    @property
    def psi(self) -> int:
        return int(sum(self.numels))

    def grad_field(self, step: int, loss_scale: float | None = None) -> Field:
        """Gradients of `step`, stored multiplied by the loss scale in force (fp16 configurations)."""
        if self.grad_kind == FP16:
            scale = self.loss_scale if loss_scale is None else loss_scale
        else:
            scale = 1.0
        return make_field(self.seed, STREAM_GRAD, step, self.grad_sigma, self.grad_kind, scale,
                          self.outlier_per_million, self.outlier_sigma)

    def master_field(self) -> Field:
        return make_field(self.seed, STREAM_MASTER, 0, self.master_sigma, F32)


def _tiny():
    return Workload("tiny", 1, [1_000_003], world=4, ranks=[0, 1, 2, 3], steps=3, grad_kind=BF16, grad_sigma=1e-3)


def _gpt2():
    return Workload("gpt2-1.5b", 2, gpt2_tensors()[1], world=8, ranks=[0], steps=3, grad_kind=BF16, grad_sigma=1e-3)


def _llama7b():
    return Workload("llama-7b", 3, llama_tensors(4096, 11008, 32)[1], world=8, ranks=[3], steps=5, grad_kind=BF16,
                    grad_sigma=1e-3, outlier_per_million=1000, outlier_sigma=1.0)


def _llama13b():
    return Workload("llama-13b", 4, llama_tensors(5120, 13824, 40)[1], world=4, ranks=[0], steps=6,
                    grad_kind=FP16, grad_sigma=1e-3, loss_scale=65536.0,
                    inject={2: (float("inf"), 1 / 3), 5: (float("-inf"), 2 / 3)})


def _t1():
    return Workload("1t-zero3", 5, [10**12], world=1024, ranks=[0], steps=10, grad_kind=FP16, grad_sigma=1e-4,
                    loss_scale=65536.0, lr=1e-4, lr_min=1e-5, flat_shard_only=True)


WORKLOADS = {w.name: w for w in (_tiny(), _gpt2(), _llama7b(), _llama13b(), _t1())}
