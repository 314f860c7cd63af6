"""Full-state GPU parity on the small configuration: flat Ψ = 1,000,003 parameters,
N = 4 simulated ranks (all four shards on the one GPU), bf16 gradients, 3 steps.
Every element of every shard is compared with the oracle after every step."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth.workloads import WORKLOADS
from tests.parity import (assert_bf16_within_ulp, assert_bits_equal, assert_f32_close, assert_grad_scale_close,
                          assert_norm_close)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixed_precision_adam_amd as Z
    from mixed_precision_adam_amd.driver import AdamWConfig, RankShard, ScalerState, rank_norms, rank_update


def bits16(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("mode", ["arrays", "slices", "tiled", "tiled-fused", "arrays-fused"])
def test_tiny_all_ranks(mode):
    """arrays: separate master/m/v per rank; slices: the ranks' shards as slices of one flat buffer per
    array; tiled: tiled optimizer state; -fused: flatten and square-norm in one pass."""
    w = WORKLOADS["tiny"]
    dev = torch.device("cuda:0")
    src = torch.empty(w.psi, dtype=torch.bfloat16, device=dev)
    shards = [RankShard(w.numels, w.world, r, Z.ZERO_BF16, dev, sources=[src], tiled=mode.startswith("tiled"),
                        fused=mode.endswith("fused")) for r in w.ranks]
    s = shards[0].n
    if mode == "slices":
        # The four shards as disjoint slices of one padded flat buffer per array (ranks 1..3 start at
        # odd multiples of 4 bytes, so they take the element path).
        flat = {k: torch.zeros(w.world * s, dtype=torch.float32, device=dev) for k in ("master", "m", "v")}
        pflat = torch.zeros(w.world * s, dtype=torch.bfloat16, device=dev)
        gflat = torch.zeros(w.world * s, dtype=torch.bfloat16, device=dev)
        for r, sh in enumerate(shards):
            for k in flat:
                setattr(sh, k, flat[k][r * s:(r + 1) * s])
            sh.param = pflat[r * s:(r + 1) * s]
            sh.grad = gflat[r * s:(r + 1) * s]
    cfg = AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, max_norm=w.clip)
    scaler = ScalerState()

    master_all = synth.fill_host(w.master_field(), 0, w.psi)
    ref = []
    for r, sh in enumerate(shards):
        lay = sh.layout
        p = np.zeros(s, np.float32)
        p[:lay.shard_valid] = master_all[lay.shard_offset:lay.shard_offset + lay.shard_valid]
        sh.load_master(torch.from_numpy(p).to(dev))
        ref.append(dict(p=p.copy(), m=np.zeros(s, np.float32), v=np.zeros(s, np.float32), q=np.zeros(s, np.uint16)))
    oscale, ogood, ostep = 1.0, 0, 0

    for t in range(1, w.steps + 1):
        synth.fill_tensor(w.grad_field(t), 0, src)
        dec = rank_norms(shards, cfg, scaler)
        flat_g = synth.fill_host(w.grad_field(t), 0, w.psi)
        assert_bits_equal(bits16(src), flat_g, f"step {t}: device generator vs host generator")
        og, sqs, fls = [], [], []
        for r, sh in enumerate(shards):
            g = oracle.flatten([flat_g], w.numels, w.world, r)
            og.append(g)
            assert_bits_equal(bits16(sh.grad), g, f"step {t} rank {r} flattened shard")
            sq, fl = oracle.sqnorm(g, oracle.BF16)
            assert dec["rank_flags"][r] == fl == 0
            assert_norm_close(dec["rank_sqnorms"][r], sq, s, f"step {t} rank {r} sqnorm")
            sqs.append(sq)
            fls.append(fl)
        od = oracle.step_decision(sqs, fls, w.clip, oscale, ogood, 2**31 - 1)
        oscale, ogood = od["loss_scale"], od["good_steps"]
        assert dec["skip"] == od["skip"] == 0
        assert_grad_scale_close(dec["grad_scale"], od["grad_scale"], w.world * s, f"step {t}")
        # several square-norms are correct; the update given a factor is unique: apply the oracle's
        rank_update(shards, cfg, scaler, dict(dec, grad_scale=od["grad_scale"]))
        torch.cuda.synchronize()
        ostep += 1
        for r, sh in enumerate(shards):
            R = ref[r]
            oracle.adamw_step(og[r], oracle.BF16, R["p"], R["m"], R["v"], R["q"], lr=w.lr, beta1=w.beta1,
                              beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, grad_scale=od["grad_scale"],
                              step=ostep)
            what = f"step {t} rank {r}"
            gp, gm, gv = (x.cpu().numpy() for x in sh.read_state())
            nd = assert_f32_close(gp, R["p"], what + " master")
            nd += assert_f32_close(gm, R["m"], what + " m")
            nd += assert_f32_close(gv, R["v"], what + " v")
            nd += assert_bf16_within_ulp(bits16(sh.param), R["q"], what + " param")
            assert nd == 0, f"{what}: {nd} elements differ in bits (within tolerance)"
    # the one padding element of rank 3 stays +0 everywhere
    last = shards[-1]
    assert last.layout.shard_valid == s - 1
    for x in last.read_state():
        assert int(x[-1:].view(torch.int32).cpu()[0]) == 0


def test_host_decision_on_a_side_stream():
    """rank_step on a stream other than torch's current one: flatten + norm, the 16-byte readback and the host
    wait all follow that stream, so the decision sees this step's norms.  The side stream is kept busy first
    (a few GB of fills), so a readback not ordered after its norm would read the previous step's values."""
    from mixed_precision_adam_amd.driver import rank_step

    w = WORKLOADS["tiny"]
    dev = torch.device("cuda:0")
    src = torch.empty(w.psi, dtype=torch.bfloat16, device=dev)
    shards = [RankShard(w.numels, w.world, r, Z.ZERO_BF16, dev, sources=[src], tiled=True, fused=True)
              for r in w.ranks]
    s = shards[0].n
    master_all = synth.fill_host(w.master_field(), 0, w.psi)
    ref = []
    for sh in shards:
        lay = sh.layout
        p = np.zeros(s, np.float32)
        p[:lay.shard_valid] = master_all[lay.shard_offset:lay.shard_offset + lay.shard_valid]
        sh.load_master(torch.from_numpy(p).to(dev))
        ref.append([p, np.zeros(s, np.float32), np.zeros(s, np.float32), np.zeros(s, np.uint16)])
    cfg = AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, max_norm=w.clip)
    scaler = ScalerState()
    side = torch.cuda.Stream()
    busy = torch.empty(1 << 29, dtype=torch.float32, device=dev)
    oscale, ogood = 1.0, 0
    for t in (1, 2):
        synth.fill_tensor(w.grad_field(t), 0, src)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(4):
                busy.fill_(float(t))
        dec = rank_step(shards, cfg, scaler, stream=side)
        side.synchronize()
        flat_g = synth.fill_host(w.grad_field(t), 0, w.psi)
        grads = [oracle.flatten([flat_g], w.numels, w.world, r) for r in w.ranks]
        norms = [oracle.sqnorm(g, oracle.BF16) for g in grads]
        for r in w.ranks:
            assert dec["rank_flags"][r] == 0
            assert_norm_close(dec["rank_sqnorms"][r], norms[r][0], s, f"side stream step {t} rank {r}")
        od = oracle.step_decision([x[0] for x in norms], [0] * w.world, w.clip, oscale, ogood, 2**31 - 1)
        oscale, ogood = od["loss_scale"], od["good_steps"]
        assert dec["skip"] == 0
        assert_grad_scale_close(dec["grad_scale"], od["grad_scale"], w.world * s, f"side stream step {t}")
        for r, sh in enumerate(shards):
            P, M, V, Q = ref[r]
            oracle.adamw_step(grads[r], oracle.BF16, P, M, V, Q, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                              weight_decay=w.weight_decay, grad_scale=dec["grad_scale"], step=t)
            gp, gm, gv = (x.cpu().numpy() for x in sh.read_state())
            what = f"side stream step {t} rank {r}"
            nd = assert_f32_close(gp, P, what + " master") + assert_f32_close(gm, M, what + " m")
            nd += assert_f32_close(gv, V, what + " v")
            nd += assert_bf16_within_ulp(bits16(sh.param), Q, what + " param")
            assert nd == 0, what
