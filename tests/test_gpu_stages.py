"""Stage equivalence on the GPU: ZeRO changes where model state lives and how
gradients travel, not what a step computes ([D] 误区与复盘, second pitfall;
[Z] section 四).  Three ways of running the same step on one GPU:

  * ZeRO-2: each rank flattens its slice of the per-tensor gradients into its
    own shard buffer (the reduce-scatter landing buffer) and updates it;
  * ZeRO-1: gradients stay in one full all-reduced flat buffer and each rank's
    norm and update read its slice of it directly, with no copy;
  * plain DP: one rank (N = 1) updates everything.

ZeRO-1 and ZeRO-2 must agree bit for bit (same bytes, same alignment, same
kernels), and ZeRO-1 must match the oracle run on the same slices: each
rank's square-norm, the 4-rank decision, and each slice's master / m / v /
param with the oracle applying the device's factor (one of the correct
ones: several fp64 summation orders are).  Gathering the N ranks' state
must equal the DP state bit for bit as long as every step's two fp32
factors have coincided.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import assert_bf16_within_ulp, assert_f32_close, assert_grad_scale_close, assert_norm_close

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixed_precision_adam_amd as Z
    from mixed_precision_adam_amd.driver import AdamWConfig, DeviceDecision, RankShard

DEV = "cuda:0"
NUMELS = [40_000, 1_600, 123_456, 8, 300_000, 97_432]  # Ψ = 562,496: N = 4 gives S = 140,624 = 8·17,578
WORLD = 4
SEED = 0x5EED0042


def _field(t):
    return synth.field(SEED, synth.STREAM_GRAD, t, 1e-3, synth.BF16)


def _master_flat(psi):
    m = torch.zeros(psi, device=DEV)
    synth.fill_tensor(synth.field(SEED, synth.STREAM_MASTER, 0, 0.02, synth.F32), 0, m)
    return m


def test_zero1_zero2_and_dp_agree():
    psi = sum(NUMELS)
    lay0, _ = Z.zero_shard_layout(NUMELS, WORLD, 0)
    s = lay0.shard_numel
    assert s % 8 == 0 and WORLD * s == psi
    cfg = AdamWConfig(lr=3e-3, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.1, max_norm=0.5)
    offs = np.cumsum([0] + NUMELS)
    master = _master_flat(psi)

    # ZeRO-2: per-tensor sources, flatten (+ fused norm) into each rank's shard buffer
    srcs = [torch.empty(n, dtype=torch.bfloat16, device=DEV) for n in NUMELS]
    z2 = [RankShard(NUMELS, WORLD, r, Z.ZERO_BF16, DEV, sources=srcs, tiled=True, fused=False) for r in range(WORLD)]
    for r, sh in enumerate(z2):
        sh.load_master(master[r * s:(r + 1) * s].contiguous())
    d2 = DeviceDecision(z2, cfg)

    # ZeRO-1: one full flat gradient buffer; each rank's grad *is* its slice (16-byte aligned: S % 8 == 0)
    flat = torch.empty(psi, dtype=torch.bfloat16, device=DEV)
    z1 = [RankShard(NUMELS, WORLD, r, Z.ZERO_BF16, DEV, tiled=True) for r in range(WORLD)]
    for r, sh in enumerate(z1):
        sh.grad = flat[r * s:(r + 1) * s]
        sh.load_master(master[r * s:(r + 1) * s].contiguous())
    d1 = DeviceDecision(z1, cfg)

    # DP: a single rank over everything
    dp = RankShard([psi], 1, 0, Z.ZERO_BF16, DEV, tiled=True)
    dp.grad = flat
    dp.load_master(master)
    ddp = DeviceDecision([dp], cfg)

    # the oracle's ZeRO-1 ranks: each reads its slice of the same full flat buffer
    master_host = master.cpu().numpy()
    oref = [[master_host[r * s:(r + 1) * s].copy(), np.zeros(s, np.float32), np.zeros(s, np.float32),
             np.zeros(s, np.uint16)] for r in range(WORLD)]
    ogood, diverged, compared = 0, False, 0
    for t in range(1, 4):
        f = _field(t)
        for k, src in enumerate(srcs):
            synth.fill_tensor(f, int(offs[k]), src)
        synth.fill_tensor(f, 0, flat)
        d2.step()                      # flatten + norm + decide + update
        d1.step(flatten=False)         # norm of the slices + decide + update, no copy
        ddp.step(flatten=False)
        torch.cuda.synchronize()
        s2, s1, sdp = d2.read(), d1.read(), ddp.read()
        # ZeRO-1 against the oracle: each slice's square-norm and flag, the 4-rank decision, each slice's state
        flat_host = synth.fill_host(f, 0, psi)
        onorms = [oracle.sqnorm(flat_host[r * s:(r + 1) * s], oracle.BF16) for r in range(WORLD)]
        sq1 = d1.norms[:WORLD].cpu().numpy()
        fl1 = d1.norms.view(torch.int32)[2 * WORLD: 3 * WORLD].cpu().numpy()
        for r in range(WORLD):
            assert fl1[r] == onorms[r][1] == 0, (t, r)
            assert_norm_close(float(sq1[r]), onorms[r][0], s, f"ZeRO-1 step {t} rank {r} sqnorm")
        od = oracle.step_decision([x[0] for x in onorms], [x[1] for x in onorms], cfg.max_norm, 1.0, ogood,
                                  2**31 - 1)
        ogood = od["good_steps"]
        assert s1["skip"] == od["skip"] == 0 and s1["adam_step"] == t and s1["loss_scale"] == od["loss_scale"]
        # the device's factor is one of the correct ones; given it, the update is unique: the oracle applies it
        assert_grad_scale_close(s1["grad_scale"], od["grad_scale"], psi, f"ZeRO-1 step {t}")
        for r, sh in enumerate(z1):
            P, M, V, Q = oref[r]
            oracle.adamw_step(flat_host[r * s:(r + 1) * s].copy(), oracle.BF16, P, M, V, Q, lr=cfg.lr,
                              beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.eps, weight_decay=cfg.weight_decay,
                              grad_scale=s1["grad_scale"], step=t)
            gp, gm, gv = (x.cpu().numpy() for x in sh.read_state())
            what = f"ZeRO-1 step {t} rank {r}"
            nd = assert_f32_close(gp, P, what + " master") + assert_f32_close(gm, M, what + " m")
            nd += assert_f32_close(gv, V, what + " v")
            nd += assert_bf16_within_ulp(sh.param.view(torch.int16).cpu().numpy().view(np.uint16), Q,
                                         what + " param")
            assert nd == 0, (what, nd)
        assert s1 == s2, (t, s1, s2)
        for a, b in zip(z1, z2):
            assert torch.equal(a.grad.view(torch.int16), b.grad.view(torch.int16))
            assert torch.equal(a.state.view(torch.int32), b.state.view(torch.int32)), t
            assert torch.equal(a.param.view(torch.int16), b.param.view(torch.int16)), t
        # DP and the gathered ZeRO ranks follow the same trajectory as long as every step's two fp32 factors
        # (from two fp64 summation orders, both correct) have coincided; then they agree bit for bit
        same = assert_grad_scale_close(sdp["grad_scale"], s2["grad_scale"], psi, f"step {t} DP vs ZeRO")
        diverged = diverged or not same
        if not diverged:
            compared += 1
            gathered = [torch.cat([x for x in zip(*[sh.read_state() for sh in z2])][k]) for k in range(3)]
            for k in range(3):
                assert torch.equal(gathered[k].view(torch.int32), dp.read_state()[k].view(torch.int32)), (t, k)
            q = torch.cat([sh.param for sh in z2])
            assert torch.equal(q.view(torch.int16), dp.param.view(torch.int16)), t
    assert compared >= 1  # the factors coincide except with probability ~1e-9 per step


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_eight_ranks_equal_dp_at_gpt2_scale():
    """All eight rank shards of the GPT-2 1.5B configuration (1,557,611,200 parameters, 47+ tensor pieces per
    rank), each flattened from the per-tensor gradients, normed, decided and updated on the GPU, then laid end
    to end, against one unsharded rank over the whole model: equal bit for bit whenever the two fp32 factors
    coincide (several fp64 summation orders are correct)."""
    from synth.workloads import WORKLOADS

    w = WORKLOADS["gpt2-1.5b"]
    psi, world = sum(w.numels), w.world
    cfg = AdamWConfig(lr=3e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_norm=1.0)
    offs = np.cumsum([0] + list(w.numels))
    srcs = [torch.empty(n, dtype=torch.bfloat16, device=DEV) for n in w.numels]
    zs = [RankShard(w.numels, world, r, Z.ZERO_BF16, DEV, sources=srcs, tiled=True, fused=True) for r in range(world)]
    s = zs[0].n
    assert world * s == psi  # 8 | Ψ here: no padding, so the shards tile the model exactly
    master = torch.empty(psi, device=DEV)
    synth.fill_tensor(synth.field(SEED, synth.STREAM_MASTER, 0, 0.02, synth.F32), 0, master)
    for r, sh in enumerate(zs):
        sh.load_master(master[r * s:(r + 1) * s].contiguous())
    dz = DeviceDecision(zs, cfg)
    flat = torch.empty(psi, dtype=torch.bfloat16, device=DEV)
    dp = RankShard([psi], 1, 0, Z.ZERO_BF16, DEV, tiled=True)
    dp.grad = flat
    dp.load_master(master)
    del master
    ddp = DeviceDecision([dp], cfg)
    compared = 0
    for t in range(1, 4):
        print(f"[gpt2 x8 vs DP] step {t}", flush=True)
        f = _field(t)
        for k, src in enumerate(srcs):
            synth.fill_tensor(f, int(offs[k]), src)
        synth.fill_tensor(f, 0, flat)
        dz.step()
        ddp.step(flatten=False)
        torch.cuda.synchronize()
        sz, sdp = dz.read(), ddp.read()
        assert sz["skip"] == sdp["skip"] == 0 and sz["adam_step"] == sdp["adam_step"] == t
        same = assert_grad_scale_close(sdp["grad_scale"], sz["grad_scale"], psi, f"step {t}")
        for r, sh in enumerate(zs):  # the gradient shards are the model's gradients, in order
            assert torch.equal(sh.grad.view(torch.int16), flat[r * s:(r + 1) * s].view(torch.int16)), (t, r)
        if same:
            compared += 1
            dpm = dp.read_state()  # untiled master / m / v of the whole model
            for r, sh in enumerate(zs):
                zm = sh.read_state()
                lo, hi = r * s, (r + 1) * s
                for k in range(3):
                    assert torch.equal(zm[k].view(torch.int32), dpm[k][lo:hi].view(torch.int32)), (t, r, k)
                assert torch.equal(sh.param.view(torch.int16), dp.param[lo:hi].view(torch.int16)), (t, r)
                del zm
            del dpm
    assert compared >= 1  # the factors coincide except with probability ~1e-4 per step
