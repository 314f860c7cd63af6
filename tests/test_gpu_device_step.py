"""The device-resident decision: one GPU thread repeats the host decision and
scalar derivation, the update kernels read them from device memory, and a
whole step can be captured in a HIP graph."""
import math

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
    from mixed_precision_adam_amd.driver import AdamWConfig, DeviceDecision, RankShard

DEV = "cuda:0"


def _f32bits(x):
    return np.array([x], dtype=np.float32).view(np.uint32)[0]


def test_decision_kernel_matches_host_decision():
    rng = np.random.default_rng(2024)
    state = torch.zeros(16, dtype=torch.float64, device=DEV)
    for trial in range(40):
        n = int(rng.integers(1, 6))
        scale = float(2.0 ** rng.integers(0, 17))
        growth = int(rng.choice([1, 2, 3, 1000]))
        hp = dict(lr=float(rng.choice([0.0, 1e-4, 3e-3, 0.05])), beta1=float(rng.choice([0.0, 0.8, 0.9, 0.99])),
                  beta2=float(rng.choice([0.0, 0.95, 0.999, 0.9999])), eps=float(rng.choice([1e-8, 1e-3])),
                  weight_decay=float(rng.choice([0.0, 0.01, 0.1])))
        max_norm = float(rng.choice([0.0, 0.5, 1.0, 5.0]))
        Z.zero_step_state_init(state, scale, growth)
        h_scale, h_good, h_t = scale, 0, 0
        for it in range(12):
            sq = rng.random(n) * 10.0 ** rng.uniform(-4, 6) * scale * scale
            fl = (rng.random(n) < 0.15).astype(np.int32)
            buf = torch.zeros(n + (n + 1) // 2, dtype=torch.float64, device=DEV)
            buf[:n] = torch.from_numpy(sq)
            buf.view(torch.int32)[2 * n: 3 * n] = torch.from_numpy(fl)
            Z.zero_step_decision_dev(buf.data_ptr(), buf.data_ptr() + 8 * n, n, max_norm, state, **hp)
            got = Z.read_step_state(state)
            host = Z.zero_step_decision(list(sq), list(fl), max_norm, h_scale, h_good, growth)
            h_scale, h_good = host["loss_scale"], host["good_steps"]
            what = f"trial {trial} it {it}"
            assert got["skip"] == host["skip"], what
            assert got["loss_scale"] == host["loss_scale"] and got["good_steps"] == host["good_steps"], what
            assert got["iteration"] == it + 1, what
            if host["skip"]:
                assert math.isnan(got["global_norm"]) and got["grad_scale"] == 0.0, what
                assert got["adam_step"] == h_t, what
                continue
            h_t += 1
            assert got["adam_step"] == h_t, what
            assert got["grad_scale"] == host["grad_scale"], (what, got["grad_scale"], host["grad_scale"])
            assert got["global_norm"] == host["global_norm"], what
            ref = oracle.adamw_scalars(grad_scale=host["grad_scale"], step=h_t, **hp)
            names = ["b1", "omb1", "b2", "omb2", "eps", "decay", "step_size", "bc2_sqrt", "gscale"]
            for k, name in enumerate(names):
                assert _f32bits(got["scalars"][k]) == ref[name].view(np.uint32), (what, name)


def test_update_skips_when_decision_says_so():
    n = 5000
    p = torch.randn(n, device=DEV)
    m, v = torch.zeros(n, device=DEV), torch.zeros(n, device=DEV)
    q = torch.full((n,), 3.0, dtype=torch.bfloat16, device=DEV)
    g = torch.randn(n, device=DEV).to(torch.bfloat16)
    state = torch.zeros(16, dtype=torch.float64, device=DEV)
    Z.zero_step_state_init(state, 1.0, 1000)  # nothing decided yet: skip
    p0 = p.clone()
    Z.zero_adamw_step_dev(g, 0, p, m, v, q, n, state)
    tiled = torch.zeros(Z.zero_state_tiled_numel(n), device=DEV)
    Z.zero_adamw_step_tiled_dev(g, 0, tiled, q, n, state)
    torch.cuda.synchronize()
    assert torch.equal(p, p0) and (m == 0).all() and (q == 3.0).all() and (tiled == 0).all()


def _setup(w, tiled=True, fused=True):
    dev = torch.device(DEV)
    src = torch.empty(w.psi, dtype=torch.bfloat16 if w.grad_kind == synth.BF16 else torch.float16, device=dev)
    gdt = Z.ZERO_BF16 if w.grad_kind == synth.BF16 else Z.ZERO_FP16
    shards = [RankShard(w.numels, w.world, r, gdt, dev, sources=[src], tiled=tiled, fused=fused) for r in w.ranks]
    master_all = synth.fill_host(w.master_field(), 0, w.psi)
    for sh in shards:
        lay = sh.layout
        p = np.zeros(sh.n, np.float32)
        p[:lay.shard_valid] = master_all[lay.shard_offset:lay.shard_offset + lay.shard_valid]
        sh.load_master(torch.from_numpy(p).to(dev))
    return src, shards, master_all


@pytest.mark.parametrize("tiled", [True, False])
def test_device_step_tiny_against_oracle(tiled):
    w = WORKLOADS["tiny"]
    src, shards, master_all = _setup(w, tiled=tiled)
    cfg = AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, max_norm=w.clip)
    dd = DeviceDecision(shards, cfg)
    s = shards[0].n
    refs = []
    for sh in shards:
        lay = sh.layout
        p = np.zeros(s, np.float32)
        p[:lay.shard_valid] = master_all[lay.shard_offset:lay.shard_offset + lay.shard_valid]
        refs.append([p, np.zeros(s, np.float32), np.zeros(s, np.float32), np.zeros(s, np.uint16)])
    oscale, ogood = 1.0, 0
    for t in range(1, w.steps + 1):
        synth.fill_tensor(w.grad_field(t), 0, src)
        dd.step()
        got = dd.read()
        flat = synth.fill_host(w.grad_field(t), 0, w.psi)
        grads = [oracle.flatten([flat], w.numels, w.world, r) for r in w.ranks]
        norms = [oracle.sqnorm(g, 0) for g in grads]
        od = oracle.step_decision([x[0] for x in norms], [x[1] for x in norms], w.clip, oscale, ogood, 2**31 - 1)
        oscale, ogood = od["loss_scale"], od["good_steps"]
        assert got["skip"] == 0 and got["adam_step"] == t
        # the device's factor is one of the correct ones; given it, the update is unique: the oracle applies it
        assert_grad_scale_close(got["grad_scale"], od["grad_scale"], w.world * s, f"step {t}")
        for r, sh in enumerate(shards):
            p, m, v, q = refs[r]
            oracle.adamw_step(grads[r], 0, p, m, v, q, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                              weight_decay=w.weight_decay, grad_scale=got["grad_scale"], step=t)
            gp, gm, gv = (x.cpu().numpy() for x in sh.read_state())
            what = f"step {t} rank {r}"
            nd = assert_f32_close(gp, p, what + " master") + assert_f32_close(gm, m, what + " m")
            nd += assert_f32_close(gv, v, what + " v")
            nd += assert_bf16_within_ulp(sh.param.view(torch.int16).cpu().numpy().view(np.uint16), q, what)
            assert nd == 0, what


def test_device_step_skips_overflow_and_halves_scale():
    w = WORKLOADS["tiny"]
    w16 = type(w)(**{**w.__dict__, "grad_kind": synth.FP16, "loss_scale": 1024.0, "ranks": [0, 1, 2, 3]})
    src, shards, _ = _setup(w16)
    cfg = AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, max_norm=w.clip)
    dd = DeviceDecision(shards, cfg, loss_scale=1024.0, growth_interval=1000)
    synth.fill_tensor(w16.grad_field(1, 1024.0), 0, src)
    dd.step()
    st1 = dd.read()
    assert st1["skip"] == 0 and st1["adam_step"] == 1
    before = [tuple(x.clone() for x in sh.read_state()) + (sh.param.clone(),) for sh in shards]
    synth.fill_tensor(w16.grad_field(2, 1024.0), 0, src)
    src.view(torch.int16)[777_777] = 0x7C00  # +inf lands in rank 3's shard
    dd.step()
    st2 = dd.read()
    assert st2["skip"] == 1 and st2["adam_step"] == 1 and st2["loss_scale"] == 512.0 and st2["iteration"] == 2
    for sh, b in zip(shards, before):
        after = sh.read_state() + (sh.param,)
        for x, y in zip(after, b):
            assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                               y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))
    synth.fill_tensor(w16.grad_field(3, 512.0), 0, src)
    dd.step()
    st3 = dd.read()
    assert st3["skip"] == 0 and st3["adam_step"] == 2 and st3["loss_scale"] == 512.0


def test_whole_step_captured_in_a_graph():
    """Two identical rank sets: one stepped eagerly, one by replaying a captured HIP graph of the whole step
    (flatten+norm, decision, update).  Fresh gradients are written eagerly between replays, with host
    synchronisation in between; every replay must match the eager step bit for bit."""
    w = WORKLOADS["tiny"]
    cfg = AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, max_norm=w.clip)
    src_a, shards_a, _ = _setup(w)
    src_b, shards_b, _ = _setup(w)
    dd_a = DeviceDecision(shards_a, cfg)
    dd_b = DeviceDecision(shards_b, cfg)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dd_b.step()
    # capture recorded the work without running it: the states are still the initial ones
    Z.zero_step_state_init(dd_b.state, 1.0, 2**31 - 1)
    torch.cuda.synchronize()
    for t in range(1, 5):
        synth.fill_tensor(w.grad_field(t), 0, src_a)
        synth.fill_tensor(w.grad_field(t), 0, src_b)
        torch.cuda.synchronize()
        dd_a.step()
        graph.replay()
        torch.cuda.synchronize()
        sa, sb = dd_a.read(), dd_b.read()
        assert sa == sb, (t, sa, sb)
        assert sa["adam_step"] == t
        for a, b in zip(shards_a, shards_b):
            assert torch.equal(a.state.view(torch.int32), b.state.view(torch.int32)), t
            assert torch.equal(a.param.view(torch.int16), b.param.view(torch.int16)), t
            assert torch.equal(a.grad.view(torch.int16), b.grad.view(torch.int16)), t


def test_checkpoint_and_resume_is_bit_exact():
    """A rank's resumable state is its fp32 master / m / v shard, its 16-bit param shard and the step state
    (Adam t, loss scale, good-step count).  Two steps, a copy to host memory, a restore into fresh buffers,
    then three more steps (scale growth and an overflow skip among them) must match the uninterrupted run
    bit for bit."""
    w = WORKLOADS["tiny"]
    cfg = AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, max_norm=w.clip)
    scale, growth = 1024.0, 2
    numels, world = w.numels, w.world

    def fresh():
        src = torch.empty(w.psi, dtype=torch.float16, device=DEV)
        shards = [RankShard(numels, world, r, Z.ZERO_FP16, DEV, sources=[src], tiled=True, fused=True)
                  for r in w.ranks]
        return src, shards

    def field(t):
        return synth.field(w.seed, synth.STREAM_GRAD, t, w.grad_sigma, synth.FP16, scale=scale)

    def grads(src, t):
        synth.fill_tensor(field(t), 0, src)
        if t == 4:
            src.view(torch.int16)[123_456] = 0x7E00  # NaN: this step is skipped and the scale halves

    src_a, a = fresh()
    master_all = torch.empty(w.psi, device=DEV)
    synth.fill_tensor(w.master_field(), 0, master_all)
    for sh in a:
        m0 = torch.zeros(sh.n, device=DEV)
        lay = sh.layout
        m0[:lay.shard_valid] = master_all[lay.shard_offset:lay.shard_offset + lay.shard_valid]
        sh.load_master(m0)
    da = DeviceDecision(a, cfg, loss_scale=scale, growth_interval=growth)
    for t in (1, 2):
        grads(src_a, t)
        da.step()
    torch.cuda.synchronize()
    # checkpoint: host copies only
    saved = [(tuple(x.cpu() for x in sh.read_state()), sh.param.cpu()) for sh in a]
    saved_state = da.state.cpu()
    # restore into a fresh set of buffers
    src_b, b = fresh()
    db = DeviceDecision(b, cfg, loss_scale=1.0, growth_interval=growth)
    for sh, ((p, m, v), q) in zip(b, saved):
        Z.zero_state_tile(p.to(DEV), m.to(DEV), v.to(DEV), sh.state, sh.n)
        sh.param.copy_(q.to(DEV))
    db.state.copy_(saved_state.to(DEV))
    assert torch.equal(db.state.view(torch.int64), da.state.view(torch.int64))
    for t in (3, 4, 5):
        grads(src_a, t)
        grads(src_b, t)
        da.step()
        db.step()
        torch.cuda.synchronize()
        # the step states byte for byte (a skipped step records a NaN norm, which never compares equal)
        assert torch.equal(da.state.view(torch.int64), db.state.view(torch.int64)), (t, da.read(), db.read())
        for x, y in zip(a, b):
            assert torch.equal(x.state.view(torch.int32), y.state.view(torch.int32)), t
            assert torch.equal(x.param.view(torch.int16), y.param.view(torch.int16)), t
    st = da.read()
    assert st["iteration"] == 5 and st["adam_step"] == 4 and st["skip"] == 0


def test_device_decision_refuses_an_underflowed_loss_scale():
    """A run of overflows halves the loss scale without a floor (GradScaler convention); once it is 0, or
    so small that scale² underflows, no decision can be taken.  The host decision refuses with
    ZERO_ERR_INVALID; the device decision must skip the step and record ZERO_STEP_ERR_LOSS_SCALE instead of
    deriving a NaN factor.  Tiny, four ranks, fp16 gradients: the state starts at the smallest positive
    double, an overflow halves it to 0, and the clean step after it must leave every byte of master / m /
    v / param as it was."""
    w = WORKLOADS["tiny"]
    w16 = type(w)(**{**w.__dict__, "grad_kind": synth.FP16, "loss_scale": 1.0, "ranks": [0, 1, 2, 3]})
    src, shards, _ = _setup(w16)
    cfg = AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, max_norm=w.clip)
    tiny_scale = 5e-324
    assert tiny_scale > 0.0 and tiny_scale * 0.5 == 0.0
    dd = DeviceDecision(shards, cfg, loss_scale=tiny_scale, growth_interval=1000)
    synth.fill_tensor(w16.grad_field(1, 1.0), 0, src)
    src.view(torch.int16)[500_001] = 0x7C00  # +inf in rank 2's shard: an ordinary overflow
    dd.step()
    st1 = dd.read()
    assert st1["skip"] == 1 and st1["error"] == 0 and st1["loss_scale"] == 0.0 and st1["adam_step"] == 0
    o1 = oracle.step_decision([1.0], [1], w.clip, tiny_scale, 0, 1000)  # the oracle halves it the same way
    assert o1["skip"] == 1 and o1["loss_scale"] == 0.0
    before = [(sh.state.clone(), sh.param.clone()) for sh in shards]
    synth.fill_tensor(w16.grad_field(2, 1.0), 0, src)  # clean gradients
    dd.step()
    st2 = dd.read()
    assert st2["skip"] == 1 and st2["error"] == Z.ZERO_STEP_ERR_LOSS_SCALE, st2
    assert st2["loss_scale"] == 0.0 and st2["adam_step"] == 0 and st2["iteration"] == 2 and st2["grad_scale"] == 0.0
    for sh, (s0, q0) in zip(shards, before):
        assert torch.equal(sh.state.view(torch.int32), s0.view(torch.int32))
        assert torch.equal(sh.param.view(torch.int16), q0.view(torch.int16))
        assert torch.isfinite(sh.state).all()
    sq = [float(x) for x in dd.norms[:4].cpu()]
    with pytest.raises(Z.ZeroError):
        Z.zero_step_decision(sq, [0, 0, 0, 0], w.clip, 0.0, 0, 1000)
    with pytest.raises(oracle.OracleError):
        oracle.step_decision(sq, [0, 0, 0, 0], w.clip, 0.0, 0, 1000)
    # a usable scale again: the error clears and the step is taken
    Z.zero_step_state_init(dd.state, 1.0, 1000)
    dd.step()
    st3 = dd.read()
    assert st3["skip"] == 0 and st3["error"] == 0 and st3["adam_step"] == 1
    for sh in shards:
        assert torch.isfinite(sh.state).all()
