"""fp16 parameter output of the update ([Z] section 四（一）: fp16 parameters and gradients stay whole on
every process; [D]: fp16 training): the kernels' binary16 rounding against the oracle's, bit for bit, on
every rounding boundary, and whole steps with fp16 parameters against the oracle for both state layouts,
the element paths and the device-resident decision."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth.workloads import WORKLOADS
from tests.parity import assert_bf16_within_ulp, assert_f32_close, assert_grad_scale_close, f16_probe_bits

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixed_precision_adam_amd as Z
    from mixed_precision_adam_amd.driver import AdamWConfig, DeviceDecision, RankShard

DEV = "cuda:0"
TORCH16 = {0: torch.bfloat16, 1: torch.float16}
HP_LR0 = dict(lr=0.0, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


def bits16(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def _expect(master, pdt):
    return oracle.f32_to_f16(master) if pdt == 1 else oracle.f32_to_bf16(master)


def _compare_rounding(got, master, pdt, what):
    ref = _expect(master, pdt)
    nan = np.isnan(master)
    bad = np.nonzero(got[~nan] != ref[~nan])[0]
    assert bad.size == 0, f"{what}: {bad.size} params differ, e.g. master bits " \
        f"{master[~nan][bad[:4]].view(np.uint32)} got {got[~nan][bad[:4]]} want {ref[~nan][bad[:4]]}"
    exp_mask = 0x7C00 if pdt == 1 else 0x7F80
    assert ((got[nan] & exp_mask) == exp_mask).all() and ((got[nan] & (0x3FF if pdt == 1 else 0x7F)) != 0).all()


@pytest.mark.parametrize("pdt", [1, 0])
@pytest.mark.parametrize("layout", ["arrays", "tiled"])
@pytest.mark.parametrize("off", [0, 1])
def test_param_rounding_on_every_boundary(pdt, layout, off):
    """lr = 0 leaves the master bits unchanged (decay 1, zero gradient), so the written parameter is the
    master rounded to the parameter format: compare with the oracle's rounding of the same master."""
    master = f16_probe_bits(n_random=400_000).view(np.float32)
    n = master.size
    g = torch.zeros(n + 8, dtype=torch.bfloat16, device=DEV)[off:off + n]
    qbuf = torch.full((n + 16,), 0x5A5A, dtype=torch.int16, device=DEV)
    q = qbuf[8 + off:8 + off + n].view(TORCH16[pdt])
    p = torch.from_numpy(master.copy()).to(DEV)
    zeros = torch.zeros(n, device=DEV)
    if layout == "tiled":
        state = torch.zeros(Z.zero_state_tiled_numel(n), device=DEV)
        Z.zero_state_tile(p, zeros, zeros, state, n)
        Z.zero_adamw_step_tiled(g, 0, state, q, n, grad_scale=1.0, step=1, param_dtype=pdt, **HP_LR0)
        out = [torch.empty(n, device=DEV) for _ in range(3)]
        Z.zero_state_untile(state, *out, n)
        p_after = out[0]
    else:
        m, v = zeros.clone(), zeros.clone()
        Z.zero_adamw_step(g, 0, p, m, v, q, n, grad_scale=1.0, step=1, param_dtype=pdt, **HP_LR0)
        p_after = p
    torch.cuda.synchronize()
    pa = p_after.cpu().numpy()
    same = (pa.view(np.uint32) == master.view(np.uint32)) | (np.isnan(pa) & np.isnan(master))
    assert same.all(), "lr = 0 must leave the master bits"
    _compare_rounding(bits16(q), master, pdt, f"{layout} pdt={pdt} off={off}")
    raw = qbuf.cpu().numpy().view(np.uint16)
    assert (raw[:8 + off] == 0x5A5A).all() and (raw[8 + off + n:] == 0x5A5A).all()


@pytest.mark.parametrize("layout", ["arrays", "tiled"])
@pytest.mark.parametrize("gdt", [0, 1])
@pytest.mark.parametrize("n,off", [(5, 0), (4096 * 3 + 7, 0), (100_003, 0), (10_007, 3)])
def test_fp16_param_steps_against_oracle(layout, gdt, n, off):
    rng = np.random.default_rng(n + 17 * gdt + off)
    hp = dict(lr=1e-2, beta1=0.8, beta2=0.95, eps=1e-3, weight_decay=0.1)
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    p0[::97] *= 4e6   # large parameters: fp16 overflow and the top binades
    p0[5::89] *= 1e-3  # tiny parameters: fp16 subnormals
    gbuf = torch.zeros(n + 8, dtype=TORCH16[gdt], device=DEV)
    g = gbuf[off:off + n]
    qbuf = torch.zeros(n + 8, dtype=torch.float16, device=DEV)
    q = qbuf[off:off + n]
    p = torch.from_numpy(p0.copy()).to(DEV)
    m, v = torch.zeros(n, device=DEV), torch.zeros(n, device=DEV)
    if layout == "tiled":
        state = torch.zeros(Z.zero_state_tiled_numel(n), device=DEV)
        Z.zero_state_tile(p, m, v, state, n)
    rp, rm, rv, rq = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    for t, gs in enumerate((1.0, 0.3, 2.0**-10), start=1):
        if gdt == 0:
            gb = oracle.f32_to_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32))
        else:
            gb = (rng.standard_normal(n) * 60.0).astype(np.float16).view(np.uint16)
        g.copy_(torch.from_numpy(gb.view(np.int16).copy()).to(DEV).view(TORCH16[gdt]))
        if layout == "tiled":
            Z.zero_adamw_step_tiled(g, gdt, state, q, n, grad_scale=gs, step=t, param_dtype=1, **hp)
            out = [torch.empty(n, device=DEV) for _ in range(3)]
            Z.zero_state_untile(state, *out, n)
        else:
            Z.zero_adamw_step(g, gdt, p, m, v, q, n, grad_scale=gs, step=t, param_dtype=1, **hp)
            out = [p, m, v]
        oracle.adamw_step(gb, gdt, rp, rm, rv, rq, grad_scale=gs, step=t, param_dtype=oracle.FP16, **hp)
        torch.cuda.synchronize()
        what = f"{layout} gdt={gdt} n={n} off={off} t={t}"
        nd = assert_f32_close(out[0].cpu().numpy(), rp, what + " master")
        nd += assert_f32_close(out[1].cpu().numpy(), rm, what + " m")
        nd += assert_f32_close(out[2].cpu().numpy(), rv, what + " v")
        nd += assert_bf16_within_ulp(bits16(q), rq, what + " fp16 param")
        assert nd == 0, f"{what}: {nd} elements not bit-identical"
    assert (bits16(q) == 0x7C00).any() or (bits16(q) == 0xFC00).any() or n < 97


@pytest.mark.parametrize("tiled", [True, False])
def test_device_step_with_fp16_params(tiled):
    """The tiny configuration with fp16 gradients under a dynamic loss scale and fp16 parameters, through
    flatten+norm, the device decision and the update, against the oracle."""
    w = WORKLOADS["tiny"]
    scale = 1024.0
    src = torch.empty(w.psi, dtype=torch.float16, device=DEV)
    shards = [RankShard(w.numels, w.world, r, Z.ZERO_FP16, DEV, sources=[src], tiled=tiled, fused=True,
                        param_dtype=Z.ZERO_FP16) for r in w.ranks]
    master_all = synth.fill_host(w.master_field(), 0, w.psi)
    s = shards[0].n
    refs = []
    for sh in shards:
        lay = sh.layout
        p = np.zeros(s, np.float32)
        p[:lay.shard_valid] = master_all[lay.shard_offset:lay.shard_offset + lay.shard_valid]
        sh.load_master(torch.from_numpy(p).to(DEV))
        refs.append([p, np.zeros(s, np.float32), np.zeros(s, np.float32), np.zeros(s, np.uint16)])
    cfg = AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, max_norm=w.clip)
    dd = DeviceDecision(shards, cfg, loss_scale=scale, growth_interval=1000)
    good = 0
    for t in range(1, 4):
        field = synth.field(w.seed, synth.STREAM_GRAD, t, w.grad_sigma, synth.FP16, scale=scale)
        synth.fill_tensor(field, 0, src)
        dd.step()
        got = dd.read()
        flat = synth.fill_host(field, 0, w.psi)
        grads = [oracle.flatten([flat], w.numels, w.world, r) for r in w.ranks]
        norms = [oracle.sqnorm(g, oracle.FP16) for g in grads]
        od = oracle.step_decision([x[0] for x in norms], [x[1] for x in norms], w.clip, scale, good, 1000)
        scale, good = od["loss_scale"], od["good_steps"]
        assert got["skip"] == 0 and got["adam_step"] == t
        same = assert_grad_scale_close(got["grad_scale"], od["grad_scale"], w.world * s, f"step {t}")
        for r, sh in enumerate(shards):
            p, m, v, q = refs[r]
            oracle.adamw_step(grads[r], oracle.FP16, p, m, v, q, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                              weight_decay=w.weight_decay, grad_scale=od["grad_scale"], step=t,
                              param_dtype=oracle.FP16)
            gp, gm, gv = (x.cpu().numpy() for x in sh.read_state())
            what = f"step {t} rank {r}"
            nd = assert_f32_close(gp, p, what + " master") + assert_f32_close(gm, m, what + " m")
            nd += assert_f32_close(gv, v, what + " v")
            assert sh.param.dtype == torch.float16
            nd += assert_bf16_within_ulp(bits16(sh.param), q, what + " fp16 param")
            assert nd == 0 or not same, what
