"""Pins for the oracle's AdamW step and flatten (CPU only).

The pages name AdamW with fp32 master/m/v but print no update equations, so the
fp32 oracle is pinned to: torch.optim.AdamW (CPU, fp64 and fp32), the oracle's
own fp64 variant (itself pinned to torch fp64), the step-1 closed form, and
special cases (lr = 0, β1 = β2 = 0, zero padding, loss-scale exactness,
shard-concatenation invariance).  Hyper-parameter sets are chosen so that every
term (decay, both bias corrections, eps, clipping scale) moves the result by
far more than the tolerance.
"""
import numpy as np
import pytest
import torch

import oracle

HP_SETS = [
    dict(lr=1e-2, beta1=0.8, beta2=0.95, eps=1e-3, weight_decay=0.1),
    dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01),
    dict(lr=3e-3, beta1=0.0, beta2=0.5, eps=1e-6, weight_decay=0.0),
    dict(lr=5e-2, beta1=0.99, beta2=0.9999, eps=1e-4, weight_decay=1.0),
]


def _inputs(n, steps, seed, gscale_list):
    rng = np.random.default_rng(seed)
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    grads = [oracle.f32_to_bf16((rng.standard_normal(n) * 1e-3 * (1 + 9 * (rng.random(n) < 0.1))).astype(np.float32))
             for _ in range(steps)]
    return master, grads


def _run_oracle(master0, grads, hp, gscales):
    n = master0.size
    p, m, v = master0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    q = np.zeros(n, np.uint16)
    for t, (g, gs) in enumerate(zip(grads, gscales), start=1):
        oracle.adamw_step(g, oracle.BF16, p, m, v, q, grad_scale=gs, step=t, **hp)
    return p, m, v, q


def _run_torch(master0, grads, hp, gscales, dtype):
    p = torch.nn.Parameter(torch.from_numpy(master0.astype(np.float64)).to(dtype))
    opt = torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"], foreach=False)
    for g, gs in zip(grads, gscales):
        gf = oracle.decode(g, oracle.BF16).astype(np.float64)
        p.grad = (torch.from_numpy(gf) * gs).to(dtype)
        opt.step()
    st = opt.state[p]
    return p.detach().double().numpy(), st["exp_avg"].double().numpy(), st["exp_avg_sq"].double().numpy()


def _run_f64(master0, grads, hp, gscales):
    n = master0.size
    p, m, v = master0.astype(np.float64), np.zeros(n), np.zeros(n)
    for t, (g, gs) in enumerate(zip(grads, gscales), start=1):
        gf = oracle.decode(g, oracle.BF16).astype(np.float64)
        oracle.adamw_step_f64(gf, p, m, v, grad_scale=gs, step=t, **hp)
    return p, m, v


@pytest.mark.parametrize("hi", range(len(HP_SETS)))
def test_f64_variant_matches_torch_adamw_fp64(hi):
    hp = HP_SETS[hi]
    gsc = [1.0, 0.37, 1.0, 2.0, 0.5]
    master0, grads = _inputs(4096, 5, 100 + hi, gsc)
    p, m, v = _run_f64(master0, grads, hp, gsc)
    tp, tm, tv = _run_torch(master0, grads, hp, gsc, torch.float64)
    np.testing.assert_allclose(p, tp, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(m, tm, rtol=1e-12, atol=1e-18)
    np.testing.assert_allclose(v, tv, rtol=1e-12, atol=1e-24)


@pytest.mark.parametrize("hi", range(len(HP_SETS)))
def test_fp32_oracle_within_rounding_of_fp64(hi):
    """fp32 evaluation vs exact-ish fp64: a few ulps of the magnitudes involved per step."""
    hp = HP_SETS[hi]
    gsc = [1.0, 0.37, 1.0, 2.0, 0.5]
    master0, grads = _inputs(4096, 5, 200 + hi, gsc)
    p, m, v, q = _run_oracle(master0, grads, hp, gsc)
    rp, rm, rv = _run_f64(master0, grads, hp, gsc)
    ulp = 2.0**-23
    steps = len(grads)
    # Bound per quantity: (ops per step · steps) ulps of the largest magnitude feeding it.
    mag_p = np.abs(master0).astype(np.float64) + steps * hp["lr"] * 2
    assert (np.abs(p - rp) <= 8 * steps * ulp * mag_p).all()
    gmax = max(float(np.abs(oracle.decode(g, 0)).max()) * s for g, s in zip(grads, gsc))
    assert (np.abs(m - rm) <= 4 * steps * ulp * gmax).all()
    assert (np.abs(v - rv) <= 4 * steps * ulp * gmax * gmax).all()
    # the bf16 output is the RNE rounding of the fp32 master (torch's conversion is RNE)
    tq = torch.from_numpy(p.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (q == tq).all()


@pytest.mark.parametrize("hi", [0, 1])
def test_fp32_oracle_close_to_torch_fp32(hi):
    hp = HP_SETS[hi]
    gsc = [1.0, 1.0, 0.25]
    master0, grads = _inputs(2048, 3, 300 + hi, gsc)
    p, m, v, _ = _run_oracle(master0, grads, hp, gsc)
    tp, tm, tv = _run_torch(master0, grads, hp, gsc, torch.float32)
    np.testing.assert_allclose(p, tp, rtol=2e-6, atol=1e-9)
    np.testing.assert_allclose(m, tm, rtol=1e-5, atol=1e-10)
    np.testing.assert_allclose(v, tv, rtol=1e-5, atol=1e-16)


@pytest.mark.parametrize("hi", range(len(HP_SETS)))
def test_step1_closed_form(hi):
    """At t = 1 with m = v = 0 the bias corrections give m̂ = g and v̂ = g², so
    p1 = p0·(1 − lr·wd) − lr·g/(|g| + eps)."""
    hp = HP_SETS[hi]
    master0, grads = _inputs(4096, 1, 400 + hi, [1.0])
    p, m, v, _ = _run_oracle(master0, grads, hp, [1.0])
    g = oracle.decode(grads[0], 0).astype(np.float64)
    p0 = master0.astype(np.float64)
    expect = p0 * (1 - hp["lr"] * hp["weight_decay"]) - hp["lr"] * g / (np.abs(g) + hp["eps"])
    assert (np.abs(p - expect) <= 1e-6 * (np.abs(p0) + hp["lr"])).all()
    np.testing.assert_allclose(m, (1 - hp["beta1"]) * g, rtol=1e-6)
    np.testing.assert_allclose(v, (1 - hp["beta2"]) * g * g, rtol=1e-6)


def test_four_element_worked_example():
    """A four-element, two-step example worked out beforehand, step by step in numpy float32 from the same
    reading (lr 1e-3, betas (0.9, 0.999), eps 1e-8, wd 0.01, no clipping, p0 = [1, -2, 0.5, 0], gradients
    [0.1, -0.2, 0, 3] then [0.05, 0.2, -0.3, -3]).  That example used fp32 gradients; here they are rounded to
    bf16 first, which leaves every master bit of both steps unchanged at these hyper-parameters (the update
    depends on the gradients through m / sqrt(v), which a common 0.1% rounding barely moves)."""
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    p = np.array([1.0, -2.0, 0.5, 0.0], np.float32)
    m, v, q = np.zeros(4, np.float32), np.zeros(4, np.float32), np.zeros(4, np.uint16)
    expect = [[0x3F7FBDCF, 0xBFFFDE93, 0x3EFFFF58, 0xBA83126E], [0x3F7F8010, 0xBFFFDFA5, 0x3F00301D, 0xBA785824]]
    for t, g in enumerate(([0.1, -0.2, 0.0, 3.0], [0.05, 0.2, -0.3, -3.0]), start=1):
        oracle.adamw_step(oracle.f32_to_bf16(np.array(g, np.float32)), oracle.BF16, p, m, v, q, grad_scale=1.0,
                          step=t, **hp)
        assert p.view(np.uint32).tolist() == expect[t - 1], (t, [hex(x) for x in p.view(np.uint32)])
    assert q[3] == 0xBA78


def test_lr_zero_leaves_master_bits():
    master0, grads = _inputs(1000, 2, 5, [1.0, 1.0])
    p, m, v, q = _run_oracle(master0, grads, dict(lr=0.0, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.5),
                             [1.0, 1.0])
    assert (p.view(np.uint32) == master0.view(np.uint32)).all()
    assert (q == oracle.f32_to_bf16(master0)).all()
    assert (m != 0).any() and (v != 0).any()


def test_fp16_param_output_is_the_rounded_master():
    """With fp16 parameters the update is unchanged and the parameter is the master rounded to binary16;
    the rounding is checked against torch's own conversion (not the oracle's codec)."""
    hp = dict(lr=1e-2, beta1=0.8, beta2=0.95, eps=1e-3, weight_decay=0.1)
    master0, grads = _inputs(5000, 3, 8, [0.5] * 3)
    master0[:4] = [70000.0, -65519.0, 3e-6, 1e-8]  # overflow, round-down, subnormal and underflow parameters
    p, m, v, qb = _run_oracle(master0, grads, hp, [0.5] * 3)
    p2, m2, v2 = master0.copy(), np.zeros_like(master0), np.zeros_like(master0)
    qh = np.zeros(master0.size, np.uint16)
    for t, g in enumerate(grads, start=1):
        oracle.adamw_step(g, oracle.BF16, p2, m2, v2, qh, grad_scale=0.5, step=t, param_dtype=oracle.FP16, **hp)
    for a, b in ((p, p2), (m, m2), (v, v2)):
        assert (a.view(np.uint32) == b.view(np.uint32)).all()
    ref = torch.from_numpy(p2.copy()).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert (qh == ref).all() and qh[0] == 0x7C00
    assert (qb == torch.from_numpy(p.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)).all()


def test_zero_betas_sign_like_update():
    hp = dict(lr=1e-3, beta1=0.0, beta2=0.0, eps=1e-8, weight_decay=0.0)
    master0, grads = _inputs(1000, 3, 6, [1.0] * 3)
    p, _, _, _ = _run_oracle(master0, grads, hp, [1.0] * 3)
    expect = master0.astype(np.float64)
    for g in grads:
        gf = oracle.decode(g, 0).astype(np.float64)
        expect = expect - 1e-3 * gf / (np.abs(gf) + 1e-8)
    np.testing.assert_allclose(p, expect, rtol=0, atol=1e-8)


def test_zero_padding_stays_positive_zero():
    n = 64
    p, m, v = np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.float32)
    q = np.full(n, 0xABCD, np.uint16)
    for t in range(1, 4):
        oracle.adamw_step(np.zeros(n, np.uint16), oracle.BF16, p, m, v, q, grad_scale=0.7, step=t, **HP_SETS[0])
    for a in (p, m, v):
        assert (a.view(np.uint32) == 0).all()
    assert (q == 0).all()


def test_loss_scale_unscale_is_exact():
    """fp16 grads stored as g·2^16 with gscale 2^-16 give the same bits as g with gscale 1."""
    rng = np.random.default_rng(9)
    g = (rng.standard_normal(5000) * 1e-3).astype(np.float16)
    scaled = (g.astype(np.float32) * 65536).astype(np.float16)
    assert (scaled.astype(np.float32) == g.astype(np.float32) * 65536).all()
    outs = []
    for gq, gs in ((g.view(np.uint16), 1.0), (scaled.view(np.uint16), 2.0**-16)):
        p = (rng.standard_normal(5000) * 0.02).astype(np.float32) if not outs else outs[0][4].copy()
        p0 = p.copy()
        m, v, q = np.zeros(5000, np.float32), np.zeros(5000, np.float32), np.zeros(5000, np.uint16)
        oracle.adamw_step(gq, oracle.FP16, p, m, v, q, grad_scale=gs, step=1, **HP_SETS[1])
        outs.append((p, m, v, q, p0))
    for a, b in zip(outs[0][:4], outs[1][:4]):
        assert (a.view(np.uint8) == b.view(np.uint8)).all()


def test_shard_concat_equals_unsharded():
    """[Z] section 四（一）: rank i updates only partition i; gathering the updated partitions must give
    the same parameters as one unsharded update."""
    n, world = 1003, 4
    master0, grads = _inputs(n, 3, 8, [1.0] * 3)
    full = _run_oracle(master0, grads, HP_SETS[0], [1.0] * 3)
    lay = oracle.layout([n], world, 0)
    s = lay.shard_numel
    parts = []
    for r in range(world):
        lo, hi = r * s, min(n, (r + 1) * s)
        parts.append(_run_oracle(master0[lo:hi].copy(), [g[lo:hi].copy() for g in grads], HP_SETS[0], [1.0] * 3))
    for k in range(4):
        cat = np.concatenate([pt[k] for pt in parts])
        assert (cat.view(np.uint8) == full[k].view(np.uint8)).all()


def test_invalid_hparams_rejected():
    with pytest.raises(oracle.OracleError):
        oracle.adamw_scalars(lr=1e-3, beta1=1.0, beta2=0.9, eps=1e-8, weight_decay=0, grad_scale=1, step=1)
    with pytest.raises(oracle.OracleError):
        oracle.adamw_scalars(lr=1e-3, beta1=0.9, beta2=0.9, eps=1e-8, weight_decay=0, grad_scale=1, step=0)


# ----------------------------------------------------------------- flatten

def test_flatten_matches_concatenation_definition():
    rng = np.random.default_rng(21)
    for trial in range(200):
        k = int(rng.integers(1, 7))
        numels = [int(x) for x in rng.integers(0, 40, k)]
        psi = sum(numels)
        if psi == 0:
            continue
        world = int(rng.integers(1, 9))
        tensors = [rng.integers(0, 65536, n, dtype=np.uint32).astype(np.uint16) for n in numels]
        flat = np.concatenate(tensors)
        s = -(-psi // world)
        padded = np.concatenate([flat, np.zeros(world * s - psi, np.uint16)])
        for r in range(world):
            got = oracle.flatten(tensors, numels, world, r)
            assert (got == padded[r * s:(r + 1) * s]).all()


def test_flatten_eight_param_example():
    """[Z] section 六（二）: after reduce-scatter GPU i holds [G_{2i}, G_{2i+1}]."""
    grads = [np.array([0x3F80 + i], np.uint16) for i in range(8)]
    for r in range(4):
        got = oracle.flatten(grads, [1] * 8, 4, r)
        assert list(got) == [0x3F80 + 2 * r, 0x3F80 + 2 * r + 1]


def test_flatten_skips_untouched_tensors():
    numels = [10, 10, 10, 10]
    tensors = [None, np.arange(10, dtype=np.uint16), np.arange(10, 20, dtype=np.uint16), None]
    got = oracle.flatten(tensors, numels, 4, 1)  # rank 1 owns flat [10, 20)
    assert list(got) == list(range(10))
