"""Pins for the oracle's codecs, grad norm, clipping, loss scale and schedule (CPU only).

Each oracle function is checked against something other than itself: exact
rational arithmetic, library routines (torch / numpy on the CPU), closed forms
and invariants.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests.parity import f16_probe_bits


# ----------------------------------------------------------------- codecs

def test_bf16_decode_all_patterns():
    pats = np.arange(65536, dtype=np.uint16)
    got = oracle.decode(pats, oracle.BF16)
    ref = torch.from_numpy(pats.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan].view(np.uint32) == ref[~nan].view(np.uint32)).all()


def test_fp16_decode_all_patterns():
    pats = np.arange(65536, dtype=np.uint16)
    got = oracle.decode(pats, oracle.FP16)
    ref = pats.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan].view(np.uint32) == ref[~nan].view(np.uint32)).all()


def test_bf16_rne_against_torch():
    hi = np.repeat(np.arange(65536, dtype=np.uint32), 7) << 16
    lo = np.tile(np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000], dtype=np.uint32), 65536)
    rng = np.random.default_rng(7)
    bits = np.concatenate([hi | lo, rng.integers(0, 2**32, 2_000_000, dtype=np.uint64).astype(np.uint32)])
    x = bits.view(np.float32)
    got = oracle.f32_to_bf16(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert (got[~nan] == ref[~nan]).all()
    assert ((got[nan] & 0x7F80) == 0x7F80).all() and ((got[nan] & 0x7F) != 0).all()


def test_f16_rne_against_numpy_and_torch():
    """fp32 -> binary16 rounding (fp16 parameter output) against two library routines."""
    x = f16_probe_bits().view(np.float32)
    got = oracle.f32_to_f16(x)
    with np.errstate(over="ignore"):
        ref_np = x.astype(np.float16).view(np.uint16)
    ref_t = torch.from_numpy(x.copy()).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert (got[~nan] == ref_np[~nan]).all()
    assert (got[~nan] == ref_t[~nan]).all()
    assert ((got[nan] & 0x7C00) == 0x7C00).all() and ((got[nan] & 0x3FF) != 0).all()


def test_f16_rne_worked_cases():
    """Hand-checked binary16 roundings: the largest finite half, the overflow tie, subnormal ties."""
    cases = [(65504.0, 0x7BFF), (65519.99, 0x7BFF), (65520.0, 0x7C00), (2.0**-24, 0x0001), (2.0**-25, 0x0000),
             (3 * 2.0**-25, 0x0002), (5 * 2.0**-25, 0x0002), (1.0 + 2.0**-11, 0x3C00), (1.0 + 3 * 2.0**-11, 0x3C02),
             (2.0**-14 - 2.0**-25, 0x0400), (-0.0, 0x8000), (1e-10, 0x0000), (-1e9, 0xFC00)]
    for v, bits in cases:
        assert oracle.f32_to_f16(np.array([v], np.float32))[0] == bits, (v, hex(bits))


# ----------------------------------------------------------------- grad norm

def test_sqnorm_hand_vector():
    x = oracle.f32_to_bf16(np.array([3.0, 4.0, 0.0, -0.0], dtype=np.float32))
    assert oracle.sqnorm(x, oracle.BF16) == (25.0, 0)
    h = np.array([3.0, 4.0], dtype=np.float16).view(np.uint16)
    assert oracle.sqnorm(h, oracle.FP16) == (25.0, 0)
    assert oracle.sqnorm(np.zeros(0, np.uint16), oracle.BF16) == (0.0, 0)


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP16])
def test_sqnorm_exact_rational_bound(dtype):
    """Sequential fp64 summation of exact squares: |err| <= (n-1)·2^-53·Σx² against the exact sum."""
    rng = np.random.default_rng(11 + dtype)
    n = 5000
    if dtype == oracle.BF16:
        x = oracle.f32_to_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32))
    else:
        x = (rng.standard_normal(n) * 30).astype(np.float16).view(np.uint16)
    vals = oracle.decode(x, dtype).astype(np.float64)
    exact = sum(Fraction(float(v)) ** 2 for v in vals)
    got, flag = oracle.sqnorm(x, dtype)
    assert flag == 0
    assert abs(Fraction(got) - exact) <= Fraction(n - 1, 2**53) * exact
    # library cross-checks: numpy fp64 and torch vector_norm in fp64
    assert math.isclose(got, float(np.dot(vals, vals)), rel_tol=1e-13)
    assert math.isclose(got, float(torch.linalg.vector_norm(torch.from_numpy(vals)) ** 2), rel_tol=1e-13)


def test_sqnorm_exact_when_representable():
    # Small integers: every partial sum is an exact integer, so the result is exact.
    x = oracle.f32_to_bf16(np.arange(-100, 101, dtype=np.float32))
    assert oracle.sqnorm(x, oracle.BF16)[0] == float(2 * sum(i * i for i in range(101)))


@pytest.mark.parametrize("dtype,pattern,flag", [
    (oracle.BF16, 0x7F80, 1), (oracle.BF16, 0xFF80, 1), (oracle.BF16, 0x7FC0, 1), (oracle.BF16, 0x7F81, 1),
    (oracle.BF16, 0x7F7F, 0), (oracle.BF16, 0x0001, 0),
    (oracle.FP16, 0x7C00, 1), (oracle.FP16, 0xFC00, 1), (oracle.FP16, 0x7E00, 1), (oracle.FP16, 0x7BFF, 0),
    (oracle.FP16, 0x0001, 0)])
def test_sqnorm_nonfinite_flag(dtype, pattern, flag):
    x = np.zeros(1000, dtype=np.uint16)
    x[437] = pattern
    assert oracle.sqnorm(x, dtype)[1] == flag


# ----------------------------------------------------------------- clipping, loss scale, schedule

@pytest.mark.parametrize("max_norm", [1.0, 0.5, 100.0])
def test_clip_coef_against_torch(max_norm):
    rng = np.random.default_rng(3)
    g = [torch.from_numpy(rng.standard_normal(s)) for s in (17, 300, 5)]
    sq = float(sum((t * t).sum() for t in g))
    coef = oracle.clip_coef(sq, max_norm)
    params = []
    for t in g:
        p = torch.nn.Parameter(torch.zeros_like(t))
        p.grad = t.clone()
        params.append(p)
    total = torch.nn.utils.clip_grad_norm_(params, max_norm, foreach=False)
    assert math.isclose(float(total), math.sqrt(sq), rel_tol=1e-14)
    for a, p in zip(g, params):
        np.testing.assert_allclose((a * coef).numpy(), p.grad.numpy(), rtol=1e-14, atol=0)


def test_clip_disabled_and_small_norm():
    assert oracle.clip_coef(1e6, 0.0) == 1.0
    assert oracle.clip_coef(1e6, -1.0) == 1.0
    assert oracle.clip_coef(0.25, 1.0) == 1.0
    assert oracle.clip_coef(4.0, 1.0) == pytest.approx(1 / (2 + 1e-6), rel=1e-15)


def test_loss_scale_against_torch_amp_update():
    scale_t = torch.tensor([65536.0])
    tracker = torch.tensor([0], dtype=torch.int32)
    scale, good = 65536.0, 0
    flags = [0, 1, 0, 0, 1, 0, 0, 0, 0, 0, 0, 1, 1, 0]
    for f in flags:
        torch._amp_update_scale_(scale_t, tracker, torch.tensor([float(f)]), 2.0, 0.5, 3)
        scale, good = oracle.loss_scale_update(scale, f, good, 3)
        assert scale == float(scale_t[0]) and good == int(tracker[0])


def test_cosine_lr_against_torch_closed_form():
    lr_max, lr_min, total = 1e-4, 1e-5, 10
    opt = torch.optim.SGD([torch.nn.Parameter(torch.zeros(1))], lr=lr_max)
    sched = torch.optim.lr_scheduler.CosineAnnealingLR(opt, T_max=total - 1, eta_min=lr_min)
    for t in range(1, total + 1):
        ref = sched._get_closed_form_lr()[0]
        assert math.isclose(oracle.cosine_lr(t, total, lr_max, lr_min), ref, rel_tol=1e-13)
        opt.step()
        sched.step()
    assert oracle.cosine_lr(1, total, lr_max, lr_min) == lr_max
    assert math.isclose(oracle.cosine_lr(total, total, lr_max, lr_min), lr_min, rel_tol=1e-15)


def test_step_decision_against_torch_unscale_and_clip():
    """Unscaling by the loss scale then clip_grad_norm_ (torch, CPU fp64) on the gradients of several
    simulated ranks gives the same per-element multiplier as the oracle's decision."""
    rng = np.random.default_rng(17)
    scale = 1024.0
    ranks = [rng.standard_normal(1000) * 1e-2 * scale for _ in range(4)]
    sq = [float(np.dot(g, g)) for g in ranks]
    dec = oracle.step_decision(sq, [0] * 4, 1.0, scale, 0, 1000)
    params = []
    for g in ranks:
        p = torch.nn.Parameter(torch.zeros(1000, dtype=torch.float64))
        p.grad = torch.from_numpy(g / scale)
        params.append(p)
    total = torch.nn.utils.clip_grad_norm_(params, 1.0, foreach=False)
    assert dec["skip"] == 0 and math.isclose(dec["global_norm"], float(total), rel_tol=1e-13)
    for g, p in zip(ranks, params):
        np.testing.assert_allclose(g * dec["grad_scale"], p.grad.numpy(), rtol=1e-13)
    assert dec["loss_scale"] == scale and dec["good_steps"] == 1


def test_step_decision_overflow_skips_and_halves():
    dec = oracle.step_decision([1.0, float("inf"), 2.0], [0, 1, 0], 1.0, 65536.0, 7, 1000)
    assert dec["skip"] == 1 and dec["loss_scale"] == 32768.0 and dec["good_steps"] == 0
    dec = oracle.step_decision([4.0], [0], 0.0, 1.0, 0, 2**31 - 1)
    assert dec["skip"] == 0 and dec["grad_scale"] == 1.0 and dec["global_norm"] == 2.0


def test_step_decision_refuses_an_unusable_loss_scale():
    """Reading: no decision without a usable loss scale.  IEEE fixes when that happens: the smallest positive
    double squared is 0 and 1e-170 squared underflows to 0, so a step without overflow has no finite unscaled
    norm; 1e-150 squared (1e-300) and 2^-537 squared (2^-1074, the smallest subnormal) are still positive."""
    assert 5e-324 * 5e-324 == 0.0 and 1e-170 * 1e-170 == 0.0
    assert 1e-150 * 1e-150 > 0.0 and 2.0**-537 * 2.0**-537 == 2.0**-1074
    for scale in (0.0, -2.0, float("inf"), float("nan"), 5e-324, 1e-170):
        with pytest.raises(oracle.OracleError):
            oracle.step_decision([2.5], [0], 1.0, scale, 0, 1000)
    for scale in (0.0, float("inf")):
        with pytest.raises(oracle.OracleError):
            oracle.step_decision([2.5], [1], 1.0, scale, 0, 1000)
    dec = oracle.step_decision([2.5], [1], 1.0, 5e-324, 4, 1000)  # an overflow is an ordinary skip
    assert dec["skip"] == 1 and dec["loss_scale"] == 0.0 and dec["good_steps"] == 0
    dec = oracle.step_decision([2.5e-300], [0], 1.0, 2.0**-537, 0, 1000)
    assert dec["skip"] == 0 and dec["global_norm"] == pytest.approx(2.5e-300**0.5 / 2.0**-537, rel=1e-15)
