"""Input generator checks (CPU only): determinism, slicing, distribution and encodings."""
import numpy as np
import torch

import synth
from synth.workloads import WORKLOADS


def test_slices_are_independent_of_chunking():
    f = synth.field(0x5EED0001, synth.STREAM_GRAD, 1, 1e-3, synth.BF16)
    whole = synth.fill_host(f, 0, 300_000)
    parts = np.concatenate([synth.fill_host(f, lo, hi - lo, threads=t)
                            for (lo, hi, t) in [(0, 7, 1), (7, 150_001, 3), (150_001, 300_000, 16)]])
    assert (whole == parts).all()
    again = synth.fill_host(f, 0, 300_000, threads=1)
    assert (whole == again).all()


def test_streams_and_steps_differ():
    a = synth.fill_host(synth.field(1, 1, 1, 1.0, synth.F32), 0, 1000)
    b = synth.fill_host(synth.field(1, 1, 2, 1.0, synth.F32), 0, 1000)
    c = synth.fill_host(synth.field(1, 2, 1, 1.0, synth.F32), 0, 1000)
    assert (a != b).mean() > 0.99 and (a != c).mean() > 0.99


def test_moments_of_the_normal_approximation():
    x = synth.fill_host(synth.field(3, 1, 0, 1.0, synth.F32), 0, 2_000_000).astype(np.float64)
    assert abs(x.mean()) < 3e-3
    assert abs(x.std() - 1.0) < 3e-3
    assert abs(np.abs(x).max()) < 6.0
    # Irwin-Hall(12) excess kurtosis is -0.1
    k = ((x - x.mean()) ** 4).mean() / x.var() ** 2 - 3
    assert abs(k + 0.1) < 0.02


def test_outlier_fraction():
    f = synth.field(4, 1, 0, 1e-3, synth.F32, outlier_per_million=1000, outlier_sigma=1.0)
    x = synth.fill_host(f, 0, 4_000_000)
    frac = (np.abs(x) > 0.01).mean()  # base values stay below 6e-3
    assert 0.0008 < frac < 0.0011


def test_bf16_and_fp16_encodings_are_rne():
    rng_f = synth.field(5, 1, 0, 3.0, synth.F32, scale=1.0)
    v = synth.fill_host(rng_f, 0, 500_000)
    bf = synth.fill_host(synth.field(5, 1, 0, 3.0, synth.BF16), 0, 500_000)
    ref_bf = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (bf == ref_bf).all()
    for sigma in (3.0, 1e-6, 2e4):  # normal, subnormal and overflowing fp16 ranges
        v = synth.fill_host(synth.field(6, 1, 0, sigma, synth.F32), 0, 500_000)
        h = synth.fill_host(synth.field(6, 1, 0, sigma, synth.FP16), 0, 500_000)
        with np.errstate(over="ignore"):
            ref = v.astype(np.float16).view(np.uint16)
        assert (h == ref).all()


def test_workloads_use_global_flat_index():
    w = WORKLOADS["tiny"]
    f = w.grad_field(1)
    flat = synth.fill_host(f, 0, w.psi)
    s = -(-w.psi // w.world)
    for r in w.ranks:
        lo, hi = r * s, min(w.psi, (r + 1) * s)
        assert (synth.fill_host(f, lo, hi - lo) == flat[lo:hi]).all()
