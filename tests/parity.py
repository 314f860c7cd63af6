"""Comparison helpers shared by the GPU parity tests (no method arithmetic).

Tolerances:
  * layout, offsets, flatten copies, the non-finite flag: bit-exact (integer and byte work);
  * fp32 master / m / v: |gpu - oracle| <= 1e-6 · |oracle| per element (zeros must match exactly); every
    element is one fixed sequence of correctly rounded fp32 operations, so equality is expected;
  * 16-bit param (bf16 or fp16): within 1 ulp (adjacent values);
  * gradient square-norm: within 1e-5 relative of the fp64 oracle, and within the 2n·2^-53 bound of two
    fp64 summation orders.
"""
from __future__ import annotations

import numpy as np

REL_STATE = 1e-6
REL_NORM = 1e-5


def assert_bits_equal(got: np.ndarray, ref: np.ndarray, what: str) -> None:
    got = np.ascontiguousarray(got).reshape(-1)
    ref = np.ascontiguousarray(ref).reshape(-1)
    k = got.dtype.itemsize
    assert ref.dtype.itemsize == k and got.size == ref.size, (what, got.dtype, ref.dtype, got.size, ref.size)
    diff = np.nonzero((got.view(np.uint8).reshape(-1, k) != ref.view(np.uint8).reshape(-1, k)).any(axis=1))[0]
    if diff.size:
        raise AssertionError(f"{what}: {diff.size} of {got.size} elements differ, first at {diff[:5]}: "
                             f"got {got[diff[:5]]} want {ref[diff[:5]]}")


def assert_f32_close(got: np.ndarray, ref: np.ndarray, what: str, rel: float = REL_STATE) -> int:
    """Returns the number of elements whose bits differ (0 expected)."""
    got = np.asarray(got, dtype=np.float32)
    ref = np.asarray(ref, dtype=np.float32)
    assert got.shape == ref.shape
    same = got.view(np.uint32) == ref.view(np.uint32)
    g64, r64 = got.astype(np.float64), ref.astype(np.float64)
    ok = same | (np.abs(g64 - r64) <= rel * np.abs(r64))
    if not ok.all():
        idx = np.nonzero(~ok)[0][:5]
        raise AssertionError(f"{what}: {int((~ok).sum())} elements beyond {rel} relative, e.g. idx {idx}: "
                             f"got {got[idx]} want {ref[idx]}")
    return int((~same).sum())


def assert_bf16_within_ulp(got: np.ndarray, ref: np.ndarray, what: str, ulps: int = 1) -> int:
    """16-bit float bit patterns (uint16; bf16 or fp16, both sign-magnitude). Compares positions on the
    ordered number line."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    got = np.asarray(got, dtype=np.uint16)
    ref = np.asarray(ref, dtype=np.uint16)
    d = np.abs(ordered(got) - ordered(ref))
    if (d > ulps).any():
        idx = np.nonzero(d > ulps)[0][:5]
        raise AssertionError(f"{what}: {int((d > ulps).sum())} params beyond {ulps} ulp, e.g. {idx}: "
                             f"got {got[idx]} want {ref[idx]}")
    return int((d != 0).sum())


def assert_norm_close(got: float, ref: float, n: int, what: str) -> None:
    assert np.isfinite(got) and np.isfinite(ref), (what, got, ref)
    if ref == 0.0:
        assert got == 0.0, (what, got)
        return
    rel = abs(got - ref) / abs(ref)
    assert rel <= REL_NORM, f"{what}: relative error {rel:.3e} > {REL_NORM}"
    # Any summation order of n non-negative fp64 terms stays within n·2^-53 of the exact sum, and so does
    # the sequential oracle: the two can differ by at most twice that.
    assert rel <= 2 * max(n, 1) * 2.0**-53, f"{what}: relative error {rel:.3e} beyond fp64 summation bound"


def assert_grad_scale_close(got: float, ref: float, n: int, what: str) -> bool:
    """The clip/unscale factor comes from each side's own fp64 square-norm; two summation orders of n terms
    differ by at most 2·n·2^-53 relative, the square root halves that, the division adds rounding.
    Returns True when both factors round to the same fp32 value (then the updates must agree bit for bit)."""
    bound = max(1e-13, 2 * max(n, 1) * 2.0**-53)
    assert abs(got - ref) <= bound * abs(ref), f"{what}: grad scale {got!r} vs {ref!r}"
    return bool(np.float32(got) == np.float32(ref))


def f16_probe_bits(n_random: int = 2_000_000, seed: int = 11) -> np.ndarray:
    """fp32 bit patterns on and next to every binary16 rounding boundary (exact ties, one fp32 ulp either
    side, the overflow threshold, the subnormal range), the specials, and random patterns; both signs."""
    h = np.arange(0, 0x7C00, dtype=np.uint32)  # every finite non-negative half
    vals = h.astype(np.uint16).view(np.float16).astype(np.float64)
    nxt = np.append(vals[1:], 65536.0)
    mb = ((vals + nxt) / 2).astype(np.float32).view(np.uint32)  # halfway points are exact in fp32
    base = np.concatenate([mb, mb - 1, mb + 1, vals.astype(np.float32).view(np.uint32)])
    special = np.array([0x477FF000, 0x477FEFFF, 0x477FF001, 0x47800000, 0x7F7FFFFF, 0x33000000, 0x33000001,
                        0x32FFFFFF, 0x33C00000, 0x387FE000, 0x387FF000, 0x38800000, 0x00000001, 0x7F800000,
                        0x7FC00000, 0x7F800001, 0x7FFFFFFF], dtype=np.uint32)
    rng = np.random.default_rng(seed)
    rand = rng.integers(0, 2**32, n_random, dtype=np.uint64).astype(np.uint32)
    near = rng.integers(0x2F000000, 0x48000000, n_random // 2, dtype=np.uint64).astype(np.uint32)
    allb = np.concatenate([base, special, rand, near])
    return np.concatenate([allb, allb | 0x80000000])
