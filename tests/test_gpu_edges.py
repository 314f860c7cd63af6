"""GPU parity on small and ragged cases: each C-ABI call against the oracle.

Cases span several tiles plus ragged tails, unaligned base addresses (scalar
paths), empty inputs, all-padding shards and non-finite gradients.  Every
operand sits inside a guard region whose sentinel bits must survive the call.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import assert_bf16_within_ulp, assert_bits_equal, assert_f32_close, assert_norm_close

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixed_precision_adam_amd as Z

DEV = "cuda:0"
GUARD = 64  # elements of sentinel on each side


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def guarded(n: int, dtype, offset: int = 0, fill=None):
    """A tensor of n elements starting `offset` elements past a 256-byte aligned base, plus its guard buffer."""
    total = GUARD + offset + n + GUARD
    buf = torch.empty(total, dtype=dtype, device=DEV)
    if dtype in (torch.float32,):
        buf.view(torch.int32).fill_(0x7FA5A5A5)
    else:
        buf.view(torch.int16).fill_(0x5A5A)
    view = buf[GUARD + offset: GUARD + offset + n]
    if fill is not None:
        view.copy_(fill)
    return buf, view


def check_guards(buf: torch.Tensor, offset: int, n: int, what: str):
    if buf.dtype == torch.float32:
        raw = buf.view(torch.int32).cpu().numpy()
        sentinel = 0x7FA5A5A5
    else:
        raw = buf.view(torch.int16).cpu().numpy().view(np.uint16)
        sentinel = 0x5A5A
    lo = GUARD + offset
    assert (raw[:lo] == sentinel).all() and (raw[lo + n:] == sentinel).all(), f"{what}: guard overwritten"


def to_dev16(bits: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16).copy()).to(DEV).view(dtype)


# ----------------------------------------------------------------------------- flatten

def _flatten_case(numels, world, src_offsets, dt, seed):
    rng = np.random.default_rng(seed)
    tdt = torch.bfloat16 if dt == 0 else torch.float16
    host = [rng.integers(0, 65536, n, dtype=np.uint32).astype(np.uint16) for n in numels]
    keep, srcs = [], []
    for h, off in zip(host, src_offsets):
        buf, view = guarded(len(h), tdt, off)
        view.copy_(to_dev16(h, tdt)) if len(h) else None
        keep.append(buf)
        srcs.append(view.data_ptr() if len(h) else 0)
    for rank in range(world):
        lay, segs = Z.zero_shard_layout(numels, world, rank)
        s = lay.shard_numel
        table = Z.zero_flatten_plan(segs, srcs)
        tab = torch.frombuffer(bytearray(table or b"\0" * 32), dtype=torch.uint8).to(DEV)
        ref = oracle.flatten(host, numels, world, rank)
        rsq, rflag = oracle.sqnorm(ref, dt)
        for dst_off in (0, 3):
            for fused in (False, True):
                sbuf, shard = guarded(s, tdt, dst_off)
                if fused:
                    wsb = Z.zero_grad_sqnorm_workspace_bytes(s)
                    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
                    out = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
                    flag = torch.full((1,), -1, dtype=torch.int32, device=DEV)
                    Z.zero_flatten_grads_sqnorm(tab, len(segs), dt, shard, s, ws, wsb, out, flag)
                else:
                    Z.zero_flatten_grads(tab, len(segs), dt, shard, s)
                torch.cuda.synchronize()
                what = f"flatten rank {rank}/{world} dst_off {dst_off} fused {fused}"
                assert_bits_equal(bits16(shard), ref, what)
                check_guards(sbuf, dst_off, s, "flatten shard")
                if fused:
                    assert int(flag.cpu()[0]) == rflag, what
                    if not rflag:
                        assert_norm_close(float(out.cpu()[0]), rsq, s, what)
    for buf, off, h in zip(keep, src_offsets, host):
        check_guards(buf, off, len(h), "flatten source")


@pytest.mark.parametrize("dt", [0, 1])
def test_flatten_ragged_lists(dt):
    _flatten_case([1000, 1, 0, 77, 4096, 5, 30011], 4, [0] * 7, dt, 1)
    _flatten_case([1000, 1, 0, 77, 4096, 5, 30011], 3, [1, 0, 0, 3, 5, 7, 2], dt, 2)  # mismatched phases
    _flatten_case([8] * 50 + [123457], 8, [8] * 51, dt, 3)


def test_flatten_many_blocks_and_padding():
    # > 1 workgroup per piece, shard not a multiple of 8, last rank mostly padding
    _flatten_case([200_003, 65_536 * 5 + 3, 17], 7, [0, 8, 1], 0, 4)


def test_flatten_fused_norm_finite_values():
    """Finite gradients (the random-bit cases above are mostly flagged), norm compared with the oracle."""
    rng = np.random.default_rng(8)
    numels = [70_001, 3, 65_536 * 2 + 1, 999]
    host = [oracle.f32_to_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32)) for n in numels]
    srcs = [to_dev16(h, torch.bfloat16) for h in host]
    for world in (1, 3):
        for rank in range(world):
            lay, segs = Z.zero_shard_layout(numels, world, rank)
            s = lay.shard_numel
            tab = torch.frombuffer(bytearray(Z.zero_flatten_plan(segs, [x.data_ptr() for x in srcs])),
                                   dtype=torch.uint8).to(DEV)
            shard = torch.empty(s, dtype=torch.bfloat16, device=DEV)
            wsb = Z.zero_grad_sqnorm_workspace_bytes(s)
            ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
            out = torch.zeros(1, dtype=torch.float64, device=DEV)
            flag = torch.full((1,), -1, dtype=torch.int32, device=DEV)
            Z.zero_flatten_grads_sqnorm(tab, len(segs), 0, shard, s, ws, wsb, out, flag)
            torch.cuda.synchronize()
            ref = oracle.flatten(host, numels, world, rank)
            assert_bits_equal(bits16(shard), ref, "fused flatten")
            rsq, rflag = oracle.sqnorm(ref, 0)
            assert int(flag.cpu()[0]) == rflag == 0
            assert_norm_close(float(out.cpu()[0]), rsq, s, f"fused norm {world}/{rank}")
            a = float(out.cpu()[0])
            Z.zero_flatten_grads_sqnorm(tab, len(segs), 0, shard, s, ws, wsb, out, flag)
            torch.cuda.synchronize()
            assert float(out.cpu()[0]) == a  # deterministic


def test_flatten_all_padding_ranks():
    _flatten_case([5], 9, [0], 0, 5)  # ranks 5..8 own only padding
    _flatten_case([1], 1, [0], 1, 6)


# ----------------------------------------------------------------------------- square-norm

def _gpu_sqnorm(bits: np.ndarray, dt: int, offset: int):
    tdt = torch.bfloat16 if dt == 0 else torch.float16
    n = bits.size
    buf, x = guarded(n, tdt, offset)
    if n:
        x.copy_(to_dev16(bits, tdt))
    wsb = Z.zero_grad_sqnorm_workspace_bytes(n)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    out = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
    flag = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    Z.zero_grad_sqnorm(x, dt, n, ws, wsb, out, flag)
    torch.cuda.synchronize()
    check_guards(buf, offset, n, "sqnorm input")
    return float(out.cpu()[0]), int(flag.cpu()[0])


@pytest.mark.parametrize("dt", [0, 1])
@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 255, 4097, 65_536 * 3 + 5, 1_000_003])
def test_sqnorm_sizes(dt, n):
    rng = np.random.default_rng(n + 10 * dt)
    if dt == 0:
        bits = oracle.f32_to_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32))
    else:  # fp16 with a loss-scale-like magnitude plus some subnormals
        v = rng.standard_normal(n) * 60.0
        v[::97] = 3e-7
        bits = v.astype(np.float16).view(np.uint16)
    ref, rflag = oracle.sqnorm(bits, dt)
    for offset in (0, 1, 5):
        got, flag = _gpu_sqnorm(bits, dt, offset)
        assert flag == rflag == 0
        assert_norm_close(got, ref, n, f"sqnorm n={n} off={offset}")


def test_sqnorm_is_deterministic():
    rng = np.random.default_rng(0)
    bits = oracle.f32_to_bf16((rng.standard_normal(3_000_001) * 1e-3).astype(np.float32))
    a = _gpu_sqnorm(bits, 0, 0)
    b = _gpu_sqnorm(bits, 0, 0)
    assert a == b


@pytest.mark.parametrize("dt,pattern", [(0, 0x7F80), (0, 0xFF80), (0, 0x7FC1), (1, 0x7C00), (1, 0xFC00), (1, 0x7E00)])
@pytest.mark.parametrize("where", [0, 3, 77_777, 199_999])
def test_sqnorm_nonfinite(dt, pattern, where):
    bits = np.zeros(200_000, dtype=np.uint16)
    bits[where] = pattern
    for offset in (0, 3):
        _, flag = _gpu_sqnorm(bits, dt, offset)
        assert flag == 1


def test_sqnorm_max_finite_is_not_flagged():
    bits = np.full(1000, 0x7F7F, dtype=np.uint16)
    got, flag = _gpu_sqnorm(bits, 0, 0)
    ref, _ = oracle.sqnorm(bits, 0)
    assert flag == 0
    assert_norm_close(got, ref, 1000, "max bf16")


# ----------------------------------------------------------------------------- AdamW

HP_SETS = [
    dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01),
    dict(lr=1e-2, beta1=0.8, beta2=0.95, eps=1e-3, weight_decay=0.1),
    dict(lr=0.0, beta1=0.0, beta2=0.0, eps=1e-6, weight_decay=0.5),
]


def _adam_case(n, dt, offset, hp, steps, seed, gscales=(1.0, 0.3, 2.0)):
    rng = np.random.default_rng(seed)
    tdt = torch.bfloat16 if dt == 0 else torch.float16
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    p0[::31] = 0.0
    bufs = {k: guarded(n, torch.float32, offset) for k in ("p", "m", "v")}
    bufs["p"][1].copy_(torch.from_numpy(p0))
    bufs["m"][1].zero_()
    bufs["v"][1].zero_()
    qbuf, q = guarded(n, torch.bfloat16, offset)
    gbuf, g = guarded(n, tdt, offset)
    rp, rm, rv = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    rq = np.zeros(n, np.uint16)
    for t in range(1, steps + 1):
        if dt == 0:
            gb = oracle.f32_to_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32))
        else:
            v = rng.standard_normal(n) * 60.0
            v[::53] = 1e-7  # subnormal fp16
            gb = v.astype(np.float16).view(np.uint16)
        gb[::29] = 0
        if n:
            g.copy_(to_dev16(gb, tdt))
        gs = gscales[(t - 1) % len(gscales)]
        Z.zero_adamw_step(g, dt, bufs["p"][1], bufs["m"][1], bufs["v"][1], q, n, grad_scale=gs, step=t, **hp)
        oracle.adamw_step(gb, dt, rp, rm, rv, rq, grad_scale=gs, step=t, **hp)
        torch.cuda.synchronize()
        what = f"adamw n={n} dt={dt} off={offset} t={t}"
        nd = assert_f32_close(bufs["p"][1].cpu().numpy(), rp, what + " master")
        nd += assert_f32_close(bufs["m"][1].cpu().numpy(), rm, what + " m")
        nd += assert_f32_close(bufs["v"][1].cpu().numpy(), rv, what + " v")
        nd += assert_bf16_within_ulp(bits16(q), rq, what + " param")
        assert nd == 0, f"{what}: {nd} elements not bit-identical (within tolerance)"
    for k, (buf, _) in bufs.items():
        check_guards(buf, offset, n, "adamw " + k)
    check_guards(qbuf, offset, n, "adamw param")
    check_guards(gbuf, offset, n, "adamw grad")


@pytest.mark.parametrize("n", [1, 7, 8, 9, 15, 16, 17, 4096 + 8 + 3, 100_003])
@pytest.mark.parametrize("dt", [0, 1])
def test_adamw_sizes_aligned(n, dt):
    _adam_case(n, dt, 0, HP_SETS[0], 3, n + dt)


@pytest.mark.parametrize("offset", [1, 4, 8])
def test_adamw_offsets(offset):
    _adam_case(10_007, 0, offset, HP_SETS[1], 2, offset)


@pytest.mark.parametrize("hi", range(len(HP_SETS)))
def test_adamw_hparam_sets(hi):
    _adam_case(65_536 + 13, 0, 0, HP_SETS[hi], 3, 100 + hi)
    _adam_case(65_536 + 13, 1, 0, HP_SETS[hi], 2, 200 + hi, gscales=(2.0**-16, 2.0**-15))


def test_adamw_zero_padding_stays_zero():
    n = 4099
    p = torch.zeros(n, device=DEV)
    m = torch.zeros(n, device=DEV)
    v = torch.zeros(n, device=DEV)
    q = torch.full((n,), 1.0, dtype=torch.bfloat16, device=DEV)
    g = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    for t in (1, 2):
        Z.zero_adamw_step(g, 0, p, m, v, q, n, grad_scale=0.5, step=t, **HP_SETS[1])
    torch.cuda.synchronize()
    for x in (p, m, v):
        assert (x.view(torch.int32) == 0).all()
    assert (q.view(torch.int16) == 0).all()


def test_adamw_empty_is_noop():
    Z.zero_adamw_step(0, 0, 0, 0, 0, 0, 0, grad_scale=1.0, step=1, **HP_SETS[0])


# ----------------------------------------------------------------------------- tiled state

def _tiled_case(n, dt, gq_offset, hp, steps, seed):
    rng = np.random.default_rng(seed)
    tdt = torch.bfloat16 if dt == 0 else torch.float16
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    tn = Z.zero_state_tiled_numel(n)
    sbuf, state = guarded(tn, torch.float32, 0)
    state.zero_()
    zeros = torch.zeros(n, device=DEV)
    Z.zero_state_tile(torch.from_numpy(p0).to(DEV), zeros, zeros, state, n)
    qbuf, q = guarded(n, torch.bfloat16, gq_offset)
    gbuf, g = guarded(n, tdt, gq_offset)
    rp, rm, rv = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    rq = np.zeros(n, np.uint16)
    for t in range(1, steps + 1):
        if dt == 0:
            gb = oracle.f32_to_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32))
        else:
            gb = (rng.standard_normal(n) * 60.0).astype(np.float16).view(np.uint16)
        g.copy_(to_dev16(gb, tdt))
        Z.zero_adamw_step_tiled(g, dt, state, q, n, grad_scale=0.5, step=t, **hp)
        oracle.adamw_step(gb, dt, rp, rm, rv, rq, grad_scale=0.5, step=t, **hp)
        out = [torch.empty(n, device=DEV) for _ in range(3)]
        Z.zero_state_untile(state, *out, n)
        torch.cuda.synchronize()
        what = f"tiled n={n} dt={dt} off={gq_offset} t={t}"
        nd = assert_f32_close(out[0].cpu().numpy(), rp, what + " master")
        nd += assert_f32_close(out[1].cpu().numpy(), rm, what + " m")
        nd += assert_f32_close(out[2].cpu().numpy(), rv, what + " v")
        nd += assert_bf16_within_ulp(bits16(q), rq, what + " param")
        assert nd == 0, what
    check_guards(sbuf, 0, tn, "tiled state")
    check_guards(qbuf, gq_offset, n, "tiled param")
    # padding floats of the last tile are never written
    T = Z.ZERO_STATE_TILE
    if n % T:
        tail = state.view(-1, 3, T)[-1][:, n % T:]
        assert (tail == 0).all()


# 192 * 1024 + 5 and 3 * 192 * 1024 + 1027: just past one and three spans of the XCD tile grouping (8 XCDs x 24
# tiles), ragged
@pytest.mark.parametrize("n", [1, 5, 1023, 1024, 1025, 2047, 2048, 2049, 2048 + 1027, 4096 * 3 + 7, 100_003,
                               192 * 1024 + 5, 3 * 192 * 1024 + 1027])
@pytest.mark.parametrize("dt", [0, 1])
def test_adamw_tiled_sizes(n, dt):
    _tiled_case(n, dt, 0, HP_SETS[0], 2, n + 7 * dt)


@pytest.mark.parametrize("off", [1, 2, 4])
def test_adamw_tiled_unaligned_grad_param(off):
    _tiled_case(5 * Z.ZERO_STATE_TILE + 3, 0, off, HP_SETS[1], 2, off)


@pytest.mark.parametrize("layout", ["arrays", "tiled"])
def test_adamw_across_launch_boundaries(layout):
    """Shards longer than one launch (2^25 elements) are updated in several launches: a ragged shard that
    spans two of them, element by element against the oracle."""
    n = (1 << 25) + 4096 + 3
    if layout == "arrays":
        _adam_case(n, 0, 0, HP_SETS[1], 2, 77)
    else:
        _tiled_case(n, 0, 0, HP_SETS[1], 2, 78)


def test_tiled_matches_separate_arrays_bitwise():
    n = 300_001
    rng = np.random.default_rng(31)
    p0 = torch.from_numpy((rng.standard_normal(n) * 0.02).astype(np.float32)).to(DEV)
    state = torch.zeros(Z.zero_state_tiled_numel(n), device=DEV)
    zeros = torch.zeros(n, device=DEV)
    Z.zero_state_tile(p0, zeros, zeros, state, n)
    p, m, v = p0.clone(), zeros.clone(), zeros.clone()
    q1 = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    q2 = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    for t in (1, 2, 3):
        g = to_dev16(oracle.f32_to_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32)), torch.bfloat16)
        Z.zero_adamw_step(g, 0, p, m, v, q1, n, grad_scale=0.9, step=t, **HP_SETS[1])
        Z.zero_adamw_step_tiled(g, 0, state, q2, n, grad_scale=0.9, step=t, **HP_SETS[1])
    out = [torch.empty(n, device=DEV) for _ in range(3)]
    Z.zero_state_untile(state, *out, n)
    torch.cuda.synchronize()
    for a, b in zip(out, (p, m, v)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(q1.view(torch.int16), q2.view(torch.int16))


def test_tile_untile_roundtrip():
    T = Z.ZERO_STATE_TILE
    for n in (1, 1000, 1024, 2048, 2049, 4097, 77_777):
        src = [torch.randn(n, device=DEV) for _ in range(3)]
        state = torch.full((Z.zero_state_tiled_numel(n),), 7.0, device=DEV)
        Z.zero_state_tile(*src, state, n)
        back = [torch.empty(n, device=DEV) for _ in range(3)]
        Z.zero_state_untile(state, *back, n)
        torch.cuda.synchronize()
        for a, b in zip(src, back):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        tiles = state.view(-1, 3, T)
        assert torch.equal(tiles[:, 0, :].reshape(-1)[:n], src[0])
        assert torch.equal(tiles[:, 2, :].reshape(-1)[:n], src[2])
        if n % T:
            assert (tiles[-1][:, n % T:] == 7.0).all()


def _same_or_both_nan(got, ref, what):
    got, ref = np.asarray(got, np.float32), np.asarray(ref, np.float32)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all(), f"{what}: NaN positions differ"
    bad = np.nonzero(got[~nan].view(np.uint32) != ref[~nan].view(np.uint32))[0]
    assert bad.size == 0, f"{what}: {bad.size} elements differ, e.g. got {got[~nan][bad[:4]]} want {ref[~nan][bad[:4]]}"


@pytest.mark.parametrize("layout", ["arrays", "tiled"])
@pytest.mark.parametrize("gscale", [1.0, 2.0**-16, 65536.0])
def test_adamw_extreme_values(layout, gscale):
    """Gradients at the edges of bf16 (largest finite, smallest normal, subnormals, signed zeros) and masters at
    the edges of fp32 (largest finite, subnormals, signed zeros), scaled so that products overflow, quotients
    reach inf/inf and results go subnormal: every element must come out bit for bit as the oracle's (both
    evaluate the same correctly rounded IEEE operations with subnormals kept), NaN where the oracle has NaN."""
    g_pat = np.array([0x7F7F, 0xFF7F, 0x0080, 0x8080, 0x0001, 0x8001, 0x007F, 0x0000, 0x8000, 0x3F80, 0xBF80,
                      0x3DCD, 0x7F00, 0x00FF], dtype=np.uint16)
    m_pat = np.array([3.4028235e38, -3.4028235e38, 1e-45, -1e-45, 1.1754944e-38, 0.0, -0.0, 1.0, -2.0, 1e30,
                      1e-30, 5.877472e-39, 65504.0, -7.0e-39], dtype=np.float32)
    rng = np.random.default_rng(int(gscale * 1000) % 2**31 + (layout == "tiled"))
    n = 4096 + 37
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
    p0 = m_pat[rng.integers(0, m_pat.size, n)]
    p = torch.from_numpy(p0.copy()).to(DEV)
    m, v = torch.zeros(n, device=DEV), torch.zeros(n, device=DEV)
    q = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    if layout == "tiled":
        state = torch.zeros(Z.zero_state_tiled_numel(n), device=DEV)
        Z.zero_state_tile(p, m, v, state, n)
    rp, rm, rv, rq = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), np.zeros(n, np.uint16)
    for t in range(1, 4):
        gb = g_pat[rng.integers(0, g_pat.size, n)]
        g = to_dev16(gb, torch.bfloat16)
        if layout == "tiled":
            Z.zero_adamw_step_tiled(g, 0, state, q, n, grad_scale=gscale, step=t, **hp)
            out = [torch.empty(n, device=DEV) for _ in range(3)]
            Z.zero_state_untile(state, *out, n)
        else:
            Z.zero_adamw_step(g, 0, p, m, v, q, n, grad_scale=gscale, step=t, **hp)
            out = [p, m, v]
        oracle.adamw_step(gb, 0, rp, rm, rv, rq, grad_scale=gscale, step=t, **hp)
        torch.cuda.synchronize()
        what = f"extreme {layout} gscale={gscale} t={t}"
        for k, (x, r) in enumerate(zip(out, (rp, rm, rv))):
            _same_or_both_nan(x.cpu().numpy(), r, f"{what} {('master', 'm', 'v')[k]}")
        qg = bits16(q)
        nanq = (rq & 0x7F80) == 0x7F80
        nanq &= (rq & 0x7F) != 0
        assert (qg[~nanq] == rq[~nanq]).all(), what
        assert (((qg[nanq] & 0x7F80) == 0x7F80) & ((qg[nanq] & 0x7F) != 0)).all(), what
