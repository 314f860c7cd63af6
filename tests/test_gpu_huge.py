"""GPU parity past 2^32 elements: one rank's shard of 2^32 + 2^21 + 1005 elements.

At this size element indices no longer fit in 32 bits, the flatten's ranges grow past 8192 elements (its
workgroup count is capped at 2^19), the norm's partials take the two-level fold, and the update is issued
in 129 launches.  The shard is the flat concatenation of two tensors (1000 elements, then the rest), N = 1.

  * flatten: every element compared with its source on the device (a bit copy), and windows around
    element 2^32 and at the ends against the generator's values on the host;
  * square-norm (fused and separate passes): the exact closed form of a constant field with a few
    distinct values, which fp64 sums exactly in any order; a NaN past 2^32 sets the flag;
  * AdamW (tiled and separate arrays): two steps, then windows (both ends, around 2^32, and hashed
    positions) against the oracle, to the usual tolerances.

Needs about 120 GB of device memory.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import assert_bf16_within_ulp, assert_f32_close

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixed_precision_adam_amd as Z

DEV = "cuda:0"
N0 = 1000
N1 = 2**32 + 2**21 + 5
S = N0 + N1
BIG = 2**32  # first shard index past 32 bits
SEED = 0x5EED0101
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
TILE = 1024


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def grad_field(step: int):
    return synth.field(SEED, synth.STREAM_GRAD, step, 1e-3, synth.BF16)


def master_field():
    return synth.field(SEED, synth.STREAM_MASTER, 0, 0.02, synth.F32)


def windows():
    """Tile-aligned [a, b) windows: both ends, around 2^32 and six hashed positions."""
    w = [(0, 4096), (BIG - 4096, BIG + 4096), ((S - 3000) // TILE * TILE, S)]
    x = 0x9E3779B97F4A7C15
    for _ in range(6):
        x = (x * 6364136223846793005 + 1442695040888963407) % 2**64
        a = (x >> 20) % (S - 8192) // TILE * TILE
        w.append((a, a + 2048))
    return w


@pytest.fixture(scope="module")
def big():
    if torch.cuda.get_device_properties(0).total_memory < 200 * 2**30:
        pytest.skip("needs about 120 GB of device memory")
    lay, segs = Z.zero_shard_layout([N0, N1], 1, 0)
    assert (lay.shard_numel, lay.shard_valid, len(segs)) == (S, S, 2)
    t0 = torch.empty(N0, dtype=torch.bfloat16, device=DEV)
    t1 = torch.empty(N1, dtype=torch.bfloat16, device=DEV)
    shard = torch.empty(S, dtype=torch.bfloat16, device=DEV)
    table = torch.frombuffer(bytearray(Z.zero_flatten_plan(segs, [t0, t1])), dtype=torch.uint8).to(DEV)
    ws_bytes = Z.zero_grad_sqnorm_workspace_bytes(S)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    out = torch.zeros(2, dtype=torch.float64, device=DEV)  # square-norm, then the int32 flag
    d = dict(t0=t0, t1=t1, shard=shard, table=table, ws=ws, ws_bytes=ws_bytes, out=out)
    yield d
    d.clear()
    del t0, t1, shard, table, ws, out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def read_norm(out: torch.Tensor):
    host = out.cpu().numpy()
    return float(host[0]), int(host[1:2].view(np.int32)[0])


def test_flatten_copies_every_element_past_2_32(big):
    t0, t1, shard = big["t0"], big["t1"], big["shard"]
    gf = grad_field(1)
    synth.fill_tensor(gf, 0, t0)
    synth.fill_tensor(gf, N0, t1)
    shard.view(torch.int16).fill_(0x5A5A)
    Z.zero_flatten_grads(big["table"], 2, Z.ZERO_BF16, shard, S)
    torch.cuda.synchronize()
    assert torch.equal(shard[:N0].view(torch.int16), t0.view(torch.int16))
    assert torch.equal(shard[N0:].view(torch.int16), t1.view(torch.int16))
    for a, b in windows():
        np.testing.assert_array_equal(bits16(shard[a:b]), synth.fill_host(gf, a, b - a), err_msg=f"window {a}")


def test_norm_past_2_32_closed_form(big):
    """A constant field of 2^-10 with four other values (two on either side of element 2^32): every partial
    sum is a multiple of 2^-20 below 2^21, so fp64 holds it exactly and the result is exact in any order."""
    t0, t1, shard, out = big["t0"], big["t1"], big["shard"], big["out"]
    t0.fill_(2.0**-10)
    t1.fill_(2.0**-10)
    special = {5: 3.0, BIG - 1: -0.5, BIG: 1.5, S - 1: 1024.0}  # shard index -> value (all exact in bf16)
    for j, x in special.items():
        if j < N0:
            t0[j] = x
        else:
            t1[j - N0] = x
    exact = (S - len(special)) * Fraction(1, 2**20) + sum(Fraction(x) ** 2 for x in special.values())
    want = float(exact)
    assert Fraction(want) == exact
    for fused in (True, False):
        out.zero_()
        if fused:
            Z.zero_flatten_grads_sqnorm(big["table"], 2, Z.ZERO_BF16, shard, S, big["ws"], big["ws_bytes"],
                                        out.data_ptr(), out.data_ptr() + 8)
        else:
            Z.zero_grad_sqnorm(shard, Z.ZERO_BF16, S, big["ws"], big["ws_bytes"], out.data_ptr(), out.data_ptr() + 8)
        sq, flag = read_norm(out)
        assert (sq, flag) == (want, 0), (fused, sq, want)
    assert torch.equal(shard[N0:].view(torch.int16), t1.view(torch.int16))
    # one NaN past 2^32 sets the flag in both passes
    t1.view(torch.int16)[BIG - N0 + 12_345] = 0x7FC0
    for fused in (True, False):
        out.zero_()
        if fused:
            Z.zero_flatten_grads_sqnorm(big["table"], 2, Z.ZERO_BF16, shard, S, big["ws"], big["ws_bytes"],
                                        out.data_ptr(), out.data_ptr() + 8)
        else:
            Z.zero_grad_sqnorm(shard, Z.ZERO_BF16, S, big["ws"], big["ws_bytes"], out.data_ptr(), out.data_ptr() + 8)
        assert read_norm(out)[1] == 1, fused


@pytest.mark.parametrize("layout", ["tiled", "arrays"])
def test_update_past_2_32_against_oracle(big, layout):
    shard = big["shard"]
    master = torch.empty(S, dtype=torch.float32, device=DEV)
    synth.fill_tensor(master_field(), 0, master)
    param = torch.zeros(S, dtype=torch.bfloat16, device=DEV)
    if layout == "tiled":
        zeros = torch.zeros(S, dtype=torch.float32, device=DEV)
        state = torch.zeros(Z.zero_state_tiled_numel(S), dtype=torch.float32, device=DEV)
        Z.zero_state_tile(master, zeros, zeros, state, S)
        torch.cuda.synchronize()
        del master, zeros
    else:
        m = torch.zeros(S, dtype=torch.float32, device=DEV)
        v = torch.zeros(S, dtype=torch.float32, device=DEV)
    scales = {1: 0.5, 2: 0.25}
    for t, gscale in scales.items():
        synth.fill_tensor(grad_field(t), 0, shard)
        if layout == "tiled":
            Z.zero_adamw_step_tiled(shard, Z.ZERO_BF16, state, param, S, grad_scale=gscale, step=t, **HP)
        else:
            Z.zero_adamw_step(shard, Z.ZERO_BF16, master, m, v, param, S, grad_scale=gscale, step=t, **HP)
    torch.cuda.synchronize()
    tiles = state.view(-1, 3, TILE) if layout == "tiled" else None
    for a, b in windows():
        n = b - a
        ref_p = synth.fill_host(master_field(), a, n)
        ref_m = np.zeros(n, np.float32)
        ref_v = np.zeros(n, np.float32)
        ref_q = np.zeros(n, np.uint16)
        for t, gscale in scales.items():
            oracle.adamw_step(synth.fill_host(grad_field(t), a, n), oracle.BF16, ref_p, ref_m, ref_v, ref_q,
                              grad_scale=gscale, step=t, **HP)
        if layout == "tiled":
            blk = tiles[a // TILE: (b + TILE - 1) // TILE]
            got = [blk[:, k, :].reshape(-1)[:n].cpu().numpy() for k in range(3)]
        else:
            got = [x[a:b].cpu().numpy() for x in (master, m, v)]
        for g, r, what in zip(got, (ref_p, ref_m, ref_v), ("master", "m", "v")):
            assert_f32_close(g, r, f"{layout} {what} window {a}")
        assert_bf16_within_ulp(bits16(param[a:b]), ref_q, f"{layout} param window {a}")
