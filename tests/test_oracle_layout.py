"""Pins for the oracle's layout and byte accounting (CPU only).

The oracle is pinned to what the pages print (tests/golden/page_memory_pins.json,
each entry cited), to the pages' per-parameter formulas written in other
algebraic forms, to the pages' worked partition examples, and to brute-force
coverage on small cases.
"""
import json
import os
import random

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_memory_pins.json")
PINS = json.load(open(GOLDEN, encoding="utf-8"))

STAGE_FIELD = {0: "bytes_dp", 1: "bytes_zero1", 2: "bytes_zero2", 3: "bytes_zero3"}


def _bytes(psi, world, stage, rank=0):
    lay = oracle.layout([int(psi)], world, rank)
    return getattr(lay, STAGE_FIELD[stage])


@pytest.mark.parametrize("pin", PINS["per_rank_bytes"], ids=lambda p: f"{p['psi']:.3g}-N{p['world']}-s{p['stage']}")
def test_printed_per_rank_bytes(pin):
    got_gb = _bytes(pin["psi"], pin["world"], pin["stage"]) / 1e9
    assert abs(got_gb - pin["printed_gb"]) <= pin["tol"], (got_gb, pin)


def test_printed_bytes_per_param_limits():
    psi, big_n = 2**40, 2**20
    for pin in PINS["bytes_per_param_limits"]:
        n = pin.get("world", big_n)
        per_param = _bytes(psi, n, pin["stage"]) / psi
        assert abs(per_param - pin["printed"]) < 1e-4, pin


def test_printed_reduction_factors_and_linear_stage3():
    psi, n = 2**40, 2**20
    dp = _bytes(psi, n, 0)
    for pin in PINS["reduction_factors"]:
        ratio = dp / _bytes(psi, n, pin["stage"])
        assert ratio < pin["printed"] and ratio > pin["printed"] * 0.9999
    # ZeRO-3 memory falls linearly with N_d ([Z] section 四（三）): exactly N_d when N_d | Ψ.
    for n in (2, 8, 64, 1024):
        assert _bytes(psi, n, 0) == n * _bytes(psi, n, 3)


def test_printed_max_model_fit():
    mm = PINS["max_model_fit"]
    cap = mm["device_gb"] * 1e9
    for stage, printed in mm["printed_psi"].items():
        stage = int(stage)
        # The printed size fits, and a model 5% larger no longer does.
        assert _bytes(printed, mm["world"], stage) <= cap
        assert _bytes(printed * 1.05, mm["world"], stage) > cap


def test_printed_fp16_weights_1p5b():
    pin = PINS["fp16_weights_1p5b_gb"]
    # In ZeRO-3 at N=1 everything is local: params are 2 of the 16 bytes per parameter.
    lay = oracle.layout([int(pin["psi"])], 1, 0)
    assert abs(2 * lay.psi / 1e9 - pin["printed_gb"]) < 0.05
    assert lay.bytes_dp == 8 * 2 * lay.psi


@pytest.mark.parametrize("world", [1, 2, 3, 4, 7, 8, 64, 1024])
def test_formula_forms_agree_when_divisible(world):
    """[X] section 三 gives (4+12/N)Ψ, (2+14/N)Ψ, 16Ψ/N; operatorworld gives 16Ψ − 12Ψ(N−1)/N for
    ZeRO-1 and a further 2Ψ(N−1)/N saving for ZeRO-2; the gitcode note gives 2Ψ+2Ψ+12Ψ/DP,
    2Ψ+2Ψ/DP+12Ψ/DP and (2Ψ+2Ψ+12Ψ)/DP.  With N | Ψ the layout must equal all of them exactly."""
    psi = world * 123457 * 8
    lay = oracle.layout([psi], world, world - 1)
    n = world
    assert lay.bytes_dp == 16 * psi
    assert lay.bytes_zero1 * n == (4 * n + 12) * psi
    assert lay.bytes_zero2 * n == (2 * n + 14) * psi
    assert lay.bytes_zero3 * n == 16 * psi
    assert lay.bytes_zero1 * n == 16 * psi * n - 12 * psi * (n - 1)
    assert lay.bytes_zero2 * n == 16 * psi * n - 12 * psi * (n - 1) - 2 * psi * (n - 1)
    assert lay.bytes_zero1 == 2 * psi + 2 * psi + 12 * psi // n
    assert lay.bytes_zero2 == 2 * psi + 2 * psi // n + 12 * psi // n
    assert lay.bytes_zero3 == (2 * psi + 2 * psi + 12 * psi) // n


def test_padding_excess_is_bounded():
    """For N ∤ Ψ the padded layout exceeds the formulas by less than one padded element's share."""
    for psi, n in [(1_000_003, 4), (10**12, 1024), (97, 8), (5, 9)]:
        lay = oracle.layout([psi], n, 0)
        pad = lay.padded_numel - psi
        assert 0 <= pad < n
        assert 0 <= lay.bytes_zero1 * n - (4 * n + 12) * psi < (4 * n + 12) * n
        assert 0 <= lay.bytes_zero3 * n - 16 * psi < 16 * n


def test_eight_param_four_gpu_example():
    """[Z] section 六（二）: 8 parameters over 4 GPUs, GPU i owns p_{2i} and p_{2i+1}."""
    for r in range(4):
        lay = oracle.layout([1] * 8, 4, r)
        assert lay.shard_numel == 2 and lay.shard_offset == 2 * r and lay.shard_valid == 2
        assert [s[0] for s in lay.segments] == [2 * r, 2 * r + 1]
        assert [s[2] for s in lay.segments] == [0, 1]
        lay1 = oracle.layout([8], 4, r)
        assert lay1.segments == [(0, 2 * r, 0, 2)]


def test_four_block_four_gpu_snapshot():
    """gitcode note section 2: blocks [P0..P3] over 4 GPUs; GPU i keeps optimizer state O_i of P_i."""
    k = 1000
    for r in range(4):
        lay = oracle.layout([k] * 4, 4, r)
        assert lay.segments == [(r, 0, 0, k)]


def test_tiny_config_layout():
    expect = [0, 250_001, 500_002, 750_003]
    for r in range(4):
        lay = oracle.layout([1_000_003], 4, r)
        assert lay.shard_numel == 250_001 and lay.padded_numel == 1_000_004
        assert lay.shard_offset == expect[r]
        assert lay.shard_valid == (250_001 if r < 3 else 250_000)
        assert (lay.bytes_dp, lay.bytes_zero1, lay.bytes_zero2, lay.bytes_zero3) == (
            16_000_048, 7_000_028, 5_500_022, 4_000_016)


def test_brute_force_coverage():
    rng = random.Random(1234)
    for psi in range(0, 65):
        for world in range(1, 10):
            # random split of psi into tensors, including empty ones
            cuts = sorted(rng.randint(0, psi) for _ in range(rng.randint(0, 5)))
            numels = [b - a for a, b in zip([0] + cuts, cuts + [psi])]
            owner = np.full(psi, -1)
            total_valid = 0
            for r in range(world):
                lay = oracle.layout(numels, world, r)
                s = lay.shard_numel
                assert s == -(-psi // world)
                assert lay.padded_numel == world * s and lay.padded_numel - psi < max(world, 1)
                starts = np.cumsum([0] + numels)
                pos = 0
                for (t, so, do, n) in lay.segments:
                    assert n > 0 and do == pos  # contiguous in the shard, in order
                    g0 = starts[t] + so
                    assert 0 <= so and so + n <= numels[t]
                    assert g0 == r * s + do
                    assert (owner[g0:g0 + n] == -1).all()
                    owner[g0:g0 + n] = r
                    pos += n
                assert pos == lay.shard_valid
                total_valid += lay.shard_valid
            assert (owner >= 0).all() and total_valid == psi
            assert all(owner[i] == i // max(1, -(-psi // world)) for i in range(psi))


def test_model_lists_shard_sizes():
    from synth.workloads import WORKLOADS

    expect = {"gpt2-1.5b": (1_557_611_200, 194_701_400), "llama-7b": (6_738_415_616, 842_301_952),
              "llama-13b": (13_015_864_320, 3_253_966_080), "1t-zero3": (10**12, 976_562_500)}
    for name, (psi, s) in expect.items():
        w = WORKLOADS[name]
        lay = oracle.layout(w.numels, w.world, w.ranks[0])
        assert lay.psi == psi and lay.shard_numel == s
    assert oracle.layout(WORKLOADS["1t-zero3"].numels, 1024, 0).bytes_zero3 == 15_625_000_000


def test_error_paths():
    assert oracle.layout_status([4], 0, 0, 4)[0] == -1
    assert oracle.layout_status([4], 2, 2, 4)[0] == -1
    assert oracle.layout_status([4], 2, -1, 4)[0] == -1
    assert oracle.layout_status([-1], 2, 0, 4)[0] == -1
    rc, need = oracle.layout_status([1] * 8, 1, 0, 3)
    assert rc == -2 and need == 8


def test_printed_communication_per_step():
    """Per-rank elements sent per step with ring collectives ([Z] section 六; [X] section 五; operatorworld
    通信账; golden file): 2Ψ / 2Ψ / 2Ψ / 3Ψ for large N, ZeRO-3 = 1.5 x DP, one ring collective (N-1)/N·Ψ."""
    pins = PINS["comm_per_step"]
    psi, n = 2**40, 2**20
    lay = oracle.layout([psi], n, 0)
    got = {"0": lay.comm_dp, "1": lay.comm_zero1, "2": lay.comm_zero2, "3": lay.comm_zero3}
    for stage, mult in pins["printed_multiple_of_psi"].items():
        assert abs(got[stage] / psi - mult) < 1e-5, (stage, got[stage] / psi)
    for n in (2, 4, 8, 64, 1024):
        lay = oracle.layout([n * 1000], n, 0)
        assert lay.comm_zero3 * 2 == lay.comm_dp * 3  # exactly 1.5x
        assert lay.comm_dp * n == 2 * (n - 1) * (n * 1000)  # 2·(N-1)/N·Ψ when N | Ψ
    assert pins["printed_zero3_over_dp"] == 1.5


def test_communication_eight_param_example():
    """[Z] section 六（一）/（二）: 8 parameters on 4 GPUs; a ring reduce-scatter takes 3 rounds of a
    2-element chunk, so each GPU sends 6 elements, and the all-gather another 6."""
    lay = oracle.layout([8], 4, 2)
    assert lay.comm_zero2 == 6 + 6 and lay.comm_dp == 12 and lay.comm_zero3 == 18
    assert oracle.layout([8], 1, 0).comm_dp == 0  # one rank: nothing to exchange
