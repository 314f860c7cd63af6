"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, rejects bad arguments before touching the device, and its host-only
entry points (layout, decision helpers) match the oracle exactly."""
import math
import os
import random
import re

import numpy as np
import pytest

import mixed_precision_adam_amd as Z
import oracle
from synth.workloads import WORKLOADS

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "zero_shard.h")


def _declared():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zero_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 11
    lib = Z.library()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(Z.EXPORTS)


def test_invalid_arguments_rejected_without_device():
    lib = Z.library()
    assert lib.zero_adamw_step(None, 0, None, None, None, None, 0, -1, None, None) == Z.ZERO_ERR_INVALID
    hp = Z.zero_adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.0, 1.0, 0)  # step 0 is invalid
    rc = lib.zero_adamw_step(16, 0, 16, 16, 16, 16, 0, 8, hp, None)
    assert rc == Z.ZERO_ERR_INVALID and "hyper" in Z.zero_last_error()
    hp = Z.zero_adamw_hparams(1e-3, 1.0, 0.999, 1e-8, 0.0, 1.0, 1)  # beta1 = 1 is invalid
    assert lib.zero_adamw_step(16, 0, 16, 16, 16, 16, 0, 8, hp, None) == Z.ZERO_ERR_INVALID
    hp = Z.zero_adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.0, float("inf"), 1)
    assert lib.zero_adamw_step(16, 0, 16, 16, 16, 16, 0, 8, hp, None) == Z.ZERO_ERR_INVALID
    hp = Z.zero_adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.0, 1.0, 1)
    assert lib.zero_adamw_step(16, 7, 16, 16, 16, 16, 0, 8, hp, None) == Z.ZERO_ERR_INVALID  # dtype
    assert lib.zero_adamw_step(16, 0, 16, 16, 16, 16, 2, 8, hp, None) == Z.ZERO_ERR_INVALID  # parameter dtype
    assert "parameter dtype" in Z.zero_last_error()
    assert lib.zero_adamw_step(16, 0, 18, 16, 16, 16, 0, 8, hp, None) == Z.ZERO_ERR_INVALID  # fp32 misaligned
    assert lib.zero_adamw_step(None, 0, 16, 16, 16, 16, 0, 8, hp, None) == Z.ZERO_ERR_INVALID
    assert lib.zero_adamw_step(None, 0, None, None, None, None, 0, 0, hp, None) == Z.ZERO_OK  # n = 0: no-op
    assert lib.zero_flatten_grads(None, 3, 0, 16, 8, None) == Z.ZERO_ERR_INVALID
    assert lib.zero_flatten_grads(16, -1, 0, 16, 8, None) == Z.ZERO_ERR_INVALID
    assert lib.zero_flatten_grads(16, 1, 0, 17, 8, None) == Z.ZERO_ERR_INVALID  # odd shard address
    assert lib.zero_flatten_grads(16, 1, 0, None, 8, None) == Z.ZERO_ERR_INVALID
    assert lib.zero_flatten_grads(None, 0, 0, None, 0, None) == Z.ZERO_OK
    ws = Z.zero_grad_sqnorm_workspace_bytes(1000)
    assert ws % 256 == 0 and ws >= 12
    assert lib.zero_grad_sqnorm(16, 0, 1000, 256, ws - 1, 16, 16, None) == Z.ZERO_ERR_INVALID
    assert lib.zero_grad_sqnorm(16, 0, 1000, 257, ws, 16, 16, None) == Z.ZERO_ERR_INVALID  # ws alignment
    assert lib.zero_grad_sqnorm(16, 0, 1000, 256, ws, None, 16, None) == Z.ZERO_ERR_INVALID
    assert lib.zero_grad_sqnorm(None, 0, 10, 256, ws, 16, 16, None) == Z.ZERO_ERR_INVALID
    assert lib.zero_grad_sqnorm(16, 2, 10, 256, ws, 16, 16, None) == Z.ZERO_ERR_INVALID


def test_workspace_size_is_bounded():
    """At most 2^19 partials of 12 bytes (6 MiB) whatever the size; one 8192-element range per partial up to
    4.3e9 elements."""
    assert Z.zero_grad_sqnorm_workspace_bytes(0) == 256
    cap = 12 * (1 << 19)
    for n in (10**9, 3_253_966_080, 1 << 32, 10**10, 10**12, 2**62):
        assert Z.zero_grad_sqnorm_workspace_bytes(n) <= cap, n
        assert Z.zero_flatten_partials_count(n) <= 1 << 19, n
    assert Z.zero_flatten_partials_count(3_253_966_080) == -(-3_253_966_080 // 8192)
    assert Z.zero_flatten_partials_count(194_701_400) == -(-194_701_400 // 8192)


def _same_layout(numels, world, rank):
    lay, segs = Z.zero_shard_layout(numels, world, rank)
    ref = oracle.layout(numels, world, rank)
    for f in ("psi", "padded_numel", "shard_numel", "shard_offset", "shard_valid", "world", "rank", "bytes_dp",
              "bytes_zero1", "bytes_zero2", "bytes_zero3", "comm_dp", "comm_zero1", "comm_zero2", "comm_zero3"):
        assert getattr(lay, f) == getattr(ref, f), (f, numels, world, rank)
    assert [(s.tensor, s.src_offset, s.dst_offset, s.numel) for s in segs] == ref.segments


def test_layout_parity_brute_force():
    rng = random.Random(99)
    for psi in range(0, 70):
        for world in range(1, 10):
            cuts = sorted(rng.randint(0, psi) for _ in range(rng.randint(0, 6)))
            numels = [b - a for a, b in zip([0] + cuts, cuts + [psi])]
            for rank in range(world):
                _same_layout(numels, world, rank)


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_layout_parity_workloads(name):
    w = WORKLOADS[name]
    for rank in sorted(set(w.ranks + [0, w.world - 1, w.world // 2])):
        _same_layout(w.numels, w.world, rank)


def test_layout_errors_and_capacity():
    lib = Z.library()
    arr = (Z.C.c_int64 * 8)(*([1] * 8))
    out = Z.zero_layout()
    n = Z.C.c_int32(-1)
    segs = (Z.zero_segment * 3)()
    assert lib.zero_shard_layout(Z.C.cast(arr, Z._P), 8, 1, 0, Z.C.byref(out), Z.C.cast(segs, Z._P), 3,
                                 Z.C.byref(n)) == Z.ZERO_ERR_CAPACITY
    assert n.value == 8 and out.psi == 8
    assert lib.zero_shard_layout(Z.C.cast(arr, Z._P), 8, 0, 0, Z.C.byref(out), None, 0, Z.C.byref(n)) == -1
    assert lib.zero_shard_layout(Z.C.cast(arr, Z._P), 8, 4, 4, Z.C.byref(out), None, 0, Z.C.byref(n)) == -1
    bad = (Z.C.c_int64 * 1)(-5)
    assert lib.zero_shard_layout(Z.C.cast(bad, Z._P), 1, 4, 0, Z.C.byref(out), None, 0, Z.C.byref(n)) == -1
    huge = (Z.C.c_int64 * 2)(2**62, 2**62)
    assert lib.zero_shard_layout(Z.C.cast(huge, Z._P), 2, 4, 0, Z.C.byref(out), None, 0, Z.C.byref(n)) == -1


def test_host_decision_parity():
    rng = np.random.default_rng(5)
    for trial in range(300):
        k = int(rng.integers(1, 9))
        sq = list(rng.random(k) * 10 ** rng.uniform(-6, 6))
        fl = [int(x) for x in (rng.random(k) < 0.1)]
        args = (float(rng.choice([0.0, 0.5, 1.0, 5.0])), float(2.0 ** rng.integers(0, 17)), int(rng.integers(0, 5)),
                int(rng.integers(1, 6)))
        a = Z.zero_step_decision(sq, fl, *args)
        b = oracle.step_decision(sq, fl, *args)
        for key in ("grad_scale", "skip", "loss_scale", "good_steps"):
            assert a[key] == b[key], (key, a, b)
        assert (math.isnan(a["global_norm"]) and math.isnan(b["global_norm"])) or a["global_norm"] == b["global_norm"]
    for t in range(1, 11):
        assert Z.zero_cosine_lr(t, 10, 1e-4, 1e-5) == oracle.cosine_lr(t, 10, 1e-4, 1e-5)
    for sq, mx in [(0.0, 1.0), (1.0, 1.0), (1e6, 1.0), (3.0, 0.0), (4.0, -1.0)]:
        assert Z.zero_clip_coef(sq, mx) == oracle.clip_coef(sq, mx)
    for flag in (0, 1):
        assert Z.zero_loss_scale_update(1024.0, flag, 2, 3) == oracle.loss_scale_update(1024.0, flag, 2, 3)


def test_flatten_plan_packs_descriptors():
    lay, segs = Z.zero_shard_layout([10, 20, 30], 2, 0)  # rank 0 owns flat [0, 30)
    blob = Z.zero_flatten_plan(segs, [0x1000, 0x2000, 0])  # tensor 2 does not land: no address needed
    rec = np.frombuffer(blob, dtype=np.int64).reshape(-1, 4)
    assert rec.shape == (2, 4)
    assert tuple(rec[0]) == (0x1000, 0, 0, 10) and tuple(rec[1]) == (0x2000, 0, 10, 20)
    with pytest.raises(Z.ZeroError):
        Z.zero_flatten_plan(segs, [0x1000, 0, 0x3000])  # a landing tensor without an address


def test_single_hip_runtime():
    import synth

    synth._load()
    paths = Z.hip_runtimes_loaded()
    assert len(paths) == 1 and "torch" in paths[0], paths


def test_tiled_numel_and_invalid_tiled_args():
    T = Z.ZERO_STATE_TILE
    assert T == 1024
    assert Z.zero_state_tiled_numel(0) == 0
    assert Z.zero_state_tiled_numel(1) == 3 * T
    assert Z.zero_state_tiled_numel(T) == 3 * T
    assert Z.zero_state_tiled_numel(T + 1) == 6 * T
    lib = Z.library()
    hp = Z.zero_adamw_hparams(1e-3, 0.9, 0.999, 1e-8, 0.0, 1.0, 1)
    assert lib.zero_adamw_step_tiled(16, 0, 24, 16, 0, 8, hp, None) == Z.ZERO_ERR_INVALID  # state not 16-B aligned
    assert lib.zero_adamw_step_tiled(16, 0, None, 16, 0, 8, hp, None) == Z.ZERO_ERR_INVALID
    assert lib.zero_adamw_step_tiled(17, 0, 16, 16, 0, 8, hp, None) == Z.ZERO_ERR_INVALID
    assert lib.zero_state_tile(None, 16, 16, 16, 5, None) == Z.ZERO_ERR_INVALID
    assert lib.zero_state_untile(16, 16, 16, 16, -1, None) == Z.ZERO_ERR_INVALID
    assert lib.zero_state_tile(16, 16, 16, 18, 5, None) == Z.ZERO_ERR_INVALID  # state not 4-B aligned
    assert lib.zero_state_untile(16, 16, 22, 16, 5, None) == Z.ZERO_ERR_INVALID  # m not 4-B aligned
    ws = Z.zero_grad_sqnorm_workspace_bytes(100)
    assert lib.zero_flatten_grads_sqnorm(16, 1, 0, 16, 100, 256, ws - 1, 16, 16, None) == Z.ZERO_ERR_INVALID
    assert lib.zero_flatten_grads_sqnorm(12, 1, 0, 16, 100, 256, ws, 16, 16, None) == Z.ZERO_ERR_INVALID


def test_bucket_segments_cover_the_shard_once():
    """Constant-capacity windows over a shard: every valid shard element is covered by exactly one clipped
    segment, offsets are window-relative, the padding is covered by none, and each clipped piece reads the
    same tensor element as the unclipped layout."""
    from synth.workloads import gpt2_tensors

    numels = gpt2_tensors(d=128, layers=2, vocab=500, ctx=32, ffn=512)[1]
    for world, rank in [(1, 0), (4, 3), (7, 2)]:
        lay, segs = Z.zero_shard_layout(numels, world, rank)
        src_of = np.full(lay.shard_numel, -1, np.int64)  # tensor-global element read into each shard slot
        starts = np.cumsum([0] + numels)
        for sg in segs:
            g0 = starts[sg.tensor] + sg.src_offset
            src_of[sg.dst_offset:sg.dst_offset + sg.numel] = np.arange(g0, g0 + sg.numel)
        for cap in (8, 1000, 4096, lay.shard_numel + 5):
            covered = np.zeros(lay.shard_numel, np.int32)
            for a in range(0, lay.shard_numel, cap):
                b = min(lay.shard_numel, a + cap)
                for sg in Z.zero_bucket_segments(segs, a, b - a):
                    assert sg.numel > 0 and 0 <= sg.dst_offset and sg.dst_offset + sg.numel <= b - a
                    lo = a + sg.dst_offset
                    covered[lo:lo + sg.numel] += 1
                    g0 = starts[sg.tensor] + sg.src_offset
                    assert (src_of[lo:lo + sg.numel] == np.arange(g0, g0 + sg.numel)).all()
            assert (covered[:lay.shard_valid] == 1).all() and (covered[lay.shard_valid:] == 0).all()
    lay, segs = Z.zero_shard_layout([10], 1, 0)
    assert Z.zero_bucket_segments(segs, 10, 0) == [] and Z.zero_bucket_segments(segs, 3, 0) == []
    with pytest.raises(Exception):
        Z.zero_bucket_segments(segs, -1, 4)



def test_flatten_partials_count_is_not_monotone():
    """Past 2^19 partials the flatten's ranges grow, so a 2^32-element window can run more workgroups
    (partials) than a larger one: a shared partials buffer is sized by summing the windows' counts."""
    n = 5_000_000_000  # past 2^19 ranges of 8192 the ranges grow
    assert Z.zero_flatten_partials_count(1 << 32) > Z.zero_flatten_partials_count(n)
    assert Z.zero_flatten_partials_count(0) == 0 and Z.zero_flatten_partials_count(1) == 1
    for m in (1, 8191, 8192, 8193, 1 << 25, n, 10**10):
        c = Z.zero_flatten_partials_count(m)
        assert c >= 1 and Z.zero_grad_sqnorm_workspace_bytes(m) >= c * 12
    lib = Z.library()
    assert lib.zero_sqnorm_reduce(None, None, 4, 16, 16, None) == Z.ZERO_ERR_INVALID
    assert lib.zero_flatten_grads_partials(16, 1, 0, 16, 8, None, None, None) == Z.ZERO_ERR_INVALID


def test_header_is_plain_c_and_links(tmp_path):
    """include/zero_shard.h compiles as strict C99 and C11 (-pedantic, warnings as errors), and a C program
    built against it links to the library and calls a host entry point (capacity query of the layout)."""
    import shutil
    import subprocess

    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = tmp_path / "use.c"
    src.write_text('#include "zero_shard.h"\n'
                   "int main(void) {\n"
                   "  zero_layout lay;\n"
                   "  int32_t n = 0;\n"
                   "  int64_t numels[2] = {10, 7};\n"
                   "  int rc = zero_shard_layout(numels, 2, 4, 3, &lay, 0, 0, &n);\n"
                   "  return (rc == ZERO_ERR_CAPACITY && n == 1 && lay.shard_numel == 5) ? 0 : 1;\n"
                   "}\n")
    inc = os.path.join(os.path.dirname(HEADER))
    for std in ("c99", "c11"):
        subprocess.run(["gcc", f"-std={std}", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", "-I", inc,
                        str(src)], check=True)
    exe = str(tmp_path / "use")
    libdir = os.path.dirname(Z.LIB_PATH)
    subprocess.run(["gcc", "-std=c11", "-I", inc, "-o", exe, str(src), "-L", libdir, "-l:libzero_shard.so",
                    f"-Wl,-rpath,{libdir}"], check=True)
    assert subprocess.run([exe]).returncode == 0



def test_host_tensors_are_refused_before_any_call():
    """A tensor in host memory never reaches a kernel: the binding refuses it before calling the library."""
    import torch

    x = torch.zeros(64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        Z.zero_grad_sqnorm(x, Z.ZERO_BF16, 64, 256, 4096, 512, 520)
    with pytest.raises(ValueError, match="GPU tensor"):
        Z.zero_adamw_step_tiled(16, Z.ZERO_BF16, torch.zeros(3 * 1024), 32, 8, lr=1e-3, beta1=0.9, beta2=0.999,
                                eps=1e-8, weight_decay=0.0, grad_scale=1.0, step=1)
    with pytest.raises(ValueError, match="GPU tensor"):
        Z.zero_flatten_plan(Z.zero_shard_layout([8], 1, 0)[1], [x])


def test_counts_beyond_a_buffer_are_refused_before_any_call():
    """An element count larger than a tensor it describes is refused by the binding (the check on sizes comes
    before the one on the device, so host tensors show it)."""
    import torch

    with pytest.raises(ValueError, match="the call touches 128"):
        Z.zero_grad_sqnorm(torch.zeros(8, dtype=torch.bfloat16), Z.ZERO_BF16, 64, 256, 4096, 512, 520)
    with pytest.raises(ValueError, match="the call touches 12288"):
        Z.zero_adamw_step_tiled(16, Z.ZERO_BF16, torch.zeros(3 * 1024 - 1), 32, 8, lr=1e-3, beta1=0.9, beta2=0.999,
                                eps=1e-8, weight_decay=0.0, grad_scale=1.0, step=1)
    _, segs = Z.zero_shard_layout([8, 100], 1, 0)
    with pytest.raises(ValueError, match="the call touches 200"):
        Z.zero_flatten_plan(segs, [0, torch.zeros(99, dtype=torch.bfloat16)])


def test_unusable_loss_scale_is_refused_by_host_decision_and_oracle():
    """A loss scale that is not a positive finite number, or one whose square underflows so that a step
    without overflow has no finite unscaled norm, gives no decision on either side (reading: the pages never
    reach this case).  An overflow at a tiny positive scale is an ordinary skip: the scale halves, to 0 from
    the smallest positive double."""
    for scale, flag in ((0.0, 0), (0.0, 1), (-1.0, 0), (float("inf"), 0), (float("inf"), 1), (float("nan"), 0),
                        (5e-324, 0), (1e-170, 0)):
        with pytest.raises(Z.ZeroError):
            Z.zero_step_decision([2.5], [flag], 1.0, scale, 0, 1000)
        with pytest.raises(oracle.OracleError):
            oracle.step_decision([2.5], [flag], 1.0, scale, 0, 1000)
    for scale in (5e-324, 1e-170):
        got = Z.zero_step_decision([2.5], [1], 1.0, scale, 3, 1000)
        ref = oracle.step_decision([2.5], [1], 1.0, scale, 3, 1000)
        assert got["skip"] == ref["skip"] == 1 and got["loss_scale"] == ref["loss_scale"] == scale * 0.5
        assert got["good_steps"] == ref["good_steps"] == 0
    assert 5e-324 * 0.5 == 0.0
    # the smallest scales that still give a finite unscaled norm are decided normally, the same on both sides
    for scale in (1e-150, 2.0**-537):
        got = Z.zero_step_decision([2.5e-300], [0], 1.0, scale, 0, 1000)
        ref = oracle.step_decision([2.5e-300], [0], 1.0, scale, 0, 1000)
        assert got == ref and got["skip"] == 0 and math.isfinite(got["grad_scale"])
