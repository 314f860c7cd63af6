"""GPU parity at the full configuration sizes, in the launch configuration the
benchmark times (tiled optimizer state, flatten fused with the square-norm).

Per step, against the oracle on the same seeded inputs:
  * the flattened gradient shard on sampled tile-aligned windows (bit-exact);
  * the rank's fp64 square-norm over the whole shard (the oracle sums every
    element sequentially) and the non-finite flag;
  * the decision: skip and dynamic loss scale exactly, the clip/unscale
    factor within the bound two fp64 summation orders allow;
  * master / m / v / bf16 param on the sampled windows, which the oracle
    carries through every step (elements are independent given the factor).
Several square-norms are correct (any summation order), so the factor is not
unique; the update given a factor is.  Both sides therefore apply the
oracle's factor, and the state must then match bit for bit.
Windows: the first and last 64Ki elements, one around every tensor boundary
inside the shard, and 16 hashed positions.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth.workloads import WORKLOADS
from tests.parity import (assert_bf16_within_ulp, assert_bits_equal, assert_f32_close, assert_grad_scale_close,
                          assert_norm_close)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

if torch.cuda.is_available():
    import mixed_precision_adam_amd as Z
    from mixed_precision_adam_amd.driver import AdamWConfig, RankShard, ScalerState, rank_norms, rank_update

WIN = 65536        # windows at both ends, around every segment boundary and around update-launch seams
HASHED = 32        # plus this many chunks of HWIN elements at hashed positions
HWIN = 1 << 20
TILE = 1024  # ZERO_STATE_TILE: windows start on tile boundaries


def windows(layout, segments):
    """Sorted, disjoint [a, b) windows of the shard (merged where they touch), each starting on a tile."""
    s = layout.shard_numel
    spans = [(0, WIN), (max(0, (s - WIN) // TILE * TILE), WIN)]
    for sg in segments[1:]:
        spans.append((max(0, (sg.dst_offset - WIN // 2) // TILE * TILE), WIN))
    launch = 1 << 25  # the update is issued in launches of this many elements: sample their seams
    for k in range(1, min(4, s // launch) + 1):
        spans.append((max(0, (k * launch - WIN // 2) // TILE * TILE), WIN))
    for k in range(HASHED):
        h = (k * 0x9E3779B97F4A7C15 + 0x632BE59BD9B4E019) % (1 << 64)
        spans.append(((h % max(1, s // TILE)) * TILE, HWIN))
    out = []
    for a, n in sorted(spans):
        b = min(s, a + n)
        if out and a <= out[-1][1]:
            out[-1] = (out[-1][0], max(out[-1][1], b))
        else:
            out.append((a, b))
    return out


def bits16(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host_shard_grads(w, field, lay, inject_at=None):
    """The rank's gradient shard on the host: flat elements offset .. offset+valid, then zero padding."""
    g = np.zeros(lay.shard_numel, dtype=np.uint16)
    synth.fill_host(field, lay.shard_offset, lay.shard_valid, out=g[:lay.shard_valid])
    if inject_at is not None:
        j, bits = inject_at
        g[j] = bits
    return g


def host_shard_grads_window(w, field, lay, a, b, inject_at=None):
    """Shard elements [a, b) of host_shard_grads, generated for the window alone."""
    g = np.zeros(b - a, dtype=np.uint16)
    va = min(b, lay.shard_valid)
    if va > a:
        synth.fill_host(field, lay.shard_offset + a, va - a, out=g[:va - a])
    if inject_at is not None and a <= inject_at[0] < b:
        g[inject_at[0] - a] = inject_at[1]
    return g


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["gpt2-1.5b", "llama-7b", "llama-13b", "1t-zero3"])
def test_config_parity(name):
    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    rank = w.ranks[0]
    gdt = Z.ZERO_BF16 if w.grad_kind == synth.BF16 else Z.ZERO_FP16
    tdt = torch.bfloat16 if gdt == Z.ZERO_BF16 else torch.float16
    lay, segs = Z.zero_shard_layout(w.numels, w.world, rank)
    olay = oracle.layout(w.numels, w.world, rank)
    assert (lay.shard_numel, lay.shard_offset, lay.shard_valid, lay.bytes_zero3) == (
        olay.shard_numel, olay.shard_offset, olay.shard_valid, olay.bytes_zero3)
    if name == "1t-zero3":
        assert lay.bytes_zero3 == 15_625_000_000  # 16·S bytes for S = 976,562,500
    starts = np.cumsum([0] + list(w.numels))

    sources = None
    if not w.flat_shard_only:
        sources = [None] * len(w.numels)
        for sg in segs:
            sources[sg.tensor] = torch.empty(w.numels[sg.tensor], dtype=tdt, device=dev)
    sh = RankShard(w.numels, w.world, rank, gdt, dev, sources=sources, tiled=True, fused=not w.flat_shard_only)
    S = sh.n
    master0 = torch.zeros(S, dtype=torch.float32, device=dev)
    synth.fill_tensor(w.master_field(), lay.shard_offset, master0[:lay.shard_valid])
    sh.load_master(master0)
    del master0
    torch.cuda.synchronize()

    wins = windows(lay, segs)
    ref = []
    for a, b in wins:
        p = np.zeros(b - a, np.float32)
        va = min(b, lay.shard_valid)
        if va > a:
            synth.fill_host(w.master_field(), lay.shard_offset + a, va - a, out=p[:va - a])
        ref.append([p, np.zeros(b - a, np.float32), np.zeros(b - a, np.float32), np.zeros(b - a, np.uint16)])

    cfg = AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, max_norm=w.clip)
    growth = 1000 if gdt == Z.ZERO_FP16 else 2**31 - 1
    scaler = ScalerState(scale=w.loss_scale, growth_interval=growth)
    oscale, ogood, ostep = w.loss_scale, 0, 0
    skips = 0
    for t in range(1, w.steps + 1):
        print(f"[{name}] step {t}", flush=True)
        field = w.grad_field(t, scaler.scale)
        if w.flat_shard_only:
            sh.grad[lay.shard_valid:].zero_()
            synth.fill_tensor(field, lay.shard_offset, sh.grad[:lay.shard_valid])
        else:
            for sg in segs:
                synth.fill_tensor(field, int(starts[sg.tensor]), sources[sg.tensor])
        inject_at = None
        if t in w.inject:
            val, frac = w.inject[t]
            j = int(frac * lay.shard_valid)
            bits = np.array([val], dtype=np.float16 if gdt == Z.ZERO_FP16 else np.float32)
            hb = int(bits.view(np.uint16)[0]) if gdt == Z.ZERO_FP16 else int(bits.view(np.uint32)[0] >> 16)
            inject_at = (j, hb)
            sg = next(x for x in segs if x.dst_offset <= j < x.dst_offset + x.numel)
            signed = hb - (1 << 16 if hb >= 1 << 15 else 0)  # the same 16 bits as a signed int16
            sources[sg.tensor].view(torch.int16)[sg.src_offset + j - sg.dst_offset] = signed
        if w.lr_min is not None:
            cfg.lr = Z.zero_cosine_lr(t, w.steps, w.lr, w.lr_min)
            olr = oracle.cosine_lr(t, w.steps, w.lr, w.lr_min)
            assert cfg.lr == olr
        else:
            olr = w.lr
        dec = rank_norms([sh], cfg, scaler, flatten=not w.flat_shard_only)

        # oracle: whole-shard square-norm and decision
        g_host = host_shard_grads(w, field, lay, inject_at)
        for a, b in wins:
            assert_bits_equal(bits16(sh.grad[a:b]), g_host[a:b], f"{name} step {t} shard [{a},{b})")
        osq, oflag = oracle.sqnorm(g_host, gdt)
        assert dec["rank_flags"][0] == oflag, (name, t)
        if not oflag:
            assert_norm_close(dec["rank_sqnorms"][0], osq, S, f"{name} step {t} sqnorm")
        od = oracle.step_decision([osq], [oflag], w.clip, oscale, ogood, growth)
        assert dec["skip"] == od["skip"] and dec["loss_scale"] == od["loss_scale"], (dec, od)
        oscale, ogood = od["loss_scale"], od["good_steps"]
        if od["skip"]:
            skips += 1
        else:
            assert_grad_scale_close(dec["grad_scale"], od["grad_scale"], S, f"{name} step {t}")
            ostep += 1
            for (a, b), R in zip(wins, ref):
                oracle.adamw_step(g_host[a:b].copy(), gdt, R[0], R[1], R[2], R[3], lr=olr, beta1=w.beta1,
                                  beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                                  grad_scale=od["grad_scale"], step=ostep)
        rank_update([sh], cfg, scaler, dict(dec, grad_scale=od["grad_scale"]))
        torch.cuda.synchronize()
        assert scaler.adam_step == ostep
        nd = 0
        for (a, b), R in zip(wins, ref):
            gp, gm, gv = (x.cpu().numpy() for x in sh.state_views(a, b))
            what = f"{name} step {t} [{a},{b})"
            nd += assert_f32_close(gp, R[0], what + " master")
            nd += assert_f32_close(gm, R[1], what + " m")
            nd += assert_f32_close(gv, R[2], what + " v")
            if ostep > 0:
                nd += assert_bf16_within_ulp(bits16(sh.param[a:b]), R[3], what + " param")
        assert nd == 0, f"{name} step {t}: {nd} sampled elements differ in bits (within tolerance)"
    expect_skips = len(w.inject)
    assert skips == expect_skips
    if name == "llama-13b":
        assert scaler.scale == 16384.0 and scaler.adam_step == 4


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,bucket", [("gpt2-1.5b", 0), ("gpt2-1.5b", 1 << 25), ("llama-7b", 0), ("llama-13b", 0),
                                         ("1t-zero3", 0)])
def test_benchmark_path_parity(name, bucket):
    """A rank shard exactly as `bench.py` steps it: fused flatten + norm (in one pass, or in constant-capacity
    buckets of 2^25 elements, last first), the decision on the device, the tiled update in launches of 2^25
    elements.  GPT-2 1.5B (bf16), Llama-7B (bf16 with 0.1% outliers: clipping active), Llama-13B (the
    benchmark's default: fp16 gradients stored multiplied by a dynamic loss scale that starts at 65536, +inf
    injected at step 2 and -inf at step 5, so the device skips those steps and halves the scale: 65536 ->
    32768 -> 16384 over 4 Adam steps) and the 1T ZeRO-3 shard (fp16 gradients in the shard, the norm as its
    own pass, cosine learning rate over 10 steps).  The GPU takes its
    own decision; the oracle takes its own.  Skip, loss scale, good steps and Adam t must agree exactly and
    the factor within the bound of two fp64 summation orders (several factors are correct).  The update given
    a factor is unique, so the oracle then applies the device's factor and the sampled states must agree bit
    for bit; a skipped step must leave every sampled byte as it was."""
    from mixed_precision_adam_amd.driver import BucketPipeline, DeviceDecision

    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    rank = w.ranks[0]
    gdt = Z.ZERO_BF16 if w.grad_kind == synth.BF16 else Z.ZERO_FP16
    tdt = torch.bfloat16 if gdt == Z.ZERO_BF16 else torch.float16
    growth = 1000 if gdt == Z.ZERO_FP16 else 2**31 - 1
    lay, segs = Z.zero_shard_layout(w.numels, w.world, rank)
    starts = np.cumsum([0] + list(w.numels))
    flat = w.flat_shard_only  # gradients generated in the shard: no flatten, the norm as its own pass
    sources = None
    if not flat:
        sources = [None] * len(w.numels)
        for sg in segs:
            sources[sg.tensor] = torch.empty(w.numels[sg.tensor], dtype=tdt, device=dev)
    sh = RankShard(w.numels, w.world, rank, gdt, dev, sources=sources, tiled=True, fused=not flat)
    S = sh.n
    master0 = torch.zeros(S, dtype=torch.float32, device=dev)
    synth.fill_tensor(w.master_field(), lay.shard_offset, master0[:lay.shard_valid])
    sh.load_master(master0)
    del master0
    cfg = AdamWConfig(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, max_norm=w.clip)
    if bucket:
        runner = BucketPipeline(sh, sources, bucket, cfg, loss_scale=w.loss_scale, growth_interval=growth)
        assert len(runner.windows) == -(-S // bucket)
    else:
        runner = DeviceDecision([sh], cfg, loss_scale=w.loss_scale, growth_interval=growth)
    wins = windows(lay, segs)
    if bucket:  # the seams between buckets too
        wins = sorted(set(wins) | {(max(0, k * bucket - WIN // 2), min(S, k * bucket + WIN // 2))
                                   for k in range(1, -(-S // bucket))})
    ref = []
    for a, b in wins:
        p = np.zeros(b - a, np.float32)
        va = min(b, lay.shard_valid)
        if va > a:
            synth.fill_host(w.master_field(), lay.shard_offset + a, va - a, out=p[:va - a])
        ref.append([p, np.zeros(b - a, np.float32), np.zeros(b - a, np.float32), np.zeros(b - a, np.uint16)])
    torch.cuda.synchronize()
    oscale, ogood, ostep, skips = w.loss_scale, 0, 0, 0
    for t in range(1, w.steps + 1):
        print(f"[{name} bucket={bucket}] step {t}", flush=True)
        field = w.grad_field(t, oscale)  # gradients stored multiplied by the scale in force
        if flat:
            sh.grad[lay.shard_valid:].zero_()
            synth.fill_tensor(field, lay.shard_offset, sh.grad[:lay.shard_valid])
        else:
            for sg in segs:
                synth.fill_tensor(field, int(starts[sg.tensor]), sources[sg.tensor])
        olr = w.lr
        if w.lr_min is not None:  # the workload's cosine schedule
            cfg.lr = Z.zero_cosine_lr(t, w.steps, w.lr, w.lr_min)
            olr = oracle.cosine_lr(t, w.steps, w.lr, w.lr_min)
            assert cfg.lr == olr
        inject_at = None
        if t in w.inject:
            val, frac = w.inject[t]
            j = int(frac * lay.shard_valid)
            bits = np.array([val], dtype=np.float16 if gdt == Z.ZERO_FP16 else np.float32)
            hb = int(bits.view(np.uint16)[0]) if gdt == Z.ZERO_FP16 else int(bits.view(np.uint32)[0] >> 16)
            inject_at = (j, hb)
            sg = next(x for x in segs if x.dst_offset <= j < x.dst_offset + x.numel)
            sources[sg.tensor].view(torch.int16)[sg.src_offset + j - sg.dst_offset] = hb - (1 << 16 if hb >= 1 << 15
                                                                                              else 0)
        if bucket:
            runner.step()
        else:
            runner.step(flatten=not flat)
        st = runner.read()
        g_host = host_shard_grads(w, field, lay, inject_at)
        for a, b in wins:
            assert_bits_equal(bits16(sh.grad[a:b]), g_host[a:b], f"{name} bucket={bucket} step {t} shard [{a},{b})")
        osq, oflag = oracle.sqnorm(g_host, gdt)
        del g_host
        od = oracle.step_decision([osq], [oflag], w.clip, oscale, ogood, growth)
        oscale, ogood = od["loss_scale"], od["good_steps"]
        what = f"{name} bucket={bucket} step {t}"
        assert st["skip"] == od["skip"] and st["loss_scale"] == od["loss_scale"], (what, st, od)
        assert st["good_steps"] == od["good_steps"] and st["error"] == 0 and st["iteration"] == t, (what, st)
        if od["skip"]:
            skips += 1
        else:
            ostep += 1
            assert_norm_close(st["global_norm"] ** 2, od["global_norm"] ** 2, S, what + " norm")
            # the device's factor is one of the correct ones (fp64 summation order) ...
            assert_grad_scale_close(st["grad_scale"], od["grad_scale"], S, what)
        assert st["adam_step"] == ostep, (what, st)
        nd = 0
        for (a, b), R in zip(wins, ref):
            if not od["skip"]:  # ... and the update given that factor is unique: the oracle applies it too
                g_win = host_shard_grads_window(w, field, lay, a, b, inject_at)
                oracle.adamw_step(g_win, gdt, R[0], R[1], R[2], R[3], lr=olr, beta1=w.beta1, beta2=w.beta2,
                                  eps=w.eps, weight_decay=w.weight_decay, grad_scale=st["grad_scale"], step=ostep)
            gp, gm, gv = (x.cpu().numpy() for x in sh.state_views(a, b))
            ww = f"{what} [{a},{b})"
            nd += assert_f32_close(gp, R[0], ww + " master") + assert_f32_close(gm, R[1], ww + " m")
            nd += assert_f32_close(gv, R[2], ww + " v")
            if ostep > 0:
                nd += assert_bf16_within_ulp(bits16(sh.param[a:b]), R[3], ww + " param")
        assert nd == 0, f"{what}: {nd} sampled elements differ in bits from the oracle given the same factor"
    assert skips == len(w.inject)
    if name == "llama-13b":
        assert oscale == 16384.0 and ostep == 4
