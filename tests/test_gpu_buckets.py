"""Constant-capacity bucketed pipeline ([Z] section 五（二）, section 四（二）): gradients produced in
backward order on a producer stream, each bucket flattened and square-normed on the compute stream as soon
as its tensors are ready, one decision over the bucket partials, one update.  Checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth.workloads import gpt2_tensors
from tests.parity import assert_bf16_within_ulp, assert_bits_equal, assert_f32_close, assert_grad_scale_close

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixed_precision_adam_amd as Z
    from mixed_precision_adam_amd.driver import AdamWConfig, BucketPipeline, RankShard

DEV = "cuda:0"
SEED = 0x5EED0077


SMALL = [5, 17, 3, 40, 11, 1, 64]  # Ψ = 141: ragged everywhere


@pytest.mark.parametrize("model,world,rank,bucket", [("gpt2", 2, 0, 65536), ("gpt2", 2, 1, 65536),
                                                     ("gpt2", 3, 2, 1024), ("gpt2", 1, 0, 1 << 24),
                                                     ("gpt2", 2, 1, 100_000), ("small", 2, 1, 8),
                                                     ("small", 3, 0, 16), ("big", 1, 0, 1 << 25)])
def test_bucket_pipeline_against_oracle(model, world, rank, bucket):
    numels = {"gpt2": gpt2_tensors(d=128, layers=3, vocab=1000, ctx=64, ffn=512)[1], "small": SMALL,
              # 40M elements in two 2^25-element buckets, the capacity the benchmark uses
              "big": [24_000_001, 16_000_000]}[model]
    psi = sum(numels)
    starts = np.cumsum([0] + numels)
    srcs = [torch.empty(n, dtype=torch.bfloat16, device=DEV) for n in numels]
    sh = RankShard(numels, world, rank, Z.ZERO_BF16, DEV, sources=srcs, tiled=True, fused=True)
    lay = sh.layout
    s = sh.n
    master = synth.fill_host(synth.field(SEED, synth.STREAM_MASTER, 0, 0.02, synth.F32), lay.shard_offset,
                             lay.shard_valid)
    p0 = np.zeros(s, np.float32)
    p0[:lay.shard_valid] = master
    sh.load_master(torch.from_numpy(p0).to(DEV))
    cfg = AdamWConfig(lr=2e-3, beta1=0.9, beta2=0.99, eps=1e-8, weight_decay=0.05, max_norm=0.3)
    pipe = BucketPipeline(sh, srcs, bucket, cfg)
    assert len(pipe.windows) == max(1, -(-s // bucket))
    producer = torch.cuda.Stream()
    ref = [p0.copy(), np.zeros(s, np.float32), np.zeros(s, np.float32), np.zeros(s, np.uint16)]
    for t in range(1, 4):
        field = synth.field(SEED, synth.STREAM_GRAD, t, 1e-3, synth.BF16)

        def produce(idx, stream):
            for k in idx:
                synth.fill_device(field, int(starts[k]), numels[k], srcs[k].data_ptr(), stream.cuda_stream)

        pipe.step(produce=produce, producer=producer)
        got = pipe.read()
        flat = synth.fill_host(field, 0, psi)
        g = oracle.flatten([flat], [psi], world, rank)
        assert_bits_equal(sh.grad.view(torch.int16).cpu().numpy().view(np.uint16), g, f"step {t} shard")
        sq, fl = oracle.sqnorm(g, oracle.BF16)
        od = oracle.step_decision([sq], [fl], cfg.max_norm, 1.0, 0, 2**31 - 1)
        assert got["skip"] == 0 and got["adam_step"] == t
        same = assert_grad_scale_close(got["grad_scale"], od["grad_scale"], s, f"step {t}")
        oracle.adamw_step(g, oracle.BF16, *ref, lr=cfg.lr, beta1=cfg.beta1, beta2=cfg.beta2, eps=cfg.eps,
                          weight_decay=cfg.weight_decay, grad_scale=od["grad_scale"], step=t)
        gp, gm, gv = (x.cpu().numpy() for x in sh.read_state())
        nd = assert_f32_close(gp, ref[0], "master") + assert_f32_close(gm, ref[1], "m") + \
            assert_f32_close(gv, ref[2], "v")
        nd += assert_bf16_within_ulp(sh.param.view(torch.int16).cpu().numpy().view(np.uint16), ref[3], "param")
        assert nd == 0 or not same, (t, nd)



def test_sqnorm_reduce_exact_on_integers_and_flags():
    """Integer partials whose total stays below 2^53 (at most 397,213 values below 2^33) sum exactly in any
    order: the fold must return the exact total, with one level and with two (past 65,536 partials, where
    the partials are overwritten); any set flag must give nonfinite = 1; zero partials give (0, 0)."""
    rng = np.random.default_rng(5)
    out = torch.zeros(2, dtype=torch.float64, device=DEV)
    sq, fl = out.data_ptr(), out.data_ptr() + 8
    for count in (0, 1, 255, 256, 257, 5000, 65_536, 65_537, 100_000, 4096 * 40, 397_213):
        vals = rng.integers(0, 2**33, max(count, 1)).astype(np.float64)[:count]
        assert sum(int(v) for v in vals) < 2**53
        ps = torch.from_numpy(np.append(vals, 0.0)).to(DEV)
        flags = np.zeros(count + 1, np.int32)
        pf = torch.from_numpy(flags).to(DEV)
        Z.zero_sqnorm_reduce(ps, pf, count, sq, fl)
        got = out.cpu().numpy()
        assert got[0] == float(sum(int(v) for v in vals)), count
        assert got[1:].view(np.int32)[0] == 0
        if count:
            for at in (count // 2, count - 1, 0):
                flags[:] = 0
                flags[at] = 7
                Z.zero_sqnorm_reduce(ps, torch.from_numpy(flags).to(DEV), count, sq, fl)
                assert out.cpu().numpy()[1:].view(np.int32)[0] == 1, (count, at)


def test_bucket_pipeline_fp16_overflow_skips_and_halves():
    """fp16 gradients under a dynamic loss scale, in buckets: a +inf in one bucket sets that bucket's partial
    flag, the fold carries it to the decision, the step is skipped (state untouched, Adam t unchanged) and the
    scale halves; the next step proceeds."""
    numels = gpt2_tensors(d=128, layers=2, vocab=1000, ctx=64, ffn=512)[1]
    starts = np.cumsum([0] + numels)
    srcs = [torch.empty(n, dtype=torch.float16, device=DEV) for n in numels]
    sh = RankShard(numels, 2, 1, Z.ZERO_FP16, DEV, sources=srcs, tiled=True, fused=True)
    lay = sh.layout
    p0 = torch.zeros(sh.n, device=DEV)
    synth.fill_tensor(synth.field(SEED, synth.STREAM_MASTER, 0, 0.02, synth.F32), lay.shard_offset,
                      p0[:lay.shard_valid])
    sh.load_master(p0)
    cfg = AdamWConfig(lr=1e-3, max_norm=1.0)
    pipe = BucketPipeline(sh, srcs, 8192, cfg, loss_scale=1024.0, growth_interval=1000)
    assert len(pipe.windows) > 3

    def fill(t, scale, inf_at=None):
        f = synth.field(SEED, synth.STREAM_GRAD, t, 1e-3, synth.FP16, scale=scale)
        for k, src in enumerate(srcs):
            synth.fill_tensor(f, int(starts[k]), src)
        if inf_at is not None:  # a shard element in the middle of one bucket
            sg = next(x for x in sh.segments if x.dst_offset <= inf_at < x.dst_offset + x.numel)
            srcs[sg.tensor].view(torch.int16)[sg.src_offset + inf_at - sg.dst_offset] = 0x7C00

    fill(1, 1024.0)
    pipe.step()
    s1 = pipe.read()
    assert s1["skip"] == 0 and s1["adam_step"] == 1 and s1["loss_scale"] == 1024.0
    before = sh.state.clone(), sh.param.clone()
    fill(2, 1024.0, inf_at=2 * 8192 + 77)
    pipe.step()
    s2 = pipe.read()
    assert s2["skip"] == 1 and s2["adam_step"] == 1 and s2["loss_scale"] == 512.0 and s2["iteration"] == 2
    assert torch.equal(sh.state.view(torch.int32), before[0].view(torch.int32))
    assert torch.equal(sh.param.view(torch.int16), before[1].view(torch.int16))
    fill(3, 512.0)
    pipe.step()
    s3 = pipe.read()
    assert s3["skip"] == 0 and s3["adam_step"] == 2 and s3["loss_scale"] == 512.0
