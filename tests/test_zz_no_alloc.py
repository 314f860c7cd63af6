"""The allocation-free fused flatten + norm (zero_flatten_grads_sqnorm_noalloc) against the entry point it
varies (zero_flatten_grads_sqnorm with a caller workspace), called through the C ABI.

Both run the same kernels over the same partial count, so the shard, the square-norm and the flag must be
identical bit for bit.  Calls follow one another on one device and share its static scratch: a large shard
first (more than 65,536 partials, so the fold takes two levels and overwrites the partials in place), then a
smaller one whose stale partials from the first call must not leak into its sum, then a third that clears
the non-finite flag the second one raised.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import assert_norm_close

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import mixed_precision_adam_amd as Z

DEV = "cuda:0"


def _run_both(numels, world, rank, dtype, seed, inject=None, oracle_check=False):
    tdt = torch.bfloat16 if dtype == Z.ZERO_BF16 else torch.float16
    lay, segs = Z.zero_shard_layout(numels, world, rank)
    print(f"[no-alloc] numels={numels} world={world} rank={rank} dtype={dtype} shard={lay.shard_numel}", flush=True)
    field = synth.field(seed, synth.STREAM_GRAD, 1, 1e-3, synth.BF16 if dtype == Z.ZERO_BF16 else synth.FP16)
    starts = np.cumsum([0] + list(numels))
    srcs = [None] * len(numels)
    for sg in segs:
        t = sg.tensor
        if srcs[t] is None:
            srcs[t] = torch.empty(numels[t], dtype=tdt, device=DEV)
            synth.fill_tensor(field, int(starts[t]), srcs[t])
    if inject is not None:
        t, i, bits = inject
        srcs[t].view(torch.int16)[i] = bits
    table = torch.frombuffer(bytearray(Z.zero_flatten_plan(segs, [s if s is not None else 0 for s in srcs])),
                             dtype=torch.uint8).to(DEV)
    n = lay.shard_numel
    ws_bytes = Z.zero_grad_sqnorm_workspace_bytes(n)
    assert ws_bytes <= Z.ZERO_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    shard_a = torch.full((n,), -1, dtype=torch.int16, device=DEV)
    shard_b = torch.full((n,), -2, dtype=torch.int16, device=DEV)
    out_a = torch.full((2,), -7.0, dtype=torch.float64, device=DEV)  # square-norm, then the flag's 4 bytes
    out_b = torch.full((2,), -9.0, dtype=torch.float64, device=DEV)
    Z.zero_flatten_grads_sqnorm(table, len(segs), dtype, shard_a, n, ws, ws_bytes, out_a.data_ptr(),
                                out_a.data_ptr() + 8)
    Z.zero_flatten_grads_sqnorm_noalloc(table, len(segs), dtype, shard_b, n, out_b.data_ptr(), out_b.data_ptr() + 8)
    torch.cuda.synchronize()
    assert torch.equal(shard_a, shard_b), "shards differ"
    ha, hb = out_a.cpu().numpy(), out_b.cpu().numpy()
    flag_a, flag_b = int(ha[1:].view(np.int32)[0]), int(hb[1:].view(np.int32)[0])
    assert flag_a == flag_b, (flag_a, flag_b)
    if not flag_a:
        assert ha[:1].view(np.uint64)[0] == hb[:1].view(np.uint64)[0], (ha[0], hb[0])
    if oracle_check:
        g = shard_b.cpu().numpy().view(np.uint16)
        host_src = [synth.fill_host(field, int(starts[t]), numels[t]) for t in range(len(numels))]
        if inject is not None:
            host_src[inject[0]][inject[1]] = np.int16(inject[2]).view(np.uint16)
        want = oracle.flatten(host_src, numels, world, rank)
        assert np.array_equal(g, want)
        osq, oflag = oracle.sqnorm(want, dtype)
        assert oflag == flag_b
        if not oflag:
            assert_norm_close(float(hb[0]), osq, len(want), "no-alloc square-norm")
    return lay.shard_numel, flag_b


def test_noalloc_matches_workspace_entry_point_on_calls_in_a_row():
    # 1: a large ragged shard with a phase-shifting 5-element tensor before a large one: 67,139 partials
    n1, f1 = _run_both([600_000_003, 5, 500_000_000, 77], 2, 1, Z.ZERO_BF16, 0x5EED0101)
    assert n1 == 550_000_043 and Z.zero_flatten_partials_count(n1) > 65536 and f1 == 0
    # 2: much smaller, fp16, with an infinity: the flag must be raised whatever the scratch held
    n2, f2 = _run_both([1000, 3, 20_000, 9_999], 3, 2, Z.ZERO_FP16, 0x5EED0102, inject=(3, 17, 0x7C00),
                       oracle_check=True)
    assert n2 < n1 and f2 == 1
    # 3: smaller again and clean: the flag clears, the sum matches the oracle
    n3, f3 = _run_both([4096, 1], 1, 0, Z.ZERO_FP16, 0x5EED0103, oracle_check=True)
    assert n3 < n2 and f3 == 0


def test_noalloc_rejects_bad_arguments_without_launching():
    lib = Z.library()
    assert lib.zero_flatten_grads_sqnorm_noalloc(16, 1, 0, 16, 8, None, 16, None) == Z.ZERO_ERR_INVALID
    assert lib.zero_flatten_grads_sqnorm_noalloc(16, 1, 0, 16, 8, 12, 16, None) == Z.ZERO_ERR_INVALID  # misaligned
    assert lib.zero_flatten_grads_sqnorm_noalloc(16, 1, 5, 16, 8, 16, 24, None) == Z.ZERO_ERR_INVALID  # dtype
    assert lib.zero_flatten_grads_sqnorm_noalloc(None, 1, 0, 16, 8, 16, 24, None) == Z.ZERO_ERR_INVALID


def test_noalloc_captured_in_a_graph_matches_eager_calls():
    """The use it exists for: a HIP graph that captures the allocation-free call (nothing is allocated during
    capture) and is replayed after fresh gradients are written eagerly, with the host synchronising in
    between.  Every replay must equal the workspace entry point run eagerly on the same gradients, bit for
    bit; the first call on the device happens eagerly, before capture."""
    numels, world, rank = [70_001, 3, 1_000_000, 4096], 2, 1
    lay, segs = Z.zero_shard_layout(numels, world, rank)
    starts = np.cumsum([0] + numels)
    srcs = [torch.empty(k, dtype=torch.bfloat16, device=DEV) for k in numels]
    table = torch.frombuffer(bytearray(Z.zero_flatten_plan(segs, srcs)), dtype=torch.uint8).to(DEV)
    n = lay.shard_numel
    ws_bytes = Z.zero_grad_sqnorm_workspace_bytes(n)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    shard_g = torch.zeros(n, dtype=torch.int16, device=DEV)
    out_g = torch.zeros(2, dtype=torch.float64, device=DEV)
    shard_e = torch.zeros(n, dtype=torch.int16, device=DEV)
    out_e = torch.zeros(2, dtype=torch.float64, device=DEV)

    def fill(t):
        f = synth.field(0x5EED0104, synth.STREAM_GRAD, t, 1e-3, synth.BF16)
        for k, src in enumerate(srcs):
            synth.fill_tensor(f, int(starts[k]), src)

    fill(0)
    Z.zero_flatten_grads_sqnorm_noalloc(table, len(segs), Z.ZERO_BF16, shard_g, n, out_g.data_ptr(),
                                        out_g.data_ptr() + 8)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        Z.zero_flatten_grads_sqnorm_noalloc(table, len(segs), Z.ZERO_BF16, shard_g, n, out_g.data_ptr(),
                                            out_g.data_ptr() + 8)
    for t in range(1, 5):
        fill(t)
        if t == 3:
            srcs[2].view(torch.int16)[900_000] = 0x7F80  # +inf inside rank 1's shard, this replay only
        torch.cuda.synchronize()
        Z.zero_flatten_grads_sqnorm(table, len(segs), Z.ZERO_BF16, shard_e, n, ws, ws_bytes, out_e.data_ptr(),
                                    out_e.data_ptr() + 8)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(shard_g, shard_e), t
        he, hg = out_e.cpu().numpy(), out_g.cpu().numpy()
        assert hg[1:].view(np.int32)[0] == he[1:].view(np.int32)[0] == (1 if t == 3 else 0), t
        if t != 3:
            assert hg[:1].view(np.uint64)[0] == he[:1].view(np.uint64)[0], (t, hg[0], he[0])
