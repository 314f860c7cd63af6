"""The input generator's device fills against its host fill, bit for bit: both sides of every parity test
start from these values, so they must be the same bits whichever side made them."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TORCH = {synth.F32: torch.float32, synth.BF16: torch.int16, synth.FP16: torch.int16}


def _bits(t):
    return t.cpu().numpy().view(np.uint32 if t.dtype == torch.float32 else np.uint16)


@pytest.mark.parametrize("kind", [synth.F32, synth.BF16, synth.FP16])
@pytest.mark.parametrize("idx0", [0, 7, 123_456_789_013])
def test_device_fill_equals_host_fill(kind, idx0):
    f = synth.field(0x5EED0099, synth.STREAM_GRAD, 3, 1e-3, kind, scale=1024.0 if kind == synth.FP16 else 1.0,
                    outlier_per_million=1000, outlier_sigma=1.0)
    n = 1_000_003
    t = torch.empty(n, dtype=TORCH[kind], device=DEV)
    synth.fill_device(f, idx0, n, t.data_ptr(), torch.cuda.current_stream().cuda_stream)
    host = synth.fill_host(f, idx0, n)
    assert (_bits(t) == host.view(_bits(t).dtype)).all()


def test_multi_buffer_fill_equals_host_fill():
    f = synth.field(0x5EED0098, synth.STREAM_GRAD, 1, 1e-3, synth.BF16)
    sizes = [0, 1, 255, 256, 257, 1_000_000, 4097, 3]
    bufs = [torch.full((max(n, 1) + 16,), 0x5A5A, dtype=torch.int16, device=DEV) for n in sizes]
    starts = np.cumsum([0] + sizes)
    pieces = [(b.data_ptr() + 16, int(starts[k]) * 5 + 11, n) for k, (b, n) in enumerate(zip(bufs, sizes))]
    table = torch.frombuffer(bytearray(synth.piece_table(pieces)), dtype=torch.uint8).to(DEV)
    synth.fill_device_many(f, table.data_ptr(), len(pieces), max(sizes), torch.cuda.current_stream().cuda_stream)
    for (ptr, i0, n), b in zip(pieces, bufs):
        raw = b.cpu().numpy().view(np.uint16)
        assert (raw[:8] == 0x5A5A).all() and (raw[8 + n:] == 0x5A5A).all()  # nothing outside the piece
        assert (raw[8:8 + n] == synth.fill_host(f, i0, n)).all(), n
