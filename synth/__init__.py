"""Seeded synthetic inputs shared by the tests and the benchmark.

Holds none of the method's arithmetic: it only makes numbers.  A value depends
on (seed, stream, step, global flat element index), so any slice can be
regenerated on the host for the oracle while the device fill writes the same
bits straight into HBM for the library (see ``synth_core.h``).

Workload recipes (model tensor lists, per-config distributions) are in
``synth.workloads``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")

F32, BF16, FP16 = 0, 1, 2

# Streams of the generator (one per kind of input).
STREAM_GRAD = 1
STREAM_MASTER = 2


class Field(C.Structure):
    _fields_ = [
        ("seed", C.c_uint64),
        ("stream", C.c_uint32),
        ("step", C.c_uint32),
        ("sigma", C.c_double),
        ("scale", C.c_double),
        ("outlier_per_million", C.c_uint32),
        ("kind", C.c_uint32),
        ("outlier_sigma", C.c_double),
    ]


def field(seed: int, stream: int, step: int, sigma: float, kind: int, scale: float = 1.0,
          outlier_per_million: int = 0, outlier_sigma: float = 0.0) -> Field:
    return Field(seed, stream, step, sigma, scale, outlier_per_million, kind, outlier_sigma)


def build() -> None:
    subprocess.run(["sh", os.path.join(_HERE, "build.sh")], check=True)


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        import torch  # noqa: F401  (PyTorch's HIP runtime first: the fills run on its streams)

        lib = C.CDLL(_LIB_PATH)
        lib.syn_fill_host.argtypes = [C.POINTER(Field), C.c_int64, C.c_int64, C.c_void_p, C.c_int32]
        lib.syn_fill_device.argtypes = [C.POINTER(Field), C.c_int64, C.c_int64, C.c_void_p, C.c_void_p]
        lib.syn_fill_device_many.argtypes = [C.POINTER(Field), C.c_void_p, C.c_int32, C.c_int64, C.c_void_p]
        _lib = lib
    return _lib


_NP = {F32: np.float32, BF16: np.uint16, FP16: np.uint16}


def host_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def fill_host(f: Field, idx0: int, n: int, out: np.ndarray | None = None, threads: int = 0) -> np.ndarray:
    """Elements idx0 .. idx0+n-1 of the field as a host array (float32 or 16-bit patterns)."""
    if out is None:
        out = np.empty(n, dtype=_NP[f.kind])
    assert out.size == n and out.dtype == _NP[f.kind] and out.flags["C_CONTIGUOUS"]
    rc = _load().syn_fill_host(C.byref(f), idx0, n, out.ctypes.data if n else None, threads or host_threads())
    if rc != 0:
        raise RuntimeError(f"syn_fill_host failed ({rc})")
    return out


def fill_device(f: Field, idx0: int, n: int, ptr: int, stream: int) -> None:
    """Same elements written to device memory at `ptr` on HIP stream `stream`."""
    rc = _load().syn_fill_device(C.byref(f), idx0, n, ptr, stream)
    if rc != 0:
        raise RuntimeError(f"syn_fill_device failed ({rc})")


class Piece(C.Structure):
    _fields_ = [("out", C.c_void_p), ("idx0", C.c_int64), ("n", C.c_int64)]


def piece_table(pieces) -> bytes:
    """Packs (device address, first flat index, element count) triples for fill_device_many; the caller
    copies the bytes to device memory once and reuses them."""
    arr = (Piece * max(len(pieces), 1))(*[Piece(p, i, n) for p, i, n in pieces])
    return bytes(arr)[:len(pieces) * C.sizeof(Piece)]


def fill_device_many(f: Field, table_dev: int, n_pieces: int, max_n: int, stream: int) -> None:
    """Every piece of a device-resident piece table written in one launch on HIP stream `stream`."""
    rc = _load().syn_fill_device_many(C.byref(f), table_dev, n_pieces, max_n, stream)
    if rc != 0:
        raise RuntimeError(f"syn_fill_device_many failed ({rc})")


def fill_tensor(f: Field, idx0: int, t) -> None:
    """Fill a contiguous torch CUDA tensor (float32, or int16/uint16/bf16/fp16 storage for 16-bit kinds)."""
    import torch

    assert t.is_cuda and t.is_contiguous()
    assert t.element_size() == (4 if f.kind == F32 else 2)
    fill_device(f, idx0, t.numel(), t.data_ptr(), torch.cuda.current_stream(t.device).cuda_stream)
