"""CPU oracle for one data-parallel rank's share of a ZeRO step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
library (``mixed_precision_adam_amd``) never imports, links or calls it, and the
two share no code.

This module is a thin ctypes wrapper around ``liboracle.so`` (plain,
single-threaded C built by ``build.sh``); every computation happens in
``oracle.c``, which cites the passages of the pages it follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_DEFAULT_LIB = os.path.join(_HERE, "liboracle.so")
# A test that plants mistakes in a copy of the oracle points this at the mutated build.
_LIB_PATH = os.environ.get("ZERO_ORACLE_LIB") or _DEFAULT_LIB

BF16 = 0
FP16 = 1


def build() -> None:
    """Compile liboracle.so with gcc (always rebuilds)."""
    subprocess.run(["sh", os.path.join(_HERE, "build.sh")], check=True)


class _Layout(C.Structure):
    _fields_ = [
        ("psi", C.c_int64),
        ("padded_numel", C.c_int64),
        ("shard_numel", C.c_int64),
        ("shard_offset", C.c_int64),
        ("shard_valid", C.c_int64),
        ("world", C.c_int32),
        ("rank", C.c_int32),
        ("bytes_dp", C.c_int64),
        ("bytes_zero1", C.c_int64),
        ("bytes_zero2", C.c_int64),
        ("bytes_zero3", C.c_int64),
        ("comm_dp", C.c_int64),
        ("comm_zero1", C.c_int64),
        ("comm_zero2", C.c_int64),
        ("comm_zero3", C.c_int64),
    ]


class _Segment(C.Structure):
    _fields_ = [
        ("tensor", C.c_int32),
        ("reserved", C.c_int32),
        ("src_offset", C.c_int64),
        ("dst_offset", C.c_int64),
        ("numel", C.c_int64),
    ]


class _HParams(C.Structure):
    _fields_ = [
        ("lr", C.c_double),
        ("beta1", C.c_double),
        ("beta2", C.c_double),
        ("eps", C.c_double),
        ("weight_decay", C.c_double),
        ("grad_scale", C.c_double),
        ("step", C.c_int64),
    ]


class _Scalars(C.Structure):
    _fields_ = [(n, C.c_float) for n in ("b1", "omb1", "b2", "omb2", "eps", "decay", "step_size", "bc2_sqrt", "gscale")]


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        if _LIB_PATH != _DEFAULT_LIB:
            raise FileNotFoundError(_LIB_PATH)
        build()
    lib = C.CDLL(_LIB_PATH)
    P = C.c_void_p
    lib.orc_layout_compute.argtypes = [P, C.c_int32, C.c_int32, C.c_int32, C.POINTER(_Layout), P, C.c_int32,
                                       C.POINTER(C.c_int32)]
    lib.orc_flatten.argtypes = [P, P, C.c_int32, C.c_int32, C.c_int32, P]
    lib.orc_sqnorm.argtypes = [P, C.c_int32, C.c_int64, C.POINTER(C.c_double), C.POINTER(C.c_int32)]
    lib.orc_clip_coef.argtypes = [C.c_double, C.c_double]
    lib.orc_clip_coef.restype = C.c_double
    lib.orc_loss_scale_update.argtypes = [C.POINTER(C.c_double), C.c_int32, C.POINTER(C.c_int32), C.c_int32]
    lib.orc_step_decision.argtypes = [P, P, C.c_int32, C.c_double, C.POINTER(C.c_double), C.POINTER(C.c_int32),
                                      C.c_int32, C.POINTER(C.c_double), C.POINTER(C.c_int32),
                                      C.POINTER(C.c_double)]
    lib.orc_cosine_lr.argtypes = [C.c_int64, C.c_int64, C.c_double, C.c_double]
    lib.orc_cosine_lr.restype = C.c_double
    lib.orc_adamw_scalars.argtypes = [C.POINTER(_HParams), C.POINTER(_Scalars)]
    lib.orc_adamw_step.argtypes = [P, C.c_int32, P, P, P, P, C.c_int32, C.c_int64, C.POINTER(_HParams)]
    lib.orc_adamw_step_f64.argtypes = [P, P, P, P, C.c_int64, C.POINTER(_HParams)]
    lib.orc_bf16_to_f32.argtypes = [C.c_uint16]
    lib.orc_bf16_to_f32.restype = C.c_float
    lib.orc_f16_to_f32.argtypes = [C.c_uint16]
    lib.orc_f16_to_f32.restype = C.c_float
    lib.orc_f32_to_bf16.argtypes = [C.c_float]
    lib.orc_f32_to_bf16.restype = C.c_uint16
    lib.orc_f32_to_bf16_array.argtypes = [P, P, C.c_int64]
    lib.orc_f32_to_f16.argtypes = [C.c_float]
    lib.orc_f32_to_f16.restype = C.c_uint16
    lib.orc_f32_to_f16_array.argtypes = [P, P, C.c_int64]
    lib.orc_decode_array.argtypes = [P, C.c_int32, P, C.c_int64]
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle buffers must be contiguous"
    return a.ctypes.data


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise OracleError(f"{what} failed with status {rc}")


@dataclass
class Layout:
    psi: int
    padded_numel: int
    shard_numel: int
    shard_offset: int
    shard_valid: int
    world: int
    rank: int
    bytes_dp: int
    bytes_zero1: int
    bytes_zero2: int
    bytes_zero3: int
    comm_dp: int
    comm_zero1: int
    comm_zero2: int
    comm_zero3: int
    segments: list  # list of (tensor, src_offset, dst_offset, numel)


def layout(numels, world: int, rank: int) -> Layout:
    lib = _load()
    arr = np.ascontiguousarray(np.asarray(numels, dtype=np.int64))
    out = _Layout()
    n_segs = C.c_int32(0)
    rc = lib.orc_layout_compute(_ptr(arr) if arr.size else None, int(arr.size), world, rank, C.byref(out), None, 0,
                                C.byref(n_segs))
    if rc not in (0, -2):
        raise OracleError(f"orc_layout_compute failed with status {rc}")
    cap = n_segs.value
    segs = (_Segment * max(cap, 1))()
    rc = lib.orc_layout_compute(_ptr(arr) if arr.size else None, int(arr.size), world, rank, C.byref(out), segs, cap,
                                C.byref(n_segs))
    _check(rc, "orc_layout_compute")
    seg_list = [(s.tensor, s.src_offset, s.dst_offset, s.numel) for s in segs[: n_segs.value]]
    return Layout(out.psi, out.padded_numel, out.shard_numel, out.shard_offset, out.shard_valid, out.world, out.rank,
                  out.bytes_dp, out.bytes_zero1, out.bytes_zero2, out.bytes_zero3, out.comm_dp, out.comm_zero1,
                  out.comm_zero2, out.comm_zero3, seg_list)


def layout_status(numels, world: int, rank: int, cap: int):
    """Raw call for error-path tests: returns (status, n_segs)."""
    lib = _load()
    arr = np.ascontiguousarray(np.asarray(numels, dtype=np.int64))
    out = _Layout()
    n_segs = C.c_int32(-1)
    segs = (_Segment * max(cap, 1))()
    rc = lib.orc_layout_compute(_ptr(arr) if arr.size else None, int(arr.size), world, rank, C.byref(out),
                                segs if cap > 0 else None, cap, C.byref(n_segs))
    return rc, n_segs.value


def flatten(tensors, numels, world: int, rank: int) -> np.ndarray:
    """tensors: list of uint16 arrays (or None for tensors outside the shard)."""
    lib = _load()
    nums = np.ascontiguousarray(np.asarray(numels, dtype=np.int64))
    psi = int(nums.sum())
    s = -(-psi // world) if psi else 0
    keep = []
    ptrs = (C.c_void_p * max(len(tensors), 1))()
    for i, t in enumerate(tensors):
        if t is None:
            ptrs[i] = None
        else:
            t = np.ascontiguousarray(t, dtype=np.uint16)
            assert t.size == nums[i]
            keep.append(t)
            ptrs[i] = t.ctypes.data
    out = np.empty(max(s, 1), dtype=np.uint16)
    rc = lib.orc_flatten(C.cast(ptrs, C.c_void_p), _ptr(nums) if nums.size else None, len(tensors), world, rank,
                         _ptr(out))
    _check(rc, "orc_flatten")
    return out[:s]


def sqnorm(x: np.ndarray, dtype: int):
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.uint16)
    sq = C.c_double(0.0)
    flag = C.c_int32(0)
    rc = lib.orc_sqnorm(_ptr(x) if x.size else None, dtype, x.size, C.byref(sq), C.byref(flag))
    _check(rc, "orc_sqnorm")
    return sq.value, flag.value


def clip_coef(global_sqnorm: float, max_norm: float) -> float:
    return _load().orc_clip_coef(global_sqnorm, max_norm)


def loss_scale_update(scale: float, nonfinite: int, good_steps: int, growth_interval: int):
    lib = _load()
    s = C.c_double(scale)
    g = C.c_int32(good_steps)
    _check(lib.orc_loss_scale_update(C.byref(s), nonfinite, C.byref(g), growth_interval), "orc_loss_scale_update")
    return s.value, g.value


def step_decision(rank_sqnorms, rank_flags, max_norm: float, loss_scale: float, good_steps: int,
                  growth_interval: int):
    """Returns dict(grad_scale, skip, global_norm, loss_scale, good_steps)."""
    lib = _load()
    sq = np.ascontiguousarray(np.asarray(rank_sqnorms, dtype=np.float64))
    fl = np.ascontiguousarray(np.asarray(rank_flags, dtype=np.int32))
    assert sq.size == fl.size
    ls = C.c_double(loss_scale)
    gd = C.c_int32(good_steps)
    gs = C.c_double(0.0)
    sk = C.c_int32(0)
    gn = C.c_double(0.0)
    _check(lib.orc_step_decision(_ptr(sq), _ptr(fl), sq.size, max_norm, C.byref(ls), C.byref(gd), growth_interval,
                                 C.byref(gs), C.byref(sk), C.byref(gn)), "orc_step_decision")
    return dict(grad_scale=gs.value, skip=sk.value, global_norm=gn.value, loss_scale=ls.value, good_steps=gd.value)


def cosine_lr(t: int, total: int, lr_max: float, lr_min: float) -> float:
    return _load().orc_cosine_lr(t, total, lr_max, lr_min)


def _hp(lr, beta1, beta2, eps, weight_decay, grad_scale, step) -> _HParams:
    return _HParams(lr, beta1, beta2, eps, weight_decay, grad_scale, step)


def adamw_scalars(lr, beta1, beta2, eps, weight_decay, grad_scale, step) -> dict:
    s = _Scalars()
    hp = _hp(lr, beta1, beta2, eps, weight_decay, grad_scale, step)
    _check(_load().orc_adamw_scalars(C.byref(hp), C.byref(s)), "orc_adamw_scalars")
    return {n: np.float32(getattr(s, n)) for n, _ in _Scalars._fields_}


def adamw_step(grad: np.ndarray, dtype: int, master: np.ndarray, m: np.ndarray, v: np.ndarray, param: np.ndarray, *,
               lr, beta1, beta2, eps, weight_decay, grad_scale, step, param_dtype: int = BF16) -> None:
    """In-place update of master / m / v (float32) and param (uint16 bits of bf16, or of fp16 when
    param_dtype is FP16)."""
    n = grad.size
    assert grad.dtype == np.uint16 and param.dtype == np.uint16
    assert master.dtype == np.float32 and m.dtype == np.float32 and v.dtype == np.float32
    assert master.size == n and m.size == n and v.size == n and param.size == n
    hp = _hp(lr, beta1, beta2, eps, weight_decay, grad_scale, step)
    rc = _load().orc_adamw_step(_ptr(grad), dtype, _ptr(master), _ptr(m), _ptr(v), _ptr(param), param_dtype, n,
                                C.byref(hp))
    _check(rc, "orc_adamw_step")


def adamw_step_f64(grad: np.ndarray, master: np.ndarray, m: np.ndarray, v: np.ndarray, *, lr, beta1, beta2, eps,
                   weight_decay, grad_scale, step) -> None:
    n = grad.size
    for a in (grad, master, m, v):
        assert a.dtype == np.float64 and a.size == n
    hp = _hp(lr, beta1, beta2, eps, weight_decay, grad_scale, step)
    _check(_load().orc_adamw_step_f64(_ptr(grad), _ptr(master), _ptr(m), _ptr(v), n, C.byref(hp)),
           "orc_adamw_step_f64")


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, dtype=np.uint16)
    _load().orc_f32_to_bf16_array(_ptr(x), _ptr(y), x.size)
    return y


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, dtype=np.uint16)
    _load().orc_f32_to_f16_array(_ptr(x), _ptr(y), x.size)
    return y


def decode(x: np.ndarray, dtype: int) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    y = np.empty(x.shape, dtype=np.float32)
    _load().orc_decode_array(_ptr(x), dtype, _ptr(y), x.size)
    return y
