"""Python binding of libzero_shard.so: one data-parallel rank's ZeRO step on MI355X.

Argument marshalling only.  Every function has the name of the C entry point
it wraps (declared in include/zero_shard.h); all device work runs in the HIP
kernels of ``csrc/zero_shard.hip``.  PyTorch supplies device memory and the
stream.  There is no fallback: if the library is missing, importing this
package raises.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzero_shard.so")

ZERO_BF16 = 0
ZERO_FP16 = 1
ZERO_OK, ZERO_ERR_INVALID, ZERO_ERR_CAPACITY, ZERO_ERR_HIP = 0, -1, -2, -3

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python mixed_precision_adam_amd/build.py` "
                      "(or __graft_entry__.build()) first")

# PyTorch's HIP runtime must be the one the library binds to (it owns the memory and streams the library
# is handed), so it is loaded first; the library's libamdhip64.so.7 dependency then resolves to it.
import torch  # noqa: E402,F401


def hip_runtimes_loaded() -> list:
    """Distinct libamdhip64 files mapped into this process (exactly one is allowed)."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                paths.add(os.path.realpath(line.split()[-1]))
    return sorted(paths)


class ZeroError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


class zero_layout(C.Structure):
    _fields_ = [("psi", C.c_int64), ("padded_numel", C.c_int64), ("shard_numel", C.c_int64),
                ("shard_offset", C.c_int64), ("shard_valid", C.c_int64), ("world", C.c_int32), ("rank", C.c_int32),
                ("bytes_dp", C.c_int64), ("bytes_zero1", C.c_int64), ("bytes_zero2", C.c_int64),
                ("bytes_zero3", C.c_int64), ("comm_dp", C.c_int64), ("comm_zero1", C.c_int64),
                ("comm_zero2", C.c_int64), ("comm_zero3", C.c_int64)]


class zero_segment(C.Structure):
    _fields_ = [("tensor", C.c_int32), ("reserved", C.c_int32), ("src_offset", C.c_int64),
                ("dst_offset", C.c_int64), ("numel", C.c_int64)]


class zero_flat_seg(C.Structure):
    _fields_ = [("src", C.c_void_p), ("src_offset", C.c_int64), ("dst_offset", C.c_int64), ("numel", C.c_int64)]


class zero_adamw_hparams(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double), ("eps", C.c_double),
                ("weight_decay", C.c_double), ("grad_scale", C.c_double), ("step", C.c_int64)]


_P = C.c_void_p
_lib = C.CDLL(LIB_PATH)
if len(hip_runtimes_loaded()) != 1:
    raise ImportError(f"more than one HIP runtime in this process: {hip_runtimes_loaded()}")
_lib.zero_last_error.restype = C.c_char_p
_lib.zero_shard_layout.argtypes = [_P, C.c_int32, C.c_int32, C.c_int32, C.POINTER(zero_layout), _P, C.c_int32,
                                   C.POINTER(C.c_int32)]
_lib.zero_flatten_plan.argtypes = [_P, C.c_int32, _P, C.c_int32, _P]
_lib.zero_bucket_segments.argtypes = [_P, C.c_int32, C.c_int64, C.c_int64, _P, C.c_int32, C.POINTER(C.c_int32)]
_lib.zero_flatten_grads.argtypes = [_P, C.c_int32, C.c_int, _P, C.c_int64, _P]
_lib.zero_grad_sqnorm_workspace_bytes.argtypes = [C.c_int64]
_lib.zero_grad_sqnorm_workspace_bytes.restype = C.c_size_t
_lib.zero_grad_sqnorm.argtypes = [_P, C.c_int, C.c_int64, _P, C.c_size_t, _P, _P, _P]
_lib.zero_step_decision.argtypes = [_P, _P, C.c_int32, C.c_double, C.POINTER(C.c_double), C.POINTER(C.c_int32),
                                    C.c_int32, C.POINTER(C.c_double), C.POINTER(C.c_int32), C.POINTER(C.c_double)]
_lib.zero_clip_coef.argtypes = [C.c_double, C.c_double]
_lib.zero_clip_coef.restype = C.c_double
_lib.zero_loss_scale_update.argtypes = [C.POINTER(C.c_double), C.c_int32, C.POINTER(C.c_int32), C.c_int32]
_lib.zero_cosine_lr.argtypes = [C.c_int64, C.c_int64, C.c_double, C.c_double]
_lib.zero_cosine_lr.restype = C.c_double
_lib.zero_adamw_step.argtypes = [_P, C.c_int, _P, _P, _P, _P, C.c_int, C.c_int64, C.POINTER(zero_adamw_hparams),
                                 _P]
_lib.zero_flatten_grads_sqnorm.argtypes = [_P, C.c_int32, C.c_int, _P, C.c_int64, _P, C.c_size_t, _P, _P, _P]
_lib.zero_flatten_partials_count.argtypes = [C.c_int64]
_lib.zero_flatten_partials_count.restype = C.c_int64
_lib.zero_flatten_grads_partials.argtypes = [_P, C.c_int32, C.c_int, _P, C.c_int64, _P, _P, _P]
_lib.zero_sqnorm_reduce.argtypes = [_P, _P, C.c_int64, _P, _P, _P]
_lib.zero_state_tiled_numel.argtypes = [C.c_int64]
_lib.zero_state_tiled_numel.restype = C.c_int64
_lib.zero_adamw_step_tiled.argtypes = [_P, C.c_int, _P, _P, C.c_int, C.c_int64, C.POINTER(zero_adamw_hparams), _P]
_lib.zero_state_tile.argtypes = [_P, _P, _P, _P, C.c_int64, _P]
_lib.zero_state_untile.argtypes = [_P, _P, _P, _P, C.c_int64, _P]

_lib.zero_step_state_init.argtypes = [_P, C.c_double, C.c_int32, _P]
_lib.zero_step_decision_dev.argtypes = [_P, _P, C.c_int32, C.c_double, C.POINTER(zero_adamw_hparams), _P, _P]
_lib.zero_adamw_step_dev.argtypes = [_P, C.c_int, _P, _P, _P, _P, C.c_int, C.c_int64, _P, _P]
_lib.zero_adamw_step_tiled_dev.argtypes = [_P, C.c_int, _P, _P, C.c_int, C.c_int64, _P, _P]
_lib.zero_flatten_grads_sqnorm_noalloc.argtypes = [_P, C.c_int32, C.c_int, _P, C.c_int64, _P, _P, _P]
_lib.zero_calibrate_tiled_rmw.argtypes = [_P, _P, _P, C.c_int64, C.c_uint32, _P]

ZERO_STATE_TILE = 1024  # include/zero_shard.h


class zero_step_state(C.Structure):
    _fields_ = [("loss_scale", C.c_double), ("global_norm", C.c_double), ("grad_scale", C.c_double),
                ("adam_step", C.c_int64), ("iteration", C.c_int64), ("good_steps", C.c_int32),
                ("growth_interval", C.c_int32), ("skip", C.c_int32), ("error", C.c_int32),
                ("scalars", C.c_float * 12)]

# Every symbol include/zero_shard.h declares.
EXPORTS = ("zero_last_error", "zero_shard_layout", "zero_flatten_plan", "zero_bucket_segments", "zero_flatten_grads",
           "zero_flatten_grads_sqnorm", "zero_flatten_partials_count", "zero_flatten_grads_partials",
           "zero_sqnorm_reduce", "zero_grad_sqnorm_workspace_bytes", "zero_grad_sqnorm", "zero_step_decision",
           "zero_clip_coef", "zero_loss_scale_update", "zero_cosine_lr", "zero_adamw_step", "zero_state_tiled_numel",
           "zero_adamw_step_tiled", "zero_state_tile", "zero_state_untile", "zero_step_state_init",
           "zero_step_decision_dev", "zero_adamw_step_dev", "zero_adamw_step_tiled_dev",
           "zero_flatten_grads_sqnorm_noalloc", "zero_calibrate_tiled_rmw")
ZERO_STEP_ERR_LOSS_SCALE = 1  # zero_step_state.error: the decision could not be taken
ZERO_NOALLOC_SCRATCH_BYTES = 6 << 20  # static scratch of zero_flatten_grads_sqnorm_noalloc, per device


def library() -> C.CDLL:
    return _lib


def zero_last_error() -> str:
    return _lib.zero_last_error().decode()


def _check(status: int) -> None:
    if status != ZERO_OK:
        raise ZeroError(status, zero_last_error())


def _addr(x) -> int | None:
    """Device address of a torch tensor, or an int address as is.  Every buffer the entry points take is
    device memory read as one flat run of elements, so a tensor must be on the GPU and contiguous: a host
    tensor's address handed to a kernel would fault, and a strided view would be read as if dense."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError(f"a GPU tensor is required, got one on {x.device}")
    if not x.is_contiguous():
        raise ValueError(f"a contiguous tensor is required, got strides {tuple(x.stride())}")
    return x.data_ptr()


def _buf(x, nbytes: int) -> int | None:
    """_addr(x), after checking that a tensor holds at least the nbytes the entry point will touch (a count
    larger than the buffer would send a kernel past its end).  Plain int addresses are taken as they are."""
    if x is not None and not isinstance(x, int) and x.numel() * x.element_size() < nbytes:
        raise ValueError(f"buffer of {x.numel() * x.element_size()} bytes, the call touches {nbytes}")
    return _addr(x)


_SEG = C.sizeof(zero_flat_seg)
_STATE = C.sizeof(zero_step_state)


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


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


def zero_shard_layout(numels, world: int, rank: int):
    """Returns (Layout, segments) where segments is a ctypes array of zero_segment."""
    arr = (C.c_int64 * max(len(numels), 1))(*[int(n) for n in numels])
    out = zero_layout()
    n = C.c_int32(0)
    st = _lib.zero_shard_layout(C.cast(arr, _P), len(numels), world, rank, C.byref(out), None, 0, C.byref(n))
    if st not in (ZERO_OK, ZERO_ERR_CAPACITY):
        _check(st)
    segs = (zero_segment * max(n.value, 1))()
    _check(_lib.zero_shard_layout(C.cast(arr, _P), len(numels), world, rank, C.byref(out), C.cast(segs, _P),
                                  n.value, C.byref(n)))
    lay = Layout(*(getattr(out, f) for f, _ in zero_layout._fields_))
    return lay, segs[:n.value]


def zero_bucket_segments(segments, win_begin: int, win_numel: int):
    """The layout segments that fall in shard window [win_begin, win_begin + win_numel), re-based to it."""
    n = len(segments)
    segs = (zero_segment * max(n, 1))(*segments)
    cnt = C.c_int32(0)
    st = _lib.zero_bucket_segments(C.cast(segs, _P), n, win_begin, win_numel, None, 0, C.byref(cnt))
    if st not in (ZERO_OK, ZERO_ERR_CAPACITY):
        _check(st)
    out = (zero_segment * max(cnt.value, 1))()
    _check(_lib.zero_bucket_segments(C.cast(segs, _P), n, win_begin, win_numel, C.cast(out, _P), cnt.value,
                                     C.byref(cnt)))
    return out[:cnt.value]


def zero_flatten_plan(segments, tensor_ptrs) -> bytes:
    """Packs segments + tensor base addresses into the 32-byte device descriptors (returned as bytes)."""
    n = len(segments)
    segs = (zero_segment * max(n, 1))(*segments)
    need = [0] * len(tensor_ptrs)
    for sg in segments:  # 16-bit elements [src_offset, src_offset + numel) of each source are read
        if 0 <= sg.tensor < len(need):
            need[sg.tensor] = max(need[sg.tensor], 2 * (sg.src_offset + sg.numel))
    ptrs = (C.c_void_p * max(len(tensor_ptrs), 1))(*[_buf(p, k) for p, k in zip(tensor_ptrs, need)])
    out = (zero_flat_seg * max(n, 1))()
    _check(_lib.zero_flatten_plan(C.cast(segs, _P), n, C.cast(ptrs, _P), len(tensor_ptrs), C.cast(out, _P)))
    return bytes(out)[: n * C.sizeof(zero_flat_seg)]


def zero_flatten_grads(segs_dev, n_segs: int, dtype: int, shard, shard_numel: int, stream=None) -> None:
    _check(_lib.zero_flatten_grads(_buf(segs_dev, _SEG * max(n_segs, 0)), n_segs, dtype,
                                   _buf(shard, 2 * max(shard_numel, 0)), shard_numel, _stream(stream)))


def zero_grad_sqnorm_workspace_bytes(n: int) -> int:
    return int(_lib.zero_grad_sqnorm_workspace_bytes(n))


def zero_grad_sqnorm(shard, dtype: int, n: int, ws, ws_bytes: int, sqnorm_out, nonfinite_out, stream=None) -> None:
    _check(_lib.zero_grad_sqnorm(_buf(shard, 2 * max(n, 0)), dtype, n, _buf(ws, ws_bytes), ws_bytes,
                                 _buf(sqnorm_out, 8), _buf(nonfinite_out, 4), _stream(stream)))


def zero_step_decision(rank_sqnorms, rank_flags, max_norm: float, loss_scale: float, good_steps: int,
                       growth_interval: int) -> dict:
    n = len(rank_sqnorms)
    sq = (C.c_double * n)(*[float(x) for x in rank_sqnorms])
    fl = (C.c_int32 * n)(*[int(x) for x in rank_flags])
    ls, gd = C.c_double(loss_scale), C.c_int32(good_steps)
    gs, sk, gn = C.c_double(0.0), C.c_int32(0), C.c_double(0.0)
    _check(_lib.zero_step_decision(C.cast(sq, _P), C.cast(fl, _P), n, max_norm, C.byref(ls), C.byref(gd),
                                   growth_interval, C.byref(gs), C.byref(sk), C.byref(gn)))
    return dict(grad_scale=gs.value, skip=sk.value, global_norm=gn.value, loss_scale=ls.value, good_steps=gd.value)


def zero_clip_coef(global_sqnorm: float, max_norm: float) -> float:
    return _lib.zero_clip_coef(global_sqnorm, max_norm)


def zero_loss_scale_update(scale: float, nonfinite: int, good_steps: int, growth_interval: int):
    s, g = C.c_double(scale), C.c_int32(good_steps)
    _check(_lib.zero_loss_scale_update(C.byref(s), nonfinite, C.byref(g), growth_interval))
    return s.value, g.value


def zero_cosine_lr(t: int, total: int, lr_max: float, lr_min: float) -> float:
    return _lib.zero_cosine_lr(t, total, lr_max, lr_min)


def zero_adamw_step(grad, dtype: int, master, m, v, param, n: int, *, lr: float, beta1: float, beta2: float,
                    eps: float, weight_decay: float, grad_scale: float, step: int, stream=None,
                    param_dtype: int = ZERO_BF16) -> None:
    hp = zero_adamw_hparams(lr, beta1, beta2, eps, weight_decay, grad_scale, step)
    k = max(n, 0)
    _check(_lib.zero_adamw_step(_buf(grad, 2 * k), dtype, _buf(master, 4 * k), _buf(m, 4 * k), _buf(v, 4 * k),
                                _buf(param, 2 * k), param_dtype, n, C.byref(hp), _stream(stream)))


def zero_flatten_grads_sqnorm(segs_dev, n_segs: int, dtype: int, shard, shard_numel: int, ws, ws_bytes: int,
                              sqnorm_out, nonfinite_out, stream=None) -> None:
    _check(_lib.zero_flatten_grads_sqnorm(_buf(segs_dev, _SEG * max(n_segs, 0)), n_segs, dtype,
                                          _buf(shard, 2 * max(shard_numel, 0)), shard_numel, _buf(ws, ws_bytes),
                                          ws_bytes, _buf(sqnorm_out, 8), _buf(nonfinite_out, 4), _stream(stream)))


def zero_flatten_grads_sqnorm_noalloc(segs_dev, n_segs: int, dtype: int, shard, shard_numel: int, sqnorm_out,
                                      nonfinite_out, stream=None) -> None:
    _check(_lib.zero_flatten_grads_sqnorm_noalloc(_buf(segs_dev, _SEG * max(n_segs, 0)), n_segs, dtype,
                                                  _buf(shard, 2 * max(shard_numel, 0)), shard_numel,
                                                  _buf(sqnorm_out, 8), _buf(nonfinite_out, 4), _stream(stream)))


def zero_calibrate_tiled_rmw(grad, state, param, n: int, key: int = 0, stream=None) -> None:
    k = max(n, 0)
    _check(_lib.zero_calibrate_tiled_rmw(_buf(grad, 2 * k), _buf(state, 4 * zero_state_tiled_numel(k)),
                                         _buf(param, 2 * k), n, key, _stream(stream)))


def zero_flatten_partials_count(numel: int) -> int:
    return int(_lib.zero_flatten_partials_count(numel))


def zero_flatten_grads_partials(segs_dev, n_segs: int, dtype: int, dst, numel: int, part_sum, part_flag,
                                stream=None) -> None:
    parts = zero_flatten_partials_count(numel)
    _check(_lib.zero_flatten_grads_partials(_buf(segs_dev, _SEG * max(n_segs, 0)), n_segs, dtype,
                                            _buf(dst, 2 * max(numel, 0)), numel, _buf(part_sum, 8 * parts),
                                            _buf(part_flag, 4 * parts), _stream(stream)))


def zero_sqnorm_reduce(part_sum, part_flag, count: int, sqnorm_out, nonfinite_out, stream=None) -> None:
    k = max(count, 0)
    _check(_lib.zero_sqnorm_reduce(_buf(part_sum, 8 * k), _buf(part_flag, 4 * k), count, _buf(sqnorm_out, 8),
                                   _buf(nonfinite_out, 4), _stream(stream)))


def zero_state_tiled_numel(n: int) -> int:
    return int(_lib.zero_state_tiled_numel(n))


def zero_adamw_step_tiled(grad, dtype: int, state, param, n: int, *, lr: float, beta1: float, beta2: float,
                          eps: float, weight_decay: float, grad_scale: float, step: int, stream=None,
                          param_dtype: int = ZERO_BF16) -> None:
    hp = zero_adamw_hparams(lr, beta1, beta2, eps, weight_decay, grad_scale, step)
    k = max(n, 0)
    _check(_lib.zero_adamw_step_tiled(_buf(grad, 2 * k), dtype, _buf(state, 4 * zero_state_tiled_numel(k)),
                                      _buf(param, 2 * k), param_dtype, n, C.byref(hp), _stream(stream)))


def zero_state_tile(master, m, v, state, n: int, stream=None) -> None:
    k = max(n, 0)
    _check(_lib.zero_state_tile(_buf(master, 4 * k), _buf(m, 4 * k), _buf(v, 4 * k),
                                _buf(state, 4 * zero_state_tiled_numel(k)), n, _stream(stream)))


def zero_state_untile(state, master, m, v, n: int, stream=None) -> None:
    k = max(n, 0)
    _check(_lib.zero_state_untile(_buf(state, 4 * zero_state_tiled_numel(k)), _buf(master, 4 * k), _buf(m, 4 * k),
                                  _buf(v, 4 * k), n, _stream(stream)))


def zero_step_state_init(state, loss_scale: float, growth_interval: int, stream=None) -> None:
    _check(_lib.zero_step_state_init(_buf(state, _STATE), loss_scale, growth_interval, _stream(stream)))


def zero_step_decision_dev(rank_sqnorms, rank_flags, n_ranks: int, max_norm: float, state, *, lr: float,
                           beta1: float, beta2: float, eps: float, weight_decay: float, stream=None) -> None:
    hp = zero_adamw_hparams(lr, beta1, beta2, eps, weight_decay, 1.0, 1)
    k = max(n_ranks, 0)
    _check(_lib.zero_step_decision_dev(_buf(rank_sqnorms, 8 * k), _buf(rank_flags, 4 * k), n_ranks, max_norm,
                                       C.byref(hp), _buf(state, _STATE), _stream(stream)))


def zero_adamw_step_dev(grad, dtype: int, master, m, v, param, n: int, step_state, stream=None,
                        param_dtype: int = ZERO_BF16) -> None:
    k = max(n, 0)
    _check(_lib.zero_adamw_step_dev(_buf(grad, 2 * k), dtype, _buf(master, 4 * k), _buf(m, 4 * k), _buf(v, 4 * k),
                                    _buf(param, 2 * k), param_dtype, n, _buf(step_state, _STATE), _stream(stream)))


def zero_adamw_step_tiled_dev(grad, dtype: int, state, param, n: int, step_state, stream=None,
                              param_dtype: int = ZERO_BF16) -> None:
    k = max(n, 0)
    _check(_lib.zero_adamw_step_tiled_dev(_buf(grad, 2 * k), dtype, _buf(state, 4 * zero_state_tiled_numel(k)),
                                          _buf(param, 2 * k), param_dtype, n, _buf(step_state, _STATE),
                                          _stream(stream)))


def read_step_state(state_tensor) -> dict:
    """Copies a device zero_step_state (held in a torch tensor) to the host (synchronizes) and decodes it."""
    raw = bytes(state_tensor.detach().cpu().view(-1).view(__import__("torch").uint8).numpy().tobytes())
    st = zero_step_state.from_buffer_copy(raw[:C.sizeof(zero_step_state)])
    out = {f: getattr(st, f) for f, _ in zero_step_state._fields_ if f != "scalars"}
    out["scalars"] = list(st.scalars)[:9]
    return out
