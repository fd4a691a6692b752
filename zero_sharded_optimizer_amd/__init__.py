"""Fused ZeRO-sharded Adam step for AMD Instinct MI355X (gfx950).

A thin Python binding over the C ABI of libzero.so (include/zero_adam.h), with
the same function names. It only marshals arguments (device pointers, the HIP
stream, the hyperparameter struct) and checks that each tensor is a
contiguous device tensor of the dtype and size the call will touch; every step
of the computation runs in the library's HIP kernels. There is no CPU
fallback: without libzero.so every call raises.

The operation is the one of "ZeRO-Sharded Adam Step" (scratchllm.com),
sections "The step", "The shards" and "What to implement", with N logical
workers sharing one GPU:
  zero_init_states(hp, param, states)   -> m = v = 0, master from param
  zero_step(hp, param, grads, states, t) -> one reduce-scatter-mean / Adam /
                                            all-gather step, in place
  zero_step_with_mean(hp, param, grads, states, t, mean)
                                         -> the same step, also storing the averaged
                                            gradient (stage 1's .grad) in one pass
  zero_step_range(hp, param, grads, states, t, begin, end)
                                         -> the same step on [begin, end) only
                                            (one bucket of a bucketed step)
  zero_step_buckets(hp, param, grads, states, t, buckets, events)
                                         -> every bucket in one call, each after
                                            its ready event (overlap with backward)
  zero_mean_grad(hp, grads, mean, sumsq)  -> the reduce-scatter mean, materialised,
                                            and its squared norm
  zero_mean_grad_noalloc(hp, grads, mean, sumsq)
                                         -> the same with no workspace (library scratch)
  zero_step_mean(hp, param, mean, states, t, clip_sumsq, max_norm)
                                         -> the step from a materialised mean,
                                            optionally clipped by the global norm
  zero_step_clipped(hp, param, grads, states, t, max_norm, sumsq, workspace)
                                         -> both, as one clipped step
  zero_step_scalars(hp, t)               -> the step-dependent scalars of step t
  zero_step_range_dev(hp, param, grads, states, scalars, begin, end)
                                         -> zero_step_range with those scalars
                                            read from device memory (for launches
                                            captured into a graph and replayed)
  zero_memory_bytes(...)                 -> per-rank memory by ZeRO stage
  zero_min_stage(n, N, mode, act, avail) -> the smallest stage that fits
  zero_shard_bounds(n, N, r)             -> np.array_split shard [a, b)
"""
import ctypes as C
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from . import _abi
from ._abi import (ZERO_EHIP, ZERO_EINVAL, ZERO_EUNSUPPORTED, ZERO_MAX_WORKERS,  # noqa: F401
                   ZERO_MODE_F32, ZERO_MODE_F64, ZERO_MODE_MIXED_BF16, ZERO_MODE_MIXED_F16, ZERO_OK,
                   ZERO_OPT_ADAM,
                   ZERO_OPT_SGD)

__all__ = ["HParams", "States", "ZeroError", "zero_init_states", "zero_step",
           "zero_memory_bytes", "zero_shard_bounds", "zero_last_error", "wd_mask_from_flags",
           "zero_mean_grad_workspace_bytes", "zero_mean_grad", "zero_step_mean",
           "zero_step_clipped_workspace_bytes", "zero_step_clipped", "zero_step_range",
           "ZERO_MODE_F64", "ZERO_MODE_F32", "ZERO_MODE_MIXED_BF16", "ZERO_MODE_MIXED_F16",
           "ZERO_MAX_WORKERS",
           "ZERO_OPT_ADAM", "ZERO_OPT_SGD", "zero_step_scalars", "zero_step_range_dev",
           "STEP_SCALARS_BYTES", "zero_min_stage", "ZERO_MODE_MIXED_F16",
           "zero_step_buckets", "zero_step_with_mean", "zero_mean_grad_noalloc"]


class ZeroError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_abi.STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


@dataclass
class HParams:
    """Mirror of zero_hparams. No defaults for Adam's hyperparameters; the SGD
    fields are used only with optimizer=ZERO_OPT_SGD (then beta1/beta2/eps are
    ignored and may be 0)."""
    n: int
    n_workers: int
    mode: int
    lr: float
    beta1: float
    beta2: float
    eps: float
    weight_decay: float = 0.0
    rank: int = -1
    wd_mask: object = None  # device int32/uint32 tensor of (n + 31) // 32 words, or None
    optimizer: int = 0      # ZERO_OPT_ADAM or ZERO_OPT_SGD
    momentum: float = 0.0
    dampening: float = 0.0
    nesterov: bool = False

    def to_c(self):
        return _abi.zero_hparams(
            n=int(self.n), n_workers=int(self.n_workers), rank=int(self.rank),
            mode=int(self.mode), optimizer=int(self.optimizer), lr=float(self.lr),
            beta1=float(self.beta1), beta2=float(self.beta2), eps=float(self.eps),
            weight_decay=float(self.weight_decay), wd_mask=_addr(self.wd_mask),
            momentum=float(self.momentum), dampening=float(self.dampening),
            nesterov=int(bool(self.nesterov)), reserved=0)


@dataclass
class States:
    """Caller-owned optimizer state (master may be None in full fp64/fp32 mode)."""
    master: object
    m: object
    v: object

    def to_c(self):
        return _abi.zero_states(master=_addr(self.master), m=_addr(self.m), v=_addr(self.v))


# element types per mode: (parameter, gradient, state)
_DTYPES = {
    ZERO_MODE_F64: ("float64", "float64", "float64"),
    ZERO_MODE_F32: ("float32", "float32", "float32"),
    ZERO_MODE_MIXED_BF16: ("bfloat16", "bfloat16", "float32"),
    ZERO_MODE_MIXED_F16: ("float16", "float16", "float32"),
}


def _addr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _check_tensor(x, dtype_name, numel, what):
    """A raw int is taken as a device address the caller vouches for; a tensor
    must be a contiguous GPU tensor of the right dtype holding >= numel elements."""
    if x is None or isinstance(x, int):
        return
    import torch
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor or a device address")
    if not x.is_cuda:
        raise ValueError(f"{what}: must be a GPU tensor")
    if not x.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    if x.dtype != getattr(torch, dtype_name):
        raise ValueError(f"{what}: dtype {x.dtype}, expected torch.{dtype_name}")
    if x.numel() < numel:
        raise ValueError(f"{what}: {x.numel()} elements, the call touches {numel}")


def _tensor_args(xs):
    for x in xs:
        if x is None or isinstance(x, int):
            continue
        if isinstance(x, (list, tuple)):
            yield from _tensor_args(x)
        elif isinstance(x, States):
            yield from _tensor_args((x.master, x.m, x.v))
        elif hasattr(x, "device") and hasattr(x, "data_ptr"):
            yield x


def _same_device(stream, *xs):
    """The tensors of one call live on one GPU, and a torch stream passed for it
    belongs to that GPU: the library launches on the stream with the pointers
    as given, so a buffer on another device would be a bad address there."""
    devs = {str(x.device) for x in _tensor_args(xs)}
    if len(devs) > 1:
        raise ValueError(f"all tensors of one call must be on one device, got {sorted(devs)}")
    sdev = getattr(stream, "device", None)
    if devs and sdev is not None and str(sdev) not in devs:
        raise ValueError(f"stream is on {sdev}, the tensors on {devs.pop()}")


def _stream_handle(stream, like):
    if stream is None:
        import torch
        dev = like.device if hasattr(like, "device") else None
        return torch.cuda.current_stream(dev).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _raise(status):
    lib = _abi.load()
    raise ZeroError(status, lib.zero_last_error().decode())


def _shard_len(hp):
    if hp.rank < 0:
        return 0, hp.n
    a, b = zero_shard_bounds(hp.n, hp.n_workers, hp.rank)
    return a, b


def _check_common(hp, param, states):
    if hp.mode not in _DTYPES:
        return None
    p_dt, g_dt, s_dt = _DTYPES[hp.mode]
    if hp.n < 1 or hp.n_workers < 1 or not (-1 <= hp.rank < hp.n_workers):
        return None  # the library rejects these with its own message
    a, b = _shard_len(hp)
    _check_tensor(param, p_dt, hp.n, "param")
    _check_tensor(states.m, s_dt, b - a, "states.m")
    if states.v is not None or hp.optimizer != ZERO_OPT_SGD:
        _check_tensor(states.v, s_dt, b - a, "states.v")
    _check_tensor(states.master, s_dt, b - a, "states.master")
    if hp.weight_decay != 0.0 and hp.wd_mask is not None and not isinstance(hp.wd_mask, int):
        import torch
        if hp.wd_mask.dtype not in (torch.int32, torch.uint32):
            raise ValueError("wd_mask: expected int32/uint32 words")
        if not hp.wd_mask.is_cuda or not hp.wd_mask.is_contiguous():
            raise ValueError("wd_mask: must be a contiguous GPU tensor")
        if hp.wd_mask.numel() < (hp.n + 31) // 32:
            raise ValueError("wd_mask: needs (n + 31) // 32 words")
    return g_dt, b - a


def zero_init_states(hp: HParams, param, states: States, stream=None) -> None:
    """Enqueue init_states: m = v = 0, master = widen(param) (see zero_adam.h)."""
    _check_common(hp, param, states)
    _same_device(stream, param, states, hp.wd_mask)
    lib = _abi.load()
    c_hp, c_st = hp.to_c(), states.to_c()
    st = lib.zero_init_states(C.byref(c_hp), _addr(param), C.byref(c_st),
                              _stream_handle(stream, states.m))
    if st != ZERO_OK:
        _raise(st)


def zero_step(hp: HParams, param, grads: Sequence, states: States, t: int, stream=None) -> None:
    """Enqueue one fused step, in place (see zero_adam.h)."""
    chk = _check_common(hp, param, states)
    if chk is not None:
        g_dt, glen = chk
        if len(grads) != hp.n_workers:
            raise ValueError(f"grads: {len(grads)} buffers for {hp.n_workers} workers")
        for k, g in enumerate(grads):
            _check_tensor(g, g_dt, glen, f"grads[{k}]")
    _same_device(stream, param, grads, states, hp.wd_mask)
    lib = _abi.load()
    c_hp, c_st = hp.to_c(), states.to_c()
    arr = (C.c_void_p * max(1, len(grads)))(*[_addr(g) for g in grads])
    st = lib.zero_step(C.byref(c_hp), _addr(param), arr, C.byref(c_st), int(t),
                       _stream_handle(stream, states.m))
    if st != ZERO_OK:
        _raise(st)


def zero_step_with_mean(hp: HParams, param, grads: Sequence, states: States, t: int, mean_out,
                        stream=None) -> None:
    """Enqueue one fused step that also stores the averaged gradient of each
    element of the call in mean_out (state dtype; see zero_adam.h)."""
    chk = _check_common(hp, param, states)
    if chk is not None:
        g_dt, glen = chk
        if len(grads) != hp.n_workers:
            raise ValueError(f"grads: {len(grads)} buffers for {hp.n_workers} workers")
        for k, g in enumerate(grads):
            _check_tensor(g, g_dt, glen, f"grads[{k}]")
        _check_tensor(mean_out, _DTYPES[hp.mode][2], glen, "mean_out")
    _same_device(stream, param, grads, states, hp.wd_mask, mean_out)
    lib = _abi.load()
    c_hp, c_st = hp.to_c(), states.to_c()
    arr = (C.c_void_p * max(1, len(grads)))(*[_addr(g) for g in grads])
    st = lib.zero_step_with_mean(C.byref(c_hp), _addr(param), arr, C.byref(c_st), int(t),
                                 _addr(mean_out), _stream_handle(stream, states.m))
    if st != ZERO_OK:
        _raise(st)


def zero_step_range(hp: HParams, param, grads: Sequence, states: States, t: int, begin: int,
                    end: int, stream=None) -> None:
    """Enqueue the step on elements [begin, end) of the call's range."""
    chk = _check_common(hp, param, states)
    if chk is not None:
        g_dt, glen = chk
        if len(grads) != hp.n_workers:
            raise ValueError(f"grads: {len(grads)} buffers for {hp.n_workers} workers")
        for k, g in enumerate(grads):
            _check_tensor(g, g_dt, glen, f"grads[{k}]")
    _same_device(stream, param, grads, states, hp.wd_mask)
    lib = _abi.load()
    c_hp, c_st = hp.to_c(), states.to_c()
    arr = (C.c_void_p * max(1, len(grads)))(*[_addr(g) for g in grads])
    st = lib.zero_step_range(C.byref(c_hp), _addr(param), arr, C.byref(c_st), int(t), int(begin),
                             int(end), _stream_handle(stream, states.m))
    if st != ZERO_OK:
        _raise(st)


def _event_handle(ev):
    if ev is None or isinstance(ev, int):
        return ev
    return ev.cuda_event  # torch.cuda.Event: its hipEvent_t (recorded before this call)


def zero_step_buckets(hp: HParams, param, grads: Sequence, states: States, t: int,
                      buckets: Sequence, events: Optional[Sequence] = None, stream=None) -> None:
    """Enqueue the step on each (begin, end) bucket in order; bucket i waits for
    events[i] (a recorded torch.cuda.Event, a raw hipEvent_t, or None) first."""
    chk = _check_common(hp, param, states)
    if chk is not None:
        g_dt, glen = chk
        if len(grads) != hp.n_workers:
            raise ValueError(f"grads: {len(grads)} buffers for {hp.n_workers} workers")
        for k, g in enumerate(grads):
            _check_tensor(g, g_dt, glen, f"grads[{k}]")
    if events is not None and len(events) != len(buckets):
        raise ValueError(f"events: {len(events)} for {len(buckets)} buckets")
    _same_device(stream, param, grads, states, hp.wd_mask)
    lib = _abi.load()
    c_hp, c_st = hp.to_c(), states.to_c()
    arr = (C.c_void_p * max(1, len(grads)))(*[_addr(g) for g in grads])
    flat = [int(x) for lo_hi in buckets for x in lo_hi]
    edges = (C.c_int64 * max(1, len(flat)))(*flat)
    evs = None
    if events is not None:
        evs = (C.c_void_p * max(1, len(events)))(*[_event_handle(e) for e in events])
    st = lib.zero_step_buckets(C.byref(c_hp), _addr(param), arr, C.byref(c_st), int(t), edges,
                               len(buckets), evs, _stream_handle(stream, states.m))
    if st != ZERO_OK:
        _raise(st)


STEP_SCALARS_BYTES = C.sizeof(_abi.zero_step_scalars)


def zero_step_scalars(hp: HParams, t: int) -> np.ndarray:
    """The step-dependent scalars of step t (host-side, no device work), as the
    STEP_SCALARS_BYTES bytes of a zero_step_scalars: copy them into the device
    buffer that zero_step_range_dev reads before the launch (or the replay)."""
    lib = _abi.load()
    out = _abi.zero_step_scalars()
    c_hp = hp.to_c()
    st = lib.zero_step_scalars_fill(C.byref(c_hp), int(t), C.byref(out))
    if st != ZERO_OK:
        _raise(st)
    return np.frombuffer(bytes(out), dtype=np.uint8).copy()


def zero_step_range_dev(hp: HParams, param, grads: Sequence, states: States, scalars,
                        begin: int, end: int, stream=None) -> None:
    """Enqueue zero_step_range with the step scalars read on the device from
    `scalars` (a device tensor of >= STEP_SCALARS_BYTES bytes holding
    zero_step_scalars(hp, t) when the launch runs). Safe to capture into a
    graph: one kernel (one per 2^32 elements), no allocation, copy or
    synchronisation."""
    chk = _check_common(hp, param, states)
    if chk is not None:
        g_dt, glen = chk
        if len(grads) != hp.n_workers:
            raise ValueError(f"grads: {len(grads)} buffers for {hp.n_workers} workers")
        for k, g in enumerate(grads):
            _check_tensor(g, g_dt, glen, f"grads[{k}]")
    _check_bytes(scalars, STEP_SCALARS_BYTES, "scalars")
    _same_device(stream, param, grads, states, hp.wd_mask, scalars)
    lib = _abi.load()
    c_hp, c_st = hp.to_c(), states.to_c()
    arr = (C.c_void_p * max(1, len(grads)))(*[_addr(g) for g in grads])
    st = lib.zero_step_range_dev(C.byref(c_hp), _addr(param), arr, C.byref(c_st), _addr(scalars),
                                 int(begin), int(end), _stream_handle(stream, states.m))
    if st != ZERO_OK:
        _raise(st)


def _check_double(x, what):
    if x is None or isinstance(x, int):
        return
    _check_tensor(x, "float64", 1, what)


def _check_bytes(x, nbytes, what):
    """A workspace tensor: any dtype, contiguous, on the GPU, >= nbytes."""
    if x is None or isinstance(x, int):
        return
    import torch
    if not isinstance(x, torch.Tensor) or not x.is_cuda or not x.is_contiguous():
        raise ValueError(f"{what}: must be a contiguous GPU tensor")
    if x.numel() * x.element_size() < nbytes:
        raise ValueError(f"{what}: {x.numel() * x.element_size()} bytes, needs {nbytes}")


def _nbytes(x):
    if x is None or isinstance(x, int):
        return 1 << 62 if isinstance(x, int) else 0
    return x.numel() * x.element_size()


def zero_mean_grad_workspace_bytes(hp: HParams) -> int:
    lib = _abi.load()
    out = C.c_size_t()
    c_hp = hp.to_c()
    st = lib.zero_mean_grad_workspace_bytes(C.byref(c_hp), C.byref(out))
    if st != ZERO_OK:
        _raise(st)
    return out.value


def zero_mean_grad(hp: HParams, grads: Sequence, mean_out, sumsq_out=None, workspace=None,
                   stream=None) -> None:
    """Enqueue the materialised reduce-scatter mean (and squared norm)."""
    if hp.mode in _DTYPES and hp.n >= 1 and 1 <= hp.n_workers and -1 <= hp.rank < hp.n_workers:
        _, g_dt, s_dt = _DTYPES[hp.mode]
        a, b = _shard_len(hp)
        if len(grads) != hp.n_workers:
            raise ValueError(f"grads: {len(grads)} buffers for {hp.n_workers} workers")
        for k, g in enumerate(grads):
            _check_tensor(g, g_dt, b - a, f"grads[{k}]")
        _check_tensor(mean_out, s_dt, b - a, "mean_out")
        _check_double(sumsq_out, "sumsq_out")
        if sumsq_out is not None:
            _check_bytes(workspace, zero_mean_grad_workspace_bytes(hp), "workspace")
    _same_device(stream, grads, mean_out, sumsq_out, workspace)
    lib = _abi.load()
    c_hp = hp.to_c()
    arr = (C.c_void_p * max(1, len(grads)))(*[_addr(g) for g in grads])
    st = lib.zero_mean_grad(C.byref(c_hp), arr, _addr(mean_out), _addr(sumsq_out),
                            _addr(workspace), _nbytes(workspace),
                            _stream_handle(stream, mean_out if mean_out is not None else grads[0]))
    if st != ZERO_OK:
        _raise(st)


def zero_mean_grad_noalloc(hp: HParams, grads: Sequence, mean_out, sumsq_out=None,
                           stream=None) -> None:
    """Enqueue zero_mean_grad with the squared norm's partial sums in the
    library's static device scratch: no workspace, no allocation (see
    zero_adam.h for the size limit and the sharing rule)."""
    if hp.mode in _DTYPES and hp.n >= 1 and 1 <= hp.n_workers and -1 <= hp.rank < hp.n_workers:
        _, g_dt, s_dt = _DTYPES[hp.mode]
        a, b = _shard_len(hp)
        if len(grads) != hp.n_workers:
            raise ValueError(f"grads: {len(grads)} buffers for {hp.n_workers} workers")
        for k, g in enumerate(grads):
            _check_tensor(g, g_dt, b - a, f"grads[{k}]")
        _check_tensor(mean_out, s_dt, b - a, "mean_out")
        _check_double(sumsq_out, "sumsq_out")
    _same_device(stream, grads, mean_out, sumsq_out)
    lib = _abi.load()
    c_hp = hp.to_c()
    arr = (C.c_void_p * max(1, len(grads)))(*[_addr(g) for g in grads])
    st = lib.zero_mean_grad_noalloc(C.byref(c_hp), arr, _addr(mean_out), _addr(sumsq_out),
                                    _stream_handle(stream, mean_out if mean_out is not None
                                                   else grads[0]))
    if st != ZERO_OK:
        _raise(st)


def zero_step_mean(hp: HParams, param, mean_grad, states: States, t: int, clip_sumsq=None,
                   max_norm: float = 0.0, stream=None) -> None:
    """Enqueue the step from a materialised mean gradient (optionally clipped)."""
    chk = _check_common(hp, param, states)
    if chk is not None:
        _, glen = chk
        _check_tensor(mean_grad, _DTYPES[hp.mode][2], glen, "mean_grad")
        _check_double(clip_sumsq, "clip_sumsq")
    _same_device(stream, param, mean_grad, states, hp.wd_mask, clip_sumsq)
    lib = _abi.load()
    c_hp, c_st = hp.to_c(), states.to_c()
    st = lib.zero_step_mean(C.byref(c_hp), _addr(param), _addr(mean_grad), C.byref(c_st), int(t),
                            _addr(clip_sumsq), float(max_norm), _stream_handle(stream, states.m))
    if st != ZERO_OK:
        _raise(st)


def zero_step_clipped_workspace_bytes(hp: HParams) -> int:
    lib = _abi.load()
    out = C.c_size_t()
    c_hp = hp.to_c()
    st = lib.zero_step_clipped_workspace_bytes(C.byref(c_hp), C.byref(out))
    if st != ZERO_OK:
        _raise(st)
    return out.value


def zero_step_clipped(hp: HParams, param, grads: Sequence, states: States, t: int,
                      max_norm: float, workspace, sumsq_out=None, stream=None) -> None:
    """Enqueue one clipped step (full mode): mean, global squared norm, step."""
    chk = _check_common(hp, param, states)
    if chk is not None:
        g_dt, glen = chk
        if len(grads) != hp.n_workers:
            raise ValueError(f"grads: {len(grads)} buffers for {hp.n_workers} workers")
        for k, g in enumerate(grads):
            _check_tensor(g, g_dt, glen, f"grads[{k}]")
        _check_double(sumsq_out, "sumsq_out")
        if hp.rank < 0:
            _check_bytes(workspace, zero_step_clipped_workspace_bytes(hp), "workspace")
    _same_device(stream, param, grads, states, hp.wd_mask, sumsq_out, workspace)
    lib = _abi.load()
    c_hp, c_st = hp.to_c(), states.to_c()
    arr = (C.c_void_p * max(1, len(grads)))(*[_addr(g) for g in grads])
    st = lib.zero_step_clipped(C.byref(c_hp), _addr(param), arr, C.byref(c_st), int(t),
                               float(max_norm), _addr(sumsq_out), _addr(workspace),
                               _nbytes(workspace), _stream_handle(stream, states.m))
    if st != ZERO_OK:
        _raise(st)


def zero_memory_bytes(n: int, n_workers: int, rank: int, stage: int, mode: int,
                      convention: int = 0) -> dict:
    lib = _abi.load()
    out = _abi.zero_mem()
    st = lib.zero_memory_bytes(n, n_workers, rank, stage, mode, convention, C.byref(out))
    if st != ZERO_OK:
        _raise(st)
    return {"params": out.params, "grads": out.grads, "optimizer": out.optimizer,
            "total": out.total}


def zero_min_stage(n: int, n_workers: int, mode: int, activation_bytes: int,
                   available_bytes: int) -> int:
    """The smallest ZeRO stage whose per-rank memory plus activation_bytes is
    below available_bytes, or -1 if none is (see zero_adam.h)."""
    lib = _abi.load()
    out = C.c_int32()
    st = lib.zero_min_stage(n, n_workers, mode, activation_bytes, available_bytes,
                            C.byref(out))
    if st != ZERO_OK:
        _raise(st)
    return out.value


def zero_shard_bounds(n: int, n_workers: int, r: int):
    lib = _abi.load()
    a, b = C.c_int64(), C.c_int64()
    st = lib.zero_shard_bounds(n, n_workers, r, C.byref(a), C.byref(b))
    if st != ZERO_OK:
        _raise(st)
    return a.value, b.value


def zero_last_error() -> str:
    return _abi.load().zero_last_error().decode()


def wd_mask_from_flags(flags, device="cuda") -> "torch.Tensor":
    """Pack per-element decay flags (bool, length n) into the ABI's bitmask:
    element i is bit i % 32 of word i // 32. Returns an int32 device tensor."""
    import torch
    f = np.asarray(flags.cpu().numpy() if hasattr(flags, "cpu") else flags, dtype=bool)
    n = f.size
    words = (n + 31) // 32
    padded = np.zeros(words * 32, dtype=bool)
    padded[:n] = f
    packed = np.packbits(padded, bitorder="little").view("<u4").view(np.int32)
    return torch.from_numpy(packed.copy()).to(device)
