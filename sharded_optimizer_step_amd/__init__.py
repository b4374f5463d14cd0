"""The per-rank ZeRO shard step for MI355X (gfx950): a thin ctypes binding
of the C ABI declared in ``include/zero_step.h``.

This module only marshals arguments (torch tensors -> device or host
pointers and the current HIP stream). Every step of the computation runs in
``libzero_step.so``: its HIP kernels, and for the CPU-offloaded step (whose
optimizer state lives in host memory by design) the host optimizer built
into the same library. There is no CPU fallback: if the library is missing
the first call raises.

Functions keep the C names:

* ``zero_shard_reduce(grads, grad_scale, g_out)``
* ``zero_grad_check_norm_workspace_bytes(n)``
* ``zero_grad_check_norm(g, hp, external_sumsq, ws, res)``
* ``zero_adamw_step(master, exp_avg, exp_avg_sq, g, param_out, hp, res=None)``
* ``zero_step_workspace_bytes(tensors, M, hp)``
* ``zero_step(tensors, hp, external_sumsq, ws, res)``; ``StepRunner(tensors, ws, res).step(hp, external_sumsq)``
  (and ``.step_amp``): the same calls with the tensor list marshalled once
* ``zero_step_noalloc(tensors, hp, external_sumsq, res)``: the same step with the library's static device scratch
  as its workspace, for callers that cannot allocate
* ``zero_loss_scale_init(cfg, ls)``, ``zero_loss_scale_update(cfg, res, ls)``
* ``zero_step_amp_workspace_bytes(tensors, M, hp)``, ``zero_step_amp(tensors, hp, cfg, ls, external_sumsq, ws, res)``
* ``zero_bucket_reduce_workspace_bytes(shards, M)``,
  ``zero_bucket_reduce(shards, flags, grad_scale, stamp, partial, ws)``
* ``zero_step_accumulated_workspace_bytes(tensors)``,
  ``zero_step_accumulated(tensors, hp, partials, nbuckets, stamp, external_sumsq, ws, res)``,
  ``BucketReducer(shards, partial, ws=None, ls=None).reduce(flags, grad_scale, stamp)``
* ``zero_bucket_step_workspace_bytes(tensors, M)``, ``zero_bucket_step(tensors, flags, hp, stamp, partial, ws)``,
  ``BucketStepper(tensors, partial, ws=None).step(flags, hp, stamp)``: a bucket's final micro-batch folded and
  applied in one pass (no clipping, no skipping); then ``zero_step_accumulated([], ...)`` writes the record
* ``zero_offload_workspace_bytes(tensors, M)``, ``zero_offload_host_workspace_bytes(tensors)``,
  ``zero_offload_step(tensors, hp, external_sumsq, ws, host_ws, threads)``,
  ``zero_offload_adamw_host(master, exp_avg, exp_avg_sq, g, param_out, hp, clip_coef, threads)``
* ``zero_bucket_reduce_amp``, ``zero_step_accumulated_amp``, ``zero_offload_step_amp``: the same under the
  dynamic loss scale
* ``zero_workspace_forget(ws)``, ``zero_status_string(status)``
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import struct
import weakref
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzero_step.so")

ZERO_OK = 0
ZERO_ERR_INVALID_ARGUMENT = 1
ZERO_ERR_WORKSPACE_TOO_SMALL = 2
ZERO_ERR_HIP = 3
ZERO_ERR_STALE_WORKSPACE = 4
ZERO_ERR_BUCKET_PARTIALS = 5
ZERO_ERR_SCRATCH_TOO_SMALL = 6
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024
RESULT_BYTES = 32
BUCKET_ACCUMULATE = 1
BUCKET_FINAL = 2
BUCKET_STREAM_STORES = 4
# steps above this many parameters write more than the 256 MiB Infinity Cache holds
STREAM_STORES_MIN_PARAMS = (256 << 20) // 14
BUCKET_PARTIAL_BYTES = 32

# Every symbol the C ABI exports (include/zero_step.h).
EXPORTS = ("zero_shard_reduce", "zero_grad_check_norm_workspace_bytes", "zero_grad_check_norm", "zero_adamw_step",
           "zero_step_workspace_bytes", "zero_step", "zero_loss_scale_init", "zero_loss_scale_update",
           "zero_step_amp_workspace_bytes", "zero_step_amp", "zero_bucket_reduce_workspace_bytes",
           "zero_bucket_reduce", "zero_step_accumulated_workspace_bytes", "zero_step_accumulated",
           "zero_offload_workspace_bytes", "zero_offload_host_workspace_bytes", "zero_offload_step",
           "zero_offload_adamw_host", "zero_bucket_reduce_amp", "zero_step_accumulated_amp",
           "zero_offload_step_amp", "zero_workspace_forget", "zero_status_string", "zero_step_noalloc",
           "zero_bucket_step_workspace_bytes", "zero_bucket_step")
LOSS_SCALE_BYTES = 16


class _CHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double), ("step", ctypes.c_int64),
                ("max_grad_norm", ctypes.c_double), ("grad_scale", ctypes.c_double),
                ("skip_on_nonfinite", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class _CTensor(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("grads", ctypes.POINTER(ctypes.c_void_p)), ("master", ctypes.c_void_p),
                ("exp_avg", ctypes.c_void_p), ("exp_avg_sq", ctypes.c_void_p), ("param_out", ctypes.c_void_p)]


class _CGradShard(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("grads", ctypes.POINTER(ctypes.c_void_p)), ("grad_acc", ctypes.c_void_p)]


class _CAccTensor(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("grad_acc", ctypes.c_void_p), ("master", ctypes.c_void_p),
                ("exp_avg", ctypes.c_void_p), ("exp_avg_sq", ctypes.c_void_p), ("param_out", ctypes.c_void_p)]


class _CBucketTensor(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("grads", ctypes.POINTER(ctypes.c_void_p)), ("grad_acc", ctypes.c_void_p),
                ("master", ctypes.c_void_p), ("exp_avg", ctypes.c_void_p), ("exp_avg_sq", ctypes.c_void_p),
                ("param_out", ctypes.c_void_p)]


class _COffloadTensor(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("grads", ctypes.POINTER(ctypes.c_void_p)), ("master", ctypes.c_void_p),
                ("exp_avg", ctypes.c_void_p), ("exp_avg_sq", ctypes.c_void_p), ("param_out", ctypes.c_void_p)]


class _CResult(ctypes.Structure):
    _fields_ = [("sumsq", ctypes.c_double), ("clip_coef", ctypes.c_double), ("grad_norm", ctypes.c_float),
                ("found_inf", ctypes.c_int32), ("skipped", ctypes.c_int32), ("status", ctypes.c_int32)]


class _CLossScaleConfig(ctypes.Structure):
    _fields_ = [("initial_scale_power", ctypes.c_int32), ("window", ctypes.c_int32), ("hysteresis", ctypes.c_int32),
                ("min_scale", ctypes.c_float)]


class ZeroError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {zero_status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, dbl, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_size_t
        L.zero_shard_reduce.argtypes = [ctypes.POINTER(vp), i32, i64, dbl, vp, vp]
        L.zero_shard_reduce.restype = ctypes.c_int
        L.zero_grad_check_norm_workspace_bytes.argtypes = [i64]
        L.zero_grad_check_norm_workspace_bytes.restype = sz
        L.zero_grad_check_norm.argtypes = [vp, i64, ctypes.POINTER(_CHparams), dbl, vp, sz, vp, vp]
        L.zero_grad_check_norm.restype = ctypes.c_int
        L.zero_adamw_step.argtypes = [vp, vp, vp, vp, vp, i64, ctypes.POINTER(_CHparams), vp, vp]
        L.zero_adamw_step.restype = ctypes.c_int
        L.zero_step_workspace_bytes.argtypes = [ctypes.POINTER(_CTensor), i32, i32, ctypes.POINTER(_CHparams)]
        L.zero_step_workspace_bytes.restype = sz
        L.zero_step.argtypes = [ctypes.POINTER(_CTensor), i32, i32, ctypes.POINTER(_CHparams), dbl, vp, sz, vp, vp]
        L.zero_step.restype = ctypes.c_int
        L.zero_step_noalloc.argtypes = [ctypes.POINTER(_CTensor), i32, i32, ctypes.POINTER(_CHparams), dbl, vp, vp]
        L.zero_step_noalloc.restype = ctypes.c_int
        L.zero_loss_scale_init.argtypes = [ctypes.POINTER(_CLossScaleConfig), vp, vp]
        L.zero_loss_scale_init.restype = ctypes.c_int
        L.zero_loss_scale_update.argtypes = [ctypes.POINTER(_CLossScaleConfig), vp, vp, vp]
        L.zero_loss_scale_update.restype = ctypes.c_int
        L.zero_step_amp_workspace_bytes.argtypes = [ctypes.POINTER(_CTensor), i32, i32, ctypes.POINTER(_CHparams)]
        L.zero_step_amp_workspace_bytes.restype = sz
        L.zero_step_amp.argtypes = [ctypes.POINTER(_CTensor), i32, i32, ctypes.POINTER(_CHparams),
                                    ctypes.POINTER(_CLossScaleConfig), vp, dbl, vp, sz, vp, vp]
        L.zero_step_amp.restype = ctypes.c_int
        u64 = ctypes.c_uint64
        L.zero_bucket_reduce_workspace_bytes.argtypes = [ctypes.POINTER(_CGradShard), i32, i32]
        L.zero_bucket_reduce_workspace_bytes.restype = sz
        L.zero_bucket_reduce.argtypes = [ctypes.POINTER(_CGradShard), i32, i32, i32, dbl, u64, vp, vp, sz, vp]
        L.zero_bucket_reduce.restype = ctypes.c_int
        L.zero_step_accumulated_workspace_bytes.argtypes = [ctypes.POINTER(_CAccTensor), i32]
        L.zero_step_accumulated_workspace_bytes.restype = sz
        L.zero_step_accumulated.argtypes = [ctypes.POINTER(_CAccTensor), i32, ctypes.POINTER(_CHparams), vp, i32,
                                            u64, dbl, vp, sz, vp, vp]
        L.zero_step_accumulated.restype = ctypes.c_int
        L.zero_bucket_step_workspace_bytes.argtypes = [ctypes.POINTER(_CBucketTensor), i32, i32]
        L.zero_bucket_step_workspace_bytes.restype = sz
        L.zero_bucket_step.argtypes = [ctypes.POINTER(_CBucketTensor), i32, i32, i32, ctypes.POINTER(_CHparams), u64,
                                       vp, vp, sz, vp]
        L.zero_bucket_step.restype = ctypes.c_int
        L.zero_offload_workspace_bytes.argtypes = [ctypes.POINTER(_COffloadTensor), i32, i32]
        L.zero_offload_workspace_bytes.restype = sz
        L.zero_offload_host_workspace_bytes.argtypes = [ctypes.POINTER(_COffloadTensor), i32]
        L.zero_offload_host_workspace_bytes.restype = sz
        L.zero_offload_step.argtypes = [ctypes.POINTER(_COffloadTensor), i32, i32, ctypes.POINTER(_CHparams), dbl, vp,
                                        sz, vp, sz, ctypes.POINTER(_CResult), i32, vp]
        L.zero_offload_step.restype = ctypes.c_int
        L.zero_offload_adamw_host.argtypes = [vp, vp, vp, vp, vp, i64, ctypes.POINTER(_CHparams), dbl, i32]
        L.zero_offload_adamw_host.restype = ctypes.c_int
        lsc = ctypes.POINTER(_CLossScaleConfig)
        L.zero_bucket_reduce_amp.argtypes = [ctypes.POINTER(_CGradShard), i32, i32, i32, dbl, vp, u64, vp, vp, sz, vp]
        L.zero_bucket_reduce_amp.restype = ctypes.c_int
        L.zero_step_accumulated_amp.argtypes = [ctypes.POINTER(_CAccTensor), i32, ctypes.POINTER(_CHparams), lsc, vp,
                                                vp, i32, u64, dbl, vp, sz, vp, vp]
        L.zero_step_accumulated_amp.restype = ctypes.c_int
        L.zero_offload_step_amp.argtypes = [ctypes.POINTER(_COffloadTensor), i32, i32, ctypes.POINTER(_CHparams), lsc,
                                            vp, dbl, vp, sz, vp, sz, ctypes.POINTER(_CResult), i32, vp]
        L.zero_offload_step_amp.restype = ctypes.c_int
        L.zero_workspace_forget.argtypes = [vp]
        L.zero_workspace_forget.restype = ctypes.c_int
        L.zero_status_string.argtypes = [ctypes.c_int]
        L.zero_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


@dataclasses.dataclass
class HParams:
    """AdamW knobs of one step (names of a deepspeed_config.json optimizer
    block), the step index t >= 1, the clip threshold (<= 0: off), the
    multiplier of the fp32 gradient sum, and the skip switch."""
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1
    step: int = 1
    max_grad_norm: float = 0.0
    grad_scale: float = 1.0
    skip_on_nonfinite: int = 0

    def _c(self) -> _CHparams:
        return _CHparams(float(self.lr), float(self.beta1), float(self.beta2), float(self.eps),
                         float(self.weight_decay), int(self.step), float(self.max_grad_norm), float(self.grad_scale),
                         int(bool(self.skip_on_nonfinite)), 0)


@dataclasses.dataclass
class ZeroTensor:
    """One tensor's shard: M bf16 gradient replicas, fp32 master/exp_avg/
    exp_avg_sq (updated in place) and the bf16 output shard."""
    grads: List[torch.Tensor]
    master: torch.Tensor
    exp_avg: torch.Tensor
    exp_avg_sq: torch.Tensor
    param_out: torch.Tensor


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, dtype, name: str, n: Optional[int] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if n is not None and t.numel() != n:
        raise ValueError(f"{name}: expected {n} elements, got {t.numel()}")


def _need_ws(ws: Optional[torch.Tensor], name: str = "ws") -> int:
    """A device workspace (any dtype, contiguous) or None; returns its bytes.
    The library writes through it from kernels: a host tensor here would be a
    host address on the GPU."""
    if ws is None:
        return 0
    if not isinstance(ws, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not ws.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not ws.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return ws.numel() * ws.element_size()


def _check(status: int, where: str):
    if status != ZERO_OK:
        raise ZeroError(status, where)


def zero_status_string(status: int) -> str:
    return lib().zero_status_string(int(status)).decode()


def new_result(device=None) -> torch.Tensor:
    """A 32-byte device buffer for the zero_result record."""
    return torch.zeros(RESULT_BYTES, dtype=torch.uint8, device=device or "cuda")


def read_result(res: torch.Tensor) -> dict:
    """Copy the record to the host (synchronizes with its stream)."""
    b = bytes(res.cpu().numpy().tobytes())
    sumsq, coef, norm, found_inf, skipped, status = struct.unpack("<ddfiii", b)
    return dict(sumsq=sumsq, grad_norm=norm, clip_coef=coef, found_inf=found_inf, skipped=skipped, status=status)


def zero_shard_reduce(grads: Sequence[torch.Tensor], grad_scale: float, g_out: torch.Tensor, stream=None) -> None:
    n = g_out.numel()
    _need(g_out, torch.float32, "g_out")
    for r, g in enumerate(grads):
        _need(g, torch.bfloat16, f"grads[{r}]", n)
    arr = (ctypes.c_void_p * max(len(grads), 1))(*[g.data_ptr() for g in grads])
    _check(lib().zero_shard_reduce(arr, len(grads), n, float(grad_scale), g_out.data_ptr(), _stream(stream)),
           "zero_shard_reduce")


def zero_grad_check_norm_workspace_bytes(n: int) -> int:
    return int(lib().zero_grad_check_norm_workspace_bytes(int(n)))


def zero_grad_check_norm(g: torch.Tensor, hp: Optional[HParams], external_sumsq: float, ws: Optional[torch.Tensor],
                         res: torch.Tensor, stream=None) -> None:
    _need(g, torch.float32, "g")
    _need(res, torch.uint8, "res", RESULT_BYTES)
    h = hp._c() if hp is not None else None
    wsb = _need_ws(ws)
    _check(lib().zero_grad_check_norm(g.data_ptr(), g.numel(), ctypes.byref(h) if h is not None else None,
                                      float(external_sumsq), _ptr(ws), wsb, res.data_ptr(), _stream(stream)),
           "zero_grad_check_norm")


def zero_adamw_step(master: torch.Tensor, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor, g: torch.Tensor,
                    param_out: torch.Tensor, hp: HParams, res: Optional[torch.Tensor] = None, stream=None) -> None:
    n = master.numel()
    for t, nm in ((master, "master"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"), (g, "g")):
        _need(t, torch.float32, nm, n)
    _need(param_out, torch.bfloat16, "param_out", n)
    if res is not None:
        _need(res, torch.uint8, "res", RESULT_BYTES)
    h = hp._c()
    _check(lib().zero_adamw_step(master.data_ptr(), exp_avg.data_ptr(), exp_avg_sq.data_ptr(), g.data_ptr(),
                                 param_out.data_ptr(), n, ctypes.byref(h), _ptr(res), _stream(stream)),
           "zero_adamw_step")


def _ctensors(tensors: Sequence[ZeroTensor], check: bool):
    M = len(tensors[0].grads) if tensors else 1
    keep = []
    arr = (_CTensor * max(len(tensors), 1))()
    for i, t in enumerate(tensors):
        n = t.master.numel()
        if check:
            if len(t.grads) != M:
                raise ValueError(f"tensor {i}: {len(t.grads)} replicas, expected {M}")
            for r, g in enumerate(t.grads):
                _need(g, torch.bfloat16, f"tensors[{i}].grads[{r}]", n)
            for x, nm in ((t.master, "master"), (t.exp_avg, "exp_avg"), (t.exp_avg_sq, "exp_avg_sq")):
                _need(x, torch.float32, f"tensors[{i}].{nm}", n)
            _need(t.param_out, torch.bfloat16, f"tensors[{i}].param_out", n)
        ptrs = (ctypes.c_void_p * max(M, 1))(*[g.data_ptr() for g in t.grads])
        keep.append(ptrs)
        arr[i] = _CTensor(n, ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)), t.master.data_ptr(),
                          t.exp_avg.data_ptr(), t.exp_avg_sq.data_ptr(), t.param_out.data_ptr())
    return arr, keep, M


def zero_step_workspace_bytes(tensors: Sequence[ZeroTensor], M: int, hp: HParams) -> int:
    arr, keep, _ = _ctensors(tensors, check=False)
    h = hp._c()
    return int(lib().zero_step_workspace_bytes(arr, len(tensors), int(M), ctypes.byref(h)))


def zero_step(tensors: Sequence[ZeroTensor], hp: HParams, external_sumsq: float, ws: Optional[torch.Tensor],
              res: torch.Tensor, stream=None) -> None:
    _need(res, torch.uint8, "res", RESULT_BYTES)
    arr, keep, M = _ctensors(tensors, check=True)
    h = hp._c()
    wsb = _need_ws(ws)
    _check(lib().zero_step(arr, len(tensors), M, ctypes.byref(h), float(external_sumsq), _ptr(ws), wsb,
                           res.data_ptr(), _stream(stream)), "zero_step")


class StepRunner:
    """A tensor list marshalled once, for a training loop that steps it every
    iteration: step() and step_amp() call zero_step and zero_step_amp with
    the pointer tables prepared here, so a call costs one small structure of
    hyperparameters instead of checking every replica of every tensor again
    (about 2 ms of host time per call on a 288-tensor list with 8 replicas).
    The tensors, the workspace and the result record must stay alive and at
    the same addresses."""

    def __init__(self, tensors: Sequence[ZeroTensor], ws: Optional[torch.Tensor], res: torch.Tensor):
        _need(res, torch.uint8, "res", RESULT_BYTES)
        self._arr, self._keep, self.M = _ctensors(tensors, check=True)
        self._tensors = list(tensors)
        self.T = len(self._tensors)
        self.ws, self.res = ws, res
        self._wsp, self._wsb = _ptr(ws), _need_ws(ws)

    def step(self, hp: HParams, external_sumsq: float = 0.0, stream=None) -> None:
        h = hp._c()
        st = lib().zero_step(self._arr, self.T, self.M, ctypes.byref(h), float(external_sumsq), self._wsp, self._wsb,
                             self.res.data_ptr(), _stream(stream))
        if st != ZERO_OK:
            raise ZeroError(st, "zero_step")

    def step_amp(self, hp: HParams, cfg: "LossScaleConfig", ls: torch.Tensor, external_sumsq: float = 0.0,
                 stream=None) -> None:
        h, c = hp._c(), cfg._c()
        st = lib().zero_step_amp(self._arr, self.T, self.M, ctypes.byref(h), ctypes.byref(c), ls.data_ptr(),
                                 float(external_sumsq), self._wsp, self._wsb, self.res.data_ptr(), _stream(stream))
        if st != ZERO_OK:
            raise ZeroError(st, "zero_step_amp")


def zero_step_noalloc(tensors: Sequence[ZeroTensor], hp: HParams, external_sumsq: float, res: torch.Tensor,
                      stream=None) -> None:
    """zero_step with the library's static device scratch as its workspace
    (NOALLOC_SCRATCH_BYTES per GPU): the call allocates nothing. Calls on one
    GPU share the scratch and must be ordered."""
    _need(res, torch.uint8, "res", RESULT_BYTES)
    arr, keep, M = _ctensors(tensors, check=True)
    h = hp._c()
    _check(lib().zero_step_noalloc(arr, len(tensors), M, ctypes.byref(h), float(external_sumsq), res.data_ptr(),
                                   _stream(stream)), "zero_step_noalloc")


@dataclasses.dataclass
class LossScaleConfig:
    """Dynamic loss-scale knobs (names of the fp16 block of a
    deepspeed_config.json; defaults are the values printed there)."""
    initial_scale_power: int = 12
    window: int = 1000
    hysteresis: int = 2
    min_scale: float = 1.0

    def _c(self) -> _CLossScaleConfig:
        return _CLossScaleConfig(int(self.initial_scale_power), int(self.window), int(self.hysteresis),
                                 float(self.min_scale))


def new_loss_scale(device=None) -> torch.Tensor:
    """A 16-byte device buffer for the zero_loss_scale state."""
    return torch.zeros(LOSS_SCALE_BYTES, dtype=torch.uint8, device=device or "cuda")


def read_loss_scale(ls: torch.Tensor) -> dict:
    """Copy the state to the host (synchronizes with its stream)."""
    scale, inv_scale, good_steps, overflows = struct.unpack("<ffii", bytes(ls.cpu().numpy().tobytes()))
    return dict(scale=scale, inv_scale=inv_scale, good_steps=good_steps, overflows=overflows)


def zero_loss_scale_init(cfg: LossScaleConfig, ls: torch.Tensor, stream=None) -> None:
    _need(ls, torch.uint8, "ls", LOSS_SCALE_BYTES)
    c = cfg._c()
    _check(lib().zero_loss_scale_init(ctypes.byref(c), ls.data_ptr(), _stream(stream)), "zero_loss_scale_init")


def zero_loss_scale_update(cfg: LossScaleConfig, res: torch.Tensor, ls: torch.Tensor, stream=None) -> None:
    _need(res, torch.uint8, "res", RESULT_BYTES)
    _need(ls, torch.uint8, "ls", LOSS_SCALE_BYTES)
    c = cfg._c()
    _check(lib().zero_loss_scale_update(ctypes.byref(c), res.data_ptr(), ls.data_ptr(), _stream(stream)),
           "zero_loss_scale_update")


def zero_step_amp_workspace_bytes(tensors: Sequence[ZeroTensor], M: int, hp: HParams) -> int:
    arr, keep, _ = _ctensors(tensors, check=False)
    h = hp._c()
    return int(lib().zero_step_amp_workspace_bytes(arr, len(tensors), int(M), ctypes.byref(h)))


def zero_step_amp(tensors: Sequence[ZeroTensor], hp: HParams, cfg: LossScaleConfig, ls: torch.Tensor,
                  external_sumsq: float, ws: Optional[torch.Tensor], res: torch.Tensor, stream=None) -> None:
    _need(res, torch.uint8, "res", RESULT_BYTES)
    _need(ls, torch.uint8, "ls", LOSS_SCALE_BYTES)
    arr, keep, M = _ctensors(tensors, check=True)
    h = hp._c()
    c = cfg._c()
    wsb = _need_ws(ws)
    _check(lib().zero_step_amp(arr, len(tensors), M, ctypes.byref(h), ctypes.byref(c), ls.data_ptr(),
                               float(external_sumsq), _ptr(ws), wsb, res.data_ptr(), _stream(stream)),
           "zero_step_amp")


# ---------------------------------------------------------------- ZeRO-2 streaming

@dataclasses.dataclass
class GradShard:
    """One tensor shard of a gradient bucket: M bf16 replicas of this
    micro-batch and the shard's fp32 gradient accumulator."""
    grads: List[torch.Tensor]
    grad_acc: torch.Tensor


@dataclasses.dataclass
class AccTensor:
    """One tensor shard of the step from accumulated gradients."""
    grad_acc: torch.Tensor
    master: torch.Tensor
    exp_avg: torch.Tensor
    exp_avg_sq: torch.Tensor
    param_out: torch.Tensor


def new_bucket_partials(nbuckets: int, device=None) -> torch.Tensor:
    """Device storage for nbuckets zero_bucket_partial records (32 bytes each)."""
    return torch.zeros(max(nbuckets, 1) * BUCKET_PARTIAL_BYTES, dtype=torch.uint8, device=device or "cuda")


def read_bucket_partial(partials: torch.Tensor, index: int = 0) -> dict:
    """Copy one bucket partial to the host (synchronizes with its stream)."""
    b = bytes(partials[index * BUCKET_PARTIAL_BYTES:(index + 1) * BUCKET_PARTIAL_BYTES].cpu().numpy().tobytes())
    sumsq, stamp, found_inf, scale, reserved = struct.unpack("<dQifq", b)
    return dict(sumsq=sumsq, stamp=stamp, found_inf=found_inf, grad_scale=scale, reserved=reserved)


def _cshards(shards: Sequence[GradShard], check: bool):
    M = len(shards[0].grads) if shards else 1
    keep = []
    arr = (_CGradShard * max(len(shards), 1))()
    for i, t in enumerate(shards):
        n = t.grad_acc.numel()
        if check:
            if len(t.grads) != M:
                raise ValueError(f"shard {i}: {len(t.grads)} replicas, expected {M}")
            for r, g in enumerate(t.grads):
                _need(g, torch.bfloat16, f"shards[{i}].grads[{r}]", n)
            _need(t.grad_acc, torch.float32, f"shards[{i}].grad_acc", n)
        ptrs = (ctypes.c_void_p * max(M, 1))(*[g.data_ptr() for g in t.grads])
        keep.append(ptrs)
        arr[i] = _CGradShard(n, ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)), t.grad_acc.data_ptr())
    return arr, keep, M


def zero_bucket_reduce_workspace_bytes(shards: Sequence[GradShard], M: int) -> int:
    arr, keep, _ = _cshards(shards, check=False)
    return int(lib().zero_bucket_reduce_workspace_bytes(arr, len(shards), int(M)))


def zero_bucket_reduce(shards: Sequence[GradShard], flags: int, grad_scale: float, stamp: int,
                       partial: Optional[torch.Tensor], ws: Optional[torch.Tensor], stream=None) -> None:
    """partial: a 32-byte slice of new_bucket_partials(...) (this bucket's
    record), required with BUCKET_FINAL."""
    if partial is not None:
        _need(partial, torch.uint8, "partial", BUCKET_PARTIAL_BYTES)
    arr, keep, M = _cshards(shards, check=True)
    wsb = _need_ws(ws)
    _check(lib().zero_bucket_reduce(arr, len(shards), M, int(flags), float(grad_scale), int(stamp) & (2**64 - 1),
                                    _ptr(partial), _ptr(ws), wsb, _stream(stream)), "zero_bucket_reduce")


class BucketReducer:
    """One gradient bucket marshalled once, for a training loop that reduces
    it every micro-batch: reduce() calls zero_bucket_reduce with the arguments
    prepared here and no per-call Python checks. The shards' tensors, the
    partial and the workspace must stay alive and at the same addresses."""

    def __init__(self, shards: Sequence[GradShard], partial: Optional[torch.Tensor], ws: Optional[torch.Tensor] = None,
                 ls: Optional[torch.Tensor] = None):
        self._arr, self._keep, self.M = _cshards(shards, check=True)
        self._shards = list(shards)
        self.T = len(self._shards)
        if partial is not None:
            _need(partial, torch.uint8, "partial", BUCKET_PARTIAL_BYTES)
        self._partial = partial
        if ws is None:
            ws = workspace(zero_bucket_reduce_workspace_bytes(self._shards, self.M))
        self.ws = ws
        self._wsp = _ptr(ws)
        self._wsb = _need_ws(ws)
        self._pp = _ptr(partial)
        if ls is not None:
            _need(ls, torch.uint8, "ls", LOSS_SCALE_BYTES)
        self._ls = ls  # AMP: the dynamic loss scale the final pass reads
        self._fn = lib().zero_bucket_reduce if ls is None else lib().zero_bucket_reduce_amp

    def reduce(self, flags: int, grad_scale: float, stamp: int, stream=None) -> None:
        if self._ls is None:
            st = self._fn(self._arr, self.T, self.M, flags, grad_scale, stamp & 0xFFFFFFFFFFFFFFFF, self._pp,
                          self._wsp, self._wsb, _stream(stream))
        else:
            st = self._fn(self._arr, self.T, self.M, flags, grad_scale, self._ls.data_ptr(),
                          stamp & 0xFFFFFFFFFFFFFFFF, self._pp, self._wsp, self._wsb, _stream(stream))
        if st != ZERO_OK:
            raise ZeroError(st, "zero_bucket_reduce")


def zero_bucket_reduce_amp(shards: Sequence[GradShard], flags: int, grad_scale: float, ls: torch.Tensor, stamp: int,
                           partial: Optional[torch.Tensor], ws: Optional[torch.Tensor], stream=None) -> None:
    _need(ls, torch.uint8, "ls", LOSS_SCALE_BYTES)
    if partial is not None:
        _need(partial, torch.uint8, "partial", BUCKET_PARTIAL_BYTES)
    arr, keep, M = _cshards(shards, check=True)
    wsb = _need_ws(ws)
    _check(lib().zero_bucket_reduce_amp(arr, len(shards), M, int(flags), float(grad_scale), ls.data_ptr(),
                                        int(stamp) & (2**64 - 1), _ptr(partial), _ptr(ws), wsb, _stream(stream)),
           "zero_bucket_reduce_amp")


def _cacc(tensors: Sequence[AccTensor], check: bool):
    arr = (_CAccTensor * max(len(tensors), 1))()
    for i, t in enumerate(tensors):
        n = t.master.numel()
        if check:
            for x, nm in ((t.grad_acc, "grad_acc"), (t.master, "master"), (t.exp_avg, "exp_avg"),
                          (t.exp_avg_sq, "exp_avg_sq")):
                _need(x, torch.float32, f"tensors[{i}].{nm}", n)
            _need(t.param_out, torch.bfloat16, f"tensors[{i}].param_out", n)
        arr[i] = _CAccTensor(n, t.grad_acc.data_ptr(), t.master.data_ptr(), t.exp_avg.data_ptr(),
                             t.exp_avg_sq.data_ptr(), t.param_out.data_ptr())
    return arr


def zero_step_accumulated_workspace_bytes(tensors: Sequence[AccTensor]) -> int:
    return int(lib().zero_step_accumulated_workspace_bytes(_cacc(tensors, check=False), len(tensors)))


def zero_step_accumulated(tensors: Sequence[AccTensor], hp: HParams, partials: Optional[torch.Tensor], nbuckets: int,
                          stamp: int, external_sumsq: float, ws: Optional[torch.Tensor], res: torch.Tensor,
                          stream=None) -> None:
    _need(res, torch.uint8, "res", RESULT_BYTES)
    if nbuckets > 0:
        _need(partials, torch.uint8, "partials")
        if partials.numel() < nbuckets * BUCKET_PARTIAL_BYTES:
            raise ValueError(f"partials: {partials.numel()} bytes for {nbuckets} buckets")
    arr = _cacc(tensors, check=True)
    h = hp._c()
    wsb = _need_ws(ws)
    _check(lib().zero_step_accumulated(arr, len(tensors), ctypes.byref(h), _ptr(partials), int(nbuckets),
                                       int(stamp) & (2**64 - 1), float(external_sumsq), _ptr(ws), wsb,
                                       res.data_ptr(), _stream(stream)), "zero_step_accumulated")


# ---------------------------------------------------------------- ZeRO-2, fused final pass

@dataclasses.dataclass
class BucketTensor:
    """One tensor shard of a bucket's fused final pass: this micro-batch's M
    bf16 replicas, the fp32 accumulator of the earlier micro-batches (read
    with BUCKET_ACCUMULATE; may be None otherwise), the fp32 state (updated in
    place) and the bf16 output shard."""
    grads: List[torch.Tensor]
    grad_acc: Optional[torch.Tensor]
    master: torch.Tensor
    exp_avg: torch.Tensor
    exp_avg_sq: torch.Tensor
    param_out: torch.Tensor


def _cbucket(tensors: Sequence[BucketTensor], check: bool):
    M = len(tensors[0].grads) if tensors else 1
    keep = []
    arr = (_CBucketTensor * max(len(tensors), 1))()
    for i, t in enumerate(tensors):
        n = t.master.numel()
        if check:
            if len(t.grads) != M:
                raise ValueError(f"tensor {i}: {len(t.grads)} replicas, expected {M}")
            for r, g in enumerate(t.grads):
                _need(g, torch.bfloat16, f"tensors[{i}].grads[{r}]", n)
            for x, nm in ((t.master, "master"), (t.exp_avg, "exp_avg"), (t.exp_avg_sq, "exp_avg_sq")):
                _need(x, torch.float32, f"tensors[{i}].{nm}", n)
            if t.grad_acc is not None:
                _need(t.grad_acc, torch.float32, f"tensors[{i}].grad_acc", n)
            _need(t.param_out, torch.bfloat16, f"tensors[{i}].param_out", n)
        ptrs = (ctypes.c_void_p * max(M, 1))(*[g.data_ptr() for g in t.grads])
        keep.append(ptrs)
        arr[i] = _CBucketTensor(n, ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)), _ptr(t.grad_acc),
                                t.master.data_ptr(), t.exp_avg.data_ptr(), t.exp_avg_sq.data_ptr(),
                                t.param_out.data_ptr())
    return arr, keep, M


def zero_bucket_step_workspace_bytes(tensors: Sequence[BucketTensor], M: int) -> int:
    arr, keep, _ = _cbucket(tensors, check=False)
    return int(lib().zero_bucket_step_workspace_bytes(arr, len(tensors), int(M)))


def zero_bucket_step(tensors: Sequence[BucketTensor], flags: int, hp: HParams, stamp: int, partial: torch.Tensor,
                     ws: Optional[torch.Tensor], stream=None) -> None:
    """The final micro-batch of one bucket, folded and applied in one pass
    (no clipping, no skipping); partial: this bucket's 32-byte record."""
    _need(partial, torch.uint8, "partial", BUCKET_PARTIAL_BYTES)
    arr, keep, M = _cbucket(tensors, check=True)
    h = hp._c()
    wsb = _need_ws(ws)
    _check(lib().zero_bucket_step(arr, len(tensors), M, int(flags), ctypes.byref(h), int(stamp) & (2**64 - 1),
                                  partial.data_ptr(), _ptr(ws), wsb, _stream(stream)), "zero_bucket_step")


class BucketStepper:
    """One bucket's fused final pass marshalled once (for a loop that runs it
    every step): step() calls zero_bucket_step with the arguments prepared
    here. The tensors, the partial and the workspace must stay alive and at
    the same addresses."""

    def __init__(self, tensors: Sequence[BucketTensor], partial: torch.Tensor, ws: Optional[torch.Tensor] = None):
        self._arr, self._keep, self.M = _cbucket(tensors, check=True)
        self._tensors = list(tensors)
        self.T = len(self._tensors)
        _need(partial, torch.uint8, "partial", BUCKET_PARTIAL_BYTES)
        self._partial = partial
        if ws is None:
            ws = workspace(zero_bucket_step_workspace_bytes(self._tensors, self.M))
        self.ws = ws
        self._wsp, self._wsb = _ptr(ws), _need_ws(ws)

    def step(self, flags: int, hp: HParams, stamp: int, stream=None) -> None:
        h = hp._c()
        st = lib().zero_bucket_step(self._arr, self.T, self.M, flags, ctypes.byref(h), stamp & 0xFFFFFFFFFFFFFFFF,
                                    self._partial.data_ptr(), self._wsp, self._wsb, _stream(stream))
        if st != ZERO_OK:
            raise ZeroError(st, "zero_bucket_step")


# ---------------------------------------------------------------- CPU-offloaded step

@dataclasses.dataclass
class OffloadTensor:
    """One tensor shard of an offloaded step: M bf16 replicas (device), the
    fp32 master/exp_avg/exp_avg_sq in host memory (updated in place) and the
    bf16 output shard (device)."""
    grads: List[torch.Tensor]
    master: torch.Tensor
    exp_avg: torch.Tensor
    exp_avg_sq: torch.Tensor
    param_out: torch.Tensor


def _need_host(t: torch.Tensor, dtype, name: str, n: Optional[int] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device.type != "cpu":
        raise ValueError(f"{name}: must be a host tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if n is not None and t.numel() != n:
        raise ValueError(f"{name}: expected {n} elements, got {t.numel()}")


def _coffload(tensors: Sequence[OffloadTensor], check: bool):
    M = len(tensors[0].grads) if tensors else 1
    keep = []
    arr = (_COffloadTensor * max(len(tensors), 1))()
    for i, t in enumerate(tensors):
        n = t.master.numel()
        if check:
            if len(t.grads) != M:
                raise ValueError(f"tensor {i}: {len(t.grads)} replicas, expected {M}")
            for r, g in enumerate(t.grads):
                _need(g, torch.bfloat16, f"tensors[{i}].grads[{r}]", n)
            for x, nm in ((t.master, "master"), (t.exp_avg, "exp_avg"), (t.exp_avg_sq, "exp_avg_sq")):
                _need_host(x, torch.float32, f"tensors[{i}].{nm}", n)
            _need(t.param_out, torch.bfloat16, f"tensors[{i}].param_out", n)
        ptrs = (ctypes.c_void_p * max(M, 1))(*[g.data_ptr() for g in t.grads])
        keep.append(ptrs)
        arr[i] = _COffloadTensor(n, ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)), t.master.data_ptr(),
                                 t.exp_avg.data_ptr(), t.exp_avg_sq.data_ptr(), t.param_out.data_ptr())
    return arr, keep, M


def zero_offload_workspace_bytes(tensors: Sequence[OffloadTensor], M: int) -> int:
    arr, keep, _ = _coffload(tensors, check=False)
    return int(lib().zero_offload_workspace_bytes(arr, len(tensors), int(M)))


def zero_offload_host_workspace_bytes(tensors: Sequence[OffloadTensor]) -> int:
    arr, keep, _ = _coffload(tensors, check=False)
    return int(lib().zero_offload_host_workspace_bytes(arr, len(tensors)))


def host_workspace(nbytes: int) -> torch.Tensor:
    """Pinned host memory of nbytes (page-aligned), for zero_offload_step."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, pin_memory=True)


def zero_offload_step(tensors: Sequence[OffloadTensor], hp: HParams, external_sumsq: float, ws: torch.Tensor,
                      host_ws: torch.Tensor, threads: int = 0, stream=None) -> dict:
    """Returns the result record (the call reads it on the host)."""
    _need(ws, torch.uint8, "ws")
    _need_host(host_ws, torch.uint8, "host_ws")
    if not host_ws.is_pinned():
        raise ValueError("host_ws: must be pinned host memory (host_workspace())")
    arr, keep, M = _coffload(tensors, check=True)
    h = hp._c()
    r = _CResult()
    _check(lib().zero_offload_step(arr, len(tensors), M, ctypes.byref(h), float(external_sumsq), ws.data_ptr(),
                                   ws.numel(), host_ws.data_ptr(), host_ws.numel(), ctypes.byref(r), int(threads),
                                   _stream(stream)), "zero_offload_step")
    return dict(sumsq=r.sumsq, grad_norm=r.grad_norm, clip_coef=r.clip_coef, found_inf=r.found_inf,
                skipped=r.skipped, status=r.status)


def zero_offload_adamw_host(master: torch.Tensor, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor, g: torch.Tensor,
                            param_out: torch.Tensor, hp: HParams, clip_coef: float = 1.0, threads: int = 0) -> None:
    """The host half of the offloaded step on host tensors (fp32 state and
    gradient, bf16 output)."""
    n = master.numel()
    for t, nm in ((master, "master"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"), (g, "g")):
        _need_host(t, torch.float32, nm, n)
    _need_host(param_out, torch.bfloat16, "param_out", n)
    h = hp._c()
    _check(lib().zero_offload_adamw_host(master.data_ptr(), exp_avg.data_ptr(), exp_avg_sq.data_ptr(), g.data_ptr(),
                                         param_out.data_ptr(), n, ctypes.byref(h), float(clip_coef), int(threads)),
           "zero_offload_adamw_host")


def zero_step_accumulated_amp(tensors: Sequence[AccTensor], hp: HParams, cfg: "LossScaleConfig", ls: torch.Tensor,
                              partials: Optional[torch.Tensor], nbuckets: int, stamp: int, external_sumsq: float,
                              ws: Optional[torch.Tensor], res: torch.Tensor, stream=None) -> None:
    _need(res, torch.uint8, "res", RESULT_BYTES)
    _need(ls, torch.uint8, "ls", LOSS_SCALE_BYTES)
    if nbuckets > 0:
        _need(partials, torch.uint8, "partials")
        if partials.numel() < nbuckets * BUCKET_PARTIAL_BYTES:
            raise ValueError(f"partials: {partials.numel()} bytes for {nbuckets} buckets")
    arr = _cacc(tensors, check=True)
    h = hp._c()
    c = cfg._c()
    wsb = _need_ws(ws)
    _check(lib().zero_step_accumulated_amp(arr, len(tensors), ctypes.byref(h), ctypes.byref(c), ls.data_ptr(),
                                           _ptr(partials), int(nbuckets), int(stamp) & (2**64 - 1),
                                           float(external_sumsq), _ptr(ws), wsb, res.data_ptr(), _stream(stream)),
           "zero_step_accumulated_amp")


def zero_offload_step_amp(tensors: Sequence[OffloadTensor], hp: HParams, cfg: "LossScaleConfig", ls: torch.Tensor,
                          external_sumsq: float, ws: torch.Tensor, host_ws: torch.Tensor, threads: int = 0,
                          stream=None) -> dict:
    _need(ws, torch.uint8, "ws")
    _need_host(host_ws, torch.uint8, "host_ws")
    if not host_ws.is_pinned():
        raise ValueError("host_ws: must be pinned host memory (host_workspace())")
    _need(ls, torch.uint8, "ls", LOSS_SCALE_BYTES)
    arr, keep, M = _coffload(tensors, check=True)
    h = hp._c()
    c = cfg._c()
    r = _CResult()
    _check(lib().zero_offload_step_amp(arr, len(tensors), M, ctypes.byref(h), ctypes.byref(c), ls.data_ptr(),
                                       float(external_sumsq), ws.data_ptr(), ws.numel(), host_ws.data_ptr(),
                                       host_ws.numel(), ctypes.byref(r), int(threads), _stream(stream)),
           "zero_offload_step_amp")
    return dict(sumsq=r.sumsq, grad_norm=r.grad_norm, clip_coef=r.clip_coef, found_inf=r.found_inf,
                skipped=r.skipped, status=r.status)


def zero_workspace_forget(ws: torch.Tensor) -> None:
    _check(lib().zero_workspace_forget(ws.data_ptr()), "zero_workspace_forget")


def workspace(nbytes: int, device=None) -> Optional[torch.Tensor]:
    """A device workspace of nbytes (torch allocations are 256-byte aligned).
    When the tensor is freed, the library forgets any plan it cached there:
    the allocator may hand the same memory out again for something else."""
    if nbytes <= 0:
        return None
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device or "cuda")
    weakref.finalize(ws, _forget_ptr, ws.data_ptr())
    return ws


def _forget_ptr(ptr: int) -> None:
    if _lib is not None:
        _lib.zero_workspace_forget(ptr)


def zero_step_workspace_bytes_for_sizes(sizes: Sequence[int], M: int, hp: HParams) -> int:
    """Workspace size of a zero_step over shards of these lengths (no tensors needed)."""
    arr = (_CTensor * max(len(sizes), 1))()
    for i, n in enumerate(sizes):
        arr[i] = _CTensor(int(n), None, None, None, None, None)
    h = hp._c()
    return int(lib().zero_step_workspace_bytes(arr, len(sizes), int(M), ctypes.byref(h)))
