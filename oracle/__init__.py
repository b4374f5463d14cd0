"""CPU oracle for the per-rank ZeRO-1 shard step (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The HIP library and its Python binding
never import it, and the two share no code.

The arithmetic lives in ``zero_oracle.c`` (plain sequential loops, binary32 for
the rank fold that the step defines in binary32, binary64 elsewhere); this file
only marshals numpy arrays through ctypes. See the header of ``zero_oracle.c``
for the step, its order and the passages of the pages each part follows.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "zero_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libzero_oracle.so")
_CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]
# Path of an already built copy of the oracle to load instead of this one. The
# mutation check of the pins sets it in a child process to a copy built from a
# deliberately broken source; nothing else does.
_OVERRIDE_ENV = "ZERO_ORACLE_LIB_OVERRIDE"


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no GPU code involved)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm", "-pthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double), ("step", ctypes.c_int64),
                ("max_grad_norm", ctypes.c_double), ("grad_scale", ctypes.c_double),
                ("skip_on_nonfinite", ctypes.c_int32)]


class _Result(ctypes.Structure):
    _fields_ = [("sumsq", ctypes.c_double), ("grad_norm", ctypes.c_double), ("clip_coef", ctypes.c_double),
                ("found_inf", ctypes.c_int32), ("skipped", ctypes.c_int32)]


class _Tensor(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("grads", ctypes.POINTER(ctypes.c_void_p)),
                ("master", ctypes.c_void_p), ("exp_avg", ctypes.c_void_p), ("exp_avg_sq", ctypes.c_void_p),
                ("param_out", ctypes.c_void_p)]


class _AccTensor(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("grad_acc", ctypes.c_void_p), ("master", ctypes.c_void_p),
                ("exp_avg", ctypes.c_void_p), ("exp_avg_sq", ctypes.c_void_p), ("param_out", ctypes.c_void_p)]


class _LossScale(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_float), ("inv_scale", ctypes.c_float), ("good_steps", ctypes.c_int32),
                ("overflows", ctypes.c_int32)]


class _LossScaleConfig(ctypes.Structure):
    _fields_ = [("initial_scale_power", ctypes.c_int32), ("window", ctypes.c_int32),
                ("hysteresis", ctypes.c_int32), ("min_scale", ctypes.c_float)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get(_OVERRIDE_ENV) or build()
        L = ctypes.CDLL(path)
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        L.oracle_bf16_to_f32.argtypes = [vp, vp, i64]
        L.oracle_f32_to_bf16.argtypes = [vp, vp, i64]
        L.oracle_reduce.argtypes = [ctypes.POINTER(vp), i32, i64, dbl, vp]
        L.oracle_check.argtypes = [vp, i64, ctypes.POINTER(dbl), ctypes.POINTER(dbl), ctypes.POINTER(i32)]
        L.oracle_sumsq_total.argtypes = [dbl, dbl]
        L.oracle_sumsq_total.restype = dbl
        L.oracle_finalize.argtypes = [dbl, dbl, i32, dbl, i32, ctypes.POINTER(_Result)]
        L.oracle_adamw.argtypes = [vp, vp, vp, vp, vp, i64, ctypes.POINTER(_Hparams), dbl]
        L.oracle_zero_step.argtypes = [ctypes.POINTER(_Tensor), i32, i32, ctypes.POINTER(_Hparams), dbl,
                                       ctypes.POINTER(_Result)]
        L.oracle_zero_step.restype = i32
        L.oracle_grad_accumulate.argtypes = [ctypes.POINTER(vp), i32, i64, vp, i32]
        L.oracle_grad_accumulate.restype = None
        L.oracle_zero_step_accumulated.argtypes = [ctypes.POINTER(_AccTensor), i32, ctypes.POINTER(_Hparams), dbl,
                                                   ctypes.POINTER(_Result)]
        L.oracle_zero_step_accumulated.restype = i32
        L.oracle_loss_scale_init.argtypes = [ctypes.POINTER(_LossScaleConfig), ctypes.POINTER(_LossScale)]
        L.oracle_loss_scale_update.argtypes = [ctypes.POINTER(_LossScaleConfig), i32, ctypes.POINTER(_LossScale)]
        L.oracle_loss_scale_init.restype = None
        L.oracle_loss_scale_update.restype = None
        for f in ("oracle_bf16_to_f32", "oracle_f32_to_bf16", "oracle_reduce", "oracle_check",
                  "oracle_finalize", "oracle_adamw"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


@dataclasses.dataclass
class HParams:
    """AdamW knobs named as in the optimizer block of a deepspeed_config.json
    ([5D post] 4.2), plus the step index, the clip threshold, the AMP gradient
    multiplier and the skip switch."""
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1
    step: int = 1
    max_grad_norm: float = 0.0
    grad_scale: float = 1.0
    skip_on_nonfinite: int = 0

    def _c(self) -> _Hparams:
        return _Hparams(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay, int(self.step),
                        self.max_grad_norm, self.grad_scale, int(self.skip_on_nonfinite))


@dataclasses.dataclass
class Result:
    sumsq: float
    grad_norm: float
    clip_coef: float
    found_inf: int
    skipped: int


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.float32, a.dtype
    return a


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


def bf16_to_f32(h) -> np.ndarray:
    h = _u16(h)
    out = np.empty(h.shape, np.float32)
    lib().oracle_bf16_to_f32(_p(h), _p(out), h.size)
    return out


def f32_to_bf16(x) -> np.ndarray:
    x = _f32(x)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_f32_to_bf16(_p(x), _p(out), x.size)
    return out


def reduce(grads: Sequence[np.ndarray], grad_scale: float = 1.0) -> np.ndarray:
    """Ascending-rank binary32 fold of M bf16 replicas, times scale32."""
    gs = [_u16(g) for g in grads]
    n = gs[0].size
    assert all(g.size == n for g in gs)
    ptrs = (ctypes.c_void_p * len(gs))(*[_p(g) for g in gs])
    out = np.empty(n, np.float32)
    lib().oracle_reduce(ptrs, len(gs), n, float(grad_scale), _p(out))
    return out


class SumSq:
    """A running sum of squares and non-finite flag over slices taken in
    index order: the compensated pair of zero_oracle.c's step 3, so that
    chaining slices gives exactly what one call over their concatenation
    gives."""

    def __init__(self, sumsq: float = 0.0, found_inf: int = 0):
        self._s = ctypes.c_double(sumsq)
        self._c = ctypes.c_double(0.0)
        self._f = ctypes.c_int32(found_inf)

    def add(self, g) -> "SumSq":
        g = _f32(g)
        lib().oracle_check(_p(g), g.size, ctypes.byref(self._s), ctypes.byref(self._c), ctypes.byref(self._f))
        return self

    @property
    def sumsq(self) -> float:
        return lib().oracle_sumsq_total(self._s.value, self._c.value)

    @property
    def found_inf(self) -> int:
        return self._f.value


def check(g, sumsq: float = 0.0, found_inf: int = 0):
    """(sum of squares, non-finite flag) of g, continuing from a plain sum
    sumsq and a flag (use SumSq to chain slices exactly)."""
    st = SumSq(sumsq, found_inf).add(g)
    return st.sumsq, st.found_inf


def finalize(sumsq: float, external_sumsq: float, found_inf: int, max_grad_norm: float,
             skip_on_nonfinite: int) -> Result:
    r = _Result()
    lib().oracle_finalize(sumsq, external_sumsq, int(found_inf), max_grad_norm, int(skip_on_nonfinite),
                          ctypes.byref(r))
    return Result(r.sumsq, r.grad_norm, r.clip_coef, r.found_inf, r.skipped)


def adamw(master, exp_avg, exp_avg_sq, g, hp: HParams, coef: float = 1.0):
    """Returns new (master, exp_avg, exp_avg_sq, param_out); inputs untouched."""
    th, m, v = _f32(master).copy(), _f32(exp_avg).copy(), _f32(exp_avg_sq).copy()
    g = _f32(g)
    out = np.empty(th.shape, np.uint16)
    h = hp._c()
    lib().oracle_adamw(_p(th), _p(m), _p(v), _p(g), _p(out), th.size, ctypes.byref(h), float(coef))
    return th, m, v, out


@dataclasses.dataclass
class TensorState:
    grads: list          # M arrays of uint16 (bf16 bits)
    master: np.ndarray   # float32
    exp_avg: np.ndarray  # float32
    exp_avg_sq: np.ndarray  # float32
    param_out: np.ndarray | None = None  # uint16; left as given on a skipped step


def zero_step(tensors: Sequence[TensorState], hp: HParams, external_sumsq: float = 0.0):
    """The whole step over a tensor list. Returns (new TensorStates, Result).
    The inputs are not modified; a skipped step returns copies of the old state."""
    T = len(tensors)
    M = len(tensors[0].grads)
    keep = []
    cts = (_Tensor * max(T, 1))()
    new = []
    for i, t in enumerate(tensors):
        gs = [_u16(g) for g in t.grads]
        assert len(gs) == M
        n = t.master.size
        st = TensorState(gs, _f32(t.master).copy(), _f32(t.exp_avg).copy(), _f32(t.exp_avg_sq).copy(),
                         (_u16(t.param_out).copy() if t.param_out is not None else np.zeros(n, np.uint16)))
        ptrs = (ctypes.c_void_p * M)(*[_p(g) for g in gs])
        keep.append(ptrs)
        cts[i] = _Tensor(n, ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)), _p(st.master), _p(st.exp_avg),
                         _p(st.exp_avg_sq), _p(st.param_out))
        new.append(st)
    h = hp._c()
    r = _Result()
    rc = lib().oracle_zero_step(cts, T, M, ctypes.byref(h), float(external_sumsq), ctypes.byref(r))
    if rc != 0:
        raise MemoryError("oracle_zero_step: out of host memory")
    return new, Result(r.sumsq, r.grad_norm, r.clip_coef, r.found_inf, r.skipped)


# --------------------------------------------------------------------------
# ZeRO-2 streaming (see the header of zero_oracle.c): each bucket's replicas
# are folded into an fp32 shard accumulator as they arrive, micro-batch after
# micro-batch; the step then runs on g = acc * scale32.
# --------------------------------------------------------------------------

def grad_accumulate(grads: Sequence[np.ndarray], acc: np.ndarray | None = None) -> np.ndarray:
    """One micro-batch of one tensor: the binary32 fold of its M bf16
    replicas, stored (acc None) or added to a copy of acc. Returns the new
    accumulator; acc is not modified."""
    gs = [_u16(g) for g in grads]
    n = gs[0].size
    assert all(g.size == n for g in gs)
    ptrs = (ctypes.c_void_p * len(gs))(*[_p(g) for g in gs])
    out = np.empty(n, np.float32) if acc is None else _f32(acc).copy()
    assert out.size == n
    lib().oracle_grad_accumulate(ptrs, len(gs), n, _p(out), 0 if acc is None else 1)
    return out


def zero_step_accumulated(accs: Sequence[np.ndarray], tensors: Sequence[TensorState], hp: HParams,
                          external_sumsq: float = 0.0):
    """The step from accumulated fp32 shard gradients accs[t] (the grads of
    `tensors` are not read). Returns (new TensorStates, Result); the inputs are
    not modified, and a skipped step returns copies of the old state."""
    T = len(tensors)
    assert len(accs) == T
    cts = (_AccTensor * max(T, 1))()
    new = []
    keep = []
    for i, (a, t) in enumerate(zip(accs, tensors)):
        a = _f32(a)
        n = t.master.size
        assert a.size == n
        st = TensorState([], _f32(t.master).copy(), _f32(t.exp_avg).copy(), _f32(t.exp_avg_sq).copy(),
                         (_u16(t.param_out).copy() if t.param_out is not None else np.zeros(n, np.uint16)))
        keep.append(a)
        cts[i] = _AccTensor(n, _p(a), _p(st.master), _p(st.exp_avg), _p(st.exp_avg_sq), _p(st.param_out))
        new.append(st)
    h = hp._c()
    r = _Result()
    rc = lib().oracle_zero_step_accumulated(cts, T, ctypes.byref(h), float(external_sumsq), ctypes.byref(r))
    if rc != 0:
        raise MemoryError("oracle_zero_step_accumulated: out of host memory")
    return new, Result(r.sumsq, r.grad_norm, r.clip_coef, r.found_inf, r.skipped)


# --------------------------------------------------------------------------
# Dynamic loss scale (see oracle_loss_scale_update in zero_oracle.c for the
# rule and the passages it reads).
# --------------------------------------------------------------------------

@dataclasses.dataclass
class LossScaleConfig:
    initial_scale_power: int = 12
    window: int = 1000
    hysteresis: int = 2
    min_scale: float = 1.0

    def _c(self) -> _LossScaleConfig:
        return _LossScaleConfig(self.initial_scale_power, self.window, self.hysteresis, self.min_scale)


@dataclasses.dataclass(frozen=True)
class LossScale:
    scale: float
    inv_scale: float
    good_steps: int = 0
    overflows: int = 0

    def _c(self) -> _LossScale:
        return _LossScale(self.scale, self.inv_scale, self.good_steps, self.overflows)


def _ls(c: _LossScale) -> LossScale:
    return LossScale(c.scale, c.inv_scale, c.good_steps, c.overflows)


def loss_scale_init(cfg: LossScaleConfig) -> LossScale:
    c = _LossScale()
    lib().oracle_loss_scale_init(ctypes.byref(cfg._c()), ctypes.byref(c))
    return _ls(c)


def loss_scale_update(state: LossScale, cfg: LossScaleConfig, found_inf: int) -> LossScale:
    c = state._c()
    lib().oracle_loss_scale_update(ctypes.byref(cfg._c()), int(bool(found_inf)), ctypes.byref(c))
    return _ls(c)


def zero_step_amp(tensors: Sequence[TensorState], hp: HParams, cfg: LossScaleConfig, state: LossScale,
                  external_sumsq: float = 0.0):
    """One AMP step with a dynamic loss scale: the fp32 sum is multiplied by
    grad_scale x inv_scale (a binary32 product), a step with a non-finite
    gradient is skipped, then the scale moves on the step's flag.
    Returns (new TensorStates, Result, new LossScale)."""
    mult = float(np.float32(hp.grad_scale) * np.float32(state.inv_scale))
    h = dataclasses.replace(hp, grad_scale=mult, skip_on_nonfinite=1)
    new, res = zero_step(tensors, h, external_sumsq)
    return new, res, loss_scale_update(state, cfg, res.found_inf)


def zero_step_accumulated_amp(accs: Sequence[np.ndarray], tensors: Sequence[TensorState], hp: HParams,
                              cfg: LossScaleConfig, state: LossScale, external_sumsq: float = 0.0):
    """The ZeRO-2 step from accumulated gradients under a dynamic loss scale:
    the multiplier is grad_scale x inv_scale (a binary32 product), a step with
    a non-finite gradient is skipped, then the scale moves on the step's flag.
    Returns (new TensorStates, Result, new LossScale)."""
    mult = float(np.float32(hp.grad_scale) * np.float32(state.inv_scale))
    h = dataclasses.replace(hp, grad_scale=mult, skip_on_nonfinite=1)
    new, res = zero_step_accumulated(accs, tensors, h, external_sumsq)
    return new, res, loss_scale_update(state, cfg, res.found_inf)


# --------------------------------------------------------------------------
# Memory accounting of mixed-precision AdamW training state
# ([CS336 L7] "训练内存的详细分析": bf16 parameter 2 B, bf16 gradient 2 B,
# fp32 master 4 B, fp32 first moment 4 B, fp32 second moment 4 B per
# parameter; [ZeRO ch.] 2.3.4 and [CS336 L7] "ZeRO Stage 1": the optimizer
# state -- master, m, v -- is split 1/N across the N data-parallel ranks).
# --------------------------------------------------------------------------

BYTES_PER_PARAM = {"param_bf16": 2, "grad_bf16": 2, "master_fp32": 4, "exp_avg_fp32": 4, "exp_avg_sq_fp32": 4}


def bytes_per_param_naive_dp() -> int:
    return sum(BYTES_PER_PARAM.values())


def bytes_per_gpu(n_params: float, n_ranks: int, stage: int) -> float:
    """Per-GPU bytes of the training state for naive DP (stage 0) or ZeRO
    stages 1-3 over n_ranks data-parallel ranks (activations excluded)."""
    p = BYTES_PER_PARAM["param_bf16"]
    g = BYTES_PER_PARAM["grad_bf16"]
    opt = BYTES_PER_PARAM["master_fp32"] + BYTES_PER_PARAM["exp_avg_fp32"] + BYTES_PER_PARAM["exp_avg_sq_fp32"]
    if stage == 0:
        per = p + g + opt
    elif stage == 1:
        per = p + g + opt / n_ranks
    elif stage == 2:
        per = p + (g + opt) / n_ranks
    elif stage == 3:
        per = (p + g + opt) / n_ranks
    else:
        raise ValueError(stage)
    return n_params * per
