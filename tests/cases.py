"""Builders shared by the GPU tests: one seeded case, materialised twice --
on the device by the GPU generator and on the host by the host generator --
plus the comparison rules of the parity gates."""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np
import torch

import oracle
import sharded_optimizer_step_amd as z
import synth

K = synth


@dataclasses.dataclass
class Case:
    sizes: Sequence[int]
    M: int
    seed: int = 5
    grad_std: float = 1e-3
    master_std: float = 0.02
    m_std: float = 1e-5
    v_std: float = 1e-8
    offsets: Optional[Sequence[Sequence[int]]] = None  # per tensor: element offsets of [grads..., master, m, v, out]
    zero_state: bool = False


def _buf(n, off, dtype, dev):
    base = torch.empty(n + off + 8, dtype=dtype, device=dev)
    return base[off:off + n]


def build(case: Case, dev="cuda"):
    """Returns (device ZeroTensors, host oracle TensorStates)."""
    dts, hts = [], []
    for t, n in enumerate(case.sizes):
        offs = case.offsets[t] if case.offsets is not None else [0] * (case.M + 4)
        grads = []
        hgrads = []
        for r in range(case.M):
            st = K.stream_id(K.KIND_GRAD, t, r)
            g = _buf(n, offs[r], torch.bfloat16, dev)
            if n:
                K.device_bf16(g, case.seed, st, case.grad_std)
            grads.append(g)
            hgrads.append(K.host_bf16(n, case.seed, st, case.grad_std))
        state_d, state_h = [], []
        for j, (kind, std, ab) in enumerate(((K.KIND_MASTER, case.master_std, False),
                                             (K.KIND_EXP_AVG, case.m_std, False),
                                             (K.KIND_EXP_AVG_SQ, case.v_std, True))):
            x = _buf(n, offs[case.M + j], torch.float32, dev)
            st = K.stream_id(kind, t, 0)
            if case.zero_state and kind != K.KIND_MASTER:
                x.zero_()
                h = np.zeros(n, np.float32)
            else:
                if n:
                    K.device_f32(x, case.seed, st, std, absval=ab)
                h = K.host_f32(n, case.seed, st, std, absval=ab)
            state_d.append(x)
            state_h.append(h)
        out = _buf(n, offs[case.M + 3], torch.bfloat16, dev)
        out.view(torch.int16).fill_(0x1234)
        dts.append(z.ZeroTensor(grads, state_d[0], state_d[1], state_d[2], out))
        hts.append(oracle.TensorState(hgrads, state_h[0], state_h[1], state_h[2], np.full(n, 0x1234, np.uint16)))
    return dts, hts


def to_np_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def to_np_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def ordered16(u: np.ndarray) -> np.ndarray:
    """bf16 codes as integers whose order is the order of the values."""
    u = u.astype(np.int64)
    return np.where(u >= 0x8000, 0x8000 - u, u)


def ordered32(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.int64)
    return np.where(u >= 2**31, 2**31 - u, u)


def hp_oracle(hp: z.HParams) -> oracle.HParams:
    return oracle.HParams(lr=hp.lr, beta1=hp.beta1, beta2=hp.beta2, eps=hp.eps, weight_decay=hp.weight_decay,
                          step=hp.step, max_grad_norm=hp.max_grad_norm, grad_scale=hp.grad_scale,
                          skip_on_nonfinite=hp.skip_on_nonfinite)


@dataclasses.dataclass
class Stats:
    max_rel: dict = dataclasses.field(default_factory=dict)
    max_ulp: dict = dataclasses.field(default_factory=dict)


def assert_state_matches(got_master, got_m, got_v, got_out, want_master, want_m, want_v, want_out, where="",
                         stats: Optional[Stats] = None):
    """The parity gate of the fp32 state and the bf16 emit:
    |d| <= max(2e-6 |ref|, 1e-7) on master, m, v; <= 1 bf16 ulp on out."""
    for name, got, want in (("master", got_master, want_master), ("exp_avg", got_m, want_m),
                            ("exp_avg_sq", got_v, want_v)):
        g = got.astype(np.float64)
        w = want.astype(np.float64)
        both_nan = np.isnan(g) & np.isnan(w)
        same = both_nan | (g == w)  # NaN in both, or equal values (infinities included)
        with np.errstate(invalid="ignore"):
            err = np.where(same, 0.0, np.abs(g - w))
        tol = np.maximum(2e-6 * np.abs(w), 1e-7)
        bad = ~same & ~(err <= tol)
        if bad.any():
            i = int(np.flatnonzero(bad)[0])
            raise AssertionError(f"{where} {name}[{i}]: got {got[i]!r} want {want[i]!r} "
                                 f"({int(bad.sum())} of {bad.size} outside the gate)")
        if stats is not None:
            nz = (np.abs(w) > 0) & ~both_nan
            rel = float(np.max(err[nz] / np.abs(w[nz]))) if nz.any() else 0.0
            ulp = int(np.max(np.abs(ordered32(got) - ordered32(want))[~both_nan])) if (~both_nan).any() else 0
            stats.max_rel[name] = max(stats.max_rel.get(name, 0.0), rel)
            stats.max_ulp[name] = max(stats.max_ulp.get(name, 0), ulp)
    nanw = (want_out & 0x7F80) == 0x7F80
    nanw &= (want_out & 0x7F) != 0
    nang = ((got_out & 0x7F80) == 0x7F80) & ((got_out & 0x7F) != 0)
    assert np.array_equal(nanw, nang), f"{where} out: NaN positions differ"
    d = np.abs(ordered16(got_out) - ordered16(want_out))[~nanw]
    if d.size and d.max() > 1:
        i = int(np.flatnonzero(~nanw)[int(np.argmax(d))])
        raise AssertionError(f"{where} out[{i}]: got {got_out[i]:#06x} want {want_out[i]:#06x}")
    if stats is not None and d.size:
        stats.max_ulp["out"] = max(stats.max_ulp.get("out", 0), int(d.max()))


def assert_tensor_matches(dt: z.ZeroTensor, ht: oracle.TensorState, where="", stats=None):
    assert_state_matches(to_np_f32(dt.master), to_np_f32(dt.exp_avg), to_np_f32(dt.exp_avg_sq),
                         to_np_u16(dt.param_out), ht.master, ht.exp_avg, ht.exp_avg_sq, ht.param_out, where, stats)


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    return np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8))


def run_step(dts: List[z.ZeroTensor], hp: z.HParams, external: float = 0.0, ws=None):
    if ws is None:
        ws = z.workspace(z.zero_step_workspace_bytes(dts, len(dts[0].grads), hp))
    res = z.new_result()
    z.zero_step(dts, hp, external, ws, res)
    return z.read_result(res), ws


# ---------------------------------------------------------------- full-size workloads

def sample_indices(n: int, rng, k: int = 40_000) -> np.ndarray:
    """Sorted unique indices: both ends, around 2048- and 65536-element tile
    boundaries, and uniform random ones."""
    parts = [np.arange(min(n, 4096)), np.arange(max(0, n - 4096), n)]
    for step in (2048, 65536):
        b = np.arange(step, n, step * max(1, n // (step * 200)))
        parts.append(np.clip(np.concatenate([b - 9, b - 1, b, b + 7]), 0, n - 1))
    parts.append(rng.integers(0, n, k))
    return np.unique(np.concatenate(parts).astype(np.int64))


def host_inputs_at(w, spec, idx: np.ndarray):
    """Host copies of the workload's inputs at shard-local indices idx."""
    g = idx + spec.start
    st = lambda k, r=0: synth.stream_id(k, spec.tensor_id, r)
    grads = [synth.host_bf16_at(g, w.seed, st(synth.KIND_GRAD, r), w.grad_std) for r in range(w.M)]
    master = synth.host_f32_at(g, w.seed, st(synth.KIND_MASTER), w.master_std)
    m = synth.host_f32_at(g, w.seed, st(synth.KIND_EXP_AVG), w.m_std) if w.m_std else np.zeros(idx.size, np.float32)
    v = synth.host_f32_at(g, w.seed, st(synth.KIND_EXP_AVG_SQ), w.v_std, absval=True) if w.v_std else \
        np.zeros(idx.size, np.float32)
    return grads, master, m, v


def oracle_sumsq_streaming(w, slice_elems: int = 1 << 22, workers: int = 16, inject=()):
    """The oracle's sum of squares and non-finite flag over the whole workload,
    regenerating the inputs on the host slice by slice (bounded memory). Slice
    partials are combined in index order. `inject` lists (tensor, rank, index)
    elements set to +inf."""
    from concurrent.futures import ThreadPoolExecutor
    jobs = []
    for ti, spec in enumerate(w.tensors):
        for s0 in range(0, spec.n, slice_elems):
            jobs.append((ti, s0, min(spec.n, s0 + slice_elems)))
    inj = {}
    for (t, r, i) in inject:
        inj.setdefault(t, []).append((r, i))

    def one(job):
        ti, s0, s1 = job
        spec = w.tensors[ti]
        grads = [synth.host_bf16(s1 - s0, w.seed, synth.stream_id(synth.KIND_GRAD, spec.tensor_id, r), w.grad_std,
                                 start=spec.start + s0) for r in range(w.M)]
        for r, i in inj.get(ti, []):
            if s0 <= i < s1:
                grads[r][i - s0] = 0x7F80
        g = oracle.reduce(grads, w.grad_scale)
        return oracle.check(g)

    with ThreadPoolExecutor(max_workers=workers) as ex:
        res = list(ex.map(one, jobs))
    total, bad = 0.0, 0
    for s, f in res:
        total += s
        bad |= f
    return total, bad
