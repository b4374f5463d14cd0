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
    """Per field: the largest relative error with no floor (elements whose
    reference is nonzero), the largest distance in binary32 (bf16 for out)
    units in the last place, the elements compared, and the elements let off
    the ulp gate because the update cancels there (see coef_sensitive)."""
    max_rel: dict = dataclasses.field(default_factory=dict)
    max_ulp: dict = dataclasses.field(default_factory=dict)
    elements: int = 0
    ulp_exempt: int = 0

    def merge(self, o: "Stats") -> None:
        for k, x in o.max_rel.items():
            self.max_rel[k] = max(self.max_rel.get(k, 0.0), x)
        for k, x in o.max_ulp.items():
            self.max_ulp[k] = max(self.max_ulp.get(k, 0), x)
        self.elements += o.elements
        self.ulp_exempt += o.ulp_exempt

    def as_dict(self) -> dict:
        return dict(elements=self.elements, max_rel_no_floor={k: float(f"{x:.3g}") for k, x in self.max_rel.items()},
                    max_ulp=dict(self.max_ulp), ulp_exempt=self.ulp_exempt)


# Largest distance, in binary32 units in the last place, allowed between the
# device's master, m and v and the oracle's. Both evaluate the same binary64
# AdamW formula on the same binary32 inputs and round once, so they agree
# bit for bit unless the clip coefficients differ in their last bits (two
# correctly rounded sums of squares taken in different orders).
ULP_GATE = 4


def ulp_gate(*records):
    """ULP_GATE when the device and the oracle took bit-identical clip
    coefficients in every step given -- records are pairs (device record dict,
    oracle Result) -- else None. The ulp gate applies where both sides evaluate
    the same binary64 formula on the same inputs; where the coefficients
    differ in their last bits (sums of squares in different orders) and the
    update cancels, a stored value can move by many ulps while the absolute
    difference stays tiny, and only the stated tolerance applies (the
    full-size tests instead let off only the elements where the oracle itself
    is that sensitive: coef_sensitive)."""
    for r, ro in records:
        if not (r["clip_coef"] == ro.clip_coef):
            return None
    return ULP_GATE


def assert_state_matches(got_master, got_m, got_v, got_out, want_master, want_m, want_v, want_out, where="",
                         stats: Optional[Stats] = None, ulp_max: Optional[int] = ULP_GATE, exempt=None):
    """The parity gates of the fp32 state and the bf16 emit:
    |d| <= max(2e-6 |ref|, 1e-7) on master, m, v (the stated tolerance);
    at most ulp_max binary32 ulps on master, m, v (equal values, NaN in both,
    count as 0); <= 1 bf16 ulp on out, NaN positions equal.
    exempt(idx) -> bool mask over idx: elements let off the ulp gate (only
    where the two sides used clip coefficients that differ in their last
    bits; see coef_sensitive). Elements it lets off still meet the stated
    tolerance."""
    over_idx = []
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
        ulp = np.where(same, 0, np.abs(ordered32(got) - ordered32(want)))
        if ulp_max is not None:
            over_idx.append(np.flatnonzero(ulp > ulp_max))
        if stats is not None:
            nz = (np.abs(w) > 0) & ~both_nan
            rel = float(np.max(err[nz] / np.abs(w[nz]))) if nz.any() else 0.0
            stats.max_rel[name] = max(stats.max_rel.get(name, 0.0), rel)
            stats.max_ulp[name] = max(stats.max_ulp.get(name, 0), int(ulp.max()) if ulp.size else 0)
    if over_idx:
        over = np.unique(np.concatenate(over_idx))
        if over.size:
            ok = np.asarray(exempt(over), bool) if exempt is not None else np.zeros(over.size, bool)
            if not ok.all():
                i = int(over[np.flatnonzero(~ok)[0]])
                raise AssertionError(
                    f"{where}: element {i} beyond {ulp_max} binary32 ulps: master {got_master[i]!r} vs "
                    f"{want_master[i]!r}, exp_avg {got_m[i]!r} vs {want_m[i]!r}, exp_avg_sq {got_v[i]!r} vs "
                    f"{want_v[i]!r} ({int((~ok).sum())} such elements)")
            if stats is not None:
                stats.ulp_exempt += int(over.size)
    if stats is not None:
        stats.elements += int(np.asarray(want_master).size)
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


def coef_sensitive(master, m, v, g, hp: oracle.HParams, coef: float, delta: float):
    """exempt() for assert_state_matches: the oracle's AdamW evaluated again
    at coef * (1 - delta) and coef * (1 + delta); an element is sensitive when
    either moves any of its master, m, v by more than one binary32 ulp. There
    the update cancels (w*(1 - lr*wd) against the Adam step, or b1*m against
    (1-b1)*g), and a coefficient that differs in its last bits can move the
    stored value by many ulps while the absolute difference stays tiny. The
    inputs are the oracle's own; delta only has to exceed the relative
    difference between the two coefficients by a wide margin."""
    def f(idx):
        idx = np.asarray(idx, np.int64)
        base = oracle.adamw(master[idx], m[idx], v[idx], g[idx], hp, coef)
        moved = np.zeros(idx.size, bool)
        for c in (coef * (1.0 - delta), coef * (1.0 + delta)):
            alt = oracle.adamw(master[idx], m[idx], v[idx], g[idx], hp, c)
            for a, b in zip(alt[:3], base[:3]):
                moved |= np.abs(ordered32(a) - ordered32(b)) > 1
        return moved
    return f


def assert_tensor_matches(dt: z.ZeroTensor, ht: oracle.TensorState, where="", stats=None, ulp_max=ULP_GATE):
    assert_state_matches(to_np_f32(dt.master), to_np_f32(dt.exp_avg), to_np_f32(dt.exp_avg_sq),
                         to_np_u16(dt.param_out), ht.master, ht.exp_avg, ht.exp_avg_sq, ht.param_out, where, stats,
                         ulp_max=ulp_max)


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


def host_replicas(w, spec, s0: int, s1: int, inject=()):
    """The workload's M bf16 replicas of tensor `spec` at shard-local
    elements [s0, s1), regenerated on the host; `inject` lists (rank, index)
    elements set to +inf."""
    grads = [synth.host_bf16(s1 - s0, w.seed, synth.stream_id(synth.KIND_GRAD, spec.tensor_id, r), w.grad_std,
                             start=spec.start + s0) for r in range(w.M)]
    for r, i in inject:
        if s0 <= i < s1:
            grads[r][i - s0] = 0x7F80
    return grads


def host_state(w, spec, s0: int, s1: int):
    """The workload's seeded fp32 master, m and v at shard-local [s0, s1)."""
    st = lambda k: synth.stream_id(k, spec.tensor_id, 0)
    n = s1 - s0
    master = synth.host_f32(n, w.seed, st(synth.KIND_MASTER), w.master_std, start=spec.start + s0)
    m = synth.host_f32(n, w.seed, st(synth.KIND_EXP_AVG), w.m_std, start=spec.start + s0) if w.m_std else \
        np.zeros(n, np.float32)
    v = synth.host_f32(n, w.seed, st(synth.KIND_EXP_AVG_SQ), w.v_std, start=spec.start + s0, absval=True) \
        if w.v_std else np.zeros(n, np.float32)
    return master, m, v


def _slices(w, slice_elems: int):
    return [(ti, s0, min(spec.n, s0 + slice_elems)) for ti, spec in enumerate(w.tensors)
            for s0 in range(0, spec.n, slice_elems)]


def _in_order(jobs, fn, workers: int, label: str):
    """fn over jobs on host threads (numpy, the oracle's C calls and device
    read-backs release the interpreter lock), results yielded in job order,
    a bounded window of jobs in flight; a progress line every tenth."""
    from concurrent.futures import ThreadPoolExecutor
    import time
    t0 = time.perf_counter()
    window = 2 * workers
    with ThreadPoolExecutor(max_workers=workers) as ex:
        futs = [ex.submit(fn, j) for j in jobs[:window]]
        nxt = len(futs)
        for k in range(len(jobs)):
            r = futs[k].result()
            futs[k] = None
            if nxt < len(jobs):
                futs.append(ex.submit(fn, jobs[nxt]))
                nxt += 1
            if (k + 1) * 10 // len(jobs) != k * 10 // len(jobs):
                print(f"  {label}: {k + 1}/{len(jobs)} slices, {time.perf_counter() - t0:.1f} s", flush=True)
            yield r


def oracle_sumsq_streaming(w, slice_elems: int = 1 << 22, workers: int = 16, inject=()):
    """The oracle's sum of squares and non-finite flag over the whole
    workload, regenerating the replicas on the host slice by slice (bounded
    memory): the folds run on host threads, and the squares are chained
    through the slices in index order, as the oracle's own step sums them
    (its compensated pair carried from slice to slice).
    `inject` lists (tensor, rank, index) elements set to +inf."""
    inj = {}
    for (t, r, i) in inject:
        inj.setdefault(t, []).append((r, i))

    def one(job):
        ti, s0, s1 = job
        return oracle.reduce(host_replicas(w, w.tensors[ti], s0, s1, inj.get(ti, ())), w.grad_scale)

    st = oracle.SumSq()
    for g in _in_order(_slices(w, slice_elems), one, workers, f"{w.name}: oracle sum of squares"):
        st.add(g)
    return st.sumsq, st.found_inf


def _read(t: torch.Tensor, s0: int, s1: int) -> np.ndarray:
    return t[s0:s1].cpu().numpy()


def _read_u16(t: torch.Tensor, s0: int, s1: int) -> np.ndarray:
    return t[s0:s1].view(torch.int16).cpu().numpy().view(np.uint16)


def assert_bits_equal_nan(got: np.ndarray, want: np.ndarray, where: str):
    """Bit-exact fp32, except that NaN payloads only have to be NaN in both."""
    nan = np.isnan(want)
    if not np.array_equal(np.isnan(got), nan):
        raise AssertionError(f"{where}: NaN positions differ")
    gu = np.ascontiguousarray(got).view(np.uint32)
    wu = np.ascontiguousarray(want).view(np.uint32)
    diff = (gu != wu) & ~nan
    if diff.any():
        i = int(np.flatnonzero(diff)[0])
        raise AssertionError(f"{where}[{i}]: got {got[i]!r} ({gu[i]:#010x}) want {want[i]!r} ({wu[i]:#010x}); "
                             f"{int(diff.sum())} of {diff.size} differ")


def full_step_parity(w, dts, hp, coef: float, coef_dev: float, stats: Stats, g_dev=None, slice_elems: int = 1 << 22,
                     workers: int = 16):
    """Every element of every tensor of workload w after one zero_step from
    its seeded state, against the oracle: the M replicas and the state are
    regenerated on the host slice by slice; the oracle folds (binary32,
    ascending rank), scales and applies AdamW with its own clip coefficient
    `coef`; the device state is read back slice by slice and held to the
    parity gates. g_dev (optional, per tensor): a device fp32 buffer that
    zero_shard_reduce wrote from the same replicas, compared bit for bit.
    coef_dev is the device's coefficient: when it differs from the oracle's
    in its last bits, elements where the update cancels are let off the ulp
    gate (coef_sensitive), still held to the stated tolerance."""
    hpo = hp_oracle(hp)
    rel = abs(coef_dev / coef - 1.0) if coef else 0.0
    delta = None if coef_dev == coef else max(1e-9, 100.0 * rel)

    def one(job):
        ti, s0, s1 = job
        spec, dt = w.tensors[ti], dts[ti]
        where = f"{spec.name}[{s0}:{s1}]"
        g = oracle.reduce(host_replicas(w, spec, s0, s1), w.grad_scale)
        if g_dev is not None:
            assert_bits_equal_nan(_read(g_dev[ti], s0, s1), g, "zero_shard_reduce " + where)
        master, m, v = host_state(w, spec, s0, s1)
        wt, wm, wv, wo = oracle.adamw(master, m, v, g, hpo, coef)
        st = Stats()
        ex = coef_sensitive(master, m, v, g, hpo, coef, delta) if delta is not None else None
        assert_state_matches(_read(dt.master, s0, s1), _read(dt.exp_avg, s0, s1), _read(dt.exp_avg_sq, s0, s1),
                             _read_u16(dt.param_out, s0, s1), wt, wm, wv, wo, where, st, exempt=ex)
        return st

    for st in _in_order(_slices(w, slice_elems), one, workers, f"{w.name}: every element"):
        stats.merge(st)


def full_zero2_parity(w, dts, accs, hp, micro_batches: int, stats: Stats, slice_elems: int = 1 << 22,
                      workers: int = 16):
    """Every element of every tensor of workload w after `micro_batches`
    deliveries of the same replicas through zero_bucket_reduce and one
    zero_step_accumulated (no clipping or skipping, so each element's
    update is local): the fp32 accumulators bit for bit against the oracle's
    accumulation, the state to the parity gates of the oracle's accumulated
    step."""
    hpo = hp_oracle(hp)
    assert not (hp.max_grad_norm > 0) and not hp.skip_on_nonfinite

    def one(job):
        ti, s0, s1 = job
        spec, dt = w.tensors[ti], dts[ti]
        where = f"{spec.name}[{s0}:{s1}]"
        grads = host_replicas(w, spec, s0, s1)
        a = None
        for _ in range(micro_batches):
            a = oracle.grad_accumulate(grads, a)
        assert_bits_equal_nan(_read(accs[ti], s0, s1), a, "accumulator " + where)
        master, m, v = host_state(w, spec, s0, s1)
        new, _ = oracle.zero_step_accumulated([a], [oracle.TensorState([], master, m, v, None)], hpo)
        h = new[0]
        st = Stats()
        assert_state_matches(_read(dt.master, s0, s1), _read(dt.exp_avg, s0, s1), _read(dt.exp_avg_sq, s0, s1),
                             _read_u16(dt.param_out, s0, s1), h.master, h.exp_avg, h.exp_avg_sq, h.param_out, where,
                             st)
        return st

    for st in _in_order(_slices(w, slice_elems), one, workers, f"{w.name}: ZeRO-2, every element"):
        stats.merge(st)
