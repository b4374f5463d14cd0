"""The five workloads at full size, built and stepped exactly as bench.py
does, checked against the oracle on every element: the M replicas and the
seeded state are regenerated on the host slice by slice on host threads, the
oracle folds and updates each slice, and the device's state is read back
slice by slice and held to the parity gates (the stated tolerance and at most
4 binary32 ulps on master, m, v; 1 bf16 ulp on the output). The same pass
compares zero_shard_reduce's fp32 output from the same replicas bit for bit,
and the global norm against the oracle's own sum of squares, chained through
the whole workload in index order."""
import json
import math

import numpy as np
import pytest
import torch

import bench
import oracle
import sharded_optimizer_step_amd as z
import synth
from cases import (Stats, assert_state_matches, coef_sensitive, full_step_parity, full_zero2_parity, hp_oracle,
                   host_inputs_at, oracle_sumsq_streaming, sample_indices, to_np_f32, to_np_u16)
from synth.workloads import workload, zero2_buckets

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    z.lib()
    torch.cuda.set_device(0)
    yield
    torch.cuda.empty_cache()


def _step(w, tensors, hp):
    ws = z.workspace(z.zero_step_workspace_bytes(tensors, w.M, hp))
    res = z.new_result()
    z.zero_step(tensors, hp, 0.0, ws, res)
    return z.read_result(res)


def _gather(t: torch.Tensor, idx: np.ndarray):
    return t[torch.from_numpy(idx).to(t.device)]


def _check_sampled(w, tensors, hp, coef, coef_dev, idx_per_tensor, stats):
    delta = None if coef_dev == coef else max(1e-9, 100.0 * abs(coef_dev / coef - 1.0))
    for spec, dt, idx in zip(w.tensors, tensors, idx_per_tensor):
        grads, master, m, v = host_inputs_at(w, spec, idx)
        g = oracle.reduce(grads, w.grad_scale)
        hpo = hp_oracle(hp)
        wt, wm, wv, wo = oracle.adamw(master, m, v, g, hpo, coef)
        ex = coef_sensitive(master, m, v, g, hpo, coef, delta) if delta is not None else None
        assert_state_matches(to_np_f32(_gather(dt.master, idx)), to_np_f32(_gather(dt.exp_avg, idx)),
                             to_np_f32(_gather(dt.exp_avg_sq, idx)), to_np_u16(_gather(dt.param_out, idx)),
                             wt, wm, wv, wo, f"{spec.name}", stats, exempt=ex)


def _hp(w):
    return z.HParams(**w.hparams())


def _report(w, what, r, ro, st):
    """One line a log reader can collect: the run's parity statistics."""
    print("PARITY " + json.dumps(dict(workload=w.index, what=what, grad_norm=r["grad_norm"],
                                      oracle_grad_norm=ro.grad_norm, clip_coef=r["clip_coef"],
                                      oracle_clip_coef=ro.clip_coef, **st.as_dict())), flush=True)


def _reduce_all(w, tensors):
    """zero_shard_reduce of every tensor's replicas into fresh fp32 buffers."""
    outs = []
    for dt in tensors:
        g = torch.empty(dt.master.numel(), dtype=torch.float32, device="cuda")
        z.zero_shard_reduce(dt.grads, w.grad_scale, g)
        outs.append(g)
    torch.cuda.synchronize()
    return outs


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wi", [0, 1, 2, 3])
def test_single_pass_and_clipped_workloads_every_element(wi):
    # workloads 0, 2 and 3 step in one pass; workload 1 clips at 1.0 (two
    # passes). Every element of the state, and zero_shard_reduce over the same
    # replicas bit for bit.
    w = workload(wi)
    tensors = bench.build_workload(w, 0)
    hp = _hp(w)
    r = _step(w, tensors, hp)
    g_dev = _reduce_all(w, tensors)
    s, f = oracle_sumsq_streaming(w)
    ro = oracle.finalize(s, 0.0, f, hp.max_grad_norm, hp.skip_on_nonfinite)
    assert r["status"] == 0 and r["found_inf"] == f == 0 and r["skipped"] == 0
    assert abs(r["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm, (r, ro)
    assert abs(r["clip_coef"] - ro.clip_coef) <= 1e-6 * ro.clip_coef, (r, ro)
    if wi == 1:
        assert ro.clip_coef < 1.0  # the 124M-parameter bucket clips at 1.0
    else:
        assert r["clip_coef"] == ro.clip_coef == 1.0
    st = Stats()
    full_step_parity(w, tensors, hp, ro.clip_coef, r["clip_coef"], st, g_dev=g_dev,
                     slice_elems=1 << 21 if w.M > 16 else 1 << 22)
    assert st.elements == w.n_total
    _report(w, "zero_step, every element; zero_shard_reduce bit-exact on every element", r, ro, st)


def _seeded_state_unchanged(w, dt, spec):
    """Every element of master, m, v still holds its seeded value (the device
    generator fills a scratch buffer to compare against)."""
    tmp = torch.empty_like(dt.master)
    for x, kind, std, ab in ((dt.master, synth.KIND_MASTER, w.master_std, False),
                             (dt.exp_avg, synth.KIND_EXP_AVG, w.m_std, False),
                             (dt.exp_avg_sq, synth.KIND_EXP_AVG_SQ, w.v_std, True)):
        synth.device_f32(tmp, w.seed, synth.stream_id(kind, spec.tensor_id, 0), std, start=spec.start, absval=ab)
        if not torch.equal(x.view(torch.int32), tmp.view(torch.int32)):
            return False
    return True


@pytest.mark.timeout(900)
def test_amp_workload_skip_then_clean_step():
    w = workload(4)
    tensors = bench.build_workload(w, 0)
    dt = tensors[0]
    spec = w.tensors[0]
    hp = _hp(w)
    # odd run: seeded +inf values planted in the replicas -> the step is skipped
    pos = synth.inject_positions(w.seed, 1, w.M, spec.n, w.inject_rate)
    assert len(pos) >= 1
    for rnk, i in pos:
        dt.grads[rnk].view(torch.int16)[i] = 0x7F80
    dt.param_out.view(torch.int16).fill_(0x1234)
    r = _step(w, tensors, hp)
    assert r["found_inf"] == 1 and r["skipped"] == 1 and r["status"] == 0
    assert _seeded_state_unchanged(w, dt, spec)  # every element of master, m, v
    assert bool((dt.param_out.view(torch.int16) == 0x1234).all())
    # even run: the planted values restored from the generator -> a clean, clipped step
    for rnk, i in pos:
        h = synth.host_bf16_at(np.array([i + spec.start], np.int64), w.seed,
                               synth.stream_id(synth.KIND_GRAD, spec.tensor_id, rnk), w.grad_std)
        dt.grads[rnk].view(torch.int16)[i] = int(h.view(np.int16)[0])
    r = _step(w, tensors, hp)
    g_dev = _reduce_all(w, tensors)
    s, f = oracle_sumsq_streaming(w)
    ro = oracle.finalize(s, 0.0, f, hp.max_grad_norm, hp.skip_on_nonfinite)
    assert r["found_inf"] == 0 and r["skipped"] == 0 and ro.skipped == 0
    assert abs(r["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm
    assert abs(r["clip_coef"] - ro.clip_coef) <= 1e-6 * ro.clip_coef
    assert ro.clip_coef < 1.0
    st = Stats()
    full_step_parity(w, tensors, hp, ro.clip_coef, r["clip_coef"], st, g_dev=g_dev)
    assert st.elements == w.n_total
    _report(w, "skipped step: state bit-identical; clean clipped step, every element; "
               "zero_shard_reduce bit-exact on every element", r, ro, st)


def test_amp_workload_under_the_dynamic_loss_scale():
    # the bench's --amp leg at full size: the scale held on the device starts
    # at 1/grad_scale = 2^16 (so a clean step is the fixed-scale step), then
    # two steps with the seeded +inf values planted are skipped and, at
    # hysteresis 2, the second halves the scale
    w = workload(4)
    tensors = bench.build_workload(w, 0)
    dt = tensors[0]
    spec = w.tensors[0]
    power = int(round(-math.log2(w.grad_scale)))
    assert 2.0 ** -power == w.grad_scale
    kw = dict(initial_scale_power=power, window=1000, hysteresis=2, min_scale=1.0)
    cfg, ocfg = z.LossScaleConfig(**kw), oracle.LossScaleConfig(**kw)
    hp = _hp(w)
    hp.grad_scale = 1.0  # the multiplier comes from the device state
    ls = z.new_loss_scale()
    z.zero_loss_scale_init(cfg, ls)
    ols = oracle.loss_scale_init(ocfg)
    ws = z.workspace(z.zero_step_amp_workspace_bytes(tensors, w.M, hp))
    res = z.new_result()

    # clean step
    z.zero_step_amp(tensors, hp, cfg, ls, 0.0, ws, res)
    r = z.read_result(res)
    s, f = oracle_sumsq_streaming(w)
    ro = oracle.finalize(s, 0.0, f, hp.max_grad_norm, 1)
    assert r["status"] == 0 and r["found_inf"] == 0 and r["skipped"] == 0
    assert abs(r["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm and ro.clip_coef < 1.0
    st = Stats()
    _check_sampled(w, tensors, hp, ro.clip_coef, r["clip_coef"],
                   [sample_indices(spec.n, np.random.default_rng(44), 40_000)], st)
    ols = oracle.loss_scale_update(ols, ocfg, 0)
    assert z.read_loss_scale(ls) == dict(scale=ols.scale, inv_scale=ols.inv_scale, good_steps=ols.good_steps,
                                         overflows=ols.overflows)

    # two overflowed steps: skipped, state untouched, the second halves the scale
    pos = synth.inject_positions(w.seed, 1, w.M, spec.n, w.inject_rate)
    for rnk, i in pos:
        dt.grads[rnk].view(torch.int16)[i] = 0x7F80
    probe = np.unique(np.array([i for _, i in pos], np.int64))
    before = [to_np_f32(_gather(x, probe)).copy() for x in (dt.master, dt.exp_avg, dt.exp_avg_sq)]
    out_before = to_np_u16(_gather(dt.param_out, probe)).copy()
    for k in range(2):
        z.zero_step_amp(tensors, hp, cfg, ls, 0.0, ws, res)
        r = z.read_result(res)
        assert r["status"] == 0 and r["found_inf"] == 1 and r["skipped"] == 1, (k, r)
        ols = oracle.loss_scale_update(ols, ocfg, 1)
        got = z.read_loss_scale(ls)
        assert got == dict(scale=ols.scale, inv_scale=ols.inv_scale, good_steps=ols.good_steps,
                           overflows=ols.overflows), (k, got, ols)
    assert got["scale"] == 2.0 ** (power - 1)
    for b, x in zip(before, (dt.master, dt.exp_avg, dt.exp_avg_sq)):
        assert np.array_equal(to_np_f32(_gather(x, probe)).view(np.uint32), b.view(np.uint32))
    assert np.array_equal(to_np_u16(_gather(dt.param_out, probe)), out_before)
    print(w.name, "AMP norm", r, ro.grad_norm, st)


def test_offloaded_step_on_the_7p5b_shard():
    # the state of the 117,187,500-parameter shard moved to host memory: the
    # offloaded step must give exactly what the fused step gives on the same
    # replicas, and match the oracle on sampled elements
    w = workload(2)
    tensors = bench.build_workload(w, 0)
    d = tensors[0]
    spec = w.tensors[0]
    hp = _hp(w)
    ot = z.OffloadTensor(d.grads, d.master.cpu(), d.exp_avg.cpu(), d.exp_avg_sq.cpu(),
                         torch.empty_like(d.param_out))
    r_off = z.zero_offload_step([ot], hp, 0.0, z.workspace(z.zero_offload_workspace_bytes([ot], w.M)),
                                z.host_workspace(z.zero_offload_host_workspace_bytes([ot])))
    torch.cuda.synchronize()
    r = _step(w, tensors, hp)
    assert r_off["status"] == r["status"] == 0 and r_off["skipped"] == r["skipped"] == 0
    assert math.isclose(r_off["sumsq"], r["sumsq"], rel_tol=1e-12)
    for name in ("master", "exp_avg", "exp_avg_sq"):
        assert torch.equal(getattr(ot, name), getattr(d, name).cpu()), name
    assert torch.equal(ot.param_out.view(torch.int16), d.param_out.view(torch.int16))
    idx = sample_indices(spec.n, np.random.default_rng(22), 40_000)
    st = Stats()
    _check_sampled(w, tensors, hp, 1.0, 1.0, [idx], st)
    print(w.name, "offloaded", st)


@pytest.mark.timeout(900)
def test_zero2_two_micro_batches_on_the_llama_list():
    # the same replicas delivered twice: every accumulator holds fold + fold,
    # compared bit for bit on every element with the oracle's two-micro-batch
    # accumulation, then the state after the step from it, on every element
    w = workload(3)
    tensors = bench.build_workload(w, 0)
    buckets = zero2_buckets(w)
    accs = [torch.empty(spec.n, dtype=torch.float32, device="cuda") for spec in w.tensors]
    parts = z.new_bucket_partials(len(buckets))
    hp = _hp(w)
    reducers = [z.BucketReducer([z.GradShard(tensors[t].grads, accs[t]) for t in idx], parts[32 * b:32 * b + 32])
                for b, idx in enumerate(buckets)]
    for k in range(2):
        for rd in reducers:
            rd.reduce((z.BUCKET_ACCUMULATE if k else 0) | (z.BUCKET_FINAL if k else 0), hp.grad_scale, 9)
    ats = [z.AccTensor(a, t.master, t.exp_avg, t.exp_avg_sq, t.param_out) for a, t in zip(accs, tensors)]
    res = z.new_result()
    z.zero_step_accumulated(ats, hp, parts, len(buckets), 9, 0.0,
                            z.workspace(z.zero_step_accumulated_workspace_bytes(ats)), res)
    r = z.read_result(res)
    assert r["status"] == 0 and r["found_inf"] == 0 and r["skipped"] == 0
    st = Stats()
    full_zero2_parity(w, tensors, accs, hp, 2, st)
    assert st.elements == w.n_total
    print("PARITY " + json.dumps(dict(workload=w.index, what="ZeRO-2, 2 micro-batches: accumulators bit-exact and "
                                      "state, every element", grad_norm=r["grad_norm"], **st.as_dict())), flush=True)


@pytest.mark.timeout(900)
def test_zero2_fused_final_pass_on_the_llama_list():
    # the 288-tensor shard through its 97 buckets in backward order, each
    # bucket's only micro-batch folded and applied in one pass
    # (zero_bucket_step), the record from the bucket partials: with one
    # micro-batch this is the fused ZeRO-1 step, checked on every element
    w = workload(3)
    tensors = bench.build_workload(w, 0)
    buckets = zero2_buckets(w)
    parts = z.new_bucket_partials(len(buckets))
    hp = _hp(w)
    steppers = [z.BucketStepper([z.BucketTensor(tensors[t].grads, None, tensors[t].master, tensors[t].exp_avg,
                                                tensors[t].exp_avg_sq, tensors[t].param_out) for t in idx],
                                parts[32 * b:32 * b + 32]) for b, idx in enumerate(buckets)]
    for sp in steppers:
        sp.step(0, hp, 21)
    res = z.new_result()
    z.zero_step_accumulated([], hp, parts, len(buckets), 21, 0.0, None, res)
    r = z.read_result(res)
    s, f = oracle_sumsq_streaming(w)
    ro = oracle.finalize(s, 0.0, f, hp.max_grad_norm, hp.skip_on_nonfinite)
    assert r["status"] == 0 and r["found_inf"] == f == 0 and r["skipped"] == 0 and r["clip_coef"] == 1.0
    assert abs(r["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm, (r, ro)
    st = Stats()
    full_step_parity(w, tensors, hp, 1.0, 1.0, st)
    assert st.elements == w.n_total
    _report(w, f"ZeRO-2 fused final pass, {len(buckets)} buckets: every element", r, ro, st)
