"""The five workloads at full size, built and stepped exactly as bench.py
does, checked against the oracle: every element for the two smaller ones,
sampled elements (both ends, tile boundaries, uniform random) for the three
large ones, and the global norm against the oracle's own sum of squares over
the whole workload, regenerated on the host slice by slice."""
import math

import numpy as np
import pytest
import torch

import bench
import oracle
import sharded_optimizer_step_amd as z
import synth
from cases import (Stats, assert_state_matches, hp_oracle, host_inputs_at, oracle_sumsq_streaming, sample_indices,
                   to_np_f32, to_np_u16)
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


def _check_sampled(w, tensors, hp, coef, idx_per_tensor, stats):
    for spec, dt, idx in zip(w.tensors, tensors, idx_per_tensor):
        grads, master, m, v = host_inputs_at(w, spec, idx)
        g = oracle.reduce(grads, w.grad_scale)
        wt, wm, wv, wo = oracle.adamw(master, m, v, g, hp_oracle(hp), coef)
        assert_state_matches(to_np_f32(_gather(dt.master, idx)), to_np_f32(_gather(dt.exp_avg, idx)),
                             to_np_f32(_gather(dt.exp_avg_sq, idx)), to_np_u16(_gather(dt.param_out, idx)),
                             wt, wm, wv, wo, f"{spec.name}", stats)


def _hp(w):
    return z.HParams(**w.hparams())


@pytest.mark.parametrize("wi", [0, 1])
def test_small_workloads_every_element(wi):
    w = workload(wi)
    tensors = bench.build_workload(w, 0)
    hp = _hp(w)
    r = _step(w, tensors, hp)
    spec = w.tensors[0]
    idx = np.arange(spec.n, dtype=np.int64)
    grads, master, m, v = host_inputs_at(w, spec, idx)
    new, ro = oracle.zero_step([oracle.TensorState(grads, master, m, v, None)], hp_oracle(hp))
    assert r["status"] == 0 and r["found_inf"] == 0 and r["skipped"] == 0
    assert abs(r["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm
    assert abs(r["clip_coef"] - ro.clip_coef) <= 1e-6 * ro.clip_coef
    if wi == 1:
        assert ro.clip_coef < 1.0  # the 124M-parameter bucket clips at 1.0
    st = Stats()
    assert_state_matches(to_np_f32(tensors[0].master), to_np_f32(tensors[0].exp_avg),
                         to_np_f32(tensors[0].exp_avg_sq), to_np_u16(tensors[0].param_out), new[0].master,
                         new[0].exp_avg, new[0].exp_avg_sq, new[0].param_out, w.name, st)
    print(w.name, st)


@pytest.mark.parametrize("wi", [2, 3])
def test_large_single_pass_workloads_sampled(wi):
    w = workload(wi)
    tensors = bench.build_workload(w, 0)
    hp = _hp(w)
    r = _step(w, tensors, hp)
    rng = np.random.default_rng(wi)
    k = 40_000 if len(w.tensors) == 1 else 400
    idx = [sample_indices(spec.n, rng, k) for spec in w.tensors]
    st = Stats()
    _check_sampled(w, tensors, hp, 1.0, idx, st)
    s, f = oracle_sumsq_streaming(w)
    assert r["status"] == 0 and r["found_inf"] == f == 0 and r["skipped"] == 0
    assert abs(r["grad_norm"] - math.sqrt(s)) <= 1e-5 * math.sqrt(s), (r, math.sqrt(s))
    assert r["clip_coef"] == 1.0
    print(w.name, "norm", r["grad_norm"], math.sqrt(s), st)


def test_amp_workload_skip_then_clean_step():
    w = workload(4)
    tensors = bench.build_workload(w, 0)
    dt = tensors[0]
    spec = w.tensors[0]
    hp = _hp(w)
    rng = np.random.default_rng(4)
    idx = sample_indices(spec.n, rng, 40_000)
    # odd run: seeded +inf values planted in the replicas -> the step is skipped
    pos = synth.inject_positions(w.seed, 1, w.M, spec.n, w.inject_rate)
    assert len(pos) >= 1
    for rnk, i in pos:
        dt.grads[rnk].view(torch.int16)[i] = 0x7F80
    dt.param_out.view(torch.int16).fill_(0x1234)
    probe = np.unique(np.concatenate([idx, np.array([i for _, i in pos], np.int64)]))
    r = _step(w, tensors, hp)
    assert r["found_inf"] == 1 and r["skipped"] == 1 and r["status"] == 0
    _, master, m, v = host_inputs_at(w, spec, probe)
    assert np.array_equal(to_np_f32(_gather(dt.master, probe)).view(np.uint32), master.view(np.uint32))
    assert np.array_equal(to_np_f32(_gather(dt.exp_avg, probe)).view(np.uint32), m.view(np.uint32))
    assert np.array_equal(to_np_f32(_gather(dt.exp_avg_sq, probe)).view(np.uint32), v.view(np.uint32))
    assert bool((dt.param_out.view(torch.int16) == 0x1234).all())
    # even run: the planted values restored from the generator -> a clean, clipped step
    for rnk, i in pos:
        h = synth.host_bf16_at(np.array([i + spec.start], np.int64), w.seed,
                               synth.stream_id(synth.KIND_GRAD, spec.tensor_id, rnk), w.grad_std)
        dt.grads[rnk].view(torch.int16)[i] = int(h.view(np.int16)[0])
    r = _step(w, tensors, hp)
    s, f = oracle_sumsq_streaming(w)
    ro = oracle.finalize(s, 0.0, f, hp.max_grad_norm, hp.skip_on_nonfinite)
    assert r["found_inf"] == 0 and r["skipped"] == 0 and ro.skipped == 0
    assert abs(r["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm
    assert ro.clip_coef < 1.0
    st = Stats()
    _check_sampled(w, tensors, hp, ro.clip_coef, [idx], st)
    print(w.name, "norm", r["grad_norm"], ro.grad_norm, "coef", r["clip_coef"], ro.clip_coef, st)


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
    _check_sampled(w, tensors, hp, ro.clip_coef, [sample_indices(spec.n, np.random.default_rng(44), 40_000)], st)
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
    _check_sampled(w, tensors, hp, 1.0, [idx], st)
    print(w.name, "offloaded", st)


def test_zero2_two_micro_batches_on_the_llama_list():
    # the same replicas delivered twice: every accumulator holds fold + fold,
    # checked against the oracle's two-micro-batch accumulation on sampled
    # elements, then the step from it
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
    rng = np.random.default_rng(34)
    st = Stats()
    for spec, dt, acc in zip(w.tensors, tensors, accs):
        idx = sample_indices(spec.n, rng, 200)
        grads, master, m, v = host_inputs_at(w, spec, idx)
        a = oracle.grad_accumulate(grads, oracle.grad_accumulate(grads))
        sel = torch.from_numpy(idx).cuda()
        got = acc[sel].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), a.view(np.uint32)), spec.name
        new, _ = oracle.zero_step_accumulated([a], [oracle.TensorState([], master, m, v, None)], hp_oracle(hp))
        h = new[0]
        assert_state_matches(to_np_f32(dt.master[sel]), to_np_f32(dt.exp_avg[sel]), to_np_f32(dt.exp_avg_sq[sel]),
                             to_np_u16(dt.param_out[sel]), h.master, h.exp_avg, h.exp_avg_sq, h.param_out, spec.name,
                             st)
    print(w.name, "ZeRO-2, 2 micro-batches", st)
