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
from synth.workloads import workload

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
