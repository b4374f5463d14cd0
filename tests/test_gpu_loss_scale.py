"""GPU parity of the dynamic loss scale (zero_loss_scale_init/_update and the
fused zero_step_amp) against the CPU oracle, through the C ABI.

Gates: the loss-scale state bit-exact after every step; found_inf and
skipped exact; the step's state as in the other parity tests (master/m/v
within max(2e-6 |ref|, 1e-7), the bf16 output within 1 ulp); a finite sum of
squares within 1e-9 relative."""
import math
import struct

import numpy as np
import pytest
import torch

import oracle
import sharded_optimizer_step_amd as z
from cases import Case, assert_state_matches, assert_tensor_matches, build, hp_oracle, to_np_u16, ulp_gate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    z.lib()
    torch.cuda.set_device(0)
    yield


def _cfg_pair(**kw):
    return z.LossScaleConfig(**kw), oracle.LossScaleConfig(**kw)


def _same_state(dev: dict, ref: oracle.LossScale, where=""):
    got = (np.float32(dev["scale"]), np.float32(dev["inv_scale"]), dev["good_steps"], dev["overflows"])
    want = (np.float32(ref.scale), np.float32(ref.inv_scale), ref.good_steps, ref.overflows)
    assert got[0].tobytes() == want[0].tobytes() and got[1].tobytes() == want[1].tobytes(), (where, got, want)
    assert got[2:] == want[2:], (where, got, want)


def _record(found_inf: int, status: int = 0) -> torch.Tensor:
    b = struct.pack("<ddfiii", 1.0, 1.0, 1.0, found_inf, found_inf, status)
    return torch.frombuffer(bytearray(b), dtype=torch.uint8).cuda()


@pytest.mark.parametrize("kw", [dict(), dict(initial_scale_power=0, window=3, hysteresis=1),
                                dict(initial_scale_power=4, window=2, hysteresis=1, min_scale=3.0),
                                dict(initial_scale_power=126, window=1, hysteresis=3),
                                dict(initial_scale_power=-120, window=5, hysteresis=2, min_scale=2.0 ** -126)])
def test_update_kernel_follows_the_oracle(kw):
    zc, oc = _cfg_pair(**kw)
    ls = z.new_loss_scale()
    z.zero_loss_scale_init(zc, ls)
    ref = oracle.loss_scale_init(oc)
    _same_state(z.read_loss_scale(ls), ref, "init")
    rng = np.random.default_rng(sum(map(hash, map(str, kw.items()))) & 0xFFFF)
    flags = (rng.random(120) < 0.3).astype(int)
    recs = {f: _record(f) for f in (0, 1)}
    for k, f in enumerate(flags):
        z.zero_loss_scale_update(zc, recs[int(f)], ls)
        ref = oracle.loss_scale_update(ref, oc, int(f))
        if k % 7 == 0 or k == len(flags) - 1:
            _same_state(z.read_loss_scale(ls), ref, f"step {k}")
    # a record of a stale workspace leaves the state alone
    z.zero_loss_scale_update(zc, _record(1, status=z.ZERO_ERR_STALE_WORKSPACE), ls)
    _same_state(z.read_loss_scale(ls), ref, "stale")


def _inject(dts, hts, where, value=0x7F80):
    """Set element i of replica r of tensor t on both sides; returns the old codes."""
    old = []
    for (t, r, i) in where:
        h = hts[t].grads[r]
        old.append(int(h[i]))
        h[i] = value
        dts[t].grads[r].view(torch.int16)[i] = int(np.int16(np.uint16(value)))
    return old


def _restore(dts, hts, where, old):
    for (t, r, i), v in zip(where, old):
        hts[t].grads[r][i] = v
        dts[t].grads[r].view(torch.int16)[i] = int(np.int16(np.uint16(v)))


@pytest.mark.parametrize("sizes,M,max_norm", [([20_003], 4, 0.0), ([100_003, 512, 4099], 8, 5.0),
                                              ([300_000], 2, 1e-2)])
def test_amp_step_run_matches_the_oracle(sizes, M, max_norm):
    # gradients as a loss scaled by 2^12 would give them; overflows planted on
    # chosen steps: the scale halves on the second one in a row and doubles
    # after every `window` clean steps
    case = Case(sizes, M, seed=31, grad_std=4.0)
    dts, hts = build(case)
    zc, oc = _cfg_pair(initial_scale_power=12, window=3, hysteresis=2, min_scale=1.0)
    hp = z.HParams(step=1, max_grad_norm=max_norm)
    ws = z.workspace(z.zero_step_amp_workspace_bytes(dts, M, hp))
    res = z.new_result()
    ls = z.new_loss_scale()
    z.zero_loss_scale_init(zc, ls)
    ref = oracle.loss_scale_init(oc)
    state = hts
    plan = {2: [(0, M - 1, 7)], 3: [(0, 0, 5)], 4: [(len(sizes) - 1, 1 % M, sizes[-1] - 1)], 9: [(0, 0, 0)]}
    t = 1
    records = []
    for k in range(14):
        where = plan.get(k, [])
        old = _inject(dts, state, where)
        hp.step = t
        z.zero_step_amp(dts, hp, zc, ls, 0.0, ws, res)
        r = z.read_result(res)
        state, ro, ref = oracle.zero_step_amp(state, hp_oracle(hp), oc, ref)
        assert r["status"] == 0
        assert (r["found_inf"], r["skipped"]) == (ro.found_inf, ro.skipped) == (int(bool(where)),) * 2, k
        if not where:
            assert math.isclose(r["sumsq"], ro.sumsq, rel_tol=1e-9), (k, r, ro)
            t += 1
            records.append((r, ro))  # the steps that updated the state
        _same_state(z.read_loss_scale(ls), ref, f"step {k}")
        for d, h in zip(dts, state):
            assert_tensor_matches(d, h, f"step {k}", ulp_max=ulp_gate(*records))
        _restore(dts, state, where, old)
    # the run moved the scale both ways
    assert ref.scale != 4096.0 or ref.good_steps != 0


def test_amp_step_on_an_empty_bucket_counts_a_clean_step():
    zc, oc = _cfg_pair(window=2)
    ls = z.new_loss_scale()
    z.zero_loss_scale_init(zc, ls)
    empty = z.ZeroTensor([torch.empty(0, dtype=torch.bfloat16, device="cuda")] * 3,
                         *[torch.empty(0, dtype=torch.float32, device="cuda") for _ in range(3)],
                         torch.empty(0, dtype=torch.bfloat16, device="cuda"))
    res = z.new_result()
    ref = oracle.loss_scale_init(oc)
    for _ in range(3):
        z.zero_step_amp([empty], z.HParams(), zc, ls, 0.0, None, res)
        ref = oracle.loss_scale_update(ref, oc, 0)
    _same_state(z.read_loss_scale(ls), ref)
    assert ref.scale == 8192.0


def test_amp_step_equals_reduce_check_update_composition():
    # the fused AMP step and the composed entry points (reduce with
    # grad_scale = inv_scale, check, AdamW, then zero_loss_scale_update) give
    # the same record, state and scale
    case = Case([50_001], 4, seed=41, grad_std=4.0)
    d1, _ = build(case)
    d2, _ = build(case)
    zc, _ = _cfg_pair(initial_scale_power=12, window=1, hysteresis=1)
    hp = z.HParams(step=3, max_grad_norm=20.0, skip_on_nonfinite=1)
    ls1, ls2 = z.new_loss_scale(), z.new_loss_scale()
    z.zero_loss_scale_init(zc, ls1)
    z.zero_loss_scale_init(zc, ls2)
    res1, res2 = z.new_result(), z.new_result()
    z.zero_step_amp(d1, hp, zc, ls1, 0.0, z.workspace(z.zero_step_amp_workspace_bytes(d1, 4, hp)), res1)
    g = torch.empty(50_001, dtype=torch.float32, device="cuda")
    inv = z.read_loss_scale(ls2)["inv_scale"]
    z.zero_shard_reduce(d2[0].grads, inv, g)
    z.zero_grad_check_norm(g, hp, 0.0, z.workspace(z.zero_grad_check_norm_workspace_bytes(g.numel())), res2)
    z.zero_adamw_step(d2[0].master, d2[0].exp_avg, d2[0].exp_avg_sq, g, d2[0].param_out, hp, res2)
    z.zero_loss_scale_update(zc, res2, ls2)
    r1, r2 = z.read_result(res1), z.read_result(res2)
    assert (r1["found_inf"], r1["skipped"]) == (r2["found_inf"], r2["skipped"]) == (0, 0)
    assert math.isclose(r1["sumsq"], r2["sumsq"], rel_tol=1e-12)
    assert z.read_loss_scale(ls1) == z.read_loss_scale(ls2)
    for a, b in ((d1[0].master, d2[0].master), (d1[0].exp_avg, d2[0].exp_avg), (d1[0].exp_avg_sq, d2[0].exp_avg_sq)):
        assert torch.equal(a, b)
    assert torch.equal(d1[0].param_out.view(torch.int16), d2[0].param_out.view(torch.int16))


def _run_plan(sizes, M):
    """Overflows planted on chosen steps: the second in a row halves the scale,
    every `window` clean steps double it."""
    return {2: [(0, M - 1, 7)], 3: [(0, 0, 5)], 6: [(len(sizes) - 1, 1 % M, sizes[-1] - 1)]}


@pytest.mark.parametrize("max_norm", [0.0, 5.0])
def test_zero2_amp_run_matches_the_oracle(max_norm):
    # the ZeRO-2 streaming step under the dynamic scale: bucket reduces read
    # inv_scale on the device, the step checks the partials' multiplier,
    # updates, then moves the scale
    sizes, M = [100_003, 512, 4099], 4
    case = Case(sizes, M, seed=33, grad_std=4.0)
    dts, hts = build(case)
    zc, oc = _cfg_pair(initial_scale_power=12, window=3, hysteresis=2, min_scale=1.0)
    ls = z.new_loss_scale()
    z.zero_loss_scale_init(zc, ls)
    ref = oracle.loss_scale_init(oc)
    buckets = [[2, 1], [0]]
    parts = z.new_bucket_partials(len(buckets))
    accs = [torch.empty(n, dtype=torch.float32, device="cuda") for n in sizes]
    reducers = [z.BucketReducer([z.GradShard(dts[t].grads, accs[t]) for t in idx], parts[32 * b:32 * b + 32], ls=ls)
                for b, idx in enumerate(buckets)]
    ats = [z.AccTensor(a, d.master, d.exp_avg, d.exp_avg_sq, d.param_out) for a, d in zip(accs, dts)]
    sws = z.workspace(z.zero_step_accumulated_workspace_bytes(ats))
    res = z.new_result()
    state = hts
    plan = _run_plan(sizes, M)
    t = 1
    records = []
    seen = set()
    for k in range(10):
        where = plan.get(k, [])
        old = _inject(dts, state, where)
        hp = z.HParams(step=t, max_grad_norm=max_norm)
        for rd in reducers:
            rd.reduce(z.BUCKET_FINAL, hp.grad_scale, 100 + k)
        z.zero_step_accumulated_amp(ats, hp, zc, ls, parts, len(buckets), 100 + k, 0.0, sws, res)
        r = z.read_result(res)
        acc_h = [oracle.grad_accumulate(s_.grads) for s_ in state]
        new, ro, ref = oracle.zero_step_accumulated_amp(acc_h, state, hp_oracle(hp), oc, ref)
        # the step from accumulators returns no replicas: keep this run's
        state = [oracle.TensorState(s_.grads, n_.master, n_.exp_avg, n_.exp_avg_sq, n_.param_out)
                 for s_, n_ in zip(state, new)]
        assert r["status"] == 0
        assert (r["found_inf"], r["skipped"]) == (ro.found_inf, ro.skipped) == (int(bool(where)),) * 2, k
        if not where:
            assert math.isclose(r["sumsq"], ro.sumsq, rel_tol=1e-9), (k, r, ro)
            t += 1
            records.append((r, ro))  # the steps that updated the state
        _same_state(z.read_loss_scale(ls), ref, f"step {k}")
        seen.add(ref.scale)
        for d, h in zip(dts, state):
            assert_tensor_matches(d, h, f"step {k}", ulp_max=ulp_gate(*records))
        _restore(dts, state, where, old)
    assert seen == {2048.0, 4096.0}  # halved on the second overflow in a row, doubled after 3 clean steps


def test_offload_amp_run_matches_the_oracle():
    # the CPU-offloaded step under the dynamic scale: the GPU's fold reads and
    # moves it, the host update is unchanged
    sizes, M = [100_003, 4099], 4
    case = Case(sizes, M, seed=35, grad_std=4.0)
    dts, hts = build(case)
    ots = [z.OffloadTensor(d.grads, torch.from_numpy(h.master.copy()), torch.from_numpy(h.exp_avg.copy()),
                           torch.from_numpy(h.exp_avg_sq.copy()), d.param_out) for d, h in zip(dts, hts)]
    zc, oc = _cfg_pair(initial_scale_power=12, window=3, hysteresis=2, min_scale=1.0)
    ls = z.new_loss_scale()
    z.zero_loss_scale_init(zc, ls)
    ref = oracle.loss_scale_init(oc)
    ws = z.workspace(z.zero_offload_workspace_bytes(ots, M))
    hws = z.host_workspace(z.zero_offload_host_workspace_bytes(ots))
    state = hts
    plan = _run_plan(sizes, M)
    t = 1
    records = []
    seen = set()
    for k in range(10):
        where = plan.get(k, [])
        old = _inject(dts, state, where)
        hp = z.HParams(step=t, max_grad_norm=5.0)
        r = z.zero_offload_step_amp(ots, hp, zc, ls, 0.0, ws, hws, 3)
        torch.cuda.synchronize()
        state, ro, ref = oracle.zero_step_amp(state, hp_oracle(hp), oc, ref)
        assert r["status"] == 0
        assert (r["found_inf"], r["skipped"]) == (ro.found_inf, ro.skipped) == (int(bool(where)),) * 2, k
        if not where:
            assert math.isclose(r["sumsq"], ro.sumsq, rel_tol=1e-9), (k, r, ro)
            t += 1
            records.append((r, ro))  # the steps that updated the state
        _same_state(z.read_loss_scale(ls), ref, f"step {k}")
        seen.add(ref.scale)
        for o, h in zip(ots, state):
            assert_state_matches(o.master.numpy(), o.exp_avg.numpy(), o.exp_avg_sq.numpy(), to_np_u16(o.param_out),
                                 h.master, h.exp_avg, h.exp_avg_sq, h.param_out, f"step {k}",
                                 ulp_max=ulp_gate(*records))
        _restore(dts, state, where, old)
    assert seen == {2048.0, 4096.0}  # halved on the second overflow in a row, doubled after 3 clean steps
