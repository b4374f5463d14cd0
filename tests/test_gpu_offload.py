"""GPU parity of the CPU-offloaded step (zero_offload_step) through the C ABI:
the fold, flag and norm on the GPU, the AdamW update on host threads over
host-resident state, the bf16 shard copied back to the device.

Gates as for zero_step: master/m/v within max(2e-6 |ref|, 1e-7) of the oracle,
the bf16 output within 1 ulp, the norm within 1e-5 relative; and, since the
host evaluates the same binary64 formula as the GPU's update pass from the
same fold, the whole state bit-identical to zero_step's on the same inputs."""
import math

import numpy as np
import pytest
import torch

import oracle
import sharded_optimizer_step_amd as z
from cases import (Case, Stats, assert_state_matches, bits_equal, build, hp_oracle, to_np_f32, to_np_u16,
                   ulp_gate)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    z.lib()
    torch.cuda.set_device(0)
    yield
    torch.cuda.empty_cache()


def offload_tensors(dts, hts):
    """Device replicas and output from dts; host copies of the state from hts."""
    return [z.OffloadTensor(d.grads, torch.from_numpy(h.master.copy()), torch.from_numpy(h.exp_avg.copy()),
                            torch.from_numpy(h.exp_avg_sq.copy()), d.param_out) for d, h in zip(dts, hts)]


def run_offload(ots, hp, external=0.0, ws=None, hws=None, threads=0):
    M = len(ots[0].grads) if ots else 1
    ws = ws if ws is not None else z.workspace(z.zero_offload_workspace_bytes(ots, M))
    hws = hws if hws is not None else z.host_workspace(z.zero_offload_host_workspace_bytes(ots))
    r = z.zero_offload_step(ots, hp, external, ws, hws, threads)
    torch.cuda.synchronize()
    return r, ws, hws


def check_against(ots, new, where, ulp_max, stats=None):
    for t, (o, h) in enumerate(zip(ots, new)):
        assert_state_matches(o.master.numpy(), o.exp_avg.numpy(), o.exp_avg_sq.numpy(), to_np_u16(o.param_out),
                             h.master, h.exp_avg, h.exp_avg_sq, h.param_out, f"{where} t{t}", stats,
                             ulp_max=ulp_max)


@pytest.mark.parametrize("sizes,M,max_norm,scale,ext", [
    ([512, 4099, 100_003, 1, 70_001], 4, 0.0, 1.0, 0.0),
    ([9_000_001], 8, 0.5, 1.0, 0.0),          # three transfer-and-update chunks of 4Mi elements
    ([5000, 3], 64, 0.01, 1.0 / 64, 0.25),
    ([262_144], 1, 1.0, 2.0**-16, 0.0),
    ([70_001, 3, 5_000_000], 5, 0.0, 0.5, 1.75),  # no clipping: the pipelined fold, with the other ranks' sum
])
def test_offload_step_matches_the_oracle(sizes, M, max_norm, scale, ext):
    case = Case(sizes, M, seed=500 + M, grad_std=1e-3 / scale if scale < 1 else 1e-3)
    dts, hts = build(case)
    ots = offload_tensors(dts, hts)
    hp = z.HParams(step=12, max_grad_norm=max_norm, grad_scale=scale)
    r, _, _ = run_offload(ots, hp, ext, threads=5)
    new, ro = oracle.zero_step(hts, hp_oracle(hp), ext)
    assert r["status"] == 0 and r["found_inf"] == ro.found_inf == 0 and r["skipped"] == 0
    assert abs(r["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm
    assert abs(r["clip_coef"] - ro.clip_coef) <= 1e-6 * ro.clip_coef
    if max_norm in (0.5, 0.01):
        assert ro.clip_coef < 1.0
    st = Stats()
    check_against(ots, new, "offload", ulp_gate((r, ro)), st)
    print(st)


@pytest.mark.parametrize("max_norm", [0.0, 0.02])
def test_offload_step_equals_zero_step_bitwise(max_norm):
    sizes, M = [100_003, 4099, 777], 8
    case = Case(sizes, M, seed=510)
    d1, h1 = build(case)
    d2, h2 = build(case)
    hp = z.HParams(step=21, max_grad_norm=max_norm, skip_on_nonfinite=1)
    res = z.new_result()
    z.zero_step(d1, hp, 0.0, z.workspace(z.zero_step_workspace_bytes(d1, M, hp)), res)
    r1 = z.read_result(res)
    ots = offload_tensors(d2, h2)
    r2, _, _ = run_offload(ots, hp)
    assert r1["sumsq"] == r2["sumsq"] and r1["clip_coef"] == r2["clip_coef"]
    for a, o in zip(d1, ots):
        assert bits_equal(to_np_f32(a.master), o.master.numpy())
        assert bits_equal(to_np_f32(a.exp_avg), o.exp_avg.numpy())
        assert bits_equal(to_np_f32(a.exp_avg_sq), o.exp_avg_sq.numpy())
        assert np.array_equal(to_np_u16(a.param_out), to_np_u16(o.param_out))


def test_offload_skip_leaves_every_state_unchanged():
    sizes, M = [4099, 70_001], 3
    case = Case(sizes, M, seed=520)
    dts, hts = build(case)
    dts[1].grads[2].view(torch.int16)[60_000] = 0x7F80  # +inf
    ots = offload_tensors(dts, hts)
    hp = z.HParams(step=5, max_grad_norm=1.0, skip_on_nonfinite=1)
    r, _, _ = run_offload(ots, hp)
    assert r["status"] == 0 and r["found_inf"] == 1 and r["skipped"] == 1
    for o, h in zip(ots, hts):
        assert bits_equal(o.master.numpy(), h.master) and bits_equal(o.exp_avg_sq.numpy(), h.exp_avg_sq)
        assert np.array_equal(to_np_u16(o.param_out), h.param_out)


def test_consecutive_offload_steps_chain_like_the_oracle():
    sizes, M = [300_001, 512], 4
    case = Case(sizes, M, seed=530)
    dts, hts = build(case)
    ots = offload_tensors(dts, hts)
    ws = hws = None
    state = hts
    records = []
    for k, ext in enumerate([0.0, 1.5, 0.0]):
        hp = z.HParams(step=1 + k, max_grad_norm=0.05)
        r, ws, hws = run_offload(ots, hp, ext, ws, hws, threads=3)
        state, ro = oracle.zero_step(state, hp_oracle(hp), ext)
        records.append((r, ro))
        assert r["status"] == 0 and abs(r["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm
        check_against(ots, state, f"step {k}", ulp_gate(*records))


def test_empty_offload_step_reports_the_external_norm():
    ws = z.workspace(z.zero_offload_workspace_bytes([], 1))
    hws = z.host_workspace(z.zero_offload_host_workspace_bytes([]))
    r = z.zero_offload_step([], z.HParams(max_grad_norm=1.0), 9.0, ws, hws)
    assert r["status"] == 0 and r["grad_norm"] == 3.0 and abs(r["clip_coef"] - 1.0 / (3.0 + 1e-6)) < 1e-15


@pytest.mark.parametrize("sizes,M,scale", [([9_000_001, 70_001, 3], 8, 2.0**-10), ([2 * 4_194_304 + 5], 3, 1.0 / 3.0),
                                           ([5000, 1], 64, 1.0)])
def test_pipelined_offload_equals_zero_step(sizes, M, scale):
    # no clipping, no skip, a fixed scale: the fold runs chunk by chunk beside
    # the host update, the host applies grad_scale to the staged fold; the
    # state must be what zero_step gives, bit for bit, and the sum of squares
    # (combined chunk by chunk instead of tile by tile) within the rounding of
    # a binary64 sum
    case = Case(sizes, M, seed=540 + M, grad_std=1e-3 / scale if scale < 1 else 1e-3)
    d1, h1 = build(case)
    d2, h2 = build(case)
    hp = z.HParams(step=21, grad_scale=scale)
    res = z.new_result()
    z.zero_step(d1, hp, 0.0, z.workspace(z.zero_step_workspace_bytes(d1, M, hp)), res)
    r1 = z.read_result(res)
    ots = offload_tensors(d2, h2)
    r2, _, _ = run_offload(ots, hp, threads=4)
    assert r1["status"] == r2["status"] == 0 and r1["found_inf"] == r2["found_inf"] == 0 and r2["skipped"] == 0
    n = sum(sizes)
    assert abs(r1["sumsq"] - r2["sumsq"]) <= (1e-12 + n * 2.0**-53) * r1["sumsq"]
    for a, o in zip(d1, ots):
        assert bits_equal(to_np_f32(a.master), o.master.numpy())
        assert bits_equal(to_np_f32(a.exp_avg), o.exp_avg.numpy())
        assert bits_equal(to_np_f32(a.exp_avg_sq), o.exp_avg_sq.numpy())
        assert np.array_equal(to_np_u16(a.param_out), to_np_u16(o.param_out))


def test_pipelined_offload_detects_a_stale_workspace():
    sizes, M = [300_001, 4099], 4
    case = Case(sizes, M, seed=560)
    dts, hts = build(case)
    ots = offload_tensors(dts, hts)
    hp = z.HParams(step=3)
    r, ws, hws = run_offload(ots, hp)
    assert r["status"] == 0
    before = [(o.master.numpy().copy(), o.exp_avg_sq.numpy().copy(), to_np_u16(o.param_out).copy()) for o in ots]
    ws.zero_()  # the caller reuses the workspace for something else
    r, _, _ = run_offload(ots, hp, ws=ws, hws=hws)
    assert r["status"] == z.ZERO_ERR_STALE_WORKSPACE
    for o, (m0, v0, out0) in zip(ots, before):
        assert bits_equal(o.master.numpy(), m0) and bits_equal(o.exp_avg_sq.numpy(), v0)
        assert np.array_equal(to_np_u16(o.param_out), out0)
    z.zero_workspace_forget(ws)
    r, _, _ = run_offload(ots, hp, ws=ws, hws=hws)
    assert r["status"] == 0 and not bits_equal(ots[0].master.numpy(), before[0][0])
