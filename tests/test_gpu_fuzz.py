"""Seeded random layouts through every form of the step, against the oracle.

Each case draws a ragged tensor list (sizes at and around the tile edges,
empty tensors, one element), a replica count, per-pointer element offsets
(one shared misalignment per tensor, or mixed offsets that force the
element-by-element path) and hyperparameters (clip on or off, skip, a scale),
then runs it through the fused step, the ZeRO-2 bucket reduce + accumulated
step, and the CPU-offloaded step. Gates as in the other parity tests. Eight
more cases draw lists large enough for the single-pass 16-vector geometries."""
import math

import numpy as np
import pytest
import torch

import oracle
import sharded_optimizer_step_amd as z
from cases import (Case, assert_state_matches, bits_equal, build, hp_oracle, to_np_f32, to_np_u16,
                   ulp_gate)

pytestmark = pytest.mark.gpu

EDGES = [0, 1, 7, 8, 9, 255, 2047, 2048, 2049, 8191, 16_385, 65_535, 65_537, 131_073]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    z.lib()
    torch.cuda.set_device(0)
    yield
    torch.cuda.empty_cache()


def draw(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 9))
    sizes = [int(rng.choice(EDGES)) if rng.random() < 0.6 else int(rng.integers(1, 200_000)) for _ in range(T)]
    M = int(rng.choice([1, 2, 3, 5, 8, 17, 64]))
    if M > 8:
        sizes = [min(s, 20_000) for s in sizes]
    offsets = []
    for _ in range(T):
        if rng.random() < 0.7:  # one shared misalignment: bf16 o, fp32 a with -o = -a (mod 4) -> vector path
            o = int(rng.integers(0, 8))
            a = o % 4 + 4 * int(rng.integers(0, 2))
            offsets.append([o] * M + [a, a, a, o])
        else:                   # mixed offsets -> element by element
            offsets.append([int(rng.integers(0, 8)) for _ in range(M + 4)])
    max_norm = float(rng.choice([0.0, 0.0, 0.05, 10.0]))
    skip = int(rng.random() < 0.3)
    scale = float(rng.choice([1.0, 0.5, 2.0**-10]))
    t = int(rng.choice([1, 2, 50, 1000]))
    return sizes, M, offsets, z.HParams(step=t, max_grad_norm=max_norm, skip_on_nonfinite=skip, grad_scale=scale)


def check_all(dts, hts, new, where, ulp_max):
    for i, (d, h) in enumerate(zip(dts, new)):
        assert_state_matches(to_np_f32(d.master), to_np_f32(d.exp_avg), to_np_f32(d.exp_avg_sq),
                             to_np_u16(d.param_out), h.master, h.exp_avg, h.exp_avg_sq, h.param_out, f"{where} t{i}",
                             ulp_max=ulp_max)


def check_record(r, ro, where):
    assert r["status"] == 0, (where, r)
    assert (r["found_inf"], r["skipped"]) == (ro.found_inf, ro.skipped), (where, r, ro)
    if ro.found_inf == 0:
        assert abs(r["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm + 1e-30, (where, r, ro)
        assert abs(r["clip_coef"] - ro.clip_coef) <= 1e-6 * ro.clip_coef, (where, r, ro)


@pytest.mark.parametrize("seed", range(64))
def test_random_layouts_through_every_form(seed):
    sizes, M, offsets, hp = draw(seed)
    std = 1e-3 / hp.grad_scale
    case = Case(sizes, M, seed=900 + seed, grad_std=std, offsets=offsets, zero_state=(hp.step == 1))
    where = f"seed {seed}: sizes {sizes}, M {M}, hp {hp}"

    # fused step
    dts, hts = build(case)
    res = z.new_result()
    z.zero_step(dts, hp, 0.0, z.workspace(z.zero_step_workspace_bytes(dts, M, hp)), res)
    new, ro = oracle.zero_step(hts, hp_oracle(hp))
    r = z.read_result(res)
    check_record(r, ro, "zero_step " + where)
    check_all(dts, hts, new, "zero_step " + where, ulp_gate((r, ro)))

    # ZeRO-2: one bucket per tensor (in reverse order), one micro-batch
    dts, hts = build(case)
    accs = []
    for n, off in zip(sizes, offsets):
        base = torch.empty(n + off[M] + 8, dtype=torch.float32, device="cuda")
        accs.append(base[off[M]:off[M] + n])
    parts = z.new_bucket_partials(len(sizes))
    for b, t in enumerate(reversed(range(len(sizes)))):
        sh = [z.GradShard(dts[t].grads, accs[t])]
        z.zero_bucket_reduce(sh, z.BUCKET_FINAL, hp.grad_scale, seed + 1, parts[32 * b:32 * b + 32],
                             z.workspace(z.zero_bucket_reduce_workspace_bytes(sh, M)))
    for a, h in zip(accs, hts):
        want = oracle.grad_accumulate(h.grads)
        got = to_np_f32(a)
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan) and bits_equal(got[~nan], want[~nan]), where
    ats = [z.AccTensor(a, d.master, d.exp_avg, d.exp_avg_sq, d.param_out) for a, d in zip(accs, dts)]
    z.zero_step_accumulated(ats, hp, parts, len(sizes), seed + 1, 0.0,
                            z.workspace(z.zero_step_accumulated_workspace_bytes(ats)), res)
    r = z.read_result(res)
    check_record(r, ro, "ZeRO-2 " + where)
    check_all(dts, hts, new, "ZeRO-2 " + where, ulp_gate((r, ro)))

    # CPU-offloaded
    dts, hts = build(case)
    ots = [z.OffloadTensor(d.grads, torch.from_numpy(h.master.copy()), torch.from_numpy(h.exp_avg.copy()),
                           torch.from_numpy(h.exp_avg_sq.copy()), d.param_out) for d, h in zip(dts, hts)]
    r = z.zero_offload_step(ots, hp, 0.0, z.workspace(z.zero_offload_workspace_bytes(ots, M)),
                            z.host_workspace(z.zero_offload_host_workspace_bytes(ots)), 3)
    torch.cuda.synchronize()
    check_record(r, ro, "offload " + where)
    for i, (o, h) in enumerate(zip(ots, new)):
        assert_state_matches(o.master.numpy(), o.exp_avg.numpy(), o.exp_avg_sq.numpy(), to_np_u16(o.param_out),
                             h.master, h.exp_avg, h.exp_avg_sq, h.param_out, f"offload {where} t{i}",
                             ulp_max=ulp_gate((r, ro)))


@pytest.mark.parametrize("seed", range(8))
def test_random_ragged_lists_on_the_long_burst_geometries(seed):
    # Single-pass steps whose lists are large enough (over two tiles per CU)
    # for the 16-vector geometries, with the update in pairs: every tensor's
    # last tile ends at a random vector, so pairs with one vector in the
    # shard and one past it occur at each tensor end; tensors of 1-8 elements
    # (no whole vector) and mixed offsets (element by element) share the
    # launch. Every element checked against the oracle.
    rng = np.random.default_rng(77_000 + seed)
    M = int(rng.choice([2, 3, 8, 17, 20]))
    tile = 32_768 if M <= 16 else 65_536
    sizes = []
    while sum(sizes) < 132 * tile:
        sizes.append(int(rng.integers(1, 3 * tile)))
    sizes += [int(rng.integers(1, 9)) for _ in range(2)]
    offsets = []
    for _ in sizes:
        if rng.random() < 0.8:
            o = int(rng.integers(0, 8))
            a = o % 4 + 4 * int(rng.integers(0, 2))
            offsets.append([o] * M + [a, a, a, o])
        else:
            offsets.append([int(rng.integers(0, 8)) for _ in range(M + 4)])
    hp = z.HParams(step=int(rng.choice([1, 10, 1000])), grad_scale=float(rng.choice([1.0, 0.5, 1.0 / 3.0])))
    case = Case(sizes, M, seed=950 + seed, grad_std=1e-3, offsets=offsets, zero_state=(hp.step == 1))
    where = f"seed {seed}: {len(sizes)} tensors, {sum(sizes)} elements, M {M}, hp {hp}"
    dts, hts = build(case)
    res = z.new_result()
    z.zero_step(dts, hp, 0.0, z.workspace(z.zero_step_workspace_bytes(dts, M, hp)), res)
    new, ro = oracle.zero_step(hts, hp_oracle(hp))
    r = z.read_result(res)
    check_record(r, ro, where)
    check_all(dts, hts, new, where, ulp_gate((r, ro)))
