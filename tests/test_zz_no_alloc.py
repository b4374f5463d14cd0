"""zero_step_noalloc -- the step with the library's static device scratch as
its workspace -- against zero_step with a caller workspace, on the same
seeded inputs: calls in a row on different tensor lists (the second smaller
than the first, then the first list's size again), single-pass and two-pass
(clipping, so the scratch also holds the fp32 gradient), and a second step
on the same tensors (the plan already in the scratch). Every result record
and every element of the state must be bit-identical to zero_step's, and
zero_step's own result meets the oracle's parity gates."""
import numpy as np
import pytest
import torch

import oracle
import sharded_optimizer_step_amd as z
from cases import Case, assert_tensor_matches, build, hp_oracle, to_np_f32, to_np_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    z.lib()
    torch.cuda.set_device(0)
    yield


def _state(dts):
    return [(to_np_f32(d.master).view(np.uint32), to_np_f32(d.exp_avg).view(np.uint32),
             to_np_f32(d.exp_avg_sq).view(np.uint32), to_np_u16(d.param_out)) for d in dts]


def _same(a, b, where):
    for ta, tb in zip(a, b):
        for x, y, name in zip(ta, tb, ("master", "exp_avg", "exp_avg_sq", "param_out")):
            assert np.array_equal(x, y), f"{where}: {name} differs from zero_step's"


def _pair(sizes, M, hp, seed, steps=1):
    """The same case built twice: stepped through zero_step_noalloc and through
    zero_step; returns both records and states after each step, and the
    oracle's check of zero_step's first step."""
    case = Case(sizes, M, seed=seed)
    d_na, h = build(case)
    d_ws, _ = build(case)
    ws = z.workspace(z.zero_step_workspace_bytes(d_ws, M, hp))
    for k in range(steps):
        hp.step = 3 + k
        r_na, r_ws = z.new_result(), z.new_result()
        z.zero_step_noalloc(d_na, hp, 0.0, r_na)
        z.zero_step(d_ws, hp, 0.0, ws, r_ws)
        torch.cuda.synchronize()
        a, b = z.read_result(r_na), z.read_result(r_ws)
        where = f"sizes {sizes}, M {M}, clip {hp.max_grad_norm}, step {hp.step}"
        assert a == b, (where, a, b)
        assert a["status"] == 0 and a["skipped"] == 0, (where, a)
        _same(_state(d_na), _state(d_ws), where)
        if k == 0:
            new, ro = oracle.zero_step(h, hp_oracle(hp))
            for dt, ht in zip(d_ws, new):
                assert_tensor_matches(dt, ht, where)
            assert abs(a["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm
    return a


@pytest.mark.parametrize("clip", [0.0, 1.0])
def test_noalloc_matches_zero_step_on_calls_in_a_row(clip):
    big = [300_001, 70_000, 4099]
    small = [5000, 17]
    r1 = _pair(big, 8, z.HParams(max_grad_norm=clip), seed=61)
    if clip:
        assert r1["clip_coef"] < 1.0  # the clip is active, so the step ran in two passes
    _pair(small, 4, z.HParams(max_grad_norm=clip), seed=62)
    _pair(big, 8, z.HParams(max_grad_norm=clip), seed=63, steps=2)  # the second step reuses the plan in the scratch
