"""HIP graph capture of the step. The plan tables reach the workspace through
small kernels (no host copy, no memset), and the fold's last workgroup
re-arms its arrival counter, so a captured step replays as a step. Each test
captures after one eager warm-up call (the plan is then cached), replays the
graph several times with eager work and synchronizations in between, and
checks every replay bit for bit against the same call made eagerly on a twin
copy of the inputs. The hyperparameters are captured with the launches: a
replay repeats the captured step counter t."""
import numpy as np
import pytest
import torch

import sharded_optimizer_step_amd as z
from cases import Case, bits_equal, build, to_np_f32, to_np_u16

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    z.lib()
    torch.cuda.set_device(0)
    yield
    torch.cuda.empty_cache()


def same_state(a, b, where):
    for i, (x, y) in enumerate(zip(a, b)):
        for nm in ("master", "exp_avg", "exp_avg_sq"):
            assert bits_equal(to_np_f32(getattr(x, nm)), to_np_f32(getattr(y, nm))), f"{where} t{i} {nm}"
        assert np.array_equal(to_np_u16(x.param_out), to_np_u16(y.param_out)), f"{where} t{i} out"


def eager_work():
    # unrelated work of the program between replays, then a full synchronization
    x = torch.randn(1 << 20, device="cuda")
    (x * 2.0 + 1.0).sum().item()
    torch.cuda.synchronize()


def capture(fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("max_norm,skip", [(0.0, 0), (0.05, 1)])
def test_captured_zero_step_replays_like_eager_calls(max_norm, skip):
    M = 4
    case = Case([100_003, 4099, 512, 1], M, seed=700)
    d_eager, _ = build(case)
    d_graph, _ = build(case)
    hp = z.HParams(step=7, max_grad_norm=max_norm, skip_on_nonfinite=skip)
    ws_e = z.workspace(z.zero_step_workspace_bytes(d_eager, M, hp))
    ws_g = z.workspace(z.zero_step_workspace_bytes(d_graph, M, hp))
    res_e, res_g = z.new_result(), z.new_result()
    z.zero_step(d_eager, hp, 0.0, ws_e, res_e)
    z.zero_step(d_graph, hp, 0.0, ws_g, res_g)  # warm-up: the plan is uploaded outside the graph
    torch.cuda.synchronize()
    g = capture(lambda: z.zero_step(d_graph, hp, 0.0, ws_g, res_g))
    same_state(d_eager, d_graph, "after capture (nothing ran)")
    for k in range(REPLAYS):
        g.replay()
        z.zero_step(d_eager, hp, 0.0, ws_e, res_e)
        eager_work()
        same_state(d_eager, d_graph, f"replay {k}")
        re, rg = z.read_result(res_e), z.read_result(res_g)
        assert re == rg and rg["status"] == 0, (k, re, rg)


def test_captured_amp_step_moves_the_loss_scale_like_eager_calls():
    M = 3
    case = Case([70_001, 2049], M, seed=710, grad_std=1e-3 * 4096)
    d_eager, _ = build(case)
    d_graph, _ = build(case)
    hp = z.HParams(step=11, max_grad_norm=0.5)
    cfg = z.LossScaleConfig(initial_scale_power=12, window=2, hysteresis=1, min_scale=1.0)
    ls_e, ls_g = z.new_loss_scale(), z.new_loss_scale()
    z.zero_loss_scale_init(cfg, ls_e)
    z.zero_loss_scale_init(cfg, ls_g)
    ws_e = z.workspace(z.zero_step_amp_workspace_bytes(d_eager, M, hp))
    ws_g = z.workspace(z.zero_step_amp_workspace_bytes(d_graph, M, hp))
    res_e, res_g = z.new_result(), z.new_result()
    z.zero_step_amp(d_eager, hp, cfg, ls_e, 0.0, ws_e, res_e)
    z.zero_step_amp(d_graph, hp, cfg, ls_g, 0.0, ws_g, res_g)
    torch.cuda.synchronize()
    g = capture(lambda: z.zero_step_amp(d_graph, hp, cfg, ls_g, 0.0, ws_g, res_g))
    scales = set()
    for k in range(REPLAYS):
        g.replay()
        z.zero_step_amp(d_eager, hp, cfg, ls_e, 0.0, ws_e, res_e)
        eager_work()
        same_state(d_eager, d_graph, f"replay {k}")
        assert z.read_result(res_e) == z.read_result(res_g)
        le, lg = z.read_loss_scale(ls_e), z.read_loss_scale(ls_g)
        assert le == lg, (k, le, lg)
        scales.add(lg["scale"])
    assert len(scales) > 1  # window 2: the scale doubles during the replays


def test_captured_zero2_step_replays_like_eager_calls():
    M = 2
    sizes = [40_000, 3001, 65_537]
    case = Case(sizes, M, seed=720)
    sides = []
    for _ in range(2):
        dts, _ = build(case)
        accs = [torch.empty(n, dtype=torch.float32, device="cuda") for n in sizes]
        parts = z.new_bucket_partials(2)
        # two buckets in backward order: the last tensor, then the first two
        buckets = [[2], [0, 1]]
        reducers = [z.BucketReducer([z.GradShard(dts[t].grads, accs[t]) for t in b],
                                    parts[32 * i:32 * i + 32]) for i, b in enumerate(buckets)]
        ats = [z.AccTensor(a, d.master, d.exp_avg, d.exp_avg_sq, d.param_out) for a, d in zip(accs, dts)]
        ws = z.workspace(z.zero_step_accumulated_workspace_bytes(ats))
        sides.append((dts, accs, parts, reducers, ats, ws, z.new_result()))
    hp = z.HParams(step=9, max_grad_norm=0.02)

    def step(side):
        dts, accs, parts, reducers, ats, ws, res = side
        for mb in range(2):  # two micro-batches (the same replicas twice)
            flags = (z.BUCKET_ACCUMULATE if mb else 0) | (z.BUCKET_FINAL if mb == 1 else 0)
            for r in reducers:
                r.reduce(flags, hp.grad_scale, 5)
        z.zero_step_accumulated(ats, hp, parts, 2, 5, 0.0, ws, res)

    step(sides[0])
    step(sides[1])
    torch.cuda.synchronize()
    g = capture(lambda: step(sides[1]))
    for k in range(REPLAYS):
        g.replay()
        step(sides[0])
        eager_work()
        same_state(sides[0][0], sides[1][0], f"replay {k}")
        for a, b in zip(sides[0][1], sides[1][1]):
            assert bits_equal(to_np_f32(a), to_np_f32(b)), f"replay {k} accumulator"
        re, rg = z.read_result(sides[0][6]), z.read_result(sides[1][6])
        assert re == rg and rg["status"] == 0, (k, re, rg)


@pytest.mark.parametrize("max_norm", [0.0, 0.05])
def test_captured_noalloc_step_replays_like_eager_calls(max_norm):
    # zero_step_noalloc (the plan in the library's static scratch) captured
    # after one eager warm-up call, replayed against zero_step with a caller
    # workspace made eagerly on a twin
    M = 4
    case = Case([100_003, 4099, 512, 1], M, seed=730)
    d_eager, _ = build(case)
    d_graph, _ = build(case)
    hp = z.HParams(step=8, max_grad_norm=max_norm)
    ws_e = z.workspace(z.zero_step_workspace_bytes(d_eager, M, hp))
    res_e, res_g = z.new_result(), z.new_result()
    z.zero_step(d_eager, hp, 0.0, ws_e, res_e)
    z.zero_step_noalloc(d_graph, hp, 0.0, res_g)  # warm-up: the plan reaches the scratch outside the graph
    torch.cuda.synchronize()
    same_state(d_eager, d_graph, "warm-up")
    g = capture(lambda: z.zero_step_noalloc(d_graph, hp, 0.0, res_g))
    for k in range(REPLAYS):
        g.replay()
        z.zero_step(d_eager, hp, 0.0, ws_e, res_e)
        eager_work()
        same_state(d_eager, d_graph, f"replay {k}")
        re, rg = z.read_result(res_e), z.read_result(res_g)
        assert re == rg and rg["status"] == 0, (k, re, rg)


def test_captured_fused_bucket_pass_replays_like_eager_calls():
    # a bucket's fused final pass and the record from its partial, captured
    # together, against the same two calls made eagerly on a twin
    M = 8
    case = Case([70_001, 4099], M, seed=740)
    d_eager, _ = build(case)
    d_graph, _ = build(case)
    hp = z.HParams(step=12)
    parts_e, parts_g = z.new_bucket_partials(1), z.new_bucket_partials(1)
    se = z.BucketStepper([z.BucketTensor(d.grads, None, d.master, d.exp_avg, d.exp_avg_sq, d.param_out)
                          for d in d_eager], parts_e)
    sg = z.BucketStepper([z.BucketTensor(d.grads, None, d.master, d.exp_avg, d.exp_avg_sq, d.param_out)
                          for d in d_graph], parts_g)
    res_e, res_g = z.new_result(), z.new_result()

    def eager():
        se.step(0, hp, 33)
        z.zero_step_accumulated([], hp, parts_e, 1, 33, 0.0, None, res_e)

    def graphed():
        sg.step(0, hp, 33)
        z.zero_step_accumulated([], hp, parts_g, 1, 33, 0.0, None, res_g)

    eager()
    graphed()  # warm-up: the bucket's plan is uploaded outside the graph
    torch.cuda.synchronize()
    g = capture(graphed)
    for k in range(REPLAYS):
        g.replay()
        eager()
        eager_work()
        same_state(d_eager, d_graph, f"replay {k}")
        re, rg = z.read_result(res_e), z.read_result(res_g)
        assert re == rg and rg["status"] == 0, (k, re, rg)
