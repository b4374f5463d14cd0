"""GPU parity of the ZeRO-2 streaming entry points (zero_bucket_reduce,
zero_step_accumulated) against the CPU oracle, through the C ABI.

Gates: the fp32 accumulator bit-exact after every micro-batch (the fold and
the running sum are fixed-order binary32); found_inf bit-exact; the bucket
partial's sum of squares within the oracle's own error bound for its
index-order binary64 sum (sumsq_tol); master/m/v within max(2e-6 |ref|, 1e-7); the bf16 output within 1 ulp;
the norm within 1e-5 relative."""
import math

import numpy as np
import pytest
import torch

import bench
import oracle
import sharded_optimizer_step_amd as z
import synth
from cases import (Case, Stats, assert_state_matches, bits_equal, build, hp_oracle, host_inputs_at,
                   oracle_sumsq_streaming, sample_indices, to_np_f32, to_np_u16, ulp_gate)
from synth.workloads import workload, zero2_buckets

pytestmark = pytest.mark.gpu

A, F = z.BUCKET_ACCUMULATE, z.BUCKET_FINAL


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    z.lib()
    torch.cuda.set_device(0)
    yield
    torch.cuda.empty_cache()


def _buf(n, off, dtype, fill=None):
    base = torch.empty(n + off + 8, dtype=dtype, device="cuda")
    if fill is not None:
        base.fill_(fill)
    return base[off:off + n]


def micro_batch(sizes, M, k, seed, std=1e-3, offs=None):
    """Micro-batch k's replicas: (device bf16 tensors, host bf16 codes) per tensor."""
    dev, host = [], []
    for t, n in enumerate(sizes):
        d, h = [], []
        for r in range(M):
            st = synth.stream_id(synth.KIND_GRAD, t, r)
            g = _buf(n, offs[r] if offs else 0, torch.bfloat16)
            if n:
                synth.device_bf16(g, seed + 7919 * k, st, std)
            d.append(g)
            h.append(synth.host_bf16(n, seed + 7919 * k, st, std))
        dev.append(d)
        host.append(h)
    return dev, host


def accumulate_all(sizes, M, K, seed, scale=1.0, stamp=1, std=1e-3, offs=None, acc_off=0, check_each=True,
                   inject=None):
    """Runs K micro-batches of one bucket; returns (device accumulators,
    oracle accumulators, partial tensor). inject: (k, t, r, i, code)."""
    accs = [_buf(n, acc_off, torch.float32, float("nan")) for n in sizes]
    part = z.new_bucket_partials(1)
    ws = None
    want = [None] * len(sizes)
    for k in range(K):
        dev, host = micro_batch(sizes, M, k, seed, std, offs)
        if inject is not None and inject[0] == k:
            _, t, r, i, code = inject
            dev[t][r].view(torch.int16)[i] = np.int16(np.uint16(code).view(np.int16))
            host[t][r][i] = code
        shards = [z.GradShard(dev[t], accs[t]) for t in range(len(sizes))]
        if ws is None:
            ws = z.workspace(z.zero_bucket_reduce_workspace_bytes(shards, M))
        flags = (A if k > 0 else 0) | (F if k == K - 1 else 0)
        z.zero_bucket_reduce(shards, flags, scale, stamp, part, ws)
        want = [oracle.grad_accumulate(host[t], want[t] if k > 0 else None) for t in range(len(sizes))]
        if check_each or k == K - 1:
            for t in range(len(sizes)):
                got = to_np_f32(accs[t])
                nan = np.isnan(want[t])
                assert np.array_equal(np.isnan(got), nan), (k, t)
                assert bits_equal(got[~nan], want[t][~nan]), (k, t)
    return accs, want, part


def sumsq_tol(n: int) -> float:
    """Relative tolerance of a device sum of squares against the oracle's
    (a compensated sum, within about one rounding of the exact sum): the
    device adds the same exact squares in a fixed tree of binary64 adds,
    whose error is at most about log2(n) * 2^-53 of the sum; n * 2^-53 bounds
    it loosely."""
    return 1e-12 + n * 2.0**-53


def oracle_partial(want, scale):
    st = oracle.SumSq()
    for a in want:
        st.add((a * np.float32(scale)).astype(np.float32))
    return st.sumsq, st.found_inf


# ---------------------------------------------------------------- zero_bucket_reduce

@pytest.mark.parametrize("sizes,M,K,scale", [
    ([512, 4099, 100_003, 1, 70_001], 3, 3, 1.0),
    ([2_000_000], 8, 2, 2.0**-3),
    ([9_000_000], 2, 2, 1.0),        # 64Ki-element tiles (1024 threads x 8 vectors)
    ([70_001], 1, 3, 0.5),
    ([9_001, 3], 64, 1, 1.0 / 64),
    ([0, 5000, 0], 4, 2, 1.0),
])
def test_bucket_reduce_bit_exact(sizes, M, K, scale):
    accs, want, part = accumulate_all(sizes, M, K, seed=400 + M, scale=scale, stamp=77)
    p = z.read_bucket_partial(part)
    s, f = oracle_partial(want, scale)
    assert p["stamp"] == 77 and p["found_inf"] == f == 0 and p["reserved"] == 0
    assert p["grad_scale"] == np.float32(scale)
    assert math.isclose(p["sumsq"], s, rel_tol=sumsq_tol(sum(sizes))), (p, s)


@pytest.mark.parametrize("offs,acc_off", [([1, 1, 1], 1), ([3, 3, 3], 3), ([1, 2, 0], 0), ([0, 0, 0], 1)])
def test_bucket_reduce_unaligned_layouts(offs, acc_off):
    # bf16 offsets o and fp32 offset a share a 16-byte head h (h = -o mod 8,
    # h = -a mod 4) -> vector path with a scalar head; otherwise element by element
    accs, want, part = accumulate_all([9_999, 70_001], 3, 2, seed=410, offs=offs, acc_off=acc_off)
    s, f = oracle_partial(want, 1.0)
    assert math.isclose(z.read_bucket_partial(part)["sumsq"], s, rel_tol=sumsq_tol(80_000))


def test_bucket_reduce_flags_nonfinite_of_the_running_sum():
    # +inf in micro-batch 0 and -inf in micro-batch 1 at one element: the
    # running sum is NaN there and the final partial says so
    sizes, M = [5000, 3001], 2
    accs = [_buf(n, 0, torch.float32) for n in sizes]
    part = z.new_bucket_partials(1)
    ws = None
    want = [None, None]
    for k, code in ((0, 0x7F80), (1, 0xFF80)):
        dev, host = micro_batch(sizes, M, k, 420)
        dev[1][k].view(torch.int16)[123] = np.int16(np.uint16(code).view(np.int16))
        host[1][k][123] = code
        shards = [z.GradShard(dev[t], accs[t]) for t in range(2)]
        ws = ws if ws is not None else z.workspace(z.zero_bucket_reduce_workspace_bytes(shards, M))
        z.zero_bucket_reduce(shards, (A if k else 0) | (F if k else 0), 1.0, 9, part, ws)
        want = [oracle.grad_accumulate(host[t], want[t] if k else None) for t in range(2)]
    got = to_np_f32(accs[1])
    assert np.isnan(got[123]) and np.isnan(want[1][123])
    assert bits_equal(np.delete(got, 123), np.delete(want[1], 123))
    p = z.read_bucket_partial(part)
    assert p["found_inf"] == 1 and p["stamp"] == 9


def test_empty_final_bucket_writes_its_partial():
    part = z.new_bucket_partials(1)
    part.fill_(0xAB)
    acc = torch.empty(0, dtype=torch.float32, device="cuda")
    z.zero_bucket_reduce([z.GradShard([torch.empty(0, dtype=torch.bfloat16, device="cuda")] * 2, acc)], F, 0.25,
                         123, part, None)
    assert z.read_bucket_partial(part) == dict(sumsq=0.0, stamp=123, found_inf=0, grad_scale=0.25, reserved=0)


def test_bucket_reducer_matches_the_oracle():
    # the prepared form: the same replica tensors regenerated in place for
    # every micro-batch, so the marshalled pointers stay valid
    sizes, M, K = [4099, 100_003], 4, 3
    dev, _ = micro_batch(sizes, M, 0, 480)
    accs = [_buf(n, 0, torch.float32) for n in sizes]
    part = z.new_bucket_partials(1)
    rd = z.BucketReducer([z.GradShard(dev[t], accs[t]) for t in range(len(sizes))], part)
    want = [None] * len(sizes)
    for k in range(K):
        host = []
        for t, n in enumerate(sizes):
            host.append([])
            for r in range(M):
                st = synth.stream_id(synth.KIND_GRAD, t, r)
                synth.device_bf16(dev[t][r], 480 + 7919 * k, st, 1e-3)
                host[t].append(synth.host_bf16(n, 480 + 7919 * k, st, 1e-3))
        rd.reduce((A if k else 0) | (F if k == K - 1 else 0), 0.5, 11)
        want = [oracle.grad_accumulate(host[t], want[t] if k else None) for t in range(len(sizes))]
    for a, w_ in zip(accs, want):
        assert bits_equal(to_np_f32(a), w_)
    s, f = oracle_partial(want, 0.5)
    p = z.read_bucket_partial(part)
    assert p["stamp"] == 11 and p["found_inf"] == f == 0 and math.isclose(p["sumsq"], s, rel_tol=sumsq_tol(sum(sizes)))


# ---------------------------------------------------------------- zero_step_accumulated

def _acc_tensors(dts, accs):
    return [z.AccTensor(a, d.master, d.exp_avg, d.exp_avg_sq, d.param_out) for a, d in zip(accs, dts)]


def _run_buckets(sizes, M, K, seed, buckets, scale, stamp, std=1e-3):
    """Every bucket (list of tensor indices) through K micro-batches; returns
    (device accumulators, oracle accumulators, partials)."""
    parts = z.new_bucket_partials(len(buckets))
    accs = [_buf(n, 0, torch.float32, float("nan")) for n in sizes]
    want = [None] * len(sizes)
    wss = [None] * len(buckets)
    for k in range(K):
        dev, host = micro_batch(sizes, M, k, seed, std)
        for b, idx in enumerate(buckets):
            shards = [z.GradShard(dev[t], accs[t]) for t in idx]
            if wss[b] is None:
                wss[b] = z.workspace(z.zero_bucket_reduce_workspace_bytes(shards, M))
            flags = (A if k > 0 else 0) | (F if k == K - 1 else 0)
            z.zero_bucket_reduce(shards, flags, scale, stamp, parts[32 * b:32 * b + 32], wss[b])
        want = [oracle.grad_accumulate(host[t], want[t] if k > 0 else None) for t in range(len(sizes))]
    return accs, want, parts


@pytest.mark.parametrize("max_norm,skip,ext,scale", [(0.0, 0, 0.0, 1.0), (0.05, 0, 0.0, 1.0), (1.0, 1, 0.5, 0.25),
                                                     (0.01, 0, 2.0, 2.0**-4)])
def test_step_accumulated_matches_oracle(max_norm, skip, ext, scale):
    sizes, M, K = [512, 4099, 100_003, 1, 70_001], 4, 2
    case = Case(sizes, M, seed=430)
    dts, hts = build(case)
    buckets = [[4, 3], [2], [1, 0]]
    accs, want, parts = _run_buckets(sizes, M, K, 431, buckets, scale, stamp=5)
    hp = z.HParams(step=20, max_grad_norm=max_norm, skip_on_nonfinite=skip, grad_scale=scale)
    ats = _acc_tensors(dts, accs)
    ws = z.workspace(z.zero_step_accumulated_workspace_bytes(ats))
    res = z.new_result()
    z.zero_step_accumulated(ats, hp, parts, len(buckets), 5, ext, ws, res)
    r = z.read_result(res)
    new, ro = oracle.zero_step_accumulated(want, hts, hp_oracle(hp), ext)
    assert r["status"] == 0 and r["found_inf"] == ro.found_inf == 0 and r["skipped"] == 0
    assert math.isclose(r["sumsq"], ro.sumsq, rel_tol=sumsq_tol(sum(sizes)))
    assert abs(r["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm
    assert abs(r["clip_coef"] - ro.clip_coef) <= 1e-6 * ro.clip_coef
    if max_norm in (0.05, 0.01):
        assert ro.clip_coef < 1.0
    st = Stats()
    for t, (d, h) in enumerate(zip(dts, new)):
        assert_state_matches(to_np_f32(d.master), to_np_f32(d.exp_avg), to_np_f32(d.exp_avg_sq),
                             to_np_u16(d.param_out), h.master, h.exp_avg, h.exp_avg_sq, h.param_out, f"t{t}", st,
                             ulp_max=ulp_gate((r, ro)))
    # the step read the accumulators and left them as they were
    for a, w_ in zip(accs, want):
        assert bits_equal(to_np_f32(a), w_)
    print(st)


@pytest.mark.parametrize("M,sizes", [(8, [512, 4099, 100_003, 1, 70_001]), (64, [9_001, 2048])])
def test_one_micro_batch_equals_zero_step_bitwise(M, sizes):
    # ZeRO-2 with one micro-batch and no clipping computes exactly what the
    # fused ZeRO-1 step computes over the same replicas
    case = Case(sizes, M, seed=440)
    d1, _ = build(case)
    d2, _ = build(case)
    hp = z.HParams(step=33, grad_scale=0.5)
    res1 = z.new_result()
    z.zero_step(d1, hp, 0.0, z.workspace(z.zero_step_workspace_bytes(d1, M, hp)), res1)
    accs = [_buf(n, 0, torch.float32) for n in sizes]
    part = z.new_bucket_partials(1)
    shards = [z.GradShard(d.grads, a) for d, a in zip(d2, accs)]
    z.zero_bucket_reduce(shards, F, hp.grad_scale, 1, part, z.workspace(z.zero_bucket_reduce_workspace_bytes(shards, M)))
    ats = _acc_tensors(d2, accs)
    res2 = z.new_result()
    z.zero_step_accumulated(ats, hp, part, 1, 1, 0.0, z.workspace(z.zero_step_accumulated_workspace_bytes(ats)), res2)
    r1, r2 = z.read_result(res1), z.read_result(res2)
    assert r1["status"] == r2["status"] == 0
    assert math.isclose(r1["sumsq"], r2["sumsq"], rel_tol=sumsq_tol(sum(sizes)))
    for a, b in zip(d1, d2):
        for f in ("master", "exp_avg", "exp_avg_sq"):
            assert bits_equal(to_np_f32(getattr(a, f)), to_np_f32(getattr(b, f))), f
        assert np.array_equal(to_np_u16(a.param_out), to_np_u16(b.param_out))


@pytest.mark.parametrize("what", ["stamp", "scale", "missing"])
def test_partials_of_another_step_are_rejected(what):
    sizes, M = [4099, 20_000], 2
    case = Case(sizes, M, seed=450)
    dts, hts = build(case)
    accs, want, parts = _run_buckets(sizes, M, 1, 451, [[0], [1]], 1.0, stamp=41)
    hp = z.HParams(step=4)
    nb = 2
    if what == "stamp":
        stamp = 42
    elif what == "scale":
        stamp, hp.grad_scale = 41, 0.5
    else:  # a third bucket that no final reduce wrote
        stamp, nb = 41, 3
        parts = torch.cat([parts, torch.zeros(32, dtype=torch.uint8, device="cuda")])
    ats = _acc_tensors(dts, accs)
    res = z.new_result()
    z.zero_step_accumulated(ats, hp, parts, nb, stamp, 0.0, z.workspace(z.zero_step_accumulated_workspace_bytes(ats)),
                            res)
    r = z.read_result(res)
    assert r["status"] == z.ZERO_ERR_BUCKET_PARTIALS and r["skipped"] == 1
    for d, h in zip(dts, hts):
        assert bits_equal(to_np_f32(d.master), h.master) and bits_equal(to_np_f32(d.exp_avg_sq), h.exp_avg_sq)
        assert np.array_equal(to_np_u16(d.param_out), h.param_out)


def test_nonfinite_micro_batch_skips_the_step():
    sizes, M, K = [4099, 70_001], 3, 2
    case = Case(sizes, M, seed=460)
    dts, hts = build(case)
    accs, want, part = accumulate_all(sizes, M, K, seed=461, stamp=3, inject=(0, 1, 2, 65_000, 0x7F80))
    assert z.read_bucket_partial(part)["found_inf"] == 1
    hp = z.HParams(step=8, max_grad_norm=1.0, skip_on_nonfinite=1)
    ats = _acc_tensors(dts, accs)
    res = z.new_result()
    z.zero_step_accumulated(ats, hp, part, 1, 3, 0.0, z.workspace(z.zero_step_accumulated_workspace_bytes(ats)), res)
    r = z.read_result(res)
    assert r["status"] == 0 and r["found_inf"] == 1 and r["skipped"] == 1
    for d, h in zip(dts, hts):
        assert bits_equal(to_np_f32(d.master), h.master) and bits_equal(to_np_f32(d.exp_avg), h.exp_avg)
        assert np.array_equal(to_np_u16(d.param_out), h.param_out)


def test_consecutive_steps_reuse_the_bucket_workspaces():
    # each bucket keeps its workspace (tables uploaded once); the arrival
    # counter of every final pass is re-armed, so every step's partials and
    # records are its own
    sizes, M = [100_003, 4099, 777], 4
    case = Case(sizes, M, seed=470)
    dts, hts = build(case)
    buckets = [[2, 1], [0]]
    parts = z.new_bucket_partials(2)
    accs = [_buf(n, 0, torch.float32) for n in sizes]
    wss = [None, None]
    ats = _acc_tensors(dts, accs)
    sws = z.workspace(z.zero_step_accumulated_workspace_bytes(ats))
    res = z.new_result()
    state = hts
    records = []
    for step in range(1, 5):
        dev, host = micro_batch(sizes, M, step, 471)
        for b, idx in enumerate(buckets):
            shards = [z.GradShard(dev[t], accs[t]) for t in idx]
            wss[b] = wss[b] if wss[b] is not None else z.workspace(z.zero_bucket_reduce_workspace_bytes(shards, M))
            z.zero_bucket_reduce(shards, F, 1.0, 1000 + step, parts[32 * b:32 * b + 32], wss[b])
        hp = z.HParams(step=step, max_grad_norm=0.02)
        z.zero_step_accumulated(ats, hp, parts, 2, 1000 + step, 0.0, sws, res)
        r = z.read_result(res)
        want = [oracle.grad_accumulate(host[t]) for t in range(len(sizes))]
        state, ro = oracle.zero_step_accumulated(want, state, hp_oracle(hp))
        assert r["status"] == 0 and math.isclose(r["sumsq"], ro.sumsq, rel_tol=sumsq_tol(sum(sizes))), (step, r, ro)
        records.append((r, ro))
        for t, (d, h) in enumerate(zip(dts, state)):
            assert_state_matches(to_np_f32(d.master), to_np_f32(d.exp_avg), to_np_f32(d.exp_avg_sq),
                                 to_np_u16(d.param_out), h.master, h.exp_avg, h.exp_avg_sq, h.param_out,
                                 f"step {step} t{t}", ulp_max=ulp_gate(*records))


def test_empty_step_reports_the_external_norm():
    res = z.new_result()
    parts = z.new_bucket_partials(1)
    z.zero_bucket_reduce([], F, 1.0, 8, parts, None)
    z.zero_step_accumulated([], z.HParams(max_grad_norm=1.0), parts, 1, 8, 4.0, None, res)
    r = z.read_result(res)
    assert r["status"] == 0 and r["grad_norm"] == 2.0 and abs(r["clip_coef"] - 1.0 / (2.0 + 1e-6)) < 1e-15


# ---------------------------------------------------------------- full size

def test_llama_bucket_workload_streamed_in_backward_order():
    # the ragged 288-tensor Llama-7B-shaped shard, reduced bucket by bucket in
    # backward order (reduce_bucket_size 5e7), one micro-batch, then the step
    w = workload(3)
    tensors = bench.build_workload(w, 0)
    buckets = zero2_buckets(w)
    accs = [torch.empty(spec.n, dtype=torch.float32, device="cuda") for spec in w.tensors]
    parts = z.new_bucket_partials(len(buckets))
    hp = z.HParams(**w.hparams())
    for b, idx in enumerate(buckets):
        shards = [z.GradShard(tensors[t].grads, accs[t]) for t in idx]
        z.zero_bucket_reduce(shards, F, hp.grad_scale, 7, parts[32 * b:32 * b + 32],
                             z.workspace(z.zero_bucket_reduce_workspace_bytes(shards, w.M)))
    ats = _acc_tensors(tensors, accs)
    res = z.new_result()
    z.zero_step_accumulated(ats, hp, parts, len(buckets), 7, 0.0,
                            z.workspace(z.zero_step_accumulated_workspace_bytes(ats)), res)
    r = z.read_result(res)
    s, f = oracle_sumsq_streaming(w)
    assert r["status"] == 0 and r["found_inf"] == f == 0 and r["skipped"] == 0
    assert abs(r["grad_norm"] - math.sqrt(s)) <= 1e-5 * math.sqrt(s)
    rng = np.random.default_rng(33)
    st = Stats()
    for spec, dt, acc in zip(w.tensors, tensors, accs):
        idx = sample_indices(spec.n, rng, 400)
        grads, master, m, v = host_inputs_at(w, spec, idx)
        a = oracle.grad_accumulate(grads)
        sel = torch.from_numpy(idx).cuda()
        assert bits_equal(to_np_f32(acc[sel]), a), spec.name
        new, _ = oracle.zero_step_accumulated([a], [oracle.TensorState([], master, m, v, None)], hp_oracle(hp))
        h = new[0]
        assert_state_matches(to_np_f32(dt.master[sel]), to_np_f32(dt.exp_avg[sel]), to_np_f32(dt.exp_avg_sq[sel]),
                             to_np_u16(dt.param_out[sel]), h.master, h.exp_avg, h.exp_avg_sq, h.param_out, spec.name,
                             st)
    print(w.name, len(buckets), "buckets, norm", r["grad_norm"], math.sqrt(s), st)
