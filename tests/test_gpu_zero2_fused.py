"""GPU parity of ZeRO-2's fused final pass (zero_bucket_step: a bucket's last
micro-batch folded, added to the accumulator, scaled and applied with AdamW
in one pass; then zero_step_accumulated with no tensors for the record)
against the CPU oracle's accumulated step, through the C ABI, and bit for
bit against the two-pass form (zero_bucket_reduce FINAL, then
zero_step_accumulated over the tensors) on the same inputs.

Gates: the state bit-identical to the two-pass form's and within the parity
gates of the oracle's (stated tolerance, 4 binary32 ulps, 1 bf16 ulp); the
accumulator untouched; found_inf exact; the norm within 1e-5 of the
oracle's."""
import math

import numpy as np
import pytest
import torch

import oracle
import sharded_optimizer_step_amd as z
import synth
from cases import Case, Stats, assert_state_matches, bits_equal, build, hp_oracle, to_np_f32, to_np_u16

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


def _buf(n, off, dtype):
    base = torch.empty(n + off + 8, dtype=dtype, device="cuda")
    return base[off:off + n]


def micro_batch(sizes, M, k, seed, offs):
    """Micro-batch k's replicas: (device bf16 tensors, host bf16 codes) per tensor."""
    dev, host = [], []
    for t, n in enumerate(sizes):
        d, h = [], []
        for r in range(M):
            st = synth.stream_id(synth.KIND_GRAD, t, r)
            g = _buf(n, offs[t][r], torch.bfloat16)
            if n:
                synth.device_bf16(g, seed + 7919 * k, st, 1e-3)
            d.append(g)
            h.append(synth.host_bf16(n, seed + 7919 * k, st, 1e-3))
        dev.append(d)
        host.append(h)
    return dev, host


def _state(dts):
    return [(to_np_f32(d.master).view(np.uint32), to_np_f32(d.exp_avg).view(np.uint32),
             to_np_f32(d.exp_avg_sq).view(np.uint32), to_np_u16(d.param_out)) for d in dts]


def run_both(sizes, M, K, buckets, hp, seed, offs=None, inject=None, extra_flags=0):
    """K micro-batches of every bucket through (1) zero_bucket_reduce for the
    first K-1 and zero_bucket_step for the last, and (2) zero_bucket_reduce
    for all K then zero_step_accumulated, on two copies of the same state.
    Returns (records 1 and 2, device tensors 1, accumulators 1 as they were
    before the fused pass and after it, oracle state and result)."""
    offs = offs or [[0] * (M + 5) for _ in sizes]
    case = Case(sizes, M, seed=seed, offsets=[o[:M + 4] for o in offs])
    d1, hts = build(case)
    d2, _ = build(case)
    acc1 = [_buf(n, offs[t][M + 4], torch.float32) for t, n in enumerate(sizes)]
    acc2 = [_buf(n, offs[t][M + 4], torch.float32) for t, n in enumerate(sizes)]
    nb = len(buckets)
    p1, p2 = z.new_bucket_partials(nb), z.new_bucket_partials(nb)
    want = [None] * len(sizes)
    acc_before = None
    stamp = 500 + seed
    for k in range(K):
        dev, host = micro_batch(sizes, M, k, seed, offs)
        if inject is not None and inject[0] == k:
            _, t, r, i, code = inject
            dev[t][r].view(torch.int16)[i] = np.int16(np.uint16(code).view(np.int16))
            host[t][r][i] = code
        last = k == K - 1
        for b, idx in enumerate(buckets):
            flags = (A if k else 0) | (F if last else 0)
            z.zero_bucket_reduce([z.GradShard(dev[t], acc2[t]) for t in idx], flags, hp.grad_scale, stamp,
                                 p2[32 * b:32 * b + 32],
                                 z.workspace(z.zero_bucket_reduce_workspace_bytes(
                                     [z.GradShard(dev[t], acc2[t]) for t in idx], M)))
            if not last:
                z.zero_bucket_reduce([z.GradShard(dev[t], acc1[t]) for t in idx], flags, hp.grad_scale, stamp,
                                     None, z.workspace(z.zero_bucket_reduce_workspace_bytes(
                                         [z.GradShard(dev[t], acc1[t]) for t in idx], M)))
            else:
                if acc_before is None:
                    torch.cuda.synchronize()
                    acc_before = [to_np_f32(a).copy() for a in acc1]
                bts = [z.BucketTensor(dev[t], acc1[t] if k else None, d1[t].master, d1[t].exp_avg,
                                      d1[t].exp_avg_sq, d1[t].param_out) for t in idx]
                z.zero_bucket_step(bts, (A if k else 0) | extra_flags, hp, stamp, p1[32 * b:32 * b + 32],
                                   z.workspace(z.zero_bucket_step_workspace_bytes(bts, M)))
        want = [oracle.grad_accumulate(host[t], want[t] if k else None) for t in range(len(sizes))]
    r1, r2 = z.new_result(), z.new_result()
    z.zero_step_accumulated([], hp, p1, nb, stamp, 0.0, None, r1)
    ats = [z.AccTensor(a, d.master, d.exp_avg, d.exp_avg_sq, d.param_out) for a, d in zip(acc2, d2)]
    z.zero_step_accumulated(ats, hp, p2, nb, stamp, 0.0, z.workspace(z.zero_step_accumulated_workspace_bytes(ats)),
                            r2)
    new, ro = oracle.zero_step_accumulated(want, hts, hp_oracle(hp))
    torch.cuda.synchronize()
    return z.read_result(r1), z.read_result(r2), d1, d2, acc1, acc_before, new, ro


@pytest.mark.parametrize("sizes,M,K,buckets,scale", [
    ([512, 4099, 100_003, 1, 70_001], 4, 1, [[4, 3], [2], [1, 0]], 1.0),
    ([512, 4099, 100_003, 1, 70_001], 4, 2, [[4, 3], [2], [1, 0]], 0.25),
    ([300_001, 7, 2049], 8, 3, [[0, 1, 2]], 1.0 / 3.0),
    ([9_001, 2048], 64, 2, [[1], [0]], 1.0 / 64),
    ([8_400_000, 4099], 8, 2, [[0], [1]], 1.0),    # 257 tiles of 32768 elements: 256 x 16, paired update
    ([8_400_000], 20, 1, [[0]], 0.5),              # M > 16: 129 tiles of 65536 elements, 512 x 16
    ([8_400_000], 20, 2, [[0]], 0.5),              # the same, accumulating
    ([0, 5000, 0], 2, 2, [[0], [1, 2]], 1.0),
])
def test_fused_final_pass_matches_the_oracle_and_the_two_pass_form(sizes, M, K, buckets, scale):
    hp = z.HParams(step=17, grad_scale=scale)
    r1, r2, d1, d2, acc1, acc_before, new, ro = run_both(sizes, M, K, buckets, hp, seed=600 + M + K)
    where = f"sizes {sizes}, M {M}, K {K}"
    assert r1["status"] == r2["status"] == 0 and r1["found_inf"] == r2["found_inf"] == ro.found_inf == 0
    assert r1["skipped"] == 0 and r1["clip_coef"] == 1.0
    assert abs(r1["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm + 1e-30, (where, r1, ro)
    assert math.isclose(r1["sumsq"], r2["sumsq"], rel_tol=1e-12), (where, r1, r2)
    for t, (a, b) in enumerate(zip(_state(d1), _state(d2))):
        for x, y, nm in zip(a, b, ("master", "exp_avg", "exp_avg_sq", "param_out")):
            assert np.array_equal(x, y), f"{where}: tensor {t} {nm} differs from the two-pass form"
    st = Stats()
    for t, (d, h) in enumerate(zip(d1, new)):
        assert_state_matches(to_np_f32(d.master), to_np_f32(d.exp_avg), to_np_f32(d.exp_avg_sq),
                             to_np_u16(d.param_out), h.master, h.exp_avg, h.exp_avg_sq, h.param_out,
                             f"{where} t{t}", st)
    for a, b in zip(acc1, acc_before):  # the fused pass reads the accumulator and leaves it as it was
        assert bits_equal(to_np_f32(a), b)
    print(where, st)


@pytest.mark.parametrize("sizes,M,K,buckets", [
    ([8_400_000, 4099], 8, 2, [[0], [1]]),   # 256 x 16, paired update, a half-filled last block
    ([8_400_000, 70_001], 20, 1, [[1, 0]]),  # 512 x 16
    ([70_001, 5, 4099], 4, 2, [[0, 1, 2]]),  # too few tiles for 16 vectors per thread: the per-vector path
])
def test_fused_final_pass_with_streamed_state_stores(sizes, M, K, buckets):
    # ZERO_BUCKET_STREAM_STORES changes only the cache policy of the state
    # stores: the state stays bit-identical to the two-pass form's
    hp = z.HParams(step=9, grad_scale=0.5)
    r1, r2, d1, d2, acc1, acc_before, new, ro = run_both(sizes, M, K, buckets, hp, seed=640 + M,
                                                         extra_flags=z.BUCKET_STREAM_STORES)
    where = f"sizes {sizes}, M {M}, K {K}, streamed"
    assert r1["status"] == 0 and r1["found_inf"] == ro.found_inf == 0
    assert math.isclose(r1["sumsq"], r2["sumsq"], rel_tol=1e-12), (where, r1, r2)
    for t, (a, b) in enumerate(zip(_state(d1), _state(d2))):
        for x, y, nm in zip(a, b, ("master", "exp_avg", "exp_avg_sq", "param_out")):
            assert np.array_equal(x, y), f"{where}: tensor {t} {nm} differs from the two-pass form"
    for t, (d, h) in enumerate(zip(d1, new)):
        assert_state_matches(to_np_f32(d.master), to_np_f32(d.exp_avg), to_np_f32(d.exp_avg_sq),
                             to_np_u16(d.param_out), h.master, h.exp_avg, h.exp_avg_sq, h.param_out,
                             f"{where} t{t}")


@pytest.mark.parametrize("offs", [
    # a shared misalignment (bf16 offset o, fp32 offset o mod 4): the vector path with a scalar head and tail
    [[3] * 4 + [3, 3, 3, 3, 3], [5] * 4 + [1, 1, 1, 5, 1]],
    # offsets that disagree: element by element
    [[1, 2, 3, 0, 0, 1, 2, 3, 2], [0, 0, 0, 0, 1, 0, 0, 0, 0]],
])
def test_fused_final_pass_on_unaligned_layouts(offs):
    sizes, M = [70_001, 4099], 4
    hp = z.HParams(step=3)
    r1, r2, d1, d2, acc1, acc_before, new, ro = run_both(sizes, M, 2, [[0, 1]], hp, seed=620, offs=offs)
    assert r1["status"] == 0 and r1["found_inf"] == 0
    for a, b in zip(_state(d1), _state(d2)):
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
    for t, (d, h) in enumerate(zip(d1, new)):
        assert_state_matches(to_np_f32(d.master), to_np_f32(d.exp_avg), to_np_f32(d.exp_avg_sq),
                             to_np_u16(d.param_out), h.master, h.exp_avg, h.exp_avg_sq, h.param_out, f"t{t}")


def test_fused_final_pass_flags_a_nonfinite_gradient_and_still_applies_it():
    # no skipping in the fused form: +inf in the last micro-batch is flagged in
    # the partial and the record, and the update runs as zero_step's would
    sizes, M = [20_000, 513], 4
    hp = z.HParams(step=9)
    r1, r2, d1, d2, acc1, acc_before, new, ro = run_both(sizes, M, 2, [[1], [0]], hp, seed=630,
                                                         inject=(1, 0, 2, 777, 0x7F80))
    assert r1["found_inf"] == r2["found_inf"] == ro.found_inf == 1
    assert r1["skipped"] == 0 and ro.skipped == 0
    m1 = to_np_f32(d1[0].master)
    assert not np.isfinite(m1[777])
    for a, b in zip(_state(d1), _state(d2)):
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
    for t, (d, h) in enumerate(zip(d1, new)):
        assert_state_matches(to_np_f32(d.master), to_np_f32(d.exp_avg), to_np_f32(d.exp_avg_sq),
                             to_np_u16(d.param_out), h.master, h.exp_avg, h.exp_avg_sq, h.param_out, f"t{t}")


def test_fused_final_pass_refuses_clipping_and_skipping():
    case = Case([1000], 2, seed=640)
    d, _ = build(case)
    bts = [z.BucketTensor(d[0].grads, None, d[0].master, d[0].exp_avg, d[0].exp_avg_sq, d[0].param_out)]
    part = z.new_bucket_partials(1)
    ws = z.workspace(z.zero_bucket_step_workspace_bytes(bts, 2))
    before = _state(d)
    for hp in (z.HParams(max_grad_norm=1.0), z.HParams(skip_on_nonfinite=1)):
        with pytest.raises(z.ZeroError) as e:
            z.zero_bucket_step(bts, 0, hp, 1, part, ws)
        assert e.value.status == z.ZERO_ERR_INVALID_ARGUMENT
    with pytest.raises(z.ZeroError):
        z.zero_bucket_step(bts, A, z.HParams(), 1, part, ws)  # accumulating without an accumulator
    with pytest.raises(z.ZeroError):
        z.zero_bucket_step(bts, F, z.HParams(), 1, part, ws)  # FINAL is implied, not a flag here
    torch.cuda.synchronize()
    for x, y in zip(_state(d)[0], before[0]):
        assert np.array_equal(x, y)


def test_bucket_stepper_runs_consecutive_steps():
    # the prepared form, two steps in a row on one workspace (the plan cached
    # there), the record of each from its bucket partials
    sizes, M = [100_003, 4099], 8
    case = Case(sizes, M, seed=650)
    d, hts = build(case)
    part = z.new_bucket_partials(1)
    stepper = z.BucketStepper([z.BucketTensor(x.grads, None, x.master, x.exp_avg, x.exp_avg_sq, x.param_out)
                               for x in d], part)
    state = hts
    for k in range(2):
        hp = z.HParams(step=4 + k)
        stepper.step(0, hp, 70 + k)
        res = z.new_result()
        z.zero_step_accumulated([], hp, part, 1, 70 + k, 0.0, None, res)
        r = z.read_result(res)
        state, ro = oracle.zero_step(state, hp_oracle(hp))
        assert r["status"] == 0 and abs(r["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm
        for t, (x, h) in enumerate(zip(d, state)):
            assert_state_matches(to_np_f32(x.master), to_np_f32(x.exp_avg), to_np_f32(x.exp_avg_sq),
                                 to_np_u16(x.param_out), h.master, h.exp_avg, h.exp_avg_sq, h.param_out,
                                 f"step {k} t{t}")
