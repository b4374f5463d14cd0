"""Pins of the oracle's ZeRO-2 streaming step (CPU only).

"CS336 Lecture 7: Parallelism 1", section "ZeRO Stage 2": as backward
produces each layer's gradient, it is reduced straight to the rank that owns
that shard, so no rank ever holds a whole gradient; gsyq.cn/news/457874
section 4.2 groups gradients in buckets (reduce_bucket_size) over
gradient_accumulation_steps micro-batches. The oracle keeps the shard's
gradient as a binary32 running sum of reduce-scatter results and then runs
the ZeRO-1 step on g = acc * scale32.

What pins it, other than itself:

* accumulation rule -> an exact rational emulation of binary32 addition
                       (IEEE 754 round-to-nearest-even, from the definition);
                       an order pin whose three candidate readings give three
                       different answers.
* one micro-batch   -> the ZeRO-1 step over the same replicas (itself pinned to
                       torch's AdamW, clip_grad_norm_ and exact arithmetic),
                       bit for bit.
* K micro-batches   -> on inputs where every add is exact, the step equals the
                       ZeRO-1 step over all K*M replicas as one large batch
                       (gradient accumulation is a larger batch).
* skip              -> an inf in any micro-batch skips the step, state unchanged.
* memory            -> the ZeRO-2 row of the per-parameter accounting.
"""
import ctypes
import math

import numpy as np
import pytest

import oracle
from test_oracle_pins import F32, bits32, random_bf16, torch_bf16_to_f32


def _bf16_of(vals) -> np.ndarray:
    h = oracle.f32_to_bf16(np.asarray(vals, np.float32))
    assert np.array_equal(oracle.bf16_to_f32(h), np.asarray(vals, np.float32)), "not exact in bf16"
    return h


def _accumulate(micro_batches):
    """micro_batches[k] = M replica arrays; returns the oracle's accumulator."""
    acc = None
    for grads in micro_batches:
        acc = oracle.grad_accumulate(grads, acc)
    return acc


def _state(n, rng):
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-5).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-8).astype(np.float32)
    return th, m, v


def _tensors(sizes, M, rng, std=1e-3):
    out = []
    for n in sizes:
        th, m, v = _state(n, rng)
        grads = [oracle.f32_to_bf16((rng.standard_normal(n) * std).astype(np.float32)) for _ in range(M)]
        out.append(oracle.TensorState(grads, th, m, v, np.full(n, 0x1234, np.uint16)))
    return out


def _same_state(a, b):
    for f in ("master", "exp_avg", "exp_avg_sq", "param_out"):
        x, y = getattr(a, f), getattr(b, f)
        if not np.array_equal(np.ascontiguousarray(x).view(np.uint8), np.ascontiguousarray(y).view(np.uint8)):
            return False
    return True


# --------------------------------------------------------------------------
# The accumulation rule
# --------------------------------------------------------------------------

def test_accumulation_order_pin():
    # Micro-batch 1 replicas (1, 0), micro-batch 2 replicas (2^-24, 2^-24):
    #   sum of reduce-scatter results: 1 + (2^-24 + 2^-24) = 1 + 2^-23
    #   one fold continued across micro-batches: ((1 + 0) + 2^-24) + 2^-24 = 1
    #   each rank's micro-batches first: (1 + 2^-24) + (0 + 2^-24) = 1 + 2^-24 -> 1
    # Element 1 swaps the roles so that a dropped micro-batch shows too.
    mb1 = [_bf16_of([1.0, 2**-24]), _bf16_of([0.0, 2**-24])]
    mb2 = [_bf16_of([2**-24, 1.0]), _bf16_of([2**-24, 0.0])]
    acc = _accumulate([mb1, mb2])
    assert acc[0] == np.float32(1.0 + 2.0**-23)
    assert acc[1] == np.float32(1.0 + 2.0**-23)


@pytest.mark.parametrize("case", range(60))
def test_accumulate_matches_exact_binary32_emulation(case):
    rng = np.random.default_rng(3000 + case)
    M = [1, 2, 3, 8][case % 4]
    K = [1, 2, 3, 5][(case // 4) % 4]
    n = int(rng.integers(16, 65))
    if case % 3 == 0:
        mbs = [[random_bf16(n, 110, 118, rng=rng) for _ in range(M)] for _ in range(K)]
    elif case % 3 == 1:
        mbs = [[random_bf16(n, 60, 180, rng=rng) for _ in range(M)] for _ in range(K)]
    else:
        mbs = [[random_bf16(n, 0, 4, p_sub=0.3, p_zero=0.2, rng=rng) for _ in range(M)] for _ in range(K)]
    got = _accumulate(mbs)
    vals = [[torch_bf16_to_f32(g) for g in grads] for grads in mbs]
    for i in range(n):
        acc = None
        for k in range(K):
            s = F32.of(float(vals[k][0][i]))
            for r in range(1, M):
                s = s.add(F32.of(float(vals[k][r][i])))
            acc = s if acc is None else acc.add(s)
        assert acc.same_as(float(got[i])), (case, i)


def test_first_micro_batch_ignores_the_accumulator_contents():
    rng = np.random.default_rng(21)
    grads = [random_bf16(100, 100, 130, rng=rng) for _ in range(3)]
    acc = np.full(100, np.nan, np.float32)
    ptrs = (ctypes.c_void_p * 3)(*[g.ctypes.data for g in grads])
    oracle.lib().oracle_grad_accumulate(ptrs, 3, 100, acc.ctypes.data, 0)
    assert np.array_equal(bits32(acc), bits32(oracle.reduce(grads)))


# --------------------------------------------------------------------------
# The step from the accumulator
# --------------------------------------------------------------------------

# Scales 1/3 and 0.1 (a mean over three ranks; a non-dyadic factor) are not
# powers of two: the product with the binary32 scale rounds, so these cases
# also pin that the accumulated step unscales exactly as the ZeRO-1 step does,
# in binary32 with the scale rounded to binary32 once.
@pytest.mark.parametrize("max_norm,scale,skip", [(0.0, 1.0, 0), (1e-2, 1.0, 0), (1.0, 2.0**-16, 1), (0.0, 0.125, 0),
                                                 (0.0, 1.0 / 3.0, 0), (1e-2, 0.1, 0)])
def test_one_micro_batch_equals_the_zero1_step(max_norm, scale, skip):
    rng = np.random.default_rng(22)
    std = 1e-3 / scale
    ts = _tensors([512, 4099, 1, 3001], 4, rng, std=std)
    hp = oracle.HParams(step=7, max_grad_norm=max_norm, grad_scale=scale, skip_on_nonfinite=skip)
    want, rw = oracle.zero_step(ts, hp, external_sumsq=0.25)
    accs = [oracle.grad_accumulate(t.grads) for t in ts]
    got, rg = oracle.zero_step_accumulated(accs, ts, hp, external_sumsq=0.25)
    assert (rg.sumsq, rg.clip_coef, rg.found_inf, rg.skipped) == (rw.sumsq, rw.clip_coef, rw.found_inf, rw.skipped)
    if max_norm == 1e-2:
        assert rg.clip_coef < 1.0
    for a, b in zip(got, want):
        assert _same_state(a, b)


def test_accumulated_micro_batches_equal_one_large_batch():
    # Integers in [-255, 255] times 2^-12 (exact in bf16), at most 16 summands: every
    # binary32 add is exact, so accumulating K micro-batches of M replicas
    # gives the same gradient as one fold of all K*M replicas, and the whole
    # step (mean gradient: scale 1/(K*M)) matches the large-batch step bitwise.
    rng = np.random.default_rng(23)
    K, M, n = 4, 4, 3000
    mbs = [[_bf16_of(rng.integers(-255, 256, n) * 2.0**-12) for _ in range(M)] for _ in range(K)]
    th, m, v = _state(n, rng)
    hp = oracle.HParams(step=12, max_grad_norm=0.05, grad_scale=1.0 / (K * M))
    acc = _accumulate(mbs)
    got, rg = oracle.zero_step_accumulated([acc], [oracle.TensorState([], th, m, v, None)], hp)
    big = oracle.TensorState([g for grads in mbs for g in grads], th, m, v, None)
    want, rw = oracle.zero_step([big], hp)
    assert rg.clip_coef < 1.0
    assert rg.sumsq == rw.sumsq and rg.clip_coef == rw.clip_coef
    assert _same_state(got[0], want[0])


@pytest.mark.parametrize("where", ["first", "last", "opposite"])
def test_nonfinite_in_any_micro_batch_skips(where):
    rng = np.random.default_rng(24)
    K, M, n = 3, 2, 700
    mbs = [[oracle.f32_to_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32)) for _ in range(M)]
           for _ in range(K)]
    if where == "first":
        mbs[0][1][5] = 0x7F80
    elif where == "last":
        mbs[2][0][699] = 0x7FC0
    else:  # +inf in one micro-batch, -inf in another: the running sum becomes NaN
        mbs[0][0][42] = 0x7F80
        mbs[1][1][42] = 0xFF80
    acc = _accumulate(mbs)
    th, m, v = _state(n, rng)
    st = oracle.TensorState([], th, m, v, np.full(n, 0x1234, np.uint16))
    hp = oracle.HParams(step=3, max_grad_norm=1.0, skip_on_nonfinite=1)
    got, r = oracle.zero_step_accumulated([acc], [st], hp)
    assert r.found_inf == 1 and r.skipped == 1
    assert _same_state(got[0], st)
    if where == "opposite":
        assert math.isnan(acc[42])


def test_zero2_memory_accounting():
    # ZeRO-2 also splits the gradient: per GPU, the bf16 parameters stay
    # whole while the gradient and the 12 optimizer bytes are split N ways
    # ("ZeRO Stage 2": peak memory = full parameters + sharded gradients +
    # sharded optimizer state).
    P, N = 7.5e9, 64
    z0, z1, z2, z3 = (oracle.bytes_per_gpu(P, N, s) for s in range(4))
    assert z2 == P * (2 + (2 + 12) / N)
    assert z3 < z2 < z1 < z0


@pytest.mark.parametrize("flag_inf", [False, True])
def test_amp_one_micro_batch_equals_the_zero1_amp_step(flag_inf):
    # the dynamic loss scale over the accumulated gradient: with one
    # micro-batch, state, record and the moved scale equal the ZeRO-1 AMP step's
    rng = np.random.default_rng(25)
    ts = _tensors([700, 33], 3, rng, std=4.0)
    if flag_inf:
        ts[1].grads[2][30] = 0x7F80
    cfg = oracle.LossScaleConfig(initial_scale_power=12, window=1, hysteresis=1)
    ls = oracle.loss_scale_init(cfg)
    hp = oracle.HParams(step=9, max_grad_norm=3.0)
    want, rw, lw = oracle.zero_step_amp(ts, hp, cfg, ls)
    accs = [oracle.grad_accumulate(t.grads) for t in ts]
    got, rg, lg = oracle.zero_step_accumulated_amp(accs, ts, hp, cfg, ls)
    assert (rg.sumsq == rw.sumsq or flag_inf) and (rg.found_inf, rg.skipped) == (rw.found_inf, rw.skipped)
    assert (rg.found_inf, rg.skipped) == (int(flag_inf),) * 2
    assert lg == lw and lw.scale == (2048.0 if flag_inf else 8192.0)
    for a, b in zip(got, want):
        assert _same_state(a, b)
