"""The oracle's brute-force tiny set, run on the GPU: 200 seeded cases of 16 to
64 elements with M in {1, 2, 3, 4, 8, 64}, adversarial bf16 replicas
(wide exponent ranges up to bf16 max, subnormals, signed zeros, +-inf and NaN
codes, order-sensitive columns) at random element offsets, through
zero_shard_reduce (bit-exact against the oracle's fold, NaN positions
included) and through zero_step with random clip/skip/scale/t (the parity
gates; found_inf and skipped exact; a finite norm within 1e-5); and 100
more such cases, with two micro-batches of replicas, through the ZeRO-2
bucket reduce (the accumulator bit-exact) and accumulated step, and through
the CPU-offloaded step."""
import math

import numpy as np
import pytest
import torch

import oracle
import sharded_optimizer_step_amd as z
from cases import assert_state_matches, bits_equal, hp_oracle, to_np_f32, to_np_u16, ulp_gate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    z.lib()
    torch.cuda.set_device(0)
    yield


def adversarial_bf16(rng, M, n):
    """M replicas of n bf16 codes drawn from one of several regimes."""
    regime = int(rng.integers(0, 5))
    lo, hi = [(100, 130), (1, 254), (240, 254), (1, 20), (110, 135)][regime]
    sign = rng.integers(0, 2, (M, n), dtype=np.uint16) << 15
    e = rng.integers(lo, hi + 1, (M, n)).astype(np.uint16) << 7
    f = rng.integers(0, 128, (M, n), dtype=np.uint16)
    h = (sign | e | f).astype(np.uint16)
    sub = rng.random((M, n)) < 0.05
    h[sub] = sign[sub] | rng.integers(1, 128, int(sub.sum()), dtype=np.uint16)   # subnormals
    zero = rng.random((M, n)) < 0.05
    h[zero] = sign[zero]                                                            # signed zeros
    if rng.random() < 0.3:                                                          # non-finite codes
        k = int(rng.integers(1, 4))
        for _ in range(k):
            h[int(rng.integers(0, M)), int(rng.integers(0, n))] = rng.choice([0x7F80, 0xFF80, 0x7FC1])
    if M >= 4 and rng.random() < 0.5:                                               # the order pin column
        j = int(rng.integers(0, n))
        h[:, j] = 0
        h[:4, j] = [0x3F80, 0x3380, 0x3380, 0xBF80]
    return [h[r].copy() for r in range(M)]


def dev_at(h: np.ndarray, off: int, dtype) -> torch.Tensor:
    """A device copy of host array h at an element offset into a fresh buffer."""
    base = torch.empty(h.size + off + 8, dtype=dtype, device="cuda")
    v = base[off:off + h.size]
    if dtype == torch.bfloat16:
        v.view(torch.int16).copy_(torch.from_numpy(h.view(np.int16)))
    else:
        v.copy_(torch.from_numpy(h))
    return v


@pytest.mark.parametrize("case", range(200))
def test_tiny_adversarial_case_on_the_gpu(case):
    rng = np.random.default_rng(31_000 + case)
    M = int(rng.choice([1, 2, 3, 4, 8, 64]))
    n = int(rng.integers(16, 65))
    hs = adversarial_bf16(rng, M, n)
    offs = [int(x) for x in rng.integers(0, 8, M + 5)]
    scale = float(rng.choice([1.0, 2.0**-16, 1.0 / 3.0, 0.125]))
    where = f"case {case}: M {M}, n {n}, scale {scale}, offsets {offs}"

    # the reduce alone: bit-exact, NaN positions included
    ds = [dev_at(h, o, torch.bfloat16) for h, o in zip(hs, offs)]
    g_out = dev_at(np.zeros(n, np.float32), offs[M], torch.float32)
    z.zero_shard_reduce(ds, scale, g_out)
    got, want = to_np_f32(g_out), oracle.reduce(hs, scale)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), where
    assert bits_equal(got[~nan], want[~nan]), where

    # the fused step
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-5).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-8).astype(np.float32)
    hp = z.HParams(step=int(rng.choice([1, 10, 1000])), max_grad_norm=float(rng.choice([0.0, 1e-3, 10.0])),
                   skip_on_nonfinite=int(rng.integers(0, 2)), grad_scale=scale)
    dt = z.ZeroTensor(ds, dev_at(master, offs[M + 1], torch.float32), dev_at(m, offs[M + 2], torch.float32),
                      dev_at(v, offs[M + 3], torch.float32),
                      dev_at(np.full(n, 0x1234, np.uint16), offs[M + 4], torch.bfloat16))
    res = z.new_result()
    z.zero_step([dt], hp, 0.0, z.workspace(z.zero_step_workspace_bytes([dt], M, hp)), res)
    r = z.read_result(res)
    ht = oracle.TensorState(hs, master.copy(), m.copy(), v.copy(), np.full(n, 0x1234, np.uint16))
    new, ro = oracle.zero_step([ht], hp_oracle(hp))
    assert r["status"] == 0, where
    assert (r["found_inf"], r["skipped"]) == (ro.found_inf, ro.skipped), (where, r, ro)
    if math.isfinite(ro.grad_norm) and ro.grad_norm < 3.4e38:  # the record holds the norm in binary32
        assert abs(r["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm + 1e-30, (where, r, ro)
    assert_state_matches(to_np_f32(dt.master), to_np_f32(dt.exp_avg), to_np_f32(dt.exp_avg_sq),
                         to_np_u16(dt.param_out), new[0].master, new[0].exp_avg, new[0].exp_avg_sq,
                         new[0].param_out, where, ulp_max=ulp_gate((r, ro)))


def check_record(r, ro, where):
    assert r["status"] == 0, (where, r)
    assert (r["found_inf"], r["skipped"]) == (ro.found_inf, ro.skipped), (where, r, ro)
    if math.isfinite(ro.grad_norm) and ro.grad_norm < 3.4e38:
        assert abs(r["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm + 1e-30, (where, r, ro)


@pytest.mark.parametrize("case", range(100))
def test_tiny_adversarial_case_through_zero2_and_offload(case):
    rng = np.random.default_rng(41_000 + case)
    M = int(rng.choice([1, 2, 3, 8, 64]))
    n = int(rng.integers(16, 65))
    mb = [adversarial_bf16(rng, M, n) for _ in range(2)]  # two micro-batches of replicas
    offs = [int(x) for x in rng.integers(0, 8, M + 6)]
    scale = float(rng.choice([1.0, 2.0**-16, 1.0 / 3.0, 0.125]))
    hp = z.HParams(step=int(rng.choice([1, 10, 1000])), max_grad_norm=float(rng.choice([0.0, 1e-3, 10.0])),
                   skip_on_nonfinite=int(rng.integers(0, 2)), grad_scale=scale)
    where = f"case {case}: M {M}, n {n}, hp {hp}, offsets {offs}"
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-5).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-8).astype(np.float32)

    # ZeRO-2: store, then accumulate-and-finish; the accumulator bit-exact (NaN positions included)
    acc = dev_at(np.zeros(n, np.float32), offs[M], torch.float32)
    parts = z.new_bucket_partials(1)
    for k, hs in enumerate(mb):
        ds = [dev_at(h, o, torch.bfloat16) for h, o in zip(hs, offs)]
        sh = [z.GradShard(ds, acc)]
        flags = (z.BUCKET_ACCUMULATE | z.BUCKET_FINAL) if k else 0
        z.zero_bucket_reduce(sh, flags, scale, 77, parts, z.workspace(z.zero_bucket_reduce_workspace_bytes(sh, M)))
    want_acc = oracle.grad_accumulate(mb[1], oracle.grad_accumulate(mb[0]))
    got_acc = to_np_f32(acc)
    nan = np.isnan(want_acc)
    assert np.array_equal(np.isnan(got_acc), nan), where
    assert bits_equal(got_acc[~nan], want_acc[~nan]), where
    st = [dev_at(x, o, torch.float32) for x, o in zip((master, m, v), offs[M + 1:M + 4])]
    out = dev_at(np.full(n, 0x1234, np.uint16), offs[M + 4], torch.bfloat16)
    ats = [z.AccTensor(acc, st[0], st[1], st[2], out)]
    res = z.new_result()
    z.zero_step_accumulated(ats, hp, parts, 1, 77, 0.0, z.workspace(z.zero_step_accumulated_workspace_bytes(ats)), res)
    ht = oracle.TensorState([], master.copy(), m.copy(), v.copy(), np.full(n, 0x1234, np.uint16))
    new, ro = oracle.zero_step_accumulated([want_acc], [ht], hp_oracle(hp))
    r = z.read_result(res)
    check_record(r, ro, "ZeRO-2 " + where)
    assert_state_matches(to_np_f32(st[0]), to_np_f32(st[1]), to_np_f32(st[2]), to_np_u16(out), new[0].master,
                         new[0].exp_avg, new[0].exp_avg_sq, new[0].param_out, "ZeRO-2 " + where,
                         ulp_max=ulp_gate((r, ro)))

    # the CPU-offloaded step on the first micro-batch: the ZeRO-1 step's result
    ds = [dev_at(h, o, torch.bfloat16) for h, o in zip(mb[0], offs)]
    out = dev_at(np.full(n, 0x1234, np.uint16), offs[M + 5], torch.bfloat16)
    ots = [z.OffloadTensor(ds, torch.from_numpy(master.copy()), torch.from_numpy(m.copy()),
                           torch.from_numpy(v.copy()), out)]
    r = z.zero_offload_step(ots, hp, 0.0, z.workspace(z.zero_offload_workspace_bytes(ots, M)),
                            z.host_workspace(z.zero_offload_host_workspace_bytes(ots)), 2)
    torch.cuda.synchronize()
    ht = oracle.TensorState(mb[0], master.copy(), m.copy(), v.copy(), np.full(n, 0x1234, np.uint16))
    new, ro = oracle.zero_step([ht], hp_oracle(hp))
    check_record(r, ro, "offload " + where)
    assert_state_matches(ots[0].master.numpy(), ots[0].exp_avg.numpy(), ots[0].exp_avg_sq.numpy(), to_np_u16(out),
                         new[0].master, new[0].exp_avg, new[0].exp_avg_sq, new[0].param_out, "offload " + where,
                         ulp_max=ulp_gate((r, ro)))
