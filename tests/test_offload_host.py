"""The host half of the CPU-offloaded step (zero_offload_adamw_host), on the
CPU: no GPU is touched. It applies the same binary64 AdamW as the GPU kernels
to host fp32 state, so it must reproduce the oracle's update bit for bit
whatever the thread count (IEEE division and square root are correctly
rounded, and contraction is off)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import sharded_optimizer_step_amd as z


def _state(n, seed, t):
    rng = np.random.default_rng(seed)
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-5).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-8).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    if t == 1:
        m[:] = 0
        v[:] = 0
    return th, m, v, g


def _host_step(th, m, v, g, hp, coef, threads):
    T = [torch.from_numpy(a.copy()) for a in (th, m, v, g)]
    out = torch.empty(th.size, dtype=torch.bfloat16)
    z.zero_offload_adamw_host(T[0], T[1], T[2], T[3], out, hp, coef, threads)
    return T[0].numpy(), T[1].numpy(), T[2].numpy(), out.view(torch.int16).numpy().view(np.uint16)


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


@pytest.mark.parametrize("n,t,coef,threads", [(100_003, 1, 1.0, 4), (65, 10, 0.37, 3), (64, 100, 1.0, 1),
                                              (63, 1000, 0.5, 8), (1, 5000, 1.0, 2), (262_147, 33, 0.999, 0)])
def test_host_adamw_matches_the_oracle_bitwise(n, t, coef, threads):
    hp = z.HParams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=t)
    th, m, v, g = _state(n, 7 + t, t)
    got = _host_step(th, m, v, g, hp, coef, threads)
    want = oracle.adamw(th, m, v, g, oracle.HParams(lr=hp.lr, beta1=hp.beta1, beta2=hp.beta2, eps=hp.eps,
                                                    weight_decay=hp.weight_decay, step=t), coef)
    for a, b, name in zip(got, want, ("master", "exp_avg", "exp_avg_sq", "param_out")):
        assert np.array_equal(_bits(a), _bits(b)), name


def test_thread_count_does_not_change_the_result():
    hp = z.HParams(step=17)
    th, m, v, g = _state(1_000_001, 3, 17)
    ref = _host_step(th, m, v, g, hp, 0.8, 1)
    for threads in (2, 5, 16):
        got = _host_step(th, m, v, g, hp, 0.8, threads)
        assert all(np.array_equal(_bits(a), _bits(b)) for a, b in zip(got, ref)), threads


def test_nonfinite_gradients_propagate_like_the_oracle():
    hp = z.HParams(step=4)
    th, m, v, g = _state(1000, 5, 4)
    g[3], g[500], g[999] = np.inf, -np.inf, np.nan
    got = _host_step(th, m, v, g, hp, 1.0, 3)
    want = oracle.adamw(th, m, v, g, oracle.HParams(step=4), 1.0)
    for a, b in zip(got[:3], want[:3]):
        assert np.array_equal(np.isnan(a), np.isnan(b))
        ok = ~np.isnan(b)
        assert np.array_equal(_bits(a[ok]), _bits(b[ok]))
    nan_out = lambda u: ((u & 0x7F80) == 0x7F80) & ((u & 0x7F) != 0)
    assert np.array_equal(nan_out(got[3]), nan_out(want[3]))
    assert np.array_equal(got[3][~nan_out(want[3])], want[3][~nan_out(want[3])])


def test_host_adamw_argument_checks():
    L = z.lib()
    h = z.HParams()._c()
    bad = z.HParams(step=0)._c()
    p = ctypes.c_void_p(4096)
    assert L.zero_offload_adamw_host(p, p, p, p, p, 10, ctypes.byref(bad), 1.0, 0) == 1
    assert L.zero_offload_adamw_host(p, p, p, p, p, -1, ctypes.byref(h), 1.0, 0) == 1
    assert L.zero_offload_adamw_host(p, p, p, p, p, 10, ctypes.byref(h), float("nan"), 0) == 1
    assert L.zero_offload_adamw_host(p, p, p, p, p, 10, ctypes.byref(h), 1.0, -1) == 1
    assert L.zero_offload_adamw_host(p, p, None, p, p, 10, ctypes.byref(h), 1.0, 0) == 1
    assert L.zero_offload_adamw_host(None, None, None, None, None, 0, ctypes.byref(h), 1.0, 0) == 0  # n == 0
