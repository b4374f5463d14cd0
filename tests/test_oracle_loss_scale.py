"""Pins of the oracle's dynamic loss scale (CPU only).

The pages configure the scale with the fp16 block of the deepspeed_config.json
listing (gsyq.cn/news/457874, section 4.2: loss_scale 0, initial_scale_power,
loss_scale_window, hysteresis, min_loss_scale) and describe the scaler's
scale / step / update cycle (section 3.2, trap 3); they print no update rule.
The rule read from the knobs is pinned here against things other than the
oracle itself: a library gradient scaler (hysteresis 1), closed forms over
runs of clean and overflowing steps, and the exactness of power-of-two
unscaling in the step.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def run(cfg, flags, state=None):
    s = state if state is not None else oracle.loss_scale_init(cfg)
    out = []
    for f in flags:
        s = oracle.loss_scale_update(s, cfg, f)
        out.append(s)
    return out


@pytest.mark.parametrize("window", [1, 2, 3, 7, 50])
@pytest.mark.parametrize("power", [0, 12, 16])
@pytest.mark.parametrize("seed", [0, 1])
def test_hysteresis_one_is_the_library_gradient_scaler(window, power, seed):
    # torch's scaler update: on an overflow multiply by the backoff factor and
    # clear the growth tracker; after growth_interval clean steps in a row
    # multiply by the growth factor. Growth 2, backoff 1/2, interval = window.
    rng = np.random.default_rng(seed)
    flags = (rng.random(300) < rng.choice([0.02, 0.1, 0.4])).astype(int)
    cfg = oracle.LossScaleConfig(initial_scale_power=power, window=window, hysteresis=1, min_scale=2.0 ** -60)
    scale = torch.tensor([2.0 ** power], dtype=torch.float32)
    tracker = torch.tensor([0], dtype=torch.int32)
    compared = 0
    for f, s in zip(flags, run(cfg, flags)):
        torch._amp_update_scale_(scale, tracker, torch.tensor([float(f)]), 2.0, 0.5, window)
        if scale.item() < cfg.min_scale:
            break  # the library scaler has no floor: the rules part here
        assert s.scale == scale.item() and s.good_steps == tracker.item()
        assert s.inv_scale == np.float32(1.0) / np.float32(s.scale)
        compared += 1
    assert compared >= 100


def test_pages_fp16_block_gives_the_initial_scale():
    cfgj = json.load(open(os.path.join(HERE, "golden", "ds_config_blocks.json")))["fp16"]
    assert cfgj["loss_scale"] == 0  # 0: dynamic
    cfg = oracle.LossScaleConfig(initial_scale_power=cfgj["initial_scale_power"], window=cfgj["loss_scale_window"],
                                 hysteresis=cfgj["hysteresis"], min_scale=float(cfgj["min_loss_scale"]))
    s = oracle.loss_scale_init(cfg)
    assert (s.scale, s.inv_scale, s.good_steps, s.overflows) == (4096.0, 2.0 ** -12, 0, 0)
    # hysteresis 2: one overflow leaves the scale, the second in a row halves it
    a, b = run(cfg, [1, 1])
    assert a.scale == 4096.0 and b.scale == 2048.0
    # an overflow, a clean step, an overflow: never two in a row, no change
    assert [x.scale for x in run(cfg, [1, 0, 1, 0, 1])] == [4096.0] * 5
    # 1000 clean steps double it
    assert run(cfg, [0] * 1000)[-1].scale == 8192.0
    assert run(cfg, [0] * 999)[-1].scale == 4096.0


@pytest.mark.parametrize("h", [1, 2, 3, 5])
def test_overflow_streak_closed_form(h):
    cfg = oracle.LossScaleConfig(initial_scale_power=20, window=10 ** 6, hysteresis=h, min_scale=2.0 ** -40)
    for q in range(0, 41):
        s = run(cfg, [1] * q)[-1] if q else oracle.loss_scale_init(cfg)
        assert s.scale == 2.0 ** (20 - q // h)
        assert s.overflows == q % h
        assert s.good_steps == 0


@pytest.mark.parametrize("window", [1, 3, 8])
@pytest.mark.parametrize("seed", [2, 3, 4])
def test_clean_runs_closed_form(window, seed):
    # with a hysteresis no streak reaches, the scale only grows: each maximal
    # run of L clean steps contributes floor(L / window) doublings
    rng = np.random.default_rng(seed)
    flags = (rng.random(120) < 0.15).astype(int)  # at most 120 doublings: below the binary32 ceiling
    cfg = oracle.LossScaleConfig(initial_scale_power=0, window=window, hysteresis=10 ** 6, min_scale=1.0)
    got = run(cfg, flags)
    runs, cur = [], 0
    for f in flags:
        if f:
            runs.append(cur)
            cur = 0
        else:
            cur += 1
    runs.append(cur)
    assert got[-1].scale == 2.0 ** sum(L // window for L in runs)
    assert got[-1].good_steps == cur % window


def test_floor_and_ceiling():
    cfg = oracle.LossScaleConfig(initial_scale_power=12, window=1000, hysteresis=2, min_scale=1.0)
    seq = run(cfg, [1] * 100)
    assert seq[23].scale == 1.0 and seq[21].scale == 2.0  # 24 overflows: 12 halvings
    assert all(s.scale == 1.0 for s in seq[23:])
    odd = oracle.LossScaleConfig(initial_scale_power=4, window=1000, hysteresis=1, min_scale=3.0)
    assert [s.scale for s in run(odd, [1, 1, 1])] == [8.0, 4.0, 3.0]
    assert run(odd, [1, 1, 1])[-1].inv_scale == np.float32(1.0) / np.float32(3.0)
    top = oracle.LossScaleConfig(initial_scale_power=127, window=1, hysteresis=1, min_scale=1.0)
    s = run(top, [0, 0])
    assert s[0].scale == 2.0 ** 127 and s[1].scale == 2.0 ** 127 and s[1].good_steps == 0
    assert math.isfinite(s[1].scale)


@pytest.mark.parametrize("power", [-126, -60, 0, 12, 64, 126, 127])
def test_inverse_of_a_power_of_two_is_exact(power):
    s = oracle.loss_scale_init(oracle.LossScaleConfig(initial_scale_power=power))
    assert s.scale == 2.0 ** power and s.inv_scale == 2.0 ** -power


def _scaled_bf16(h, k):
    x = oracle.bf16_to_f32(h).astype(np.float64) * 2.0 ** k
    out = oracle.f32_to_bf16(x.astype(np.float32))
    assert np.array_equal(oracle.bf16_to_f32(out).astype(np.float64), x)  # exact power-of-two scaling
    return out


def _tensors(rng, n, M, k=0):
    grads = [oracle.f32_to_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32)) for _ in range(M)]
    if k:
        grads = [_scaled_bf16(g, k) for g in grads]
    mk = lambda s: (rng.standard_normal(n) * s).astype(np.float32)
    return grads, mk(0.02), mk(1e-5), np.abs(mk(1e-8))


def test_amp_step_unscales_exactly():
    # gradients of a loss scaled by S = 2^12, unscaled by the step, give the
    # same state bit for bit as the unscaled gradients with no loss scale
    rng = np.random.default_rng(7)
    n, M = 3001, 4
    grads, w, m, v = _tensors(rng, n, M)
    sgrads = [_scaled_bf16(g, 12) for g in grads]
    hp = oracle.HParams(step=5, max_grad_norm=0.5)
    cfg = oracle.LossScaleConfig()
    plain, rp = oracle.zero_step([oracle.TensorState(grads, w, m, v)], hp)
    amp, ra, s1 = oracle.zero_step_amp([oracle.TensorState(sgrads, w, m, v)], hp, cfg, oracle.loss_scale_init(cfg))
    for a, b in zip((plain[0].master, plain[0].exp_avg, plain[0].exp_avg_sq, plain[0].param_out),
                    (amp[0].master, amp[0].exp_avg, amp[0].exp_avg_sq, amp[0].param_out)):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    assert ra.sumsq == rp.sumsq and ra.found_inf == 0 and ra.skipped == 0
    assert s1 == oracle.LossScale(4096.0, 2.0 ** -12, 1, 0)


def test_amp_step_overflow_skips_then_backs_off():
    rng = np.random.default_rng(8)
    n, M = 1000, 2
    grads, w, m, v = _tensors(rng, n, M, k=12)
    grads[1] = grads[1].copy()
    grads[1][17] = 0x7F80  # +inf in one replica
    cfg = oracle.LossScaleConfig()
    t0 = [oracle.TensorState(grads, w, m, v, np.full(n, 0x1234, np.uint16))]
    hp = oracle.HParams(step=3)
    t1, r1, s1 = oracle.zero_step_amp(t0, hp, cfg, oracle.loss_scale_init(cfg))
    assert r1.found_inf == 1 and r1.skipped == 1
    assert np.array_equal(t1[0].master, w) and np.array_equal(t1[0].param_out, t0[0].param_out)
    assert (s1.scale, s1.overflows) == (4096.0, 1)
    t2, r2, s2 = oracle.zero_step_amp(t1, hp, cfg, s1)
    assert r2.skipped == 1 and (s2.scale, s2.overflows) == (2048.0, 0)
    # the caller's skip_on_nonfinite does not matter: the AMP step always skips
    t3, r3, _ = oracle.zero_step_amp(t0, oracle.HParams(step=3, skip_on_nonfinite=0), cfg, s2)
    assert r3.skipped == 1 and np.array_equal(t3[0].exp_avg, m)
