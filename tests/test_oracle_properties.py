"""Property-based pins of the oracle (CPU, hypothesis): searched and shrunk
inputs instead of fixed seeds.

* The rank fold of any finite bf16 replicas (M up to 12, any exponent that
  cannot overflow binary32 in 12 adds, subnormals and signed zeros included),
  times a binary32 scale, equals the exact rational emulation of the
  ascending-rank binary32 left fold (the IEEE 754 definition, written in the
  pin module).
* AdamW on one element, over wide ranges of the state, the gradient and every
  hyperparameter, equals the formula evaluated in 80-digit decimal arithmetic
  and rounded to binary32, within one binary32 ulp plus the rounding error a
  binary64 evaluation of the formula can make (a bound of 2e-11 of the
  magnitudes of the terms, far below what a dropped term, a wrong sign or a
  binary32 intermediate would change)."""
import decimal
import math

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from test_oracle_pins import F32, torch_bf16_to_f32

# finite bf16 codes whose magnitude stays below 2^124 (twelve of them cannot
# overflow binary32 when added); signed zeros, the smallest subnormals, +-1
# and the 2^-24 of the order pin are drawn often
FINITE_BF16 = st.one_of(st.sampled_from([0x0000, 0x8000, 0x0001, 0x8001, 0x3F80, 0xBF80, 0x3380, 0xB380]),
                        st.integers(0, 0xFFFF).filter(lambda h: ((h >> 7) & 0xFF) <= 250))


@st.composite
def replicas(draw):
    M = draw(st.integers(1, 12))
    n = draw(st.integers(1, 6))
    return [np.array([draw(FINITE_BF16) for _ in range(n)], np.uint16) for _ in range(M)]


@settings(max_examples=400, deadline=None, suppress_health_check=[HealthCheck.filter_too_much])
@given(grads=replicas(), scale=st.sampled_from([1.0, 2.0**-16, 1.0 / 3.0, 0.125, 1.0 / 64, 3.0]))
def test_fold_is_the_ascending_binary32_left_fold(grads, scale):
    got = oracle.reduce(grads, scale)
    vals = [torch_bf16_to_f32(g) for g in grads]
    sc = F32.of(float(np.float32(scale)))
    for i in range(grads[0].size):
        s = F32.of(float(vals[0][i]))
        for r in range(1, len(grads)):
            s = s.add(F32.of(float(vals[r][i])))
        s = s.mul(sc)
        assert s.same_as(float(got[i])), (i, [int(g[i]) for g in grads], scale, float(got[i]))


def f32(lo, hi, **kw):
    lo, hi = float(np.float32(lo)), float(np.float32(hi))  # binary32 bounds
    return st.floats(lo, hi, width=32, allow_nan=False, allow_infinity=False, **kw)


def ulp32(x: float) -> float:
    x = abs(float(np.float32(x)))
    if x == 0.0:
        return float(np.nextafter(np.float32(0), np.float32(1)))
    return float(np.spacing(np.float32(x)))


@settings(max_examples=300, deadline=None)
@given(th=f32(-4.0, 4.0), m=f32(-1e-2, 1e-2), v=f32(0.0, 1e-3), g=f32(-1.0, 1.0),
       lr=st.floats(0.0, 1e-2), b1=st.floats(0.0, 0.999), b2=st.floats(0.0, 0.9999), eps=st.floats(1e-12, 1e-6),
       wd=st.floats(0.0, 0.2), t=st.integers(1, 10_000), coef=st.floats(1e-3, 1.0))
def test_adamw_is_the_formula_within_binary64_rounding(th, m, v, g, lr, b1, b2, eps, wd, t, coef):
    hp = oracle.HParams(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd, step=t)
    a = lambda x: np.array([x], np.float32)
    o_th, o_m, o_v, _ = oracle.adamw(a(th), a(m), a(v), a(g), hp, coef)

    decimal.getcontext().prec = 80
    D = decimal.Decimal
    B1, B2, LR, EPS, WD = D(b1), D(b2), D(lr), D(eps), D(wd)
    gi = D(float(np.float32(g))) * D(coef)
    mn = B1 * D(float(np.float32(m))) + (1 - B1) * gi
    vn = B2 * D(float(np.float32(v))) + (1 - B2) * gi * gi
    bc1, bc2 = 1 - B1 ** t, 1 - B2 ** t
    decay_term = D(float(np.float32(th))) * (1 - LR * WD)
    step_term = LR * (mn / bc1) / ((vn / bc2).sqrt() + EPS)
    tn = decay_term - step_term

    def close(got, exact, scale_terms):
        e = float(exact)
        err = abs(float(got) - e)
        return err <= ulp32(e) + 2e-11 * scale_terms, (float(got), e, err)

    ok, info = close(o_m[0], mn, abs(float(B1 * D(float(np.float32(m))))) + abs(float((1 - B1) * gi)))
    assert ok, ("exp_avg", info)
    ok, info = close(o_v[0], vn, abs(float(B2 * D(float(np.float32(v))))) + abs(float((1 - B2) * gi * gi)))
    assert ok, ("exp_avg_sq", info)
    ok, info = close(o_th[0], tn, abs(float(decay_term)) + abs(float(step_term)))
    assert ok, ("master", info)
    assert math.isfinite(float(o_th[0]))
