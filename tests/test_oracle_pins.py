"""Pins of the CPU oracle to things other than itself (CPU only).

Each pin is chosen so that a plausible mistake in the oracle (a dropped term,
a wrong sign, a wrong order of accumulation, a wrong rounding rule) fails at
least one of them:

* bf16 decode/encode   -> torch's bfloat16 conversions (library routines).
* rank fold            -> exact rational emulation of binary32 round-to-nearest-even
                          addition, written here from the IEEE 754 definition; an
                          order pin whose three candidate orders give three
                          different answers; signed-zero rule; M = 1 special case.
* sum of squares       -> exact rational sums; closed form for a constant vector.
* clip coefficient     -> torch.nn.utils.clip_grad_norm_ (library routine).
* AdamW update         -> torch.optim.AdamW in float64 (library routine); the
                          step-1 closed form theta1 = theta0 - lr*wd*theta0
                          - lr*g/(|g|+eps); a 60-digit decimal evaluation.
* skip                 -> a step with an inf anywhere leaves all state unchanged.
* memory accounting    -> the per-parameter table the pages print (golden file).
"""
import decimal
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(20251207)
F32_MAX = Fraction(2) ** 128 - Fraction(2) ** 104


# --------------------------------------------------------------------------
# Helpers: torch conversions and an exact binary32 model.
# --------------------------------------------------------------------------

def torch_bf16_to_f32(h: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(h.astype(np.uint16).view(np.int16).copy()).view(torch.bfloat16)
    return t.float().numpy()


def torch_f32_to_bf16(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(x.astype(np.float32).copy()).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits32(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def rnd32(q: Fraction) -> Fraction | float:
    """Round an exact rational to binary32, nearest, ties to even (IEEE 754).
    Returns a Fraction, or +-inf on overflow. Zero results carry no sign."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    qe = max(e - 23, -149)  # exponent of the last significand bit
    k = a / Fraction(2) ** qe
    fl = k.numerator // k.denominator
    rem = k - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * Fraction(2) ** qe
    if r > F32_MAX:
        return sign * math.inf
    return sign * r


class F32:
    """A binary32 value as (exact rational, negative-zero flag)."""

    def __init__(self, val, negzero=False):
        self.val = val
        self.negzero = negzero

    @staticmethod
    def of(x: float) -> "F32":
        if x == 0:
            return F32(Fraction(0), math.copysign(1.0, x) < 0)
        return F32(Fraction(x))

    def add(self, o: "F32") -> "F32":
        if self.val == 0 and o.val == 0:
            return F32(Fraction(0), self.negzero and o.negzero)
        if self.val == 0:
            return o
        if o.val == 0:
            return self
        q = self.val + o.val
        if q == 0:
            return F32(Fraction(0), False)  # x + (-x) = +0 when rounding to nearest
        return F32(rnd32(q))

    def mul(self, o: "F32") -> "F32":
        neg = (self.val < 0 or self.negzero) != (o.val < 0 or o.negzero)
        q = self.val * o.val
        if q == 0:
            return F32(Fraction(0), neg)
        r = rnd32(q)
        if r == 0:
            return F32(Fraction(0), neg)
        return F32(r)

    def same_as(self, x: float) -> bool:
        if x == 0:
            return self.val == 0 and self.negzero == (math.copysign(1.0, x) < 0)
        if math.isinf(x) or math.isnan(x):
            return False
        return Fraction(x) == self.val


def random_bf16(shape, exp_lo=100, exp_hi=140, p_sub=0.0, p_zero=0.0, rng=RNG) -> np.ndarray:
    """bf16 bit patterns with exponent fields in [exp_lo, exp_hi], random sign
    and fraction, plus optional subnormals and signed zeros."""
    sign = rng.integers(0, 2, shape, dtype=np.uint16) << 15
    e = rng.integers(exp_lo, exp_hi + 1, shape).astype(np.uint16) << 7
    f = rng.integers(0, 128, shape, dtype=np.uint16)
    h = sign | e | f
    if p_sub:
        m = rng.random(shape) < p_sub
        h[m] = (sign[m] | rng.integers(1, 128, int(m.sum()), dtype=np.uint16))
    if p_zero:
        m = rng.random(shape) < p_zero
        h[m] = sign[m]
    return h.astype(np.uint16)


# --------------------------------------------------------------------------
# bf16 format
# --------------------------------------------------------------------------

def test_bf16_decode_all_patterns_matches_torch():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f32(h)
    ref = torch_bf16_to_f32(h)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(bits32(ours[~nan]), bits32(ref[~nan]))
    # the pattern is the upper half of the binary32 encoding
    assert np.array_equal(bits32(ours[~nan]) >> 16, h[~nan].astype(np.uint32))


def test_bf16_round_nearest_even_matches_torch():
    u = RNG.integers(0, 2**32, 1 << 20, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    # exact halfway points between adjacent bf16 values (ties), both parities
    hb = RNG.integers(0, 0x7F7F, 4096, dtype=np.uint32)
    ties = ((hb << 16) | 0x8000).view(np.float32)
    near = np.concatenate([((hb << 16) | 0x7FFF), ((hb << 16) | 0x8001)]).view(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 3.3961775e38, 3.4e38, -3.4e38,
                        1e-40, -1e-40, 1.4e-45, 1.1754942e-38, 9.2e-41], np.float32)
    edge = np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0x7F7FFFFF, 0x007F8000, 0x007FFFFF, 0x00008000,
                     0x00018000, 0x80018000], np.uint32).view(np.float32)
    allx = np.concatenate([x, ties, -ties, near, special, edge]).astype(np.float32)
    ours = oracle.f32_to_bf16(allx)
    ref = torch_f32_to_bf16(allx)
    isn = np.isnan(allx)
    assert np.array_equal(ours[~isn], ref[~isn])
    # NaN stays NaN (quiet, sign kept)
    on = ours[isn]
    assert np.all((on & 0x7F80) == 0x7F80) and np.all((on & 0x7F) != 0)
    assert np.array_equal(on >> 15, (bits32(allx[isn]) >> 31).astype(np.uint16))


def test_bf16_round_ties_go_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: goes to 1 (even);
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: goes to 1+2^-6 (even).
    x = np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8)], np.float32)
    out = oracle.f32_to_bf16(x)
    assert list(out) == [0x3F80, 0x3F82, 0xBF80]


# --------------------------------------------------------------------------
# Rank fold (reduce-scatter arithmetic at one rank) and unscale
# --------------------------------------------------------------------------

def _bf16_of(vals) -> np.ndarray:
    h = oracle.f32_to_bf16(np.asarray(vals, np.float32))
    assert np.array_equal(oracle.bf16_to_f32(h), np.asarray(vals, np.float32)), "not exact in bf16"
    return h


def test_fold_order_pin():
    # element 0: [1, 2^-24, 2^-24, -1]; element 1: [-1, 2^-24, 2^-24, 1]
    # ascending left fold: 0 and 2^-23; descending: 2^-23 and 0; pairwise: 2^-24 and 2^-24.
    cols = [[1.0, -1.0], [2**-24, 2**-24], [2**-24, 2**-24], [-1.0, 1.0]]
    grads = [_bf16_of(c) for c in cols]
    s = oracle.reduce(grads)
    assert s[0] == 0.0 and s[1] == 2.0**-23


def test_fold_signed_zero_starts_from_rank0():
    grads = [_bf16_of([-0.0, -0.0, 0.0]), _bf16_of([-0.0, 0.0, -0.0]), _bf16_of([-0.0, -0.0, -0.0])]
    s = oracle.reduce(grads)
    assert np.array_equal(np.signbit(s), [True, False, False])


def test_fold_M1_is_exact_conversion():
    h = random_bf16(4096, 1, 254, p_sub=0.05, p_zero=0.02)
    s = oracle.reduce([h])
    assert np.array_equal(bits32(s), bits32(torch_bf16_to_f32(h)))


@pytest.mark.parametrize("case", range(200))
def test_fold_matches_exact_binary32_emulation(case):
    rng = np.random.default_rng(1000 + case)
    M = [1, 2, 3, 4, 8, 64][case % 6]
    n = int(rng.integers(16, 65)) if M < 64 else 16
    if case % 3 == 0:   # similar magnitudes, like real gradients
        grads = [random_bf16(n, 110, 118, rng=rng) for _ in range(M)]
    elif case % 3 == 1:  # wide range: stresses rounding
        grads = [random_bf16(n, 60, 180, rng=rng) for _ in range(M)]
    else:                # tiny: subnormals and signed zeros
        grads = [random_bf16(n, 0, 4, p_sub=0.3, p_zero=0.2, rng=rng) for _ in range(M)]
    scale = [1.0, 2.0**-16, 1.0 / 3.0, 0.125][case % 4]
    got = oracle.reduce(grads, scale)
    vals = [torch_bf16_to_f32(g) for g in grads]
    sc = F32.of(float(np.float32(scale)))
    for i in range(n):
        s = F32.of(float(vals[0][i]))
        for r in range(1, M):
            s = s.add(F32.of(float(vals[r][i])))
        s = s.mul(sc)
        assert s.same_as(float(got[i])), (case, i)


def test_fold_error_bound_against_exact_sum():
    rng = np.random.default_rng(7)
    for M in (2, 8, 64):
        grads = [random_bf16(64, 100, 130, rng=rng) for _ in range(M)]
        got = oracle.reduce(grads)
        vals = [torch_bf16_to_f32(g).astype(np.float64) for g in grads]
        u = 2.0 ** -24
        gamma = (M - 1) * u / (1 - (M - 1) * u)
        for i in range(64):
            exact = sum(Fraction(float(v[i])) for v in vals)
            absum = sum(abs(Fraction(float(v[i]))) for v in vals)
            assert abs(Fraction(float(got[i])) - exact) <= Fraction(gamma) * absum


def test_reduce_scatter_concat_equals_all_reduce():
    # All-Reduce = Reduce-Scatter + All-Gather ([CS336 L7] "核心恒等式"):
    # concatenating every rank's reduced shard gives the unsharded reduction.
    N, M = 10007, 4
    full = [random_bf16(N, 105, 120) for _ in range(M)]
    whole = oracle.reduce(full)
    per = -(-N // M)
    parts = [oracle.reduce([g[r * per:min(N, (r + 1) * per)] for g in full]) for r in range(M)]
    assert np.array_equal(bits32(np.concatenate(parts)), bits32(whole))


def test_unscale_after_sum_is_invariant_for_power_of_two_scale(golden_dir):
    # AMP: gradients carry a loss scale S = 2^k; the fp16 block of the page's
    # deepspeed config starts at 2^initial_scale_power.
    cfg = json.load(open(os.path.join(golden_dir, "ds_config_blocks.json")))
    S = 2.0 ** cfg["fp16"]["initial_scale_power"]
    assert S == 4096.0
    M, n = 8, 5000
    grads = [random_bf16(n, 105, 118) for _ in range(M)]
    scaled = [_bf16_of(torch_bf16_to_f32(g) * np.float32(S)) for g in grads]
    a = oracle.reduce(grads)
    b = oracle.reduce(scaled, 1.0 / S)
    assert np.array_equal(bits32(a), bits32(b))


# --------------------------------------------------------------------------
# Non-finite flag and sum of squares
# --------------------------------------------------------------------------

def test_sumsq_matches_exact_rational():
    g = (RNG.standard_normal(777) * 1e-3).astype(np.float32)
    s, f = oracle.check(g)
    exact = sum(Fraction(float(x)) ** 2 for x in g)
    assert f == 0
    assert abs(Fraction(s) - exact) <= exact * Fraction(777 * 2**-53)
    assert math.isclose(s, math.fsum(float(x) * float(x) for x in g), rel_tol=1e-14)


def test_sumsq_chains_across_slices_in_index_order():
    g = (RNG.standard_normal(100000) * 1e-4).astype(np.float32)
    s_all, _ = oracle.check(g)
    st = oracle.SumSq()
    for k in range(0, g.size, 9973):
        st.add(g[k:k + 9973])
    assert st.sumsq == s_all and st.found_inf == 0


def test_sumsq_is_the_exact_sum_where_a_plain_sum_drops_terms():
    # 1024^2 = 2^20 first, then 100,000 squares of 2^-17 (2^-34 each): every
    # small square is a quarter of an ulp of 2^20, so a plain left-to-right
    # binary64 sum never leaves 2^20; the exact sum, 2^20 + 100,000 * 2^-34,
    # is representable, and the oracle must return it
    g = np.concatenate([[np.float32(1024.0)], np.full(100_000, np.float32(2.0**-17))]).astype(np.float32)
    s, f = oracle.check(g)
    assert f == 0
    assert s == 2.0**20 + 100_000 * 2.0**-34 != 2.0**20
    assert s == math.fsum(float(x) * float(x) for x in g)


def test_sumsq_of_many_terms_is_correctly_rounded():
    # 2^20 squares of wide-range binary32 values: within one binary64 ulp of
    # the correctly rounded exact sum (math.fsum)
    g = (RNG.standard_normal(1 << 20) * np.exp(RNG.uniform(-8, 8, 1 << 20))).astype(np.float32)
    s, _ = oracle.check(g)
    exact = math.fsum((g.astype(np.float64) ** 2).tolist())
    assert abs(s - exact) <= math.ulp(exact)


def test_norm_of_constant_vector_closed_form():
    n, c = 1 << 16, np.float32(-0.0029296875)  # exact in binary32 and bf16
    g = np.full(n, c, np.float32)
    s, _ = oracle.check(g)
    r = oracle.finalize(s, 0.0, 0, 0.0, 0)
    assert r.grad_norm == abs(float(c)) * math.sqrt(n)
    assert r.clip_coef == 1.0


@pytest.mark.parametrize("bad", ["pinf", "ninf", "nan", "pinf_ninf", "overflow"])
def test_nonfinite_is_flagged(bad):
    M, n = 4, 64
    grads = [random_bf16(n, 110, 118) for _ in range(M)]
    if bad == "pinf":
        grads[2][17] = 0x7F80
    elif bad == "ninf":
        grads[0][63] = 0xFF80
    elif bad == "nan":
        grads[3][0] = 0x7FC1
    elif bad == "pinf_ninf":  # +inf + -inf at one element -> NaN, still caught
        grads[1][5] = 0x7F80
        grads[2][5] = 0xFF80
    else:  # finite bf16 max twice overflows the binary32 sum
        grads[0][9] = 0x7F7F
        grads[1][9] = 0x7F7F
        grads[2][9] = 0x0000
        grads[3][9] = 0x0000
    g = oracle.reduce(grads)
    _, f = oracle.check(g)
    assert f == 1
    _, f0 = oracle.check(oracle.reduce([random_bf16(n, 110, 118) for _ in range(M)]))
    assert f0 == 0


# --------------------------------------------------------------------------
# Clip coefficient vs torch.nn.utils.clip_grad_norm_
# --------------------------------------------------------------------------

@pytest.mark.parametrize("max_norm,std", [(1.0, 1e-2), (1.0, 1e-4), (0.05, 1e-3), (3.0, 1.0)])
def test_clip_matches_torch_clip_grad_norm(max_norm, std):
    sizes = [513, 4096, 37]
    gs = [(RNG.standard_normal(k) * std).astype(np.float32) for k in sizes]
    st = oracle.SumSq()
    for g in gs:
        st.add(g)
    r = oracle.finalize(st.sumsq, 0.0, st.found_inf, max_norm, 0)
    ps = [torch.zeros(k, dtype=torch.float64, requires_grad=True) for k in sizes]
    for p, g in zip(ps, gs):
        p.grad = torch.from_numpy(g.astype(np.float64))
    tn = torch.nn.utils.clip_grad_norm_(ps, max_norm, norm_type=2.0, foreach=False)
    assert math.isclose(r.grad_norm, float(tn), rel_tol=1e-14)
    for p, g in zip(ps, gs):
        np.testing.assert_allclose(g.astype(np.float64) * r.clip_coef, p.grad.numpy(), rtol=1e-14, atol=0)


def test_clip_with_external_sumsq_and_nonfinite_norm():
    r = oracle.finalize(3.0, 1.0, 0, 1.0, 0)
    assert r.grad_norm == 2.0 and math.isclose(r.clip_coef, 1.0 / (2.0 + 1e-6), rel_tol=1e-15)
    r = oracle.finalize(math.inf, 0.0, 1, 1.0, 0)
    assert r.clip_coef == 0.0 and r.skipped == 0 and r.found_inf == 1
    r = oracle.finalize(math.nan, 0.0, 1, 1.0, 1)
    assert math.isnan(r.clip_coef) and r.skipped == 1
    r = oracle.finalize(4.0, 0.0, 0, 0.0, 1)  # max <= 0: clipping off
    assert r.clip_coef == 1.0 and r.skipped == 0


def test_clipped_gradient_norm_identity():
    g = (RNG.standard_normal(20000) * 1e-2).astype(np.float32)
    s, _ = oracle.check(g)
    r = oracle.finalize(s, 0.0, 0, 1.0, 0)
    assert r.clip_coef < 1.0
    clipped = math.sqrt(math.fsum((float(x) * r.clip_coef) ** 2 for x in g))
    assert math.isclose(clipped, 1.0 * r.grad_norm / (r.grad_norm + 1e-6), rel_tol=1e-12)
    # doubling every gradient barely moves the clipped gradient
    s2, _ = oracle.check(g * np.float32(2))
    r2 = oracle.finalize(s2, 0.0, 0, 1.0, 0)
    assert math.isclose(2 * r2.clip_coef, r.clip_coef, rel_tol=2e-6)


# --------------------------------------------------------------------------
# AdamW vs torch.optim.AdamW (float64) and closed forms
# --------------------------------------------------------------------------

def _state(n, rng, m_std=1e-5, v_std=1e-8, th_std=0.02, g_std=1e-4):
    th = (rng.standard_normal(n) * th_std).astype(np.float32)
    m = (rng.standard_normal(n) * m_std).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * v_std).astype(np.float32)
    g = (rng.standard_normal(n) * g_std).astype(np.float32)
    return th, m, v, g


def _torch_adamw(th, m, v, g, hp: oracle.HParams, coef):
    p = torch.from_numpy(th.astype(np.float64)).requires_grad_(True)
    opt = torch.optim.AdamW([p], lr=hp.lr, betas=(hp.beta1, hp.beta2), eps=hp.eps,
                            weight_decay=hp.weight_decay, foreach=False, fused=False)
    p.grad = torch.from_numpy(g.astype(np.float64) * coef)
    opt.state[p] = {"step": torch.tensor(float(hp.step - 1), dtype=torch.float64),
                    "exp_avg": torch.from_numpy(m.astype(np.float64)),
                    "exp_avg_sq": torch.from_numpy(v.astype(np.float64))}
    with torch.no_grad():
        opt.step()
    st = opt.state[p]
    return (p.detach().numpy().astype(np.float32), st["exp_avg"].numpy().astype(np.float32),
            st["exp_avg_sq"].numpy().astype(np.float32))


def _ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ia = bits32(a).astype(np.int64)
    ib = bits32(b).astype(np.int64)
    ia = np.where(ia >= 2**31, 2**31 - ia, ia)  # ordered integers
    ib = np.where(ib >= 2**31, 2**31 - ib, ib)
    return np.abs(ia - ib)


@pytest.mark.parametrize("t", [1, 2, 10, 100, 1000, 5000])
@pytest.mark.parametrize("hpset", ["c0", "ds"])
def test_adamw_matches_torch_adamw_float64(t, hpset, golden_dir):
    if hpset == "ds":
        p = json.load(open(os.path.join(golden_dir, "ds_config_blocks.json")))["optimizer"]["params"]
        hp = oracle.HParams(lr=p["lr"], beta1=p["betas"][0], beta2=p["betas"][1], eps=p["eps"],
                            weight_decay=p["weight_decay"], step=t)
    else:
        hp = oracle.HParams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=t)
    rng = np.random.default_rng(t * 7 + len(hpset))
    th, m, v, g = _state(8192, rng)
    if t == 1:
        m[:] = 0
        v[:] = 0
    coef = 0.8993
    o_th, o_m, o_v, o_out = oracle.adamw(th, m, v, g, hp, coef)
    r_th, r_m, r_v = _torch_adamw(th, m, v, g, hp, coef)
    # both evaluate in binary64 and round once; allow one ulp for double rounding
    for a, b in ((o_th, r_th), (o_m, r_m), (o_v, r_v)):
        d = _ulp_diff(a, b)
        assert d.max() <= 1
        assert (d == 0).mean() > 0.99
    assert np.array_equal(o_out, torch_f32_to_bf16(o_th))


def test_step1_closed_form():
    # With m = v = 0 at t = 1, the bias corrections cancel: m1 = (1-b1) g,
    # v1 = (1-b2) g^2, theta1 = theta0 - lr*wd*theta0 - lr*g/(|g|+eps).
    hp = oracle.HParams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1)
    rng = np.random.default_rng(11)
    th, _, _, g = _state(50000, rng, g_std=1e-3)
    z = np.zeros_like(th)
    o_th, o_m, o_v, _ = oracle.adamw(th, z, z, g, hp)
    th64, g64 = th.astype(np.float64), g.astype(np.float64)
    want = th64 - hp.lr * hp.weight_decay * th64 - hp.lr * g64 / (np.abs(g64) + hp.eps)
    assert _ulp_diff(o_th, want.astype(np.float32)).max() <= 1
    np.testing.assert_allclose(o_th, want, rtol=2e-6, atol=1e-7)
    assert _ulp_diff(o_m, (0.1 * g64).astype(np.float32)).max() <= 1
    assert _ulp_diff(o_v, (0.05 * g64 * g64).astype(np.float32)).max() <= 1


def test_adamw_against_60_digit_decimal():
    decimal.getcontext().prec = 60
    D = decimal.Decimal
    hp = oracle.HParams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=10)
    rng = np.random.default_rng(5)
    th, m, v, g = _state(64, rng)
    coef = 0.75
    o_th, o_m, o_v, _ = oracle.adamw(th, m, v, g, hp, coef)
    b1, b2, lr, eps, wd = (D(repr(x)) for x in (hp.beta1, hp.beta2, hp.lr, hp.eps, hp.weight_decay))
    bc1 = 1 - b1 ** hp.step
    bc2 = 1 - b2 ** hp.step
    for i in range(64):
        gi = D(float(g[i])) * D(coef)
        mi = b1 * D(float(m[i])) + (1 - b1) * gi
        vi = b2 * D(float(v[i])) + (1 - b2) * gi * gi
        ti = D(float(th[i])) * (1 - lr * wd) - lr * (mi / bc1) / ((vi / bc2).sqrt() + eps)
        for got, want in ((o_th[i], ti), (o_m[i], mi), (o_v[i], vi)):
            assert _ulp_diff(np.float32(got), np.float32(float(want))).max() <= 1


def test_adamw_degenerate_cases():
    rng = np.random.default_rng(3)
    th, m, v, g = _state(4096, rng)
    # lr = 0 leaves the master bit-identical
    o_th, _, _, _ = oracle.adamw(th, m, v, g, oracle.HParams(lr=0.0, step=7))
    assert np.array_equal(bits32(o_th), bits32(th))
    # wd = 0 is plain Adam: compare with torch Adam (no decay)
    hp = oracle.HParams(weight_decay=0.0, step=7)
    o_th, _, _, _ = oracle.adamw(th, m, v, g, hp)
    p = torch.from_numpy(th.astype(np.float64)).requires_grad_(True)
    opt = torch.optim.Adam([p], lr=hp.lr, betas=(hp.beta1, hp.beta2), eps=hp.eps, foreach=False)
    p.grad = torch.from_numpy(g.astype(np.float64))
    opt.state[p] = {"step": torch.tensor(6.0, dtype=torch.float64), "exp_avg": torch.from_numpy(m.astype(np.float64)),
                    "exp_avg_sq": torch.from_numpy(v.astype(np.float64))}
    with torch.no_grad():
        opt.step()
    assert _ulp_diff(o_th, p.detach().numpy().astype(np.float32)).max() <= 1
    # t >= 1000 with beta2 = 0.95: both bias corrections are 1 in binary64
    hp = oracle.HParams(step=1000)
    o_th, o_m, o_v, _ = oracle.adamw(th, m, v, g, hp)
    g64 = g.astype(np.float64)
    m1 = 0.9 * m.astype(np.float64) + 0.1 * g64
    v1 = 0.95 * v.astype(np.float64) + 0.05 * g64 * g64
    want = th.astype(np.float64) * (1 - 1e-4) - 1e-3 * m1 / (np.sqrt(v1) + 1e-8)
    assert _ulp_diff(o_th, want.astype(np.float32)).max() <= 1


# --------------------------------------------------------------------------
# Whole step: skip, multi-tensor, resume
# --------------------------------------------------------------------------

def _tensors(sizes, M, rng, t_std=1e-4):
    out = []
    for n in sizes:
        th, m, v, _ = _state(n, rng)
        grads = [oracle.f32_to_bf16((rng.standard_normal(n) * t_std).astype(np.float32)) for _ in range(M)]
        out.append(oracle.TensorState(grads, th, m, v, np.full(n, 0x1234, np.uint16)))
    return out


@pytest.mark.parametrize("val", [0x7F80, 0xFF80, 0x7FC0])
def test_skipped_step_leaves_state_unchanged(val):
    rng = np.random.default_rng(9)
    ts = _tensors([100, 4099, 512], 4, rng)
    ts[1].grads[3][4000] = val
    hp = oracle.HParams(step=5000, max_grad_norm=1.0, grad_scale=2.0**-16, skip_on_nonfinite=1)
    new, r = oracle.zero_step(ts, hp)
    assert r.found_inf == 1 and r.skipped == 1
    for a, b in zip(ts, new):
        for x, y in ((a.master, b.master), (a.exp_avg, b.exp_avg), (a.exp_avg_sq, b.exp_avg_sq)):
            assert np.array_equal(bits32(x), bits32(y))
        assert np.array_equal(a.param_out, b.param_out)


def test_nonfinite_without_skip_still_updates():
    rng = np.random.default_rng(10)
    ts = _tensors([300], 2, rng)
    ts[0].grads[0][7] = 0x7F80
    new, r = oracle.zero_step(ts, oracle.HParams(step=3))
    assert r.found_inf == 1 and r.skipped == 0
    assert np.isnan(new[0].master[7]) or np.isinf(new[0].master[7])
    assert np.isfinite(new[0].master[8])


def test_multi_tensor_list_equals_flat_concatenation():
    rng = np.random.default_rng(12)
    sizes = [512, 2048, 1, 4099, 11011, 512, 4097]
    M = 8
    ts = _tensors(sizes, M, rng, t_std=3e-3)
    hp = oracle.HParams(step=10, max_grad_norm=1.0)
    new, r = oracle.zero_step(ts, hp)
    flat = oracle.TensorState([np.concatenate([t.grads[k] for t in ts]) for k in range(M)],
                              np.concatenate([t.master for t in ts]), np.concatenate([t.exp_avg for t in ts]),
                              np.concatenate([t.exp_avg_sq for t in ts]), np.concatenate([t.param_out for t in ts]))
    newf, rf = oracle.zero_step([flat], hp)
    assert r.clip_coef < 1.0
    assert r.sumsq == rf.sumsq and r.clip_coef == rf.clip_coef
    for f in ("master", "exp_avg", "exp_avg_sq", "param_out"):
        cat = np.concatenate([getattr(t, f) for t in new])
        assert np.array_equal(cat.view(np.uint8), getattr(newf[0], f).view(np.uint8)), f


def test_resume_equals_uninterrupted():
    rng = np.random.default_rng(13)
    ts = _tensors([777], 3, rng)
    hp = lambda t: oracle.HParams(step=t, max_grad_norm=0.5)
    a = ts
    for t in range(1, 6):
        a, _ = oracle.zero_step(a, hp(t))
    b = ts
    for t in range(1, 3):
        b, _ = oracle.zero_step(b, hp(t))
    saved = [oracle.TensorState([g.copy() for g in x.grads], x.master.copy(), x.exp_avg.copy(), x.exp_avg_sq.copy(),
                                x.param_out.copy()) for x in b]
    for t in range(3, 6):
        saved, _ = oracle.zero_step(saved, hp(t))
    assert np.array_equal(bits32(a[0].master), bits32(saved[0].master))
    assert np.array_equal(bits32(a[0].exp_avg_sq), bits32(saved[0].exp_avg_sq))


# --------------------------------------------------------------------------
# Memory accounting vs the pages' table
# --------------------------------------------------------------------------

def test_memory_table_matches_pages(golden_dir):
    gold = {}
    for line in open(os.path.join(golden_dir, "cs336_memory_table.txt")):
        line = line.strip()
        if line and not line.startswith("#") and not line.startswith("key"):
            k, v = line.split()
            gold[k] = float(v)
    for k in ("param_bf16", "grad_bf16", "master_fp32", "exp_avg_fp32", "exp_avg_sq_fp32"):
        assert oracle.BYTES_PER_PARAM[k] == gold[k]
    assert oracle.bytes_per_param_naive_dp() == gold["total"]
    opt = oracle.BYTES_PER_PARAM["master_fp32"] + oracle.BYTES_PER_PARAM["exp_avg_fp32"] + \
        oracle.BYTES_PER_PARAM["exp_avg_sq_fp32"]
    assert opt == gold["optimizer_state"] and opt / gold["total"] == gold["optimizer_share"]
    per_gpu = oracle.bytes_per_gpu(gold["example_params"], int(gold["example_ranks"]), 0)
    assert per_gpu == gold["example_naive_dp_bytes_per_gpu"] and per_gpu > gold["example_a100_bytes"]
    # ZeRO-1 keeps parameters and gradients whole and splits the 12 optimizer bytes
    z1 = oracle.bytes_per_gpu(gold["example_params"], int(gold["example_ranks"]), 1)
    assert z1 < gold["example_a100_bytes"] < per_gpu
