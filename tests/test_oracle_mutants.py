"""Mutation check of the oracle's pins (CPU only; nothing here runs on a GPU).

Each mutant below is one plausible mistake planted in a copy of the oracle's C
source: a dropped term, a wrong sign, constant or index, a transposed operand,
a binary32 step taken in binary64 or the reverse, a branch turned the wrong
way. The copy is compiled with the oracle's own flags into a temporary
directory, and the oracle's pin suites (closed forms, exact emulations,
torch's AdamW and GradScaler, the pages' worked figures) run against it in a
child process that loads the copy in place of the oracle. Every mutant must
make at least one pin fail; the unmutated copy, built and run the same way,
must pass them all, so a failure comes from the planted mistake and not from
the harness.

Mutants that cannot change any result (equivalent mutants) are left out: for
example removing the explicit overflow-to-infinity branch of the bf16 encoder,
whose fall-through already encodes 2^128 as the infinity pattern, or moving
its normal/subnormal test up one binade, since both branches give the
smallest normal binade the same spacing, 2^-133."""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_SUITES = ["test_oracle_pins.py", "test_oracle_properties.py", "test_oracle_zero2.py",
              "test_oracle_loss_scale.py"]

FOLD_REDUCE = ("        float s = bf16_to_float(grads[0][i]);\n"
               "        for (int32_t r = 1; r < M; ++r) s = s + bf16_to_float(grads[r][i]);\n"
               "        g_out[i] = s * scale;\n")
FOLD_ACC = ("        float s = bf16_to_float(grads[0][i]);\n"
            "        for (int32_t r = 1; r < M; ++r) s = s + bf16_to_float(grads[r][i]);\n"
            "        acc[i] = accumulate ? acc[i] + s : s;\n")
UPDATE_CALL = "    if (!res->skipped)\n        for (int32_t t = 0; t < T; ++t)\n"
FINALIZE_CALL = "oracle_finalize(sumsq, external_sumsq, found_inf, hp->max_grad_norm, hp->skip_on_nonfinite, res);"

# (name, [(old, new) or (old, new, occurrence)]): old must occur exactly once,
# or, with an occurrence index, at least that many times.
MUTANTS = [
    # step 1-2: the rank fold and the unscale
    ("fold from +0 instead of rank 0's value",
     [(FOLD_REDUCE, FOLD_REDUCE.replace("float s = bf16_to_float(grads[0][i]);", "float s = 0.0f;")
       .replace("int32_t r = 1", "int32_t r = 0"))]),
    ("fold in descending rank order",
     [(FOLD_REDUCE, FOLD_REDUCE.replace("grads[0][i]", "grads[M - 1][i]")
       .replace("for (int32_t r = 1; r < M; ++r)", "for (int32_t r = M - 2; r >= 0; --r)"))]),
    ("fold in binary64",
     [(FOLD_REDUCE, FOLD_REDUCE.replace("float s =", "double s =").replace("g_out[i] = s * scale;",
                                                                           "g_out[i] = (float)(s * scale);"))]),
    ("every rank read from rank 0's replica",
     [(FOLD_REDUCE, FOLD_REDUCE.replace("bf16_to_float(grads[r][i])", "bf16_to_float(grads[0][i])"))]),
    ("last rank dropped from the fold",
     [(FOLD_REDUCE, FOLD_REDUCE.replace("r < M;", "r < M - 1;"))]),
    ("unscale by the binary64 scale",
     [("    const float scale = (float)grad_scale;\n    for (int64_t i = 0; i < n; ++i) {\n        float s",
       "    const double scale = grad_scale;\n    for (int64_t i = 0; i < n; ++i) {\n        float s"),
      ("        g_out[i] = s * scale;\n", "        g_out[i] = (float)((double)s * scale);\n")]),
    ("unscale each replica before the fold",
     [(FOLD_REDUCE, FOLD_REDUCE.replace("float s = bf16_to_float(grads[0][i]);",
                                        "float s = bf16_to_float(grads[0][i]) * scale;")
       .replace("s = s + bf16_to_float(grads[r][i]);", "s = s + bf16_to_float(grads[r][i]) * scale;")
       .replace("g_out[i] = s * scale;", "g_out[i] = s;"))]),
    # bf16 decode and encode
    ("bf16 subnormals decoded a binade low",
     [("ldexp((double)f, -126 - 7)", "ldexp((double)f, -127 - 7)")]),
    ("bf16 exponent bias off by one", [("ldexp((double)(128 + f), e - 127 - 7)", "ldexp((double)(128 + f), e - 126 - 7)")]),
    ("bf16 emit truncates", [("nearbyint(ldexp(a, -q))", "trunc(ldexp(a, -q))")]),
    ("bf16 emit rounds ties away from zero", [("nearbyint(ldexp(a, -q))", "round(ldexp(a, -q))")]),
    ("bf16 emit drops the sign of NaN", [("signbit(x) ? 0xFFC0 : 0x7FC0", "0x7FC0")]),
    ("bf16 emit keeps one fraction bit too few",
     [("const int q = (e - 1 >= -126) ? (e - 1 - 7) : (-126 - 7);",
       "const int q = (e - 1 >= -126) ? (e - 1 - 6) : (-126 - 7);")]),
    ("bf16 NaN codes decoded as infinities", [("        if (f != 0) return sign ? -NAN : NAN;\n", "")]),
    ("bf16 negative zero decoded as +0",
     [("return (float)(sign ? -mag : mag);", "return (float)(sign && mag != 0.0 ? -mag : mag);")]),
    ("bf16 emit: normal spacing used for the largest subnormals",
     [("const int q = (e - 1 >= -126) ? (e - 1 - 7) : (-126 - 7);",
       "const int q = (e - 1 >= -127) ? (e - 1 - 7) : (-126 - 7);")]),
    ("bf16 emit: exponent field off by one", [("((e - 1 + 127) << 7)", "((e - 1 + 126) << 7)")]),
    ("bf16 emit: infinity loses its sign", [("if (isinf(x)) return (uint16_t)(s | 0x7F80);", "if (isinf(x)) return 0x7F80;")]),
    # step 3: flag and sum of squares
    ("flag misses infinities", [("if (!isfinite(g[i])) bad = 1;", "if (isnan(g[i])) bad = 1;")]),
    ("flag misses NaN", [("if (!isfinite(g[i])) bad = 1;", "if (isinf(g[i])) bad = 1;")]),
    ("sum of |g| instead of g^2", [("const double x = (double)g[i] * (double)g[i];",
                                     "const double x = fabs((double)g[i]);")]),
    ("squares taken in binary32", [("const double x = (double)g[i] * (double)g[i];",
                                    "const double x = (double)(g[i] * g[i]);")]),
    ("sum of squares not chained across tensors", [("double s = *sumsq, c = *comp;", "double s = 0.0, c = *comp;")]),
    ("plain left-to-right sum of squares (no compensation)",
     [("if (isfinite(t)) c += fabs(s) >= fabs(x) ? (s - t) + x : (x - t) + s;", "(void)x;")]),
    ("compensation with the operands' roles swapped",
     [("if (isfinite(t)) c += fabs(s) >= fabs(x) ? (s - t) + x : (x - t) + s;",
       "if (isfinite(t)) c += fabs(s) >= fabs(x) ? (x - t) + s : (s - t) + x;")]),
    ("compensation dropped from the total", [("return isfinite(sumsq) ? sumsq + comp : sumsq;", "return sumsq;")]),
    ("flag not chained across tensors", [("int32_t bad = *found_inf;", "int32_t bad = 0;")]),
    # step 4: finalize
    ("external sum of squares dropped", [("const double total = sumsq + external_sumsq;", "const double total = sumsq;")]),
    ("norm without the square root", [("const double norm = sqrt(total);", "const double norm = total;")]),
    ("clip without the 1e-6", [("coef = max_grad_norm / (norm + 1e-6);", "coef = max_grad_norm / norm;")]),
    ("clip coefficient not capped at 1", [("        if (coef > 1.0) coef = 1.0; /* a NaN coefficient stays NaN */\n", "")]),
    ("clip applied when max_grad_norm is 0", [("if (max_grad_norm > 0.0) {", "if (max_grad_norm >= 0.0) {")]),
    ("skip ignores the switch",
     [("res->skipped = (found_inf && skip_on_nonfinite) ? 1 : 0;", "res->skipped = found_inf ? 1 : 0;")]),
    ("skip never taken", [("res->skipped = (found_inf && skip_on_nonfinite) ? 1 : 0;", "res->skipped = 0;")]),
    ("ZeRO-1 step ignores external_sumsq",
     [(FINALIZE_CALL, FINALIZE_CALL.replace("external_sumsq", "0.0"), 0)]),
    ("flag reported only when the step skips",
     [("res->found_inf = found_inf ? 1 : 0;", "res->found_inf = (found_inf && skip_on_nonfinite) ? 1 : 0;")]),
    ("NaN clip coefficient replaced by 1", [("if (coef > 1.0) coef = 1.0;", "if (!(coef <= 1.0)) coef = 1.0;")]),
    # step 5-6: AdamW and the emit
    ("clip coefficient not applied", [("const double gi = (double)g[i] * coef;", "const double gi = (double)g[i];")]),
    ("no bias correction of m", [("const double m_hat = m / bc1;", "const double m_hat = m;")]),
    ("no bias correction of v", [("const double v_hat = v / bc2;", "const double v_hat = v;")]),
    ("bias correction of m at t + 1", [("pow(hp->beta1, t)", "pow(hp->beta1, t + 1.0)")]),
    ("bias correction of m with beta2", [("const double bc1 = 1.0 - pow(hp->beta1, t);", "const double bc1 = 1.0 - pow(hp->beta2, t);")]),
    ("v's bias correction under the root twice", [("const double v_hat = v / bc2;", "const double v_hat = v / sqrt(bc2);")]),
    ("eps inside the square root", [("(sqrt(v_hat) + hp->eps)", "sqrt(v_hat + hp->eps)")]),
    ("weight decay not scaled by lr", [("(1.0 - hp->lr * hp->weight_decay)", "(1.0 - hp->weight_decay)")]),
    ("weight decay dropped", [("(double)master[i] * (1.0 - hp->lr * hp->weight_decay)", "(double)master[i]")]),
    ("L2 penalty in the gradient (Adam, not AdamW)",
     [("const double gi = (double)g[i] * coef;",
       "const double gi = (double)g[i] * coef + hp->weight_decay * (double)master[i];"),
      ("(double)master[i] * (1.0 - hp->lr * hp->weight_decay)", "(double)master[i]")]),
    ("Adam step added instead of subtracted", [("- hp->lr * m_hat", "+ hp->lr * m_hat")]),
    ("beta1 in the second moment",
     [("hp->beta2 * (double)exp_avg_sq[i] + (1.0 - hp->beta2)", "hp->beta1 * (double)exp_avg_sq[i] + (1.0 - hp->beta1)")]),
    ("betas' complements swapped",
     [("hp->beta1 * (double)exp_avg[i] + (1.0 - hp->beta1) * gi", "hp->beta1 * (double)exp_avg[i] + hp->beta1 * gi")]),
    ("first power of g in the second moment", [("(1.0 - hp->beta2) * gi * gi", "(1.0 - hp->beta2) * gi")]),
    ("second moment from the unclipped gradient",
     [("(1.0 - hp->beta2) * gi * gi", "(1.0 - hp->beta2) * (double)g[i] * (double)g[i]")]),
    ("moments stored into each other's arrays",
     [("        exp_avg[i] = (float)m;\n        exp_avg_sq[i] = (float)v;\n",
       "        exp_avg[i] = (float)v;\n        exp_avg_sq[i] = (float)m;\n")]),
    ("moment terms rounded to binary32",
     [("const double m = hp->beta1 * (double)exp_avg[i] + (1.0 - hp->beta1) * gi;",
       "const double m = (double)((float)(hp->beta1 * (double)exp_avg[i]) + (float)((1.0 - hp->beta1) * gi));"),
      ("const double v = hp->beta2 * (double)exp_avg_sq[i] + (1.0 - hp->beta2) * gi * gi;",
       "const double v = (double)((float)(hp->beta2 * (double)exp_avg_sq[i]) + (float)((1.0 - hp->beta2) * gi * gi));")]),
    ("emit from the old master",
     [("        master[i] = (float)theta;\n        out[i] = bf16_round_nearest_even(master[i]);\n",
       "        out[i] = bf16_round_nearest_even(master[i]);\n        master[i] = (float)theta;\n")]),
    ("skipped ZeRO-1 step still updates", [(UPDATE_CALL, "    if (1)\n        for (int32_t t = 0; t < T; ++t)\n", 0)]),
    ("ZeRO-1 step updates only the first tensor",
     [("        for (int32_t t = 0; t < T; ++t)\n            oracle_adamw(", "        for (int32_t t = 0; t < 1 && t < T; ++t)\n            oracle_adamw(", 0)]),
    # ZeRO-2 accumulation
    ("accumulate always adds", [("acc[i] = accumulate ? acc[i] + s : s;", "acc[i] = acc[i] + s;")]),
    ("accumulate never adds", [("acc[i] = accumulate ? acc[i] + s : s;", "acc[i] = s;")]),
    ("accumulate folds in descending rank order",
     [(FOLD_ACC, FOLD_ACC.replace("grads[0][i]", "grads[M - 1][i]")
       .replace("for (int32_t r = 1; r < M; ++r)", "for (int32_t r = M - 2; r >= 0; --r)"))]),
    ("accumulated step drops the scale", [("gs[t][i] = ts[t].grad_acc[i] * scale;", "gs[t][i] = ts[t].grad_acc[i];")]),
    ("accumulated step scales in binary64",
     [("gs[t][i] = ts[t].grad_acc[i] * scale;", "gs[t][i] = (float)((double)ts[t].grad_acc[i] * hp->grad_scale);")]),
    ("skipped accumulated step still updates",
     [(UPDATE_CALL, "    if (1)\n        for (int32_t t = 0; t < T; ++t)\n", 1)]),
    ("accumulated step ignores external_sumsq",
     [(FINALIZE_CALL, FINALIZE_CALL.replace("external_sumsq", "0.0"), 1)]),
    # the dynamic loss scale
    ("initial scale a power low", [("ldexp(1.0, c->initial_scale_power)", "ldexp(1.0, c->initial_scale_power - 1)")]),
    ("hysteresis ignored", [("if (s->overflows >= c->hysteresis) {", "if (1) {")]),
    ("hysteresis off by one", [("if (s->overflows >= c->hysteresis) {", "if (s->overflows > c->hysteresis) {")]),
    ("floor test reversed", [("s->scale = half < c->min_scale ? c->min_scale : half;", "s->scale = half > c->min_scale ? c->min_scale : half;")]),
    ("no floor at min_loss_scale", [("s->scale = half < c->min_scale ? c->min_scale : half;", "s->scale = half;")]),
    ("clean step keeps the overflow count",
     [("        s->overflows = 0;\n        s->good_steps += 1;\n", "        s->good_steps += 1;\n")]),
    ("overflow keeps the clean-step count",
     [("        s->good_steps = 0;\n        s->overflows += 1;\n", "        s->overflows += 1;\n")]),
    ("window off by one", [("if (s->good_steps >= c->window) {", "if (s->good_steps > c->window) {")]),
    ("growth to infinity", [("if (isfinite(twice)) s->scale = twice;", "s->scale = twice;")]),
    ("inverse scale not refreshed", [("    s->inv_scale = 1.0f / s->scale;\n}\n", "}\n")]),
]


def plant(src: str, edits) -> str:
    for e in edits:
        old, new = e[0], e[1]
        count = src.count(old)
        if len(e) == 2:
            assert count == 1, (old, count)
            src = src.replace(old, new)
        else:
            k = e[2]
            assert count > k, (old, count)
            at = -1
            for _ in range(k + 1):
                at = src.index(old, at + 1)
            src = src[:at] + new + src[at + len(old):]
    return src


def build_copy(src: str, where: str) -> str:
    c, so = os.path.join(where, "zero_oracle.c"), os.path.join(where, "libzero_oracle.so")
    with open(c, "w") as f:
        f.write(src)
    subprocess.run(["gcc", *oracle._CFLAGS, "-o", so, c, "-lm", "-pthread"], check=True, capture_output=True)
    return so


def run_pins(so: str, where: str) -> subprocess.CompletedProcess:
    """The pin suites against the library at so, in a child process whose
    working directory (and so its example database) is the scratch directory."""
    env = dict(os.environ, **{oracle._OVERRIDE_ENV: so})
    tests = [os.path.join(ROOT, "tests", f) for f in PIN_SUITES]
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
           "--hypothesis-seed=0", f"--rootdir={ROOT}", *tests]
    return subprocess.run(cmd, cwd=where, env=env, capture_output=True, text=True, timeout=600)


def workers() -> int:
    return max(1, min(6, (os.cpu_count() or 2) - 1))


@pytest.fixture(scope="module")
def source():
    with open(oracle._SRC) as f:
        return f.read()


def test_every_mutant_applies_to_the_current_source(source):
    names = [m[0] for m in MUTANTS]
    assert len(set(names)) == len(names)
    for name, edits in MUTANTS:
        assert plant(source, edits) != source, name


def test_pins_kill_every_planted_mistake(source):
    def one(job):
        name, edits = job
        with tempfile.TemporaryDirectory(prefix="oracle_mutant_") as d:
            so = build_copy(plant(source, edits), d)
            r = run_pins(so, d)
        tail = (r.stdout + r.stderr).strip().splitlines()[-3:]
        return name, r.returncode, tail

    jobs = [("unmutated copy", [])] + MUTANTS
    with cf.ThreadPoolExecutor(workers()) as ex:
        results = list(ex.map(one, jobs))

    control = results[0]
    assert control[1] == 0, f"the unmutated copy fails its own pins: {control}"
    survivors = [(n, t) for n, rc, t in results[1:] if rc != 1]
    assert not survivors, "mistakes no pin catches (or a harness error): " + repr(survivors)
