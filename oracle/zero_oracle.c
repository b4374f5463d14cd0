/*
 * zero_oracle.c -- plain, slow, sequential CPU oracle for the per-rank
 * ZeRO-1 shard step of mixed-precision data-parallel training.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load or call this code. The HIP library
 * never includes, links or calls it, and it shares no source with that
 * library (no headers, helpers, tables or constants).
 *
 * Pages cited below:
 *   [ZeRO ch.]  "第2章 软件程序与专用硬件的结合" (zhurongshuo.com), section
 *               2.3.4 "ZeRO：数据并行的革命性优化", Stage 1 paragraph.
 *   [CS336 L7]  "CS336 Lecture 7: Parallelism 1" (hqhq1025.github.io),
 *               sections "五种基本集合通信操作" (collective primitives),
 *               "核心恒等式" (All-Reduce = Reduce-Scatter + All-Gather),
 *               "训练内存的详细分析" (the 16-bytes-per-parameter table), and
 *               "ZeRO Stage 1：优化器状态分片" (the four-step workflow).
 *   [5D post]   gsyq.cn/news/457874, section 3.2 trap 3 (AMP gradient
 *               scaling, loss going to inf) and section 4.2 (the
 *               deepspeed_config.json optimizer block: AdamW with lr, betas,
 *               eps, weight_decay; the fp16 loss-scale block).
 *
 * What one step computes, in this order ([CS336 L7] ZeRO Stage 1 workflow:
 * reduce-scatter the gradients, update the local shard, all-gather the
 * parameters):
 *
 *   1. reduce    s[i] = fold over ranks r = 0..M-1, ascending, of the bf16
 *                gradient replicas converted to binary32, starting from the
 *                rank-0 value; every add is one binary32 add rounded to
 *                nearest even. GPU i receives the *summed* gradient of its
 *                shard ([CS336 L7] Stage 1 step 2, Reduce-Scatter).
 *   2. unscale   g[i] = s[i] * scale32, scale32 = the scale rounded once to
 *                binary32 (AMP: the gradient is multiplied by 1/S after the
 *                sum; [5D post] 3.2 trap 3).
 *   3. check     found_inf = any g[i] not finite; sumsq = sum of g[i]^2:
 *                the exact squares added in index order with a compensated
 *                binary64 sum (within about one rounding of the exact sum).
 *   4. finalize  norm = sqrt(sumsq + external_sumsq);
 *                coef = min(1, max_norm / (norm + 1e-6)) when max_norm > 0,
 *                else 1 (NaN propagates); skip = found_inf && skip_on_nonfinite.
 *                Clipping by the global L2 norm is not described on the pages;
 *                this is the common framework convention, read as such.
 *   5. update    (only when not skipped; a skipped step writes nothing)
 *                AdamW with bias correction, eps outside the square root and
 *                weight decay decoupled from the gradient and scaled by lr
 *                ([5D post] 4.2 names the optimizer "AdamW" and its knobs;
 *                [CS336 L7] memory table: fp32 master, fp32 first and second
 *                moments). Evaluated in binary64 from the binary32 state and
 *                rounded once to binary32 on store.
 *   6. emit      out[i] = bf16 round-to-nearest-even of the new binary32
 *                master value (the shard the all-gather would broadcast;
 *                [CS336 L7] Stage 1 step 4).
 *
 *   7. scale     (AMP with a dynamic loss scale) after the step, the loss
 *                scale S moves on the step's non-finite flag: see
 *                oracle_loss_scale_update below ([5D post] 4.2 fp16 block,
 *                3.2 trap 3).
 *
 * ZeRO-2, streaming ([CS336 L7] "ZeRO Stage 2": each layer's gradient is
 * reduced to the rank that owns it as soon as backward has produced it, so
 * no rank holds a whole gradient; [5D post] 4.2: gradients travel in buckets
 * of reduce_bucket_size, over gradient_accumulation_steps micro-batches):
 *
 *   1'. accumulate  for each micro-batch k and each tensor of a bucket:
 *                s = the step-1 fold of that micro-batch's M replicas;
 *                acc[i] = s (first micro-batch) or acc[i] + s (later ones),
 *                one binary32 add: the fp32 shard gradient is a running sum
 *                of reduce-scatter results.
 *   2'-6'.       the step then runs steps 2-6 on g[i] = acc[i] * scale32.
 *   With one micro-batch this is exactly the ZeRO-1 step above.
 *
 * Compile with -O2 -ffp-contract=off and without -ffast-math: the binary32
 * fold of step 1 must be exactly the sequence of rounded adds written here.
 */
#define _POSIX_C_SOURCE 200809L /* pthread_once */

#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* bf16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.           */
/* ------------------------------------------------------------------------ */

/* Value of one bf16 bit pattern, read from its fields. */
static float bf16_value_from_fields(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 7) & 0xFF;
    const int f = h & 0x7F;
    double mag;
    if (e == 0xFF) {
        if (f != 0) return sign ? -NAN : NAN;
        return sign ? -INFINITY : INFINITY;
    }
    if (e == 0)
        mag = ldexp((double)f, -126 - 7);           /* 0.f x 2^-126 */
    else
        mag = ldexp((double)(128 + f), e - 127 - 7); /* 1.f x 2^(e-127) */
    return (float)(sign ? -mag : mag);               /* exact in binary32 */
}

static float g_bf16_table[65536];
static pthread_once_t g_bf16_table_once = PTHREAD_ONCE_INIT;

static void bf16_table_fill(void)
{
    for (uint32_t h = 0; h < 65536u; ++h) g_bf16_table[h] = bf16_value_from_fields((uint16_t)h);
}

/* Filled once per process, also when several threads call in at once. */
static void bf16_table_init(void) { pthread_once(&g_bf16_table_once, bf16_table_fill); }

static inline float bf16_to_float(uint16_t h) { return g_bf16_table[h]; }

/* Largest finite bf16: (2 - 2^-7) * 2^127 = 255 * 2^120. */
#define BF16_MAX_FINITE (255.0 * 0x1p120)

/* Encode a value that is already exactly representable in bf16. */
static uint16_t bf16_encode_exact(double r, uint16_t s)
{
    int e;
    if (r == 0.0) return s;
    frexp(r, &e); /* r = f * 2^e, 0.5 <= f < 1: unbiased exponent e-1 */
    if (e - 1 >= -126) {
        const int frac = (int)ldexp(r, -(e - 1 - 7)) - 128;
        return (uint16_t)(s | ((e - 1 + 127) << 7) | frac);
    }
    return (uint16_t)(s | (int)ldexp(r, 126 + 7));
}

/* Round a binary32 value to bf16, to nearest, ties to even (IEEE 754). */
static uint16_t bf16_round_nearest_even(float x)
{
    if (isnan(x)) return signbit(x) ? 0xFFC0 : 0x7FC0; /* quiet NaN, sign kept */
    const uint16_t s = signbit(x) ? 0x8000 : 0;
    if (isinf(x)) return (uint16_t)(s | 0x7F80);
    const double a = fabs((double)x);
    if (a == 0.0) return s;
    int e;
    frexp(a, &e);
    /* exponent of the last bit bf16 keeps: 7 fraction bits below the leading
     * bit for normals, fixed at 2^-133 for subnormals */
    const int q = (e - 1 >= -126) ? (e - 1 - 7) : (-126 - 7);
    const double k = nearbyint(ldexp(a, -q)); /* ties to even */
    const double r = ldexp(k, q);
    if (r > BF16_MAX_FINITE) return (uint16_t)(s | 0x7F80);
    return bf16_encode_exact(r, s);
}

/* ------------------------------------------------------------------------ */
/* Exported helpers for the pins.                                           */
/* ------------------------------------------------------------------------ */

void oracle_bf16_to_f32(const uint16_t* in, float* out, int64_t n)
{
    bf16_table_init();
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_to_float(in[i]);
}

void oracle_f32_to_bf16(const float* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_round_nearest_even(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Step 1 + 2: reduce the M replicas of one shard, then unscale.            */
/* ------------------------------------------------------------------------ */

void oracle_reduce(const uint16_t* const* grads, int32_t M, int64_t n, double grad_scale, float* g_out)
{
    bf16_table_init();
    const float scale = (float)grad_scale;
    for (int64_t i = 0; i < n; ++i) {
        float s = bf16_to_float(grads[0][i]);
        for (int32_t r = 1; r < M; ++r) s = s + bf16_to_float(grads[r][i]);
        g_out[i] = s * scale;
    }
}

/* ------------------------------------------------------------------------ */
/* Step 3: non-finite flag and sum of squares.                              */
/* ------------------------------------------------------------------------ */
/*
 * The sum of squares is the exact sum of the squares, rounded to binary64.
 * Each square is exact in binary64 (a binary32 value has 24 significant bits,
 * its square at most 48). The terms are added in index order with Neumaier's
 * compensated summation (A. Neumaier, "Rundungsfehleranalyse einiger
 * Verfahren zur Summation endlicher Summen", ZAMM 54, 1974): a second binary64
 * word carries the rounding error of every add, and s + c is then within
 * about one rounding of the exact sum at any length. A plain left-to-right
 * binary64 sum is not: over the 2e9 squares of the AMP workload, whose terms
 * have few significant bits, it drifts below the exact sum by 5e-9 relative.
 * Once the sum is not finite the correction is no longer tracked and the
 * result is the plain sum's inf or NaN. The pair (*sumsq, *comp) is in/out,
 * so that consecutive slices chain in index order.
 */
void oracle_check(const float* g, int64_t n, double* sumsq, double* comp, int32_t* found_inf)
{
    double s = *sumsq, c = *comp;
    int32_t bad = *found_inf;
    for (int64_t i = 0; i < n; ++i) {
        if (!isfinite(g[i])) bad = 1;
        const double x = (double)g[i] * (double)g[i];
        const double t = s + x;
        if (isfinite(t)) c += fabs(s) >= fabs(x) ? (s - t) + x : (x - t) + s;
        s = t;
    }
    *sumsq = s;
    *comp = c;
    *found_inf = bad;
}

/* The sum that a pair (sumsq, comp) of oracle_check stands for. */
double oracle_sumsq_total(double sumsq, double comp) { return isfinite(sumsq) ? sumsq + comp : sumsq; }

/* ------------------------------------------------------------------------ */
/* Step 4: norm, clip coefficient, skip decision.                           */
/* ------------------------------------------------------------------------ */

typedef struct {
    double sumsq;     /* local sum of squares plus external_sumsq */
    double grad_norm; /* sqrt(sumsq) */
    double clip_coef; /* multiplier applied to g before the update */
    int32_t found_inf;
    int32_t skipped;
} oracle_result;

void oracle_finalize(double sumsq, double external_sumsq, int32_t found_inf, double max_grad_norm,
                     int32_t skip_on_nonfinite, oracle_result* res)
{
    const double total = sumsq + external_sumsq;
    const double norm = sqrt(total);
    double coef = 1.0;
    if (max_grad_norm > 0.0) {
        coef = max_grad_norm / (norm + 1e-6);
        if (coef > 1.0) coef = 1.0; /* a NaN coefficient stays NaN */
    }
    res->sumsq = total;
    res->grad_norm = norm;
    res->clip_coef = coef;
    res->found_inf = found_inf ? 1 : 0;
    res->skipped = (found_inf && skip_on_nonfinite) ? 1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Step 5 + 6: AdamW on the fp32 master, m, v, then the bf16 emit.          */
/* ------------------------------------------------------------------------ */

typedef struct {
    double lr, beta1, beta2, eps, weight_decay;
    int64_t step;         /* t >= 1: the index of this update */
    double max_grad_norm; /* <= 0: no clipping */
    double grad_scale;    /* multiplies the fp32 sum */
    int32_t skip_on_nonfinite;
} oracle_hparams;

void oracle_adamw(float* master, float* exp_avg, float* exp_avg_sq, const float* g, uint16_t* out, int64_t n,
                  const oracle_hparams* hp, double coef)
{
    const double t = (double)hp->step;
    const double bc1 = 1.0 - pow(hp->beta1, t); /* bias corrections of m and v */
    const double bc2 = 1.0 - pow(hp->beta2, t);
    for (int64_t i = 0; i < n; ++i) {
        const double gi = (double)g[i] * coef;
        const double m = hp->beta1 * (double)exp_avg[i] + (1.0 - hp->beta1) * gi;
        const double v = hp->beta2 * (double)exp_avg_sq[i] + (1.0 - hp->beta2) * gi * gi;
        const double m_hat = m / bc1;
        const double v_hat = v / bc2;
        const double theta = (double)master[i] * (1.0 - hp->lr * hp->weight_decay)
                             - hp->lr * m_hat / (sqrt(v_hat) + hp->eps);
        exp_avg[i] = (float)m;
        exp_avg_sq[i] = (float)v;
        master[i] = (float)theta;
        out[i] = bf16_round_nearest_even(master[i]);
    }
}

/* ------------------------------------------------------------------------ */
/* The whole step over a list of tensors (one shard each).                  */
/* ------------------------------------------------------------------------ */

typedef struct {
    int64_t n;
    const uint16_t* const* grads; /* M pointers, n bf16 values each */
    float* master;
    float* exp_avg;
    float* exp_avg_sq;
    uint16_t* param_out; /* n bf16 values */
} oracle_tensor;

/* Returns 0, or -1 when scratch memory cannot be had. */
int32_t oracle_zero_step(const oracle_tensor* ts, int32_t T, int32_t M, const oracle_hparams* hp,
                         double external_sumsq, oracle_result* res)
{
    float** gs = (float**)calloc((size_t)(T > 0 ? T : 1), sizeof(float*));
    if (!gs) return -1;
    double sumsq = 0.0, comp = 0.0;
    int32_t found_inf = 0;
    int32_t rc = 0;
    for (int32_t t = 0; t < T; ++t) {
        gs[t] = (float*)malloc((size_t)(ts[t].n > 0 ? ts[t].n : 1) * sizeof(float));
        if (!gs[t]) { rc = -1; goto done; }
        oracle_reduce(ts[t].grads, M, ts[t].n, hp->grad_scale, gs[t]);
        oracle_check(gs[t], ts[t].n, &sumsq, &comp, &found_inf);
    }
    sumsq = oracle_sumsq_total(sumsq, comp);
    oracle_finalize(sumsq, external_sumsq, found_inf, hp->max_grad_norm, hp->skip_on_nonfinite, res);
    if (!res->skipped)
        for (int32_t t = 0; t < T; ++t)
            oracle_adamw(ts[t].master, ts[t].exp_avg, ts[t].exp_avg_sq, gs[t], ts[t].param_out, ts[t].n, hp,
                         res->clip_coef);
done:
    for (int32_t t = 0; t < T; ++t) free(gs[t]);
    free(gs);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* ZeRO-2 streaming: per-bucket accumulation, then the step from the        */
/* accumulated fp32 shard gradient.                                         */
/* ------------------------------------------------------------------------ */

/* One micro-batch of one tensor: fold its M replicas (step 1, without the
 * scale) and store the fold (accumulate == 0) or add it to acc (binary32). */
void oracle_grad_accumulate(const uint16_t* const* grads, int32_t M, int64_t n, float* acc, int32_t accumulate)
{
    bf16_table_init();
    for (int64_t i = 0; i < n; ++i) {
        float s = bf16_to_float(grads[0][i]);
        for (int32_t r = 1; r < M; ++r) s = s + bf16_to_float(grads[r][i]);
        acc[i] = accumulate ? acc[i] + s : s;
    }
}

typedef struct {
    int64_t n;
    const float* grad_acc; /* n fp32: the accumulated (unscaled) shard gradient */
    float* master;
    float* exp_avg;
    float* exp_avg_sq;
    uint16_t* param_out;
} oracle_acc_tensor;

/* Steps 2-6 on g = acc * scale32 over a tensor list. Returns 0, or -1 when
 * scratch memory cannot be had. */
int32_t oracle_zero_step_accumulated(const oracle_acc_tensor* ts, int32_t T, const oracle_hparams* hp,
                                     double external_sumsq, oracle_result* res)
{
    float** gs = (float**)calloc((size_t)(T > 0 ? T : 1), sizeof(float*));
    if (!gs) return -1;
    const float scale = (float)hp->grad_scale;
    double sumsq = 0.0, comp = 0.0;
    int32_t found_inf = 0;
    int32_t rc = 0;
    for (int32_t t = 0; t < T; ++t) {
        gs[t] = (float*)malloc((size_t)(ts[t].n > 0 ? ts[t].n : 1) * sizeof(float));
        if (!gs[t]) { rc = -1; goto done; }
        for (int64_t i = 0; i < ts[t].n; ++i) gs[t][i] = ts[t].grad_acc[i] * scale;
        oracle_check(gs[t], ts[t].n, &sumsq, &comp, &found_inf);
    }
    sumsq = oracle_sumsq_total(sumsq, comp);
    oracle_finalize(sumsq, external_sumsq, found_inf, hp->max_grad_norm, hp->skip_on_nonfinite, res);
    if (!res->skipped)
        for (int32_t t = 0; t < T; ++t)
            oracle_adamw(ts[t].master, ts[t].exp_avg, ts[t].exp_avg_sq, gs[t], ts[t].param_out, ts[t].n, hp,
                         res->clip_coef);
done:
    for (int32_t t = 0; t < T; ++t) free(gs[t]);
    free(gs);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Step 7: the dynamic loss scale.                                          */
/* ------------------------------------------------------------------------ */
/*
 * [5D post] 4.2 configures the fp16 loss scale with loss_scale 0 (dynamic),
 * initial_scale_power, loss_scale_window, hysteresis and min_loss_scale, and
 * 3.2 trap 3 describes the scaler's cycle (scale the loss, step on unscaled
 * gradients, update the scale). The pages print the knobs, not the rule; the
 * reading taken from their names:
 *   - S starts at 2^initial_scale_power.
 *   - A step whose unscaled gradient holds a non-finite value is an overflow
 *     (the step itself is skipped). The hysteresis-th overflow in a row,
 *     counted since the last clean step or the last halving, halves S, never
 *     below min_loss_scale, and restarts the count.
 *   - A clean step clears the overflow count. The loss_scale_window-th clean
 *     step in a row, counted since the last overflow or the last doubling,
 *     doubles S, unless 2S is not a finite binary32 value, and restarts the
 *     count.
 *   - S is a binary32 value; the step multiplies the fp32 sum by
 *     inv_scale = 1/S rounded to binary32 (exact while S is a power of two).
 * With hysteresis 1 this is the growth/backoff rule of a gradient scaler
 * with growth factor 2, backoff factor 1/2 and growth interval
 * loss_scale_window.
 */

typedef struct {
    float scale;        /* S */
    float inv_scale;    /* 1/S, rounded to binary32 */
    int32_t good_steps; /* clean steps in a row since the last overflow or doubling */
    int32_t overflows;  /* overflows in a row since the last clean step or halving */
} oracle_loss_scale;

typedef struct {
    int32_t initial_scale_power;
    int32_t window;     /* loss_scale_window, >= 1 */
    int32_t hysteresis; /* >= 1 */
    float min_scale;    /* min_loss_scale, > 0 */
} oracle_loss_scale_config;

void oracle_loss_scale_init(const oracle_loss_scale_config* c, oracle_loss_scale* s)
{
    s->scale = (float)ldexp(1.0, c->initial_scale_power);
    s->inv_scale = 1.0f / s->scale;
    s->good_steps = 0;
    s->overflows = 0;
}

void oracle_loss_scale_update(const oracle_loss_scale_config* c, int32_t found_inf, oracle_loss_scale* s)
{
    if (found_inf) {
        s->good_steps = 0;
        s->overflows += 1;
        if (s->overflows >= c->hysteresis) {
            const float half = s->scale / 2.0f;
            s->scale = half < c->min_scale ? c->min_scale : half;
            s->overflows = 0;
        }
    } else {
        s->overflows = 0;
        s->good_steps += 1;
        if (s->good_steps >= c->window) {
            const float twice = s->scale * 2.0f;
            if (isfinite(twice)) s->scale = twice;
            s->good_steps = 0;
        }
    }
    s->inv_scale = 1.0f / s->scale;
}
