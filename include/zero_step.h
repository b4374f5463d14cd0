/*
 * zero_step.h -- C ABI of the fused per-rank ZeRO-1 shard step for MI355X
 * (gfx950).
 *
 * The operation ("CS336 Lecture 7: Parallelism 1", section "ZeRO Stage 1：
 * 优化器状态分片", the four-step workflow; "第2章 软件程序与专用硬件的结合",
 * section 2.3.4, Stage 1): every data-parallel rank holds a full bf16
 * gradient; a reduce-scatter gives rank i the *sum* over ranks of shard i;
 * rank i updates shard i with the optimizer state it alone keeps (fp32
 * master weights, fp32 first and second moments: the 16-bytes-per-parameter
 * table of section "训练内存的详细分析"); an all-gather then broadcasts the
 * updated bf16 parameters. This library performs the part of that step that
 * runs at one rank, on one GPU: the M gradient replicas of the shard are M
 * buffers in this GPU's memory.
 *
 *   g[i]  = (((g_0[i] + g_1[i]) + g_2[i]) + ... + g_{M-1}[i]) * grad_scale
 *           in binary32, ranks in ascending order, from the rank-0 value;
 *   found_inf = any g[i] is inf or NaN;
 *   norm  = sqrt(sum of g[i]^2 + external_sumsq)        (binary64 partials)
 *   coef  = min(1, max_grad_norm / (norm + 1e-6)) if max_grad_norm > 0 else 1
 *   skip  = found_inf && skip_on_nonfinite      (a skipped step writes nothing)
 *   AdamW (bias-corrected, eps outside the root, decay scaled by lr),
 *   evaluated in binary64 from the fp32 state and rounded once on store:
 *     m   = b1*m + (1-b1)*(coef*g);   v = b2*v + (1-b2)*(coef*g)^2
 *     w   = w*(1 - lr*wd) - lr * (m/(1-b1^t)) / (sqrt(v/(1-b2^t)) + eps)
 *   out   = bf16 round-to-nearest-even of the new fp32 w (the all-gather payload)
 *
 * AMP unscaling (grad_scale = 1/S) and the inf/NaN skip follow the
 * loss-scaling behaviour described in gsyq.cn/news/457874, section 3.2 trap 3;
 * the AdamW knob names follow its section 4.2 optimizer block. Clipping by the
 * global L2 norm is not on the pages; the coefficient is the common framework
 * convention above.
 *
 * Conventions for every entry point:
 *  - Pointers named *_dev, and every tensor pointer, are device pointers on the
 *    current HIP device. Arrays of pointers (grads) are HOST arrays holding
 *    device pointers. Structs passed by pointer (hparams, tensors) are host
 *    memory, read during the call only.
 *  - bf16 data are raw 16-bit codes (uint16). fp32 data are IEEE binary32.
 *  - The caller owns all memory. The library allocates no device memory; it
 *    keeps a small host-side cache of workspace plans. (The one exception is
 *    zero_step_noalloc's static scratch, a device array that is part of the
 *    library's code and is loaded with it.)
 *  - Every call is asynchronous on `stream` (0 = the null stream) and returns
 *    after enqueueing. Results are device-resident.
 *  - Errors: an int status (ZERO_OK or ZERO_ERR_*). On any error nothing is
 *    launched and no memory is written. n == 0 is a valid no-op. No C++
 *    exception crosses the ABI.
 *  - Any alignment is accepted; when all pointers of a tensor share their
 *    alignment modulo 16 bytes the kernels use 16-byte vector accesses.
 *  - The fused forms launch one workgroup per tile of a pass, at most
 *    2^31 - 1 tiles (an update pass's tiles hold 2048 elements: about 4.4e12
 *    elements per call); a larger call is ZERO_ERR_INVALID_ARGUMENT.
 *  - Outputs must not alias inputs, except the in-place master/exp_avg/
 *    exp_avg_sq. The library never advances `step`: the caller increments it
 *    when the result record says `skipped == 0`.
 */
#ifndef ZERO_STEP_H
#define ZERO_STEP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define ZERO_OK 0
#define ZERO_ERR_INVALID_ARGUMENT 1    /* null pointer, bad size or hyperparameter */
#define ZERO_ERR_WORKSPACE_TOO_SMALL 2 /* ws_bytes below the size query's answer */
#define ZERO_ERR_HIP 3                 /* a HIP runtime call failed (launch, copy) */
#define ZERO_ERR_STALE_WORKSPACE 4     /* set in zero_result.status by the device when a
                                          workspace no longer holds the plan of this call;
                                          the step then wrote nothing */
#define ZERO_ERR_BUCKET_PARTIALS 5     /* set in zero_result.status by zero_step_accumulated
                                          when a bucket partial was not written by a final
                                          zero_bucket_reduce with this stamp and grad_scale;
                                          the step then wrote nothing */
#define ZERO_ERR_SCRATCH_TOO_SMALL 6   /* zero_step_noalloc: the call's workspace would exceed
                                          ZERO_NOALLOC_SCRATCH_BYTES; nothing was launched */

/* Largest M accepted (ranks, i.e. gradient replicas per shard). */
#define ZERO_MAX_RANKS 65536

/* AdamW hyperparameters of one step (names as in a deepspeed_config.json
 * optimizer block, gsyq.cn/news/457874 section 4.2). Host memory. */
typedef struct zero_adamw_hparams {
    double lr;                 /* learning rate, finite, >= 0 */
    double beta1;              /* first-moment decay, in [0, 1) */
    double beta2;              /* second-moment decay, in [0, 1) */
    double eps;                /* added to sqrt of the bias-corrected v, finite, >= 0 */
    double weight_decay;       /* decoupled: w *= (1 - lr*weight_decay); finite */
    int64_t step;              /* t >= 1: index of this update (bias corrections) */
    double max_grad_norm;      /* > 0: clip g to this global L2 norm; <= 0: off */
    double grad_scale;         /* multiplies the fp32 sum, rounded to fp32 once: 1,
                                  1/S for an AMP loss scale S, 1/M for a mean; finite, > 0 */
    int32_t skip_on_nonfinite; /* nonzero: any inf/NaN in g skips the whole update */
    int32_t reserved;          /* must be 0 */
} zero_adamw_hparams;

/* One tensor's shard in a zero_step bucket list. Host memory. */
typedef struct zero_tensor {
    int64_t n;                /* elements in this shard, >= 0 */
    const void* const* grads; /* HOST array of M device pointers, n bf16 each (read only) */
    float* master;            /* device, n fp32 master weights, updated in place */
    float* exp_avg;           /* device, n fp32 first moments, updated in place */
    float* exp_avg_sq;        /* device, n fp32 second moments, updated in place */
    void* param_out;          /* device, n bf16 codes, written (the all-gather payload) */
} zero_tensor;

/* Device-resident result record of a step, 32 bytes, written by the library. */
typedef struct zero_result {
    double sumsq;      /* sum of g^2 over every element of the call, plus external_sumsq */
    double clip_coef;  /* coefficient applied to g, binary64 (1 when clipping is off) */
    float grad_norm;   /* sqrt(sumsq) rounded to fp32 (inf/NaN when found_inf) */
    int32_t found_inf; /* 1 when any unscaled reduced gradient is inf or NaN */
    int32_t skipped;   /* 1 when the update was not applied */
    int32_t status;    /* ZERO_OK, or ZERO_ERR_STALE_WORKSPACE */
} zero_result;

/*
 * zero_shard_reduce -- the reduce-scatter arithmetic at one rank
 * ("CS336 Lecture 7", section "五种基本集合通信操作", Reduce-Scatter; section
 * "ZeRO Stage 1", step 2: GPU i receives the summed gradient of shard i).
 *   g_out[i] = fl32(fold_{r=0..M-1} bf16->fp32(grads[r][i])) * fl32(grad_scale)
 * grads: host array of M device pointers to n bf16 codes. g_out: device, n
 * fp32, must not overlap any replica. 1 <= M <= ZERO_MAX_RANKS, n >= 0,
 * grad_scale finite and > 0. Bit-exact: the fold order is fixed.
 */
int zero_shard_reduce(const void* const* grads, int32_t M, int64_t n, double grad_scale, float* g_out,
                      hipStream_t stream);

/*
 * zero_grad_check_norm_workspace_bytes -- workspace size for
 * zero_grad_check_norm over n elements (0 when n == 0).
 */
size_t zero_grad_check_norm_workspace_bytes(int64_t n);

/*
 * zero_grad_check_norm -- non-finite check, global L2 norm, clip coefficient
 * and skip decision over an fp32 gradient g (device, n elements), written to
 * the device record res_dev. The check and the skip follow the loss-scaling
 * cycle of gsyq.cn/news/457874 section 3.2 trap 3 (a step whose unscaled
 * gradient holds inf or NaN is not applied); the norm is global because each
 * rank holds one shard of the summed gradient ("CS336 Lecture 7", "ZeRO
 * Stage 1" step 2), so the other ranks' share enters as external_sumsq.
 * Clipping by that norm is not on the pages: the coefficient is the common
 * framework rule stated at the top of this header. hp may be NULL (no clipping, no skip); only its
 * max_grad_norm and skip_on_nonfinite are read. external_sumsq is the other
 * ranks' sum of squares for a multi-GPU caller, 0 on one GPU: NaN and +inf
 * propagate into the norm, a negative value is ZERO_ERR_INVALID_ARGUMENT (as
 * in every call that takes it). ws: device workspace of at least
 * zero_grad_check_norm_workspace_bytes(n) bytes, contents irrelevant on entry.
 * The sum of squares uses exact binary64 squares and a fixed reduction tree
 * (bitwise repeatable on one device).
 */
int zero_grad_check_norm(const float* g, int64_t n, const zero_adamw_hparams* hp, double external_sumsq,
                         void* ws, size_t ws_bytes, zero_result* res_dev, hipStream_t stream);

/*
 * zero_adamw_step -- AdamW on fp32 master/exp_avg/exp_avg_sq (device, n each,
 * in place) from the fp32 gradient g (device, n), plus the bf16 emit into
 * param_out (device, n bf16 codes): the local update of "CS336 Lecture 7",
 * "ZeRO Stage 1" step 3 (rank i updates shard i with the optimizer state it
 * alone keeps: the fp32 master copy and both moments of the table in section
 * "训练内存的详细分析") and the bf16 payload of the all-gather in step 4; the
 * knobs are those of the AdamW optimizer block in gsyq.cn/news/457874
 * section 4.2, and the formula is the one stated at the top of this header. hp is required (max_grad_norm and
 * skip_on_nonfinite are ignored here). res_dev (device, may be NULL) supplies
 * clip_coef and skipped from zero_grad_check_norm: when skipped is set the
 * kernel writes nothing; when res_dev is NULL the coefficient is 1.
 */
int zero_adamw_step(float* master, float* exp_avg, float* exp_avg_sq, const float* g, void* param_out, int64_t n,
                    const zero_adamw_hparams* hp, const zero_result* res_dev, hipStream_t stream);

/*
 * zero_step_workspace_bytes -- workspace size for zero_step over this tensor
 * list and hyperparameters (pointers inside `tensors` are not read). Returns 0
 * on invalid arguments.
 */
size_t zero_step_workspace_bytes(const zero_tensor* tensors, int32_t T, int32_t M, const zero_adamw_hparams* hp);

/*
 * zero_step -- the fused step over a bucket list of T tensor shards, each with
 * M bf16 replicas ("CS336 Lecture 7", "ZeRO Stage 1" steps 2-3 and the
 * payload of step 4; per-layer buckets as in its section "ZeRO Stage 2").
 * The norm and found_inf are global over all T tensors. Without clipping and
 * skipping it is one streaming pass; with either, a first pass writes the fp32
 * reduced gradient to the workspace and a second pass applies the update.
 * Above ZERO_STREAM_STORES_MIN_PARAMS parameters in all the call's tensors
 * together, the state stores of the updating pass stream out to memory (see
 * ZERO_BUCKET_STREAM_STORES); the results do not depend on it.
 * ws: device workspace of zero_step_workspace_bytes(...) bytes, 256-byte
 * aligned. The workspace caches the tensor table of the call; it belongs to
 * the library from this call until the caller reuses it for anything else,
 * and two calls that share a workspace must not run concurrently. res_dev:
 * device result record. external_sumsq as for zero_grad_check_norm. Returns
 * ZERO_ERR_WORKSPACE_TOO_SMALL if ws_bytes is short.
 */
int zero_step(const zero_tensor* tensors, int32_t T, int32_t M, const zero_adamw_hparams* hp,
              double external_sumsq, void* ws, size_t ws_bytes, zero_result* res_dev, hipStream_t stream);

/* Bytes of the static device workspace of zero_step_noalloc (64 MiB per GPU). */
#define ZERO_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)

/*
 * zero_step_noalloc -- zero_step for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the workspace is a static device array inside the
 * library, ZERO_NOALLOC_SCRATCH_BYTES bytes on each GPU, taken when the
 * library's code is loaded on that GPU and held until the process ends. The
 * call itself allocates nothing (no hipMalloc, no hipFree, no allocating
 * library routine); the caller still passes the tensors and res_dev.
 * Arguments, results and errors as for zero_step, plus
 * ZERO_ERR_SCRATCH_TOO_SMALL, returned before anything is launched, when
 * zero_step_workspace_bytes(tensors, T, M, hp) exceeds the scratch: the
 * single-pass plan takes about 12 bytes per 1024 elements plus 112 + 8*M
 * bytes per tensor (every workload up to billions of elements fits), a
 * two-pass plan (clipping or skipping) also holds the fp32 gradient, 4 bytes
 * per element (up to about 16 million elements).
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's plan and re-arms its own counters: calls on one GPU must be ordered
 * (one stream, or events); calls that overlap on one GPU race and corrupt
 * each other's results. A HIP graph that captures a call holds the scratch's
 * address, so a replay is valid only while no other call with a different
 * tensor list has used the scratch since the capture.
 */
int zero_step_noalloc(const zero_tensor* tensors, int32_t T, int32_t M, const zero_adamw_hparams* hp,
                      double external_sumsq, zero_result* res_dev, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Dynamic loss scale (AMP).
 *
 * gsyq.cn/news/457874 configures the fp16 loss scale with the fp16 block of
 * its section 4.2 listing (loss_scale 0 = dynamic, initial_scale_power,
 * loss_scale_window, hysteresis, min_loss_scale) and describes the scaler's
 * cycle in section 3.2 trap 3 (scale the loss, step on unscaled gradients,
 * update the scale). The pages name the knobs, not the rule; the rule read
 * from them:
 *   - S starts at 2^initial_scale_power;
 *   - a step whose unscaled reduced gradient holds inf/NaN is skipped and is
 *     an overflow; the hysteresis-th overflow in a row (counted since the last
 *     clean step or halving) halves S, never below min_scale, and restarts the
 *     count;
 *   - a clean step clears the overflow count; the window-th clean step in a
 *     row (counted since the last overflow or doubling) doubles S unless 2S is
 *     not a finite binary32 value, and restarts the count;
 *   - inv_scale = 1/S rounded to binary32 (exact while S is a power of two).
 * The state stays in device memory: a training loop moves it without a host
 * synchronisation.
 * ------------------------------------------------------------------------ */

/* Loss-scale state, 16 bytes, device memory, written by the library. */
typedef struct zero_loss_scale {
    float scale;        /* S: the factor the loss was multiplied by */
    float inv_scale;    /* 1/S rounded to binary32 */
    int32_t good_steps; /* clean steps in a row since the last overflow or doubling */
    int32_t overflows;  /* overflowing steps in a row since the last clean step or halving */
} zero_loss_scale;

/* Loss-scale knobs (host memory, read during the call). */
typedef struct zero_loss_scale_config {
    int32_t initial_scale_power; /* S starts at 2^power; -126 <= power <= 127 */
    int32_t window;              /* loss_scale_window: clean steps per doubling, >= 1 */
    int32_t hysteresis;          /* overflows in a row per halving, >= 1 */
    float min_scale;             /* min_loss_scale: finite, > 0 */
} zero_loss_scale_config;

/*
 * zero_loss_scale_init -- write the initial state (S = 2^initial_scale_power,
 * counts 0) to ls_dev (device, 16 bytes).
 */
int zero_loss_scale_init(const zero_loss_scale_config* cfg, zero_loss_scale* ls_dev, hipStream_t stream);

/*
 * zero_loss_scale_update -- move the state ls_dev on the found_inf flag of
 * the result record res_dev (device) of a step that used it, e.g. after
 * zero_shard_reduce with grad_scale = inv_scale and zero_grad_check_norm.
 * A record whose status is not ZERO_OK leaves the state unchanged.
 */
int zero_loss_scale_update(const zero_loss_scale_config* cfg, const zero_result* res_dev, zero_loss_scale* ls_dev,
                           hipStream_t stream);

/*
 * zero_step_amp_workspace_bytes -- workspace size for zero_step_amp (always
 * the two-pass plan). Returns 0 on invalid arguments.
 */
size_t zero_step_amp_workspace_bytes(const zero_tensor* tensors, int32_t T, int32_t M, const zero_adamw_hparams* hp);

/*
 * zero_step_amp -- zero_step with the dynamic loss scale in ls_dev: the fp32
 * sum is multiplied by fl32(grad_scale) * inv_scale (a binary32 product read
 * from ls_dev by the device, so the host never needs S); a step with any
 * inf/NaN in the unscaled gradient is always skipped (skip_on_nonfinite is
 * ignored); after the fold, the state moves on the step's found_inf. No
 * extra launch: the workgroup that writes the result record also updates
 * ls_dev. ls_dev must not change while the call runs, and two calls that share
 * ls_dev must be ordered (one stream). Other arguments and errors as for
 * zero_step; the workspace size is zero_step_amp_workspace_bytes(...).
 */
int zero_step_amp(const zero_tensor* tensors, int32_t T, int32_t M, const zero_adamw_hparams* hp,
                  const zero_loss_scale_config* cfg, zero_loss_scale* ls_dev, double external_sumsq, void* ws,
                  size_t ws_bytes, zero_result* res_dev, hipStream_t stream);

/* ------------------------------------------------------------------------
 * ZeRO-2, streaming.
 *
 * "CS336 Lecture 7: Parallelism 1", section "ZeRO Stage 2": as backward
 * produces each layer's gradient, it is reduced at once to the rank that owns
 * its shard, and the local copy is freed, so no rank holds a whole gradient.
 * gsyq.cn/news/457874 section 4.2 sends gradients in buckets
 * (reduce_bucket_size) and accumulates gradient_accumulation_steps
 * micro-batches per step. At one rank, on one GPU:
 *   - zero_bucket_reduce, once per bucket and micro-batch, as the bucket's M
 *     replicas arrive: acc[i] = fold(replicas) for the first micro-batch, or
 *     acc[i] = acc[i] + fold(replicas) (one binary32 add) for later ones. The
 *     fold is zero_shard_reduce's, without the scale: acc is the running sum
 *     of the reduce-scatter results. On the last micro-batch (FINAL) the call
 *     also writes the bucket's sum of squares and non-finite flag of
 *     g = acc * fl32(grad_scale) to a 32-byte bucket partial, stamped;
 *   - zero_step_accumulated, once per step: combines the bucket partials in
 *     index order into the result record (norm, clip coefficient, skip), then
 *     applies AdamW and the bf16 emit from g = acc * fl32(grad_scale), as
 *     zero_step does from its fold.
 * With one micro-batch, the state this writes is bit-identical to zero_step's
 * over the same replicas when clipping is off (the norm's summation tree
 * differs, so a clipped step may differ by the last bit of the coefficient).
 * ------------------------------------------------------------------------ */

/* flags of zero_bucket_reduce */
#define ZERO_BUCKET_ACCUMULATE 1 /* add the fold to acc; otherwise store it (first micro-batch) */
#define ZERO_BUCKET_FINAL 2      /* last micro-batch of the step: also write the bucket partial */
/* flag of zero_bucket_step: the state stores of the pass stream out to memory
 * (non-temporal, system scope) instead of waiting in the caches. Results are
 * the same either way; it is faster when the step's buckets together write
 * more than the GPU's 256 MiB Infinity Cache holds, i.e. above
 * ZERO_STREAM_STORES_MIN_PARAMS parameters (12 bytes of state and 2 of bf16
 * output each), and slower below. zero_step and zero_step_accumulated make
 * this choice themselves from the size of the step. */
#define ZERO_BUCKET_STREAM_STORES 4
#define ZERO_STREAM_STORES_MIN_PARAMS ((256ll << 20) / 14)

/* One tensor shard of a gradient bucket. Host memory. */
typedef struct zero_grad_shard {
    int64_t n;                /* elements in this shard, >= 0 */
    const void* const* grads; /* HOST array of M device pointers, n bf16 each (read only) */
    float* grad_acc;          /* device, n fp32: the shard's accumulated gradient, updated */
} zero_grad_shard;

/* One bucket's share of the step's norm and flag, 32 bytes, device memory. */
typedef struct zero_bucket_partial {
    double sumsq;      /* sum over the bucket of g^2, g = acc * fl32(grad_scale) (binary64) */
    uint64_t stamp;    /* the stamp of the final zero_bucket_reduce that wrote it */
    int32_t found_inf; /* 1 when any g of the bucket is inf or NaN */
    float grad_scale;  /* fl32(grad_scale) of that call */
    int64_t reserved;  /* written 0 */
} zero_bucket_partial;

/* One tensor shard of a zero_step_accumulated list. Host memory. */
typedef struct zero_acc_tensor {
    int64_t n;              /* elements in this shard, >= 0 */
    const float* grad_acc;  /* device, n fp32: the accumulated gradient (read only) */
    float* master;          /* device, n fp32, updated in place */
    float* exp_avg;         /* device, n fp32, updated in place */
    float* exp_avg_sq;      /* device, n fp32, updated in place */
    void* param_out;        /* device, n bf16 codes, written */
} zero_acc_tensor;

/*
 * zero_bucket_reduce_workspace_bytes -- workspace size for zero_bucket_reduce
 * over this bucket (pointers inside `shards` are not read); 0 on invalid
 * arguments.
 */
size_t zero_bucket_reduce_workspace_bytes(const zero_grad_shard* shards, int32_t T, int32_t M);

/*
 * zero_bucket_reduce -- fold one micro-batch of one bucket (T tensor shards,
 * M bf16 replicas each) into the shards' fp32 accumulators, per `flags`
 * (ZERO_BUCKET_ACCUMULATE, ZERO_BUCKET_FINAL; other bits are an error).
 * With ZERO_BUCKET_FINAL, grad_scale (finite, > 0; the step's) and stamp (any
 * value that differs from the previous step's, e.g. an iteration count) go
 * into *partial_dev (device, 32 bytes); without it they are ignored and
 * partial_dev may be NULL. ws: device workspace of
 * zero_bucket_reduce_workspace_bytes(...) bytes, 256-byte aligned, one per
 * bucket (it caches the bucket's tables; calls that share one must not run
 * concurrently). A workspace that no longer holds this bucket's tables is
 * detected on the device: nothing is written but *partial_dev, whose stamp is
 * then invalid (zero_step_accumulated reports it; a later final call on a
 * valid workspace would overwrite it, so call zero_workspace_forget before
 * reusing a bucket workspace for anything else). The accumulators must not
 * overlap the replicas or each other.
 */
int zero_bucket_reduce(const zero_grad_shard* shards, int32_t T, int32_t M, int32_t flags, double grad_scale,
                       uint64_t stamp, zero_bucket_partial* partial_dev, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/*
 * zero_bucket_reduce_amp -- zero_bucket_reduce under the dynamic loss scale
 * ls_dev (device): the final pass squares acc * (fl32(grad_scale) *
 * inv_scale), the binary32 product read from ls_dev on the device, and
 * stores that product in the partial's grad_scale. ls_dev is only read; it
 * must not move between a bucket's final pass and the step that consumes the
 * partials (zero_step_accumulated_amp moves it at the end of the step).
 */
int zero_bucket_reduce_amp(const zero_grad_shard* shards, int32_t T, int32_t M, int32_t flags, double grad_scale,
                           const zero_loss_scale* ls_dev, uint64_t stamp, zero_bucket_partial* partial_dev, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/*
 * zero_step_accumulated_workspace_bytes -- workspace size for
 * zero_step_accumulated over this tensor list; 0 on invalid arguments.
 */
size_t zero_step_accumulated_workspace_bytes(const zero_acc_tensor* tensors, int32_t T);

/*
 * zero_step_accumulated -- the step from the accumulated shard gradients:
 * partials_dev (device, nbuckets >= 0 records, each written by the final
 * zero_bucket_reduce of one bucket with this `stamp` and hp->grad_scale) are
 * combined in index order, with external_sumsq, into res_dev (norm, clip
 * coefficient, skip, as zero_step); unless skipped, AdamW and the bf16 emit
 * are applied to every tensor from g = acc * fl32(hp->grad_scale). A partial
 * with another stamp or scale sets res_dev->status = ZERO_ERR_BUCKET_PARTIALS
 * and nothing is written. The state stores stream out above
 * ZERO_STREAM_STORES_MIN_PARAMS parameters, as in zero_step. ws: device
 * workspace of zero_step_accumulated_workspace_bytes(...) bytes, 256-byte
 * aligned, as for zero_step.
 */
int zero_step_accumulated(const zero_acc_tensor* tensors, int32_t T, const zero_adamw_hparams* hp,
                          const zero_bucket_partial* partials_dev, int32_t nbuckets, uint64_t stamp,
                          double external_sumsq, void* ws, size_t ws_bytes, zero_result* res_dev,
                          hipStream_t stream);

/*
 * zero_step_accumulated_amp -- zero_step_accumulated under the dynamic loss
 * scale ls_dev (device, with its config cfg): the multiplier is
 * fl32(hp->grad_scale) * inv_scale read on the device (the partials must
 * carry that product, as zero_bucket_reduce_amp writes it); a step with any
 * inf/NaN is always skipped (skip_on_nonfinite is ignored); after the update
 * the state moves on the step's found_inf (one more small launch). Workspace
 * as for zero_step_accumulated.
 */
int zero_step_accumulated_amp(const zero_acc_tensor* tensors, int32_t T, const zero_adamw_hparams* hp,
                              const zero_loss_scale_config* cfg, zero_loss_scale* ls_dev,
                              const zero_bucket_partial* partials_dev, int32_t nbuckets, uint64_t stamp,
                              double external_sumsq, void* ws, size_t ws_bytes, zero_result* res_dev,
                              hipStream_t stream);

/* ------------------------------------------------------------------------
 * ZeRO-2, the final micro-batch fused with the update.
 *
 * Without clipping and without skipping, no element's update waits for the
 * global norm, so the last micro-batch of a bucket can be folded and applied
 * in one pass instead of being stored to the accumulator and read back by
 * zero_step_accumulated ("CS336 Lecture 7", "ZeRO Stage 2": each bucket is
 * reduced to its owner as soon as backward has produced it; here its owner
 * also updates it then). Per element of the bucket:
 *   g   = (acc + fold(replicas)) * fl32(grad_scale)   with ZERO_BUCKET_ACCUMULATE
 *   g   = fold(replicas) * fl32(grad_scale)           without (one micro-batch)
 *   AdamW on master, m, v and the bf16 emit, exactly as zero_step; acc is read,
 *   never written. The bucket's sum of squares and non-finite flag of g go to
 *   a stamped bucket partial, as a final zero_bucket_reduce writes it.
 * The step's result record then comes from zero_step_accumulated with no
 * tensors (T = 0, ws may be NULL): it combines the bucket partials in index
 * order with external_sumsq. The state equals, bit for bit, what
 * zero_bucket_reduce (FINAL) followed by zero_step_accumulated writes.
 * Traffic per element: 2M + 26 bytes for one micro-batch (2M + 30 with the
 * accumulator), against 2M + 4 + 30 in two passes.
 * ------------------------------------------------------------------------ */

/* One tensor shard of a fused final bucket pass. Host memory. */
typedef struct zero_bucket_tensor {
    int64_t n;                /* elements in this shard, >= 0 */
    const void* const* grads; /* HOST array of M device pointers, n bf16 each (read only) */
    const float* grad_acc;    /* device, n fp32: the earlier micro-batches' sum, read with
                                 ZERO_BUCKET_ACCUMULATE (may be NULL otherwise); not written */
    float* master;            /* device, n fp32, updated in place */
    float* exp_avg;           /* device, n fp32, updated in place */
    float* exp_avg_sq;        /* device, n fp32, updated in place */
    void* param_out;          /* device, n bf16 codes, written */
} zero_bucket_tensor;

/*
 * zero_bucket_step_workspace_bytes -- workspace size for zero_bucket_step over
 * this bucket (pointers inside `tensors` are not read); 0 on invalid arguments.
 */
size_t zero_bucket_step_workspace_bytes(const zero_bucket_tensor* tensors, int32_t T, int32_t M);

/*
 * zero_bucket_step -- the final micro-batch of one bucket (T tensor shards,
 * M bf16 replicas each), folded, added to the accumulator when `flags` has
 * ZERO_BUCKET_ACCUMULATE (without it: the bucket's only micro-batch), scaled
 * and applied with AdamW and the bf16 emit in one pass, its state stores
 * streamed when `flags` has ZERO_BUCKET_STREAM_STORES (any other bit is an
 * error);
 * the bucket partial *partial_dev (device, 32 bytes) gets the bucket's sum of
 * squares and flag with `stamp` and fl32(hp->grad_scale). hp must have
 * max_grad_norm <= 0 and skip_on_nonfinite == 0 (otherwise
 * ZERO_ERR_INVALID_ARGUMENT: the update would have to wait for the norm).
 * A non-finite gradient is flagged in the partial and still applied, as
 * zero_step does without skipping. ws: device workspace of
 * zero_bucket_step_workspace_bytes(...) bytes, 256-byte aligned, one per
 * bucket (it caches the bucket's tables; calls that share one must not run
 * concurrently); a workspace that no longer holds the bucket's tables is
 * detected on the device, and then nothing is written but an invalid
 * partial. Buckets are independent: different buckets may run on different
 * streams.
 */
int zero_bucket_step(const zero_bucket_tensor* tensors, int32_t T, int32_t M, int32_t flags,
                     const zero_adamw_hparams* hp, uint64_t stamp, zero_bucket_partial* partial_dev, void* ws,
                     size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * CPU-offloaded step (ZeRO-Offload).
 *
 * "第2章 软件程序与专用硬件的结合" section 2.3.4 names ZeRO-Offload, which
 * moves the optimizer state to CPU memory; gsyq.cn/news/457874 section 4.2
 * configures it (offload_optimizer: device cpu, pin_memory true) and reports
 * its trade: less GPU memory, a slower step, CPU-GPU transfers of ~20 GB/s.
 * Here the fp32 master, m and v of the shard live in host memory. The GPU
 * folds the M replicas, unscales, flags and squares (the first pass of the
 * two-pass step, into a device fp32 gradient); the gradient goes to pinned
 * host memory in chunks; host threads apply AdamW to each chunk as it lands
 * (binary64, the same formula and rounding as the GPU kernels) and emit bf16;
 * each bf16 chunk goes back to the device shard. The result equals zero_step's
 * over the same replicas: 4 + 2 bytes per parameter cross the host link
 * instead of 12 bytes of state living in HBM.
 * ------------------------------------------------------------------------ */

/* One tensor shard of an offloaded step. Host memory. */
typedef struct zero_offload_tensor {
    int64_t n;                /* elements in this shard, >= 0 */
    const void* const* grads; /* HOST array of M device pointers, n bf16 each (read only) */
    float* master;            /* HOST memory, n fp32, updated in place */
    float* exp_avg;           /* HOST memory, n fp32, updated in place */
    float* exp_avg_sq;        /* HOST memory, n fp32, updated in place */
    void* param_out;          /* DEVICE, n bf16 codes, written by host-to-device copies */
} zero_offload_tensor;

/* Device workspace size of zero_offload_step (plan, result record, the fp32
 * gradient, one 32-byte partial per fold group); 0 on invalid arguments. */
size_t zero_offload_workspace_bytes(const zero_offload_tensor* tensors, int32_t T, int32_t M);

/* Pinned host workspace size of zero_offload_step (staging: 4 bytes of
 * gradient and 2 bytes of bf16 output per element); 0 on invalid arguments. */
size_t zero_offload_host_workspace_bytes(const zero_offload_tensor* tensors, int32_t T);

/*
 * zero_offload_step -- the step with the optimizer state in host memory.
 * hp, external_sumsq and the result as for zero_step (*res_host, HOST memory,
 * is written before the call returns). ws: device workspace of
 * zero_offload_workspace_bytes(...) bytes, 256-byte aligned (it caches the
 * call's tables, as for zero_step). host_ws: PINNED host memory
 * (hipHostMalloc) of zero_offload_host_workspace_bytes(...) bytes, 64-byte
 * aligned. threads: host threads of the update (0: the size of the process's
 * CPU affinity mask). The call waits for the GPU's fold and returns once
 * master, m and v are updated on the host (or the step is skipped); the
 * bf16 copies into param_out are then enqueued, and `stream` is made to wait
 * for them, so work later on `stream` sees the new shard. Those copies read
 * host_ws: it stays allocated and untouched until `stream` has passed them,
 * and calls that share a host workspace must be issued on one stream.
 * Argument errors are reported before anything is launched; a HIP error
 * during the transfers (ZERO_ERR_HIP) can leave the host state partly
 * updated, and the call drains its copies before returning it.
 * Without clipping, skipping or a dynamic loss scale the update needs nothing
 * global, so the fold runs in groups of tiles and the host updates each piece
 * of the gradient as it arrives; the state is the same as with one fold pass
 * (and as zero_step's), while the reported sum of squares combines the group
 * partials in group order (it may differ from zero_step's in the last bits).
 */
int zero_offload_step(const zero_offload_tensor* tensors, int32_t T, int32_t M, const zero_adamw_hparams* hp,
                      double external_sumsq, void* ws, size_t ws_bytes, void* host_ws, size_t host_ws_bytes,
                      zero_result* res_host, int32_t threads, hipStream_t stream);

/*
 * zero_offload_step_amp -- zero_offload_step under the dynamic loss scale
 * ls_dev (device, with its config cfg): the GPU's fold multiplies by
 * fl32(hp->grad_scale) * inv_scale read on the device, a step with any inf/NaN
 * is always skipped, and the fold's last workgroup moves the state, as in
 * zero_step_amp; the host update is unchanged. Workspaces as for
 * zero_offload_step.
 */
int zero_offload_step_amp(const zero_offload_tensor* tensors, int32_t T, int32_t M, const zero_adamw_hparams* hp,
                          const zero_loss_scale_config* cfg, zero_loss_scale* ls_dev, double external_sumsq, void* ws,
                          size_t ws_bytes, void* host_ws, size_t host_ws_bytes, zero_result* res_host,
                          int32_t threads, hipStream_t stream);

/*
 * zero_offload_adamw_host -- the host half alone: AdamW on host fp32
 * master/exp_avg/exp_avg_sq (n each, in place) from the host fp32 gradient g
 * (multiplied by clip_coef in binary64), bf16 output into host param_out;
 * hp as for zero_adamw_step; threads as above. For a caller that moves the
 * gradient itself. Synchronous; launches nothing on the GPU.
 */
int zero_offload_adamw_host(float* master, float* exp_avg, float* exp_avg_sq, const float* g, void* param_out,
                            int64_t n, const zero_adamw_hparams* hp, double clip_coef, int32_t threads);

/*
 * zero_workspace_forget -- drop the host-side record that `ws` holds the
 * tensor table of an earlier zero_step, zero_step_amp, zero_bucket_reduce,
 * zero_step_accumulated or zero_offload_step call. Call it before freeing or
 * repurposing such a workspace; the next zero_step on it then rewrites the
 * table. (A workspace whose table was overwritten without this call is
 * detected on the device: zero_result.status = ZERO_ERR_STALE_WORKSPACE and
 * nothing is written.) Host only; launches nothing.
 */
int zero_workspace_forget(const void* ws);

/* Human-readable text of a status code (static storage). */
const char* zero_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_STEP_H */
