// zero_kernels.hip -- gfx950 kernels of the per-rank ZeRO shard step.
//
// The step ("CS336 Lecture 7: Parallelism 1", section "ZeRO Stage 1", steps
// 2-4): the M bf16 gradient replicas of this rank's shard are summed in fp32
// (the reduce-scatter arithmetic), unscaled, checked for inf/NaN and squared
// into the global norm; AdamW then updates the fp32 master, m and v of the
// shard (the 12 optimizer bytes of the table in section "训练内存的详细分析")
// and the new master is rounded to the bf16 shard an all-gather would send.
// The same tile loop serves the step's other forms: ZeRO-2 streaming (section
// "ZeRO Stage 2"; Mode::Acc folds each bucket into the caller's fp32 shard
// accumulator, its final pass emitting the bucket's norm partial, and
// Mode::PassB then updates from the accumulator), the CPU-offloaded step
// (the GPU's side of it: Mode::PassA, or, when neither clipping nor skipping
// has to wait for the norm, Mode::Acc over groups of tiles so that each
// group's copy to the host starts while the next folds) and the dynamic loss scale
// (the multiplier read from device memory, the scale moved by the fold's
// last workgroup).
//
// This is streaming, HBM-bound work with no contraction, so there is no MFMA
// here. Design points for CDNA4:
//  - Each thread owns runs of 8 consecutive elements, so every replica read
//    is one 16-byte load and a wave reads a contiguous 1 KiB per replica.
//  - The fused step launches one workgroup per tile (grid = tiles, in
//    order), with a tile geometry per pass (threads x 8-element vectors per
//    thread). Inside a tile the workgroup sweeps the replicas in lockstep, a
//    barrier after each, so the reads in flight on the chip stay within a
//    compact window of every replica (few open DRAM pages and TLB entries
//    with 64+ streams).
//  - The rank fold is a fixed ascending left fold in fp32; the sum of squares
//    uses exact binary64 squares, a per-thread binary64 accumulator, a fixed
//    wave butterfly and a fixed LDS order, and the per-workgroup partials are
//    combined in index order by the last workgroup to finish: bitwise
//    repeatable (atomics publish and count, they never add values).
//  - The composed entry points (reduce, check, AdamW) use grid-stride sweeps
//    of 2048-element tiles over a grid sized to the resident capacity.
//  - Replica reads and the bf16 emit use non-temporal accesses.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <utility>

#include "zero_internal.h"

namespace zero {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ helpers

// Every buffer of the step is device (global) memory, so the 16-byte accesses
// go through the global address space: global_* instructions with a scalar
// base, rather than flat accesses that also count against the LDS counter.
#define ZERO_GLOBAL __attribute__((address_space(1)))
#define ZERO_CONSTANT __attribute__((address_space(4)))

__device__ __forceinline__ u32x4 ld_nt(const uint16_t* p)
{
    return __builtin_nontemporal_load((const ZERO_GLOBAL u32x4*)p);
}
__device__ __forceinline__ f32x4 ld4(const float* p) { return *(const ZERO_GLOBAL f32x4*)p; }
__device__ __forceinline__ void st4(float* p, f32x4 v) { *(ZERO_GLOBAL f32x4*)p = v; }
__device__ __forceinline__ void st_nt(uint16_t* p, u32x4 v) { __builtin_nontemporal_store(v, (ZERO_GLOBAL u32x4*)p); }

// Base address of replica r from a plan's rank-pointer table in the
// workspace. The table is written before the launch and not modified during
// it, so it is read through the constant address space: a scalar load served
// by the scalar cache instead of a vector round trip in front of every
// replica sweep.
__device__ __forceinline__ const uint16_t* rank_ptr(const uint16_t* const* gp, int r)
{
    return reinterpret_cast<const uint16_t*>(((const ZERO_CONSTANT uint64_t*)gp)[r]);
}

// bf16 -> fp32 is exact: the code is the upper half of the binary32 encoding.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf1(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

__device__ __forceinline__ void set8(float (&s)[8], u32x4 w)
{
    s[0] = bf_lo(w.x); s[1] = bf_hi(w.x); s[2] = bf_lo(w.y); s[3] = bf_hi(w.y);
    s[4] = bf_lo(w.z); s[5] = bf_hi(w.z); s[6] = bf_lo(w.w); s[7] = bf_hi(w.w);
}
__device__ __forceinline__ void add8(float (&s)[8], u32x4 w)
{
    s[0] = s[0] + bf_lo(w.x); s[1] = s[1] + bf_hi(w.x); s[2] = s[2] + bf_lo(w.y); s[3] = s[3] + bf_hi(w.y);
    s[4] = s[4] + bf_lo(w.z); s[5] = s[5] + bf_hi(w.z); s[6] = s[6] + bf_lo(w.w); s[7] = s[7] + bf_hi(w.w);
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN with its sign.
__device__ __forceinline__ uint32_t bf16_rne(float x)
{
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t nonfinite(float x) { return (__float_as_uint(x) & 0x7F800000u) == 0x7F800000u; }

// Ascending left fold of the M replicas at elements [e0, e0+8). FROM0: start
// from rank 0's value; otherwise continue the fold from s.
template <int MT, bool FROM0>
__device__ __forceinline__ void fold_vec(const uint16_t* const* __restrict__ gp, int M, int64_t e0, float (&s)[8])
{
    constexpr int B = 8;  // loads issued before the adds that consume them
    const int Mr = MT > 0 ? MT : M;
    if constexpr (FROM0) set8(s, ld_nt(gp[0] + e0));
    auto batch = [&](int r0) {
        u32x4 buf[B];
#pragma unroll
        for (int j = 0; j < B; ++j)
            if (r0 + j < Mr) buf[j] = ld_nt(gp[r0 + j] + e0);
#pragma unroll
        for (int j = 0; j < B; ++j)
            if (r0 + j < Mr) add8(s, buf[j]);
    };
    if constexpr (MT > 0) {
#pragma unroll
        for (int r0 = FROM0 ? 1 : 0; r0 < MT; r0 += B) batch(r0);
    } else {
        for (int r0 = FROM0 ? 1 : 0; r0 < Mr; r0 += B) batch(r0);
    }
}

template <int MT, bool FROM0>
__device__ __forceinline__ float fold_one(const uint16_t* const* __restrict__ gp, int M, int64_t e, float s)
{
    const int Mr = MT > 0 ? MT : M;
    if constexpr (FROM0) s = bf1(gp[0][e]);
    for (int r = FROM0 ? 1 : 0; r < Mr; ++r) s = s + bf1(gp[r][e]);
    return s;
}

// One AdamW element: bias-corrected, eps outside the root, decay decoupled
// and scaled by lr. Evaluated in binary64 from the fp32 state and rounded
// once on store; every operation is a separate IEEE binary64 operation
// (no contraction), so the new state is what a binary64 evaluation of the
// formula gives, also where w*(1 - lr*wd) and the Adam step nearly cancel.
__device__ __forceinline__ void adam1(float g32, double coef, const AdamScalars& c, float& w, float& m, float& v)
{
    const double g = static_cast<double>(g32) * coef;
    const double mn = c.b1 * static_cast<double>(m) + c.omb1 * g;
    const double vn = c.b2 * static_cast<double>(v) + c.omb2 * g * g;
    const double m_hat = mn / c.bc1;
    const double v_hat = vn / c.bc2;
    const double wn = static_cast<double>(w) * c.decay - c.lr * m_hat / (sqrt(v_hat) + c.eps);
    m = static_cast<float>(mn);
    v = static_cast<float>(vn);
    w = static_cast<float>(wn);
}

// Per-workgroup reduction of (sum of squares, non-finite flag) in a fixed
// order: a wave butterfly, then the waves in index order. The result is valid
// in thread 0 only.
template <int NT = kThreads>
__device__ __forceinline__ void block_reduce(double& acc, uint32_t& bad)
{
    __shared__ double s_acc[NT / 64];
    __shared__ uint32_t s_bad[NT / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        acc += __shfl_xor(acc, off, 64);
        bad |= __shfl_xor(bad, off, 64);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        s_acc[wave] = acc;
        s_bad[wave] = bad;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        acc = s_acc[0];
        bad = s_bad[0];
#pragma unroll
        for (int w = 1; w < NT / 64; ++w) {
            acc += s_acc[w];
            bad |= s_bad[w];
        }
    }
}

// block_reduce, written to one partial record.
template <int NT = kThreads>
__device__ __forceinline__ void block_partial(double acc, uint32_t bad, Partial* __restrict__ out)
{
    block_reduce<NT>(acc, bad);
    if (threadIdx.x == 0) {
        Partial p;
        p.sumsq = acc;
        p.bad = bad;
        p.pad = 0;
        *out = p;
    }
}

// ------------------------------------------------------------------ last-workgroup finalize
//
// A fold pass ends with its last-arriving workgroup turning the per-workgroup
// partials into the result record, so a step needs no separate finalize
// launch. Each workgroup publishes its partial with agent-scope atomic
// exchanges and only then counts itself in with an agent-scope atomic add.
// An atomic read-modify-write returns its old value once it has been
// performed where the whole device sees it, and the add's operand is made to
// depend on both returned values, so no workgroup is counted before its
// partial is visible on every XCD. The workgroup that counts last reads the
// partials with agent-scope atomic loads, which do not take a stale line
// from its own XCD's L2. No release fence is used on purpose: on CDNA4 an
// agent-scope release writes back the whole L2 of the XCD, and making every
// workgroup wait for the write-back of the others' output lines cost 5-7% of
// a two-pass step.

// Zero, computed from x by an instruction the compiler cannot see through:
// whatever consumes the result is issued only after x has arrived.
__device__ __forceinline__ uint32_t zero_after(uint32_t x)
{
    uint32_t z;
    asm volatile("v_and_b32 %0, 0, %1" : "=v"(z) : "v"(x));
    return z;
}

// One thread: publish (sumsq, bad) as the partial at `slot`, then count the
// workgroup in; returns the counter's value before the add.
__device__ __forceinline__ unsigned publish_and_arrive(Partial* slot, double sumsq, uint32_t bad, unsigned* counter)
{
    const unsigned long long o1 = __hip_atomic_exchange(reinterpret_cast<unsigned long long*>(&slot->sumsq),
                                                        static_cast<unsigned long long>(__double_as_longlong(sumsq)),
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t o2 = __hip_atomic_exchange(&slot->bad, bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t dep = zero_after(static_cast<uint32_t>(o1) | static_cast<uint32_t>(o1 >> 32) | o2);
    return __hip_atomic_fetch_add(counter, 1u + dep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The published partials 0..n-1 combined in a fixed order (thread i takes i,
// i+NT, ...; then block_reduce); valid in thread 0.
template <int NT>
__device__ __forceinline__ void combine_published(Partial* parts, int64_t n, double& sumsq, uint32_t& bad)
{
    sumsq = 0.0;
    bad = 0;
    for (int64_t i = threadIdx.x; i < n; i += NT) {
        sumsq += __longlong_as_double(static_cast<long long>(__hip_atomic_load(
            reinterpret_cast<unsigned long long*>(&parts[i].sumsq), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
        bad |= __hip_atomic_load(&parts[i].bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    block_reduce<NT>(sumsq, bad);
}

// ------------------------------------------------------------------ tile body

enum class Op : int { Reduce, Check, Adam, Full, PassA, Acc };

// Pointers and layout of one shard, as seen by one tile.
struct Ctx {
    const uint16_t* const* gp;
    int M;
    float* master;
    float* m;
    float* v;
    uint16_t* out;
    float* gout;        // fp32 gradient written (Reduce, PassA, Acc)
    const float* gin;   // fp32 gradient read (Check, Adam, Acc; Reduce continuing a fold)
    int64_t n, nvec;
    int32_t head, tail;
};

struct Scal {
    float gscale;     // multiplier of the fp32 sum (Reduce: applied when `last`); Adam: of the stored g
    double coef;      // clip coefficient (Adam, Full)
    bool last;        // Reduce: this pass ends the fold
    bool accumulate;  // Acc: add the fold to the accumulator (else store it)
    bool final;       // Acc: also check and square g = acc * gscale
    bool stream;      // 16-vector Full and PassA, Adam: whole-line stores stream past the caches
};

// One element, scalar path. PREADD (Full only): when k.accumulate, the fold
// is added to the caller's accumulator x.gin before the scale (the final
// micro-batch of a ZeRO-2 bucket, updated in the same pass).
template <Op OP, int MT, bool FROM0, bool PREADD = false>
__device__ __forceinline__ void do_one(const Ctx& x, const Scal& k, const AdamScalars& c, int64_t e, double& acc,
                                       uint32_t& bad)
{
    float g;
    if constexpr (OP == Op::Reduce) {
        g = fold_one<MT, FROM0>(x.gp, x.M, e, FROM0 ? 0.0f : x.gin[e]);
        if (k.last) g = g * k.gscale;
        x.gout[e] = g;
        return;
    }
    if constexpr (OP == Op::Acc) {
        float a = fold_one<MT, true>(x.gp, x.M, e, 0.0f);
        if (k.accumulate) a = x.gin[e] + a;
        x.gout[e] = a;
        if (k.final) {
            g = a * k.gscale;
            bad |= nonfinite(g);
            const double d = static_cast<double>(g);
            acc = fma(d, d, acc);
        }
        return;
    }
    if constexpr (OP == Op::Full && PREADD) {
        float a = fold_one<MT, true>(x.gp, x.M, e, 0.0f);
        if (k.accumulate) a = x.gin[e] + a;
        g = a * k.gscale;
    } else if constexpr (OP == Op::Full || OP == Op::PassA) {
        g = fold_one<MT, true>(x.gp, x.M, e, 0.0f) * k.gscale;
    }
    if constexpr (OP == Op::Check) g = x.gin[e];
    if constexpr (OP == Op::Adam) g = x.gin[e] * k.gscale;
    if constexpr (OP != Op::Adam) {
        bad |= nonfinite(g);
        const double d = static_cast<double>(g);
        acc = fma(d, d, acc);
    }
    if constexpr (OP == Op::PassA) x.gout[e] = g;
    if constexpr (OP == Op::Full || OP == Op::Adam) {
        float w = x.master[e], m = x.m[e], v = x.v[e];
        adam1(g, k.coef, c, w, m, v);
        x.master[e] = w;
        x.m[e] = m;
        x.v[e] = v;
        x.out[e] = static_cast<uint16_t>(bf16_rne(w));
    }
}

// The fp32 master, exp_avg and exp_avg_sq of elements [e0, e0+8).
struct State8 {
    f32x4 w0, w1, m0, m1, v0, v1;
};

__device__ __forceinline__ State8 load_state8(const Ctx& x, int64_t e0)
{
    State8 q;
    q.w0 = ld4(x.master + e0);
    q.w1 = ld4(x.master + e0 + 4);
    q.m0 = ld4(x.m + e0);
    q.m1 = ld4(x.m + e0 + 4);
    q.v0 = ld4(x.v + e0);
    q.v1 = ld4(x.v + e0 + 4);
    return q;
}

// AdamW + bf16 emit of elements [e0, e0+8) from their gradient g and their
// state q as loaded.
__device__ __forceinline__ void adam8_from(const Ctx& x, const Scal& k, const AdamScalars& c, int64_t e0,
                                           const float (&g)[8], const State8& q)
{
    float w[8] = {q.w0.x, q.w0.y, q.w0.z, q.w0.w, q.w1.x, q.w1.y, q.w1.z, q.w1.w};
    float m[8] = {q.m0.x, q.m0.y, q.m0.z, q.m0.w, q.m1.x, q.m1.y, q.m1.z, q.m1.w};
    float v[8] = {q.v0.x, q.v0.y, q.v0.z, q.v0.w, q.v1.x, q.v1.y, q.v1.z, q.v1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) adam1(g[j], k.coef, c, w[j], m[j], v[j]);
    st4(x.master + e0, f32x4{w[0], w[1], w[2], w[3]});
    st4(x.master + e0 + 4, f32x4{w[4], w[5], w[6], w[7]});
    st4(x.m + e0, f32x4{m[0], m[1], m[2], m[3]});
    st4(x.m + e0 + 4, f32x4{m[4], m[5], m[6], m[7]});
    st4(x.v + e0, f32x4{v[0], v[1], v[2], v[3]});
    st4(x.v + e0 + 4, f32x4{v[4], v[5], v[6], v[7]});
    u32x4 o;
    o.x = bf16_rne(w[0]) | (bf16_rne(w[1]) << 16);
    o.y = bf16_rne(w[2]) | (bf16_rne(w[3]) << 16);
    o.z = bf16_rne(w[4]) | (bf16_rne(w[5]) << 16);
    o.w = bf16_rne(w[6]) | (bf16_rne(w[7]) << 16);
    st_nt(x.out + e0, o);
}

// AdamW + bf16 emit of elements [e0, e0+8) from their gradient g.
__device__ __forceinline__ void adam8(const Ctx& x, const Scal& k, const AdamScalars& c, int64_t e0,
                                      const float (&g)[8])
{
    adam8_from(x, k, c, e0, g, load_state8(x, e0));
}

// ------------------------------------------------------------------ whole-line state I/O
//
// The paired update of the 16-vector geometries, the update pass and the
// first pass's gradient stores work on half vectors: lane l of a wave takes
// elements 4l..4l+3 (half A) and 256+4l..256+4l+3 (half B) of the wave's
// 512-element block, so that each fp32 load or store instruction of the wave
// covers 1 KiB of whole 128-byte lines (with 8 consecutive elements per lane,
// two instructions each write half of every line).

// Store 16 bytes at byte offset `off` of the 512-element fp32 block that
// starts at `blk` (the same address in every lane of the wave), as a buffer
// store whose range is that block. STREAM: with the non-temporal and
// system-scope cache-policy bits (nt, sc1), so that the lines go out to
// memory in the order they are written instead of waiting, dirty, in the
// caches; otherwise a plain store.
template <bool STREAM>
__device__ __forceinline__ void st_line(float* blk, uint32_t off, f32x4 v)
{
    // word 3 of the resource (0x00020000): a raw, unformatted gfx9 buffer
    constexpr int kNt = 2, kSc1 = 16;  // CDNA3/CDNA4 buffer cache-policy bits
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(static_cast<void*>(blk), 0, 2048, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, static_cast<int>(off), 0,
                                           STREAM ? (kNt | kSc1) : 0);
}

__device__ __forceinline__ void st_nt2(uint16_t* p, u32x2 v) { __builtin_nontemporal_store(v, (ZERO_GLOBAL u32x2*)p); }

// The state of the lane's two halves of the block at element `blk` (uniform
// over the wave); a half that is not valid reads the block's first element.
__device__ __forceinline__ State8 load_halves(const Ctx& x, int64_t blk, int lane, bool oa, bool ob)
{
    const int64_t a = oa ? blk + 4 * lane : blk, b = ob ? blk + 256 + 4 * lane : blk;
    State8 q;
    q.w0 = ld4(x.master + a);
    q.w1 = ld4(x.master + b);
    q.m0 = ld4(x.m + a);
    q.m1 = ld4(x.m + b);
    q.v0 = ld4(x.v + a);
    q.v1 = ld4(x.v + b);
    return q;
}

// The lane's 4-element half at byte offset `off` of the block at `blk`, as
// four fp32 stores of master, m and v and the bf16 output.
template <bool STREAM>
__device__ __forceinline__ void store_half(const Ctx& x, int64_t blk, uint32_t off, const float* w, const float* m,
                                           const float* v)
{
    st_line<STREAM>(x.master + blk, off, f32x4{w[0], w[1], w[2], w[3]});
    st_line<STREAM>(x.m + blk, off, f32x4{m[0], m[1], m[2], m[3]});
    st_line<STREAM>(x.v + blk, off, f32x4{v[0], v[1], v[2], v[3]});
    st_nt2(x.out + blk + off / 4u,
           u32x2{bf16_rne(w[0]) | (bf16_rne(w[1]) << 16), bf16_rne(w[2]) | (bf16_rne(w[3]) << 16)});
}

// AdamW + bf16 emit of the lane's two halves (g[0..3]: half A, g[4..7]: half
// B) from their state q; a half is stored only when valid.
__device__ __forceinline__ void adam_halves(const Ctx& x, const Scal& k, const AdamScalars& c, int64_t blk, int lane,
                                            bool oa, bool ob, const float (&g)[8], const State8& q)
{
    float w[8] = {q.w0.x, q.w0.y, q.w0.z, q.w0.w, q.w1.x, q.w1.y, q.w1.z, q.w1.w};
    float m[8] = {q.m0.x, q.m0.y, q.m0.z, q.m0.w, q.m1.x, q.m1.y, q.m1.z, q.m1.w};
    float v[8] = {q.v0.x, q.v0.y, q.v0.z, q.v0.w, q.v1.x, q.v1.y, q.v1.z, q.v1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) adam1(g[j], k.coef, c, w[j], m[j], v[j]);
    const uint32_t off = 16u * static_cast<uint32_t>(lane);
    if (k.stream) {
        if (oa) store_half<true>(x, blk, off, w, m, v);
        if (ob) store_half<true>(x, blk, off + 1024u, w + 4, m + 4, v + 4);
    } else {
        if (oa) store_half<false>(x, blk, off, w, m, v);
        if (ob) store_half<false>(x, blk, off + 1024u, w + 4, m + 4, v + 4);
    }
}

// Eight elements [e0, e0+8), 16-byte vector path.
template <Op OP, int MT, bool FROM0>
__device__ __forceinline__ void do_vec(const Ctx& x, const Scal& k, const AdamScalars& c, int64_t e0, double& acc,
                                       uint32_t& bad)
{
    float g[8];
    if constexpr (OP == Op::Reduce) {
        if constexpr (!FROM0) {
            const f32x4 a = ld4(x.gin + e0), b = ld4(x.gin + e0 + 4);
            g[0] = a.x; g[1] = a.y; g[2] = a.z; g[3] = a.w; g[4] = b.x; g[5] = b.y; g[6] = b.z; g[7] = b.w;
        }
        fold_vec<MT, FROM0>(x.gp, x.M, e0, g);
        if (k.last) {
#pragma unroll
            for (int j = 0; j < 8; ++j) g[j] = g[j] * k.gscale;
        }
        st4(x.gout + e0, f32x4{g[0], g[1], g[2], g[3]});
        st4(x.gout + e0 + 4, f32x4{g[4], g[5], g[6], g[7]});
        return;
    }
    if constexpr (OP == Op::Full || OP == Op::PassA) {
        fold_vec<MT, true>(x.gp, x.M, e0, g);
#pragma unroll
        for (int j = 0; j < 8; ++j) g[j] = g[j] * k.gscale;
    }
    if constexpr (OP == Op::Check || OP == Op::Adam) {
        const f32x4 a = ld4(x.gin + e0), b = ld4(x.gin + e0 + 4);
        g[0] = a.x; g[1] = a.y; g[2] = a.z; g[3] = a.w; g[4] = b.x; g[5] = b.y; g[6] = b.z; g[7] = b.w;
    }
    if constexpr (OP == Op::Adam) {
#pragma unroll
        for (int j = 0; j < 8; ++j) g[j] = g[j] * k.gscale;
    }
    if constexpr (OP != Op::Adam) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            bad |= nonfinite(g[j]);
            const double d = static_cast<double>(g[j]);
            acc = fma(d, d, acc);
        }
    }
    if constexpr (OP == Op::PassA) {
        st4(x.gout + e0, f32x4{g[0], g[1], g[2], g[3]});
        st4(x.gout + e0 + 4, f32x4{g[4], g[5], g[6], g[7]});
    }
    if constexpr (OP == Op::Full || OP == Op::Adam) adam8(x, k, c, e0, g);
}

// Tile `t` of one shard.
template <Op OP, int MT, bool FROM0>
__device__ __forceinline__ void do_tile(const Ctx& x, const Scal& k, const AdamScalars& c, int64_t t, double& acc,
                                        uint32_t& bad)
{
    const int tid = threadIdx.x;
    if (x.nvec >= 0) {
        const int64_t v = t * kThreads + tid;
        if (v < x.nvec) do_vec<OP, MT, FROM0>(x, k, c, x.head + v * kVec, acc, bad);
        if (t == 0 && tid < x.head) do_one<OP, MT, FROM0>(x, k, c, tid, acc, bad);
        const int64_t last = x.nvec > 0 ? (x.nvec - 1) / kThreads : 0;
        if (t == last && tid < x.tail) do_one<OP, MT, FROM0>(x, k, c, x.head + x.nvec * kVec + tid, acc, bad);
    } else {
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            const int64_t e = t * kTileElems + j * kThreads + tid;
            if (e < x.n) do_one<OP, MT, FROM0>(x, k, c, e, acc, bad);
        }
    }
}

// Tile `t` of one shard in the fused kernels' geometry (NT threads, U
// vectors per thread). The fold sweeps the replicas in ascending rank order
// with a workgroup barrier after each replica, so the workgroup requests
// NT*U*16 contiguous bytes of one replica together: long runs per DRAM page
// with 64+ concurrent replica streams.
template <Op OP, int NT, int U, bool PREADD = false>
__device__ __forceinline__ void big_tile(const Ctx& x, const Scal& k, const AdamScalars& c, int64_t t, double& acc,
                                         uint32_t& bad)
{
    const int tid = threadIdx.x;
    constexpr int64_t kTileVecs = static_cast<int64_t>(NT) * U;
    if (x.nvec < 0) {  // scalar layout: element by element
        const int64_t base = t * kTileVecs * kVec;
        for (int j = 0; j < U * kVec; ++j) {
            const int64_t e = base + static_cast<int64_t>(j) * NT + tid;
            if (e < x.n) do_one<OP, 0, true, PREADD>(x, k, c, e, acc, bad);
        }
        return;
    }
    const int lane = tid & 63, wave = tid >> 6;
    const int64_t v0 = t * kTileVecs + static_cast<int64_t>(wave) * 64 * U + lane;
    if constexpr (OP == Op::Full || OP == Op::PassA || OP == Op::Acc) {
        bool ok[U];
        float s[U][8];
        const uint16_t* p0 = rank_ptr(x.gp, 0) + x.head;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            ok[u] = v0 + u * 64 < x.nvec;
            if (ok[u]) {
                set8(s[u], ld_nt(p0 + (v0 + u * 64) * kVec));
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) s[u][j] = 0.0f;
            }
        }
        __syncthreads();
#pragma unroll 1
        for (int r = 1; r < x.M; ++r) {
            const uint16_t* p = rank_ptr(x.gp, r) + x.head;
            u32x4 w[U];
#pragma unroll
            for (int u = 0; u < U; ++u) w[u] = ok[u] ? ld_nt(p + (v0 + u * 64) * kVec) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int u = 0; u < U; ++u) add8(s[u], w[u]);
            __syncthreads();
        }
        if constexpr (PREADD) {
            // the final micro-batch of a ZeRO-2 bucket: acc + fold, one
            // binary32 add per element, before the scale; four vectors'
            // accumulator loads in flight at a time
            if (k.accumulate) {
#pragma unroll
                for (int u0 = 0; u0 < U; u0 += 4) {
                    f32x4 a[4][2];
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        if (u0 + h < U && ok[u0 + h]) {
                            const int64_t e0 = x.head + (v0 + (u0 + h) * 64) * kVec;
                            a[h][0] = ld4(x.gin + e0);
                            a[h][1] = ld4(x.gin + e0 + 4);
                        }
                    }
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        if (u0 + h < U && ok[u0 + h]) {
                            float (&q)[8] = s[u0 + h];
                            q[0] = a[h][0].x + q[0]; q[1] = a[h][0].y + q[1]; q[2] = a[h][0].z + q[2]; q[3] = a[h][0].w + q[3];
                            q[4] = a[h][1].x + q[4]; q[5] = a[h][1].y + q[5]; q[6] = a[h][1].z + q[6]; q[7] = a[h][1].w + q[7];
                        }
                    }
                }
            }
        }
        bool paired = false;
        if constexpr (OP == Op::Full && U == 16) {
            // The update in pairs of vectors, on half vectors (whole-line
            // state I/O above): the fold's sums are first moved across lanes
            // so that lane l holds elements 4l..4l+3 and 256+4l..256+4l+3 of
            // each of its wave's 512-element blocks; both vectors' state is
            // loaded, then both are updated, which halves the dependent round
            // trips of the update. A half past the shard's last vector loads
            // the block's first element and stores nothing, so the loads take
            // no per-lane branch; the scheduling barriers keep each pair's
            // loads together, ahead of its arithmetic. (The 1024-thread
            // geometries run four waves per SIMD, within 128 registers, where
            // a second state does not fit.)
            paired = x.nvec > 0;
            if (paired) {
                const int64_t vb = t * kTileVecs + static_cast<int64_t>(__builtin_amdgcn_readfirstlane(wave)) * 64 * U;
                const int srcA = lane >> 1, srcB = 32 + (lane >> 1);
                const bool odd = (lane & 1) != 0;
#pragma unroll
                for (int u = 0; u < U; u += 2) {
                    bool oa[2], ob[2];
                    int64_t blk[2];
                    State8 q[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int64_t vv = vb + (u + h) * 64;  // the block's first vector
                        oa[h] = vv + (lane >> 1) < x.nvec;
                        ob[h] = vv + 32 + (lane >> 1) < x.nvec;
                        blk[h] = x.head + (vv < x.nvec ? vv : 0) * kVec;
                        q[h] = load_halves(x, blk[h], lane, oa[h], ob[h]);
                    }
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        // element 4l+j of the block sits in lane l/2, slot
                        // 4(l%2)+j; element 256+4l+j in lane 32+l/2
                        float nw[8];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float a0 = __shfl(s[u + h][j], srcA, 64), a1 = __shfl(s[u + h][4 + j], srcA, 64);
                            const float b0 = __shfl(s[u + h][j], srcB, 64), b1 = __shfl(s[u + h][4 + j], srcB, 64);
                            nw[j] = odd ? a1 : a0;
                            nw[4 + j] = odd ? b1 : b0;
                        }
#pragma unroll
                        for (int j = 0; j < 8; ++j) s[u + h][j] = nw[j];
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        if (oa[h] || ob[h]) {
                            float g[8];
#pragma unroll
                            for (int j = 0; j < 8; ++j) g[j] = s[u + h][j] * k.gscale;
                            if (oa[h]) {
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    bad |= nonfinite(g[j]);
                                    const double d = static_cast<double>(g[j]);
                                    acc = fma(d, d, acc);
                                }
                            }
                            if (ob[h]) {
#pragma unroll
                                for (int j = 4; j < 8; ++j) {
                                    bad |= nonfinite(g[j]);
                                    const double d = static_cast<double>(g[j]);
                                    acc = fma(d, d, acc);
                                }
                            }
                            adam_halves(x, k, c, blk[h], lane, oa[h], ob[h], g, q[h]);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        }
        if constexpr (OP == Op::PassA && U == 16) {
            // the first pass of a two-pass step stores its fp32 gradient on
            // half vectors too: whole lines, streamed as the state stores are
            if (x.nvec > 0) {
                const int64_t vb = t * kTileVecs + static_cast<int64_t>(__builtin_amdgcn_readfirstlane(wave)) * 64 * U;
                const int srcA = lane >> 1, srcB = 32 + (lane >> 1);
                const bool odd = (lane & 1) != 0;
                const uint32_t off = 16u * static_cast<uint32_t>(lane);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t vv = vb + u * 64;  // the block's first vector
                    const bool oa = vv + (lane >> 1) < x.nvec, ob = vv + 32 + (lane >> 1) < x.nvec;
                    const int64_t blk = x.head + (vv < x.nvec ? vv : 0) * kVec;
                    float g[8];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float a0 = __shfl(s[u][j], srcA, 64), a1 = __shfl(s[u][4 + j], srcA, 64);
                        const float b0 = __shfl(s[u][j], srcB, 64), b1 = __shfl(s[u][4 + j], srcB, 64);
                        g[j] = (odd ? a1 : a0) * k.gscale;
                        g[4 + j] = (odd ? b1 : b0) * k.gscale;
                    }
                    if (oa) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            bad |= nonfinite(g[j]);
                            const double d = static_cast<double>(g[j]);
                            acc = fma(d, d, acc);
                        }
                        const f32x4 ga = {g[0], g[1], g[2], g[3]};
                        if (k.stream) st_line<true>(x.gout + blk, off, ga); else st_line<false>(x.gout + blk, off, ga);
                    }
                    if (ob) {
#pragma unroll
                        for (int j = 4; j < 8; ++j) {
                            bad |= nonfinite(g[j]);
                            const double d = static_cast<double>(g[j]);
                            acc = fma(d, d, acc);
                        }
                        const f32x4 gb = {g[4], g[5], g[6], g[7]};
                        if (k.stream) st_line<true>(x.gout + blk, off + 1024u, gb);
                        else st_line<false>(x.gout + blk, off + 1024u, gb);
                    }
                }
            }
        }
        // Every other pass and geometry takes the per-vector loop (in the
        // paired kernels a tile with no whole vector has only its scalar head
        // and tail to do).
        if (!(OP == Op::Full && U == 16) && !(OP == Op::PassA && U == 16) && !paired) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (!ok[u]) continue;
                const int64_t e0 = x.head + (v0 + u * 64) * kVec;
                if constexpr (OP == Op::Acc) {
                    // the running sum of the reduce-scatter results: acc + fold
                    float a[8];
                    if (k.accumulate) {
                        const f32x4 p = ld4(x.gin + e0), q = ld4(x.gin + e0 + 4);
                        a[0] = p.x + s[u][0]; a[1] = p.y + s[u][1]; a[2] = p.z + s[u][2]; a[3] = p.w + s[u][3];
                        a[4] = q.x + s[u][4]; a[5] = q.y + s[u][5]; a[6] = q.z + s[u][6]; a[7] = q.w + s[u][7];
                    } else {
#pragma unroll
                        for (int j = 0; j < 8; ++j) a[j] = s[u][j];
                    }
                    st4(x.gout + e0, f32x4{a[0], a[1], a[2], a[3]});
                    st4(x.gout + e0 + 4, f32x4{a[4], a[5], a[6], a[7]});
                    if (k.final) {
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const float g = a[j] * k.gscale;
                            bad |= nonfinite(g);
                            const double d = static_cast<double>(g);
                            acc = fma(d, d, acc);
                        }
                    }
                    continue;
                }
                float g[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    g[j] = s[u][j] * k.gscale;
                    bad |= nonfinite(g[j]);
                    const double d = static_cast<double>(g[j]);
                    acc = fma(d, d, acc);
                }
                if constexpr (OP == Op::PassA) {
                    st4(x.gout + e0, f32x4{g[0], g[1], g[2], g[3]});
                    st4(x.gout + e0 + 4, f32x4{g[4], g[5], g[6], g[7]});
                } else {
                    adam8(x, k, c, e0, g);
                }
            }
        }
    } else {
        static_assert(OP == Op::Adam, "fused tiles fold, or update from the stored gradient");
        // on half vectors, like the paired update: whole-line state I/O
        const int64_t vw = t * kTileVecs + static_cast<int64_t>(__builtin_amdgcn_readfirstlane(wave)) * 64 * U;
#pragma unroll 1
        for (int u = 0; u < U; ++u) {
            const int64_t vv = vw + u * 64;  // the block's first vector
            if (vv >= x.nvec) break;
            const bool oa = vv + (lane >> 1) < x.nvec, ob = vv + 32 + (lane >> 1) < x.nvec;
            const int64_t blk = x.head + vv * kVec;
            const f32x4 a = ld4(x.gin + (oa ? blk + 4 * lane : blk)), b = ld4(x.gin + (ob ? blk + 256 + 4 * lane : blk));
            const State8 q = load_halves(x, blk, lane, oa, ob);
            const float g[8] = {a.x * k.gscale, a.y * k.gscale, a.z * k.gscale, a.w * k.gscale,
                                b.x * k.gscale, b.y * k.gscale, b.z * k.gscale, b.w * k.gscale};
            adam_halves(x, k, c, blk, lane, oa, ob, g, q);
        }
    }
    if (t == 0 && tid < x.head) do_one<OP, 0, true, PREADD>(x, k, c, tid, acc, bad);
    const int64_t last = x.nvec > 0 ? (x.nvec - 1) / kTileVecs : 0;
    if (t == last && tid < x.tail) do_one<OP, 0, true, PREADD>(x, k, c, x.head + x.nvec * kVec + tid, acc, bad);
}

__device__ __forceinline__ Ctx ctx_of(const TensorDesc& d, int M)
{
    Ctx x;
    x.gp = d.grads;
    x.M = M;
    x.master = d.master;
    x.m = d.exp_avg;
    x.v = d.exp_avg_sq;
    x.out = d.out;
    x.gout = d.gbuf;
    x.gin = d.gbuf;
    x.n = d.n;
    x.nvec = d.nvec;
    x.head = d.head;
    x.tail = d.tail;
    return x;
}

__device__ __forceinline__ Ctx ctx_flat(const Layout& L)
{
    Ctx x = {};
    x.n = L.n;
    x.nvec = L.nvec;
    x.head = L.head;
    x.tail = L.tail;
    return x;
}

// ------------------------------------------------------------------ kernels

template <int MT, bool FROM0>
__global__ __launch_bounds__(kThreads) void reduce_kernel(RankPtrs ptrs, int Mc, int last, float scale, Layout L,
                                                          float* __restrict__ g_out)
{
    Ctx x = ctx_flat(L);
    x.gp = ptrs.p;
    x.M = Mc;
    x.gout = g_out;
    x.gin = g_out;
    const Scal k{scale, 1.0, last != 0, false, false};
    const AdamScalars c{};
    double acc = 0.0;
    uint32_t bad = 0;
    const int64_t tiles = layout_tiles(L);
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) do_tile<Op::Reduce, MT, FROM0>(x, k, c, t, acc, bad);
}

__global__ __launch_bounds__(kThreads) void check_kernel(const float* __restrict__ g, Layout L,
                                                         Partial* __restrict__ parts)
{
    Ctx x = ctx_flat(L);
    x.gin = g;
    const Scal k{1.0f, 1.0, false, false, false};
    const AdamScalars c{};
    double acc = 0.0;
    uint32_t bad = 0;
    const int64_t tiles = layout_tiles(L);
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) do_tile<Op::Check, 1, true>(x, k, c, t, acc, bad);
    block_partial(acc, bad, parts + blockIdx.x);
}

__global__ __launch_bounds__(kThreads) void adamw_kernel(float* __restrict__ master, float* __restrict__ m,
                                                         float* __restrict__ v, const float* __restrict__ g,
                                                         uint16_t* __restrict__ out, Layout L, AdamScalars c,
                                                         const zero_result* __restrict__ res)
{
    double coef = 1.0;
    if (res != nullptr) {
        if (res->skipped != 0 || res->status != 0) return;
        coef = res->clip_coef;
    }
    Ctx x = ctx_flat(L);
    x.master = master;
    x.m = m;
    x.v = v;
    x.out = out;
    x.gin = g;
    const Scal k{1.0f, coef, false, false, false};
    double acc = 0.0;
    uint32_t bad = 0;
    const int64_t tiles = layout_tiles(L);
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) do_tile<Op::Adam, 1, true>(x, k, c, t, acc, bad);
}

// The result record from the combined partials: norm, clip coefficient,
// skip decision (clip rule: min(1, max/(norm + 1e-6)); NaN propagates).
__device__ __forceinline__ zero_result make_record(double sumsq, uint32_t bad, double external, double max_norm,
                                                   int skip)
{
    const double total = sumsq + external;
    const double norm = sqrt(total);
    double coef = 1.0;
    if (max_norm > 0.0) {
        coef = max_norm / (norm + 1e-6);
        if (coef > 1.0) coef = 1.0;
    }
    zero_result r;
    r.sumsq = total;
    r.clip_coef = coef;
    r.grad_norm = static_cast<float>(norm);
    r.found_inf = bad != 0 ? 1 : 0;
    r.skipped = (bad != 0 && skip != 0) ? 1 : 0;
    r.status = ZERO_OK;
    return r;
}

__device__ __forceinline__ zero_bucket_partial bucket_partial(double sumsq, uint32_t bad, uint64_t stamp, float scale)
{
    zero_bucket_partial p;
    p.sumsq = sumsq;
    p.stamp = stamp;
    p.found_inf = bad != 0 ? 1 : 0;
    p.grad_scale = scale;
    p.reserved = 0;
    return p;
}

__device__ __forceinline__ zero_result error_record(int32_t status)
{
    zero_result r;
    r.sumsq = __builtin_nan("");
    r.clip_coef = __builtin_nan("");
    r.grad_norm = __builtin_nanf("");
    r.found_inf = 0;
    r.skipped = 1;
    r.status = status;
    return r;
}

__device__ __forceinline__ zero_result stale_record() { return error_record(ZERO_ERR_STALE_WORKSPACE); }

// One move of the dynamic loss scale on a step's overflow flag (the rule is
// stated with zero_loss_scale in zero_step.h: hysteresis-th overflow in a row
// halves S down to min_scale, window-th clean step in a row doubles it while
// 2S is finite). 1/S is formed in binary64 and rounded once, which equals the
// correctly rounded binary32 quotient (53 >= 2*24 + 2).
__device__ __forceinline__ void loss_scale_move(const zero_loss_scale_config& c, bool overflow,
                                                zero_loss_scale* __restrict__ p)
{
    zero_loss_scale s = *p;
    if (overflow) {
        s.good_steps = 0;
        s.overflows += 1;
        if (s.overflows >= c.hysteresis) {
            const float half = s.scale / 2.0f;
            s.scale = half < c.min_scale ? c.min_scale : half;
            s.overflows = 0;
        }
    } else {
        s.overflows = 0;
        s.good_steps += 1;
        if (s.good_steps >= c.window) {
            const float twice = s.scale * 2.0f;
            if (__builtin_isfinite(twice)) s.scale = twice;
            s.good_steps = 0;
        }
    }
    s.inv_scale = static_cast<float>(1.0 / static_cast<double>(s.scale));
    *p = s;
}

// Partials 0..n-1 written by an earlier launch, combined in the same fixed
// order as combine_published; valid in thread 0.
template <int NT>
__device__ __forceinline__ void combine_partials(const Partial* __restrict__ parts, int64_t n, double& sumsq,
                                                 uint32_t& bad)
{
    sumsq = 0.0;
    bad = 0;
    for (int64_t i = threadIdx.x; i < n; i += NT) {
        sumsq += parts[i].sumsq;
        bad |= parts[i].bad;
    }
    block_reduce<NT>(sumsq, bad);
}

// One workgroup per tile (grid = tiles): the workgroups in flight cover a
// compact window of the buffers that advances as the dispatcher hands out
// tiles in order, and the partial of tile t is written to parts[t] whatever
// the order in which tiles run.
template <Mode MODE, int NT, int U>
__global__ __launch_bounds__(NT) void fused_kernel(const PlanHeader* __restrict__ hdr,
                                                   const TensorDesc* __restrict__ desc,
                                                   const TileRef* __restrict__ map, uint64_t sig, int M, float gscale,
                                                   AdamScalars c, Partial* __restrict__ parts, FinalizeArgs fin,
                                                   const zero_result* __restrict__ res)
{
    if (hdr->signature != sig) {  // the workspace no longer holds this plan: write nothing but the record
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            if constexpr (MODE == Mode::Acc || MODE == Mode::BucketFull) {
                if (fin.slot != nullptr) *fin.slot = bucket_partial(0.0, 0, ~fin.stamp, gscale);
            } else if constexpr (MODE != Mode::PassB) {
                *fin.res = stale_record();
            }
        }
        return;
    }
    double coef = 1.0;
    if constexpr (MODE == Mode::PassB) {
        if (res->skipped != 0 || res->status != 0) return;
        coef = res->clip_coef;
    }
    if (fin.scale_from != nullptr) gscale = gscale * fin.scale_from->inv_scale;  // AMP: the scale of this step
    constexpr Op OP = MODE == Mode::Full || MODE == Mode::BucketFull ? Op::Full
                      : MODE == Mode::PassA                          ? Op::PassA
                      : MODE == Mode::Acc                            ? Op::Acc
                                                                     : Op::Adam;
    const Scal k{gscale, coef, false, fin.accumulate != 0, fin.final != 0, fin.stream != 0};
    double acc = 0.0;
    uint32_t bad = 0;
    const TileRef tr = map[blockIdx.x];
    const Ctx x = ctx_of(desc[tr.tensor], M);
    big_tile<OP, NT, U, MODE == Mode::BucketFull>(x, k, c, tr.local, acc, bad);
    if constexpr (MODE == Mode::Acc) {
        if (!k.final) return;  // uniform over the launch
    }
    if constexpr (MODE != Mode::PassB) {
        // the last workgroup to arrive writes the record (the bucket partial
        // when accumulating) and re-arms the counter for the next launch
        block_reduce<NT>(acc, bad);
        __shared__ int s_last;
        if (threadIdx.x == 0) s_last = publish_and_arrive(parts + blockIdx.x, acc, bad, fin.counter) == gridDim.x - 1;
        __syncthreads();
        if (s_last) {
            double sumsq;
            uint32_t nbad;
            combine_published<NT>(parts, gridDim.x, sumsq, nbad);
            if (threadIdx.x == 0) {
                if constexpr (MODE == Mode::Acc || MODE == Mode::BucketFull) {
                    *fin.slot = bucket_partial(sumsq, nbad, fin.stamp, gscale);
                } else {
                    *fin.res = make_record(sumsq, nbad, fin.external, fin.max_norm, fin.skip);
                    // every other workgroup has arrived, so none still reads inv_scale
                    if (fin.ls != nullptr) loss_scale_move(fin.lscfg, nbad != 0, fin.ls);
                }
                __hip_atomic_store(fin.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// One workgroup: combine the partials in index order, then the norm, the
// clip coefficient and the skip decision.
__global__ __launch_bounds__(kThreads) void finalize_kernel(const Partial* __restrict__ parts, int64_t nparts,
                                                            double external, double max_norm, int skip,
                                                            zero_result* __restrict__ res)
{
    double sumsq;
    uint32_t bad;
    combine_partials<kThreads>(parts, nparts, sumsq, bad);
    if (threadIdx.x == 0) *res = make_record(sumsq, bad, external, max_norm, skip);
}

// One workgroup: the bucket partials of a ZeRO-2 step in index order (the
// same fixed tree as combine_partials), each checked against the step's
// stamp and fp32 scale, then the norm, clip coefficient and skip decision.
// hdr (null when the step has no elements) is the plan of the update pass
// that follows: a stale one is reported here, before that pass skips.
__global__ __launch_bounds__(kThreads) void bucket_finalize_kernel(const PlanHeader* __restrict__ hdr, uint64_t sig,
                                                                   const zero_bucket_partial* __restrict__ parts,
                                                                   int32_t nb, uint64_t stamp, float scale,
                                                                   const zero_loss_scale* __restrict__ ls,
                                                                   double external, double max_norm, int skip,
                                                                   zero_result* __restrict__ res)
{
    if (ls != nullptr) scale = scale * ls->inv_scale;  // AMP: the multiplier the buckets were squared with
    if (hdr != nullptr && hdr->signature != sig) {
        if (threadIdx.x == 0) *res = stale_record();
        return;
    }
    double sumsq = 0.0;
    uint32_t flags = 0;  // bit 0: a non-finite gradient; bit 1: a partial of another step or scale
    for (int32_t i = threadIdx.x; i < nb; i += kThreads) {
        const zero_bucket_partial p = parts[i];
        sumsq += p.sumsq;
        flags |= p.found_inf != 0 ? 1u : 0u;
        flags |= (p.stamp != stamp || __float_as_uint(p.grad_scale) != __float_as_uint(scale)) ? 2u : 0u;
    }
    block_reduce<kThreads>(sumsq, flags);
    if (threadIdx.x == 0)
        *res = (flags & 2u) ? error_record(ZERO_ERR_BUCKET_PARTIALS)
                            : make_record(sumsq, flags & 1u, external, max_norm, skip);
}

__global__ void bucket_partial_empty_kernel(zero_bucket_partial* __restrict__ slot, uint64_t stamp, float scale,
                                            const zero_loss_scale* __restrict__ ls)
{
    if (threadIdx.x == 0) *slot = bucket_partial(0.0, 0, stamp, ls != nullptr ? scale * ls->inv_scale : scale);
}

__global__ void loss_scale_init_kernel(zero_loss_scale s, zero_loss_scale* __restrict__ ls)
{
    if (threadIdx.x == 0) *ls = s;
}

__global__ void loss_scale_update_kernel(zero_loss_scale_config c, const zero_result* __restrict__ res,
                                         zero_loss_scale* __restrict__ ls)
{
    if (threadIdx.x == 0 && res->status == ZERO_OK) loss_scale_move(c, res->found_inf != 0, ls);
}

__global__ __launch_bounds__(kThreads) void plan_write_kernel(uint8_t* __restrict__ ws, WriteChunk c)
{
    uint32_t* dst = reinterpret_cast<uint32_t*>(ws + c.offset);
    for (uint32_t i = threadIdx.x; i < c.words; i += kThreads) dst[i] = c.data[i];
}

__global__ __launch_bounds__(kThreads) void plan_tiles_kernel(const TensorDesc* __restrict__ desc, int T,
                                                              TileRef* __restrict__ map0, TileRef* __restrict__ map1)
{
    for (int t = blockIdx.x; t < T; t += gridDim.x) {
        for (int p = 0; p < 2; ++p) {
            TileRef* map = p == 0 ? map0 : map1;
            if (map == nullptr) continue;
            const int64_t b = desc[t].tile_begin[p], nt = desc[t].ntiles[p];
            for (int64_t j = threadIdx.x; j < nt; j += kThreads) {
                TileRef r;
                r.tensor = t;
                r.local = static_cast<int32_t>(j);
                map[b + j] = r;
            }
        }
    }
}

// ------------------------------------------------------------------ occupancy

int device_cus()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        cached[dev] = v;
    }
    return cached[dev];
}

// Resident workgroups of one kernel on the current device, cached per
// (kernel, device).
template <typename K>
int resident(K kernel, int block = kThreads)
{
    static std::mutex mu;
    static std::map<std::pair<const void*, int>, int> cache;
    int dev = 0;
    (void)hipGetDevice(&dev);
    const auto key = std::make_pair(reinterpret_cast<const void*>(kernel), dev);
    {
        std::lock_guard<std::mutex> lk(mu);
        auto it = cache.find(key);
        if (it != cache.end()) return it->second;
    }
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess || per_cu <= 0)
        per_cu = 1;
    int g = per_cu * device_cus();
    g = g < kMaxPartials ? g : kMaxPartials;
    std::lock_guard<std::mutex> lk(mu);
    cache[key] = g;
    return g;
}

template <bool FROM0>
hipError_t reduce_dispatch(const RankPtrs& ptrs, int Mc, int last, float scale, const Layout& L, float* g_out,
                           int grid, hipStream_t s)
{
    switch (Mc) {
    case 1: reduce_kernel<1, FROM0><<<grid, kThreads, 0, s>>>(ptrs, Mc, last, scale, L, g_out); break;
    case 2: reduce_kernel<2, FROM0><<<grid, kThreads, 0, s>>>(ptrs, Mc, last, scale, L, g_out); break;
    case 4: reduce_kernel<4, FROM0><<<grid, kThreads, 0, s>>>(ptrs, Mc, last, scale, L, g_out); break;
    case 8: reduce_kernel<8, FROM0><<<grid, kThreads, 0, s>>>(ptrs, Mc, last, scale, L, g_out); break;
    case 16: reduce_kernel<16, FROM0><<<grid, kThreads, 0, s>>>(ptrs, Mc, last, scale, L, g_out); break;
    case 32: reduce_kernel<32, FROM0><<<grid, kThreads, 0, s>>>(ptrs, Mc, last, scale, L, g_out); break;
    case 64: reduce_kernel<64, FROM0><<<grid, kThreads, 0, s>>>(ptrs, Mc, last, scale, L, g_out); break;
    default: reduce_kernel<0, FROM0><<<grid, kThreads, 0, s>>>(ptrs, Mc, last, scale, L, g_out); break;
    }
    return hipGetLastError();
}

#define ZERO_FOR_EACH_GEOM(X) \
    X(0, 256, 1) X(1, 1024, 1) X(2, 1024, 2) X(3, 1024, 4) X(4, 1024, 8) X(5, 512, 16) X(6, 256, 16)

// The geometries each mode is launched with, from the plan's rules: the
// single-pass step never takes 1024 x 8, a pass that only folds never takes
// 256 x 16, and the update pass always runs 256 x 1. Only these are built; any
// other pair is an error at launch.
template <Mode MODE>
constexpr bool geom_used(int g)
{
    return MODE == Mode::PassB ? g == 0 : (MODE == Mode::Full || MODE == Mode::BucketFull) ? g != 4 : g != 6;
}

template <Mode MODE>
hipError_t fused_dispatch(int geom, const PlanHeader* hdr, const TensorDesc* desc, const TileRef* map, int64_t tiles,
                          uint64_t sig, int M, float gscale, const AdamScalars& c, Partial* parts,
                          const FinalizeArgs& fin, const zero_result* res, hipStream_t s)
{
    if (tiles <= 0 || tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    const unsigned grid = static_cast<unsigned>(tiles);
    switch (geom) {
#define ZERO_CASE(I, NTV, UV)                                                                              \
    case I:                                                                                                \
        if constexpr (geom_used<MODE>(I))                                                                  \
            fused_kernel<MODE, NTV, UV><<<grid, NTV, 0, s>>>(hdr, desc, map, sig, M, gscale, c, parts, fin, res); \
        else                                                                                               \
            return hipErrorInvalidValue;                                                                   \
        break;
        ZERO_FOR_EACH_GEOM(ZERO_CASE)
#undef ZERO_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

// ------------------------------------------------------------------ wrappers

hipError_t launch_reduce(const RankPtrs& ptrs, int Mc, bool first, bool last, float scale, const Layout& L,
                         float* g_out, int grid, hipStream_t s)
{
    if (first) return reduce_dispatch<true>(ptrs, Mc, last ? 1 : 0, scale, L, g_out, grid, s);
    return reduce_dispatch<false>(ptrs, Mc, last ? 1 : 0, scale, L, g_out, grid, s);
}

hipError_t launch_check(const float* g, const Layout& L, Partial* parts, int grid, hipStream_t s)
{
    check_kernel<<<grid, kThreads, 0, s>>>(g, L, parts);
    return hipGetLastError();
}

hipError_t launch_adamw(float* master, float* m, float* v, const float* g, uint16_t* out, const Layout& L,
                        const AdamScalars& c, const zero_result* res, int grid, hipStream_t s)
{
    adamw_kernel<<<grid, kThreads, 0, s>>>(master, m, v, g, out, L, c, res);
    return hipGetLastError();
}

hipError_t launch_finalize(const Partial* parts, int64_t nparts, double external, double max_norm, int skip,
                           zero_result* res, hipStream_t s)
{
    finalize_kernel<<<1, kThreads, 0, s>>>(parts, nparts, external, max_norm, skip, res);
    return hipGetLastError();
}

hipError_t launch_bucket_finalize(const PlanHeader* hdr, uint64_t sig, const zero_bucket_partial* parts, int32_t nb,
                                  uint64_t stamp, float scale, const zero_loss_scale* ls, double external,
                                  double max_norm, int skip, zero_result* res, hipStream_t s)
{
    bucket_finalize_kernel<<<1, kThreads, 0, s>>>(hdr, sig, parts, nb, stamp, scale, ls, external, max_norm, skip,
                                                  res);
    return hipGetLastError();
}

hipError_t launch_bucket_partial_empty(zero_bucket_partial* slot, uint64_t stamp, float scale,
                                       const zero_loss_scale* ls, hipStream_t s)
{
    bucket_partial_empty_kernel<<<1, 64, 0, s>>>(slot, stamp, scale, ls);
    return hipGetLastError();
}

hipError_t launch_loss_scale_init(const zero_loss_scale& s, zero_loss_scale* ls, hipStream_t st)
{
    loss_scale_init_kernel<<<1, 64, 0, st>>>(s, ls);
    return hipGetLastError();
}

hipError_t launch_loss_scale_update(const zero_loss_scale_config& c, const zero_result* res, zero_loss_scale* ls,
                                    hipStream_t st)
{
    loss_scale_update_kernel<<<1, 64, 0, st>>>(c, res, ls);
    return hipGetLastError();
}

hipError_t launch_plan_write(uint8_t* ws, const WriteChunk& c, hipStream_t s)
{
    plan_write_kernel<<<1, kThreads, 0, s>>>(ws, c);
    return hipGetLastError();
}

hipError_t launch_plan_tiles(const TensorDesc* desc, int T, TileRef* map0, TileRef* map1, hipStream_t s)
{
    const int grid = T < 4096 ? (T > 0 ? T : 1) : 4096;
    plan_tiles_kernel<<<grid, kThreads, 0, s>>>(desc, T, map0, map1);
    return hipGetLastError();
}

hipError_t launch_fused(Mode mode, int geom, const PlanHeader* hdr, const TensorDesc* desc, const TileRef* map,
                        int64_t tiles, uint64_t sig, int M, float gscale, const AdamScalars& c, Partial* parts,
                        const FinalizeArgs& fin, const zero_result* res, hipStream_t s)
{
    switch (mode) {
    case Mode::Full:
        return fused_dispatch<Mode::Full>(geom, hdr, desc, map, tiles, sig, M, gscale, c, parts, fin, res, s);
    case Mode::PassA:
        return fused_dispatch<Mode::PassA>(geom, hdr, desc, map, tiles, sig, M, gscale, c, parts, fin, res, s);
    case Mode::PassB:
        return fused_dispatch<Mode::PassB>(geom, hdr, desc, map, tiles, sig, M, gscale, c, parts, fin, res, s);
    case Mode::Acc:
        return fused_dispatch<Mode::Acc>(geom, hdr, desc, map, tiles, sig, M, gscale, c, parts, fin, res, s);
    case Mode::BucketFull:
        return fused_dispatch<Mode::BucketFull>(geom, hdr, desc, map, tiles, sig, M, gscale, c, parts, fin, res, s);
    }
    return hipErrorInvalidValue;
}

int resident_grid_reduce(int Mc, bool first)
{
    // every instantiation has the same launch bounds; the widest one decides
    (void)Mc;
    return first ? resident(reduce_kernel<64, true>) : resident(reduce_kernel<64, false>);
}

int resident_grid_check() { return resident(check_kernel); }
int resident_grid_adamw() { return resident(adamw_kernel); }

int compute_units() { return device_cus(); }

// ------------------------------------------------------------------ static scratch
//
// The workspace of zero_step_noalloc: one zero_step plan (header, tensor
// table, rank pointers, tile maps, per-tile partials and, for a two-pass
// plan, the fp32 gradient) kept in a file-scope device array instead of
// caller memory, for callers that cannot allocate. Each device holds its own
// copy from the moment the library's code is loaded on it until the process
// ends. In host code `scratch` names a host-side stand-in, not the device
// array: its device address is taken once per device with
// hipGetSymbolAddress, with that device current, and only that address is
// handed to kernels and copies.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t scratch_workspace(void** ptr)
{
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr || reinterpret_cast<uintptr_t>(p) % kAlign != 0) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace zero
