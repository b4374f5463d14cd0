/*
 * synth_host.c -- host side of the seeded synthetic-input generator.
 *
 * Shared input generator for tests and benchmark: it produces gradient
 * replicas and optimizer state, and holds none of the optimizer step's
 * arithmetic. synth_gpu.hip implements the identical generator for the GPU;
 * both must give the same bits for every index.
 *
 * Generator (a pure function of seed, stream and element index i):
 *   w[0..3] = Philox4x32-10(counter = {lo32(i), hi32(i), 0, 0},
 *                           key = {seed, stream})
 *     (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
 *      1, 2, 3", SC 2011: 10 rounds, multipliers 0xD2511F53 / 0xCD9E8D57,
 *      Weyl key increments 0x9E3779B9 / 0xBB67AE85.)
 *   h[0..7] = the eight 16-bit halves of w; S = sum of h (Irwin-Hall of 8).
 *   z = (2*S - 8*65535) * C, C = sqrt(3 / (8 * (2^32 - 1))), in binary64:
 *       zero mean, unit variance, support about +-4.9.
 *   normal:     f = (float)(z * std)
 *   abs normal: f = (float)(|z| * std)
 *   bf16 codes: the upper 16 bits of f (rounded toward zero).
 * Every step is an integer operation or one IEEE binary64 multiply or
 * conversion, so both implementations give identical bits.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u
#define IRWIN_HALL_C 0x1.3988e1412ed76p-17

void synth_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += PHILOX_W0; k1 += PHILOX_W1; }
        const uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        const uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n1 = (uint32_t)p1;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        const uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static double synth_z(uint64_t i, uint32_t seed, uint32_t stream)
{
    const uint32_t ctr[4] = {(uint32_t)i, (uint32_t)(i >> 32), 0u, 0u};
    const uint32_t key[2] = {seed, stream};
    uint32_t w[4];
    synth_philox4x32_10(ctr, key, w);
    int32_t s = 0;
    for (int k = 0; k < 4; ++k) s += (int32_t)(w[k] & 0xFFFFu) + (int32_t)(w[k] >> 16);
    const int32_t d = 2 * s - 8 * 65535;
    return (double)d * IRWIN_HALL_C;
}

static float synth_f32_at(uint64_t i, uint32_t seed, uint32_t stream, double std, int32_t absval)
{
    double z = synth_z(i, seed, stream);
    if (absval) z = fabs(z);
    return (float)(z * std);
}

static uint16_t synth_bf16_at(uint64_t i, uint32_t seed, uint32_t stream, double std)
{
    const float f = synth_f32_at(i, seed, stream, std, 0);
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* Contiguous fill of elements [start, start + n). */
void synth_fill_f32(float* out, int64_t n, int64_t start, uint32_t seed, uint32_t stream, double std, int32_t absval)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = synth_f32_at((uint64_t)(start + i), seed, stream, std, absval);
}

void synth_fill_bf16(uint16_t* out, int64_t n, int64_t start, uint32_t seed, uint32_t stream, double std)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = synth_bf16_at((uint64_t)(start + i), seed, stream, std);
}

/* Values at arbitrary indices. */
void synth_gather_f32(float* out, const int64_t* idx, int64_t k, uint32_t seed, uint32_t stream, double std,
                      int32_t absval)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < k; ++j) out[j] = synth_f32_at((uint64_t)idx[j], seed, stream, std, absval);
}

void synth_gather_bf16(uint16_t* out, const int64_t* idx, int64_t k, uint32_t seed, uint32_t stream, double std)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < k; ++j) out[j] = synth_bf16_at((uint64_t)idx[j], seed, stream, std);
}

/* Raw 4x32 blocks for counters {lo32(i), hi32(i), 0, 0}, i in [start, start+k). */
void synth_raw_blocks(uint32_t* out, int64_t k, int64_t start, uint32_t seed, uint32_t stream)
{
    const uint32_t key[2] = {seed, stream};
    for (int64_t j = 0; j < k; ++j) {
        const uint64_t i = (uint64_t)(start + j);
        const uint32_t ctr[4] = {(uint32_t)i, (uint32_t)(i >> 32), 0u, 0u};
        synth_philox4x32_10(ctr, key, out + 4 * j);
    }
}
