/*
 * Seeded synthetic-input generator shared by the tests, the benchmark and the
 * oracle's callers.  It draws random numbers and rounds them to the storage
 * type of each input; it holds none of the decode-tail arithmetic.
 *
 * Counter-based generator: Philox4x32-10, as defined in Salmon, Moraes, Dror
 * and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11), section 3
 * (Philox S-box: two 32x32->64 multiplies per round, Weyl key schedule,
 * ten rounds).  Every output element is a pure function of
 * (seed, stream, element index), so any slice can be produced on any number
 * of threads and the result never depends on the order of draws.
 *
 * Normals: Box-Muller on two 53-bit uniforms taken from one Philox block;
 * element 2p uses the cosine branch and element 2p+1 the sine branch of
 * block p.  The value mean + std*z is formed in double and rounded to
 * float32 (round to nearest even); a bfloat16 output is then the
 * round-to-nearest-even bfloat16 of that float32.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static void philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
        k0 += PHILOX_W0; k1 += PHILOX_W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* block `p` of stream (seed, stream, lane) */
static void block(uint64_t seed, uint32_t stream, uint32_t lane, uint64_t p, uint32_t out[4]) {
    uint32_t ctr[4] = {(uint32_t)p, (uint32_t)(p >> 32), stream, lane};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    philox4x32_10(ctr, key, out);
}

static double u53(uint32_t hi, uint32_t lo) { /* [0, 1) on a 2^-53 grid */
    uint64_t x = ((uint64_t)hi << 32) | lo;
    return (double)(x >> 11) * 0x1.0p-53;
}

static uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u) { /* inf / nan: keep, quiet the nan */
        uint16_t h = (uint16_t)(u >> 16);
        if (u & 0x007FFFFFu) h |= 0x0040u;
        return h;
    }
    uint32_t bias = 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)((u + bias) >> 16);
}

static float normal_at(uint64_t seed, uint32_t stream, uint64_t i, double mean, double std) {
    uint32_t b[4];
    block(seed, stream, 0u, i >> 1, b);
    double u1 = 1.0 - u53(b[0], b[1]); /* (0, 1] */
    double u2 = u53(b[2], b[3]);
    double r = sqrt(-2.0 * log(u1));
    double t = 6.283185307179586476925286766559 * u2;
    double z = (i & 1) ? r * sin(t) : r * cos(t);
    return (float)(mean + std * z);
}

/* out[i] = float32(mean + std*z_i), i in [offset, offset+n) of the stream */
void synth_normal_f32(uint64_t seed, uint32_t stream, uint64_t offset, size_t n,
                      double mean, double std, float* out) {
    #pragma omp parallel for schedule(static)
    for (long long j = 0; j < (long long)n; ++j)
        out[j] = normal_at(seed, stream, offset + (uint64_t)j, mean, std);
}

/* out[i] = bf16_rne(float32(mean + std*z_i)), as raw bfloat16 bits */
void synth_normal_bf16(uint64_t seed, uint32_t stream, uint64_t offset, size_t n,
                       double mean, double std, uint16_t* out) {
    #pragma omp parallel for schedule(static)
    for (long long j = 0; j < (long long)n; ++j)
        out[j] = f32_to_bf16_rne(normal_at(seed, stream, offset + (uint64_t)j, mean, std));
}

/* out[i] in [0, 1) on a 2^-53 grid */
void synth_uniform_f64(uint64_t seed, uint32_t stream, uint64_t offset, size_t n, double* out) {
    #pragma omp parallel for schedule(static)
    for (long long j = 0; j < (long long)n; ++j) {
        uint32_t b[4];
        block(seed, stream, 1u, offset + (uint64_t)j, b);
        out[j] = u53(b[0], b[1]);
    }
}

/* out[i] in [0, 1) on a 2^-24 grid, so every value is exact in float32 */
void synth_uniform_f32(uint64_t seed, uint32_t stream, uint64_t offset, size_t n, float* out) {
    #pragma omp parallel for schedule(static)
    for (long long j = 0; j < (long long)n; ++j) {
        uint32_t b[4];
        block(seed, stream, 2u, offset + (uint64_t)j, b);
        out[j] = (float)(b[0] >> 8) * 0x1.0p-24f;
    }
}

/* raw Philox4x32-10 blocks, for the known-answer test of the generator */
void synth_philox_block(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    philox4x32_10(ctr, key, out);
}

/* bfloat16 round-to-nearest-even of float32 values, as raw bits */
void synth_round_bf16(const float* in, size_t n, uint16_t* out) {
    #pragma omp parallel for schedule(static)
    for (long long j = 0; j < (long long)n; ++j) out[j] = f32_to_bf16_rne(in[j]);
}
