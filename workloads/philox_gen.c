/*
 * Seeded synthetic-input generator shared by the oracle tests, the GPU tests and the benchmark.
 *
 * It holds none of the drafter's arithmetic: it only turns (key, stream, index) into random numbers.
 * Random bits come from Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and Shaw,
 * "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011), written here from that definition.
 * Normal deviates use the Box-Muller transform (Box and Muller, 1958) in double precision; each value
 * is then scaled, rounded to float32, and optionally rounded to bfloat16 (round to nearest, ties to even).
 * Every output element depends only on (key, stream, index), so the result does not depend on threading.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void mulhilo(uint32_t a, uint32_t b, uint32_t *hi, uint32_t *lo) {
    uint64_t p = (uint64_t)a * (uint64_t)b;
    *hi = (uint32_t)(p >> 32);
    *lo = (uint32_t)p;
}

/* Ten rounds of Philox4x32 on counter c under key k (the key is bumped by the Weyl constants). */
static inline void philox4x32_10(const uint32_t in[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c0 = in[0], c1 = in[1], c2 = in[2], c3 = in[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        uint32_t hi0, lo0, hi1, lo1;
        mulhilo(PHILOX_M0, c0, &hi0, &lo0);
        mulhilo(PHILOX_M1, c2, &hi1, &lo1);
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += PHILOX_W0;
        k1 += PHILOX_W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Counter for block b of stream s: (b_lo, b_hi, s_lo, s_hi). */
static inline void block_bits(uint64_t key64, uint64_t stream, uint64_t b, uint32_t out[4]) {
    uint32_t ctr[4] = {(uint32_t)b, (uint32_t)(b >> 32), (uint32_t)stream, (uint32_t)(stream >> 32)};
    uint32_t key[2] = {(uint32_t)key64, (uint32_t)(key64 >> 32)};
    philox4x32_10(ctr, key, out);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Raw 32-bit words of elements start..start+n-1: element i is word (i % 4) of Philox block i / 4. */
void synth_u32(uint64_t key, uint64_t stream, int64_t start, int64_t n, uint32_t *out) {
    if (n <= 0) return;
    int64_t b0 = start / 4, b1 = (start + n - 1) / 4;
    #pragma omp parallel for schedule(static)
    for (int64_t b = b0; b <= b1; ++b) {
        uint32_t w[4];
        block_bits(key, stream, (uint64_t)b, w);
        for (int j = 0; j < 4; ++j) {
            int64_t i = 4 * b + j;
            if (i >= start && i < start + n) out[i - start] = w[j];
        }
    }
}

/* Normal deviates times `scale` for elements start..start+n-1 of the stream.
 * mode 0: float32 output; mode 1: bfloat16 bit patterns (uint16).
 * Block b yields elements 4b..4b+3: two Box-Muller pairs from its four words. */
void synth_normal(uint64_t key, uint64_t stream, int64_t start, int64_t n, double scale, int mode, void *out) {
    const double two_pi = 6.283185307179586476925286766559;
    const double inv32 = 1.0 / 4294967296.0;
    if (n <= 0) return;
    int64_t b0 = start / 4, b1 = (start + n - 1) / 4;
    #pragma omp parallel for schedule(static)
    for (int64_t b = b0; b <= b1; ++b) {
        uint32_t w[4];
        block_bits(key, stream, (uint64_t)b, w);
        double z[4];
        for (int p = 0; p < 2; ++p) {
            double u1 = ((double)w[2 * p] + 1.0) * inv32; /* (0, 1] */
            double u2 = (double)w[2 * p + 1] * inv32;     /* [0, 1) */
            double r = sqrt(-2.0 * log(u1));
            z[2 * p] = r * cos(two_pi * u2);
            z[2 * p + 1] = r * sin(two_pi * u2);
        }
        for (int j = 0; j < 4; ++j) {
            int64_t i = 4 * b + j;
            if (i < start || i >= start + n) continue;
            float v = (float)(z[j] * scale);
            if (mode == 0) ((float *)out)[i - start] = v;
            else ((uint16_t *)out)[i - start] = f32_to_bf16_rne(v);
        }
    }
}

/* One raw Philox4x32-10 block, exposed for the known-answer test. */
void synth_philox_block(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    philox4x32_10(ctr, key, out);
}
