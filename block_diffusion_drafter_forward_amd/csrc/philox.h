// Counter-based random draws for sampling at temperature 1.
//
// Generator: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
// SC 2011): ten rounds, each multiplying counter words 0 and 2 by two fixed multipliers into 64-bit products
// and recombining their halves with the other two words and the key; the key advances by two Weyl constants
// between rounds.  Being counter-based, the draw for any (stream, index) is made where it is consumed -- in
// the epilogue of the LM head for each logit -- with no state and no stored random numbers.
//
// Stream layout: the 32-bit word for (tag, row, index j) under a 64-bit seed is word j % 4 of the block at
// counter (j / 4, row, tag, 0), key (seed low word, seed high word).  Tags: 1 drafting (row = request * L +
// block row, j = vocabulary id), 2 acceptance uniforms (row = request, j = draft position), 3 residual or
// bonus sampling (row = request, j = vocabulary id).  A word c stands for the uniform u = (c + 1/2) / 2^32
// and the standard Gumbel variable G = -ln(-ln(1 - u)).
#pragma once
#include <stdint.h>

namespace df {

enum { RNG_TAG_DRAFT = 1, RNG_TAG_ACCEPT = 2, RNG_TAG_RESAMPLE = 3 };

struct RngKey {
    uint32_t lo, hi;
};

// The four words of the block at counter (quad, row, tag, 0).
__device__ __forceinline__ void philox_block(RngKey key, uint32_t quad, uint32_t row, uint32_t tag, uint32_t (&w)[4]) {
    uint32_t c0 = quad, c1 = row, c2 = tag, c3 = 0u;
    uint32_t k0 = key.lo, k1 = key.hi;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
        const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
        const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    w[0] = c0;
    w[1] = c1;
    w[2] = c2;
    w[3] = c3;
}

// One word of stream (tag, row) at index j.
__device__ __forceinline__ uint32_t rng_word(RngKey key, uint32_t j, uint32_t row, uint32_t tag) {
    uint32_t w[4];
    philox_block(key, j >> 2, row, tag, w);
    const uint32_t e = j & 3u;
    return e == 0 ? w[0] : e == 1 ? w[1] : e == 2 ? w[2] : w[3];
}

// u = (c + 1/2) / 2^32 in float32, kept below 1 (the conversion of the largest words rounds up to 2^32).
__device__ __forceinline__ float rng_uniform(uint32_t c) {
    return fminf(((float)c + 0.5f) * 2.3283064365386963e-10f, 0.99999994f);
}

// G = -ln(-ln(1 - u)); log1p keeps full relative precision for small u, where G is large (the draws that
// decide a Gumbel-max sample).
__device__ __forceinline__ float rng_gumbel(uint32_t c) { return -logf(-log1pf(-rng_uniform(c))); }

}  // namespace df
