/* Seeded synthetic inputs for the ZeRO per-rank shard step.
 *
 * This header is the ONE definition of every synthetic input (gradient
 * contributions, initial fp32 master weights, outlier masks).  It is compiled
 * twice: by gcc into the host generator and by hipcc into the device
 * generator, so both produce bit-identical values for the same
 * (seed, stream, step, k, element index).  It holds none of the shard step's
 * arithmetic: no reduction, no scaling policy, no optimizer.
 *
 * The includer defines SYNTH_FN (host-only `static inline` for C, or
 * `__host__ __device__ static inline` for HIP) before including this file.
 *
 * Every floating-point expression below is exact in binary64 except where a
 * single rounding is noted, and both builds use -ffp-contract=off, so no
 * fused multiply-add can make the two builds differ.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <stdint.h>

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ull /* splitmix64 increment (odd golden-ratio constant) */

#define SYNTH_STREAM_MASTER 0u   /* initial fp32 master weights */
#define SYNTH_STREAM_CONTRIB 1u  /* gradient contributions, by (step, k) */
#define SYNTH_STREAM_OUTLIER 2u  /* Bernoulli outlier mask, by (step, k) */

#define SYNTH_F16 1
#define SYNTH_BF16 2

/* splitmix64 output function (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014). */
SYNTH_FN uint64_t synth_mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* Starting state of the sequence for one (seed, stream, step, k). */
SYNTH_FN uint64_t synth_stream_key(uint64_t seed, uint32_t stream, uint32_t step, uint32_t k) {
    uint64_t z = synth_mix64(seed + SYNTH_GAMMA * (1ull + stream));
    z = synth_mix64(z + SYNTH_GAMMA * (1ull + step));
    z = synth_mix64(z + SYNTH_GAMMA * (1ull + k));
    return z;
}

/* Output number idx (0-based) of the splitmix64 sequence whose state starts
 * at `key`: the state after idx+1 increments, mixed.  Counter-based, so any
 * element can be drawn on its own. */
SYNTH_FN uint64_t synth_bits(uint64_t key, uint64_t idx) {
    return synth_mix64(key + (idx + 1ull) * SYNTH_GAMMA);
}

/* Approximately standard-normal deviate from 64 random bits: the sum of four
 * 16-bit uniforms u_j = (b_j + 1/2) / 2^16 on (0,1) (Irwin-Hall with n = 4:
 * mean 2, variance 1/3), centred and rescaled to unit variance:
 *   z = (sum_j u_j - 2) * sqrt(3) = (b_0 + b_1 + b_2 + b_3 - 131070) * 2^-16 * sqrt(3).
 * Bounded by +-2*sqrt(3).  Everything before the product by sqrt(3) is exact;
 * that product is the only rounding. */
SYNTH_FN double synth_normal(uint64_t bits) {
    int32_t s = (int32_t)(bits & 0xFFFFu) + (int32_t)((bits >> 16) & 0xFFFFu) +
                (int32_t)((bits >> 32) & 0xFFFFu) + (int32_t)(bits >> 48);
    return ((double)(s - 131070) * 0x1p-16) * 1.7320508075688772;
}

SYNTH_FN uint32_t synth_f32_bits(float f) {
    union { float f; uint32_t u; } c;
    c.f = f;
    return c.u;
}

/* binary32 -> binary16, round to nearest even (integer form). */
SYNTH_FN uint16_t synth_f32_to_f16(float f) {
    uint32_t x = synth_f32_bits(f);
    uint32_t sign = (x >> 16) & 0x8000u;
    x &= 0x7FFFFFFFu;
    if (x >= 0x7F800000u) return (uint16_t)(sign | (x > 0x7F800000u ? 0x7E00u : 0x7C00u));
    if (x >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u); /* >= 65520 rounds past 65504 */
    if (x < 0x38800000u) {                                    /* below 2^-14: subnormal result */
        if (x < 0x33000000u) return (uint16_t)sign;           /* <= 2^-25 rounds to zero */
        uint32_t e = x >> 23;
        uint32_t mant = (x & 0x7FFFFFu) | 0x800000u;
        uint32_t sh = 126u - e; /* value in units of 2^-24 is mant >> sh */
        uint32_t q = mant >> sh;
        uint32_t rem = mant & ((1u << sh) - 1u);
        uint32_t half = 1u << (sh - 1u);
        q += (uint32_t)(rem > half) | ((uint32_t)(rem == half) & q & 1u);
        return (uint16_t)(sign | q);
    }
    uint32_t e = x >> 23;
    uint32_t mant = x & 0x7FFFFFu;
    uint32_t h = ((e - 112u) << 10) | (mant >> 13);
    uint32_t rem = mant & 0x1FFFu;
    h += (uint32_t)(rem > 0x1000u) | ((uint32_t)(rem == 0x1000u) & h & 1u);
    return (uint16_t)(sign | h);
}

/* binary32 -> bfloat16, round to nearest even (integer form). */
SYNTH_FN uint16_t synth_f32_to_bf16(float f) {
    uint32_t x = synth_f32_bits(f);
    if ((x & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((x >> 16) | 0x40u);
    x += 0x7FFFu + ((x >> 16) & 1u);
    return (uint16_t)(x >> 16);
}

/* One gradient contribution element, as 16-bit storage bits.
 * value = N(0,1) * sigma [* mult if the outlier draw fires] * scale,
 * rounded binary64 -> binary32 -> dtype. */
SYNTH_FN uint16_t synth_contrib_value(uint64_t key_c, uint64_t key_o, uint64_t outlier_thresh,
                                      double sigma, double scale, double outlier_mult, int dtype,
                                      uint64_t idx) {
    double x = synth_normal(synth_bits(key_c, idx)) * sigma;
    if (outlier_thresh != 0ull && synth_bits(key_o, idx) < outlier_thresh) x = x * outlier_mult;
    x = x * scale;
    float f = (float)x;
    return dtype == SYNTH_BF16 ? synth_f32_to_bf16(f) : synth_f32_to_f16(f);
}

/* One initial fp32 master weight: N(0,1) * sigma rounded to binary32. */
SYNTH_FN float synth_master_value(uint64_t key_m, double sigma, uint64_t idx) {
    return (float)(synth_normal(synth_bits(key_m, idx)) * sigma);
}

#endif
