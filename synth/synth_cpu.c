/* Host build of the synthetic-input generator (definitions in synth_core.h).
 * Used by the oracle side of the tests and by the bench's CPU baseline. */
#define SYNTH_FN static inline
#include "synth_core.h"

#include <stddef.h>

/* Contribution rows k = 0..n-1 for global elements [idx0, idx0+len):
 * out[k*stride + i] for i < len; columns [len, stride) are set to zero. */
void synth_contrib_rows(uint64_t seed, uint32_t step, int32_t n, int32_t dtype, double sigma,
                        double scale, uint64_t outlier_thresh, double outlier_mult, int64_t idx0,
                        int64_t len, int64_t stride, uint16_t *out) {
    for (int32_t k = 0; k < n; ++k) {
        uint64_t kc = synth_stream_key(seed, SYNTH_STREAM_CONTRIB, step, (uint32_t)k);
        uint64_t ko = synth_stream_key(seed, SYNTH_STREAM_OUTLIER, step, (uint32_t)k);
        uint16_t *row = out + (size_t)k * (size_t)stride;
        for (int64_t i = 0; i < len; ++i)
            row[i] = synth_contrib_value(kc, ko, outlier_thresh, sigma, scale, outlier_mult, dtype,
                                         (uint64_t)(idx0 + i));
        for (int64_t i = len; i < stride; ++i) row[i] = 0;
    }
}

/* Contributions at arbitrary global elements: out[k*count + j] is contribution
 * k of element idx[j]. */
void synth_contrib_at(uint64_t seed, uint32_t step, int32_t n, int32_t dtype, double sigma,
                      double scale, uint64_t outlier_thresh, double outlier_mult,
                      const int64_t *idx, int64_t count, uint16_t *out) {
    for (int32_t k = 0; k < n; ++k) {
        uint64_t kc = synth_stream_key(seed, SYNTH_STREAM_CONTRIB, step, (uint32_t)k);
        uint64_t ko = synth_stream_key(seed, SYNTH_STREAM_OUTLIER, step, (uint32_t)k);
        for (int64_t j = 0; j < count; ++j)
            out[(size_t)k * (size_t)count + (size_t)j] = synth_contrib_value(
                kc, ko, outlier_thresh, sigma, scale, outlier_mult, dtype, (uint64_t)idx[j]);
    }
}

void synth_master_range(uint64_t seed, double sigma, int64_t idx0, int64_t len, float *out) {
    uint64_t km = synth_stream_key(seed, SYNTH_STREAM_MASTER, 0u, 0u);
    for (int64_t i = 0; i < len; ++i) out[i] = synth_master_value(km, sigma, (uint64_t)(idx0 + i));
}

void synth_master_at(uint64_t seed, double sigma, const int64_t *idx, int64_t count, float *out) {
    uint64_t km = synth_stream_key(seed, SYNTH_STREAM_MASTER, 0u, 0u);
    for (int64_t j = 0; j < count; ++j) out[j] = synth_master_value(km, sigma, (uint64_t)idx[j]);
}

/* Raw generator words, for distribution tests. */
void synth_bits_range(uint64_t seed, uint32_t stream, uint32_t step, uint32_t k, int64_t idx0,
                      int64_t len, uint64_t *out) {
    uint64_t key = synth_stream_key(seed, stream, step, k);
    for (int64_t i = 0; i < len; ++i) out[i] = synth_bits(key, (uint64_t)(idx0 + i));
}

void synth_normal_range(uint64_t seed, uint32_t stream, uint32_t step, uint32_t k, int64_t idx0,
                        int64_t len, double *out) {
    uint64_t key = synth_stream_key(seed, stream, step, k);
    for (int64_t i = 0; i < len; ++i) out[i] = synth_normal(synth_bits(key, (uint64_t)(idx0 + i)));
}

/* Initial 16-bit parameters: the generator's master values rounded to dtype. */
void synth_param_range(uint64_t seed, double sigma, int32_t dtype, int64_t idx0, int64_t len,
                       uint16_t *out) {
    uint64_t km = synth_stream_key(seed, SYNTH_STREAM_MASTER, 0u, 0u);
    for (int64_t i = 0; i < len; ++i) {
        float f = synth_master_value(km, sigma, (uint64_t)(idx0 + i));
        out[i] = dtype == SYNTH_BF16 ? synth_f32_to_bf16(f) : synth_f32_to_f16(f);
    }
}

void synth_param_at(uint64_t seed, double sigma, int32_t dtype, const int64_t *idx, int64_t count,
                    uint16_t *out) {
    uint64_t km = synth_stream_key(seed, SYNTH_STREAM_MASTER, 0u, 0u);
    for (int64_t j = 0; j < count; ++j) {
        float f = synth_master_value(km, sigma, (uint64_t)idx[j]);
        out[j] = dtype == SYNTH_BF16 ? synth_f32_to_bf16(f) : synth_f32_to_f16(f);
    }
}
