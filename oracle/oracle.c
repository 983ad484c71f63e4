/* oracle.c -- CPU oracle for the ZeRO per-rank shard step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  The GPU library
 * never calls, links or includes anything here, and this file includes
 * nothing of the GPU library; the two share no code.
 *
 * Plain, slow and single-threaded.  Each function states the passage of the
 * ZeRO pages it follows.  Page names used below:
 *   [sim]  "zero-stages-simulation" README (riteshverma), the per-GPU model-state
 *          table and the paragraph on flat contiguous partitioning.
 *   [bea]  "ZeRO Stage 1/2/3" (infra.bea.ai guide), sections 1-5.
 *   [pg]   "ZeRO: Memory Optimizations Toward Training Trillion Parameter Models"
 *          (paper-graph summary), section 3.4 (model-state analysis, Stage 1/2/3,
 *          residual states).
 *   [cmu]  "CMU 11-868 L18: How ZeRO Cuts Data-Parallel Memory", "Mechanism 1"
 *          steps 3-6.
 *   [grasp] "ZeRO: Memory Optimization for Large Models", "Stage 1" and "Stage 2".
 *
 * Precision: the pages fix fp16/bf16 gradients and parameters and fp32 master,
 * momentum, variance and reduced gradient ([pg] 3.4 "16 Psi baseline"; [cmu]
 * Mechanism 1 step 3, fp32 reduced gradient).  The oracle computes exactly those types,
 * every operation rounded once in the order written (compiled with
 * -ffp-contract=off, SSE scalar arithmetic).  The squared-norm is exact.
 *
 * Readings the pages leave open, and their pins: the clip rule and the loss
 * scaler's schedule (the pages give neither) are pinned to PyTorch's own
 * routines on the CPU (clip_grads_with_norm_, _amp_update_scale_), with the
 * one departure stated above oracle_finalize (the scale never drops below
 * min_scale); the block quantisation's zero-point form and rounding (the
 * page names the form, not the arithmetic) are pinned to PyTorch's affine
 * quantiser, block by block.  Adam is pinned by closed forms and by
 * torch.optim.AdamW (within 1e-5 of each array's RMS; its operations are
 * ordered differently).  Parity unpinned: the quantisation block length of
 * 2048 elements (no page gives one; the tests only check that it is what
 * the reading says) and the S = 1 / NaN conventions for empty and
 * non-finite blocks.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 and bfloat16 (the upper half of binary32), written from  */
/* the format definitions.  Mixed precision keeps parameters and gradients in  */
/* a 16-bit format ([pg] 3.4 "16 Psi baseline"; [bea] section 1 uses bf16).   */
/* ------------------------------------------------------------------------ */

#define ORACLE_F16 1
#define ORACLE_BF16 2

typedef struct {
    int p;           /* significand bits including the implicit one */
    int emin;        /* exponent of the smallest normal number */
    int emax;        /* exponent of the largest finite number */
    int ebias;       /* exponent bias */
    uint16_t inf;    /* bits of +infinity */
    uint16_t qnan;   /* bits of the quiet NaN returned for NaN input */
} fmt16;

static const fmt16 FMT_F16 = {11, -14, 15, 15, 0x7C00u, 0x7E00u};
static const fmt16 FMT_BF16 = {8, -126, 127, 127, 0x7F80u, 0x7FC0u};

static const fmt16 *fmt_of(int dtype) { return dtype == ORACLE_BF16 ? &FMT_BF16 : &FMT_F16; }

/* 2^k as a binary64, built from its encoding (exact for -1022 <= k <= 1023). */
static double pow2i(int k) {
    uint64_t b = (uint64_t)(k + 1023) << 52;
    double d;
    memcpy(&d, &b, 8);
    return d;
}

/* floor(log2 x) of a positive normal binary64 (its unbiased exponent field). */
static int exponent_of(double x) {
    uint64_t b;
    memcpy(&b, &x, 8);
    return (int)((b >> 52) & 0x7FF) - 1023;
}

/* 16-bit pattern -> value.  Normal: (-1)^s 2^(e-bias) (1 + frac/2^(p-1));
 * subnormal (e == 0): (-1)^s 2^emin (frac/2^(p-1)).  Exact in binary32. */
float oracle_to_f32(uint16_t h, int32_t dtype) {
    const fmt16 *F = fmt_of(dtype);
    int fb = F->p - 1;
    int emax_field = (1 << (15 - fb)) - 1;
    int s = h >> 15;
    int e = (h >> fb) & emax_field;
    int f = h & ((1 << fb) - 1);
    double mag;
    if (e == emax_field) {
        if (f != 0) return copysignf(NAN, s ? -1.0f : 1.0f);
        return s ? -INFINITY : INFINITY;
    }
    if (e == 0)
        mag = (double)f * pow2i(F->emin - fb);
    else
        mag = (double)((1 << fb) + f) * pow2i(e - F->ebias - fb);
    return (float)(s ? -mag : mag);
}

/* binary32 -> 16-bit pattern, round to nearest, ties to even.
 * x = |v| is exact in binary64.  With E = max(floor(log2 x), emin), the
 * representable numbers near x are r * 2^(E-(p-1)) for integers r; the
 * result is the nearest such r (ties to the even r), re-normalised when r
 * reaches 2^p, infinite when its exponent passes emax. */
uint16_t oracle_from_f32(float v, int32_t dtype) {
    const fmt16 *F = fmt_of(dtype);
    int fb = F->p - 1;
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return (uint16_t)(sign | F->qnan);
    if (isinf(v)) return (uint16_t)(sign | F->inf);
    double x = fabs((double)v);
    if (x == 0.0) return sign;
    int E = exponent_of(x);
    if (E < F->emin) E = F->emin;
    double q = x * pow2i(fb - E);     /* exact: a power-of-two scaling, q < 2^p */
    int64_t r = (int64_t)q;           /* floor, q >= 0 */
    double frac = q - (double)r;      /* exact */
    if (frac > 0.5 || (frac == 0.5 && (r & 1) != 0)) r += 1;
    if (r == ((int64_t)1 << F->p)) {  /* rounded up into the next binade */
        r >>= 1;
        E += 1;
    }
    if (E > F->emax) return (uint16_t)(sign | F->inf);
    if (r < ((int64_t)1 << fb))       /* subnormal (E == emin) or zero */
        return (uint16_t)(sign | (uint16_t)r);
    return (uint16_t)(sign | ((uint32_t)(E + F->ebias) << fb) | (uint32_t)(r - ((int64_t)1 << fb)));
}

void oracle_to_f32_array(const uint16_t *h, int64_t n, int32_t dtype, float *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_to_f32(h[i], dtype);
}

void oracle_from_f32_array(const float *v, int64_t n, int32_t dtype, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_from_f32(v[i], dtype);
}

/* Bit patterns b = b0 .. b0+n-1 read as binary32, converted (exhaustive tests). */
void oracle_from_f32_bits_range(uint32_t b0, int64_t n, int32_t dtype, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) {
        uint32_t b = b0 + (uint32_t)i;
        float v;
        memcpy(&v, &b, 4);
        out[i] = oracle_from_f32(v, dtype);
    }
}

/* ------------------------------------------------------------------------ */
/* Partition.  The flat buffer is cut into N contiguous pieces of (almost)    */
/* the same length, piece r belonging to rank r ([sim] partitioning          */
/* paragraph; [pg] 3.4 Stage 1; [grasp] Stage 1 step 3).                      */
/* Equal ceil(Psi/N) chunks, so the tail ranks are short or empty.            */
/* ------------------------------------------------------------------------ */
int oracle_partition(int64_t psi, int32_t nranks, int32_t rank, int64_t *shard, int64_t *offset,
                     int64_t *valid) {
    if (psi < 1 || nranks < 1 || rank < 0 || rank >= nranks) return -1;
    int64_t s = psi / nranks + (psi % nranks != 0 ? 1 : 0);
    int64_t off = (int64_t)rank * s;
    int64_t rem = psi - off;
    *shard = s;
    *offset = off;
    *valid = rem < 0 ? 0 : (rem > s ? s : rem);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Reduce.  The reduce-scatter sums the N ranks' gradients for the owned slice */
/* and averages them, delivering fp32 ([cmu] Mechanism 1 step 3; [sim] data-  */
/* flow table, gradient-sync column; [pg] 3.4 Stage 2).  Sum in fp32 in rank  */
/* order k = 0..N-1; overflow is tested on the sum; then multiply by           */
/* inv = fl32(1 / (N * S)), which removes the loss scale S and averages.       */
/* C is laid out [n][stride] (16-bit patterns); only columns < len are read.   */
/* ------------------------------------------------------------------------ */
float oracle_inv_scale(int32_t nranks, float loss_scale) {
    return (float)(1.0 / ((double)nranks * (double)loss_scale));
}

void oracle_reduce(const uint16_t *C, int32_t dtype, int32_t n, int64_t stride, int64_t len,
                   float inv, float *g, int32_t *nonfinite) {
    int32_t flag = 0;
    for (int64_t i = 0; i < len; ++i) {
        float acc = 0.0f;
        for (int32_t k = 0; k < n; ++k) acc = acc + oracle_to_f32(C[(int64_t)k * stride + i], dtype);
        if (!isfinite(acc)) flag = 1;
        g[i] = acc * inv;
    }
    *nonfinite = flag;
}

/* ------------------------------------------------------------------------ */
/* Squared L2 norm of the reduced gradient, exactly.  Gradient-norm           */
/* computation over all gradients ([pg] 3.4 residual states, temporary       */
/* buffers; [cmu] "The memory bill").  Each g is M 2^(e-24) with M < 2^24,    */
/* so g^2 = M^2 2^(2e-48) is an integer below 2^48 placed at bit 2e+296 of a   */
/* 640-bit fixed-point accumulator (least significant bit 2^-344, enough for   */
/* every binary32 square and 2^34 terms).  The sum is therefore independent of */
/* the order and grouping of the terms.  NaN anywhere gives NaN; otherwise an  */
/* infinity gives +inf.                                                        */
/* ------------------------------------------------------------------------ */
#define ORACLE_LIMBS 10

typedef struct {
    uint64_t limb[ORACLE_LIMBS];
    int32_t has_nan;
    int32_t has_inf;
} oracle_sumsq;

static void limbs_add(uint64_t *limb, int li, uint64_t v) {
    for (int j = li; j < ORACLE_LIMBS && v != 0; ++j) {
        uint64_t old = limb[j];
        limb[j] = old + v;
        v = limb[j] < old ? 1u : 0u;
    }
}

void oracle_sumsq_clear(oracle_sumsq *a) { memset(a, 0, sizeof(*a)); }

void oracle_sumsq_add(oracle_sumsq *a, const float *g, int64_t len) {
    for (int64_t i = 0; i < len; ++i) {
        float x = g[i];
        if (isnan(x)) { a->has_nan = 1; continue; }
        if (isinf(x)) { a->has_inf = 1; continue; }
        if (x == 0.0f) continue;
        int e;
        float f = frexpf(fabsf(x), &e);          /* |x| = f 2^e, f in [0.5, 1) */
        uint64_t M = (uint64_t)ldexpf(f, 24);    /* integer in [2^23, 2^24) */
        uint64_t sq = M * M;                     /* exact, below 2^48 */
        int p = 2 * e + 296;                     /* bit position of 2^(2e-48) */
        int li = p >> 6, sh = p & 63;
        limbs_add(a->limb, li, sq << sh);
        if (sh != 0) limbs_add(a->limb, li + 1, sq >> (64 - sh));
    }
}

void oracle_sumsq_merge(oracle_sumsq *dst, const oracle_sumsq *src) {
    for (int j = 0; j < ORACLE_LIMBS; ++j) limbs_add(dst->limb, j, src->limb[j]);
    dst->has_nan |= src->has_nan;
    dst->has_inf |= src->has_inf;
}

/* The accumulated value rounded to binary64: limbs summed from the most
 * significant down in x87 extended precision (64-bit significand, so each limb
 * is exact and the total relative error is far below one binary64 ulp). */
double oracle_sumsq_value(const oracle_sumsq *a) {
    if (a->has_nan) return NAN;
    if (a->has_inf) return INFINITY;
    long double s = 0.0L;
    for (int j = ORACLE_LIMBS - 1; j >= 0; --j) s += ldexpl((long double)a->limb[j], 64 * j - 344);
    return (double)s;
}

/* ------------------------------------------------------------------------ */
/* Scalar decisions after the reduction.                                       */
/* The pages name the gradient-norm computation but give no skip, loss-scale   */
/* or clipping rule; mixed precision is cited to Micikevicius et al. ([pg] 3.4 */
/* "16 Psi baseline").  Readings taken: a step whose reduced gradient holds    */
/* inf/NaN is skipped (parameters, moments and step count unchanged); the      */
/* dynamic scaler halves S (not below min_scale) on a skipped step and, after  */
/* growth_interval consecutive finite steps, doubles it unless the doubled     */
/* value is not finite (then S stays; the run count restarts either way);      */
/* unlike PyTorch's scaler, S never drops below min_scale;                     */
/* clipping multiplies g by min(1, max/(norm + 1e-6)), the coefficient formed  */
/* in binary64 and rounded once to binary32.  The bias-correction powers       */
/* beta^t are running binary64 products, one factor per applied step.          */
/* ------------------------------------------------------------------------ */
typedef struct {
    float lr, beta1, beta2, eps, weight_decay, max_grad_norm;
    int32_t scaler; /* 0: none (S = 1), 1: static, 2: dynamic */
    float min_scale;
    int32_t growth_interval;
} oracle_hparams;

typedef struct {
    double pow1, pow2; /* beta1^t, beta2^t */
    float scale;       /* loss scale S for the next step */
    int32_t good;      /* consecutive finite steps since the last change of S */
    int32_t t;         /* applied optimizer steps */
    int32_t pad;
} oracle_scalars;

typedef struct {
    double sumsq, norm;
    float scale_used, clip;
    int32_t nonfinite, skip;
} oracle_report;

void oracle_scalars_init(oracle_scalars *st, float loss_scale) {
    st->pow1 = 1.0;
    st->pow2 = 1.0;
    st->scale = loss_scale;
    st->good = 0;
    st->t = 0;
    st->pad = 0;
}

void oracle_finalize(const oracle_hparams *hp, oracle_scalars *st, int32_t nonfinite,
                     const oracle_sumsq *acc, oracle_report *rep) {
    rep->nonfinite = nonfinite ? 1 : 0;
    rep->sumsq = oracle_sumsq_value(acc);
    rep->norm = sqrt(rep->sumsq);
    rep->scale_used = st->scale;
    rep->skip = rep->nonfinite;
    rep->clip = 1.0f;
    if (hp->scaler == 2) {
        if (rep->skip) {
            float half = st->scale * 0.5f;
            st->scale = half > hp->min_scale ? half : hp->min_scale;
            st->good = 0;
        } else {
            st->good += 1;
            if (st->good == hp->growth_interval) {
                float twice = st->scale * 2.0f;
                if (isfinite(twice)) st->scale = twice;
                st->good = 0;
            }
        }
    }
    if (!rep->skip) {
        if (hp->max_grad_norm > 0.0f) {
            double coef = (double)hp->max_grad_norm / (rep->norm + 1e-6);
            if (coef < 1.0) rep->clip = (float)coef;
        }
        st->t += 1;
        st->pow1 = st->pow1 * (double)hp->beta1;
        st->pow2 = st->pow2 * (double)hp->beta2;
    }
}

/* ------------------------------------------------------------------------ */
/* Adam on the owned slice: the rank's fp32 master weights and both moments    */
/* are the only optimizer state it touches ([cmu] Mechanism 1 step 4; [pg] 3.4 */
/* Stage 1; [grasp] Stage 1 step 3).  The pages cite Kingma and Ba and name    */
/* AdamW with weight_decay ([bea] section 5) without printing the update, so   */
/* the textbook bias-corrected form is used, epsilon outside the square root,  */
/* decoupled weight decay on the pre-update parameter.  st->pow1/pow2 hold     */
/* beta^t for the step being applied.  Every operation is binary32.            */
/* ------------------------------------------------------------------------ */
void oracle_adam(float *p, float *m, float *v, const float *g, int64_t len,
                 const oracle_hparams *hp, float clip, double pow1, double pow2) {
    const float b1 = hp->beta1, b2 = hp->beta2;
    const float omb1 = 1.0f - b1, omb2 = 1.0f - b2;
    const float bc1 = (float)(1.0 - pow1), bc2 = (float)(1.0 - pow2);
    const float lr = hp->lr, eps = hp->eps, wd = hp->weight_decay;
    for (int64_t i = 0; i < len; ++i) {
        float gi = g[i] * clip;
        float mi = b1 * m[i] + omb1 * gi;
        float vi = b2 * v[i] + omb2 * (gi * gi);
        float mhat = mi / bc1;
        float vhat = vi / bc2;
        float u = mhat / (sqrtf(vhat) + eps);
        p[i] = p[i] - lr * (u + wd * p[i]);
        m[i] = mi;
        v[i] = vi;
    }
}

/* ------------------------------------------------------------------------ */
/* Cast.  The new master weights, rounded to the 16-bit format, go into the   */
/* rank's slot of the full parameter buffer that the all-gather fills ([cmu]   */
/* Mechanism 1 steps 5-6; [grasp] Stage 1 step 4).                              */
/* ------------------------------------------------------------------------ */
void oracle_cast(const float *p, int64_t len, int32_t dtype, uint16_t *out) {
    for (int64_t i = 0; i < len; ++i) out[i] = oracle_from_f32(p[i], dtype);
}

/* ------------------------------------------------------------------------ */
/* Block quantisation (ZeRO++).  [cmu] "Other memory optimizations" names     */
/* ZeRO++'s quantised communication: parameters block-wise from 16 bits to    */
/* INT8 with a zero point for the forward all-gather, and the gradient         */
/* reduce-scatter in INT8 or INT4.  The page fixes neither block size nor      */
/* rounding; the reading taken here:                                          */
/*   blocks of ORACLE_QBLOCK = 2048 consecutive elements from the start of    */
/*   the buffer (the last one may be short); Q = 2^bits - 1;                   */
/*   a block holding a non-finite value gets scale NaN, zero 0, codes 0, so   */
/*   every element of it dequantises to NaN and an overflow check downstream  */
/*   still fires;                                                             */
/*   otherwise, the affine (zero-point) mapping whose range contains 0:       */
/*     lo = min(0, min x), hi = max(0, max x)           (exact)               */
/*     S  = (hi - lo) / Q, replaced by 1 when it is 0   (fp32, rounded)       */
/*     Z  = clamp(rint(-lo / S), 0, Q)                  (integer)             */
/*     q  = clamp(rint(x * fl32(1 / S)) + Z, 0, Q)      (integer)             */
/*     x' = S * (q - Z)                                 (fp32, rounded once)  */
/*   a block whose S overflows counts as non-finite;                           */
/*   rint rounds half to even; INT4 codes are packed two to a byte, the       */
/*   element with the even index in the low nibble.                            */
/* For finite blocks whose S is at least fp32's epsilon this is PyTorch's    */
/* per-tensor affine quantisation of the block (MinMaxObserver's scale and   */
/* zero point, quantize_per_tensor's codes, quint4x2's packing, dequantize); */
/* torch floors S at epsilon where this reading takes S = 1 for an empty     */
/* range, and has no NaN convention.                                          */
/* Real zero maps to Z and back to exactly 0; |x - x'| <= S/2 up to the       */
/* fp32 roundings.                                                            */
/* ------------------------------------------------------------------------ */
#define ORACLE_QBLOCK 2048

int64_t oracle_qblock(void) { return ORACLE_QBLOCK; }

static float q_clamp_code(float r, float qmax) { return r < 0.0f ? 0.0f : (r > qmax ? qmax : r); }

void oracle_quantize(const uint16_t *src, int32_t dtype, int64_t len, int32_t bits, uint8_t *codes,
                     float *scale, int32_t *zero) {
    const float qmax = (float)((1 << bits) - 1);
    const int64_t nblk = (len + ORACLE_QBLOCK - 1) / ORACLE_QBLOCK;
    const int64_t ncode_bytes = bits == 8 ? len : (len + 1) / 2;
    for (int64_t i = 0; i < ncode_bytes; ++i) codes[i] = 0;
    for (int64_t b = 0; b < nblk; ++b) {
        const int64_t i0 = b * ORACLE_QBLOCK;
        const int64_t i1 = i0 + ORACLE_QBLOCK < len ? i0 + ORACLE_QBLOCK : len;
        float lo = 0.0f, hi = 0.0f;
        int finite = 1;
        for (int64_t i = i0; i < i1; ++i) {
            const float x = oracle_to_f32(src[i], dtype);
            if (!isfinite(x)) finite = 0;
            else {
                if (x < lo) lo = x;
                if (x > hi) hi = x;
            }
        }
        float s = (hi - lo) / qmax;
        if (finite && !isfinite(s)) finite = 0;
        if (!finite) {
            scale[b] = NAN;
            zero[b] = 0;
            continue;  /* codes stay 0 */
        }
        if (s == 0.0f) s = 1.0f;
        const float z = q_clamp_code(rintf(-lo / s), qmax);
        const float inv = 1.0f / s;  /* codes use the reciprocal, as torch's quantizer does */
        scale[b] = s;
        zero[b] = (int32_t)z;
        for (int64_t i = i0; i < i1; ++i) {
            const float x = oracle_to_f32(src[i], dtype);
            const uint8_t q = (uint8_t)q_clamp_code(rintf(x * inv) + z, qmax);
            if (bits == 8) codes[i] = q;
            else codes[i / 2] = (uint8_t)(codes[i / 2] | (q << (4 * (i % 2))));
        }
    }
}

/* Code of element i of a quantised buffer. */
static int32_t q_code(const uint8_t *codes, int32_t bits, int64_t i) {
    if (bits == 8) return codes[i];
    return (codes[i / 2] >> (4 * (i % 2))) & 15;
}

/* x'_i = S_b * (q_i - Z_b), b = i / 2048, in fp32. */
void oracle_dequantize(const uint8_t *codes, const float *scale, const int32_t *zero, int32_t bits,
                       int64_t len, float *out) {
    for (int64_t i = 0; i < len; ++i) {
        const int64_t b = i / ORACLE_QBLOCK;
        out[i] = scale[b] * (float)(q_code(codes, bits, i) - zero[b]);
    }
}

/* The reduce of Reduce above over quantised contributions: row k is given as */
/* codes[k] with per-block scale[k] and zero[k]; each value is dequantised    */
/* as in oracle_dequantize, then summed in fp32 in rank order; the overflow   */
/* test and the multiplication by inv are unchanged.                          */
void oracle_reduce_q(const uint8_t *const *codes, const float *const *scale,
                     const int32_t *const *zero, int32_t bits, int32_t n, int64_t len, float inv,
                     float *g, int32_t *nonfinite) {
    int32_t flag = 0;
    for (int64_t i = 0; i < len; ++i) {
        const int64_t b = i / ORACLE_QBLOCK;
        float acc = 0.0f;
        for (int32_t k = 0; k < n; ++k)
            acc = acc + scale[k][b] * (float)(q_code(codes[k], bits, i) - zero[k][b]);
        if (!isfinite(acc)) flag = 1;
        g[i] = acc * inv;
    }
    *nonfinite = flag;
}
