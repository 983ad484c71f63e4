// Kernels and C ABI of the ZeRO per-rank shard step, written for gfx950 (MI355X).
//
// Every kernel here streams HBM: the work per element is a handful of fp32
// operations against 26 + 2N bytes, so nothing is a contraction and nothing
// uses the matrix cores.  The design points are
//   * 16-byte vector loads/stores (8 sixteen-bit or 4 fp32 values per access)
//     with non-temporal hints: every byte is touched once per step, so it
//     should not displace anything in L2 or the Infinity Cache;
//   * a grid of at most kMaxParts workgroups of 4 waves looping over the
//     shard (grid-stride), so each workgroup leaves exactly one 16-byte
//     partial of the norm reduction and the second level is a single small
//     workgroup;
//   * fp32 reduction in rank order k = 0..N-1 and each Adam operation rounded
//     once in the written order (compiled with -ffp-contract=off, correctly
//     rounded division and square root), so results are reproducible and
//     agree with a scalar reference operation for operation;
//   * the squared norm accumulated in fp64 per lane, reduced per wave with
//     cross-lane shuffles, per workgroup through LDS, then across workgroups
//     in a fixed order: deterministic and far inside the clip tolerance;
//   * all step-to-step scalars (loss scale, t, beta powers, skip, clip, the
//     current state set) live in a device control block, so a step never
//     waits for the host.
// Sources: see include/zero_shard.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "zero_shard.h"

namespace {

constexpr int kBlock = 256;           // threads per workgroup: 4 wave64s
constexpr int kWaves = kBlock / 64;
constexpr int kVec = 8;               // elements per thread per iteration
constexpr int64_t kMaxParts = 2048;   // workgroups of a streaming pass (8 per CU)
constexpr int64_t kMaxLen = int64_t(1) << 40;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Partial {
    double sumsq;
    uint32_t nonfinite;
    uint32_t pad;
};
static_assert(sizeof(Partial) == 16, "partial layout");
static_assert(sizeof(zero_ctrl) == 64, "ctrl layout");

int64_t parts_for(int64_t len) {
    if (len <= 0) return 0;
    int64_t nvec = (len + kVec - 1) / kVec;
    int64_t g = (nvec + kBlock - 1) / kBlock;
    return g > kMaxParts ? kMaxParts : g;
}

// ---------------------------------------------------------------- conversions
template <int DT>
__device__ __forceinline__ float widen_lo(uint32_t w);
template <int DT>
__device__ __forceinline__ float widen_hi(uint32_t w);

template <>
__device__ __forceinline__ float widen_lo<ZERO_F16>(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
template <>
__device__ __forceinline__ float widen_hi<ZERO_F16>(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
template <>
__device__ __forceinline__ float widen_lo<ZERO_BF16>(uint32_t w) {
    return __uint_as_float(w << 16);
}
template <>
__device__ __forceinline__ float widen_hi<ZERO_BF16>(uint32_t w) {
    return __uint_as_float(w & 0xFFFF0000u);
}

template <int DT>
__device__ __forceinline__ float widen1(uint16_t h) {
    return widen_lo<DT>((uint32_t)h);
}

// fp32 -> 16-bit, round to nearest even (hardware conversions).
template <int DT>
__device__ __forceinline__ uint32_t narrow(float x);
template <>
__device__ __forceinline__ uint32_t narrow<ZERO_F16>(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}
template <>
__device__ __forceinline__ uint32_t narrow<ZERO_BF16>(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Adds contribution word vector w (8 sixteen-bit values) into acc[0..7].
template <int DT>
__device__ __forceinline__ void add8(float acc[kVec], u32x4 w) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        acc[2 * j] = acc[2 * j] + widen_lo<DT>(w[j]);
        acc[2 * j + 1] = acc[2 * j + 1] + widen_hi<DT>(w[j]);
    }
}

// acc[j] = sum over rows k = 0..n-1, in that order, of element j of the
// 8-element group at p + k*stride.  Loads are issued eight rows at a time.
template <int DT>
__device__ __forceinline__ void sum_rows(const uint16_t* __restrict__ p, int n, int64_t stride,
                                         float acc[kVec]) {
#pragma unroll
    for (int j = 0; j < kVec; ++j) acc[j] = 0.0f;
    int k = 0;
    for (; k + 8 <= n; k += 8) {
        u32x4 w[8];
#pragma unroll
        for (int r = 0; r < 8; ++r)
            w[r] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(p + (int64_t)(k + r) * stride));
#pragma unroll
        for (int r = 0; r < 8; ++r) add8<DT>(acc, w[r]);
    }
    for (; k < n; ++k)
        add8<DT>(acc, __builtin_nontemporal_load(
                          reinterpret_cast<const u32x4*>(p + (int64_t)k * stride)));
}

template <int DT>
__device__ __forceinline__ float sum_rows1(const uint16_t* __restrict__ p, int n, int64_t stride) {
    float acc = 0.0f;
    for (int k = 0; k < n; ++k) acc = acc + widen1<DT>(p[(int64_t)k * stride]);
    return acc;
}

// ---------------------------------------------------------------- Adam element
struct AdamK {
    float b1, b2, omb1, omb2, bc1, bc2, lr, eps, wd;
};

__device__ __forceinline__ AdamK make_adam(const zero_hparams& hp, double pow1, double pow2) {
    AdamK k;
    k.b1 = hp.beta1;
    k.b2 = hp.beta2;
    k.omb1 = 1.0f - hp.beta1;
    k.omb2 = 1.0f - hp.beta2;
    k.bc1 = (float)(1.0 - pow1);
    k.bc2 = (float)(1.0 - pow2);
    k.lr = hp.lr;
    k.eps = hp.eps;
    k.wd = hp.weight_decay;
    return k;
}

// One bias-corrected AdamW update; every operation is one fp32 rounding.
__device__ __forceinline__ void adam_elem(const AdamK& k, float g, float& p, float& m, float& v) {
    const float mi = k.b1 * m + k.omb1 * g;
    const float vi = k.b2 * v + k.omb2 * (g * g);
    const float mhat = mi / k.bc1;
    const float vhat = vi / k.bc2;
    const float u = mhat / (sqrtf(vhat) + k.eps);
    p = p - k.lr * (u + k.wd * p);
    m = mi;
    v = vi;
}

// ---------------------------------------------------------------- vector I/O
__device__ __forceinline__ void load8(const float* __restrict__ p, float x[kVec]) {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void store8(float* __restrict__ p, const float x[kVec]) {
    f32x4 a, b;
    a.x = x[0]; a.y = x[1]; a.z = x[2]; a.w = x[3];
    b.x = x[4]; b.y = x[5]; b.z = x[6]; b.w = x[7];
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(p));
    __builtin_nontemporal_store(b, reinterpret_cast<f32x4*>(p + 4));
}

// Stores 8 sixteen-bit values h[0..7] at dst with accesses of GW elements
// (GW = 8, 4, 2, 1 for 16-, 8-, 4-, 2-byte aligned dst).
template <int GW>
__device__ __forceinline__ void store_h8(uint16_t* __restrict__ dst, const uint32_t h[kVec]) {
    if constexpr (GW == 8) {
        u32x4 w;
        w.x = h[0] | (h[1] << 16);
        w.y = h[2] | (h[3] << 16);
        w.z = h[4] | (h[5] << 16);
        w.w = h[6] | (h[7] << 16);
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(dst));
    } else if constexpr (GW == 4) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            u32x2 w;
            w.x = h[4 * q] | (h[4 * q + 1] << 16);
            w.y = h[4 * q + 2] | (h[4 * q + 3] << 16);
            __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(dst + 4 * q));
        }
    } else if constexpr (GW == 2) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            __builtin_nontemporal_store(h[2 * q] | (h[2 * q + 1] << 16),
                                        reinterpret_cast<uint32_t*>(dst + 2 * q));
    } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) __builtin_nontemporal_store((uint16_t)h[q], dst + q);
    }
}

// ---------------------------------------------------------------- norm partials
// Reduces (sumsq, nonfinite) over the workgroup: cross-lane within each wave,
// then the kWaves wave results in wave order.  Thread 0 gets the result.
__device__ __forceinline__ void block_reduce(double& ss, uint32_t& bad) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        ss += __shfl_xor(ss, off, 64);
        bad |= __shfl_xor(bad, off, 64);
    }
    __shared__ double s_ss[kWaves];
    __shared__ uint32_t s_bad[kWaves];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (lane == 0) {
        s_ss[wave] = ss;
        s_bad[wave] = bad;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        uint32_t b = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            t += s_ss[w];
            b |= s_bad[w];
        }
        ss = t;
        bad = b;
    }
}

__device__ __forceinline__ void write_partial(Partial* __restrict__ ws, double ss, uint32_t bad) {
    block_reduce(ss, bad);
    if (threadIdx.x == 0) {
        Partial p;
        p.sumsq = ss;
        p.nonfinite = bad ? 1u : 0u;
        p.pad = 0u;
        ws[blockIdx.x] = p;
    }
}

// ---------------------------------------------------------------- kernels
__global__ void ctrl_init_kernel(zero_ctrl* __restrict__ c, float loss_scale) {
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        zero_ctrl z;
        z.sumsq = 0.0;
        z.norm = 0.0;
        z.beta1_pow = 1.0;
        z.beta2_pow = 1.0;
        z.loss_scale = loss_scale;
        z.scale_used = loss_scale;
        z.clip = 1.0f;
        z.nonfinite = 0;
        z.skip = 0;
        z.t = 0;
        z.good_steps = 0;
        z.cur = 0;
        *c = z;
    }
}

struct ReduceArgs {
    const uint16_t* contrib;
    int64_t stride;
    int64_t len;
    const zero_ctrl* ctrl;
    float* g;
    Partial* ws;
    int32_t n;
};

// Pass 1 of the two-pass step: g = fl32(sum_k C[k]) * inv, plus partials.
template <int DT>
__global__ void __launch_bounds__(kBlock) reduce_kernel(ReduceArgs a) {
    const float inv = (float)(1.0 / ((double)a.n * (double)a.ctrl->loss_scale));
    double ss = 0.0;
    uint32_t bad = 0;
    const int64_t nvec = a.len / kVec;
    const int64_t gstride = (int64_t)gridDim.x * kBlock;
    const int64_t tid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    for (int64_t vi = tid; vi < nvec; vi += gstride) {
        float acc[kVec], out[kVec];
        sum_rows<DT>(a.contrib + vi * kVec, a.n, a.stride, acc);
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            bad |= __builtin_isfinite(acc[j]) ? 0u : 1u;
            const float gj = acc[j] * inv;
            ss += (double)gj * (double)gj;
            out[j] = gj;
        }
        store8(a.g + vi * kVec, out);
    }
    const int64_t e = nvec * kVec + tid;  // the < 8 tail elements: threads 0.. of workgroup 0
    if (e < a.len) {
        const float acc = sum_rows1<DT>(a.contrib + e, a.n, a.stride);
        bad |= __builtin_isfinite(acc) ? 0u : 1u;
        const float gj = acc * inv;
        ss += (double)gj * (double)gj;
        a.g[e] = gj;
    }
    write_partial(a.ws, ss, bad);
}

struct CombineArgs {
    const Partial* ws[ZERO_MAX_RANKS];
    zero_ctrl* ctrl[ZERO_MAX_RANKS];
    int32_t nparts[ZERO_MAX_RANKS];
    int32_t nranks;
    int32_t pingpong;
    zero_hparams hp;
};

// Second level of the norm/overflow reduction and the step decisions.
__global__ void __launch_bounds__(kBlock) finalize_kernel(CombineArgs a) {
    double ss = 0.0;
    uint32_t bad = 0;
    for (int r = 0; r < a.nranks; ++r) {
        const Partial* __restrict__ w = a.ws[r];
        for (int i = threadIdx.x; i < a.nparts[r]; i += kBlock) {
            ss += w[i].sumsq;
            bad |= w[i].nonfinite;
        }
    }
    block_reduce(ss, bad);
    if (threadIdx.x != 0) return;
    const zero_hparams& hp = a.hp;
    zero_ctrl c = *a.ctrl[0];
    c.sumsq = ss;
    c.norm = sqrt(ss);
    c.nonfinite = bad ? 1 : 0;
    c.skip = c.nonfinite;
    c.scale_used = c.loss_scale;
    c.clip = 1.0f;
    if (hp.scaler == ZERO_SCALER_DYNAMIC) {
        if (c.skip) {
            const float half = c.loss_scale * 0.5f;
            c.loss_scale = half > hp.min_scale ? half : hp.min_scale;
            c.good_steps = 0;
        } else {
            c.good_steps += 1;
            if (c.good_steps == hp.growth_interval) {
                c.loss_scale = c.loss_scale * 2.0f;
                c.good_steps = 0;
            }
        }
    }
    if (!c.skip) {
        if (hp.max_grad_norm > 0.0f && c.norm > (double)hp.max_grad_norm)
            c.clip = (float)((double)hp.max_grad_norm / (c.norm + 1e-6));
        c.t += 1;
        c.beta1_pow = c.beta1_pow * (double)hp.beta1;
        c.beta2_pow = c.beta2_pow * (double)hp.beta2;
        if (a.pingpong) c.cur ^= 1;
    }
    for (int r = 0; r < a.nranks; ++r) *a.ctrl[r] = c;
}

struct AdamArgs {
    float* master;
    float* m;
    float* v;
    const float* g;
    uint16_t* slot;  // gather + offset, or null
    int64_t len;
    const zero_ctrl* ctrl;
    zero_hparams hp;
};

// Pass 2 of the two-pass step: Adam in place (+ cast into the gather slot).
template <int DT, int GW>
__global__ void __launch_bounds__(kBlock) adam_kernel(AdamArgs a) {
    const zero_ctrl* __restrict__ c = a.ctrl;
    if (c->skip) return;
    const float clip = c->clip;
    const AdamK k = make_adam(a.hp, c->beta1_pow, c->beta2_pow);
    const int64_t nvec = a.len / kVec;
    const int64_t gstride = (int64_t)gridDim.x * kBlock;
    const int64_t tid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    for (int64_t vi = tid; vi < nvec; vi += gstride) {
        const int64_t o = vi * kVec;
        float g[kVec], p[kVec], m[kVec], v[kVec];
        uint32_t h[kVec];
        load8(a.g + o, g);
        load8(a.master + o, p);
        load8(a.m + o, m);
        load8(a.v + o, v);
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            adam_elem(k, g[j] * clip, p[j], m[j], v[j]);
            h[j] = narrow<DT>(p[j]);
        }
        store8(a.master + o, p);
        store8(a.m + o, m);
        store8(a.v + o, v);
        if (GW > 0) store_h8<(GW > 0 ? GW : 1)>(a.slot + o, h);
    }
    const int64_t e = nvec * kVec + tid;
    if (e < a.len) {
        float p = a.master[e], m = a.m[e], v = a.v[e];
        adam_elem(k, a.g[e] * clip, p, m, v);
        a.master[e] = p;
        a.m[e] = m;
        a.v[e] = v;
        if (GW > 0) a.slot[e] = (uint16_t)narrow<DT>(p);
    }
}

struct CastArgs {
    const float* master0;
    const float* master1;
    uint16_t* slot;
    int64_t len;
    const zero_ctrl* ctrl;  // restore only
};

// gather slot <- RNE(master).  RESTORE: only when ctrl->skip, from the
// current set (master0 or master1 as ctrl->cur says).
template <int DT, int GW, bool RESTORE>
__global__ void __launch_bounds__(kBlock) cast_kernel(CastArgs a) {
    const float* __restrict__ src = a.master0;
    if (RESTORE) {
        if (!a.ctrl->skip) return;
        src = a.ctrl->cur ? a.master1 : a.master0;
    }
    const int64_t nvec = a.len / kVec;
    const int64_t gstride = (int64_t)gridDim.x * kBlock;
    const int64_t tid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    for (int64_t vi = tid; vi < nvec; vi += gstride) {
        float p[kVec];
        uint32_t h[kVec];
        load8(src + vi * kVec, p);
#pragma unroll
        for (int j = 0; j < kVec; ++j) h[j] = narrow<DT>(p[j]);
        store_h8<GW>(a.slot + vi * kVec, h);
    }
    const int64_t e = nvec * kVec + tid;
    if (e < a.len) a.slot[e] = (uint16_t)narrow<DT>(src[e]);
}

struct FusedArgs {
    const uint16_t* contrib;
    int64_t stride;
    float* set0[3];  // master, m, v
    float* set1[3];
    uint16_t* slot;
    int64_t len;
    const zero_ctrl* ctrl;
    Partial* ws;
    zero_hparams hp;
    int32_t n;
};

// Single pass: reduce + partials + Adam (read set cur, write set 1-cur) + cast.
template <int DTI, int DTO, int GW>
__global__ void __launch_bounds__(kBlock) fused_kernel(FusedArgs a) {
    const zero_ctrl* __restrict__ c = a.ctrl;
    const int cur = c->cur;
    const float* __restrict__ ps = cur ? a.set1[0] : a.set0[0];
    const float* __restrict__ ms = cur ? a.set1[1] : a.set0[1];
    const float* __restrict__ vs = cur ? a.set1[2] : a.set0[2];
    float* __restrict__ pd = cur ? a.set0[0] : a.set1[0];
    float* __restrict__ md = cur ? a.set0[1] : a.set1[1];
    float* __restrict__ vd = cur ? a.set0[2] : a.set1[2];
    const float inv = (float)(1.0 / ((double)a.n * (double)c->loss_scale));
    const AdamK k = make_adam(a.hp, c->beta1_pow * (double)a.hp.beta1,
                              c->beta2_pow * (double)a.hp.beta2);
    double ss = 0.0;
    uint32_t bad = 0;
    const int64_t nvec = a.len / kVec;
    const int64_t gstride = (int64_t)gridDim.x * kBlock;
    const int64_t tid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    for (int64_t vi = tid; vi < nvec; vi += gstride) {
        const int64_t o = vi * kVec;
        float acc[kVec], p[kVec], m[kVec], v[kVec];
        uint32_t h[kVec];
        load8(ps + o, p);
        load8(ms + o, m);
        load8(vs + o, v);
        sum_rows<DTI>(a.contrib + o, a.n, a.stride, acc);
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            bad |= __builtin_isfinite(acc[j]) ? 0u : 1u;
            const float gj = acc[j] * inv;
            ss += (double)gj * (double)gj;
            adam_elem(k, gj, p[j], m[j], v[j]);
            h[j] = narrow<DTO>(p[j]);
        }
        store8(pd + o, p);
        store8(md + o, m);
        store8(vd + o, v);
        store_h8<GW>(a.slot + o, h);
    }
    const int64_t e = nvec * kVec + tid;
    if (e < a.len) {
        const float acc = sum_rows1<DTI>(a.contrib + e, a.n, a.stride);
        bad |= __builtin_isfinite(acc) ? 0u : 1u;
        const float gj = acc * inv;
        ss += (double)gj * (double)gj;
        float p = ps[e], m = ms[e], v = vs[e];
        adam_elem(k, gj, p, m, v);
        pd[e] = p;
        md[e] = m;
        vd[e] = v;
        a.slot[e] = (uint16_t)narrow<DTO>(p);
    }
    write_partial(a.ws, ss, bad);
}

// ---------------------------------------------------------------- host side
thread_local char g_err[512];

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return ZERO_OK;
}

int launched(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int32_t dt) { return dt == ZERO_F16 || dt == ZERO_BF16; }

// Store width (elements) for a 16-bit destination: 8, 4, 2 or 1.
int store_width(const void* p) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    if ((a & 15u) == 0) return 8;
    if ((a & 7u) == 0) return 4;
    if ((a & 3u) == 0) return 2;
    return 1;
}

int check_hp(const zero_hparams* hp) {
    if (hp == nullptr) return fail(ZERO_EINVAL, "hparams pointer is null");
    if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f && hp->beta2 >= 0.0f && hp->beta2 < 1.0f))
        return fail(ZERO_EINVAL, "betas must lie in [0, 1)");
    if (!(hp->eps >= 0.0f) || !(hp->lr == hp->lr) || !(hp->weight_decay == hp->weight_decay))
        return fail(ZERO_EINVAL, "lr, eps and weight_decay must be numbers (eps >= 0)");
    if (hp->scaler < ZERO_SCALER_NONE || hp->scaler > ZERO_SCALER_DYNAMIC)
        return fail(ZERO_EINVAL, "unknown scaler %d", hp->scaler);
    if (hp->scaler == ZERO_SCALER_DYNAMIC && (hp->growth_interval < 1 || !(hp->min_scale > 0.0f)))
        return fail(ZERO_EINVAL, "dynamic scaler needs growth_interval >= 1 and min_scale > 0");
    return ZERO_OK;
}

int check_contrib(const void* contrib, int32_t dtype, int32_t n, int64_t stride, int64_t len) {
    if (len < 0 || len > kMaxLen) return fail(ZERO_ERANGE, "valid_len %lld out of range", (long long)len);
    if (!valid_dtype(dtype)) return fail(ZERO_EINVAL, "unknown contribution dtype %d", dtype);
    if (n < 1 || n > ZERO_MAX_CONTRIB)
        return fail(ZERO_EINVAL, "nranks %d outside [1, %d]", n, ZERO_MAX_CONTRIB);
    if (stride < len || stride > kMaxLen)
        return fail(ZERO_EINVAL, "stride %lld must be >= valid_len %lld", (long long)stride,
                    (long long)len);
    if (stride % kVec != 0)
        return fail(ZERO_EALIGN, "stride %lld is not a multiple of 8 elements", (long long)stride);
    if (contrib == nullptr) return fail(ZERO_EINVAL, "contribution pointer is null");
    if (!aligned16(contrib)) return fail(ZERO_EALIGN, "contribution buffer not 16-byte aligned");
    return ZERO_OK;
}

int check_state(const zero_state* s, const char* what) {
    if (s == nullptr || s->master == nullptr || s->m == nullptr || s->v == nullptr)
        return fail(ZERO_EINVAL, "%s: null state pointer", what);
    if (!aligned16(s->master) || !aligned16(s->m) || !aligned16(s->v))
        return fail(ZERO_EALIGN, "%s: state arrays must be 16-byte aligned", what);
    return ZERO_OK;
}

int check_ws(const void* ws, size_t ws_bytes, int64_t len) {
    const size_t need = zero_workspace_bytes(len);
    if (ws == nullptr) return fail(ZERO_EINVAL, "workspace pointer is null");
    if (ws_bytes < need)
        return fail(ZERO_ESPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
    if ((reinterpret_cast<uintptr_t>(ws) & 15u) != 0)
        return fail(ZERO_EALIGN, "workspace not 16-byte aligned");
    return ZERO_OK;
}

int check_slot(const void* gather, int32_t dtype, int64_t offset) {
    if (gather == nullptr) return fail(ZERO_EINVAL, "gather pointer is null");
    if (!valid_dtype(dtype)) return fail(ZERO_EINVAL, "unknown gather dtype %d", dtype);
    if (offset < 0 || offset > kMaxLen * 64) return fail(ZERO_ERANGE, "offset %lld out of range", (long long)offset);
    if ((reinterpret_cast<uintptr_t>(gather) & 1u) != 0)
        return fail(ZERO_EALIGN, "gather buffer not 2-byte aligned");
    return ZERO_OK;
}

template <int GW>
void* select_fused_gw(int dti, int dto) {
    if (dti == ZERO_F16 && dto == ZERO_F16) return (void*)fused_kernel<ZERO_F16, ZERO_F16, GW>;
    if (dti == ZERO_F16 && dto == ZERO_BF16) return (void*)fused_kernel<ZERO_F16, ZERO_BF16, GW>;
    if (dti == ZERO_BF16 && dto == ZERO_F16) return (void*)fused_kernel<ZERO_BF16, ZERO_F16, GW>;
    return (void*)fused_kernel<ZERO_BF16, ZERO_BF16, GW>;
}

template <int DT>
void* select_adam_gw(int gw) {
    switch (gw) {
        case 8: return (void*)adam_kernel<DT, 8>;
        case 4: return (void*)adam_kernel<DT, 4>;
        case 2: return (void*)adam_kernel<DT, 2>;
        case 1: return (void*)adam_kernel<DT, 1>;
        default: return (void*)adam_kernel<DT, 0>;
    }
}

template <bool RESTORE, int DT>
void* select_cast_gw(int gw) {
    switch (gw) {
        case 8: return (void*)cast_kernel<DT, 8, RESTORE>;
        case 4: return (void*)cast_kernel<DT, 4, RESTORE>;
        case 2: return (void*)cast_kernel<DT, 2, RESTORE>;
        default: return (void*)cast_kernel<DT, 1, RESTORE>;
    }
}

template <class Args>
int launch(void* kernel, unsigned grid, hipStream_t s, const Args& args, const char* what) {
    void* params[] = {const_cast<Args*>(&args)};
    const hipError_t e = hipLaunchKernel(kernel, dim3(grid), dim3(kBlock), params, 0, s);
    if (e != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return launched(what);
}

}  // namespace

extern "C" {

int zero_partition(int64_t psi, int32_t nranks, int32_t rank, int64_t* shard_len, int64_t* offset,
                   int64_t* valid_len) {
    if (shard_len == nullptr || offset == nullptr || valid_len == nullptr)
        return fail(ZERO_EINVAL, "zero_partition: null output pointer");
    if (psi < 1) return fail(ZERO_EINVAL, "zero_partition: psi must be >= 1");
    if (nranks < 1) return fail(ZERO_EINVAL, "zero_partition: nranks must be >= 1");
    if (rank < 0 || rank >= nranks)
        return fail(ZERO_EINVAL, "zero_partition: rank %d outside [0, %d)", rank, nranks);
    const int64_t shard = psi / nranks + (psi % nranks ? 1 : 0);
    const int64_t off = (int64_t)rank * shard;
    const int64_t rem = psi - off;
    *shard_len = shard;
    *offset = off;
    *valid_len = rem <= 0 ? 0 : (rem < shard ? rem : shard);
    return ok();
}

size_t zero_ctrl_bytes(void) { return sizeof(zero_ctrl); }

size_t zero_workspace_bytes(int64_t valid_len) {
    const int64_t p = parts_for(valid_len);
    return (size_t)(p > 0 ? p : 1) * sizeof(Partial);
}

int zero_ctrl_init(zero_ctrl* ctrl, float loss_scale, void* stream) {
    if (ctrl == nullptr) return fail(ZERO_EINVAL, "zero_ctrl_init: null ctrl");
    if (!(loss_scale > 0.0f) || loss_scale > 3.0e38f)
        return fail(ZERO_EINVAL, "zero_ctrl_init: loss scale must be finite and > 0");
    if ((reinterpret_cast<uintptr_t>(ctrl) & 7u) != 0)
        return fail(ZERO_EALIGN, "zero_ctrl_init: ctrl not 8-byte aligned");
    hipLaunchKernelGGL(ctrl_init_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, ctrl,
                       loss_scale);
    return launched("zero_ctrl_init");
}

int zero_reduce_grads(const void* contrib, int32_t dtype, int32_t nranks, int64_t stride,
                      int64_t valid_len, const zero_ctrl* ctrl, float* g, void* ws,
                      size_t ws_bytes, void* stream) {
    int rc;
    if ((rc = check_contrib(contrib, dtype, nranks, stride, valid_len)) != ZERO_OK) return rc;
    if (ctrl == nullptr || g == nullptr) return fail(ZERO_EINVAL, "zero_reduce_grads: null ctrl or g");
    if (!aligned16(g)) return fail(ZERO_EALIGN, "zero_reduce_grads: g not 16-byte aligned");
    if ((rc = check_ws(ws, ws_bytes, valid_len)) != ZERO_OK) return rc;
    if (valid_len == 0) return ok();
    ReduceArgs a{(const uint16_t*)contrib, stride, valid_len, ctrl, g, (Partial*)ws, nranks};
    void* k = dtype == ZERO_F16 ? (void*)reduce_kernel<ZERO_F16> : (void*)reduce_kernel<ZERO_BF16>;
    return launch(k, (unsigned)parts_for(valid_len), (hipStream_t)stream, a, "zero_reduce_grads");
}

int zero_grad_norm_overflow(int32_t nranks, void* const* ws, const int64_t* valid_len,
                            zero_ctrl* const* ctrl, const zero_hparams* hp, int32_t pingpong,
                            void* stream) {
    int rc;
    if (nranks < 1 || nranks > ZERO_MAX_RANKS)
        return fail(ZERO_EINVAL, "zero_grad_norm_overflow: nranks %d outside [1, %d]", nranks,
                    ZERO_MAX_RANKS);
    if (ws == nullptr || valid_len == nullptr || ctrl == nullptr)
        return fail(ZERO_EINVAL, "zero_grad_norm_overflow: null array");
    if ((rc = check_hp(hp)) != ZERO_OK) return rc;
    CombineArgs a{};
    for (int r = 0; r < nranks; ++r) {
        if (ctrl[r] == nullptr) return fail(ZERO_EINVAL, "zero_grad_norm_overflow: null ctrl[%d]", r);
        if (valid_len[r] < 0 || valid_len[r] > kMaxLen)
            return fail(ZERO_ERANGE, "zero_grad_norm_overflow: valid_len[%d] out of range", r);
        const int64_t np = parts_for(valid_len[r]);
        if (np > 0 && ws[r] == nullptr)
            return fail(ZERO_EINVAL, "zero_grad_norm_overflow: null ws[%d]", r);
        a.ws[r] = (const Partial*)ws[r];
        a.ctrl[r] = ctrl[r];
        a.nparts[r] = (int32_t)np;
    }
    a.nranks = nranks;
    a.pingpong = pingpong ? 1 : 0;
    a.hp = *hp;
    return launch((void*)finalize_kernel, 1u, (hipStream_t)stream, a, "zero_grad_norm_overflow");
}

int zero_adam_step(const zero_state* state, const float* g, int64_t valid_len,
                   const zero_hparams* hp, const zero_ctrl* ctrl, void* gather,
                   int32_t gather_dtype, int64_t offset, void* stream) {
    int rc;
    if (valid_len < 0 || valid_len > kMaxLen) return fail(ZERO_ERANGE, "zero_adam_step: valid_len out of range");
    if ((rc = check_state(state, "zero_adam_step")) != ZERO_OK) return rc;
    if ((rc = check_hp(hp)) != ZERO_OK) return rc;
    if (g == nullptr || ctrl == nullptr) return fail(ZERO_EINVAL, "zero_adam_step: null g or ctrl");
    if (!aligned16(g)) return fail(ZERO_EALIGN, "zero_adam_step: g not 16-byte aligned");
    uint16_t* slot = nullptr;
    int gw = 0;
    if (gather != nullptr) {
        if ((rc = check_slot(gather, gather_dtype, offset)) != ZERO_OK) return rc;
        slot = (uint16_t*)gather + offset;
        gw = store_width(slot);
    }
    if (valid_len == 0) return ok();
    AdamArgs a{state->master, state->m, state->v, g, slot, valid_len, ctrl, *hp};
    void* k = gather_dtype == ZERO_BF16 && gather != nullptr ? select_adam_gw<ZERO_BF16>(gw)
                                                              : select_adam_gw<ZERO_F16>(gw);
    return launch(k, (unsigned)parts_for(valid_len), (hipStream_t)stream, a, "zero_adam_step");
}

int zero_cast_to_gather(const float* master, int64_t valid_len, void* gather, int32_t dtype,
                        int64_t offset, void* stream) {
    int rc;
    if (valid_len < 0 || valid_len > kMaxLen) return fail(ZERO_ERANGE, "zero_cast_to_gather: valid_len out of range");
    if (master == nullptr) return fail(ZERO_EINVAL, "zero_cast_to_gather: null master");
    if (!aligned16(master)) return fail(ZERO_EALIGN, "zero_cast_to_gather: master not 16-byte aligned");
    if ((rc = check_slot(gather, dtype, offset)) != ZERO_OK) return rc;
    if (valid_len == 0) return ok();
    uint16_t* slot = (uint16_t*)gather + offset;
    CastArgs a{master, master, slot, valid_len, nullptr};
    const int gw = store_width(slot);
    void* k = dtype == ZERO_F16 ? select_cast_gw<false, ZERO_F16>(gw) : select_cast_gw<false, ZERO_BF16>(gw);
    return launch(k, (unsigned)parts_for(valid_len), (hipStream_t)stream, a, "zero_cast_to_gather");
}

int zero_fused_step(const void* contrib, int32_t contrib_dtype, int32_t nranks, int64_t stride,
                    const zero_state* state0, const zero_state* state1, int64_t valid_len,
                    void* gather, int32_t gather_dtype, int64_t offset, const zero_hparams* hp,
                    const zero_ctrl* ctrl, void* ws, size_t ws_bytes, void* stream) {
    int rc;
    if ((rc = check_contrib(contrib, contrib_dtype, nranks, stride, valid_len)) != ZERO_OK) return rc;
    if ((rc = check_state(state0, "zero_fused_step state0")) != ZERO_OK) return rc;
    if ((rc = check_state(state1, "zero_fused_step state1")) != ZERO_OK) return rc;
    if (state0->master == state1->master || state0->m == state1->m || state0->v == state1->v)
        return fail(ZERO_EINVAL, "zero_fused_step: the two state sets must be distinct buffers");
    if ((rc = check_hp(hp)) != ZERO_OK) return rc;
    if (hp->max_grad_norm > 0.0f)
        return fail(ZERO_EINVAL, "zero_fused_step: clipping needs the two-pass path");
    if (ctrl == nullptr) return fail(ZERO_EINVAL, "zero_fused_step: null ctrl");
    if ((rc = check_slot(gather, gather_dtype, offset)) != ZERO_OK) return rc;
    if ((rc = check_ws(ws, ws_bytes, valid_len)) != ZERO_OK) return rc;
    if (valid_len == 0) return ok();
    uint16_t* slot = (uint16_t*)gather + offset;
    FusedArgs a{(const uint16_t*)contrib, stride,
                {state0->master, state0->m, state0->v}, {state1->master, state1->m, state1->v},
                slot, valid_len, ctrl, (Partial*)ws, *hp, nranks};
    void* k;
    switch (store_width(slot)) {
        case 8: k = select_fused_gw<8>(contrib_dtype, gather_dtype); break;
        case 4: k = select_fused_gw<4>(contrib_dtype, gather_dtype); break;
        case 2: k = select_fused_gw<2>(contrib_dtype, gather_dtype); break;
        default: k = select_fused_gw<1>(contrib_dtype, gather_dtype); break;
    }
    return launch(k, (unsigned)parts_for(valid_len), (hipStream_t)stream, a, "zero_fused_step");
}

int zero_fused_restore(const zero_state* state0, const zero_state* state1, int64_t valid_len,
                       void* gather, int32_t dtype, int64_t offset, const zero_ctrl* ctrl,
                       void* stream) {
    int rc;
    if (valid_len < 0 || valid_len > kMaxLen) return fail(ZERO_ERANGE, "zero_fused_restore: valid_len out of range");
    if ((rc = check_state(state0, "zero_fused_restore state0")) != ZERO_OK) return rc;
    if ((rc = check_state(state1, "zero_fused_restore state1")) != ZERO_OK) return rc;
    if (ctrl == nullptr) return fail(ZERO_EINVAL, "zero_fused_restore: null ctrl");
    if ((rc = check_slot(gather, dtype, offset)) != ZERO_OK) return rc;
    if (valid_len == 0) return ok();
    uint16_t* slot = (uint16_t*)gather + offset;
    CastArgs a{state0->master, state1->master, slot, valid_len, ctrl};
    const int gw = store_width(slot);
    void* k = dtype == ZERO_F16 ? select_cast_gw<true, ZERO_F16>(gw) : select_cast_gw<true, ZERO_BF16>(gw);
    return launch(k, (unsigned)parts_for(valid_len), (hipStream_t)stream, a, "zero_fused_restore");
}

const char* zero_last_error(void) { return g_err; }

}  // extern "C"
