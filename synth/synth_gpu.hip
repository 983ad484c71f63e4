// Device build of the synthetic-input generator (definitions in synth_core.h),
// plus a plain 16-byte copy kernel used to calibrate HBM byte counters and to
// give a reachable-bandwidth reference line.  Test and bench infrastructure:
// the shard-step library does not link against it.
#include <hip/hip_runtime.h>

#define SYNTH_FN __host__ __device__ static inline
#include "synth_core.h"

namespace {

constexpr int kBlock = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kBlock)
contrib_rows_kernel(uint64_t seed, uint32_t step, int32_t dtype, double sigma, double scale,
                    uint64_t thresh, double mult, int64_t idx0, int64_t len, int64_t stride,
                    uint16_t* out) {
    const uint32_t k = blockIdx.y;
    const uint64_t kc = synth_stream_key(seed, SYNTH_STREAM_CONTRIB, step, k);
    const uint64_t ko = synth_stream_key(seed, SYNTH_STREAM_OUTLIER, step, k);
    uint16_t* row = out + (int64_t)k * stride;
    const int64_t nvec = stride / 8;  // stride is a multiple of 8 (checked on the host)
    for (int64_t v = (int64_t)blockIdx.x * kBlock + threadIdx.x; v < nvec;
         v += (int64_t)gridDim.x * kBlock) {
        uint16_t h[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t i = v * 8 + j;
            h[j] = i < len ? synth_contrib_value(kc, ko, thresh, sigma, scale, mult, dtype,
                                                 (uint64_t)(idx0 + i))
                           : (uint16_t)0;
        }
        uint4 w;
        w.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
        w.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
        w.z = (uint32_t)h[4] | ((uint32_t)h[5] << 16);
        w.w = (uint32_t)h[6] | ((uint32_t)h[7] << 16);
        *reinterpret_cast<uint4*>(row + v * 8) = w;
    }
}

__global__ void __launch_bounds__(kBlock)
master_range_kernel(uint64_t seed, double sigma, int64_t idx0, int64_t len, float* out) {
    const uint64_t km = synth_stream_key(seed, SYNTH_STREAM_MASTER, 0u, 0u);
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < len;
         i += (int64_t)gridDim.x * kBlock)
        out[i] = synth_master_value(km, sigma, (uint64_t)(idx0 + i));
}

__global__ void __launch_bounds__(kBlock)
param_range_kernel(uint64_t seed, double sigma, int32_t dtype, int64_t idx0, int64_t len,
                   uint16_t* out) {
    const uint64_t km = synth_stream_key(seed, SYNTH_STREAM_MASTER, 0u, 0u);
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < len;
         i += (int64_t)gridDim.x * kBlock) {
        const float f = synth_master_value(km, sigma, (uint64_t)(idx0 + i));
        out[i] = dtype == SYNTH_BF16 ? synth_f32_to_bf16(f) : synth_f32_to_f16(f);
    }
}

// One 16-byte vector per thread over a grid covering the buffer (the
// fastest plain copy measured on MI355X).
__global__ void __launch_bounds__(kBlock)
copy16_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t nvec) {
    const int64_t v = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (v < nvec) __builtin_nontemporal_store(__builtin_nontemporal_load(src + v), dst + v);
}

// Plain streams for the benchmark's reference lines.  Each workgroup moves
// 8 KiB of every array it touches (256 threads, two 16-byte vectors each,
// every wave instruction one contiguous 4 KiB span); kind 0 reads a, 1 writes
// d, 2 copies a to d, 3 writes d = a + b (two bytes read per byte written,
// the read:write mix of the fused shard step), 4 writes d = a + a' + b + b'
// where a' and b' are a and b one stream length further on (four bytes read
// per byte written, the mix of the reduce pass).
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int64_t stream_base() {
    return (int64_t)blockIdx.x * 2048 + threadIdx.x * 4;  // floats
}

__global__ void __launch_bounds__(kBlock) stream_read_kernel(const float* __restrict__ a,
                                                             float* __restrict__ d) {
    const int64_t i = stream_base();
    const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a + i));
    const f32x4 y = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a + i + 1024));
    const float s = x.x + x.y + x.z + x.w + y.x + y.y + y.z + y.w;
    if (s == -1.5e38f) d[threadIdx.x] = s;  // keeps the loads; not met by finite data
}

__global__ void __launch_bounds__(kBlock) stream_write_kernel(float* __restrict__ d) {
    const int64_t i = stream_base();
    const f32x4 v = {1.0f, 2.0f, 3.0f, 4.0f};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(d + i));
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(d + i + 1024));
}

__global__ void __launch_bounds__(kBlock) stream_copy_kernel(const float* __restrict__ a,
                                                             float* __restrict__ d) {
    const int64_t i = stream_base();
    const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a + i));
    const f32x4 y = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a + i + 1024));
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(d + i));
    __builtin_nontemporal_store(y, reinterpret_cast<f32x4*>(d + i + 1024));
}

__global__ void __launch_bounds__(kBlock) stream_mix_kernel(const float* __restrict__ a,
                                                            const float* __restrict__ b,
                                                            float* __restrict__ d) {
    const int64_t i = stream_base();
    const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a + i));
    const f32x4 y = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a + i + 1024));
    const f32x4 u = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(b + i));
    const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(b + i + 1024));
    __builtin_nontemporal_store(x + u, reinterpret_cast<f32x4*>(d + i));
    __builtin_nontemporal_store(y + w, reinterpret_cast<f32x4*>(d + i + 1024));
}

__global__ void __launch_bounds__(kBlock) stream_mix4_kernel(const float* __restrict__ a,
                                                             const float* __restrict__ b,
                                                             float* __restrict__ d, int64_t far) {
    const int64_t i = stream_base();
    f32x4 s[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t j = i + h * 1024;
        const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a + j));
        const f32x4 y = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a + far + j));
        const f32x4 u = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(b + j));
        const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(b + far + j));
        s[h] = (x + y) + (u + w);
    }
    __builtin_nontemporal_store(s[0], reinterpret_cast<f32x4*>(d + i));
    __builtin_nontemporal_store(s[1], reinterpret_cast<f32x4*>(d + i + 1024));
}

unsigned grid_for(int64_t work, int64_t per_block) {
    int64_t g = (work + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > 65536) g = 65536;
    return (unsigned)g;
}

int status(hipError_t e) { return e == hipSuccess ? 0 : -(int)e - 1000; }

}  // namespace

extern "C" {

// Contribution rows k = 0..n-1 of global elements [idx0, idx0+len) into a
// device buffer laid out [n][stride] (16-bit storage); columns [len, stride)
// are zero.  stride must be a multiple of 8 and `out` 16-byte aligned.
int synth_gpu_contrib_rows(uint64_t seed, uint32_t step, int32_t n, int32_t dtype, double sigma,
                           double scale, uint64_t outlier_thresh, double outlier_mult, int64_t idx0,
                           int64_t len, int64_t stride, void* out, void* stream) {
    if (n < 1 || n > 65535 || stride % 8 != 0 || len > stride || len < 0 || out == nullptr ||
        (reinterpret_cast<uintptr_t>(out) & 15u) != 0)
        return -1;
    if (stride == 0) return 0;
    dim3 grid(grid_for(stride / 8, kBlock), (unsigned)n);
    hipLaunchKernelGGL(contrib_rows_kernel, grid, dim3(kBlock), 0, (hipStream_t)stream, seed, step,
                       dtype, sigma, scale, outlier_thresh, outlier_mult, idx0, len, stride,
                       (uint16_t*)out);
    return status(hipGetLastError());
}

int synth_gpu_master_range(uint64_t seed, double sigma, int64_t idx0, int64_t len, float* out,
                           void* stream) {
    if (len < 0 || (len > 0 && out == nullptr)) return -1;
    if (len == 0) return 0;
    hipLaunchKernelGGL(master_range_kernel, dim3(grid_for(len, kBlock)), dim3(kBlock), 0,
                       (hipStream_t)stream, seed, sigma, idx0, len, out);
    return status(hipGetLastError());
}

// Initial 16-bit parameters: the generator's master values rounded to dtype.
int synth_gpu_param_range(uint64_t seed, double sigma, int32_t dtype, int64_t idx0, int64_t len,
                          void* out, void* stream) {
    if (len < 0 || (len > 0 && out == nullptr)) return -1;
    if (len == 0) return 0;
    hipLaunchKernelGGL(param_range_kernel, dim3(grid_for(len, kBlock)), dim3(kBlock), 0,
                       (hipStream_t)stream, seed, sigma, dtype, idx0, len, (uint16_t*)out);
    return status(hipGetLastError());
}

// Plain streaming copy of `bytes` (multiple of 16, both pointers 16-byte aligned);
// `grid` is ignored (kept for the call's signature).
int synth_gpu_copy(const void* src, void* dst, int64_t bytes, int32_t grid, void* stream) {
    if (bytes < 0 || bytes % 16 != 0 || src == nullptr || dst == nullptr ||
        ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) != 0)
        return -1;
    if (bytes == 0) return 0;
    const int64_t nvec = bytes / 16;
    const int64_t blocks = (nvec + kBlock - 1) / kBlock;
    if (blocks > 0x7FFFFFFF) return -1;
    (void)grid;
    hipLaunchKernelGGL(copy16_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, (hipStream_t)stream,
                       (const u32x4*)src, (u32x4*)dst, nvec);
    return status(hipGetLastError());
}

// One plain stream (kind as above) over `bytes` of each array (a multiple of
// 8 KiB; pointers 16-byte aligned; d at least 1 KiB for kind 0; for kind 4, a
// and b hold 2 * bytes each), issued as launches of at most `chunk`
// workgroups, each reserving `lds` bytes of LDS (which sets how many are
// resident per CU).
int synth_gpu_stream(int32_t kind, const void* a, const void* b, void* d, int64_t bytes,
                     int64_t chunk, uint32_t lds, void* stream) {
    if (kind < 0 || kind > 4 || bytes < 0 || bytes % 8192 != 0 || chunk < 1 || lds > 65536)
        return -1;
    if (((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) |
          reinterpret_cast<uintptr_t>(d)) & 15u) != 0)
        return -1;
    if ((kind != 1 && a == nullptr) || (kind >= 3 && b == nullptr) || d == nullptr) return -1;
    const int64_t wgs = bytes / 8192;
    hipStream_t s = (hipStream_t)stream;
    for (int64_t w0 = 0; w0 < wgs; w0 += chunk) {
        const int64_t g = wgs - w0 < chunk ? wgs - w0 : chunk;
        const int64_t off = w0 * 2048;  // floats
        const float* pa = (const float*)a + (kind != 1 ? off : 0);
        const float* pb = (const float*)b + (kind >= 3 ? off : 0);
        float* pd = (float*)d + (kind != 0 ? off : 0);
        switch (kind) {
            case 0: hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)g), dim3(kBlock), lds, s, pa, pd); break;
            case 1: hipLaunchKernelGGL(stream_write_kernel, dim3((unsigned)g), dim3(kBlock), lds, s, pd); break;
            case 2: hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)g), dim3(kBlock), lds, s, pa, pd); break;
            case 3: hipLaunchKernelGGL(stream_mix_kernel, dim3((unsigned)g), dim3(kBlock), lds, s, pa, pb, pd); break;
            default: hipLaunchKernelGGL(stream_mix4_kernel, dim3((unsigned)g), dim3(kBlock), lds, s, pa, pb, pd, bytes / 4); break;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return status(e);
    }
    return 0;
}

// Device facts for the benchmark's peak figures: peak memory clock (kHz),
// memory bus width (bits), compute units and peak shader clock (kHz).
int synth_gpu_device_info(int32_t device, int32_t* mem_clock_khz, int32_t* bus_bits, int32_t* cus,
                          int32_t* clock_khz) {
    if (!mem_clock_khz || !bus_bits || !cus || !clock_khz) return -1;
    hipError_t e;
    if ((e = hipDeviceGetAttribute(mem_clock_khz, hipDeviceAttributeMemoryClockRate, device)) != hipSuccess)
        return status(e);
    if ((e = hipDeviceGetAttribute(bus_bits, hipDeviceAttributeMemoryBusWidth, device)) != hipSuccess)
        return status(e);
    if ((e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, device)) != hipSuccess)
        return status(e);
    return status(hipDeviceGetAttribute(clock_khz, hipDeviceAttributeClockRate, device));
}

}  // extern "C"
