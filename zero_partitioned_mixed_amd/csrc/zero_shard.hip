// Kernels and C ABI of the ZeRO per-rank shard step, written for gfx950 (MI355X).
//
// Every kernel here streams HBM: the work per element is a handful of fp32
// operations against 26 + 2N bytes, so nothing is a contraction and nothing
// uses the matrix cores.  The design points are
//   * one workgroup per tile of ZERO_TILE = 2048 elements (4 wave64s x 64
//     lanes x 8 elements), launched as full grids of at most 32,768 tiles
//     (2^17 / N over N > 8 contribution rows), with few workgroups resident
//     per CU (two or three, by pass), so that the set of tiles in flight
//     stays compact (a grid-stride loop, one grid over a whole 13B shard and
//     six or eight workgroups per CU all measured slower);
//   * wave-contiguous lanes: lane l of wave w owns two runs of four elements,
//     [512w + 4l, +4) and 256 elements later, so every memory instruction of a
//     wave covers one contiguous span and fills whole cache lines;
//   * every load of an element group is issued before its first use (a
//     scheduling barrier keeps the compiler from sinking loads behind the
//     arithmetic), with non-temporal hints: each byte is touched once a step;
//   * the contributions come from a source: one [N, stride] buffer, a table
//     of one pointer per row (peer-mapped slices), or block-quantised INT8 /
//     INT4 rows (ZeRO++ payloads); the rest of the step is shared;
//   * the fused path double-buffers the optimizer state with the two sets of
//     a tile adjacent in memory, so reading one set and writing the other
//     keeps the locality of an in-place update;
//   * a quantisation block (ZeRO++) is one tile, so the fused step can also
//     emit the block-quantised all-gather payload of the new parameters in
//     the same pass: the block's range is one more workgroup reduction;
//   * fp32 reduction in rank order k = 0..N-1 and each Adam operation rounded
//     once in the written order (compiled with -ffp-contract=off, correctly
//     rounded division and square root), so results are reproducible and
//     agree with a scalar reference operation for operation;
//   * the squared norm accumulated in fp64: per lane, per wave with
//     cross-lane shuffles, per workgroup through LDS (one 16-byte partial per
//     tile), then over contiguous ranges of partials and finally over those
//     ranges in index order: deterministic and far inside the clip tolerance;
//   * all step-to-step scalars (loss scale, t, beta powers, skip, clip, the
//     current state set) live in a device control block, so a step never
//     waits for the host.
// Sources: see include/zero_shard.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "zero_shard.h"

namespace {

constexpr int kBlock = 256;                 // threads per streaming workgroup: 4 wave64s
constexpr int kVec = 8;                     // elements per thread (two runs of four)
constexpr int64_t kTile = ZERO_TILE;        // elements per workgroup
static_assert(kTile == (int64_t)kBlock * kVec, "tile = threads x elements per thread");
constexpr int kFinBlock = 1024;             // threads per finalize workgroup
constexpr int kFinGroups = 256;             // most first-level groups of the finalize
constexpr int64_t kFinPer = 16384;          // partials per first-level finalize group
constexpr int kFinLoads = 4;                // partial loads in flight per finalize thread
// The restore pass: a fixed grid that, on a skipped step, walks the tiles
// kRestoreUnroll at a time with all their loads in flight.  Measured on a
// skipped 13B step (6 bytes per element): 256 x 1 moved 4.2-4.5 TB/s, 256 x 4
// and 512 x 2 5.4, 256 x 8 5.6, 1024 x 4 5.1; with no skip every grid costs
// what a one-wave kernel does (1.6 us back to back in a graph).
constexpr int kRestoreGrid = 256;           // workgroups of the (usually idle) restore pass
constexpr int kRestoreUnroll = 8;           // whole tiles per restore iteration
// The restore that also rebuilds a quantised payload meets a workgroup
// barrier per tile (the block's range), so it needs more workgroups: on a
// skipped 13B step with the INT8 payload, 256 workgroups took 5.8 ms without
// the 16-bit slot and 6.2 ms with it; 1024 took 1.9 and 2.3 ms, 2048 took
// 1.7 and 2.5 ms, 4096 took 1.8 and 2.5 ms.
constexpr int kRestoreQGrid = 2048;         // workgroups of the restore that rebuilds a payload
// Workgroups resident per CU, set by the LDS each streaming workgroup reserves
// (and leaves unused) out of a CU's 160 KB.  Each wave already has every
// load of its group in flight, so few workgroups per CU still cover HBM
// latency, and fewer tiles in flight read and write DRAM with more locality.
// The best count differs by pass.  Without a reservation the registers allow
// six per CU for the 16-bit fused kernels and eight for the others; in one
// process on the same buffers:
//   fused step over 16-bit rows: two per CU; the 13B step 4.5% faster than
//     without a reservation, one per CU 23% slower;
//   Adam pass: two per CU (the 7B step 3% faster, mostly here);
//   reduce over 16-bit rows: three per CU; the 7B step 7.08 ms, against
//     7.18 without a reservation and 7.32 at two;
//   passes that also quantise the all-gather payload wait at one more
//     workgroup barrier per tile: three per CU; the 13B step 10.9 ms against
//     11.2 without a reservation and 11.5 at two; over quantised
//     contributions no reservation (Residency below);
//   fused step over quantised contributions: two per CU; INT8 rows 9.41 ms
//     against 9.63 at three and 9.78 without a reservation, INT4 rows 8.26
//     against 8.37 and 8.50;
//   reduce over quantised contributions, which loads each row's block record
//     through the scalar cache and touches no paired state: no reservation;
//     the 7B step over INT8 rows 6.05 ms against 6.21 at three.
constexpr unsigned kLdsTwoPerCu = 64 * 1024;    // more than a third, at most half
constexpr unsigned kLdsThreePerCu = 48 * 1024;  // more than a quarter, at most a third
constexpr unsigned kResidencyLds = kLdsTwoPerCu;     // fused (16-bit rows) and Adam passes
constexpr unsigned kResidencyLdsQ = kLdsThreePerCu;  // passes writing the all-gather payload

constexpr int64_t kMaxLen = int64_t(1) << 40;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Partial {
    double sumsq;
    uint32_t nonfinite;
    uint32_t pad;
};
static_assert(sizeof(Partial) == ZERO_PARTIAL_BYTES, "one workspace partial per tile");
static_assert(sizeof(zero_ctrl) == 128, "ctrl layout");

int64_t tiles_for(int64_t len) { return len <= 0 ? 0 : (len + kTile - 1) / kTile; }

// ---------------------------------------------------------------- element mapping
// A tile of 2048 elements belongs to one workgroup of 4 waves; wave w covers
// elements [512w, 512w + 512) of the tile.  Lane l owns two runs of four:
// [512w + 4l, +4) ("run a") and the same 256 elements later ("run b").  Each
// memory instruction of a wave therefore covers one contiguous span (1 KiB
// of fp32, 512 B of 16-bit data), and every cache line is filled by a single
// instruction: no line is ever written back half-filled.
constexpr int kRun = 4;

struct Runs {
    int64_t a, b;  // first element of run a and of run b
};

__device__ __forceinline__ Runs runs_of(int64_t tile) {
    const int64_t a = tile * kTile + (threadIdx.x >> 6) * 512 + (threadIdx.x & 63) * kRun;
    return Runs{a, a + 256};
}

// The paired state is one buffer: per tile, set 0 then set 1, each set
// master, m, v of ZERO_TILE floats ([tile][set][master|m|v][ZERO_TILE]).  The
// three array pointers of a paired zero_state are the buffer and the buffer
// plus one and two ZERO_TILE, so pair_index gives the offset of shard element
// i of set s from any of them.
constexpr int64_t kPairTile = 6 * kTile;  // floats of one tile's two sets
__device__ __host__ __forceinline__ int64_t pair_index(int64_t i, int s) {
    const int64_t tile = i / kTile;
    return tile * kPairTile + (int64_t)s * 3 * kTile + (i - tile * kTile);
}

// Element j (0..7) of the thread's group: run a for j < 4, run b otherwise.
__device__ __forceinline__ int64_t elem(const Runs& r, int j) {
    return j < kRun ? r.a + j : r.b + (j - kRun);
}

// ---------------------------------------------------------------- tile order
// The hardware hands consecutive workgroups of a launch to the 8 XCDs in
// turn, and each XCD has its own L2.  A pass over block-quantised
// contributions reads one 8-byte block record per row per tile, and the
// records of 16 consecutive tiles share a 128-byte line; in launch order
// those 16 tiles run on 8 different XCDs, and each fetches the whole line.
// Such passes take the tiles in an order that gives the 16 tiles of a line
// to one XCD: within each group of 128 workgroups, workgroup w takes tile
// 16 * (w % 8) + (w / 8) % 16 of the group; a launch's last, partial group
// keeps the launch order.  Every tile is still taken exactly once.  In one
// process on the same buffers, the 13B step over INT8 rows went from
// 9.11-9.26 to 8.97-9.02 ms and over INT4 rows from 8.25-8.27 to 8.20-8.21
// ms.  The dequantisation of one payload row (one record per tile) ran 5%
// slower in this order, so it and the quantisation keep the launch order.
constexpr int kXcds = 8;
constexpr int kRecordsPerLine = 16;
constexpr int kTileGroup = kXcds * kRecordsPerLine;

template <bool XCD_GROUPED>
__device__ __forceinline__ int64_t tile_index() {
    const int64_t w = blockIdx.x;
    if constexpr (!XCD_GROUPED) {
        return w;
    } else {
        const int64_t whole = (int64_t)(gridDim.x / kTileGroup) * kTileGroup;
        if (w >= whole) return w;
        const int64_t r = w % kTileGroup;
        return w - r + (r % kXcds) * kRecordsPerLine + r / kXcds;
    }
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

// ---------------------------------------------------------------- contribution rows
// Where the N contribution rows of the shard live.  StridedRows: one
// allocation, row k at base + k * stride.  TableRows: row k anywhere in
// device-accessible memory (a local buffer, or a peer GPU's slice mapped into
// this process), one pointer per row carried in the kernel arguments.  Both
// are read-only and index elements of the shard from 0.
struct StridedRows {
    const uint16_t* base;
    int64_t stride;
    __device__ __forceinline__ const uint16_t* row(int k) const {
        return base + (int64_t)k * stride;
    }
};

struct TableRows {
    const uint16_t* p[ZERO_MAX_RANKS];
    __device__ __forceinline__ const uint16_t* row(int k) const { return p[k]; }
};

// One row's 8 values of the thread's group: 4 at run a, 4 at run b.
struct Row {
    u32x2 a, b;
};

__device__ __forceinline__ Row load_row(const uint16_t* __restrict__ base, const Runs& r) {
    Row w;
    w.a = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(base + r.a));
    w.b = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(base + r.b));
    return w;
}

template <int DT>
__device__ __forceinline__ void add_row(float acc[kVec], const Row& w) {
    acc[0] = acc[0] + widen_lo<DT>(w.a.x);
    acc[1] = acc[1] + widen_hi<DT>(w.a.x);
    acc[2] = acc[2] + widen_lo<DT>(w.a.y);
    acc[3] = acc[3] + widen_hi<DT>(w.a.y);
    acc[4] = acc[4] + widen_lo<DT>(w.b.x);
    acc[5] = acc[5] + widen_hi<DT>(w.b.x);
    acc[6] = acc[6] + widen_lo<DT>(w.b.y);
    acc[7] = acc[7] + widen_hi<DT>(w.b.y);
}

template <class RS>
__device__ __forceinline__ void load_rows8(const RS& R, int k0, const Runs& r, Row w[8]) {
#pragma unroll
    for (int q = 0; q < 8; ++q) w[q] = load_row(R.row(k0 + q), r);
}

template <int DT>
__device__ __forceinline__ void add_rows8(float acc[kVec], const Row w[8]) {
#pragma unroll
    for (int q = 0; q < 8; ++q) add_row<DT>(acc, w[q]);
}

// Row sums of the thread's 8 elements over rows k = 0..n-1, added in that
// order, in two phases so that callers can issue all of an element group's
// loads before its first use.  sum_rows_issue loads the first eight rows
// (n >= 8); sum_rows_finish adds them and streams the remaining rows eight
// at a time (all eight loads in flight before the first add).  NR = 8
// compiles the common case of exactly eight rows without the loop; NR = 0
// takes any n.
struct RowLoads {
    Row w[8];
};

template <int NR, class RS>
__device__ __forceinline__ void sum_rows_issue(const RS& R, int n, const Runs& r, RowLoads& L) {
    if (NR == 8 || n >= 8) load_rows8(R, 0, r, L.w);
}

template <int DT, int NR, class RS>
__device__ __forceinline__ void sum_rows_finish(const RS& R, int n, const Runs& r, RowLoads& L,
                                                float acc[kVec]) {
#pragma unroll
    for (int j = 0; j < kVec; ++j) acc[j] = 0.0f;
    if constexpr (NR == 8) {
        add_rows8<DT>(acc, L.w);
        return;
    }
    int k = 0;
    if (n >= 8) {
        add_rows8<DT>(acc, L.w);
        for (k = 8; k + 8 <= n; k += 8) {
            load_rows8(R, k, r, L.w);
            __builtin_amdgcn_sched_barrier(0);
            add_rows8<DT>(acc, L.w);
        }
    }
    // the last n % 8 rows: all loads in flight, then the adds in row order
    const int rem = n - k;
    if (rem > 0) {
#pragma unroll
        for (int q = 0; q < 7; ++q)
            if (q < rem) L.w[q] = load_row(R.row(k + q), r);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < 7; ++q)
            if (q < rem) add_row<DT>(acc, L.w[q]);
    }
}

// Scalar row sum of element i (partial tiles).
template <int DT, class RS>
__device__ __forceinline__ float sum_rows1(const RS& R, int n, int64_t i) {
    float acc = 0.0f;
    for (int k = 0; k < n; ++k) acc = acc + widen1<DT>(R.row(k)[i]);
    return acc;
}

// ---------------------------------------------------------------- contribution sources
// What the streaming kernels sum: for the thread's 8 elements, the N rows'
// values widened to fp32 and added in rank order k = 0..N-1.  A source
// provides issue<NR> (start the first loads), finish<NR> (add them and
// stream the rest) and sum1 (one element of a partial tile).
//
// Src16: 16-bit rows (fp16 or bf16), strided or through a row table.
template <int DT, class RS>
struct Src16 {
    RS rows;
    using Loads = RowLoads;
    static constexpr bool kGrouped = false;  // tiles in launch order
    template <int NR>
    __device__ __forceinline__ void issue(int n, const Runs& r, Loads& L, int64_t) const {
        sum_rows_issue<NR>(rows, n, r, L);
    }
    template <int NR>
    __device__ __forceinline__ void finish(int n, const Runs& r, Loads& L, float acc[kVec],
                                           int64_t) const {
        sum_rows_finish<DT, NR>(rows, n, r, L, acc);
    }
    __device__ __forceinline__ float sum1(int n, int64_t i, int64_t) const {
        return sum_rows1<DT>(rows, n, i);
    }
};

// SrcQ: block-quantised rows (ZeRO++ gradient payloads).  Row k is codes[k]
// (BITS = 8: one byte per element; BITS = 4: two elements per byte, the even
// one in the low nibble) with one zero_qblock per ZERO_QBLOCK elements in
// blocks[k]; both counted from the start of the shard, so the tile of a
// workgroup is exactly one block of every row, and its parameters are
// workgroup-uniform (indexed by the workgroup's tile, taken in the
// XCD-grouped order of tile_index).  Element value: scale * (code - zero),
// one fp32 rounding, then added in rank order.
static_assert(ZERO_QBLOCK == ZERO_TILE, "a quantisation block is one tile");

struct QTable {
    const uint8_t* codes[ZERO_MAX_RANKS];
    const zero_qblock* blocks[ZERO_MAX_RANKS];
};

struct QRow {
    uint32_t a, b;  // the four codes of run a and of run b
};

struct QLoads {
    QRow w[8];
    zero_qblock q[8];
};

template <int BITS>
__device__ __forceinline__ QRow load_qrow(const uint8_t* __restrict__ base, const Runs& r) {
    QRow w;
    if constexpr (BITS == 8) {
        w.a = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(base + r.a));
        w.b = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(base + r.b));
    } else {
        w.a = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(base + (r.a >> 1)));
        w.b = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(base + (r.b >> 1)));
    }
    return w;
}

template <int BITS>
__device__ __forceinline__ int32_t code_at(uint32_t w, int j) {
    return BITS == 8 ? (int32_t)((w >> (8 * j)) & 0xFFu) : (int32_t)((w >> (4 * j)) & 0xFu);
}

__device__ __forceinline__ float dequant(const zero_qblock& q, int32_t code) {
    return q.scale * (float)(code - q.zero);
}

template <int BITS>
__device__ __forceinline__ void add_qrow(float acc[kVec], const QRow& w, const zero_qblock& q) {
#pragma unroll
    for (int j = 0; j < kRun; ++j) acc[j] = acc[j] + dequant(q, code_at<BITS>(w.a, j));
#pragma unroll
    for (int j = 0; j < kRun; ++j) acc[kRun + j] = acc[kRun + j] + dequant(q, code_at<BITS>(w.b, j));
}

template <int BITS>
struct SrcQ {
    QTable t;
    using Loads = QLoads;
    static constexpr bool kGrouped = true;  // a line of records to one XCD
    __device__ __forceinline__ void load8(int k0, const Runs& r, Loads& L, int64_t blk) const {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            L.w[q] = load_qrow<BITS>(t.codes[k0 + q], r);
            L.q[q] = t.blocks[k0 + q][blk];
        }
    }
    __device__ __forceinline__ void add8(float acc[kVec], const Loads& L) const {
#pragma unroll
        for (int q = 0; q < 8; ++q) add_qrow<BITS>(acc, L.w[q], L.q[q]);
    }
    template <int NR>
    __device__ __forceinline__ void issue(int n, const Runs& r, Loads& L, int64_t blk) const {
        if (NR == 8 || n >= 8) load8(0, r, L, blk);
    }
    template <int NR>
    __device__ __forceinline__ void finish(int n, const Runs& r, Loads& L, float acc[kVec],
                                           int64_t blk) const {
#pragma unroll
        for (int j = 0; j < kVec; ++j) acc[j] = 0.0f;
        if constexpr (NR == 8) {
            add8(acc, L);
            return;
        }
        int k = 0;
        if (n >= 8) {
            add8(acc, L);
            for (k = 8; k + 8 <= n; k += 8) {
                load8(k, r, L, blk);
                __builtin_amdgcn_sched_barrier(0);
                add8(acc, L);
            }
        }
        // the last n % 8 rows: all loads in flight, then the adds in row order
        const int rem = n - k;
        if (rem > 0) {
#pragma unroll
            for (int q = 0; q < 7; ++q) {
                if (q < rem) {
                    L.w[q] = load_qrow<BITS>(t.codes[k + q], r);
                    L.q[q] = t.blocks[k + q][blk];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < 7; ++q)
                if (q < rem) add_qrow<BITS>(acc, L.w[q], L.q[q]);
        }
    }
    __device__ __forceinline__ float sum1(int n, int64_t i, int64_t blk) const {
        float acc = 0.0f;  // blk == i / ZERO_QBLOCK
        for (int k = 0; k < n; ++k) {
            const int32_t code = BITS == 8 ? (int32_t)t.codes[k][i]
                                           : (int32_t)((t.codes[k][i >> 1] >> (4 * (i & 1))) & 0xFu);
            acc = acc + dequant(t.blocks[k][blk], code);
        }
        return acc;
    }
};

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
// fp32 values of the thread's group: x[0..3] at pa, x[4..7] at pb.
__device__ __forceinline__ void load8(const float* __restrict__ pa, const float* __restrict__ pb,
                                      float x[kVec]) {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(pa));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(pb));
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void store8(float* __restrict__ pa, float* __restrict__ pb,
                                       const float x[kVec]) {
    f32x4 a, b;
    a.x = x[0]; a.y = x[1]; a.z = x[2]; a.w = x[3];
    b.x = x[4]; b.y = x[5]; b.z = x[6]; b.w = x[7];
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(pa));
    __builtin_nontemporal_store(b, reinterpret_cast<f32x4*>(pb));
}

// Stores 4 sixteen-bit values at dst with accesses of GW elements (GW = 4,
// 2, 1 for an 8-, 4-, 2-byte aligned dst).
template <int GW>
__device__ __forceinline__ void store_h4(uint16_t* __restrict__ dst, const uint32_t* h) {
    if constexpr (GW == 4) {
        u32x2 w;
        w.x = h[0] | (h[1] << 16);
        w.y = h[2] | (h[3] << 16);
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(dst));
    } else if constexpr (GW == 2) {
        __builtin_nontemporal_store(h[0] | (h[1] << 16), reinterpret_cast<uint32_t*>(dst));
        __builtin_nontemporal_store(h[2] | (h[3] << 16), reinterpret_cast<uint32_t*>(dst + 2));
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) __builtin_nontemporal_store((uint16_t)h[q], dst + q);
    }
}

template <int GW>
__device__ __forceinline__ void store_slot(uint16_t* __restrict__ slot, const Runs& r,
                                           const uint32_t h[kVec]) {
    store_h4<GW>(slot + r.a, h);
    store_h4<GW>(slot + r.b, h + kRun);
}

// ---------------------------------------------------------------- norm partials
// Reduces (sumsq, nonfinite) over a workgroup of NT threads: cross-lane within
// each wave, then the wave results in wave order.  Thread 0 gets the result.
template <int NT>
__device__ __forceinline__ void block_reduce(double& ss, uint32_t& bad) {
    constexpr int kW = NT / 64;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        ss += __shfl_xor(ss, off, 64);
        bad |= __shfl_xor(bad, off, 64);
    }
    __shared__ double s_ss[kW];
    __shared__ uint32_t s_bad[kW];
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
        for (int w = 0; w < kW; ++w) {
            t += s_ss[w];
            b |= s_bad[w];
        }
        ss = t;
        bad = b;
    }
}

__device__ __forceinline__ void write_partial(Partial* __restrict__ ws, int64_t tile, double ss,
                                              uint32_t bad) {
    block_reduce<kBlock>(ss, bad);
    if (threadIdx.x == 0) {
        Partial p;
        p.sumsq = ss;
        p.nonfinite = bad ? 1u : 0u;
        p.pad = 0u;
        ws[tile] = p;
    }
}

// ---------------------------------------------------------------- kernels
struct InitArgs {
    zero_ctrl* ctrl;
    float loss_scale;
};

__global__ void ctrl_init_kernel(InitArgs a) {
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        zero_ctrl z = {};
        z.beta1_pow = 1.0;
        z.beta2_pow = 1.0;
        z.loss_scale = a.loss_scale;
        z.scale_used = a.loss_scale;
        z.clip = 1.0f;
        *a.ctrl = z;
    }
}

template <class SRC>
struct ReduceArgs {
    SRC src;
    int64_t len;
    const zero_ctrl* ctrl;
    float* g;
    Partial* ws;
    int32_t n;
};

// Pass 1 of the two-pass step over one tile (the workgroup's, or tile_at when
// AT): g = fl32(sum_k C[k]) * inv, plus the tile's partial.
template <int NR, class SRC, bool AT = false>
__device__ __forceinline__ void reduce_tile(const ReduceArgs<SRC>& a, int64_t tile_at = 0) {
    const float inv = (float)(1.0 / ((double)a.n * (double)a.ctrl->loss_scale));
    double ss = 0.0;
    uint32_t bad = 0;
    const int64_t tile = AT ? tile_at : tile_index<SRC::kGrouped>();
    const Runs r = runs_of(tile);
    if (r.b + kRun <= a.len) {
        float acc[kVec], out[kVec];
        typename SRC::Loads L;
        a.src.template issue<NR>(a.n, r, L, tile);
        __builtin_amdgcn_sched_barrier(0);
        a.src.template finish<NR>(a.n, r, L, acc, tile);
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            bad |= __builtin_isfinite(acc[j]) ? 0u : 1u;
            const float gj = acc[j] * inv;
            ss += (double)gj * (double)gj;
            out[j] = gj;
        }
        store8(a.g + r.a, a.g + r.b, out);
    } else {
        for (int j = 0; j < kVec; ++j) {
            const int64_t i = elem(r, j);
            if (i >= a.len) continue;
            const float acc = a.src.sum1(a.n, i, tile);
            bad |= __builtin_isfinite(acc) ? 0u : 1u;
            const float gj = acc * inv;
            ss += (double)gj * (double)gj;
            a.g[i] = gj;
        }
    }
    write_partial(a.ws, tile, ss, bad);
}

template <int NR, class SRC>
__global__ void __launch_bounds__(kBlock) reduce_kernel(ReduceArgs<SRC> a) {
    reduce_tile<NR, SRC>(a);
}

struct CombineArgs {
    const Partial* ws[ZERO_MAX_RANKS];
    zero_ctrl* ctrl[ZERO_MAX_RANKS];
    int64_t first[ZERO_MAX_RANKS + 1];  // prefix offsets of each rank's partials
    Partial* level1;                    // kFinGroups slots (behind rank 0's partials)
    int64_t per;                        // partials per first-level group
    int32_t nranks;
    int32_t pingpong;
    zero_hparams hp;
};

// Second level of the norm/overflow reduction and the step decisions.  Group
// g sums partials [g*per, (g+1)*per) of the ranks' concatenated lists in
// order; with several groups, the last group to arrive sums the group results
// in group order.  Which group finishes last changes nothing in the result.
__global__ void __launch_bounds__(kFinBlock) finalize_kernel(CombineArgs a) {
    const int64_t total = a.first[a.nranks];
    const int64_t lo = (int64_t)blockIdx.x * a.per;
    const int64_t hi = lo + a.per < total ? lo + a.per : total;
    // the step's scalars, read now so their latency overlaps the reduction
    // (nothing else writes them during this kernel; arrive is reset below)
    zero_ctrl c;
    if (threadIdx.x == 0) c = *a.ctrl[0];
    double ss = 0.0;
    uint32_t bad = 0;
    if (a.nranks == 1) {
        // one rank: kFinLoads independent loads in flight per thread, added in index order
        const Partial* __restrict__ w = a.ws[0];
        int64_t i = lo + threadIdx.x;
        for (; i + (kFinLoads - 1) * kFinBlock < hi; i += kFinLoads * kFinBlock) {
            Partial p[kFinLoads];
#pragma unroll
            for (int q = 0; q < kFinLoads; ++q) p[q] = w[i + q * kFinBlock];
#pragma unroll
            for (int q = 0; q < kFinLoads; ++q) {
                ss += p[q].sumsq;
                bad |= p[q].nonfinite;
            }
        }
        for (; i < hi; i += kFinBlock) {
            ss += w[i].sumsq;
            bad |= w[i].nonfinite;
        }
    } else {
        int r = 0;
        for (int64_t i = lo + threadIdx.x; i < hi; i += kFinBlock) {
            while (i >= a.first[r + 1]) ++r;
            const Partial p = a.ws[r][i - a.first[r]];
            ss += p.sumsq;
            bad |= p.nonfinite;
        }
    }
    block_reduce<kFinBlock>(ss, bad);
    if (gridDim.x > 1) {
        __shared__ uint32_t s_last;
        if (threadIdx.x == 0) {
            Partial p;
            p.sumsq = ss;
            p.nonfinite = bad;
            p.pad = 0u;
            a.level1[blockIdx.x] = p;
            __threadfence();
            const uint32_t prev = atomicAdd(&a.ctrl[0]->arrive, 1u);
            s_last = prev == gridDim.x - 1 ? 1u : 0u;
        }
        __syncthreads();
        if (!s_last) return;
        __threadfence();
        ss = 0.0;
        bad = 0;
        for (int g = threadIdx.x; g < (int)gridDim.x; g += kFinBlock) {
            const Partial p = a.level1[g];
            ss += p.sumsq;
            bad |= p.nonfinite;
        }
        block_reduce<kFinBlock>(ss, bad);
    }
    if (threadIdx.x != 0) return;
    const zero_hparams& hp = a.hp;
    c.arrive = 0u;
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
                // a doubling that overflows keeps the scale (the run restarts either way)
                const float twice = c.loss_scale * 2.0f;
                if (__builtin_isfinite(twice)) c.loss_scale = twice;
                c.good_steps = 0;
            }
        }
    }
    if (!c.skip) {
        // g is multiplied by min(1, max / (norm + 1e-6)), formed in fp64
        if (hp.max_grad_norm > 0.0f) {
            const double coef = (double)hp.max_grad_norm / (c.norm + 1e-6);
            if (coef < 1.0) c.clip = (float)coef;
        }
        c.t += 1;
        c.beta1_pow = c.beta1_pow * (double)hp.beta1;
        c.beta2_pow = c.beta2_pow * (double)hp.beta2;
        if (a.pingpong) c.cur ^= 1;
    }
    for (int q = 0; q < a.nranks; ++q) *a.ctrl[q] = c;
}

// The quantised all-gather payload a fused step may also write: codes and
// block records of the new 16-bit parameters, and the slot's store width
// (4, 2, 1, or 0 for no 16-bit slot), chosen at launch.
struct QGatherOut {
    uint8_t* codes;
    zero_qblock* blocks;
    int32_t gw;
};

constexpr int kGwRuntime = -1;  // slot store width taken from QGatherOut::gw

// Slot store with the width chosen at launch (a workgroup-uniform branch).
__device__ __forceinline__ void store_slot_rt(int gw, uint16_t* __restrict__ slot, const Runs& r,
                                              const uint32_t h[kVec]) {
    if (gw == 4)
        store_slot<4>(slot, r, h);
    else if (gw == 2)
        store_slot<2>(slot, r, h);
    else if (gw == 1)
        store_slot<1>(slot, r, h);
}

template <int BITS>
__device__ __forceinline__ void quant_tile(const float x[kVec], const Runs& r, bool full, int64_t len,
                                           uint8_t* __restrict__ codes,
                                           zero_qblock* __restrict__ blocks, int64_t blk);

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

// Pass 2 of the two-pass step over one tile: Adam in place (+ cast into the
// gather slot).  QB = 8 or 4 also quantises the tile's new 16-bit parameters
// as one block of the all-gather payload.  A skipped step returns from every
// workgroup (the flag is the same for all its threads) before writing
// anything, so slot and payload keep the previous step's values.
template <int DT, int GW, int QB, bool AT = false>
__device__ __forceinline__ void adam_tile(const AdamArgs& a, const QGatherOut& qo,
                                          int64_t tile_at = 0) {
    const zero_ctrl* __restrict__ c = a.ctrl;
    if (c->skip) return;
    const float clip = c->clip;
    const AdamK k = make_adam(a.hp, c->beta1_pow, c->beta2_pow);
    const Runs r = runs_of(AT ? tile_at : (int64_t)blockIdx.x);
    float xq[kVec];  // QB: the new 16-bit parameters widened to fp32, 0 past the end
    if (r.b + kRun <= a.len) {
        float g[kVec], p[kVec], m[kVec], v[kVec];
        uint32_t h[kVec];
        load8(a.g + r.a, a.g + r.b, g);
        load8(a.master + r.a, a.master + r.b, p);
        load8(a.m + r.a, a.m + r.b, m);
        load8(a.v + r.a, a.v + r.b, v);
        __builtin_amdgcn_sched_barrier(0);  // every load of the group is in flight first
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            adam_elem(k, g[j] * clip, p[j], m[j], v[j]);
            h[j] = narrow<DT>(p[j]);
            if constexpr (QB != 0) xq[j] = widen1<DT>((uint16_t)h[j]);
        }
        store8(a.master + r.a, a.master + r.b, p);
        store8(a.m + r.a, a.m + r.b, m);
        store8(a.v + r.a, a.v + r.b, v);
        if constexpr (GW == kGwRuntime)
            store_slot_rt(qo.gw, a.slot, r, h);
        else if constexpr (GW > 0)
            store_slot<GW>(a.slot, r, h);
    } else {
        for (int j = 0; j < kVec; ++j) {
            const int64_t i = elem(r, j);
            if (i >= a.len) {
                if constexpr (QB != 0) xq[j] = 0.0f;
                continue;
            }
            float p = a.master[i], m = a.m[i], v = a.v[i];
            adam_elem(k, a.g[i] * clip, p, m, v);
            a.master[i] = p;
            a.m[i] = m;
            a.v[i] = v;
            if constexpr (QB == 0 && GW == kGwRuntime) {
                if (qo.gw != 0) a.slot[i] = (uint16_t)narrow<DT>(p);
            } else if constexpr (QB == 0) {
                if constexpr (GW > 0) a.slot[i] = (uint16_t)narrow<DT>(p);
            } else {
                const uint32_t hj = narrow<DT>(p);
                if (qo.gw != 0) a.slot[i] = (uint16_t)hj;
                xq[j] = widen1<DT>((uint16_t)hj);
            }
        }
    }
    if constexpr (QB != 0)
        quant_tile<QB>(xq, r, r.b + kRun <= a.len, a.len, qo.codes, qo.blocks, blockIdx.x);
}

template <int DT, int GW>
__global__ void __launch_bounds__(kBlock) adam_kernel(AdamArgs a) {
    adam_tile<DT, GW, 0>(a, QGatherOut{nullptr, nullptr, 0});
}

struct AdamQArgs {
    AdamArgs a;
    QGatherOut q;
};

// Pass 2 that also writes the quantised all-gather payload (BITS = 8 or 4);
// the 16-bit slot is written when q.gw != 0.
template <int DT, int BITS>
__global__ void __launch_bounds__(kBlock) adam_qgather_kernel(AdamQArgs a) {
    adam_tile<DT, kGwRuntime, BITS>(a.a, a.q);
}

struct CastArgs {
    const float* master;  // flat master, or the paired master (restore)
    uint16_t* slot;
    int64_t len;
    const zero_ctrl* ctrl;  // restore only
};

// gather slot <- RNE(master), one tile per workgroup.
template <int DT, int GW>
__global__ void __launch_bounds__(kBlock) cast_kernel(CastArgs a) {
    const Runs r = runs_of(blockIdx.x);
    if (r.b + kRun <= a.len) {
        float p[kVec];
        uint32_t h[kVec];
        load8(a.master + r.a, a.master + r.b, p);
#pragma unroll
        for (int j = 0; j < kVec; ++j) h[j] = narrow<DT>(p[j]);
        store_slot<GW>(a.slot, r, h);
    } else {
        for (int j = 0; j < kVec; ++j) {
            const int64_t i = elem(r, j);
            if (i < a.len) a.slot[i] = (uint16_t)narrow<DT>(a.master[i]);
        }
    }
}

// After a skipped fused step: gather slot <- RNE(current set of the paired
// master).  A fixed grid walks the tiles (with no skip every workgroup
// returns after reading the flag), kRestoreUnroll whole tiles at a time with
// all their loads in flight before the first store, then the rest one by one.
template <int DT, int GW>
__global__ void __launch_bounds__(kBlock) restore_kernel(CastArgs a) {
    if (!a.ctrl->skip) return;
    const int cur = a.ctrl->cur;
    const int64_t ntile = (a.len + kTile - 1) / kTile;
    const int64_t nwhole = a.len / kTile;  // tiles wholly inside len
    const int64_t stride = gridDim.x;
    int64_t tile = blockIdx.x;
    for (; tile + (kRestoreUnroll - 1) * stride < nwhole; tile += kRestoreUnroll * stride) {
        float p[kRestoreUnroll][kVec];
#pragma unroll
        for (int u = 0; u < kRestoreUnroll; ++u) {
            const int64_t sa = pair_index(runs_of(tile + u * stride).a, cur);
            load8(a.master + sa, a.master + sa + 256, p[u]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kRestoreUnroll; ++u) {
            uint32_t h[kVec];
#pragma unroll
            for (int j = 0; j < kVec; ++j) h[j] = narrow<DT>(p[u][j]);
            store_slot<GW>(a.slot, runs_of(tile + u * stride), h);
        }
    }
    for (; tile < ntile; tile += stride) {
        const Runs r = runs_of(tile);
        if (r.b + kRun <= a.len) {
            const int64_t sa = pair_index(r.a, cur);
            float p[kVec];
            uint32_t h[kVec];
            load8(a.master + sa, a.master + sa + 256, p);
#pragma unroll
            for (int j = 0; j < kVec; ++j) h[j] = narrow<DT>(p[j]);
            store_slot<GW>(a.slot, r, h);
        } else {
            for (int j = 0; j < kVec; ++j) {
                const int64_t i = elem(r, j);
                if (i < a.len) a.slot[i] = (uint16_t)narrow<DT>(a.master[pair_index(i, cur)]);
            }
        }
    }
}

struct PackArgs {
    float* flat[3];
    float* pair[3];
    int64_t len;
    const zero_ctrl* ctrl;
};

// TO_PAIR: flat -> current set of the pair; otherwise current set -> flat.
// Full tiles move 16-byte vectors (run a and run b sit 256 elements apart in
// both layouts); the partial last tile goes element by element.
template <bool TO_PAIR>
__global__ void __launch_bounds__(kBlock) pack_kernel(PackArgs a) {
    const int cur = a.ctrl->cur;
    const Runs r = runs_of(blockIdx.x);
    if (r.b + kRun <= a.len) {
        const int64_t pa = pair_index(r.a, cur), pb = pa + 256;
        float x[3][kVec];
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            if (TO_PAIR)
                load8(a.flat[q] + r.a, a.flat[q] + r.b, x[q]);
            else
                load8(a.pair[q] + pa, a.pair[q] + pb, x[q]);
        }
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            if (TO_PAIR)
                store8(a.pair[q] + pa, a.pair[q] + pb, x[q]);
            else
                store8(a.flat[q] + r.a, a.flat[q] + r.b, x[q]);
        }
        return;
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        for (int j = 0; j < kVec; ++j) {
            const int64_t i = elem(r, j);
            if (i >= a.len) continue;
            if (TO_PAIR)
                a.pair[q][pair_index(i, cur)] = a.flat[q][i];
            else
                a.flat[q][i] = a.pair[q][pair_index(i, cur)];
        }
    }
}

template <class SRC>
struct FusedArgs {
    SRC src;
    float* pair[3];  // master, m, v in the paired layout
    uint16_t* slot;
    int64_t len;
    const zero_ctrl* ctrl;
    Partial* ws;
    zero_hparams hp;
    int32_t n;
};

// Single pass over one tile: reduce + partial + Adam (read set cur, write set
// 1-cur of the tile) + cast.  The tile is the workgroup's (tile_index), or
// tile_at when AT (a launch over several shards).  QB = 8 or 4 also quantises the tile's new
// 16-bit parameters as one block (the payload of a quantised all-gather),
// after the per-thread work so that every thread reaches the block's barrier.
template <int DTO, int GW, int NR, class SRC, int QB, bool AT = false>
__device__ __forceinline__ void fused_tile(const FusedArgs<SRC>& a, const QGatherOut& qo,
                                           int64_t tile_at = 0) {
    const zero_ctrl* __restrict__ c = a.ctrl;
    const int cur = c->cur;
    const float inv = (float)(1.0 / ((double)a.n * (double)c->loss_scale));
    const AdamK k = make_adam(a.hp, c->beta1_pow * (double)a.hp.beta1,
                              c->beta2_pow * (double)a.hp.beta2);
    const int64_t tile = AT ? tile_at : tile_index<SRC::kGrouped>();
    const Runs r = runs_of(tile);
    double ss = 0.0;
    uint32_t bad = 0;
    float xq[kVec];  // QB: the new 16-bit parameters widened to fp32, 0 past the end
    if (r.b + kRun <= a.len) {
        // run a and run b of one tile sit at the same distance from their
        // set's start in the paired layout
        const int64_t sa = pair_index(r.a, cur), sb = sa + 256;
        const int64_t da = pair_index(r.a, cur ^ 1), db = da + 256;
        float acc[kVec], p[kVec], m[kVec], v[kVec];
        uint32_t h[kVec];
        typename SRC::Loads L;
        if constexpr (NR == 8) {
            // eight rows and the state: every load of the group in flight first
            a.src.template issue<NR>(a.n, r, L, tile);
            load8(a.pair[0] + sa, a.pair[0] + sb, p);
            load8(a.pair[1] + sa, a.pair[1] + sb, m);
            load8(a.pair[2] + sa, a.pair[2] + sb, v);
            __builtin_amdgcn_sched_barrier(0);
            a.src.template finish<NR>(a.n, r, L, acc, tile);
        } else {
            // any n: the rows stream in chunks of eight first and the state is
            // loaded after them, so it is not held in registers across the
            // chunks (56 instead of 82 VGPRs for bf16 rows: more waves resident)
            a.src.template issue<NR>(a.n, r, L, tile);
            __builtin_amdgcn_sched_barrier(0);
            a.src.template finish<NR>(a.n, r, L, acc, tile);
            __builtin_amdgcn_sched_barrier(0);
            load8(a.pair[0] + sa, a.pair[0] + sb, p);
            load8(a.pair[1] + sa, a.pair[1] + sb, m);
            load8(a.pair[2] + sa, a.pair[2] + sb, v);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            bad |= __builtin_isfinite(acc[j]) ? 0u : 1u;
            const float gj = acc[j] * inv;
            ss += (double)gj * (double)gj;
            adam_elem(k, gj, p[j], m[j], v[j]);
            h[j] = narrow<DTO>(p[j]);
            if constexpr (QB != 0) xq[j] = widen1<DTO>((uint16_t)h[j]);
        }
        store8(a.pair[0] + da, a.pair[0] + db, p);
        store8(a.pair[1] + da, a.pair[1] + db, m);
        store8(a.pair[2] + da, a.pair[2] + db, v);
        if constexpr (GW == kGwRuntime)
            store_slot_rt(qo.gw, a.slot, r, h);
        else
            store_slot<GW>(a.slot, r, h);
    } else {
        for (int j = 0; j < kVec; ++j) {
            const int64_t i = elem(r, j);
            if (i >= a.len) {
                if constexpr (QB != 0) xq[j] = 0.0f;
                continue;
            }
            const float acc = a.src.sum1(a.n, i, tile);
            bad |= __builtin_isfinite(acc) ? 0u : 1u;
            const float gj = acc * inv;
            ss += (double)gj * (double)gj;
            const int64_t si = pair_index(i, cur), di = pair_index(i, cur ^ 1);
            float p = a.pair[0][si], m = a.pair[1][si], v = a.pair[2][si];
            adam_elem(k, gj, p, m, v);
            a.pair[0][di] = p;
            a.pair[1][di] = m;
            a.pair[2][di] = v;
            if constexpr (QB == 0) {
                a.slot[i] = (uint16_t)narrow<DTO>(p);
            } else {
                const uint32_t hj = narrow<DTO>(p);
                if (qo.gw != 0) a.slot[i] = (uint16_t)hj;
                xq[j] = widen1<DTO>((uint16_t)hj);
            }
        }
    }
    if constexpr (QB != 0)
        quant_tile<QB>(xq, r, r.b + kRun <= a.len, a.len, qo.codes, qo.blocks, tile);
    write_partial(a.ws, tile, ss, bad);
}

template <int DTO, int GW, int NR, class SRC>
__global__ void __launch_bounds__(kBlock) fused_kernel(FusedArgs<SRC> a) {
    fused_tile<DTO, GW, NR, SRC, 0>(a, QGatherOut{nullptr, nullptr, 0});
}

template <class SRC>
struct FusedQArgs {
    FusedArgs<SRC> f;
    QGatherOut q;
};

// The fused step that also writes the quantised all-gather payload of the
// new parameters (BITS = 8 or 4); the 16-bit slot is written when q.gw != 0.
template <int DTO, int NR, class SRC, int BITS>
__global__ void __launch_bounds__(kBlock) fused_qgather_kernel(FusedQArgs<SRC> a) {
    fused_tile<DTO, kGwRuntime, NR, SRC, BITS>(a.f, a.q);
}

// ---------------------------------------------------------------- several shards per launch
// Small shards of several ranks on one GPU: one launch covers the tiles of up
// to ZERO_BATCH_SHARDS shards, shard k taking workgroups [tile0_k, tile0_k +
// its tiles).  Each tile does the arithmetic of its shard's own launch, in the
// same order (the slot's store width is chosen per shard at run time), so the
// results are bit-identical to one launch per shard.
struct ShardArg {
    const uint16_t* rows;  // [n, stride] 16-bit rows
    int64_t stride;
    float* pair;           // paired state; m and v one and two ZERO_TILE further
    uint16_t* slot;        // gather buffer + offset
    int64_t len;
    Partial* ws;
    const zero_ctrl* ctrl;
    int32_t tile0;         // the shard's first workgroup in the launch
    int32_t gw;            // slot store width: 4, 2 or 1 values
};

struct ShardsArgs {
    ShardArg s[ZERO_BATCH_SHARDS];
    zero_hparams hp;
    int32_t nshards;
    int32_t n;
};

// The workgroup's shard: the last one whose first workgroup is at or below
// blockIdx.x (tile0 increases with k; a workgroup-uniform scan).
template <class Args>
__device__ __forceinline__ int shard_of(const Args& a) {
    const int64_t w = blockIdx.x;
    int k = 0;
    for (int q = 1; q < a.nshards; ++q)
        if (a.s[q].tile0 <= w) k = q;
    return k;
}

template <int DT, int DTO, int NR>
__global__ void __launch_bounds__(kBlock) fused_shards_kernel(ShardsArgs a) {
    using SRC = Src16<DT, StridedRows>;
    const ShardArg& s = a.s[shard_of(a)];
    const FusedArgs<SRC> f{SRC{StridedRows{s.rows, s.stride}},
                           {s.pair, s.pair + kTile, s.pair + 2 * kTile},
                           s.slot, s.len, s.ctrl, s.ws, a.hp, a.n};
    fused_tile<DTO, kGwRuntime, NR, SRC, 0, true>(f, QGatherOut{nullptr, nullptr, s.gw},
                                                   (int64_t)blockIdx.x - s.tile0);
}

// The restore check of several shards: each workgroup rewrites one tile of
// its shard's slot from the current set of the paired master when that
// shard's step was skipped, and returns at once otherwise.
template <int DT>
__global__ void __launch_bounds__(kBlock) restore_shards_kernel(ShardsArgs a) {
    const ShardArg& s = a.s[shard_of(a)];
    if (!s.ctrl->skip) return;
    const int cur = s.ctrl->cur;
    const Runs r = runs_of((int64_t)blockIdx.x - s.tile0);
    if (r.b + kRun <= s.len) {
        const int64_t sa = pair_index(r.a, cur);
        float p[kVec];
        uint32_t h[kVec];
        load8(s.pair + sa, s.pair + sa + 256, p);
#pragma unroll
        for (int j = 0; j < kVec; ++j) h[j] = narrow<DT>(p[j]);
        store_slot_rt(s.gw, s.slot, r, h);
    } else {
        for (int j = 0; j < kVec; ++j) {
            const int64_t i = elem(r, j);
            if (i < s.len) s.slot[i] = (uint16_t)narrow<DT>(s.pair[pair_index(i, cur)]);
        }
    }
}

// The two passes of the two-pass step for several shards: the reduce (rows
// to g and partials) and, after the decision, the Adam pass (in place on the
// flat state, cast into the slot), each one launch over the shards' tiles.
struct PassArg {
    const uint16_t* rows;  // [n, stride] 16-bit rows (reduce)
    int64_t stride;
    float* master;         // flat state (Adam)
    float* m;
    float* v;
    float* g;
    uint16_t* slot;        // gather buffer + offset, or null (Adam)
    int64_t len;
    Partial* ws;           // (reduce)
    const zero_ctrl* ctrl;
    int32_t tile0;
    int32_t gw;            // slot store width: 4, 2, 1, or 0 for no slot
};

struct PassesArgs {
    PassArg s[ZERO_BATCH_SHARDS];
    zero_hparams hp;
    int32_t nshards;
    int32_t n;
};

template <int DT, int NR>
__global__ void __launch_bounds__(kBlock) reduce_shards_kernel(PassesArgs a) {
    using SRC = Src16<DT, StridedRows>;
    const PassArg& s = a.s[shard_of(a)];
    const ReduceArgs<SRC> r{SRC{StridedRows{s.rows, s.stride}}, s.len, s.ctrl, s.g, s.ws, a.n};
    reduce_tile<NR, SRC, true>(r, (int64_t)blockIdx.x - s.tile0);
}

template <int DT>
__global__ void __launch_bounds__(kBlock) adam_shards_kernel(PassesArgs a) {
    const PassArg& s = a.s[shard_of(a)];
    const AdamArgs aa{s.master, s.m, s.v, s.g, s.slot, s.len, s.ctrl, a.hp};
    adam_tile<DT, kGwRuntime, 0, true>(aa, QGatherOut{nullptr, nullptr, s.gw},
                                       (int64_t)blockIdx.x - s.tile0);
}

// ---------------------------------------------------------------- block quantisation
// One workgroup per block of ZERO_QBLOCK elements (one tile).  The block's
// range [lo, hi] always contains 0: lo starts at +0 and is replaced only by
// a strictly smaller finite value, hi likewise, so the result does not depend
// on the order in which the lanes are combined.  Then
//   S = (hi - lo) / Q (1 if 0), Z = clamp(rint(-lo / S)), q = clamp(rint(x * fl32(1 / S)) + Z),
// every operation one fp32 rounding, rint half to even; a block with a
// non-finite value, or whose S overflows, gets scale NaN, zero 0, codes 0.
struct QuantArgs {
    const uint16_t* src;
    uint8_t* codes;
    zero_qblock* blocks;
    int64_t len;
};

__device__ __forceinline__ float take_lo(float a, float b) { return b < a ? b : a; }
__device__ __forceinline__ float take_hi(float a, float b) { return b > a ? b : a; }

// Range and non-finite flag of the workgroup's values, returned to every thread.
__device__ __forceinline__ void block_range(float& lo, float& hi, uint32_t& bad) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        lo = take_lo(lo, __shfl_xor(lo, off, 64));
        hi = take_hi(hi, __shfl_xor(hi, off, 64));
        bad |= __shfl_xor(bad, off, 64);
    }
    constexpr int kW = kBlock / 64;
    __shared__ float s_lo[kW], s_hi[kW];
    __shared__ uint32_t s_bad[kW];
    if ((threadIdx.x & 63) == 0) {
        s_lo[threadIdx.x >> 6] = lo;
        s_hi[threadIdx.x >> 6] = hi;
        s_bad[threadIdx.x >> 6] = bad;
    }
    __syncthreads();
    lo = 0.0f;
    hi = 0.0f;
    bad = 0u;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
        lo = take_lo(lo, s_lo[w]);
        hi = take_hi(hi, s_hi[w]);
        bad |= s_bad[w];
    }
}

__device__ __forceinline__ float clamp_code(float r, float qmax) {
    return r < 0.0f ? 0.0f : (r > qmax ? qmax : r);
}

// Quantises one block (one tile) from the thread's 8 values x (0 for
// positions past len, which leaves the range unchanged): the block's range
// over the whole workgroup, its record at blocks[blk], and the codes at the
// thread's two runs.  Every thread of the workgroup must call it (it holds a
// workgroup barrier); `full` says whether both of the thread's runs are inside
// len.
template <int BITS>
__device__ __forceinline__ void quant_tile(const float x[kVec], const Runs& r, bool full, int64_t len,
                                           uint8_t* __restrict__ codes,
                                           zero_qblock* __restrict__ blocks, int64_t blk) {
    constexpr float qmax = (float)((1 << BITS) - 1);
    float lo = 0.0f, hi = 0.0f;
    uint32_t bad = 0u;
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
        if (!__builtin_isfinite(x[j])) {
            bad = 1u;
        } else {
            lo = take_lo(lo, x[j]);
            hi = take_hi(hi, x[j]);
        }
    }
    block_range(lo, hi, bad);
    float sc = (hi - lo) / qmax;
    const bool ok = bad == 0u && __builtin_isfinite(sc);
    if (sc == 0.0f) sc = 1.0f;
    const float z = ok ? clamp_code(__builtin_rintf(-lo / sc), qmax) : 0.0f;
    const float inv = 1.0f / sc;  // codes by the reciprocal, as torch's quantizer forms them
    uint32_t c[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j)
        c[j] = ok ? (uint32_t)clamp_code(__builtin_rintf(x[j] * inv) + z, qmax) : 0u;
    if (threadIdx.x == 0) {
        zero_qblock q;
        q.scale = ok ? sc : __builtin_nanf("");
        q.zero = (int32_t)z;
        blocks[blk] = q;
    }
    if (full) {
        if constexpr (BITS == 8) {
            __builtin_nontemporal_store(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                                        reinterpret_cast<uint32_t*>(codes + r.a));
            __builtin_nontemporal_store(c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24),
                                        reinterpret_cast<uint32_t*>(codes + r.b));
        } else {
            __builtin_nontemporal_store((uint16_t)(c[0] | (c[1] << 4) | (c[2] << 8) | (c[3] << 12)),
                                        reinterpret_cast<uint16_t*>(codes + (r.a >> 1)));
            __builtin_nontemporal_store((uint16_t)(c[4] | (c[5] << 4) | (c[6] << 8) | (c[7] << 12)),
                                        reinterpret_cast<uint16_t*>(codes + (r.b >> 1)));
        }
    } else if constexpr (BITS == 8) {
        for (int j = 0; j < kVec; ++j) {
            const int64_t i = elem(r, j);
            if (i < len) codes[i] = (uint8_t)c[j];
        }
    } else {
        // element pairs (2m, 2m + 1) never straddle a run, so each byte has one writer
        for (int j = 0; j < kVec; j += 2) {
            const int64_t i = elem(r, j);
            if (i < len) codes[i >> 1] = (uint8_t)(c[j] | (i + 1 < len ? c[j + 1] << 4 : 0u));
        }
    }
}

// VEC: src is 8-byte aligned (vector loads); otherwise 16-bit loads.
template <int DT, int BITS, bool VEC>
__global__ void __launch_bounds__(kBlock) quantize_kernel(QuantArgs a) {
    const Runs r = runs_of(blockIdx.x);
    const bool full = r.b + kRun <= a.len;
    float x[kVec];
    if (VEC && full) {
        const Row w = load_row(a.src, r);
        x[0] = widen_lo<DT>(w.a.x); x[1] = widen_hi<DT>(w.a.x);
        x[2] = widen_lo<DT>(w.a.y); x[3] = widen_hi<DT>(w.a.y);
        x[4] = widen_lo<DT>(w.b.x); x[5] = widen_hi<DT>(w.b.x);
        x[6] = widen_lo<DT>(w.b.y); x[7] = widen_hi<DT>(w.b.y);
    } else {
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            const int64_t i = elem(r, j);
            x[j] = i < a.len ? widen1<DT>(a.src[i]) : 0.0f;  // 0 leaves the range unchanged
        }
    }
    quant_tile<BITS>(x, r, full, a.len, a.codes, a.blocks, blockIdx.x);
}

struct RestoreQArgs {
    const float* master;  // paired master
    uint16_t* slot;       // NULL when gw == 0
    int64_t len;
    const zero_ctrl* ctrl;
    QGatherOut q;
};

// After a skipped fused step that wrote a quantised all-gather payload: the
// slot (when gw != 0) and the payload rebuilt from the current set of the
// paired master, exactly as the step would have written them.  A fixed small
// grid walks the tiles; with no skip every workgroup returns after reading
// the flag (uniform per workgroup, so the barriers below are reached by all
// or none of its threads).
template <int DT, int BITS>
__global__ void __launch_bounds__(kBlock) restore_q_kernel(RestoreQArgs a) {
    if (!a.ctrl->skip) return;
    const int cur = a.ctrl->cur;
    const int64_t ntile = (a.len + kTile - 1) / kTile;
    for (int64_t tile = blockIdx.x; tile < ntile; tile += gridDim.x) {
        const Runs r = runs_of(tile);
        const bool full = r.b + kRun <= a.len;
        float x[kVec];
        if (full) {
            const int64_t sa = pair_index(r.a, cur);
            float p[kVec];
            uint32_t h[kVec];
            load8(a.master + sa, a.master + sa + 256, p);
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                h[j] = narrow<DT>(p[j]);
                x[j] = widen1<DT>((uint16_t)h[j]);
            }
            store_slot_rt(a.q.gw, a.slot, r, h);
        } else {
            for (int j = 0; j < kVec; ++j) {
                const int64_t i = elem(r, j);
                if (i >= a.len) {
                    x[j] = 0.0f;
                    continue;
                }
                const uint32_t hj = narrow<DT>(a.master[pair_index(i, cur)]);
                if (a.q.gw != 0) a.slot[i] = (uint16_t)hj;
                x[j] = widen1<DT>((uint16_t)hj);
            }
        }
        quant_tile<BITS>(x, r, full, a.len, a.q.codes, a.q.blocks, tile);
        __syncthreads();  // the next tile's block range reuses the same LDS
    }
}

struct DequantArgs {
    const uint8_t* codes;
    const zero_qblock* blocks;
    uint16_t* dst;
    int64_t len;
};

// dst = RNE16(scale * (code - zero)), one block per workgroup; GW is the
// store width of dst as for the gather slot (4, 2 or 1 elements).
template <int DT, int BITS, int GW>
__global__ void __launch_bounds__(kBlock) dequantize_kernel(DequantArgs a) {
    const Runs r = runs_of(blockIdx.x);
    const zero_qblock q = a.blocks[blockIdx.x];
    if (r.b + kRun <= a.len) {
        const QRow w = load_qrow<BITS>(a.codes, r);
        uint32_t h[kVec];
#pragma unroll
        for (int j = 0; j < kRun; ++j) {
            h[j] = narrow<DT>(dequant(q, code_at<BITS>(w.a, j)));
            h[kRun + j] = narrow<DT>(dequant(q, code_at<BITS>(w.b, j)));
        }
        store_slot<GW>(a.dst, r, h);
    } else {
        for (int j = 0; j < kVec; ++j) {
            const int64_t i = elem(r, j);
            if (i >= a.len) continue;
            const int32_t code = BITS == 8 ? (int32_t)a.codes[i]
                                           : (int32_t)((a.codes[i >> 1] >> (4 * (i & 1))) & 0xFu);
            a.dst[i] = (uint16_t)narrow<DT>(dequant(q, code));
        }
    }
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

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int32_t dt) { return dt == ZERO_F16 || dt == ZERO_BF16; }

// Store width (elements) for 16-bit runs of four at dst: 4, 2 or 1.
int store_width(const void* p) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    if ((a & 7u) == 0) return 4;
    if ((a & 3u) == 0) return 2;
    return 1;
}

int check_len(int64_t len, const char* what) {
    if (len < 0 || len > kMaxLen)
        return fail(ZERO_ERANGE, "%s: valid_len %lld out of range", what, (long long)len);
    return ZERO_OK;
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
    int rc;
    if ((rc = check_len(len, "contributions")) != ZERO_OK) return rc;
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

// Row table: nranks in [1, ZERO_MAX_RANKS] pointers, each non-null and
// 8-byte aligned (the widest contribution access is four 16-bit values).
int check_rows(const void* const* rows, int32_t dtype, int32_t n, int64_t len, TableRows* out,
               const char* what) {
    int rc;
    if ((rc = check_len(len, what)) != ZERO_OK) return rc;
    if (!valid_dtype(dtype)) return fail(ZERO_EINVAL, "%s: unknown contribution dtype %d", what, dtype);
    if (n < 1 || n > ZERO_MAX_RANKS)
        return fail(ZERO_EINVAL, "%s: nranks %d outside [1, %d]", what, n, ZERO_MAX_RANKS);
    if (rows == nullptr) return fail(ZERO_EINVAL, "%s: null row table", what);
    for (int k = 0; k < ZERO_MAX_RANKS; ++k) out->p[k] = nullptr;
    for (int k = 0; k < n; ++k) {
        if (rows[k] == nullptr) return fail(ZERO_EINVAL, "%s: row %d is null", what, k);
        if ((reinterpret_cast<uintptr_t>(rows[k]) & 7u) != 0)
            return fail(ZERO_EALIGN, "%s: row %d not 8-byte aligned", what, k);
        out->p[k] = (const uint16_t*)rows[k];
    }
    return ZERO_OK;
}

int check_state(const zero_state* s, const char* what) {
    if (s == nullptr || s->master == nullptr || s->m == nullptr || s->v == nullptr)
        return fail(ZERO_EINVAL, "%s: null state pointer", what);
    if (!aligned16(s->master) || !aligned16(s->m) || !aligned16(s->v))
        return fail(ZERO_EALIGN, "%s: state arrays must be 16-byte aligned", what);
    if (s->master == s->m || s->master == s->v || s->m == s->v)
        return fail(ZERO_EINVAL, "%s: master, m and v must be distinct arrays", what);
    return ZERO_OK;
}

// A paired state: one buffer, with m and v at one and two ZERO_TILE past it.
int check_pair(const zero_state* s, const char* what) {
    if (s == nullptr || s->master == nullptr)
        return fail(ZERO_EINVAL, "%s: null paired state", what);
    if (!aligned16(s->master))
        return fail(ZERO_EALIGN, "%s: paired state not 16-byte aligned", what);
    if (s->m != s->master + kTile || s->v != s->master + 2 * kTile)
        return fail(ZERO_EINVAL, "%s: a paired state is one buffer with m = master + ZERO_TILE and "
                    "v = master + 2 * ZERO_TILE", what);
    return ZERO_OK;
}

int check_ws(const void* ws, size_t ws_bytes, int64_t len) {
    const size_t need = zero_workspace_bytes(len);
    if (ws == nullptr) return fail(ZERO_EINVAL, "workspace pointer is null");
    if (ws_bytes < need)
        return fail(ZERO_ESPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
    if (!aligned16(ws)) return fail(ZERO_EALIGN, "workspace not 16-byte aligned");
    return ZERO_OK;
}

int check_slot(const void* gather, int32_t dtype, int64_t offset) {
    if (gather == nullptr) return fail(ZERO_EINVAL, "gather pointer is null");
    if (!valid_dtype(dtype)) return fail(ZERO_EINVAL, "unknown gather dtype %d", dtype);
    if (offset < 0 || offset > kMaxLen * 64)
        return fail(ZERO_ERANGE, "offset %lld out of range", (long long)offset);
    if ((reinterpret_cast<uintptr_t>(gather) & 1u) != 0)
        return fail(ZERO_EALIGN, "gather buffer not 2-byte aligned");
    return ZERO_OK;
}

int check_ctrl(const zero_ctrl* c, const char* what) {
    if (c == nullptr) return fail(ZERO_EINVAL, "%s: null ctrl", what);
    if ((reinterpret_cast<uintptr_t>(c) & 7u) != 0)
        return fail(ZERO_EALIGN, "%s: ctrl not 8-byte aligned", what);
    return ZERO_OK;
}

template <class Args>
using Kernel = void (*)(Args);

template <int GW, int NR, class SRC>
Kernel<FusedArgs<SRC>> fused_for_nr(int dto) {
    return dto == ZERO_F16 ? fused_kernel<ZERO_F16, GW, NR, SRC> : fused_kernel<ZERO_BF16, GW, NR, SRC>;
}

// Fused kernel for a slot store width gw, output dtype dto and n rows.
template <class SRC>
Kernel<FusedArgs<SRC>> fused_for(int gw, int dto, int n) {
    const bool n8 = n == 8;
    switch (gw) {
        case 4: return n8 ? fused_for_nr<4, 8, SRC>(dto) : fused_for_nr<4, 0, SRC>(dto);
        case 2: return n8 ? fused_for_nr<2, 8, SRC>(dto) : fused_for_nr<2, 0, SRC>(dto);
        default: return n8 ? fused_for_nr<1, 8, SRC>(dto) : fused_for_nr<1, 0, SRC>(dto);
    }
}

template <int DT, int BITS>
Kernel<DequantArgs> dequant_for_bits(int gw) {
    switch (gw) {
        case 4: return dequantize_kernel<DT, BITS, 4>;
        case 2: return dequantize_kernel<DT, BITS, 2>;
        default: return dequantize_kernel<DT, BITS, 1>;
    }
}

template <int DT>
Kernel<DequantArgs> dequant_for(int bits, int gw) {
    return bits == 8 ? dequant_for_bits<DT, 8>(gw) : dequant_for_bits<DT, 4>(gw);
}

template <class SRC>
Kernel<ReduceArgs<SRC>> reduce_for(int n) {
    return n == 8 ? reduce_kernel<8, SRC> : reduce_kernel<0, SRC>;
}

template <int DT>
Kernel<AdamArgs> adam_for(int gw) {
    switch (gw) {
        case 4: return adam_kernel<DT, 4>;
        case 2: return adam_kernel<DT, 2>;
        case 1: return adam_kernel<DT, 1>;
        default: return adam_kernel<ZERO_F16, 0>;  // no slot: the format is not used
    }
}

template <int DT>
Kernel<CastArgs> cast_for(int gw) {
    switch (gw) {
        case 4: return cast_kernel<DT, 4>;
        case 2: return cast_kernel<DT, 2>;
        default: return cast_kernel<DT, 1>;
    }
}

// Launches a kernel whose only parameter is its argument struct (the type
// check below keeps the two in step).
template <class Args>
int launch(Kernel<Args> kernel, int64_t grid, int block, hipStream_t s, const Args& args,
           const char* what, unsigned lds = 0) {
    if (grid < 1 || grid > 0x7FFFFFFF) return fail(ZERO_ERANGE, "%s: grid of %lld workgroups", what, (long long)grid);
    void* params[] = {const_cast<Args*>(&args)};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)grid),
                                         dim3(block), params, lds, s);
    if (e != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    const hipError_t e2 = hipGetLastError();
    if (e2 != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e2));
    return ok();
}

// LDS reserved per workgroup of the fused, fused-with-payload and reduce
// passes, by source.  Over quantised rows the payload pass runs best with no
// reservation (13B shard, INT4 rows: 8.14 against 8.43 ms at three per CU and
// 9.52 ms at two; INT8 rows: equal at none and three per CU).
template <class SRC>
struct Residency {
    static constexpr unsigned fused = kLdsTwoPerCu;
    static constexpr unsigned fused_q = kResidencyLdsQ;
    static constexpr unsigned reduce = kLdsThreePerCu;
};
template <int BITS>
struct Residency<SrcQ<BITS>> {
    static constexpr unsigned fused = kLdsTwoPerCu;
    static constexpr unsigned fused_q = 0;
    static constexpr unsigned reduce = 0;
};

// A streaming pass over a long shard is issued as consecutive launches of at
// most launch_tiles(N) tiles, each with every per-element pointer advanced to
// its first element (the same arithmetic as the bucket contract in the
// header, so the results are those of one launch, bit for bit).  In one launch
// of many thousands of workgroups the slowest ones fall further and further
// behind and the set of tiles in flight spreads over more memory; a new launch
// every few tens of thousands of tiles keeps it compact (the 13B fused step:
// 1-7% shorter than one launch).  The memory that drift spreads over grows
// with the rows each tile reads, so the best launch size falls as N grows: in
// one process per shape, 2,048 tiles at N = 64 (+7% against 16,384), 4,096 at
// N = 32 (+1.5%), flat from 8,192 up at N = 16; at N <= 8 and in the Adam
// passes 32,768 (0.5-0.9% ahead of 16,384 on two machines), except the fused
// step that also writes the payload, which waits at one more workgroup
// barrier per tile: 16,384 (INT4 payload 1.4% ahead, INT8 equal).  Below
// 2,048 tiles the launches' fill and drain cost more than the compact window
// gains.
int64_t launch_tiles(int32_t nranks) {
    if (nranks <= 8) return ZERO_LAUNCH_TILES;
    const int64_t t = ZERO_LAUNCH_ROW_TILES / nranks;
    return t < ZERO_LAUNCH_MIN_TILES ? ZERO_LAUNCH_MIN_TILES : t;
}

// at(x, b0): x advanced by b0 elements of the shard (b0 a multiple of kTile).
StridedRows at(StridedRows r, int64_t b0) {
    r.base += b0;
    return r;
}

TableRows at(TableRows t, int64_t b0) {
    for (int k = 0; k < ZERO_MAX_RANKS; ++k)
        if (t.p[k] != nullptr) t.p[k] += b0;
    return t;
}

template <int DT, class RS>
Src16<DT, RS> at(Src16<DT, RS> s, int64_t b0) {
    s.rows = at(s.rows, b0);
    return s;
}

template <int BITS>
SrcQ<BITS> at(SrcQ<BITS> s, int64_t b0) {
    for (int k = 0; k < ZERO_MAX_RANKS; ++k) {
        if (s.t.codes[k] != nullptr) s.t.codes[k] += b0 * BITS / 8;
        if (s.t.blocks[k] != nullptr) s.t.blocks[k] += b0 / kTile;
    }
    return s;
}

QGatherOut at(QGatherOut q, int64_t b0, int bits) {
    q.codes += b0 * bits / 8;
    q.blocks += b0 / kTile;
    return q;
}

template <class SRC>
FusedArgs<SRC> at(FusedArgs<SRC> a, int64_t b0, int64_t len) {
    a.src = at(a.src, b0);
    for (int q = 0; q < 3; ++q) a.pair[q] += b0 / kTile * kPairTile;
    if (a.slot != nullptr) a.slot += b0;
    a.len = len;
    a.ws += b0 / kTile;
    return a;
}

template <class SRC>
ReduceArgs<SRC> at(ReduceArgs<SRC> a, int64_t b0, int64_t len) {
    a.src = at(a.src, b0);
    a.len = len;
    a.g += b0;
    a.ws += b0 / kTile;
    return a;
}

AdamArgs at(AdamArgs a, int64_t b0, int64_t len) {
    a.master += b0;
    a.m += b0;
    a.v += b0;
    a.g += b0;
    if (a.slot != nullptr) a.slot += b0;
    a.len = len;
    return a;
}

// Launches kernel over len elements in chunks of at most `tiles` tiles;
// at(args, b0, n) gives the arguments of the chunk [b0, b0 + n).  A launch
// error stops the loop, with the earlier chunks already enqueued.
template <class Args, class At>
int launch_chunked(Kernel<Args> kernel, const Args& args, int64_t len, int64_t tiles,
                   hipStream_t s, const char* what, At&& at_chunk, unsigned lds = kResidencyLds) {
    const int64_t chunk = tiles * kTile;
    for (int64_t b0 = 0; b0 < len; b0 += chunk) {
        const int64_t n = len - b0 < chunk ? len - b0 : chunk;
        const int rc = launch(kernel, tiles_for(n), kBlock, s, at_chunk(args, b0, n), what, lds);
        if (rc != ZERO_OK) return rc;
    }
    return ok();
}

template <class Args>
int launch_chunked(Kernel<Args> kernel, const Args& args, int64_t len, int64_t tiles,
                   hipStream_t s, const char* what, unsigned lds = kResidencyLds) {
    return launch_chunked(
        kernel, args, len, tiles, s, what,
        [](const Args& a, int64_t b0, int64_t n) { return at(a, b0, n); }, lds);
}

// Checks and launches shared by the fused entry points (the contribution
// source is already checked).
template <class SRC>
int fused_launch(const SRC& src, int32_t nranks, const zero_state* pair, int64_t valid_len,
                 void* gather, int32_t gather_dtype, int64_t offset, const zero_hparams* hp,
                 const zero_ctrl* ctrl, void* ws, size_t ws_bytes, void* stream, const char* what) {
    int rc;
    if ((rc = check_pair(pair, what)) != ZERO_OK) return rc;
    if ((rc = check_hp(hp)) != ZERO_OK) return rc;
    if (hp->max_grad_norm > 0.0f) return fail(ZERO_EINVAL, "%s: clipping needs the two-pass path", what);
    if ((rc = check_ctrl(ctrl, what)) != ZERO_OK) return rc;
    if ((rc = check_slot(gather, gather_dtype, offset)) != ZERO_OK) return rc;
    if ((rc = check_ws(ws, ws_bytes, valid_len)) != ZERO_OK) return rc;
    if (valid_len == 0) return ok();
    uint16_t* slot = (uint16_t*)gather + offset;
    const FusedArgs<SRC> a{src, {pair->master, pair->m, pair->v}, slot, valid_len, ctrl,
                           (Partial*)ws, *hp, nranks};
    return launch_chunked(fused_for<SRC>(store_width(slot), gather_dtype, nranks), a, valid_len,
                          launch_tiles(nranks), (hipStream_t)stream, what, Residency<SRC>::fused);
}

// Checks and launch shared by the reduce entry points (source already checked).
template <class SRC>
int reduce_launch(const SRC& src, int32_t nranks, int64_t valid_len, const zero_ctrl* ctrl,
                  float* g, void* ws, size_t ws_bytes, void* stream, const char* what) {
    int rc;
    if ((rc = check_ctrl(ctrl, what)) != ZERO_OK) return rc;
    if (g == nullptr) return fail(ZERO_EINVAL, "%s: null g", what);
    if (!aligned16(g)) return fail(ZERO_EALIGN, "%s: g not 16-byte aligned", what);
    if ((rc = check_ws(ws, ws_bytes, valid_len)) != ZERO_OK) return rc;
    if (valid_len == 0) return ok();
    const ReduceArgs<SRC> a{src, valid_len, ctrl, g, (Partial*)ws, nranks};
    return launch_chunked(reduce_for<SRC>(nranks), a, valid_len, launch_tiles(nranks),
                          (hipStream_t)stream, what, Residency<SRC>::reduce);
}

// Quantised row tables: bits 8 or 4, nranks in [1, ZERO_MAX_RANKS], every
// code row and block row non-null and 8-byte aligned.
int check_qrows(const void* const* codes, const zero_qblock* const* blocks, int32_t bits,
                int32_t n, int64_t len, QTable* out, const char* what) {
    int rc;
    if ((rc = check_len(len, what)) != ZERO_OK) return rc;
    if (bits != 8 && bits != 4) return fail(ZERO_EINVAL, "%s: bits must be 8 or 4, not %d", what, bits);
    if (n < 1 || n > ZERO_MAX_RANKS)
        return fail(ZERO_EINVAL, "%s: nranks %d outside [1, %d]", what, n, ZERO_MAX_RANKS);
    if (codes == nullptr || blocks == nullptr) return fail(ZERO_EINVAL, "%s: null row table", what);
    for (int k = 0; k < ZERO_MAX_RANKS; ++k) {
        out->codes[k] = nullptr;
        out->blocks[k] = nullptr;
    }
    for (int k = 0; k < n; ++k) {
        if (codes[k] == nullptr || blocks[k] == nullptr)
            return fail(ZERO_EINVAL, "%s: row %d is null", what, k);
        if (((reinterpret_cast<uintptr_t>(codes[k]) | reinterpret_cast<uintptr_t>(blocks[k])) & 7u) != 0)
            return fail(ZERO_EALIGN, "%s: row %d not 8-byte aligned", what, k);
        out->codes[k] = (const uint8_t*)codes[k];
        out->blocks[k] = blocks[k];
    }
    return ZERO_OK;
}

// Output of a quantised all-gather payload: bits 8 or 4, codes and blocks
// non-null and 8-byte aligned.
int check_qout(int32_t bits, const void* codes, const zero_qblock* blocks, const char* what) {
    if (bits != 8 && bits != 4) return fail(ZERO_EINVAL, "%s: bits must be 8 or 4, not %d", what, bits);
    if (codes == nullptr || blocks == nullptr) return fail(ZERO_EINVAL, "%s: null codes or blocks", what);
    if (((reinterpret_cast<uintptr_t>(codes) | reinterpret_cast<uintptr_t>(blocks)) & 7u) != 0)
        return fail(ZERO_EALIGN, "%s: codes and blocks must be 8-byte aligned", what);
    return ZERO_OK;
}

// The 16-bit slot of a step that also writes a quantised payload: optional
// (gather NULL writes no slot), the dtype always names the parameters' format.
int check_opt_slot(const void* gather, int32_t dtype, int64_t offset) {
    if (gather != nullptr) return check_slot(gather, dtype, offset);
    if (!valid_dtype(dtype)) return fail(ZERO_EINVAL, "unknown gather dtype %d", dtype);
    return ZERO_OK;
}

template <class SRC, int BITS>
Kernel<FusedQArgs<SRC>> fused_qgather_bits(int dto, int n) {
    if (n == 8)
        return dto == ZERO_F16 ? fused_qgather_kernel<ZERO_F16, 8, SRC, BITS>
                               : fused_qgather_kernel<ZERO_BF16, 8, SRC, BITS>;
    return dto == ZERO_F16 ? fused_qgather_kernel<ZERO_F16, 0, SRC, BITS>
                           : fused_qgather_kernel<ZERO_BF16, 0, SRC, BITS>;
}

// Checks and launch shared by the fused entry points that also write the
// quantised all-gather payload (the contribution source is already checked).
template <class SRC>
int fused_qgather_launch(const SRC& src, int32_t nranks, const zero_state* pair, int64_t valid_len,
                         void* gather, int32_t gather_dtype, int64_t offset, int32_t bits,
                         void* codes, zero_qblock* blocks, const zero_hparams* hp,
                         const zero_ctrl* ctrl, void* ws, size_t ws_bytes, void* stream,
                         const char* what) {
    int rc;
    if ((rc = check_pair(pair, what)) != ZERO_OK) return rc;
    if ((rc = check_hp(hp)) != ZERO_OK) return rc;
    if (hp->max_grad_norm > 0.0f) return fail(ZERO_EINVAL, "%s: clipping needs the two-pass path", what);
    if ((rc = check_ctrl(ctrl, what)) != ZERO_OK) return rc;
    if ((rc = check_opt_slot(gather, gather_dtype, offset)) != ZERO_OK) return rc;
    if ((rc = check_qout(bits, codes, blocks, what)) != ZERO_OK) return rc;
    if ((rc = check_ws(ws, ws_bytes, valid_len)) != ZERO_OK) return rc;
    if (valid_len == 0) return ok();
    uint16_t* slot = gather == nullptr ? nullptr : (uint16_t*)gather + offset;
    using A = FusedQArgs<SRC>;
    const A a{{src, {pair->master, pair->m, pair->v}, slot, valid_len, ctrl, (Partial*)ws, *hp,
               nranks},
              {(uint8_t*)codes, blocks, slot == nullptr ? 0 : store_width(slot)}};
    const Kernel<A> k = bits == 8 ? fused_qgather_bits<SRC, 8>(gather_dtype, nranks)
                                  : fused_qgather_bits<SRC, 4>(gather_dtype, nranks);
    const int64_t tiles = launch_tiles(nranks);
    return launch_chunked(k, a, valid_len,
                          tiles < ZERO_LAUNCH_PAYLOAD_TILES ? tiles : ZERO_LAUNCH_PAYLOAD_TILES,
                          (hipStream_t)stream, what,
                          [bits](const A& x, int64_t b0, int64_t n) {
                              return A{at(x.f, b0, n), at(x.q, b0, bits)};
                          },
                          Residency<SRC>::fused_q);
}

// What a batched call does with its shards, for the checks below.
enum class ShardCall { kFused, kRestore, kReduce, kAdam };

// Checks every shard of a batched call before anything is enqueued: the
// shard count, each shard's length (at most one launch of tiles: launch_tiles(n)
// for a pass over rows, ZERO_LAUNCH_TILES otherwise), and the buffers the call
// reads or writes: rows and workspace (fused, reduce), paired state (fused,
// restore), flat state and g (reduce: g; Adam: both), ctrl, and the slot
// (fused, restore; Adam when gather is not null).
int check_shards(const zero_shard* shards, int32_t nshards, int32_t contrib_dtype, int32_t n,
                 const void* gather, int32_t gather_dtype, ShardCall call, const char* what) {
    int rc;
    if (shards == nullptr) return fail(ZERO_EINVAL, "%s: null shard array", what);
    if (nshards < 1 || nshards > ZERO_MAX_RANKS)
        return fail(ZERO_EINVAL, "%s: nshards %d outside [1, %d]", what, nshards, ZERO_MAX_RANKS);
    const bool rows = call == ShardCall::kFused || call == ShardCall::kReduce;
    const int64_t cap = rows ? launch_tiles(n) : ZERO_LAUNCH_TILES;
    for (int i = 0; i < nshards; ++i) {
        const zero_shard& z = shards[i];
        if ((rc = check_len(z.valid_len, what)) != ZERO_OK) return rc;
        if (tiles_for(z.valid_len) > cap)
            return fail(ZERO_ERANGE, "%s: shard %d has %lld tiles, more than the %lld of one "
                        "launch; step it with its own calls", what, i,
                        (long long)tiles_for(z.valid_len), (long long)cap);
        if (rows) {
            if ((rc = check_contrib(z.contrib_dev, contrib_dtype, n, z.stride, z.valid_len)) != ZERO_OK)
                return rc;
            if ((rc = check_ws(z.ws_dev, z.ws_bytes, z.valid_len)) != ZERO_OK) return rc;
        }
        if ((call == ShardCall::kFused || call == ShardCall::kRestore) &&
            (z.pair_dev == nullptr || !aligned16(z.pair_dev)))
            return fail(ZERO_EINVAL, "%s: shard %d: paired state null or not 16-byte aligned", what, i);
        if ((call == ShardCall::kReduce || call == ShardCall::kAdam) &&
            (z.g_dev == nullptr || !aligned16(z.g_dev)))
            return fail(ZERO_EINVAL, "%s: shard %d: g null or not 16-byte aligned", what, i);
        if (call == ShardCall::kAdam && (rc = check_state(&z.state, what)) != ZERO_OK) return rc;
        if ((rc = check_ctrl(z.ctrl_dev, what)) != ZERO_OK) return rc;
        if (call == ShardCall::kReduce || (call == ShardCall::kAdam && gather == nullptr)) continue;
        if ((rc = check_slot(gather, gather_dtype, z.offset)) != ZERO_OK) return rc;
    }
    return ZERO_OK;
}

// Packs the non-empty shards into launches of at most ZERO_BATCH_SHARDS shards
// and `cap` tiles; fill(entry, shard) fills an entry of the kernel arguments
// and launch_one(args, tiles) launches, in shard order.
template <class Args, class Fill, class LaunchOne>
int for_each_shard_launch(const zero_shard* shards, int32_t nshards, int64_t cap, Fill&& fill,
                          LaunchOne&& launch_one) {
    Args a{};
    int64_t tiles = 0;
    for (int i = 0; i < nshards; ++i) {
        const zero_shard& z = shards[i];
        const int64_t t = tiles_for(z.valid_len);
        if (t == 0) continue;
        if (a.nshards == ZERO_BATCH_SHARDS || tiles + t > cap) {
            const int rc = launch_one(a, tiles);
            if (rc != ZERO_OK) return rc;
            a = Args{};
            tiles = 0;
        }
        auto& e = a.s[a.nshards++];
        fill(e, z);
        e.tile0 = (int32_t)tiles;
        tiles += t;
    }
    return a.nshards > 0 ? launch_one(a, tiles) : ok();
}

// A shard's entry for the fused step and the restore.
void fill_shard(ShardArg& e, const zero_shard& z, uint16_t* gather) {
    e.rows = (const uint16_t*)z.contrib_dev;
    e.stride = z.stride;
    e.pair = z.pair_dev;
    e.slot = gather + z.offset;
    e.len = z.valid_len;
    e.ws = (Partial*)z.ws_dev;
    e.ctrl = z.ctrl_dev;
    e.gw = store_width(e.slot);
}

// A shard's entry for the two passes of the two-pass step.
void fill_pass(PassArg& e, const zero_shard& z, uint16_t* gather) {
    e.rows = (const uint16_t*)z.contrib_dev;
    e.stride = z.stride;
    e.master = z.state.master;
    e.m = z.state.m;
    e.v = z.state.v;
    e.g = z.g_dev;
    e.slot = gather == nullptr ? nullptr : gather + z.offset;
    e.len = z.valid_len;
    e.ws = (Partial*)z.ws_dev;
    e.ctrl = z.ctrl_dev;
    e.gw = e.slot == nullptr ? 0 : store_width(e.slot);
}

template <int DT>
Kernel<ShardsArgs> fused_shards_for(int dto, int n) {
    if (n == 8)
        return dto == ZERO_F16 ? fused_shards_kernel<DT, ZERO_F16, 8> : fused_shards_kernel<DT, ZERO_BF16, 8>;
    return dto == ZERO_F16 ? fused_shards_kernel<DT, ZERO_F16, 0> : fused_shards_kernel<DT, ZERO_BF16, 0>;
}

}  // namespace

// ---------------------------------------------------------------- allocation-free step
// For callers that cannot allocate device memory, zero_fused_step_noalloc
// keeps the norm and overflow partials of one fused step in this array: one
// per tile of a shard of at most ZERO_NOALLOC_MAX_LEN elements, plus the
// second-level slots.  Every GPU the library runs on holds its own copy
// until the process ends.  Nothing in it must start at zero: the fused pass
// writes every partial the decision then reads, and the decision's arrival
// counter lives in the ctrl block.
constexpr int64_t kScratchPartials = ZERO_NOALLOC_MAX_LEN / ZERO_TILE + kFinGroups;
static __device__ __align__(256) Partial scratch[kScratchPartials];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The device address of `scratch` on the device that `stream` belongs to,
// looked up once per device with that device current.  In host code the
// array's name is only a stand-in for the symbol, never a device address.
int scratch_on(hipStream_t stream, void** out, const char* what) {
    int dev = -1;
    hipError_t e = stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ZERO_EHIP, "%s: no device for the stream: %s", what, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(ZERO_ERANGE, "%s: device %d out of range", what, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        int cur = -1;
        if ((e = hipGetDevice(&cur)) != hipSuccess)
            return fail(ZERO_EHIP, "%s: hipGetDevice: %s", what, hipGetErrorString(e));
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(ZERO_EHIP, "%s: hipSetDevice(%d): %s", what, dev, hipGetErrorString(e));
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess || p == nullptr)
            return fail(ZERO_EHIP, "%s: hipGetSymbolAddress(scratch): %s", what, hipGetErrorString(e));
        if (e2 != hipSuccess)
            return fail(ZERO_EHIP, "%s: hipSetDevice(%d): %s", what, cur, hipGetErrorString(e2));
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return ZERO_OK;
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
    return (size_t)(tiles_for(valid_len) + kFinGroups) * sizeof(Partial);
}

int64_t zero_launch_tiles(int32_t nranks) { return launch_tiles(nranks); }

size_t zero_pair_elems(int64_t valid_len) {
    return (size_t)(tiles_for(valid_len) * kPairTile);
}

int zero_ctrl_init(zero_ctrl* ctrl, float loss_scale, void* stream) {
    int rc;
    if ((rc = check_ctrl(ctrl, "zero_ctrl_init")) != ZERO_OK) return rc;
    if (!(loss_scale > 0.0f) || loss_scale > 3.0e38f)
        return fail(ZERO_EINVAL, "zero_ctrl_init: loss scale must be finite and > 0");
    const InitArgs a{ctrl, loss_scale};
    return launch<InitArgs>(ctrl_init_kernel, 1, 64, (hipStream_t)stream, a, "zero_ctrl_init");
}

int zero_reduce_grads(const void* contrib, int32_t dtype, int32_t nranks, int64_t stride,
                      int64_t valid_len, const zero_ctrl* ctrl, float* g, void* ws,
                      size_t ws_bytes, void* stream) {
    int rc;
    if ((rc = check_contrib(contrib, dtype, nranks, stride, valid_len)) != ZERO_OK) return rc;
    const StridedRows rows{(const uint16_t*)contrib, stride};
    const char* what = "zero_reduce_grads";
    return dtype == ZERO_F16
               ? reduce_launch(Src16<ZERO_F16, StridedRows>{rows}, nranks, valid_len, ctrl, g, ws,
                               ws_bytes, stream, what)
               : reduce_launch(Src16<ZERO_BF16, StridedRows>{rows}, nranks, valid_len, ctrl, g, ws,
                               ws_bytes, stream, what);
}

int zero_reduce_grads_rows(const void* const* rows, int32_t dtype, int32_t nranks,
                           int64_t valid_len, const zero_ctrl* ctrl, float* g, void* ws,
                           size_t ws_bytes, void* stream) {
    int rc;
    const char* what = "zero_reduce_grads_rows";
    TableRows t;
    if ((rc = check_rows(rows, dtype, nranks, valid_len, &t, what)) != ZERO_OK) return rc;
    return dtype == ZERO_F16
               ? reduce_launch(Src16<ZERO_F16, TableRows>{t}, nranks, valid_len, ctrl, g, ws,
                               ws_bytes, stream, what)
               : reduce_launch(Src16<ZERO_BF16, TableRows>{t}, nranks, valid_len, ctrl, g, ws,
                               ws_bytes, stream, what);
}

int zero_reduce_grads_q(const void* const* codes, const zero_qblock* const* blocks, int32_t bits,
                        int32_t nranks, int64_t valid_len, const zero_ctrl* ctrl, float* g,
                        void* ws, size_t ws_bytes, void* stream) {
    int rc;
    const char* what = "zero_reduce_grads_q";
    QTable t;
    if ((rc = check_qrows(codes, blocks, bits, nranks, valid_len, &t, what)) != ZERO_OK) return rc;
    return bits == 8 ? reduce_launch(SrcQ<8>{t}, nranks, valid_len, ctrl, g, ws, ws_bytes, stream, what)
                     : reduce_launch(SrcQ<4>{t}, nranks, valid_len, ctrl, g, ws, ws_bytes, stream, what);
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
    a.first[0] = 0;
    for (int r = 0; r < nranks; ++r) {
        if ((rc = check_ctrl(ctrl[r], "zero_grad_norm_overflow")) != ZERO_OK) return rc;
        if ((rc = check_len(valid_len[r], "zero_grad_norm_overflow")) != ZERO_OK) return rc;
        if (ws[r] == nullptr || !aligned16(ws[r]))
            return fail(ZERO_EINVAL, "zero_grad_norm_overflow: ws[%d] null or misaligned", r);
        a.ws[r] = (const Partial*)ws[r];
        a.ctrl[r] = ctrl[r];
        a.first[r + 1] = a.first[r] + tiles_for(valid_len[r]);
    }
    const int64_t total = a.first[nranks];
    int64_t groups = (total + kFinPer - 1) / kFinPer;
    groups = groups < 1 ? 1 : (groups > kFinGroups ? kFinGroups : groups);
    a.per = groups == 1 ? (total > 0 ? total : 1) : (total + groups - 1) / groups;
    a.level1 = (Partial*)ws[0] + tiles_for(valid_len[0]);
    a.nranks = nranks;
    a.pingpong = pingpong ? 1 : 0;
    a.hp = *hp;
    return launch<CombineArgs>(finalize_kernel, groups, kFinBlock, (hipStream_t)stream, a,
                  "zero_grad_norm_overflow");
}

int zero_adam_step(const zero_state* state, const float* g, int64_t valid_len,
                   const zero_hparams* hp, const zero_ctrl* ctrl, void* gather,
                   int32_t gather_dtype, int64_t offset, void* stream) {
    int rc;
    if ((rc = check_len(valid_len, "zero_adam_step")) != ZERO_OK) return rc;
    if ((rc = check_state(state, "zero_adam_step")) != ZERO_OK) return rc;
    if ((rc = check_hp(hp)) != ZERO_OK) return rc;
    if ((rc = check_ctrl(ctrl, "zero_adam_step")) != ZERO_OK) return rc;
    if (g == nullptr) return fail(ZERO_EINVAL, "zero_adam_step: null g");
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
    Kernel<AdamArgs> k = gather != nullptr && gather_dtype == ZERO_BF16 ? adam_for<ZERO_BF16>(gw)
                                                              : adam_for<ZERO_F16>(gw);
    return launch_chunked(k, a, valid_len, launch_tiles(0), (hipStream_t)stream,
                          "zero_adam_step");
}

int zero_adam_step_qgather(const zero_state* state, const float* g, int64_t valid_len,
                           const zero_hparams* hp, const zero_ctrl* ctrl, void* gather,
                           int32_t gather_dtype, int64_t offset, int32_t bits, void* codes,
                           zero_qblock* blocks, void* stream) {
    int rc;
    const char* what = "zero_adam_step_qgather";
    if ((rc = check_len(valid_len, what)) != ZERO_OK) return rc;
    if ((rc = check_state(state, what)) != ZERO_OK) return rc;
    if ((rc = check_hp(hp)) != ZERO_OK) return rc;
    if ((rc = check_ctrl(ctrl, what)) != ZERO_OK) return rc;
    if (g == nullptr) return fail(ZERO_EINVAL, "%s: null g", what);
    if (!aligned16(g)) return fail(ZERO_EALIGN, "%s: g not 16-byte aligned", what);
    if ((rc = check_opt_slot(gather, gather_dtype, offset)) != ZERO_OK) return rc;
    if ((rc = check_qout(bits, codes, blocks, what)) != ZERO_OK) return rc;
    if (valid_len == 0) return ok();
    uint16_t* slot = gather == nullptr ? nullptr : (uint16_t*)gather + offset;
    const AdamQArgs a{{state->master, state->m, state->v, g, slot, valid_len, ctrl, *hp},
                      {(uint8_t*)codes, blocks, slot == nullptr ? 0 : store_width(slot)}};
    Kernel<AdamQArgs> k;
    if (gather_dtype == ZERO_F16)
        k = bits == 8 ? adam_qgather_kernel<ZERO_F16, 8> : adam_qgather_kernel<ZERO_F16, 4>;
    else
        k = bits == 8 ? adam_qgather_kernel<ZERO_BF16, 8> : adam_qgather_kernel<ZERO_BF16, 4>;
    return launch_chunked(k, a, valid_len, launch_tiles(0), (hipStream_t)stream, what,
                          [bits](const AdamQArgs& x, int64_t b0, int64_t n) {
                              return AdamQArgs{at(x.a, b0, n), at(x.q, b0, bits)};
                          },
                          kResidencyLdsQ);
}

int zero_cast_to_gather(const float* master, int64_t valid_len, void* gather, int32_t dtype,
                        int64_t offset, void* stream) {
    int rc;
    if ((rc = check_len(valid_len, "zero_cast_to_gather")) != ZERO_OK) return rc;
    if (master == nullptr) return fail(ZERO_EINVAL, "zero_cast_to_gather: null master");
    if (!aligned16(master)) return fail(ZERO_EALIGN, "zero_cast_to_gather: master not 16-byte aligned");
    if ((rc = check_slot(gather, dtype, offset)) != ZERO_OK) return rc;
    if (valid_len == 0) return ok();
    uint16_t* slot = (uint16_t*)gather + offset;
    CastArgs a{master, slot, valid_len, nullptr};
    const int gw = store_width(slot);
    Kernel<CastArgs> k = dtype == ZERO_F16 ? cast_for<ZERO_F16>(gw) : cast_for<ZERO_BF16>(gw);
    return launch(k, tiles_for(valid_len), kBlock, (hipStream_t)stream, a, "zero_cast_to_gather");
}

int zero_fused_step(const void* contrib, int32_t contrib_dtype, int32_t nranks, int64_t stride,
                    const zero_state* pair, int64_t valid_len, void* gather, int32_t gather_dtype,
                    int64_t offset, const zero_hparams* hp, const zero_ctrl* ctrl, void* ws,
                    size_t ws_bytes, void* stream) {
    int rc;
    if ((rc = check_contrib(contrib, contrib_dtype, nranks, stride, valid_len)) != ZERO_OK) return rc;
    const StridedRows rows{(const uint16_t*)contrib, stride};
    const char* what = "zero_fused_step";
    return contrib_dtype == ZERO_F16
               ? fused_launch(Src16<ZERO_F16, StridedRows>{rows}, nranks, pair, valid_len, gather,
                              gather_dtype, offset, hp, ctrl, ws, ws_bytes, stream, what)
               : fused_launch(Src16<ZERO_BF16, StridedRows>{rows}, nranks, pair, valid_len, gather,
                              gather_dtype, offset, hp, ctrl, ws, ws_bytes, stream, what);
}

int zero_fused_step_rows(const void* const* rows, int32_t contrib_dtype, int32_t nranks,
                         const zero_state* pair, int64_t valid_len, void* gather,
                         int32_t gather_dtype, int64_t offset, const zero_hparams* hp,
                         const zero_ctrl* ctrl, void* ws, size_t ws_bytes, void* stream) {
    int rc;
    const char* what = "zero_fused_step_rows";
    TableRows t;
    if ((rc = check_rows(rows, contrib_dtype, nranks, valid_len, &t, what)) != ZERO_OK) return rc;
    return contrib_dtype == ZERO_F16
               ? fused_launch(Src16<ZERO_F16, TableRows>{t}, nranks, pair, valid_len, gather,
                              gather_dtype, offset, hp, ctrl, ws, ws_bytes, stream, what)
               : fused_launch(Src16<ZERO_BF16, TableRows>{t}, nranks, pair, valid_len, gather,
                              gather_dtype, offset, hp, ctrl, ws, ws_bytes, stream, what);
}

int zero_fused_step_q(const void* const* codes, const zero_qblock* const* blocks, int32_t bits,
                      int32_t nranks, const zero_state* pair, int64_t valid_len, void* gather,
                      int32_t gather_dtype, int64_t offset, const zero_hparams* hp,
                      const zero_ctrl* ctrl, void* ws, size_t ws_bytes, void* stream) {
    int rc;
    const char* what = "zero_fused_step_q";
    QTable t;
    if ((rc = check_qrows(codes, blocks, bits, nranks, valid_len, &t, what)) != ZERO_OK) return rc;
    return bits == 8 ? fused_launch(SrcQ<8>{t}, nranks, pair, valid_len, gather, gather_dtype,
                                    offset, hp, ctrl, ws, ws_bytes, stream, what)
                     : fused_launch(SrcQ<4>{t}, nranks, pair, valid_len, gather, gather_dtype,
                                    offset, hp, ctrl, ws, ws_bytes, stream, what);
}

size_t zero_qblock_count(int64_t len) { return (size_t)tiles_for(len); }

size_t zero_qcode_bytes(int64_t len, int32_t bits) {
    if (len <= 0) return 0;
    return bits == 4 ? (size_t)((len + 1) / 2) : (size_t)len;
}

int zero_quantize_blocks(const void* src, int32_t dtype, int64_t len, int32_t bits, void* codes,
                         zero_qblock* blocks, void* stream) {
    int rc;
    const char* what = "zero_quantize_blocks";
    if ((rc = check_len(len, what)) != ZERO_OK) return rc;
    if (!valid_dtype(dtype)) return fail(ZERO_EINVAL, "%s: unknown dtype %d", what, dtype);
    if (bits != 8 && bits != 4) return fail(ZERO_EINVAL, "%s: bits must be 8 or 4, not %d", what, bits);
    if (src == nullptr || codes == nullptr || blocks == nullptr)
        return fail(ZERO_EINVAL, "%s: null pointer", what);
    if (((reinterpret_cast<uintptr_t>(codes) | reinterpret_cast<uintptr_t>(blocks)) & 7u) != 0)
        return fail(ZERO_EALIGN, "%s: codes and blocks must be 8-byte aligned", what);
    if ((reinterpret_cast<uintptr_t>(src) & 1u) != 0)
        return fail(ZERO_EALIGN, "%s: src not 2-byte aligned", what);
    if (len == 0) return ok();
    const QuantArgs a{(const uint16_t*)src, (uint8_t*)codes, blocks, len};
    const bool vec = (reinterpret_cast<uintptr_t>(src) & 7u) == 0;
    Kernel<QuantArgs> k;
    if (dtype == ZERO_F16) {
        if (bits == 8) k = vec ? quantize_kernel<ZERO_F16, 8, true> : quantize_kernel<ZERO_F16, 8, false>;
        else k = vec ? quantize_kernel<ZERO_F16, 4, true> : quantize_kernel<ZERO_F16, 4, false>;
    } else {
        if (bits == 8) k = vec ? quantize_kernel<ZERO_BF16, 8, true> : quantize_kernel<ZERO_BF16, 8, false>;
        else k = vec ? quantize_kernel<ZERO_BF16, 4, true> : quantize_kernel<ZERO_BF16, 4, false>;
    }
    return launch(k, tiles_for(len), kBlock, (hipStream_t)stream, a, what);
}

int zero_dequantize_blocks(const void* codes, const zero_qblock* blocks, int32_t bits, int64_t len,
                           void* dst, int32_t dtype, void* stream) {
    int rc;
    const char* what = "zero_dequantize_blocks";
    if ((rc = check_len(len, what)) != ZERO_OK) return rc;
    if (!valid_dtype(dtype)) return fail(ZERO_EINVAL, "%s: unknown dtype %d", what, dtype);
    if (bits != 8 && bits != 4) return fail(ZERO_EINVAL, "%s: bits must be 8 or 4, not %d", what, bits);
    if (dst == nullptr || codes == nullptr || blocks == nullptr)
        return fail(ZERO_EINVAL, "%s: null pointer", what);
    if (((reinterpret_cast<uintptr_t>(codes) | reinterpret_cast<uintptr_t>(blocks)) & 7u) != 0)
        return fail(ZERO_EALIGN, "%s: codes and blocks must be 8-byte aligned", what);
    if ((reinterpret_cast<uintptr_t>(dst) & 1u) != 0)
        return fail(ZERO_EALIGN, "%s: dst not 2-byte aligned", what);
    if (len == 0) return ok();
    const DequantArgs a{(const uint8_t*)codes, blocks, (uint16_t*)dst, len};
    const Kernel<DequantArgs> k = dtype == ZERO_F16 ? dequant_for<ZERO_F16>(bits, store_width(dst))
                                                    : dequant_for<ZERO_BF16>(bits, store_width(dst));
    return launch(k, tiles_for(len), kBlock, (hipStream_t)stream, a, what);
}

int zero_fused_restore(const zero_state* pair, int64_t valid_len, void* gather, int32_t dtype,
                       int64_t offset, const zero_ctrl* ctrl, void* stream) {
    int rc;
    if ((rc = check_len(valid_len, "zero_fused_restore")) != ZERO_OK) return rc;
    if ((rc = check_pair(pair, "zero_fused_restore")) != ZERO_OK) return rc;
    if ((rc = check_ctrl(ctrl, "zero_fused_restore")) != ZERO_OK) return rc;
    if ((rc = check_slot(gather, dtype, offset)) != ZERO_OK) return rc;
    if (valid_len == 0) return ok();
    CastArgs a{pair->master, (uint16_t*)gather + offset, valid_len, ctrl};
    const int64_t nt = tiles_for(valid_len);
    const int gw = store_width((uint16_t*)gather + offset);
    Kernel<CastArgs> k;
    switch (gw) {
        case 4: k = dtype == ZERO_F16 ? restore_kernel<ZERO_F16, 4> : restore_kernel<ZERO_BF16, 4>; break;
        case 2: k = dtype == ZERO_F16 ? restore_kernel<ZERO_F16, 2> : restore_kernel<ZERO_BF16, 2>; break;
        default: k = dtype == ZERO_F16 ? restore_kernel<ZERO_F16, 1> : restore_kernel<ZERO_BF16, 1>; break;
    }
    return launch(k, nt < kRestoreGrid ? nt : kRestoreGrid, kBlock, (hipStream_t)stream, a,
                  "zero_fused_restore");
}

int zero_fused_step_shards(const zero_shard* shards, int32_t nshards, int32_t contrib_dtype,
                           int32_t nranks, void* gather, int32_t gather_dtype,
                           const zero_hparams* hp, void* stream) {
    int rc;
    const char* what = "zero_fused_step_shards";
    if ((rc = check_hp(hp)) != ZERO_OK) return rc;
    if (hp->max_grad_norm > 0.0f) return fail(ZERO_EINVAL, "%s: clipping needs the two-pass path", what);
    if ((rc = check_shards(shards, nshards, contrib_dtype, nranks, gather, gather_dtype,
                           ShardCall::kFused, what)) != ZERO_OK)
        return rc;
    const Kernel<ShardsArgs> k = contrib_dtype == ZERO_F16
                                     ? fused_shards_for<ZERO_F16>(gather_dtype, nranks)
                                     : fused_shards_for<ZERO_BF16>(gather_dtype, nranks);
    return for_each_shard_launch<ShardsArgs>(
        shards, nshards, launch_tiles(nranks),
        [&](ShardArg& e, const zero_shard& z) { fill_shard(e, z, (uint16_t*)gather); },
        [&](ShardsArgs& a, int64_t tiles) {
            a.hp = *hp;
            a.n = nranks;
            return launch(k, tiles, kBlock, (hipStream_t)stream, a, what, kResidencyLds);
        });
}

int zero_fused_restore_shards(const zero_shard* shards, int32_t nshards, void* gather,
                              int32_t gather_dtype, void* stream) {
    int rc;
    const char* what = "zero_fused_restore_shards";
    if ((rc = check_shards(shards, nshards, ZERO_F16, 1, gather, gather_dtype, ShardCall::kRestore,
                           what)) != ZERO_OK)
        return rc;
    const Kernel<ShardsArgs> k = gather_dtype == ZERO_F16 ? restore_shards_kernel<ZERO_F16>
                                                          : restore_shards_kernel<ZERO_BF16>;
    return for_each_shard_launch<ShardsArgs>(
        shards, nshards, ZERO_LAUNCH_TILES,
        [&](ShardArg& e, const zero_shard& z) { fill_shard(e, z, (uint16_t*)gather); },
        [&](ShardsArgs& a, int64_t tiles) {
            return launch(k, tiles, kBlock, (hipStream_t)stream, a, what);
        });
}

int zero_reduce_grads_shards(const zero_shard* shards, int32_t nshards, int32_t contrib_dtype,
                             int32_t nranks, void* stream) {
    int rc;
    const char* what = "zero_reduce_grads_shards";
    if ((rc = check_shards(shards, nshards, contrib_dtype, nranks, nullptr, ZERO_F16,
                           ShardCall::kReduce, what)) != ZERO_OK)
        return rc;
    Kernel<PassesArgs> k;
    if (nranks == 8)
        k = contrib_dtype == ZERO_F16 ? reduce_shards_kernel<ZERO_F16, 8> : reduce_shards_kernel<ZERO_BF16, 8>;
    else
        k = contrib_dtype == ZERO_F16 ? reduce_shards_kernel<ZERO_F16, 0> : reduce_shards_kernel<ZERO_BF16, 0>;
    return for_each_shard_launch<PassesArgs>(
        shards, nshards, launch_tiles(nranks),
        [&](PassArg& e, const zero_shard& z) { fill_pass(e, z, nullptr); },
        [&](PassesArgs& a, int64_t tiles) {
            a.n = nranks;
            return launch(k, tiles, kBlock, (hipStream_t)stream, a, what,
                          Residency<Src16<ZERO_F16, StridedRows>>::reduce);
        });
}

int zero_adam_step_shards(const zero_shard* shards, int32_t nshards, const zero_hparams* hp,
                          void* gather, int32_t gather_dtype, void* stream) {
    int rc;
    const char* what = "zero_adam_step_shards";
    if ((rc = check_hp(hp)) != ZERO_OK) return rc;
    if (gather == nullptr && !valid_dtype(gather_dtype))
        return fail(ZERO_EINVAL, "%s: unknown gather dtype %d", what, gather_dtype);
    if ((rc = check_shards(shards, nshards, ZERO_F16, 1, gather, gather_dtype, ShardCall::kAdam,
                           what)) != ZERO_OK)
        return rc;
    const Kernel<PassesArgs> k = gather_dtype == ZERO_F16 ? adam_shards_kernel<ZERO_F16>
                                                          : adam_shards_kernel<ZERO_BF16>;
    return for_each_shard_launch<PassesArgs>(
        shards, nshards, ZERO_LAUNCH_TILES,
        [&](PassArg& e, const zero_shard& z) { fill_pass(e, z, (uint16_t*)gather); },
        [&](PassesArgs& a, int64_t tiles) {
            a.hp = *hp;
            return launch(k, tiles, kBlock, (hipStream_t)stream, a, what, kResidencyLds);
        });
}

int zero_fused_step_qgather(const void* contrib, int32_t contrib_dtype, int32_t nranks,
                            int64_t stride, const zero_state* pair, int64_t valid_len, void* gather,
                            int32_t gather_dtype, int64_t offset, int32_t bits, void* codes,
                            zero_qblock* blocks, const zero_hparams* hp, const zero_ctrl* ctrl,
                            void* ws, size_t ws_bytes, void* stream) {
    int rc;
    const char* what = "zero_fused_step_qgather";
    if ((rc = check_contrib(contrib, contrib_dtype, nranks, stride, valid_len)) != ZERO_OK) return rc;
    const StridedRows rows{(const uint16_t*)contrib, stride};
    return contrib_dtype == ZERO_F16
               ? fused_qgather_launch(Src16<ZERO_F16, StridedRows>{rows}, nranks, pair, valid_len,
                                      gather, gather_dtype, offset, bits, codes, blocks, hp, ctrl,
                                      ws, ws_bytes, stream, what)
               : fused_qgather_launch(Src16<ZERO_BF16, StridedRows>{rows}, nranks, pair, valid_len,
                                      gather, gather_dtype, offset, bits, codes, blocks, hp, ctrl,
                                      ws, ws_bytes, stream, what);
}

int zero_fused_step_rows_qgather(const void* const* rows, int32_t contrib_dtype, int32_t nranks,
                                 const zero_state* pair, int64_t valid_len, void* gather,
                                 int32_t gather_dtype, int64_t offset, int32_t bits, void* codes,
                                 zero_qblock* blocks, const zero_hparams* hp,
                                 const zero_ctrl* ctrl, void* ws, size_t ws_bytes, void* stream) {
    int rc;
    const char* what = "zero_fused_step_rows_qgather";
    TableRows t;
    if ((rc = check_rows(rows, contrib_dtype, nranks, valid_len, &t, what)) != ZERO_OK) return rc;
    return contrib_dtype == ZERO_F16
               ? fused_qgather_launch(Src16<ZERO_F16, TableRows>{t}, nranks, pair, valid_len, gather,
                                      gather_dtype, offset, bits, codes, blocks, hp, ctrl, ws,
                                      ws_bytes, stream, what)
               : fused_qgather_launch(Src16<ZERO_BF16, TableRows>{t}, nranks, pair, valid_len,
                                      gather, gather_dtype, offset, bits, codes, blocks, hp, ctrl,
                                      ws, ws_bytes, stream, what);
}

int zero_fused_step_q_qgather(const void* const* qcodes, const zero_qblock* const* qblocks,
                              int32_t qbits, int32_t nranks, const zero_state* pair,
                              int64_t valid_len, void* gather, int32_t gather_dtype, int64_t offset,
                              int32_t bits, void* codes, zero_qblock* blocks, const zero_hparams* hp,
                              const zero_ctrl* ctrl, void* ws, size_t ws_bytes, void* stream) {
    int rc;
    const char* what = "zero_fused_step_q_qgather";
    QTable t;
    if ((rc = check_qrows(qcodes, qblocks, qbits, nranks, valid_len, &t, what)) != ZERO_OK) return rc;
    return qbits == 8 ? fused_qgather_launch(SrcQ<8>{t}, nranks, pair, valid_len, gather,
                                             gather_dtype, offset, bits, codes, blocks, hp, ctrl, ws,
                                             ws_bytes, stream, what)
                      : fused_qgather_launch(SrcQ<4>{t}, nranks, pair, valid_len, gather,
                                             gather_dtype, offset, bits, codes, blocks, hp, ctrl, ws,
                                             ws_bytes, stream, what);
}

int zero_fused_restore_q(const zero_state* pair, int64_t valid_len, void* gather, int32_t dtype,
                         int64_t offset, int32_t bits, void* codes, zero_qblock* blocks,
                         const zero_ctrl* ctrl, void* stream) {
    int rc;
    const char* what = "zero_fused_restore_q";
    if ((rc = check_len(valid_len, what)) != ZERO_OK) return rc;
    if ((rc = check_pair(pair, what)) != ZERO_OK) return rc;
    if ((rc = check_ctrl(ctrl, what)) != ZERO_OK) return rc;
    if ((rc = check_opt_slot(gather, dtype, offset)) != ZERO_OK) return rc;
    if ((rc = check_qout(bits, codes, blocks, what)) != ZERO_OK) return rc;
    if (valid_len == 0) return ok();
    uint16_t* slot = gather == nullptr ? nullptr : (uint16_t*)gather + offset;
    const RestoreQArgs a{pair->master, slot, valid_len, ctrl,
                         {(uint8_t*)codes, blocks, slot == nullptr ? 0 : store_width(slot)}};
    Kernel<RestoreQArgs> k;
    if (dtype == ZERO_F16)
        k = bits == 8 ? restore_q_kernel<ZERO_F16, 8> : restore_q_kernel<ZERO_F16, 4>;
    else
        k = bits == 8 ? restore_q_kernel<ZERO_BF16, 8> : restore_q_kernel<ZERO_BF16, 4>;
    const int64_t nt = tiles_for(valid_len);
    return launch(k, nt < kRestoreQGrid ? nt : kRestoreQGrid, kBlock, (hipStream_t)stream, a, what);
}

static int pair_copy(const zero_state* flat, const zero_state* pair, int64_t valid_len,
                     const zero_ctrl* ctrl, void* stream, bool to_pair, const char* what) {
    int rc;
    if ((rc = check_len(valid_len, what)) != ZERO_OK) return rc;
    if ((rc = check_state(flat, what)) != ZERO_OK) return rc;
    if ((rc = check_pair(pair, what)) != ZERO_OK) return rc;
    if ((rc = check_ctrl(ctrl, what)) != ZERO_OK) return rc;
    if (valid_len == 0) return ok();
    PackArgs a{{flat->master, flat->m, flat->v}, {pair->master, pair->m, pair->v}, valid_len, ctrl};
    Kernel<PackArgs> k = to_pair ? pack_kernel<true> : pack_kernel<false>;
    return launch(k, tiles_for(valid_len), kBlock, (hipStream_t)stream, a, what);
}

int zero_pair_store(const zero_state* flat, const zero_state* pair, int64_t valid_len,
                    const zero_ctrl* ctrl, void* stream) {
    return pair_copy(flat, pair, valid_len, ctrl, stream, true, "zero_pair_store");
}

int zero_pair_load(const zero_state* pair, const zero_state* flat, int64_t valid_len,
                   const zero_ctrl* ctrl, void* stream) {
    return pair_copy(flat, pair, valid_len, ctrl, stream, false, "zero_pair_load");
}

int zero_fused_step_noalloc(const void* contrib, int32_t contrib_dtype, int32_t nranks,
                            int64_t stride, const zero_state* pair, int64_t valid_len, void* gather,
                            int32_t gather_dtype, int64_t offset, const zero_hparams* hp,
                            zero_ctrl* ctrl, void* stream) {
    int rc;
    const char* what = "zero_fused_step_noalloc";
    // every argument checked before the scratch is looked up or anything enqueued
    if ((rc = check_contrib(contrib, contrib_dtype, nranks, stride, valid_len)) != ZERO_OK) return rc;
    if (valid_len > ZERO_NOALLOC_MAX_LEN)
        return fail(ZERO_ERANGE, "%s: valid_len %lld exceeds the scratch's %lld elements "
                    "(ZERO_NOALLOC_MAX_LEN); use zero_fused_step with a workspace", what,
                    (long long)valid_len, (long long)ZERO_NOALLOC_MAX_LEN);
    if ((rc = check_pair(pair, what)) != ZERO_OK) return rc;
    if ((rc = check_hp(hp)) != ZERO_OK) return rc;
    if (hp->max_grad_norm > 0.0f) return fail(ZERO_EINVAL, "%s: clipping needs the two-pass path", what);
    if ((rc = check_ctrl(ctrl, what)) != ZERO_OK) return rc;
    if ((rc = check_slot(gather, gather_dtype, offset)) != ZERO_OK) return rc;
    void* ws = nullptr;
    if ((rc = scratch_on((hipStream_t)stream, &ws, what)) != ZERO_OK) return rc;
    const size_t ws_bytes = (size_t)kScratchPartials * sizeof(Partial);
    // the three calls of a fused step, the partials in the scratch
    if ((rc = zero_fused_step(contrib, contrib_dtype, nranks, stride, pair, valid_len, gather,
                              gather_dtype, offset, hp, ctrl, ws, ws_bytes, stream)) != ZERO_OK)
        return rc;
    zero_ctrl* ctrls[1] = {ctrl};
    void* wss[1] = {ws};
    if ((rc = zero_grad_norm_overflow(1, wss, &valid_len, ctrls, hp, 1, stream)) != ZERO_OK) return rc;
    return zero_fused_restore(pair, valid_len, gather, gather_dtype, offset, ctrl, stream);
}

const char* zero_last_error(void) { return g_err; }

}  // extern "C"
