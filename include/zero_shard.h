/* zero_shard.h -- C ABI of the ZeRO per-rank shard step on AMD Instinct MI355X (gfx950).
 *
 * One data-parallel rank owns a contiguous slice ("shard") of a flat buffer of
 * Psi parameters.  After the gradient reduce-scatter, the rank holds the N
 * ranks' 16-bit gradient contributions for its slice.  The shard step
 *   1. sums them in fp32, removes the loss scale and averages,
 *   2. checks for inf/NaN and computes the global L2 norm (with optional
 *      clipping and loss-scale-driven skipping),
 *   3. runs mixed-precision Adam(W) on the fp32 master weights, momentum and
 *      variance of the slice,
 *   4. casts the new master weights to fp16/bf16 into the rank's slot of the
 *      full parameter buffer that the all-gather fills.
 * Sources (page titles and sections):
 *   "CMU 11-868 L18: How ZeRO Cuts Data-Parallel Memory", Mechanism 1, steps 3-6
 *     (reduce-scatter to fp32, update own slice of variance/momentum/params,
 *     copy to fp16, all-gather);
 *   "ZeRO: Memory Optimizations Toward Training Trillion Parameter Models"
 *     (paper-graph summary), 3.4: model-state analysis (16 Psi bill), Stage 1
 *     (Pos) and Stage 2 (Pos+g), and the residual-state note on gradient-norm
 *     buffers;
 *   "zero-stages-simulation" README, partitioning paragraph: the flattened
 *     buffer is cut into N contiguous pieces of (almost) the same length and
 *     rank r holds piece r;
 *   "ZeRO: Memory Optimization for Large Models" (lesson), Stage 1 and 2;
 *   "ZeRO Stage 1/2/3" guide, section 5 (AdamW with weight decay, the
 *     reduce bucket size);
 *   "CMU 11-868 L18", Other memory optimizations (ZeRO++ block-quantised
 *     payloads); paper summary 3.4, Stage 2 bucketization (gradients reduced
 *     bucket by bucket during the backward pass).
 *
 * Conventions for every call below.
 *   - Pointers named *_dev are device pointers (hipMalloc'd or torch tensors);
 *     all other pointers are host pointers.  Every buffer is owned by the
 *     caller.  The library never allocates or frees device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls that touch device memory only enqueue work on `stream` and return;
 *     they never synchronise.  Results are visible after the caller syncs.
 *   - Arguments are validated before anything is enqueued: on an argument
 *     error (EINVAL, EALIGN, ERANGE, ESPACE) nothing was enqueued and nothing
 *     was written.  EHIP (the runtime refused a launch) can follow earlier
 *     launches of the same call (a pass is issued as several launches, see
 *     ZERO_LAUNCH_TILES).  zero_last_error() describes the problem.  Faults
 *     inside kernels surface at the next sync.
 *   - 16-bit data is passed as raw storage (uint16 bit patterns); `dtype`
 *     selects ZERO_F16 (IEEE binary16) or ZERO_BF16 (bfloat16).
 *   - Element counts and offsets are int64 (Psi reaches 1.3e10 elements).
 *   - Alignment: contribution buffers, their row stride (a multiple of 8
 *     elements), g and the fp32 state arrays must be 16-byte aligned; rows of
 *     a row table need 8 bytes.  The gather slot needs only 2-byte alignment.
 *   - valid_len == 0 (an empty tail rank) is legal: nothing is enqueued except
 *     where the call says otherwise.
 *   - Calls on different streams are independent as long as they use
 *     different ctrl blocks and workspaces.
 *   - Sizes the library cannot see are the caller's to guarantee: a gather
 *     buffer holds at least offset + valid_len elements; contribution rows
 *     hold valid_len elements (and a [N, stride] buffer N * stride); g and
 *     flat state arrays valid_len floats; a paired state's buffer
 *     zero_pair_elems;
 *     workspaces ws_bytes (checked against zero_workspace_bytes); quantised
 *     codes zero_qcode_bytes and block records zero_qblock_count entries.
 *     A buffer shorter than that is read or written out of bounds.
 */
#ifndef ZERO_SHARD_H
#define ZERO_SHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ZERO_F16 = 1, ZERO_BF16 = 2 };

enum {
    ZERO_OK = 0,
    ZERO_EINVAL = -1, /* bad argument (null pointer, count, dtype, ...) */
    ZERO_EALIGN = -2, /* misaligned pointer or stride */
    ZERO_ERANGE = -3, /* size or offset out of the supported range */
    ZERO_ESPACE = -4, /* workspace too small */
    ZERO_EHIP = -5    /* the HIP runtime refused a launch */
};

enum { ZERO_SCALER_NONE = 0, ZERO_SCALER_STATIC = 1, ZERO_SCALER_DYNAMIC = 2 };

#define ZERO_MAX_CONTRIB 1024 /* largest N accepted by the reduce */
#define ZERO_MAX_RANKS 64     /* most ctrl blocks combined in one call; most rows in a row table */
#define ZERO_QBLOCK 2048      /* elements per quantisation block (one tile) */

/* Parameters of one quantisation block: value = scale * (code - zero).  A
 * block that held a non-finite value has scale NaN and zero 0. */
typedef struct {
    float scale;
    int32_t zero;
} zero_qblock;

/* Optimizer, clipping and loss-scale settings, passed by host pointer and
 * copied into the kernel arguments.  The pages name Adam (Kingma and Ba) and
 * AdamW with weight_decay but print no update; the library applies
 * bias-corrected Adam with epsilon outside the square root and decoupled
 * weight decay:  m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g*g;
 * p = p - lr ((m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps) + wd p),
 * every operation rounded to fp32, b^t a running fp64 product.
 * max_grad_norm > 0 turns clipping on: g is multiplied by
 * min(1, max_grad_norm / (norm + 1e-6)), the coefficient formed in fp64 and
 * rounded to fp32 (the rule of torch.nn.utils.clip_grad_norm_ given an fp64
 * norm).
 * scaler: NONE keeps S = 1; STATIC keeps the initial S; DYNAMIC halves S
 * (not below min_scale) on a skipped step and doubles it after
 * growth_interval consecutive applied steps, unless the doubled value is
 * not finite, when S stays (torch._amp_update_scale_'s schedule, plus the
 * min_scale floor).  A step whose reduced gradient holds inf or NaN is
 * always skipped. */
typedef struct zero_hparams {
    float lr, beta1, beta2, eps, weight_decay, max_grad_norm;
    int32_t scaler;
    float min_scale;
    int32_t growth_interval;
} zero_hparams;

/* Control block: 128 bytes in DEVICE memory, one per rank, written only by the
 * library's kernels.  Host code may copy it back to read the decisions.
 * It carries the step-to-step scalars so that no step needs a host sync. */
typedef struct zero_ctrl {
    double sumsq;       /* last step: global sum of g^2 over all ranks (fp64) */
    double norm;        /* last step: sqrt(sumsq) (inf/NaN when the gradient was) */
    double beta1_pow;   /* beta1^t */
    double beta2_pow;   /* beta2^t */
    float loss_scale;   /* S that the next step's contributions carry */
    float scale_used;   /* S of the last step */
    float clip;         /* clip factor applied by the last step (1 when none) */
    int32_t nonfinite;  /* last step: 1 if any reduced element was inf/NaN */
    int32_t skip;       /* last step was skipped (state, slot and t unchanged) */
    int32_t t;          /* applied optimizer steps */
    int32_t good_steps; /* applied steps since the last skip or doubling point */
    int32_t cur;        /* fused path: which set of the paired state is current */
    uint32_t arrive;    /* internal: arrival counter of the norm reduction, 0 between calls */
    uint32_t reserved[15];
} zero_ctrl;

/* Elements per workgroup tile of every streaming pass.  The fused path's
 * double-buffered state interleaves its two sets tile by tile. */
#define ZERO_TILE 2048

/* Launch sizes: a streaming pass (reduce, fused step, Adam) over valid_len
 * elements is issued as ceil(ceil(valid_len / ZERO_TILE) / T) consecutive
 * launches of at most T tiles on the caller's stream, which a profiler lists
 * one by one; the results are those of one launch.  T = ZERO_LAUNCH_TILES
 * for the Adam passes and for a pass that reads N <= 8 contribution rows;
 * over N > 8 rows (reduce and fused step, every source) T =
 * max(ZERO_LAUNCH_MIN_TILES, ZERO_LAUNCH_ROW_TILES / N) (zero_launch_tiles).
 * The fused step that also writes the quantised all-gather payload takes at
 * most ZERO_LAUNCH_PAYLOAD_TILES of those. */
#define ZERO_LAUNCH_TILES 32768
#define ZERO_LAUNCH_ROW_TILES 131072
#define ZERO_LAUNCH_MIN_TILES 2048
#define ZERO_LAUNCH_PAYLOAD_TILES 16384

/* One rank's fp32 optimizer state: master weights, Adam m, Adam v.
 * Flat form (two-pass path, pack/unpack): three arrays of valid_len
 * contiguous floats.
 * Paired form (fused path): ONE buffer of zero_pair_elems(valid_len) floats
 * holding two copies (sets) of the whole state, interleaved per tile of
 * ZERO_TILE elements as [tile][set][master | m | v][ZERO_TILE]: array q
 * (0 master, 1 m, 2 v) of set s for element i lives at buffer
 * [(i / ZERO_TILE) * 6 * ZERO_TILE + s * 3 * ZERO_TILE + q * ZERO_TILE
 * + i % ZERO_TILE].  Its zero_state is {buffer, buffer + ZERO_TILE,
 * buffer + 2 * ZERO_TILE}; the paired calls check that and return EINVAL
 * otherwise.  A tile's whole state (both sets, all three arrays, 48 KiB) is
 * one contiguous block, so the fused pass reads one set and writes the other
 * in one region of memory; with the launch configuration of the passes this
 * measured 1-2% faster than three separately allocated arrays. */
typedef struct zero_state {
    float *master;
    float *m;
    float *v;
} zero_state;

/* Partition ("zero-stages-simulation" README, flat partitioning paragraph;
 * lesson "ZeRO: Memory Optimization for Large Models", Stage 1 step 3):
 * the flat buffer is split into N contiguous shards of ceil(Psi/N) elements,
 * rank r owns [r*shard, r*shard + valid) with valid = clamp(Psi - r*shard, 0,
 * shard); tail ranks are short or empty.  Pure host arithmetic.
 * Returns ZERO_EINVAL for psi < 1, nranks < 1, rank outside [0, nranks) or a
 * null output pointer. */
int zero_partition(int64_t psi, int32_t nranks, int32_t rank, int64_t *shard_len,
                   int64_t *offset, int64_t *valid_len);

/* Bytes of the device workspace per tile of ZERO_TILE elements: the first
 * level of the norm and overflow reduction keeps one partial per tile. */
#define ZERO_PARTIAL_BYTES 16

/* Buckets (paper summary 3.4, Stage 2, bucketization: gradients are reduced
 * bucket by bucket as the backward pass produces them; "ZeRO Stage 1/2/3"
 * guide, section 5: reduce_bucket_size).  The per-element calls
 * (zero_reduce_grads and its _rows/_q forms, zero_fused_step and its
 * _rows/_q/_qgather forms) may be issued as several calls over consecutive
 * pieces of one shard, each piece [b0, b0 + len) starting at a multiple of
 * ZERO_TILE, as the pieces arrive.  The call for a piece takes every
 * per-element pointer advanced by b0 elements (contribution rows, g, the
 * 16-bit slot's offset; the paired state's pointers by 6 * b0 floats; INT8 codes
 * by b0 bytes, INT4 codes by b0 / 2, block records by b0 / ZERO_TILE), and
 * the workspace advanced by (b0 / ZERO_TILE) * ZERO_PARTIAL_BYTES bytes with
 * ws_bytes reduced by as much; ctrl, hparams and the row stride stay the
 * same.  After the last piece, zero_grad_norm_overflow over the whole
 * workspace and valid_len, then the rest of the step over the whole shard
 * (zero_adam_step or zero_adam_step_qgather; zero_fused_restore or
 * zero_fused_restore_q), complete the step: the results equal those of one
 * call over the whole shard, bit for bit.  On the fused path each piece's
 * Adam update can therefore run as soon as its gradient has arrived; the
 * skip decision still waits for the last piece. */

/* sizeof(zero_ctrl); allocate that many bytes of device memory per rank. */
size_t zero_ctrl_bytes(void);

/* Device workspace (bytes) needed by zero_reduce_grads and zero_fused_step
 * for a shard of valid_len elements: one 16-byte partial (fp64 sum of
 * squares, non-finite flag) per tile of ZERO_TILE elements, plus 256 slots
 * for the second level of the reduction (about 0.8% of the shard's fp16
 * size). */
size_t zero_workspace_bytes(int64_t valid_len);

/* Most tiles per launch T of a pass that reads nranks contribution rows, as
 * defined with ZERO_LAUNCH_TILES; nranks <= 0 gives the Adam passes' T. */
int64_t zero_launch_tiles(int32_t nranks);

/* Floats of the one buffer of a paired (fused-path) state for valid_len
 * elements: 6 * ceil(valid_len / ZERO_TILE) * ZERO_TILE. */
size_t zero_pair_elems(int64_t valid_len);

/* Initialise a ctrl block on `stream`: t = 0, beta powers 1, loss scale S
 * (must be finite and > 0; use 1 without a scaler), cur = 0, arrive = 0. */
int zero_ctrl_init(zero_ctrl *ctrl_dev, float loss_scale, void *stream);

/* Reduce ("CMU 11-868 L18", Mechanism 1 step 3: the reduce-scatter leaves each
 * rank the fp32 mean of all ranks' gradients over its own slice only; paper
 * summary 3.4 Stage 2, reduce-scatter of gradients):
 *   g[i] = fl32( sum_{k=0..N-1} C[k][i] ) * fl32(1 / (N * S)),   i < valid_len,
 * summed in fp32 in rank order k = 0..N-1; S is ctrl->loss_scale.
 * contrib_dev: N rows of `stride` elements (16-bit, dtype), row k at
 * contrib_dev + k*stride; only columns < valid_len are read.
 * g_dev: valid_len floats, written.
 * The same pass writes the first level of the norm and overflow reduction,
 * one partial per workgroup, into ws_dev (ws_bytes >= zero_workspace_bytes).
 * Errors: EINVAL (null, dtype, nranks outside [1, ZERO_MAX_CONTRIB],
 * stride < valid_len), EALIGN, ESPACE. */
int zero_reduce_grads(const void *contrib_dev, int32_t dtype, int32_t nranks, int64_t stride,
                      int64_t valid_len, const zero_ctrl *ctrl_dev, float *g_dev, void *ws_dev,
                      size_t ws_bytes, void *stream);

/* zero_reduce_grads with the N contribution rows in separate places: row k
 * starts at rows_dev[k] (valid_len 16-bit values; element i of the shard at
 * rows_dev[k][i]).  This is the form a reduce-scatter takes when every rank
 * reads its slice of the N ranks' gradient buffers directly, each slice
 * mapped into this process from its owner's memory ("CMU 11-868 L18",
 * Mechanism 1 step 3; paper summary 3.4 Stage 2): no staging copy into one
 * [N, stride] buffer.  The result is bit-identical to zero_reduce_grads on
 * the same rows (same order k = 0..N-1).  rows_dev is a host array of nranks
 * device pointers, copied into the launch (reusable on return); each pointer
 * must be non-NULL and 8-byte aligned, rows may alias (they are only read).
 * Errors: EINVAL (null table or row, dtype, nranks outside
 * [1, ZERO_MAX_RANKS]), EALIGN (a row not 8-byte aligned, g), ESPACE. */
int zero_reduce_grads_rows(const void *const *rows_dev, int32_t dtype, int32_t nranks,
                           int64_t valid_len, const zero_ctrl *ctrl_dev, float *g_dev,
                           void *ws_dev, size_t ws_bytes, void *stream);

/* Norm, overflow and step decisions (paper summary 3.4, residual states:
 * gradient-norm computation over all gradients; "CMU 11-868 L18", The memory
 * bill, same note).  Combines the per-tile partials that the previous
 * zero_reduce_grads or zero_fused_step left in each ws_dev[r] (valid_len[r]
 * elements) into the global sum of squares and the global non-finite flag of
 * the `nranks` ranks given (nranks > 1 stands in for the scalar all-reduce
 * between data-parallel ranks; with one rank they are its own).  The
 * reduction is deterministic: contiguous ranges of the concatenated partials
 * are summed in order, then the ranges in index order.  Then, in every ctrl
 * block: norm = sqrt(sumsq); skip = nonfinite; loss-scale update; clip
 * factor; if applied: t += 1, beta powers advance and, when `pingpong` is
 * nonzero, cur flips to the state set the fused step just wrote.  Enqueued
 * even when every valid_len is 0.
 * ws_dev, valid_len and ctrl_dev are host arrays of nranks entries (ws_dev and
 * ctrl_dev entries are device pointers).  Each ws_dev[r] must be the whole
 * workspace of zero_workspace_bytes(valid_len[r]) bytes that the step used
 * (the reduction keeps its second level behind rank 0's partials).  All ctrl
 * blocks must hold the same scalars (they do when they are always updated
 * together), and calls sharing ctrl_dev[0] must not overlap.
 * Errors: EINVAL (null, nranks outside [1, ZERO_MAX_RANKS], bad hparams),
 * EALIGN, ERANGE. */
int zero_grad_norm_overflow(int32_t nranks, void *const *ws_dev, const int64_t *valid_len,
                            zero_ctrl *const *ctrl_dev, const zero_hparams *hp,
                            int32_t pingpong, void *stream);

/* Adam on the owned slice ("CMU 11-868 L18", Mechanism 1 step 4: the rank's
 * fp32 master weights and both Adam moments are the only optimizer state it
 * touches; paper summary 3.4 Stage 1), fused with the cast into the gather
 * slot (Mechanism 1 step 5: the new master weights, rounded to the 16-bit
 * format).
 * Two-pass path: runs after zero_reduce_grads and zero_grad_norm_overflow
 * (pingpong = 0), reads g_dev and ctrl (skip, clip, t, beta powers), updates
 * state in place.  When gather_dev is not NULL, writes
 * RNE_dtype(master[i]) to gather_dev[offset + i].  A skipped step returns
 * from every workgroup without writing.
 * Errors: EINVAL, EALIGN, ERANGE (offset < 0). */
int zero_adam_step(const zero_state *state, const float *g_dev, int64_t valid_len,
                   const zero_hparams *hp, const zero_ctrl *ctrl_dev, void *gather_dev,
                   int32_t gather_dtype, int64_t offset, void *stream);

/* zero_adam_step that also writes the quantised all-gather payload of the
 * new parameters (ZeRO++, "CMU 11-868 L18", Other memory optimizations; see
 * zero_fused_step_qgather): codes_dev and blocks_dev equal, bit for bit,
 * what zero_quantize_blocks(gather_dtype, bits) would write from the 16-bit
 * slot after the step.  gather_dev may be NULL (no 16-bit slot written);
 * gather_dtype always names the 16-bit format that is quantised.  A skipped
 * step writes nothing, so slot and payload keep the previous step's values;
 * the caller initialises the payload with the slot (zero_quantize_blocks
 * over the initial slot), since the first step may be skipped.
 * Errors: as zero_adam_step, plus EINVAL (bits not 8 or 4, null codes or
 * blocks, gather dtype) and EALIGN (codes or blocks not 8-byte aligned). */
int zero_adam_step_qgather(const zero_state *state, const float *g_dev, int64_t valid_len,
                           const zero_hparams *hp, const zero_ctrl *ctrl_dev, void *gather_dev,
                           int32_t gather_dtype, int64_t offset, int32_t bits, void *codes_dev,
                           zero_qblock *blocks_dev, void *stream);

/* Cast ("CMU 11-868 L18", Mechanism 1 steps 5-6; lesson Stage 1 step 4):
 * gather_dev[offset + i] = RNE_dtype(master_dev[i]) for i < valid_len,
 * unconditionally (also used to fill the initial parameters). */
int zero_cast_to_gather(const float *master_dev, int64_t valid_len, void *gather_dev,
                        int32_t dtype, int64_t offset, void *stream);

/* Fused single pass (clipping off): reduce + norm/overflow partials + Adam +
 * cast, reading each contribution and each state word once.  Because the
 * skip decision is only known after every element has been summed, the
 * state is double-buffered in the paired layout (zero_state above): the
 * kernel reads the set ctrl->cur names and writes the other one;
 * zero_grad_norm_overflow with pingpong = 1 then makes the written set
 * current, or keeps the old one on a skipped step, and zero_fused_restore
 * rewrites the gather slot from the kept master on a skipped step.  Bias
 * correction uses t+1.  pair: a paired state (one 16-byte aligned buffer of
 * zero_pair_elems(valid_len) floats, see zero_state).  Requires hp->max_grad_norm <= 0
 * (EINVAL otherwise).  Other arguments as in zero_reduce_grads and
 * zero_adam_step; gather_dev must not be NULL. */
int zero_fused_step(const void *contrib_dev, int32_t contrib_dtype, int32_t nranks,
                    int64_t stride, const zero_state *pair, int64_t valid_len, void *gather_dev,
                    int32_t gather_dtype, int64_t offset, const zero_hparams *hp,
                    const zero_ctrl *ctrl_dev, void *ws_dev, size_t ws_bytes, void *stream);

/* zero_fused_step with the contribution rows given as a table of row
 * pointers, as in zero_reduce_grads_rows (same requirements on rows_dev and
 * nranks <= ZERO_MAX_RANKS): the one-pass reduce-scatter + Adam + cast of a
 * rank that reads the N ranks' slices where they lie.  Bit-identical to
 * zero_fused_step on the same rows.  Speed depends on where the rows lie:
 * on the 13B shard, rows that start at the same offset in their pages (N
 * separate, equally aligned allocations) ran about 4% slower than rows in
 * one [N, stride] buffer, and row k started k * 4 KiB into its allocation
 * recovered about half of that; the table itself costs 0.3%. */
int zero_fused_step_rows(const void *const *rows_dev, int32_t contrib_dtype, int32_t nranks,
                         const zero_state *pair, int64_t valid_len, void *gather_dev,
                         int32_t gather_dtype, int64_t offset, const zero_hparams *hp,
                         const zero_ctrl *ctrl_dev, void *ws_dev, size_t ws_bytes, void *stream);

/* After a fused step's zero_grad_norm_overflow: if ctrl->skip, rewrite
 * gather_dev[offset + i] from the current master of the paired state;
 * otherwise every workgroup returns at once. */
int zero_fused_restore(const zero_state *pair, int64_t valid_len, void *gather_dev,
                       int32_t dtype, int64_t offset, const zero_ctrl *ctrl_dev, void *stream);

/* Copies a flat state (valid_len floats per array) into the current set of a
 * paired state (set ctrl->cur), e.g. to load initial or checkpointed weights. */
int zero_pair_store(const zero_state *flat, const zero_state *pair, int64_t valid_len,
                    const zero_ctrl *ctrl_dev, void *stream);

/* Copies the current set of a paired state out to a flat state. */
int zero_pair_load(const zero_state *pair, const zero_state *flat, int64_t valid_len,
                   const zero_ctrl *ctrl_dev, void *stream);

/* ---- Several ranks' shards on one GPU ---------------------------------------
 * "zero-stages-simulation" README (riteshverma), the per-stage data-flow
 * table: its toy runs every rank of the data-parallel group in one process,
 * each rank owning one shard.  When several ranks' shards share a GPU and
 * each is small (the toy's 32 shards have ten tiles each), one launch per
 * shard leaves the chip idle between launches.  The calls below are
 * zero_fused_step and zero_fused_restore (fused path), and zero_reduce_grads
 * and zero_adam_step (two-pass path), for up to ZERO_MAX_RANKS shards at
 * once, as one launch per ZERO_BATCH_SHARDS shards: every shard's results are
 * bit-identical to its own calls'.  Between the two launches of a step,
 * zero_grad_norm_overflow over the shards' workspaces and ctrl blocks takes
 * the shared decision. */

/* One shard of a batched call: what the single-shard calls take for it.  Each
 * call reads only the fields it needs (see below). */
typedef struct zero_shard {
    const void *contrib_dev; /* [nranks, stride] 16-bit rows, 16-byte aligned */
    int64_t stride;          /* elements between rows: >= valid_len, a multiple of 8 */
    float *pair_dev;         /* fused path: paired state, zero_pair_elems(valid_len) floats,
                                16-byte aligned (the buffer zero_state's master points to) */
    int64_t valid_len;       /* at most one launch of tiles (see the calls) */
    int64_t offset;          /* the shard's slot in the gather buffer, in elements */
    zero_ctrl *ctrl_dev;     /* the shard's (rank's) ctrl block */
    void *ws_dev;            /* zero_workspace_bytes(valid_len) bytes, 16-byte aligned */
    size_t ws_bytes;
    zero_state state;        /* two-pass path: flat master, m, v of valid_len floats */
    float *g_dev;            /* two-pass path: the reduced gradient, valid_len floats,
                                16-byte aligned */
} zero_shard;

#define ZERO_BATCH_SHARDS 32 /* most shards in one launch of a batched call */

/* zero_fused_step for each of the nshards (1..ZERO_MAX_RANKS) shards in the
 * host array `shards` (contrib_dev, stride, pair_dev, valid_len, offset,
 * ctrl_dev, ws_dev and ws_bytes are read), which share contrib_dtype, nranks,
 * the gather buffer and its dtype, and hp (no clipping).  The shards' states,
 * slots, ctrl blocks and workspaces must not overlap.  Every shard is checked
 * before anything is enqueued, with the errors of zero_fused_step; a shard of
 * more than zero_launch_tiles(nranks) tiles returns ERANGE (step it with its
 * own calls).  Shards with valid_len 0 launch nothing; so in the calls below. */
int zero_fused_step_shards(const zero_shard *shards, int32_t nshards, int32_t contrib_dtype,
                           int32_t nranks, void *gather_dev, int32_t gather_dtype,
                           const zero_hparams *hp, void *stream);

/* zero_fused_restore for each shard after the decision (only pair_dev,
 * valid_len, offset and ctrl_dev are read; at most ZERO_LAUNCH_TILES tiles
 * per shard). */
int zero_fused_restore_shards(const zero_shard *shards, int32_t nshards, void *gather_dev,
                              int32_t gather_dtype, void *stream);

/* zero_reduce_grads for each shard (contrib_dev, stride, valid_len, ctrl_dev,
 * ws_dev, ws_bytes and g_dev are read; at most zero_launch_tiles(nranks)
 * tiles per shard, ERANGE otherwise). */
int zero_reduce_grads_shards(const zero_shard *shards, int32_t nshards, int32_t contrib_dtype,
                             int32_t nranks, void *stream);

/* zero_adam_step for each shard after the decision (state, g_dev, valid_len,
 * offset and ctrl_dev are read; at most ZERO_LAUNCH_TILES tiles per shard);
 * gather_dev NULL writes no slot.  Clipping as in zero_adam_step. */
int zero_adam_step_shards(const zero_shard *shards, int32_t nshards, const zero_hparams *hp,
                          void *gather_dev, int32_t gather_dtype, void *stream);

/* ---- Block-quantised payloads (ZeRO++) --------------------------------------
 * "CMU 11-868 L18", Other memory optimizations: ZeRO++ quantises the
 * parameters of the forward all-gather block-wise from 16 bits to INT8 with a
 * zero point, and the gradient reduce-scatter to INT8 or INT4.  The page
 * gives neither block size nor rounding; this library's reading:
 *   blocks of ZERO_QBLOCK consecutive elements from the start of the buffer
 *   (the last may be short), Q = 2^bits - 1, and per block
 *     lo = min(0, min x), hi = max(0, max x),
 *     scale = (hi - lo) / Q (1 when that is 0),
 *     zero  = clamp(rint(-lo / scale), 0, Q),
 *     code  = clamp(rint(x * (1 / scale)) + zero, 0, Q),
 *   each operation one fp32 rounding, rint half to even: per block, the
 *   affine quantisation of PyTorch (MinMaxObserver's scale and zero point,
 *   quantize_per_tensor's codes, quint4x2's nibble order), which floors the
 *   scale at fp32 epsilon instead.  Real 0 is exact; |x - value| <= scale / 2
 *   up to the roundings.  A block holding inf or
 *   NaN, or whose scale overflows, gets scale NaN, zero 0 and codes 0, so it
 *   dequantises to NaN and a downstream overflow check still fires.
 *   Codes: bits = 8, one byte per element; bits = 4, two per byte, the
 *   even-indexed element in the low nibble.
 * codes and blocks must be 8-byte aligned; a 16-bit src or dst needs only
 * 2-byte alignment (a parameter slot at any offset), with vector accesses
 * where its alignment allows. */

/* Blocks of a quantised buffer of len elements: ceil(len / ZERO_QBLOCK). */
size_t zero_qblock_count(int64_t len);

/* Code bytes of a quantised buffer of len elements: len (8 bits) or
 * ceil(len / 2) (4 bits); 0 for len <= 0. */
size_t zero_qcode_bytes(int64_t len, int32_t bits);

/* Quantises len 16-bit values (dtype) at src_dev into codes_dev
 * (zero_qcode_bytes) and blocks_dev (zero_qblock_count entries): a sender's
 * gradient slice for a quantised reduce-scatter, or a rank's parameter slot
 * for a quantised all-gather.  Deterministic (no atomics).
 * Errors: EINVAL (null, dtype, bits not 8 or 4), EALIGN, ERANGE. */
int zero_quantize_blocks(const void *src_dev, int32_t dtype, int64_t len, int32_t bits,
                         void *codes_dev, zero_qblock *blocks_dev, void *stream);

/* dst_dev[i] = RNE_dtype(scale_b * (code_i - zero_b)), b = i / ZERO_QBLOCK:
 * the receiving side of a quantised all-gather. */
int zero_dequantize_blocks(const void *codes_dev, const zero_qblock *blocks_dev, int32_t bits,
                           int64_t len, void *dst_dev, int32_t dtype, void *stream);

/* zero_reduce_grads over quantised contributions: row k is codes_dev[k] with
 * blocks_dev[k], each quantised from the start of this rank's slice (the
 * sender quantises every destination's slice on its own), so block b covers
 * shard elements [b * ZERO_QBLOCK, ...).  Each value is dequantised as above
 * (one fp32 rounding) and the N values are summed in fp32 in rank order;
 * overflow flag, 1/(N*S) and the norm partials are as in zero_reduce_grads.
 * codes_dev and blocks_dev are host arrays of nranks device pointers
 * (nranks <= ZERO_MAX_RANKS), copied into the launch.
 * Errors: EINVAL (null table or row, bits, nranks), EALIGN, ESPACE, ERANGE. */
int zero_reduce_grads_q(const void *const *codes_dev, const zero_qblock *const *blocks_dev,
                        int32_t bits, int32_t nranks, int64_t valid_len,
                        const zero_ctrl *ctrl_dev, float *g_dev, void *ws_dev, size_t ws_bytes,
                        void *stream);

/* zero_fused_step over quantised contributions (rows as in
 * zero_reduce_grads_q): the one-pass step of a rank whose gradient
 * reduce-scatter arrives as INT8 or INT4 blocks. */
int zero_fused_step_q(const void *const *codes_dev, const zero_qblock *const *blocks_dev,
                      int32_t bits, int32_t nranks, const zero_state *pair, int64_t valid_len,
                      void *gather_dev, int32_t gather_dtype, int64_t offset,
                      const zero_hparams *hp, const zero_ctrl *ctrl_dev, void *ws_dev,
                      size_t ws_bytes, void *stream);

/* zero_fused_step (strided rows) that also writes the quantised all-gather
 * payload of the rank's new parameters ("CMU 11-868 L18", Other memory
 * optimizations: ZeRO++ quantises the parameters block-wise to INT8 with a
 * zero point for the forward all-gather).  Block b covers shard elements
 * [b * ZERO_QBLOCK, ...), which is exactly one tile of the pass, so the
 * block's range, record and codes come out of the same pass as the new
 * parameters: codes_dev (zero_qcode_bytes(valid_len, bits)) and blocks_dev
 * (zero_qblock_count(valid_len) records) equal, bit for bit, what
 * zero_quantize_blocks(gather_dtype, bits) would write from the 16-bit slot
 * after the step.  gather_dev may be NULL: then no 16-bit slot is written
 * (every rank rebuilds the parameters from the gathered payload with
 * zero_dequantize_blocks, this one included); gather_dtype still names the
 * 16-bit format that is quantised.  bits is 8 (the page's choice) or 4.
 * On a skipped step, zero_fused_restore_q (not zero_fused_restore) rewrites
 * the slot and the payload.  Other arguments and errors as in zero_fused_step
 * and zero_quantize_blocks (codes_dev and blocks_dev 8-byte aligned). */
int zero_fused_step_qgather(const void *contrib_dev, int32_t contrib_dtype, int32_t nranks,
                            int64_t stride, const zero_state *pair, int64_t valid_len,
                            void *gather_dev, int32_t gather_dtype, int64_t offset, int32_t bits,
                            void *codes_dev, zero_qblock *blocks_dev, const zero_hparams *hp,
                            const zero_ctrl *ctrl_dev, void *ws_dev, size_t ws_bytes,
                            void *stream);

/* zero_fused_step_qgather with the contribution rows given as a table of row
 * pointers (rows_dev as in zero_reduce_grads_rows, nranks <= ZERO_MAX_RANKS).
 * Bit-identical to zero_fused_step_qgather on the same rows.  Errors: those
 * of zero_fused_step_rows for the table, then those of
 * zero_fused_step_qgather for the rest. */
int zero_fused_step_rows_qgather(const void *const *rows_dev, int32_t contrib_dtype,
                                 int32_t nranks, const zero_state *pair, int64_t valid_len,
                                 void *gather_dev, int32_t gather_dtype, int64_t offset,
                                 int32_t bits, void *codes_dev, zero_qblock *blocks_dev,
                                 const zero_hparams *hp, const zero_ctrl *ctrl_dev, void *ws_dev,
                                 size_t ws_bytes, void *stream);

/* zero_fused_step_qgather over quantised contributions (qcodes_dev,
 * qblocks_dev and qbits as codes_dev, blocks_dev and bits of
 * zero_reduce_grads_q): ZeRO++ end to end in one pass, with the gradient
 * reduce-scatter arriving as INT8 or INT4 blocks and the parameters leaving
 * as the bits-bit all-gather payload (codes_dev, blocks_dev).  The two widths
 * are independent.  Errors: those of zero_fused_step_q for the quantised
 * rows (qbits, tables, 8-byte alignment), then those of
 * zero_fused_step_qgather for the rest. */
int zero_fused_step_q_qgather(const void *const *qcodes_dev, const zero_qblock *const *qblocks_dev,
                              int32_t qbits, int32_t nranks, const zero_state *pair,
                              int64_t valid_len, void *gather_dev, int32_t gather_dtype,
                              int64_t offset, int32_t bits, void *codes_dev,
                              zero_qblock *blocks_dev, const zero_hparams *hp,
                              const zero_ctrl *ctrl_dev, void *ws_dev, size_t ws_bytes,
                              void *stream);

/* After a zero_fused_step_qgather's (or its _rows/_q form's)
 * zero_grad_norm_overflow: if ctrl->skip,
 * rewrite the slot (when gather_dev is not NULL) and the payload from the
 * current master of the paired state, as the step would have written them;
 * otherwise every workgroup returns at once. */
int zero_fused_restore_q(const zero_state *pair, int64_t valid_len, void *gather_dev,
                         int32_t dtype, int64_t offset, int32_t bits, void *codes_dev,
                         zero_qblock *blocks_dev, const zero_ctrl *ctrl_dev, void *stream);

/* ---- Allocation-free step ---------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): one rank's
 * whole fused step without a workspace argument.  It is zero_fused_step
 * followed by zero_grad_norm_overflow (this rank alone, pingpong = 1) and
 * zero_fused_restore, with the per-tile norm and overflow partials kept in
 * a static device array inside the library (ZERO_NOALLOC_MAX_LEN /
 * ZERO_TILE + 256 partials of ZERO_PARTIAL_BYTES, about 16 MiB, held by every
 * GPU the library runs on until the process ends); the results equal those
 * three calls' bit for bit.  The caller passes inputs, state, slot and ctrl
 * as for zero_fused_step; the call allocates nothing.  All calls on one GPU
 * share that array: calls that overlap on one GPU (on different streams, or
 * from different threads without ordering) race, so they must be ordered.
 * Errors: those of zero_fused_step, ERANGE for valid_len above
 * ZERO_NOALLOC_MAX_LEN (nothing enqueued), EHIP if the array's device
 * address cannot be obtained (first call on each device). */
#define ZERO_NOALLOC_MAX_LEN 2147483648LL
int zero_fused_step_noalloc(const void *contrib_dev, int32_t contrib_dtype, int32_t nranks,
                            int64_t stride, const zero_state *pair, int64_t valid_len,
                            void *gather_dev, int32_t gather_dtype, int64_t offset,
                            const zero_hparams *hp, zero_ctrl *ctrl_dev, void *stream);

/* Message for the last nonzero return on the calling thread ("" if none). */
const char *zero_last_error(void);

#ifdef __cplusplus
}
#endif

#endif
