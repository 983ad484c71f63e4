/* A plain C consumer of the shard-step C ABI (include/zero_shard.h): no Python,
 * no torch.  Device memory comes from the HIP runtime's C API, inputs from the
 * seeded host generator (libsynth_cpu), and every step of the path from
 * libzero_shard.
 *
 *   shard_step_demo host        partition, size queries and argument checks
 *                               (needs no GPU)
 *   shard_step_demo gpu FILE    runs five ranks' steps of a small workload on
 *                               the GPU and writes their results to FILE for
 *                               the test to compare with the oracle:
 *     rank 2, fused path, dynamic loss scale, +inf in contribution 1 at step 2
 *     rank 1, two-pass path, clipping at 0.01
 *     rank 0, fused path as rank 2, writing only the INT8 all-gather payload
 *     rank 2, two-pass path as rank 1, writing the slot and an INT4 payload
 *     rank 1, fused path as rank 2 over INT8-quantised contributions, writing
 *       only the INT8 payload (ZeRO++ end to end)
 *     all three ranks at once through the batched calls, fused path as rank 2
 *       (the +inf in rank 1's contribution 2), then two-pass path as rank 1
 *   all of Psi = 120,007 (fp16) over N = 3 ranks, 3 steps.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zero_shard.h"

/* libsynth_cpu (the seeded input generator shared by both sides of the tests) */
void synth_contrib_rows(uint64_t seed, uint32_t step, int32_t n, int32_t dtype, double sigma,
                        double scale, uint64_t outlier_thresh, double outlier_mult, int64_t idx0,
                        int64_t len, int64_t stride, uint16_t *out);
void synth_master_range(uint64_t seed, double sigma, int64_t idx0, int64_t len, float *out);
void synth_param_range(uint64_t seed, double sigma, int32_t dtype, int64_t idx0, int64_t len,
                       uint16_t *out);

enum { PSI = 120007, NR = 3, STEPS = 3 };
static const double SCALE = 1024.0;

#define HIP(x)                                                                          \
    do {                                                                                \
        hipError_t e_ = (x);                                                            \
        if (e_ != hipSuccess) {                                                         \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
            exit(3);                                                                    \
        }                                                                               \
    } while (0)

#define ZERO(x)                                                                          \
    do {                                                                                 \
        int rc_ = (x);                                                                   \
        if (rc_ != ZERO_OK) {                                                            \
            fprintf(stderr, "%s:%d %s -> %d: %s\n", __FILE__, __LINE__, #x, rc_, zero_last_error()); \
            exit(4);                                                                     \
        }                                                                                \
    } while (0)

static int host_mode(void) {
    int64_t shard, off, valid;
    ZERO(zero_partition(PSI, NR, 2, &shard, &off, &valid));
    if (shard != 40003 || off != 80006 || valid != 40001) return fprintf(stderr, "partition\n"), 1;
    ZERO(zero_partition(10, 7, 6, &shard, &off, &valid));
    if (shard != 2 || off != 12 || valid != 0) return fprintf(stderr, "empty rank\n"), 1;
    if (zero_ctrl_bytes() != 128 || zero_workspace_bytes(4097) != (3 + 256) * 16 ||
        zero_pair_elems(4097) != 18 * 2048 || zero_qcode_bytes(5, 4) != 3)
        return fprintf(stderr, "sizes\n"), 1;
    if (zero_partition(0, 3, 0, &shard, &off, &valid) != ZERO_EINVAL || zero_last_error()[0] == 0)
        return fprintf(stderr, "error path\n"), 1;
    if (zero_reduce_grads(NULL, ZERO_F16, 3, 64, 64, NULL, NULL, NULL, 0, NULL) != ZERO_EINVAL)
        return fprintf(stderr, "validation\n"), 1;
    printf("host ok\n");
    return 0;
}

/* One rank's STEPS steps; appends ctrl after each step, then master, m, v
 * (valid floats each), the slot (valid 16-bit words) unless slot is 0, and
 * with qbits (8 or 4) the quantised all-gather payload: codes
 * (zero_qcode_bytes) and block records (zero_qblock_count of them).  With
 * cbits (8 or 4, fused path only) each contribution row is block-quantised on
 * the device (zero_quantize_blocks) and the step reads the quantised rows. */
static void run_rank(FILE *f, int32_t rank, float max_grad_norm, int inject, int slot,
                     int32_t qbits, int32_t cbits) {
    int64_t shard, off, valid;
    ZERO(zero_partition(PSI, NR, rank, &shard, &off, &valid));
    const int64_t stride = (shard + 63) / 64 * 64;
    const int fused = !(max_grad_norm > 0.0f);
    zero_hparams hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.0f, max_grad_norm,
                       fused ? ZERO_SCALER_DYNAMIC : ZERO_SCALER_STATIC, 1.0f, 1000};
    const float loss_scale = (float)SCALE;

    uint16_t *C = malloc(sizeof(uint16_t) * NR * stride);
    float *p0 = malloc(sizeof(float) * valid);
    uint16_t *gather = malloc(sizeof(uint16_t) * PSI);
    synth_master_range(0, 0.02, off, valid, p0);
    synth_param_range(0, 0.02, ZERO_F16, 0, PSI, gather);

    void *dC, *dG, *dCtrl, *dWs, *dg = NULL;
    float *flat[3], *pair[3], *pair_buf;
    const size_t ws_bytes = zero_workspace_bytes(valid);
    HIP(hipMalloc(&dC, sizeof(uint16_t) * NR * stride));
    HIP(hipMalloc(&dG, sizeof(uint16_t) * PSI));
    HIP(hipMalloc(&dCtrl, zero_ctrl_bytes()));
    HIP(hipMalloc(&dWs, ws_bytes));
    /* the paired state is one buffer; m and v start one and two tiles into it */
    HIP(hipMalloc((void **)&pair_buf, sizeof(float) * zero_pair_elems(valid)));
    for (int q = 0; q < 3; ++q) {
        HIP(hipMalloc((void **)&flat[q], sizeof(float) * valid));
        HIP(hipMemset(flat[q], 0, sizeof(float) * valid));
        pair[q] = pair_buf + q * ZERO_TILE;
    }
    HIP(hipMemcpy(flat[0], p0, sizeof(float) * valid, hipMemcpyHostToDevice));
    HIP(hipMemcpy(dG, gather, sizeof(uint16_t) * PSI, hipMemcpyHostToDevice));
    if (!fused) HIP(hipMalloc(&dg, sizeof(float) * valid));
    void *dCodes = NULL, *dBlocks = NULL;
    const size_t code_bytes = qbits ? zero_qcode_bytes(valid, qbits) : 0;
    const size_t nblk = qbits ? zero_qblock_count(valid) : 0;
    if (qbits) {
        HIP(hipMalloc(&dCodes, code_bytes));
        HIP(hipMalloc(&dBlocks, nblk * sizeof(zero_qblock)));
    }
    void *slot_dev = slot ? dG : NULL; /* NULL: no 16-bit slot is written */
    void *qc[NR] = {NULL}, *qb[NR] = {NULL}; /* quantised contribution rows */
    if (cbits) {
        for (int k = 0; k < NR; ++k) {
            HIP(hipMalloc(&qc[k], zero_qcode_bytes(valid, cbits)));
            HIP(hipMalloc(&qb[k], zero_qblock_count(valid) * sizeof(zero_qblock)));
        }
    }

    zero_state st_flat = {flat[0], flat[1], flat[2]}, st_pair = {pair[0], pair[1], pair[2]};
    ZERO(zero_ctrl_init(dCtrl, loss_scale, NULL));
    if (fused) ZERO(zero_pair_store(&st_flat, &st_pair, valid, dCtrl, NULL));
    for (uint32_t s = 1; s <= STEPS; ++s) {
        synth_contrib_rows(0, s, NR, ZERO_F16, 1e-3, SCALE, 0, 100.0, off, valid, stride, C);
        if (inject && s == 2) C[1 * stride + 123] = 0x7C00; /* +inf in contribution 1 */
        HIP(hipMemcpy(dC, C, sizeof(uint16_t) * NR * stride, hipMemcpyHostToDevice));
        void *ws_arr[1] = {dWs};
        int64_t len_arr[1] = {valid};
        zero_ctrl *ctrl_arr[1] = {dCtrl};
        if (cbits) {
            for (int k = 0; k < NR; ++k)
                ZERO(zero_quantize_blocks((uint16_t *)dC + k * stride, ZERO_F16, valid, cbits, qc[k],
                                          (zero_qblock *)qb[k], NULL));
            ZERO(zero_fused_step_q_qgather((const void *const *)qc, (const zero_qblock *const *)qb,
                                           cbits, NR, &st_pair, valid, slot_dev, ZERO_F16, off,
                                           qbits, dCodes, dBlocks, &hp, dCtrl, dWs, ws_bytes, NULL));
            ZERO(zero_grad_norm_overflow(1, ws_arr, len_arr, ctrl_arr, &hp, 1, NULL));
            ZERO(zero_fused_restore_q(&st_pair, valid, slot_dev, ZERO_F16, off, qbits, dCodes,
                                      dBlocks, dCtrl, NULL));
        } else if (fused && qbits) {
            ZERO(zero_fused_step_qgather(dC, ZERO_F16, NR, stride, &st_pair, valid, slot_dev,
                                         ZERO_F16, off, qbits, dCodes, dBlocks, &hp, dCtrl, dWs,
                                         ws_bytes, NULL));
            ZERO(zero_grad_norm_overflow(1, ws_arr, len_arr, ctrl_arr, &hp, 1, NULL));
            ZERO(zero_fused_restore_q(&st_pair, valid, slot_dev, ZERO_F16, off, qbits, dCodes,
                                      dBlocks, dCtrl, NULL));
        } else if (fused) {
            ZERO(zero_fused_step(dC, ZERO_F16, NR, stride, &st_pair, valid, dG, ZERO_F16, off, &hp,
                                 dCtrl, dWs, ws_bytes, NULL));
            ZERO(zero_grad_norm_overflow(1, ws_arr, len_arr, ctrl_arr, &hp, 1, NULL));
            ZERO(zero_fused_restore(&st_pair, valid, dG, ZERO_F16, off, dCtrl, NULL));
        } else {
            ZERO(zero_reduce_grads(dC, ZERO_F16, NR, stride, valid, dCtrl, dg, dWs, ws_bytes, NULL));
            ZERO(zero_grad_norm_overflow(1, ws_arr, len_arr, ctrl_arr, &hp, 0, NULL));
            if (qbits)
                ZERO(zero_adam_step_qgather(&st_flat, dg, valid, &hp, dCtrl, slot_dev, ZERO_F16, off,
                                            qbits, dCodes, dBlocks, NULL));
            else
                ZERO(zero_adam_step(&st_flat, dg, valid, &hp, dCtrl, dG, ZERO_F16, off, NULL));
        }
        zero_ctrl c;
        HIP(hipMemcpy(&c, dCtrl, sizeof c, hipMemcpyDeviceToHost));
        fwrite(&c, sizeof c, 1, f);
    }
    if (fused) ZERO(zero_pair_load(&st_pair, &st_flat, valid, dCtrl, NULL));
    HIP(hipDeviceSynchronize());
    float *out = malloc(sizeof(float) * valid);
    for (int q = 0; q < 3; ++q) {
        HIP(hipMemcpy(out, flat[q], sizeof(float) * valid, hipMemcpyDeviceToHost));
        fwrite(out, sizeof(float), (size_t)valid, f);
    }
    if (slot) {
        HIP(hipMemcpy(gather, dG, sizeof(uint16_t) * PSI, hipMemcpyDeviceToHost));
        fwrite(gather + off, sizeof(uint16_t), (size_t)valid, f);
    }
    if (qbits) {
        unsigned char *codes = malloc(code_bytes);
        zero_qblock *blocks = malloc(nblk * sizeof(zero_qblock));
        HIP(hipMemcpy(codes, dCodes, code_bytes, hipMemcpyDeviceToHost));
        HIP(hipMemcpy(blocks, dBlocks, nblk * sizeof(zero_qblock), hipMemcpyDeviceToHost));
        fwrite(codes, 1, code_bytes, f);
        fwrite(blocks, sizeof(zero_qblock), nblk, f);
        free(codes);
        free(blocks);
        HIP(hipFree(dCodes));
        HIP(hipFree(dBlocks));
    }
    for (int k = 0; k < NR && cbits; ++k) {
        HIP(hipFree(qc[k]));
        HIP(hipFree(qb[k]));
    }
    for (int q = 0; q < 3; ++q) HIP(hipFree(flat[q]));
    HIP(hipFree(pair_buf));
    HIP(hipFree(dC));
    HIP(hipFree(dG));
    HIP(hipFree(dCtrl));
    HIP(hipFree(dWs));
    if (dg) HIP(hipFree(dg));
    free(C);
    free(p0);
    free(gather);
    free(out);
}

/* All NR ranks' STEPS steps through the batched calls (one launch per pass
 * for all of them) with one shared decision per step; appends every rank's
 * ctrl after each step, then each rank's master, m, v (its valid floats
 * each), then the whole parameter buffer (PSI 16-bit words). */
static void run_batched(FILE *f, float max_grad_norm) {
    const int fused = !(max_grad_norm > 0.0f);
    zero_hparams hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.0f, max_grad_norm,
                       fused ? ZERO_SCALER_DYNAMIC : ZERO_SCALER_STATIC, 1.0f, 1000};
    zero_shard sh[NR];
    void *ws_arr[NR];
    int64_t len_arr[NR], off_arr[NR];
    zero_ctrl *ctrl_arr[NR];
    uint16_t *C[NR];
    float *bufs[NR][5]; /* flat master, m, v; g; paired buffer */
    uint16_t *gather = malloc(sizeof(uint16_t) * PSI);
    void *dG;
    synth_param_range(0, 0.02, ZERO_F16, 0, PSI, gather);
    HIP(hipMalloc(&dG, sizeof(uint16_t) * PSI));
    HIP(hipMemcpy(dG, gather, sizeof(uint16_t) * PSI, hipMemcpyHostToDevice));
    memset(sh, 0, sizeof sh);
    for (int r = 0; r < NR; ++r) {
        int64_t shard, off, valid;
        ZERO(zero_partition(PSI, NR, r, &shard, &off, &valid));
        const int64_t stride = (shard + 63) / 64 * 64;
        float *p0 = malloc(sizeof(float) * valid);
        synth_master_range(0, 0.02, off, valid, p0);
        C[r] = malloc(sizeof(uint16_t) * NR * stride);
        void *dC, *dWs;
        zero_ctrl *dCtrl;
        HIP(hipMalloc(&dC, sizeof(uint16_t) * NR * stride));
        HIP(hipMalloc((void **)&dCtrl, zero_ctrl_bytes()));
        HIP(hipMalloc(&dWs, zero_workspace_bytes(valid)));
        for (int q = 0; q < 4; ++q) {
            HIP(hipMalloc((void **)&bufs[r][q], sizeof(float) * valid));
            HIP(hipMemset(bufs[r][q], 0, sizeof(float) * valid));
        }
        HIP(hipMalloc((void **)&bufs[r][4], sizeof(float) * zero_pair_elems(valid)));
        HIP(hipMemcpy(bufs[r][0], p0, sizeof(float) * valid, hipMemcpyHostToDevice));
        ZERO(zero_ctrl_init(dCtrl, (float)SCALE, NULL));
        zero_state flat = {bufs[r][0], bufs[r][1], bufs[r][2]};
        zero_state pair = {bufs[r][4], bufs[r][4] + ZERO_TILE, bufs[r][4] + 2 * ZERO_TILE};
        if (fused) ZERO(zero_pair_store(&flat, &pair, valid, dCtrl, NULL));
        sh[r].contrib_dev = dC;
        sh[r].stride = stride;
        sh[r].pair_dev = bufs[r][4];
        sh[r].valid_len = valid;
        sh[r].offset = off;
        sh[r].ctrl_dev = dCtrl;
        sh[r].ws_dev = dWs;
        sh[r].ws_bytes = zero_workspace_bytes(valid);
        sh[r].state = flat;
        sh[r].g_dev = bufs[r][3];
        ws_arr[r] = dWs;
        len_arr[r] = valid;
        off_arr[r] = off;
        ctrl_arr[r] = dCtrl;
        free(p0);
    }
    for (uint32_t s = 1; s <= STEPS; ++s) {
        for (int r = 0; r < NR; ++r) {
            synth_contrib_rows(0, s, NR, ZERO_F16, 1e-3, SCALE, 0, 100.0, off_arr[r], len_arr[r],
                               sh[r].stride, C[r]);
            if (fused && r == 1 && s == 2) C[r][2 * sh[r].stride + 77] = 0x7C00; /* +inf */
            HIP(hipMemcpy((void *)sh[r].contrib_dev, C[r], sizeof(uint16_t) * NR * sh[r].stride,
                          hipMemcpyHostToDevice));
        }
        if (fused) {
            ZERO(zero_fused_step_shards(sh, NR, ZERO_F16, NR, dG, ZERO_F16, &hp, NULL));
            ZERO(zero_grad_norm_overflow(NR, ws_arr, len_arr, ctrl_arr, &hp, 1, NULL));
            ZERO(zero_fused_restore_shards(sh, NR, dG, ZERO_F16, NULL));
        } else {
            ZERO(zero_reduce_grads_shards(sh, NR, ZERO_F16, NR, NULL));
            ZERO(zero_grad_norm_overflow(NR, ws_arr, len_arr, ctrl_arr, &hp, 0, NULL));
            ZERO(zero_adam_step_shards(sh, NR, &hp, dG, ZERO_F16, NULL));
        }
        for (int r = 0; r < NR; ++r) {
            zero_ctrl c;
            HIP(hipMemcpy(&c, ctrl_arr[r], sizeof c, hipMemcpyDeviceToHost));
            fwrite(&c, sizeof c, 1, f);
        }
    }
    for (int r = 0; r < NR; ++r) {
        const int64_t valid = len_arr[r];
        zero_state pair = {bufs[r][4], bufs[r][4] + ZERO_TILE, bufs[r][4] + 2 * ZERO_TILE};
        if (fused) ZERO(zero_pair_load(&pair, &sh[r].state, valid, ctrl_arr[r], NULL));
        HIP(hipDeviceSynchronize());
        float *out = malloc(sizeof(float) * (valid ? valid : 1));
        for (int q = 0; q < 3; ++q) {
            HIP(hipMemcpy(out, bufs[r][q], sizeof(float) * valid, hipMemcpyDeviceToHost));
            fwrite(out, sizeof(float), (size_t)valid, f);
        }
        free(out);
    }
    HIP(hipMemcpy(gather, dG, sizeof(uint16_t) * PSI, hipMemcpyDeviceToHost));
    fwrite(gather, sizeof(uint16_t), PSI, f);
    for (int r = 0; r < NR; ++r) {
        for (int q = 0; q < 5; ++q) HIP(hipFree(bufs[r][q]));
        HIP(hipFree((void *)sh[r].contrib_dev));
        HIP(hipFree(sh[r].ws_dev));
        HIP(hipFree(ctrl_arr[r]));
        free(C[r]);
    }
    HIP(hipFree(dG));
    free(gather);
}

int main(int argc, char **argv) {
    if (argc >= 2 && strcmp(argv[1], "host") == 0) return host_mode();
    if (argc >= 3 && strcmp(argv[1], "gpu") == 0) {
        FILE *f = fopen(argv[2], "wb");
        if (!f) return 2;
        run_rank(f, 2, 0.0f, 1, 1, 0, 0);
        run_rank(f, 1, 0.01f, 0, 1, 0, 0);
        run_rank(f, 0, 0.0f, 1, 0, 8, 0);
        run_rank(f, 2, 0.01f, 0, 1, 4, 0);
        run_rank(f, 1, 0.0f, 1, 0, 8, 8);
        run_batched(f, 0.0f);
        run_batched(f, 0.01f);
        fclose(f);
        printf("gpu ok\n");
        return 0;
    }
    fprintf(stderr, "usage: %s host | gpu FILE\n", argv[0]);
    return 2;
}
