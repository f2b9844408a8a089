/*
 * fp64 CPU oracle for the mixed-adapter LoRA linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
 * GPU path is checked against.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header, table
 * or constant with the HIP library.
 *
 * What it computes, per token row t (in the original row order):
 *
 *   y[t,n] = sum_{i<d_in} x[t,i] * W[i,n]                     (ascending i)
 *   if row t names a usable adapter a:
 *     u[j]     = sum_{i<d_in} x[t,i] * A_a[i,j]     for j < r_a   (ascending i)
 *     delta[n] = sum_{j<r_a}  u[j] * B_a[j,n]                     (ascending j)
 *     y[t,n]  += s_a * delta[n]
 *
 * Sources:
 *  - "Serving multiple LoRAs: segmented matrix multiplies and adapter
 *    scheduling", section "Not merging the weights, computing in batches":
 *    the forward y = xW + s(xA)B with A of shape d x r and B of shape r x d',
 *    and the per-request loop (one product per request) used as the structure.
 *  - "LoRAX, in depth", section "Computing a batch that mixes adapters": the
 *    same row-vector form, s = alpha / r, the base product over all tokens and
 *    y += scale[aid] * ((x A) B) per adapter, with "no adapter" rows skipped.
 *  - "Multi-LoRA Serving 与 Adapter 隔离", runnable grouped-batch experiment:
 *    each row gets only its own adapter; rows without one get x W.
 *
 * Every product and sum is carried out in IEEE double.  Inputs are read in
 * their storage type (fp32, or bf16 stored as the upper 16 bits of an fp32)
 * and widened exactly to double.  A usable adapter is a slot index
 * 0 <= id < n_slots whose rank is > 0; any other id (the "no adapter" marker
 * -1, an out-of-range id, an empty slot) yields the base row only.
 *
 * Rows may be processed in blocks that share one pass over W, purely for
 * cache reuse: each y[t,n] is still accumulated in ascending i exactly as the
 * per-row formula above states.  Threads split the list of rows; a row is
 * computed by one thread only, so results do not depend on the thread count.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* Exact widening of one stored element to double. */
static double widen(int dtype, const void *base, int64_t idx) {
    if (dtype == ORACLE_F32) return (double)((const float *)base)[idx];
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

typedef struct {
    int dtype;
    const void *x;           /* [T, d_in] row-major                           */
    int64_t d_in, d_out;
    const void *W;           /* [d_in, d_out] row-major                       */
    const int32_t *ids;      /* [T]: adapter slot per token row               */
    const int64_t *rows;     /* rows to evaluate (indices into x / ids)       */
    int64_t n_rows;
    const void *const *A;    /* per slot: [d_in, ranks[s]] row-major or NULL  */
    const void *const *B;    /* per slot: [ranks[s], d_out] row-major or NULL */
    const int32_t *ranks;    /* per slot true rank, 0 = empty slot            */
    const double *scales;    /* per slot s                                    */
    int32_t n_slots;
    int32_t u_stride;        /* columns of u_out                              */
    double *y_out;           /* [n_rows, d_out]                               */
    double *u_out;           /* [n_rows, u_stride] or NULL                    */
    double *delta_out;       /* [n_rows, d_out] or NULL                       */
    int64_t row_block;
    int n_threads;
    int thread_id;
} job_t;

static int usable(const job_t *j, int32_t id) {
    return id >= 0 && id < j->n_slots && j->ranks[id] > 0 && j->A[id] && j->B[id];
}

static void *run_rows(void *arg) {
    const job_t *j = (const job_t *)arg;
    const int64_t d_in = j->d_in, d_out = j->d_out;
    double *wrow = (double *)malloc(sizeof(double) * (size_t)d_out);
    double *xv = (double *)malloc(sizeof(double) * (size_t)j->row_block);
    double *u = NULL, *delta = (double *)malloc(sizeof(double) * (size_t)d_out);
    int32_t max_r = 0;
    for (int32_t s = 0; s < j->n_slots; ++s)
        if (j->ranks[s] > max_r) max_r = j->ranks[s];
    u = (double *)malloc(sizeof(double) * (size_t)(max_r > 0 ? max_r : 1));

    const int64_t n_blocks = (j->n_rows + j->row_block - 1) / j->row_block;
    for (int64_t blk = j->thread_id; blk < n_blocks; blk += j->n_threads) {
        const int64_t r0 = blk * j->row_block;
        const int64_t nb = (j->n_rows - r0 < j->row_block) ? j->n_rows - r0 : j->row_block;

        /* Base term: y[t,n] = sum_i x[t,i] W[i,n], ascending i. */
        for (int64_t b = 0; b < nb; ++b) {
            double *y = j->y_out + (r0 + b) * d_out;
            for (int64_t n = 0; n < d_out; ++n) y[n] = 0.0;
        }
        for (int64_t i = 0; i < d_in; ++i) {
            for (int64_t n = 0; n < d_out; ++n) wrow[n] = widen(j->dtype, j->W, i * d_out + n);
            for (int64_t b = 0; b < nb; ++b) xv[b] = widen(j->dtype, j->x, j->rows[r0 + b] * d_in + i);
            for (int64_t b = 0; b < nb; ++b) {
                double *y = j->y_out + (r0 + b) * d_out;
                const double xi = xv[b];
                for (int64_t n = 0; n < d_out; ++n) y[n] += xi * wrow[n];
            }
        }

        /* Low-rank term, row by row: shrink u = x A, expand delta = u B. */
        for (int64_t b = 0; b < nb; ++b) {
            const int64_t t = j->rows[r0 + b];
            const int32_t id = j->ids[t];
            double *y = j->y_out + (r0 + b) * d_out;
            double *uo = j->u_out ? j->u_out + (r0 + b) * j->u_stride : NULL;
            double *dout = j->delta_out ? j->delta_out + (r0 + b) * d_out : NULL;
            if (uo)
                for (int32_t c = 0; c < j->u_stride; ++c) uo[c] = 0.0;
            if (dout)
                for (int64_t n = 0; n < d_out; ++n) dout[n] = 0.0;
            if (!usable(j, id)) continue;
            const int32_t r = j->ranks[id];
            const void *A = j->A[id], *B = j->B[id];
            for (int32_t c = 0; c < r; ++c) {
                double acc = 0.0;
                for (int64_t i = 0; i < d_in; ++i)
                    acc += widen(j->dtype, j->x, t * d_in + i) * widen(j->dtype, A, i * r + c);
                u[c] = acc;
            }
            for (int64_t n = 0; n < d_out; ++n) {
                double acc = 0.0;
                for (int32_t c = 0; c < r; ++c) acc += u[c] * widen(j->dtype, B, (int64_t)c * d_out + n);
                delta[n] = acc;
            }
            const double s = j->scales[id];
            for (int64_t n = 0; n < d_out; ++n) y[n] += s * delta[n];
            if (uo)
                for (int32_t c = 0; c < r && c < j->u_stride; ++c) uo[c] = u[c];
            if (dout)
                for (int64_t n = 0; n < d_out; ++n) dout[n] = delta[n];
        }
    }
    free(wrow);
    free(xv);
    free(u);
    free(delta);
    return NULL;
}

/*
 * Evaluate the rows listed in `rows`.  Returns 0 on success, -1 on a bad
 * argument.  y_out receives the full output row in fp64; u_out (optional)
 * the rank-width shrink result (zero beyond the slot's rank and for rows
 * without an adapter); delta_out (optional) the unscaled low-rank product.
 */
int oracle_lora_rows(int dtype, const void *x, int64_t d_in, int64_t d_out, const void *W,
                     const int32_t *ids, const int64_t *rows, int64_t n_rows,
                     const void *const *A, const void *const *B, const int32_t *ranks,
                     const double *scales, int32_t n_slots, double *y_out, double *u_out,
                     int32_t u_stride, double *delta_out, int n_threads) {
    if ((dtype != ORACLE_F32 && dtype != ORACLE_BF16) || !x || !W || !ids || !rows || !y_out)
        return -1;
    if (d_in <= 0 || d_out <= 0 || n_rows < 0 || n_slots < 0) return -1;
    if (n_slots > 0 && (!A || !B || !ranks || !scales)) return -1;
    if (u_out && u_stride <= 0) return -1;
    if (n_threads < 1) n_threads = 1;
    if (n_rows == 0) return 0;

    job_t base = {dtype, x, d_in, d_out, W, ids, rows, n_rows, A, B, ranks, scales, n_slots,
                  u_stride, y_out, u_out, delta_out, 8, n_threads, 0};
    const int64_t n_blocks = (n_rows + base.row_block - 1) / base.row_block;
    if (n_threads > n_blocks) n_threads = (int)n_blocks;
    base.n_threads = n_threads;

    job_t *jobs = (job_t *)malloc(sizeof(job_t) * (size_t)n_threads);
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    for (int k = 0; k < n_threads; ++k) {
        jobs[k] = base;
        jobs[k].thread_id = k;
    }
    for (int k = 1; k < n_threads; ++k) pthread_create(&th[k], NULL, run_rows, &jobs[k]);
    run_rows(&jobs[0]);
    for (int k = 1; k < n_threads; ++k) pthread_join(th[k], NULL);
    free(jobs);
    free(th);
    return 0;
}
