/*
 * oracle_omp.c -- the oracle's timing mode, TEST INFRASTRUCTURE ONLY (like
 * oracle.c, which it includes unchanged; only the benchmark's CPU-baseline leg
 * calls it).
 *
 * Embedding columns are independent (each owns its table, its output slice and
 * its gradient slice), so the reference oracle's forward and backward run here
 * column by column, the columns spread over OpenMP threads.  Each column is the
 * reference call with one column: its CSR offsets are the slice of the batch's
 * offsets (positions stay absolute, so ids / fvals are shared), its output and
 * its upstream gradient are contiguous [B, dim] arrays of its own.  No
 * arithmetic differs from the single-threaded oracle.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC oracle_omp.c -o liboracle_omp.so -lm
 */
#include <omp.h>

#include "oracle.c"

/*
 * Y_col[c]  fp32 [B, dim_c]  pooled output of column c
 * G_col[c]  fp32 [B, dim_c]  upstream gradient of column c (read when training)
 * opt, lr, eps               row update as in oracle_backward
 * Returns the number of threads the parallel loop ran on.
 */
int32_t oracle_step_columns(const oracle_col *cols, int32_t C, int32_t B, const int32_t *offsets,
                            const int64_t *ids, const float *fvals, float *const *Y_col,
                            const float *const *G_col, int32_t training, int32_t opt, double lr,
                            double eps, int32_t threads)
{
    int32_t used = 1;
#pragma omp parallel num_threads(threads)
    {
#pragma omp single
        used = (int32_t)omp_get_num_threads();
#pragma omp for schedule(dynamic, 1)
        for (int32_t c = 0; c < C; c++) {
            const int32_t *off = offsets + (int64_t)c * B;
            oracle_forward(&cols[c], 1, B, off, ids, fvals, NULL, NULL, NULL, Y_col[c], NULL,
                           NULL, NULL);
            if (training)
                oracle_backward(&cols[c], 1, B, off, ids, fvals, NULL, NULL, NULL, G_col[c], opt,
                                lr, eps, NULL, NULL, NULL, NULL, INT64_MAX);
        }
    }
    return used;
}
