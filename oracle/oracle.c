/*
 * oracle.c -- plain, slow CPU oracle of the fused multi-column embedding stage.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header, table or constant generator with the
 * HIP library.
 *
 * What it computes (one embedding column = one table; RECom explainer, the
 * paragraph "Why this problem is worth solving": the index comes from a hash or
 * a bucket, out-of-range indices are dropped, a default stands in for a
 * missing feature, and the rows are looked up and reduced to one vector):
 *
 *   transform  HASH      valid iff id_lo <= id < id_hi, row = splitmix64(id) mod rows
 *              IDENTITY  valid iff 0 <= id < rows,      row = id
 *              BUCKET    valid iff x is not NaN,        row = #{ j : b_j <= x }
 *              KEYED     row handed in by the keyed-table step (or DEFAULT / dropped)
 *   forward    Y[s, p] = sum over the bag's valid positions r of w_r * E[i_r, p]
 *              (RecIS Sec. 3.2 "Index-aware segment reduction", Algorithm 1,
 *              forward half); w_r = v_r (sum) or v_r / n (mean), with v_r the
 *              caller's per-position weight (1 when none is given) and n the
 *              valid positions including DEFAULT ones.  A bag with no valid
 *              position (a missing feature) gives the zero vector, or, when the
 *              column names a default row, that row (RECom explainer: a default
 *              fills in a missing feature, and RECom merges this empty-row filling
 *              into the lookup): the bag then reads as one position at that row
 *              with weight 1, in the forward and in the backward.
 *   backward   dE[u] = sum over contributors r with i_r = u of w_r * G[s(r), :]
 *              (same section, Algorithm 1 backward half), over the distinct rows
 *              u touched in the step, then a sparse row update.
 *
 * Floating point: inputs are widened exactly (fp32 / bf16 -> fp64), every sum is
 * accumulated in fp64, and each stored result is rounded once to its storage type
 * (fp32 round-to-nearest-even by the C conversion; bf16 by rint() on an 8-bit
 * significand).  Alongside each sum it returns sum |term|, the scale of the error
 * bound a reordered fp32 sum must meet.
 *
 * Build: gcc -O2 -ffp-contract=off -shared -fPIC oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { O_HASH = 0, O_IDENTITY = 1, O_BUCKET = 2, O_KEYED = 3 };
enum { O_SUM = 0, O_MEAN = 1 };
enum { O_F32 = 0, O_BF16 = 1 };
enum { O_EMIT = 0, O_SGD = 1, O_ADAGRAD = 2 };

#define ROW_DROPPED (-1)
#define ROW_DEFAULT (-2)

typedef struct {
    int32_t kind, pool, dtype, dim;
    int64_t rows, id_lo, id_hi;
    const float *boundaries;
    int64_t n_boundaries;
    void *weights;  /* [rows, dim], fp32 or bf16 (raw uint16 bits) */
    float *state;   /* Adagrad accumulator [rows, dim] fp32, or NULL */
    int32_t seq_max;        /* SeqTrunc: keep at most this many positions per bag (0 = all) */
    int32_t seq_keep_last;  /* ... the last seq_max (1) or the first seq_max (0) */
    int64_t default_row;    /* row that fills a bag with no valid position, or -1 (zero vector) */
} oracle_col;

/* ---------------------------------------------------------------- hashing */

/* SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): the output function applied to
 * x + golden gamma, i.e. the first output of a SplitMix64 generator seeded with x. */
uint64_t oracle_splitmix64(uint64_t x)
{
    uint64_t z = x + 0x9E3779B97F4A7C15ULL;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

void oracle_splitmix64_array(const uint64_t *in, uint64_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; i++) out[i] = oracle_splitmix64(in[i]);
}

/* unsigned 64-bit remainder of the hash; C's % on uint64_t is exactly that */
int64_t oracle_hash_mod(uint64_t id_bits, int64_t rows)
{
    return (int64_t)(oracle_splitmix64(id_bits) % (uint64_t)rows);
}

/* ------------------------------------------------------------- bucketize */

/* number of boundaries b_j with b_j <= x, by a linear scan; -1 for NaN */
int64_t oracle_bucketize(const float *b, int64_t nb, float x)
{
    if (isnan(x)) return ROW_DROPPED;
    int64_t k = 0;
    for (int64_t j = 0; j < nb; j++)
        if (b[j] <= x) k++;
    return k;
}

/* -------------------------------------------------------------- storage */

static double bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* round a double once to bfloat16 (8 significant bits, fp32 exponent range),
 * ties to even */
uint16_t oracle_double_to_bf16(double v)
{
    float f;
    uint32_t u;
    if (isnan(v)) return 0x7FC0;
    if (v == 0.0) {
        f = (float)v;
        memcpy(&u, &f, 4);
        return (uint16_t)(u >> 16);
    }
    double a = fabs(v), r;
    if (a < ldexp(1.0, -126)) {
        r = rint(a * ldexp(1.0, 133)) * ldexp(1.0, -133);       /* subnormal quantum */
    } else {
        int e;
        double m = frexp(a, &e);                                /* a = m 2^e, m in [0.5,1) */
        r = ldexp(rint(ldexp(m, 8)), e - 8);                    /* 8 significant bits */
    }
    if (r > 3.3895313892515355e38) r = INFINITY;                /* above max bf16 */
    f = (float)(v < 0 ? -r : r);                                /* exact */
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static double weight_at(const oracle_col *col, int64_t row, int32_t d)
{
    int64_t i = row * col->dim + d;
    if (col->dtype == O_BF16) return bf16_to_double(((const uint16_t *)col->weights)[i]);
    return (double)((const float *)col->weights)[i];
}

static void weight_store(const oracle_col *col, int64_t row, int32_t d, double v)
{
    int64_t i = row * col->dim + d;
    if (col->dtype == O_BF16)
        ((uint16_t *)col->weights)[i] = oracle_double_to_bf16(v);
    else
        ((float *)col->weights)[i] = (float)v;
}

/* ------------------------------------------------------------- transform */

/* row of one position of column `col`: >= 0, ROW_DROPPED or ROW_DEFAULT */
int64_t oracle_row(const oracle_col *col, int64_t id, float x, int32_t keyed_row)
{
    switch (col->kind) {
    case O_HASH:
        if (id < col->id_lo || id >= col->id_hi) return ROW_DROPPED;
        return oracle_hash_mod((uint64_t)id, col->rows);
    case O_IDENTITY:
        if (id < 0 || id >= col->rows) return ROW_DROPPED;
        return id;
    case O_BUCKET:
        return oracle_bucketize(col->boundaries, col->n_boundaries, x);
    case O_KEYED:
        if (keyed_row == ROW_DEFAULT) return ROW_DEFAULT;
        if (keyed_row < 0 || keyed_row >= col->rows) return ROW_DROPPED;
        return keyed_row;
    }
    return ROW_DROPPED;
}

static int64_t position_row(const oracle_col *col, int64_t p, const int64_t *ids,
                            const float *fvals, const int32_t *keyed_rows)
{
    return oracle_row(col, ids ? ids[p] : 0, fvals ? fvals[p] : 0.0f,
                      keyed_rows ? keyed_rows[p] : ROW_DROPPED);
}

/* Sequence truncation and masking (RecIS Sec. 3.1 and Figure 2, where SeqTrunc and
 * masking are two of the per-field transformations, SeqTrunc ordered before Hash).
 * Both act on the raw positions before the transform: position p of the bag
 * [start, end) survives iff its
 * mask byte is nonzero (no mask: all survive) and, when the column truncates,
 * its index in the bag is among the first seq_max (or the last seq_max).  A
 * position that does not survive is dropped: no row, not counted in a mean. */
static int position_kept(const oracle_col *col, int64_t p, int64_t start, int64_t end,
                         const uint8_t *mask)
{
    if (mask && mask[p] == 0) return 0;
    if (col->seq_max > 0) {
        int64_t i = p - start, len = end - start;
        if (col->seq_keep_last) return i >= len - col->seq_max;
        return i < col->seq_max;
    }
    return 1;
}

/* ---------------------------------------------------------------- forward */

/*
 * Y      [B, sumD] fp32   pooled output, columns concatenated in order
 * pweights [N] fp32       per-position weights v_r, or NULL (all 1)
 * Ybound [B, sumD] fp64   sum |w_r E[i_r, d]| (may be NULL)
 * bag_n  [C*B]            valid positions per bag (may be NULL)
 * rows   [N]              transformed row per position (may be NULL)
 * Returns N (= offsets[C*B]).
 */
int64_t oracle_forward(const oracle_col *cols, int32_t C, int32_t B, const int32_t *offsets,
                       const int64_t *ids, const float *fvals, const int32_t *keyed_rows,
                       const uint8_t *mask, const float *pweights, float *Y, double *Ybound,
                       int32_t *bag_n, int32_t *rows)
{
    int64_t sumD = 0;
    for (int32_t c = 0; c < C; c++) sumD += cols[c].dim;
    int64_t off_c = 0;
    for (int32_t c = 0; c < C; c++) {
        const oracle_col *col = &cols[c];
        int32_t D = col->dim;
        double *acc = (double *)calloc((size_t)D, sizeof(double));
        double *mag = (double *)calloc((size_t)D, sizeof(double));
        for (int32_t s = 0; s < B; s++) {
            int64_t b = (int64_t)c * B + s;
            int64_t n = 0;
            memset(acc, 0, sizeof(double) * D);
            memset(mag, 0, sizeof(double) * D);
            for (int64_t p = offsets[b]; p < offsets[b + 1]; p++) {
                int64_t r = position_kept(col, p, offsets[b], offsets[b + 1], mask)
                                ? position_row(col, p, ids, fvals, keyed_rows) : ROW_DROPPED;
                if (rows) rows[p] = (int32_t)r;
                if (r == ROW_DROPPED) continue;
                n++;
                if (r == ROW_DEFAULT) continue;      /* the zero row: counted, adds nothing */
                double v = pweights ? (double)pweights[p] : 1.0;
                for (int32_t d = 0; d < D; d++) {
                    double e = v * weight_at(col, r, d);   /* exact: 24 x 24 bits */
                    acc[d] += e;
                    mag[d] += fabs(e);
                }
            }
            if (bag_n) bag_n[b] = (int32_t)n;
            for (int32_t d = 0; d < D; d++) {
                double y = 0.0, m = 0.0;
                if (n > 0) {
                    y = (col->pool == O_MEAN) ? acc[d] / (double)n : acc[d];
                    m = (col->pool == O_MEAN) ? mag[d] / (double)n : mag[d];
                } else if (col->default_row >= 0) {
                    y = weight_at(col, col->default_row, d);
                    m = fabs(y);
                }
                Y[s * sumD + off_c + d] = (float)y;
                if (Ybound) Ybound[s * sumD + off_c + d] = m;
            }
        }
        free(acc);
        free(mag);
        off_c += D;
    }
    return offsets[(int64_t)C * B];
}

/* --------------------------------------------------------------- backward */

typedef struct {
    int64_t row, pos;
} rowpos;

static int cmp_rowpos(const void *a, const void *b)
{
    const rowpos *x = (const rowpos *)a, *y = (const rowpos *)b;
    if (x->row != y->row) return x->row < y->row ? -1 : 1;
    if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;
    return 0;
}

/* Adagrad on one element, element-wise accumulator starting at zero:
 * A' = A + g^2 ; E' = E - lr g / (sqrt(A') + eps).  Returns E', writes A'. */
double oracle_adagrad_elem(double e, double a, double g, double lr, double eps, double *a_out)
{
    double a2 = a + g * g;
    *a_out = a2;
    return e - lr * g / (sqrt(a2) + eps);
}

/*
 * Gradient of the pooled output G [B, sumD] fp32 with respect to every table row
 * touched by the batch, then the row update `opt` (EMIT leaves tables alone).
 *
 * uniq_col/uniq_row [max_uniq]              distinct (column, row), ascending
 * uniq_grad/uniq_bound [max_uniq * maxD]    fp64 sum and sum |term|, row-padded to maxD
 * Returns U, or -1 if U would exceed max_uniq.
 */
int64_t oracle_backward(const oracle_col *cols, int32_t C, int32_t B, const int32_t *offsets,
                        const int64_t *ids, const float *fvals, const int32_t *keyed_rows,
                        const uint8_t *mask, const float *pweights, const float *G, int32_t opt,
                        double lr, double eps,
                        int32_t *uniq_col, int64_t *uniq_row, double *uniq_grad,
                        double *uniq_bound, int64_t max_uniq)
{
    int64_t sumD = 0, maxD = 0;
    for (int32_t c = 0; c < C; c++) {
        sumD += cols[c].dim;
        if (cols[c].dim > maxD) maxD = cols[c].dim;
    }
    int64_t U = 0, off_c = 0;
    for (int32_t c = 0; c < C; c++) {
        const oracle_col *col = &cols[c];
        int32_t D = col->dim;
        int64_t a = offsets[(int64_t)c * B], e = offsets[(int64_t)(c + 1) * B];
        /* pass 1: valid count per bag (the mean's denominator) */
        int32_t *n_of_bag = (int32_t *)calloc((size_t)B, sizeof(int32_t));
        int32_t *bag_of_pos = (int32_t *)malloc(sizeof(int32_t) * (size_t)(e - a + 1));
        /* contributors: the valid non-DEFAULT positions, then one pseudo position
         * e + s per empty bag s when the column has a default row */
        rowpos *list = (rowpos *)malloc(sizeof(rowpos) * (size_t)(e - a + B + 1));
        int64_t L = 0;
        for (int32_t s = 0; s < B; s++) {
            int64_t b = (int64_t)c * B + s;
            for (int64_t p = offsets[b]; p < offsets[b + 1]; p++) {
                int64_t r = position_kept(col, p, offsets[b], offsets[b + 1], mask)
                                ? position_row(col, p, ids, fvals, keyed_rows) : ROW_DROPPED;
                bag_of_pos[p - a] = s;
                if (r == ROW_DROPPED) continue;
                n_of_bag[s]++;
                if (r == ROW_DEFAULT) continue;     /* the default row takes no gradient */
                list[L].row = r;
                list[L].pos = p;
                L++;
            }
        }
        if (col->default_row >= 0) {
            for (int32_t s = 0; s < B; s++) {
                if (n_of_bag[s] > 0) continue;
                list[L].row = col->default_row;
                list[L].pos = e + s;
                L++;
            }
        }
        /* pass 2: sort contributors by (row, position) and sum each run */
        qsort(list, (size_t)L, sizeof(rowpos), cmp_rowpos);
        double *g = (double *)malloc(sizeof(double) * (size_t)D);
        double *m = (double *)malloc(sizeof(double) * (size_t)D);
        for (int64_t i = 0; i < L;) {
            int64_t j = i;
            memset(g, 0, sizeof(double) * D);
            memset(m, 0, sizeof(double) * D);
            for (; j < L && list[j].row == list[i].row; j++) {
                int32_t s;
                double w;
                if (list[j].pos >= e) {          /* an empty bag's default row: weight 1 */
                    s = (int32_t)(list[j].pos - e);
                    w = 1.0;
                } else {
                    s = bag_of_pos[list[j].pos - a];
                    w = (col->pool == O_MEAN) ? 1.0 / (double)n_of_bag[s] : 1.0;
                    if (pweights) w *= (double)pweights[list[j].pos];
                }
                for (int32_t d = 0; d < D; d++) {
                    double t = w * (double)G[s * sumD + off_c + d];
                    g[d] += t;
                    m[d] += fabs(t);
                }
            }
            if (U >= max_uniq) {
                free(g); free(m); free(list); free(bag_of_pos); free(n_of_bag);
                return -1;
            }
            int64_t r = list[i].row;
            if (uniq_col) uniq_col[U] = c;
            if (uniq_row) uniq_row[U] = r;
            for (int32_t d = 0; d < D; d++) {
                if (uniq_grad) uniq_grad[U * maxD + d] = g[d];
                if (uniq_bound) uniq_bound[U * maxD + d] = m[d];
            }
            /* the row update */
            for (int32_t d = 0; d < D; d++) {
                double w0 = weight_at(col, r, d);
                if (opt == O_SGD) {
                    weight_store(col, r, d, w0 - lr * g[d]);
                } else if (opt == O_ADAGRAD) {
                    double a2;
                    double a0 = (double)col->state[r * D + d];
                    double w1 = oracle_adagrad_elem(w0, a0, g[d], lr, eps, &a2);
                    col->state[r * D + d] = (float)a2;
                    weight_store(col, r, d, w1);
                }
            }
            U++;
            i = j;
        }
        free(g);
        free(m);
        free(list);
        free(bag_of_pos);
        free(n_of_bag);
        off_c += D;
    }
    return U;
}

/* ------------------------------------------------------- keyed-table rows */

/* Initial value of a newly admitted keyed row (the pages leave it open; a
 * deterministic, key-seeded uniform draw with standard deviation `std`):
 *   u = (splitmix64(splitmix64(key) + d) >> 40) * 2^-24,   e = fp32(std*sqrt(3)) * (2u - 1)
 * computed exactly in fp64 (24-bit x 24-bit product) and rounded once to fp32. */
void oracle_init_row(int64_t key, int32_t dim, double std, float *out)
{
    float a = (float)(std * sqrt(3.0));
    uint64_t h = oracle_splitmix64((uint64_t)key);
    for (int32_t d = 0; d < dim; d++) {
        uint64_t z = oracle_splitmix64(h + (uint64_t)d);
        double u = ldexp((double)(z >> 40), -24);
        out[d] = (float)((double)a * (2.0 * u - 1.0));
    }
}

/* ------------------------------------------------------- array helpers */

/* oracle_adagrad_elem over arrays (used to bound a reordered-sum result) */
void oracle_adagrad_array(const double *e, const double *a, const double *g, int64_t n, double lr,
                          double eps, double *e_out, double *a_out)
{
    for (int64_t i = 0; i < n; i++) e_out[i] = oracle_adagrad_elem(e[i], a[i], g[i], lr, eps, &a_out[i]);
}

void oracle_to_bf16_array(const double *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++) out[i] = oracle_double_to_bf16(v[i]);
}
