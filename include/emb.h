/*
 * emb.h -- C ABI of the fused multi-column embedding stage for AMD MI355X (gfx950).
 *
 * The stage turns many embedding columns into one pass over a jagged batch:
 * raw ID or float transform (hash, bucketize), safety filtering (out-of-range IDs
 * dropped, empty bags given the zero default), row lookup (hash-mod, identity, or
 * a collisionless keyed table), gather with sum/mean pooling into one
 * concatenated [B, sum(dim)] output, and the backward that deduplicates the
 * touched rows, segment-reduces their gradients and applies a sparse row update.
 *
 * Sources of the definitions (the web pages this library implements):
 *  - RECom explainer, "Why this problem is worth solving": an embedding column
 *    turns a raw feature into an index with a hash or a bucket, discards indices
 *    outside its table, substitutes a default for a missing feature, gathers the
 *    table rows and reduces them to one vector; each column has its own table.
 *  - RecIS, Sec. 3.2 "Index-aware segment reduction" and Algorithm 1: CSR
 *    offsets define segments; forward Y[s,:] = sum_r w_r E[i_r,:] over segment s,
 *    empty segments produce zero; backward dE[u] = sum over contributors r with
 *    i_r = u of w_r G[s(r),:].
 *  - RecIS, Sec. 3.1 "Fused and Vectorized Feature Processing": all fields'
 *    elements are flattened into one index space cut into equal tiles, so work
 *    follows element count rather than field count.
 *  - Monolith, Sec. 2.1 "Hash Table": a collisionless key-value table (distinct
 *    IDs never share an embedding) that admits an ID only after its occurrence
 *    count reaches a tunable threshold; lookup and update are native ops.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE memory owned by the caller unless marked (host).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls only enqueue work on it; none synchronizes the host and none
 *    allocates device memory.  The caller keeps every buffer alive until the
 *    stream work that uses it has completed.
 *  - Host-detectable argument problems return a status before anything is
 *    enqueued; emb_last_error() then holds a message.  A failed kernel launch
 *    returns EMB_ERR_HIP.
 *  - Data conditions are not errors: out-of-range IDs and NaN values are
 *    dropped, empty bags give zero, keys not (yet) admitted read the DEFAULT
 *    (zero) row; all are counted in the optional stats array.
 */
#ifndef EMB_H
#define EMB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EMB_OK = 0,
    EMB_ERR_INVALID_ARG = 1,   /* bad descriptor, pointer, size or alignment */
    EMB_ERR_UNSUPPORTED = 2,   /* a valid request the library does not handle (e.g. dim) */
    EMB_ERR_WORKSPACE = 3,     /* a caller buffer is smaller than the query returned */
    EMB_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed */
} emb_status;

/* column kinds: how a raw input becomes a row index (RECom explainer: a hash or a bucket) */
#define EMB_COL_HASH     0  /* ids int64; valid iff id_lo <= id < id_hi; row = splitmix64(id) mod rows */
#define EMB_COL_IDENTITY 1  /* ids int64; valid iff 0 <= id < rows;      row = id                    */
#define EMB_COL_BUCKET   2  /* fvals fp32; valid iff not NaN;            row = #{j : boundaries[j] <= x} */
#define EMB_COL_KEYED    3  /* keyed_rows int32 from emb_table_lookup_or_insert                      */

#define EMB_POOL_SUM  0     /* w_r = 1                                                  */
#define EMB_POOL_MEAN 1     /* w_r = 1/n, n = valid positions of the bag, DEFAULT included */

#define EMB_F32  0
#define EMB_BF16 1          /* weights bf16, accumulation fp32, updated weights rounded to nearest even */

#define EMB_OPT_EMIT    0   /* backward writes (unique key, gradient) and leaves tables alone */
#define EMB_OPT_SGD     1   /* E <- E - lr g                                                  */
#define EMB_OPT_ADAGRAD 2   /* A <- A + g^2 ; E <- E - lr g / (sqrt(A) + eps), element-wise   */

#define EMB_ROW_DROPPED (-1) /* keyed row code: the position is dropped                       */
#define EMB_ROW_DEFAULT (-2) /* keyed row code: the zero DEFAULT row (counted in a mean)        */

/* stats[] indices: int64 device counters, accumulated (the caller zeroes them) */
#define EMB_STAT_IDS            0  /* positions transformed by emb_forward           */
#define EMB_STAT_VALID          1  /* positions with a table row                     */
#define EMB_STAT_DROPPED        2  /* positions dropped (out of range, NaN, key < 1) */
#define EMB_STAT_DEFAULT        3  /* positions reading the DEFAULT row              */
#define EMB_STAT_ZERO_BAGS      4  /* bags with no valid position (zero or default row) */
#define EMB_STAT_UNIQUE         5  /* distinct (column, row) pairs in emb_backward   */
#define EMB_STAT_TABLE_INSERTED 6  /* keys newly placed in a keyed table             */
#define EMB_STAT_TABLE_ADMITTED 7  /* keys that received a row (admission)           */
#define EMB_STAT_TABLE_FULL     8  /* key occurrences refused: no free slot or row   */
#define EMB_STAT_MAX_PROBE      9  /* longest probe sequence seen (max, not sum)     */
#define EMB_STAT_FILTERED      10  /* positions removed by sequence truncation or the mask */
#define EMB_STAT_TABLE_EVICTED 11  /* keys removed by emb_table_evict                  */
#define EMB_STAT_COUNT         16

/* One embedding column (host struct), in output order.  Row-major tables. */
typedef struct emb_column_desc {
    int32_t kind;              /* EMB_COL_*                                             */
    int32_t pool;              /* EMB_POOL_*                                            */
    int32_t dtype;             /* EMB_F32 | EMB_BF16 (KEYED: EMB_F32)                    */
    int32_t dim;               /* D: a multiple of 4, <= 256                              */
    int64_t rows;              /* table rows, 1 .. 2^31-1                               */
    int64_t id_lo, id_hi;      /* HASH: valid raw IDs are [id_lo, id_hi)                  */
    const float *boundaries;   /* BUCKET: device, sorted ascending fp32                 */
    int64_t n_boundaries;      /* BUCKET: rows >= n_boundaries + 1                      */
    void *weights;             /* device [rows, dim] in dtype; updated in place by emb_backward */
    float *opt_state;          /* ADAGRAD: device fp32 [rows, dim], zero before the first step  */
    int32_t seq_max;           /* sequence truncation: keep at most seq_max positions of  */
                               /* each bag (0 = keep all), counted on the raw positions   */
                               /* before the transform (RecIS Sec. 3.1 and Figure 2:      */
                               /* SeqTrunc is a per-field step ordered before Hash)      */
    int32_t seq_keep_last;     /* 1: keep a bag's last seq_max positions, 0: its first. */
                               /* KEYED: the table lookup before the forward still sees */
                               /* (and counts) every key; truncation acts on pooling.   */
    int64_t default_row;       /* -1: a bag with no valid position pools to the zero     */
                               /* vector.  0 .. rows-1: it reads this row instead, as one */
                               /* position of weight 1, and the row gets that bag's      */
                               /* gradient (RECom explainer: a default fills in a missing */
                               /* feature; RECom merges that empty-row filling into the  */
                               /* lookup).  Plans with a default row use the global     */
                               /* radix sort in emb_backward and have no atomic backward. */
} emb_column_desc;

typedef struct emb_plan_opts {
    int32_t opt;               /* EMB_OPT_*                                            */
    float lr;                  /* learning rate (SGD, ADAGRAD)                          */
    float eps;                 /* ADAGRAD epsilon, outside the square root              */
    int32_t tile;              /* positions per wavefront tile: 0 = default (256), else a multiple of 64 <= 256 */
    int32_t fwd_tile;          /* positions per forward tile: 0 = `tile` when that is set, else chosen */
                               /* per call: 512 when the batch has at least 64 positions per bag on   */
                               /* average (long sequences: a longer tile cuts fewer bags into pieces) */
                               /* and at least 512 x 6144 positions (tiles enough to fill the chip    */
                               /* twice), 256 otherwise.  Else a multiple of 64 <= 512.               */
} emb_plan_opts;

typedef struct emb_plan emb_plan;    /* host object owned by the library */
typedef struct emb_table emb_table;  /* host object owned by the library */

/* Sizes of the device buffers a plan needs: `plan_bytes` of column metadata and
 * `workspace_bytes` of per-step workspace for batches of `batch` samples with at
 * most `max_ids` positions.  Host only; validates the descriptors. */
emb_status emb_plan_query(const emb_column_desc *cols /* host [n_cols] */, int32_t n_cols,
                          int32_t batch, int64_t max_ids, const emb_plan_opts *opts /* host */,
                          size_t *plan_bytes /* host */, size_t *workspace_bytes /* host */);

/* Creates a plan.  Copies the column metadata into `plan_mem` (>= plan_bytes,
 * 256-byte aligned) on `stream`.  The plan keeps pointers to the caller's tables. */
emb_status emb_plan_create(const emb_column_desc *cols, int32_t n_cols, int32_t batch,
                           int64_t max_ids, const emb_plan_opts *opts, void *plan_mem,
                           void *stream, emb_plan **out /* host */);

emb_status emb_plan_destroy(emb_plan *plan);

/* Positions per tile of the forward kernels for a batch of `n_ids` positions: the
 * plan's fixed size, or the one it chooses for that batch (emb_plan_opts.fwd_tile).
 * Host only.  The allocation-free forward's scratch grows with ceil(n_ids / tile).
 * n_ids outside [0, max_ids]: EMB_ERR_WORKSPACE. */
emb_status emb_plan_forward_tile(const emb_plan *plan, int64_t n_ids, int32_t *tile /* host */);

/*
 * Forward of all columns in ONE kernel launch.
 *   offsets  int32 [n_cols*batch + 1]: bag (c, s) is positions [offsets[c*B+s], offsets[c*B+s+1]),
 *            column-major (all bags of column 0, then column 1, ...); offsets[0] = 0,
 *            non-decreasing, offsets[n_cols*batch] = n_ids.
 *   ids      int64 [n_ids] raw IDs (HASH, IDENTITY positions), or NULL if no such column.
 *   fvals    fp32  [n_ids] raw values (BUCKET positions), or NULL if no such column.
 *   keyed_rows int32 [n_ids] rows from emb_table_lookup_or_insert (KEYED positions), or NULL.
 *   out      fp32 [batch, sum(dim)]: every element is written (zero for empty bags).
 *   workspace >= workspace_bytes, 256-byte aligned, ZERO-FILLED once before the
 *            plan's first call; it holds per-step state that the library
 *            restores before each call returns.  With training != 0 the forward
 *            records what the matching emb_backward needs in it, so the same
 *            workspace must reach that backward unmodified.  A workspace serves
 *            one call at a time.
 *   stats    int64 [EMB_STAT_COUNT] or NULL.
 */
emb_status emb_forward(emb_plan *plan, const int32_t *offsets, const int64_t *ids,
                       const float *fvals, const int32_t *keyed_rows, int64_t n_ids, float *out,
                       void *workspace, int32_t training, int64_t *stats, void *stream);

/*
 * emb_forward with optional per-position inputs (all device memory, caller-owned):
 *   pweights fp32 [n_ids] or NULL: the weight w_r of each contributor in
 *            RecIS Sec. 3.2 ("Index-aware segment reduction": Y_s is the sum of
 *            w_r E[i_r] over the bag, and each contributor sends w_r G[s(r)]
 *            back).  A sum bag pools sum v_r E[i_r]; a mean bag divides that sum
 *            by its count of valid positions (DEFAULT ones included, as without
 *            weights).  NULL: all weights 1.
 *   mask     uint8 [n_ids] or NULL: masking, one of the per-field
 *            transformations of RecIS Sec. 3.1 / Figure 2 (the pages give no
 *            detail, so a mask here is one byte per position).  A position whose
 *            byte is 0 is removed before the transform, like a truncated one: it
 *            reads no row, does not count in a mean and gets no gradient.
 * A position survives iff the mask keeps it AND its column's truncation keeps it
 * (both look at raw positions, so their order does not matter).  The matching
 * emb_backward needs neither input again: a training call records the removed
 * positions and copies the weights into the workspace.  With both NULL and no
 * truncating column this is emb_forward.  Arguments, layout, ownership and errors
 * otherwise as emb_forward.
 */
emb_status emb_forward_ex(emb_plan *plan, const int32_t *offsets, const int64_t *ids,
                          const float *fvals, const int32_t *keyed_rows, const float *pweights,
                          const uint8_t *mask, int64_t n_ids, float *out, void *workspace,
                          int32_t training, int64_t *stats, void *stream);

/*
 * The forward in two launches, so that the transform of the next batch can run
 * on another stream while this step's backward still uses the workspace (the
 * pipelined preparation of RecIS Sec. 3.3: feature transformation for iteration
 * t + 1 overlaps the training work of iteration t, since it neither reads nor
 * updates parameters).
 *
 * emb_transform: the transform and filter of every position (hash + mod, identity,
 * bucketize, keyed rows; truncation and the mask) and nothing else.
 *   rows_out  int32 [n_ids], caller-owned device memory: the row of each position,
 *             EMB_ROW_DROPPED (-1) for a dropped or removed one, EMB_ROW_DEFAULT (-2)
 *             for a keyed DEFAULT one.
 *   Touches no workspace; stats (or NULL) gets the per-position counters.  Other
 *   arguments as emb_forward_ex.
 * emb_forward_rows: emb_forward_ex from row codes made by emb_transform for the
 *   same plan and batch (offsets, n_ids): gather, pool, and with training != 0
 *   the record the backward needs.  Row codes outside [0, rows) other than -2 are
 *   dropped.  stats gets the bag counter only (the transform counted the rest).
 */
emb_status emb_transform(emb_plan *plan, const int32_t *offsets, const int64_t *ids,
                         const float *fvals, const int32_t *keyed_rows, const uint8_t *mask,
                         int64_t n_ids, int32_t *rows_out, int64_t *stats, void *stream);
emb_status emb_forward_rows(emb_plan *plan, const int32_t *offsets, const int32_t *rows,
                            const float *pweights, int64_t n_ids, float *out, void *workspace,
                            int32_t training, int64_t *stats, void *stream);

/*
 * emb_forward (inference, training = 0) for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It takes no workspace: the split-bag partials and tickets
 * live in a fixed 32 MiB array inside the library, one per GPU, held until the
 * process exits; the call allocates nothing.  A batch whose scratch would exceed
 * the array (1 KB plus about (8 max(dim) + 44) bytes per tile, tiles =
 * ceil(n_ids / forward tile)) returns EMB_ERR_WORKSPACE before anything is enqueued.  Each
 * call first clears the tickets it uses and a 1 KB zero row with a fill kernel on
 * `stream`.  All calls on one GPU share
 * its array: calls that overlap on one GPU (unordered streams) race; order them.
 * Other arguments, layout and errors as emb_forward.
 */
emb_status emb_forward_noalloc(emb_plan *plan, const int32_t *offsets, const int64_t *ids,
                               const float *fvals, const int32_t *keyed_rows, int64_t n_ids,
                               float *out, int64_t *stats, void *stream);

/*
 * Backward of the last training forward on this workspace: deduplicates the
 * touched (column, row) pairs by a radix sort of their keys, sums each pair's
 * contributions w_r * grad_out[s(r), off_c:off_c+dim] and applies opts->opt.
 *   grad_out   fp32 [batch, sum(dim)].
 *   uniq_keys  uint32 [n_ids + n_def] or NULL: the distinct keys, ascending, key =
 *              row_base_c + row with row_base_c = sum of rows of the columns before c;
 *              n_def = the number of columns with a default row (0 without).
 *   uniq_grads fp32 [n_ids + n_def, max(dim)] or NULL (EMIT only): gradient of
 *              uniq_keys[u] in row u.
 *   n_uniq     int64 device scalar or NULL: number of distinct keys.
 * SGD / ADAGRAD update the columns' weights (and opt_state) in place; rows that
 * no position touched are left bit-identical.
 */
emb_status emb_backward(emb_plan *plan, const float *grad_out, void *workspace,
                        uint32_t *uniq_keys, float *uniq_grads, int64_t *n_uniq, int64_t *stats,
                        void *stream);

/* emb_backward in two parts, for callers that schedule them apart (the
 * deduplication does not read grad_out, so it can run while the upstream
 * gradient is still being computed):
 *   emb_backward_dedup  radix sort of the touched row keys and the distinct
 *                       keys (RecIS Fig. 3 "Reduce-ID": each row once, with the
 *                       map back to its contributors); uniq_keys / n_uniq as above;
 *   emb_backward_apply  segment-sum of grad_out per distinct row and the row
 *                       update (or uniq_grads for EMIT).
 * apply must follow dedup on the same workspace. */
emb_status emb_backward_dedup(emb_plan *plan, void *workspace, uint32_t *uniq_keys,
                              int64_t *n_uniq, int64_t *stats, void *stream);
emb_status emb_backward_apply(emb_plan *plan, const float *grad_out, void *workspace,
                              float *uniq_grads, void *stream);

/* SGD backward by atomic scatter, the pages' own design (RecIS Sec. 3.2,
 * Algorithm 1): every contribution -lr w_r grad_out[s(r), off_c:off_c+dim] is
 * added to its row with fp32 atomic adds, with no sort and no unique-row list
 * (repeats of a row inside a small batch are merged first).  Needs the SGD
 * optimizer and fp32 tables (EMB_ERR_UNSUPPORTED otherwise).  The order of the
 * adds is not fixed, so the updated rows are not bit-reproducible; they agree
 * with emb_backward within the rounding of the sums.  Kept for comparison with
 * the sorted path. */
emb_status emb_backward_atomic(emb_plan *plan, const float *grad_out, void *workspace, void *stream);

/* A plain streaming copy of `bytes` (a multiple of 16, both buffers 16-byte
 * aligned device memory): dst[i] = src[i].  Not part of the stage; it measures
 * the bandwidth a purely contiguous read + write kernel reaches on this GPU, the
 * practical ceiling next to the specified peak that the stage's kernels are
 * reported against.  EMB_ERR_INVALID_ARG for bad sizes or alignment. */
emb_status emb_stream_copy(void *dst, const void *src, int64_t bytes, void *stream);

/* Device views into a workspace after a training forward (parity checks):
 * keys uint32 [n_ids] (row_base_c + row; sum(rows) for a dropped position,
 * sum(rows)+1 for a DEFAULT one), bags int32 [n_ids] (bag index c*B+s),
 * bag_n int32 [n_cols*batch] (valid positions per bag). */
typedef struct emb_workspace_view {
    uint32_t *keys;
    int32_t *bags;
    int32_t *bag_n;
} emb_workspace_view;
emb_status emb_plan_workspace_view(emb_plan *plan, void *workspace, emb_workspace_view *out /* host */);

/* ------------------------------------------------------------------------
 * Collisionless keyed table (Monolith, Sec. 2.1): open addressing over a
 * power-of-two slot array (buckets of 16 slots from splitmix64(key), then a
 * per-key odd stride over the buckets; tables under 16 slots probe slot by slot),
 * insertion by atomic compare-and-swap on the slot key, an occurrence count per
 * slot and a frequency filter: a key gets a row from the row pool once its count
 * reaches `threshold`.  Distinct keys never share a row.  Valid keys are >= 1.
 * Rows are fp32 [row_capacity, dim]; emb_table_rows() gives the pool, which a
 * KEYED column uses as its weights (rows = row_capacity).
 * ------------------------------------------------------------------------ */

/* Bytes of device memory for a table. */
emb_status emb_table_query(int64_t capacity /* power of two, <= 2^30 */, int64_t row_capacity,
                           int32_t dim, size_t *table_bytes /* host */);

/* Creates an empty table in `table_mem` (>= table_bytes, 256-byte aligned; cleared
 * on `stream`).  New rows start as fp32(init_std*sqrt(3)) * (2u - 1) with
 * u = (splitmix64(splitmix64(key) + d) >> 40) * 2^-24 (uniform, std init_std),
 * or zero if init_std == 0. */
emb_status emb_table_create(int64_t capacity, int64_t row_capacity, int32_t dim,
                            int32_t threshold, float init_std, void *table_mem, void *stream,
                            emb_table **out /* host */);

emb_status emb_table_destroy(emb_table *table);

/* Device pointer to the row pool, fp32 [row_capacity, dim]. */
float *emb_table_rows(emb_table *table);

/* Inserts distinct keys as already admitted (count 0) with row values `rows`
 * fp32 [n, dim] (or the initializer above if rows is NULL).  Keys already
 * present keep their row; keys < 1 are skipped. */
emb_status emb_table_bulk_insert(emb_table *table, const int64_t *keys, const float *rows,
                                 int64_t n, int64_t *stats, void *stream);

/*
 * One step's lookup-or-insert.  Every occurrence of a valid key adds one to its
 * count (absent keys are inserted first); afterwards a key without a row whose
 * count reached the threshold is admitted.  The rule is batch-level: all
 * occurrences in the step see the same outcome, whatever the thread order.
 *   rows_out int32 [n]: the key's row, EMB_ROW_DEFAULT (not admitted, or refused
 *            because the table or row pool is full) or EMB_ROW_DROPPED (key < 1).
 */
emb_status emb_table_lookup_or_insert(emb_table *table, const int64_t *keys, int64_t n,
                                      int32_t *rows_out, int64_t *stats, void *stream);

/* Read-only lookup: rows_out int32 [n] (row, EMB_ROW_DEFAULT if present but not
 * admitted, EMB_ROW_DROPPED if absent); counts_out int32 [n] or NULL. */
emb_status emb_table_find(emb_table *table, const int64_t *keys, int64_t n, int32_t *rows_out,
                          int32_t *counts_out, void *stream);

/* Writes every occupied slot (in unspecified order): keys int64, counts int32,
 * rows int32 (-1 if not admitted), each [capacity]; n_out int64 device scalar. */
emb_status emb_table_export(emb_table *table, int64_t *keys, int32_t *counts, int32_t *rows,
                            int64_t *n_out, void *stream);

/*
 * Table lifecycle (Monolith Sec. 2.1 expires IDs that stay inactive, so that the
 * table holds the live features only).  Every emb_table_lookup_or_insert is one
 * table step: step k (k = 0, 1, ...) records k as the last-seen step of each key
 * it finds or inserts, once tracking is on (emb_table_track_seen; off by
 * default: the record costs one scattered store per distinct key per 1024
 * occurrences, about 7 % of the keyed training step, and keys inserted while it
 * is off keep last-seen 0); emb_table_bulk_insert and emb_table_load always
 * record the current step.  Rows freed by eviction go to a free list that admission takes
 * from before the unused end of the pool.  None of these calls may overlap
 * another call on the same table.
 *
 * emb_table_step: the step the next lookup-or-insert will record (host value).
 * emb_table_set_step: sets it (restoring a checkpoint).
 *
 * emb_table_evict: removes every key whose last-seen step is < min_seen: its slot,
 *   count and admission are dropped and its row goes to the free list (a later
 *   occurrence starts the key anew).  The slot array is rebuilt from the live keys
 *   (compaction), so probe sequences stay short.  Row indices of live keys do not
 *   change.  opt_state: fp32 [row_capacity, dim] optimizer state of the column
 *   using the table, or NULL: the freed rows' state is zeroed.  n_live: int64
 *   device scalar or NULL (live keys after the call); stats gets
 *   EMB_STAT_TABLE_EVICTED.  Callers evict by age (min_seen = step - max_age)
 *   or when their count of keys reaches a load limit.
 *
 * emb_table_save: a checkpoint of every key, in unspecified order: keys int64,
 *   counts int32, last-seen steps int32, admitted uint8 (1 = has a row), values
 *   fp32 [capacity, dim] (the row, or zeros), each with room for `capacity`
 *   entries; n_out int64 device scalar.  Together with emb_table_step it is the
 *   table's whole state.
 * emb_table_load: inserts n checkpoint entries in that layout into a table:
 *   absent keys get their count and last-seen step, and admitted ones a row with
 *   the saved values (row pool full: not admitted, counted in
 *   EMB_STAT_TABLE_FULL); keys already present are left as they are.
 */
/*
 * Count-min admission (a probabilistic frequency filter; Monolith Sec. 2.1 admits
 * an ID once its frequency reaches a threshold): with a sketch set, a key that
 * is not in the table takes no slot; its occurrences add to `depth` counters,
 * counter j in row j at x_j mod width, where x_0, x_1, ... are the outputs of a
 * SplitMix64 generator seeded with the key.  After all occurrences of a step are
 * added, an absent key whose estimate (the least of its counters) reaches the
 * threshold enters the table with that count and gets a row; the others read
 * DEFAULT.  Keys in the table count exactly in their slots.
 *   sketch  int32 [depth, width] device memory, caller-owned, zero-filled before
 *           first use; NULL switches the filter off (exact counting in slots).
 *   depth in [1, 8]; width a power of two in [2, 2^30].
 * The sketch is not part of emb_table_save; its owner keeps it.
 */
emb_status emb_table_use_count_min(emb_table *table, int32_t depth, int64_t width, int32_t *sketch);

int64_t emb_table_step(const emb_table *table);
emb_status emb_table_track_seen(emb_table *table, int32_t on);
emb_status emb_table_set_step(emb_table *table, int64_t step);
emb_status emb_table_evict(emb_table *table, int64_t min_seen, float *opt_state, int64_t *n_live,
                           int64_t *stats, void *stream);
emb_status emb_table_save(emb_table *table, int64_t *keys, int32_t *counts, int32_t *seen,
                          uint8_t *admitted, float *values, int64_t *n_out, void *stream);
emb_status emb_table_load(emb_table *table, const int64_t *keys, const int32_t *counts,
                          const int32_t *seen, const uint8_t *admitted, const float *values,
                          int64_t n, int64_t *stats, void *stream);

/* Message for the last non-OK status on this host thread. */
const char *emb_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EMB_H */
