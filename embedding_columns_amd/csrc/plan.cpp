// plan.cpp -- host side of a plan: descriptor validation, metadata, workspace layout.
//
// Validation and layout are plain C++ (no HIP call), so emb_plan_query works on a
// machine without a GPU; emb_plan_create adds one asynchronous copy of the column
// metadata to the caller's device buffer.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <string>

#include "internal.h"

namespace emb {

static thread_local std::string g_last_error;

emb_status fail(emb_status s, const std::string &msg)
{
    g_last_error = msg;
    return s;
}

emb_status ok() { return EMB_OK; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static int pow2_ceil(int x)
{
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

emb_status plan_validate(const emb_column_desc *cols, int32_t n_cols, int32_t batch,
                         int64_t max_ids, const emb_plan_opts *opts)
{
    if (!cols || n_cols <= 0) return fail(EMB_ERR_INVALID_ARG, "n_cols must be >= 1 with a descriptor array");
    if (batch <= 0) return fail(EMB_ERR_INVALID_ARG, "batch must be >= 1");
    if ((int64_t)n_cols * batch >= (int64_t(1) << 31) - 1)
        return fail(EMB_ERR_UNSUPPORTED, "n_cols * batch must be < 2^31 - 1 (int32 bag index)");
    if (max_ids < 0 || max_ids >= (int64_t(1) << 31) - 1)
        return fail(EMB_ERR_UNSUPPORTED, "max_ids must be in [0, 2^31 - 1) (int32 offsets)");
    if (!opts) return fail(EMB_ERR_INVALID_ARG, "opts is NULL");
    if (opts->opt < EMB_OPT_EMIT || opts->opt > EMB_OPT_ADAGRAD)
        return fail(EMB_ERR_INVALID_ARG, "unknown optimizer");
    if (opts->tile != 0 && (opts->tile % kWave != 0 || opts->tile < kWave || opts->tile > kTileMax))
        return fail(EMB_ERR_INVALID_ARG, "tile must be 0 or a multiple of 64 in [64, 256]");
    if (opts->fwd_tile != 0 &&
        (opts->fwd_tile % kWave != 0 || opts->fwd_tile < kWave || opts->fwd_tile > kFwdTileMax))
        return fail(EMB_ERR_INVALID_ARG, "fwd_tile must be 0 or a multiple of 64 in [64, 512]");
    if (opts->opt != EMB_OPT_EMIT && !(opts->lr >= 0.f && std::isfinite(opts->lr)))
        return fail(EMB_ERR_INVALID_ARG, "lr must be finite and >= 0");
    if (opts->opt == EMB_OPT_ADAGRAD && !(opts->eps >= 0.f && std::isfinite(opts->eps)))
        return fail(EMB_ERR_INVALID_ARG, "eps must be finite and >= 0");
    uint64_t total_rows = 0;
    int64_t sum_dim = 0;
    for (int32_t c = 0; c < n_cols; c++) {
        const emb_column_desc &d = cols[c];
        std::string at = "column " + std::to_string(c) + ": ";
        if (d.kind < EMB_COL_HASH || d.kind > EMB_COL_KEYED) return fail(EMB_ERR_INVALID_ARG, at + "unknown kind");
        if (d.pool != EMB_POOL_SUM && d.pool != EMB_POOL_MEAN) return fail(EMB_ERR_INVALID_ARG, at + "unknown pooling");
        if (d.dtype != EMB_F32 && d.dtype != EMB_BF16) return fail(EMB_ERR_INVALID_ARG, at + "unknown dtype");
        if (d.kind == EMB_COL_KEYED && d.dtype != EMB_F32) return fail(EMB_ERR_UNSUPPORTED, at + "keyed rows are fp32");
        if (d.rows <= 0 || d.rows > (int64_t(1) << 31) - 1) return fail(EMB_ERR_INVALID_ARG, at + "rows must be in [1, 2^31-1]");
        if (d.dim <= 0) return fail(EMB_ERR_INVALID_ARG, at + "dim must be >= 1");
        if (d.dtype == EMB_F32 && (d.dim % 4 != 0 || d.dim > kMaxDimF32))
            return fail(EMB_ERR_UNSUPPORTED, at + "fp32 dim must be a multiple of 4 and <= 256");
        if (d.dtype == EMB_BF16 && (d.dim % 4 != 0 || d.dim > kMaxDimF32))
            return fail(EMB_ERR_UNSUPPORTED, at + "bf16 dim must be a multiple of 4 and <= 256");
        if (d.kind == EMB_COL_HASH && d.id_lo >= d.id_hi) return fail(EMB_ERR_INVALID_ARG, at + "id_lo must be < id_hi");
        if (d.kind == EMB_COL_BUCKET) {
            if (d.n_boundaries < 0 || (d.n_boundaries > 0 && !d.boundaries))
                return fail(EMB_ERR_INVALID_ARG, at + "bucket boundaries missing");
            if (d.rows < d.n_boundaries + 1) return fail(EMB_ERR_INVALID_ARG, at + "rows must be >= n_boundaries + 1");
            if (d.n_boundaries > (int64_t(1) << 30)) return fail(EMB_ERR_UNSUPPORTED, at + "too many boundaries");
        }
        if (d.seq_max < 0) return fail(EMB_ERR_INVALID_ARG, at + "seq_max must be >= 0");
        if (d.default_row < -1 || d.default_row >= d.rows)
            return fail(EMB_ERR_INVALID_ARG, at + "default_row must be -1 or in [0, rows)");
        if (d.seq_keep_last != 0 && d.seq_keep_last != 1)
            return fail(EMB_ERR_INVALID_ARG, at + "seq_keep_last must be 0 or 1");
        if (!d.weights) return fail(EMB_ERR_INVALID_ARG, at + "weights is NULL");
        if (!aligned(d.weights, 16)) return fail(EMB_ERR_INVALID_ARG, at + "weights must be 16-byte aligned");
        if (opts->opt == EMB_OPT_ADAGRAD && (!d.opt_state || !aligned(d.opt_state, 16)))
            return fail(EMB_ERR_INVALID_ARG, at + "Adagrad needs a 16-byte aligned opt_state");
        total_rows += (uint64_t)d.rows;
        sum_dim += d.dim;
    }
    if (total_rows + 2 > 0xFFFFFFFFull)
        return fail(EMB_ERR_UNSUPPORTED, "sum of rows over all columns must be < 2^32 - 2 (32-bit row keys)");
    if (sum_dim > (int64_t(1) << 30)) return fail(EMB_ERR_UNSUPPORTED, "sum of dims too large");
    return EMB_OK;
}

void plan_layout(emb_plan &P)
{
    const int64_t nb = (int64_t)P.n_cols * P.batch;
    // sort entries: the positions, plus one per bag when a column has a default row
    const int64_t N = std::max<int64_t>(P.max_ids, 1) + (P.has_default ? nb : 0);
    // the forward's tiles are never shorter than the backward's unless fixed so
    const int64_t tmin = P.fwd_tile ? std::min(P.tile, P.fwd_tile) : P.tile;
    P.max_tiles = std::max<int64_t>(1, (N + tmin - 1) / tmin);
    P.sort_blocks = std::max<int64_t>(1, (N + kSortTile - 1) / kSortTile);
    P.uq_blocks = std::max<int64_t>(1, (N + kUqTile - 1) / kUqTile);
    WsLayout &L = P.ws;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
    L.keys = take(4 * N);
    L.bags = take(4 * N);
    L.bag_n = take(4 * nb);
    L.fpart = take(sizeof(float) * 2 * P.max_tiles * P.max_dim);
    L.fcnt = take(4 * 2 * P.max_tiles);
    L.ftick = take(4 * P.max_tiles);
    L.keys2 = take(4 * N);
    L.vals2 = take(4 * N);
    L.hist = take(4 * (size_t)kRadix * P.sort_blocks);
    L.dtot = take(4 * kRadix);
    L.seg = take(4 * (N + 1));
    L.ukeys = take(4 * N);
    L.ucnt = take(4 * P.uq_blocks);
    L.uscan = take(4 * (P.uq_blocks + 1));
    L.misc = take(64);
    L.bpart = take(sizeof(float) * 2 * P.max_tiles * P.max_dim);
    L.bcnt = take(4 * 2 * P.max_tiles);
    L.btick = take(4 * P.max_tiles);
    L.cstart = take(4 * ((size_t)P.n_cols + 1));
    L.bw = take(8 * N);
    L.posid = take(4 * N);
    L.ccnt = take(4 * (2 * ((size_t)P.n_cols + 1) + 1));
    L.fstat = take(4 * 8 * P.max_tiles);
    L.zrow = take(kZeroRow);
    L.pairs_n = (size_t)((N + 31) / 32 * 32);
    L.pairs = take(8 * 2 * L.pairs_n);
    L.total = o;
}

int32_t fwd_tile_for(const emb_plan *P, int64_t n_ids)
{
    if (P->fwd_tile) return P->fwd_tile;
    const bool long_bags = n_ids >= (int64_t)kLongBag * P->n_cols * P->batch;
    const bool many = n_ids >= (int64_t)kFwdTileMax * kLongTilesMin;
    return long_bags && many ? kFwdTileMax : P->tile;
}

}  // namespace emb

using namespace emb;

extern "C" {

const char *emb_last_error(void) { return g_last_error.c_str(); }

static size_t plan_mem_bytes(int32_t n_cols)
{
    return align256(sizeof(DevCol) * (size_t)n_cols) + sizeof(uint32_t) * (size_t)(n_cols + 1);
}

static emb_status fill_plan(const emb_column_desc *cols, int32_t n_cols, int32_t batch,
                            int64_t max_ids, const emb_plan_opts *opts, emb_plan &P)
{
    emb_status s = plan_validate(cols, n_cols, batch, max_ids, opts);
    if (s != EMB_OK) return s;
    P.n_cols = n_cols;
    P.batch = batch;
    P.max_ids = max_ids;
    P.tile = opts->tile ? opts->tile : kTileDefault;
    // a fixed tile fixes the forward's too, unless fwd_tile sets that apart
    P.fwd_tile = opts->fwd_tile ? opts->fwd_tile : opts->tile;
    P.opt = opts->opt;
    P.lr = opts->lr;
    P.eps = opts->eps;
    P.hcols = new (std::nothrow) DevCol[n_cols];
    if (!P.hcols) return fail(EMB_ERR_INVALID_ARG, "out of host memory");
    uint64_t row_base = 0;
    int32_t off = 0, maxd = 0;
    for (int32_t c = 0; c < n_cols; c++) {
        const emb_column_desc &d = cols[c];
        DevCol &h = P.hcols[c];
        std::memset(&h, 0, sizeof(h));
        h.kind = d.kind;
        h.pool = d.pool;
        h.dtype = d.dtype;
        h.dim = d.dim;
        h.rows = d.rows;
        h.id_lo = d.id_lo;
        h.id_hi = d.id_hi;
        h.magic = ~uint64_t(0) / (uint64_t)d.rows;
        h.weights = d.weights;
        h.state = d.opt_state;
        h.boundaries = d.boundaries;
        h.n_bnd = (int32_t)d.n_boundaries;
        h.out_off = off;
        h.row_base = (uint32_t)row_base;
        // forward: 8 bf16 elements per lane (16-byte loads) where the dim allows
        h.vec = (d.dtype == EMB_BF16 && d.dim % 8 == 0) ? 8 : 4;
        h.lanes = pow2_ceil(d.dim / h.vec);
        h.glanes = pow2_ceil(d.dim / 4);
        h.seq_max = d.seq_max;
        h.seq_keep_last = d.seq_keep_last;
        h.default_row = d.default_row;
        row_base += (uint64_t)d.rows;
        off += d.dim;
        maxd = std::max(maxd, d.dim);
        P.has_hash |= d.kind == EMB_COL_HASH || d.kind == EMB_COL_IDENTITY;
        P.has_bucket |= d.kind == EMB_COL_BUCKET;
        P.has_keyed |= d.kind == EMB_COL_KEYED;
        P.any_mean |= d.pool == EMB_POOL_MEAN;
        P.all_mean &= d.pool == EMB_POOL_MEAN;
        P.has_trunc |= d.seq_max > 0;
        P.has_default |= d.default_row >= 0;
    }
    P.total_rows = (uint32_t)row_base;
    P.hrow_base = new (std::nothrow) uint32_t[n_cols + 1];
    if (!P.hrow_base) return fail(EMB_ERR_INVALID_ARG, "out of host memory");
    for (int32_t c = 0; c < n_cols; c++) P.hrow_base[c] = P.hcols[c].row_base;
    P.hrow_base[n_cols] = P.total_rows;
    P.sum_dim = off;
    P.max_dim = maxd;
    int bits = 1;
    while (bits < 32 && ((uint64_t(1) << bits) <= (uint64_t)P.total_rows + 1)) bits++;
    P.key_bits = bits;
    plan_layout(P);
    return EMB_OK;
}

emb_status emb_plan_query(const emb_column_desc *cols, int32_t n_cols, int32_t batch,
                          int64_t max_ids, const emb_plan_opts *opts, size_t *plan_bytes,
                          size_t *workspace_bytes)
{
    if (!plan_bytes || !workspace_bytes) return fail(EMB_ERR_INVALID_ARG, "NULL size output");
    emb_plan P;
    emb_status s = fill_plan(cols, n_cols, batch, max_ids, opts, P);
    delete[] P.hcols;
    delete[] P.hrow_base;
    if (s != EMB_OK) return s;
    *plan_bytes = plan_mem_bytes(n_cols);
    *workspace_bytes = P.ws.total;
    return EMB_OK;
}

emb_status emb_plan_create(const emb_column_desc *cols, int32_t n_cols, int32_t batch,
                           int64_t max_ids, const emb_plan_opts *opts, void *plan_mem,
                           void *stream, emb_plan **out)
{
    if (!out) return fail(EMB_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!plan_mem || !aligned(plan_mem, 256)) return fail(EMB_ERR_INVALID_ARG, "plan_mem must be 256-byte aligned device memory");
    emb_plan *P = new (std::nothrow) emb_plan();
    if (!P) return fail(EMB_ERR_INVALID_ARG, "out of host memory");
    emb_status s = fill_plan(cols, n_cols, batch, max_ids, opts, *P);
    if (s != EMB_OK) {
        delete[] P->hcols;
        delete[] P->hrow_base;
        delete P;
        return s;
    }
    P->dcols = static_cast<DevCol *>(plan_mem);
    P->drow_base = reinterpret_cast<uint32_t *>(static_cast<char *>(plan_mem) +
                                                align256(sizeof(DevCol) * (size_t)n_cols));
    hipError_t e = hipMemcpyAsync(P->dcols, P->hcols, sizeof(DevCol) * (size_t)n_cols,
                                  hipMemcpyHostToDevice, static_cast<hipStream_t>(stream));
    if (e == hipSuccess)
        e = hipMemcpyAsync(P->drow_base, P->hrow_base, sizeof(uint32_t) * (size_t)(n_cols + 1),
                           hipMemcpyHostToDevice, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        delete[] P->hcols;
        delete[] P->hrow_base;
        delete P;
        return fail(EMB_ERR_HIP, std::string("hipMemcpyAsync: ") + hipGetErrorString(e));
    }
    // the host copy must outlive the asynchronous copy: it lives until destroy
    *out = P;
    return EMB_OK;
}

emb_status emb_plan_destroy(emb_plan *plan)
{
    if (!plan) return EMB_OK;
    delete[] plan->hcols;
    delete[] plan->hrow_base;
    delete plan;
    return EMB_OK;
}

emb_status emb_plan_forward_tile(const emb_plan *plan, int64_t n_ids, int32_t *tile)
{
    if (!plan || !tile) return fail(EMB_ERR_INVALID_ARG, "NULL argument");
    if (n_ids < 0 || n_ids > plan->max_ids) return fail(EMB_ERR_WORKSPACE, "n_ids exceeds the plan's max_ids");
    *tile = fwd_tile_for(plan, n_ids);
    return EMB_OK;
}

emb_status emb_plan_workspace_view(emb_plan *plan, void *workspace, emb_workspace_view *out)
{
    if (!plan || !workspace || !out) return fail(EMB_ERR_INVALID_ARG, "NULL argument");
    char *w = static_cast<char *>(workspace);
    out->keys = reinterpret_cast<uint32_t *>(w + plan->ws.keys);
    out->bags = reinterpret_cast<int32_t *>(w + plan->ws.bags);
    out->bag_n = reinterpret_cast<int32_t *>(w + plan->ws.bag_n);
    return EMB_OK;
}

}  // extern "C"
