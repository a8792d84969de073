// forward.hip -- the fused multi-column forward: transform, filter, gather, pool.
//
// ONE launch covers every column.  Work follows element count, not column count
// (RecIS Sec. 3.1, "Thread mapping for skewed inputs"): all columns' positions
// form one flat index space (column-major bags), cut into tiles of about T
// positions, one tile per wavefront.  Inside a tile:
//   1. a wavefront-parallel search over the CSR offsets finds the tile's first
//      bag and the offsets around it are staged in LDS; the nominal tile ends
//      k T and (k+1) T move to the end of a short bag they cut, so short bags
//      are never split;
//   2. per column segment, each lane transforms positions (hash + exact mod,
//      identity, bucketize on LDS-staged boundaries, keyed rows), with the
//      validity filter of an embedding column (RECom explainer: out-of-range
//      indices dropped), into LDS; a training step also records the row key and
//      bag of every position for the backward;
//   3. the wavefront splits into groups of P lanes (P * 16 bytes = one table row);
//      each group walks a contiguous run of positions, issuing 8 independent
//      row loads per lane before accumulating them in fp32 registers, and
//      a bag that ends inside the run is written by that group alone -- the
//      unique-writer forward of RecIS Sec. 3.2 / Algorithm 1, no atomics on Y,
//      empty bags produce zero;
//   4. bags cut by group boundaries are combined in LDS; long bags cut by tile
//      boundaries leave fp32 partials in the workspace and the last tile to
//      arrive (atomic ticket) sums the pieces in tile order, so the result does
//      not depend on arrival order.
#include <algorithm>
#include <string>

#include "device.h"

namespace emb {

struct FwdArgs {
    const DevCol *cols;
    int32_t C, B, sumD, maxD, T, training;
    int64_t N, ntiles;
    const int32_t *off;
    const int64_t *ids;
    const float *fvals;
    const int32_t *krows;
    const uint8_t *mask;     // per-position keep byte, or NULL
    const float *pw_in;      // per-position weight, or NULL (all 1)
    uint2 *bw;               // training with weights: (bag, weight bits) of each position
    uint32_t *posid;         // ... and each position's own index (the sort's values)
    int32_t has_default;     // training entries N + bag record the default-row fills
    int32_t *rows_out;       // transform-only launch: the row code of every position
    float *Y;
    uint32_t *keys;
    int32_t *bags;
    int32_t *bag_n;
    float *part;
    int32_t *pcnt;
    uint32_t *tick;
    int64_t *stats;
    int32_t *fstat;          // with stats: each tile's counters [ntiles][kFStat], summed
                             // by fwd_stats afterwards (NULL: atomics on stats)
    uint32_t total_rows;
    uint32_t *cstart;        // training: first position of each column, [C + 1]
    const char *zrow;        // kZeroRow bytes of zeros
};

constexpr int kColCache = 8;
constexpr int kFStat = 8;          // counters per tile record (6 used)

// What one launch of the forward kernel does:
//   kFused      transform + gather + pool (emb_forward, emb_forward_ex);
//   kTransform  the transform only: the row code of every position goes to rows_out
//               (emb_transform; it touches no workspace, so it may run on another
//               stream while the previous step's backward still uses it);
//   kFromRows   gather + pool from row codes a transform-only launch made
//               (emb_forward_rows); truncation and the mask were applied there.
enum FwdMode { kFused = 0, kTransform = 1, kFromRows = 2 };
constexpr int kFeatFilter = 1;    // truncation or a mask: positions are removed
constexpr int kFeatWeights = 2;   // per-position weights or default rows
// A bag of at most kShort positions is never cut by a tile boundary: the tile
// holding its start finishes it (tiles span at most T + kShort - 1 positions).
// Only longer bags are split and combined through the workspace.
constexpr int kShort = 64;

// One wavefront's LDS for tiles of up to TM positions.  The kernel exists for two
// capacities: kTileMax, and kFwdTileMax for batches of long bags, where a longer
// tile cuts fewer bags (fewer pieces through the workspace) at the price of fewer
// waves per SIMD.
template <int TM, bool WT>
struct WaveLds {
    static constexpr int kSpan = TM + kShort;
    static_assert(kSpan >= 8, "the walk's row reads run up to 7 entries past rows[] into pbag[]");
    static constexpr int kOff = TM + 128;   // offsets window: kMargin bags before, the tile's after
    int32_t rows[kSpan];             // transformed row of each tile position
    int32_t pbag[kSpan];             // bag of each tile position (training)
    float wt[WT ? kSpan : 1];        // weight of each tile position (weighted instances)
    int32_t off[kOff];               // window of CSR offsets
    union {
        float part[kWave][8];        // per-lane partial sum of each run's first bag
        float bnd[kBndCap];          // bucket boundaries of the current column
    } x;
    int32_t hbag[kWave], hcnt[kWave], hpass[kWave];
    int32_t cout[kColCache], cdim[kColCache];   // output offset and dim of columns c_first + i
};

struct TileCtx {
    int64_t k;
    int p0;          // k * T: the tile's inputs were loaded from here
    int t0, t1;      // positions of this tile
    int bf, bl;      // first / last non-empty bag touching the tile
    int wb, wn;      // LDS window: offsets[wb .. wb+wn)
};

template <class LT>
__device__ __forceinline__ int offat(const FwdArgs &a, const LT &L, const TileCtx &t, int b)
{
    const unsigned i = (unsigned)(b - t.wb);
    return i < (unsigned)t.wn ? L.off[i] : *gp(a.off + b);
}

// Offsets of the bags the walk touches (bf .. bl + 1).  When the LDS window
// covers them all (W, the usual case) the walk reads LDS only: a global
// fallback inside the walk makes the compiler wait for every outstanding load
// and store before each lookup.
template <bool W, class LT>
__device__ __forceinline__ int offw(const FwdArgs &a, const LT &L, const TileCtx &t, int b)
{
    if (W) return L.off[b - t.wb];
    return offat(a, L, t, b);
}

// the non-empty bag containing position p (p inside the tile)
template <bool W, class LT>
__device__ __forceinline__ int bag_of(const FwdArgs &a, const LT &L, const TileCtx &t, int p)
{
    int lo = t.bf, hi = t.bl + 1;   // off[lo] <= p < off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offw<W>(a, L, t, mid) <= p) lo = mid; else hi = mid;
    }
    return lo;
}

// the next non-empty bag after b (a later position exists)
template <bool W, class LT>
__device__ __forceinline__ int next_bag(const FwdArgs &a, const LT &L, const TileCtx &t, int b)
{
    int nb = b + 1;
    while (offw<W>(a, L, t, nb + 1) == offw<W>(a, L, t, nb)) nb++;
    return nb;
}

// A bag with no valid position in a column with a default row: sort entry N + bag
// gives that row the bag's gradient; other bags leave a sentinel there.  Written
// by the bag's one writer (lane q == 0 of bag_out, or the empty-bag pass).
__device__ __forceinline__ void default_entry(const FwdArgs &a, const DevCol &col, int bag, int n)
{
    const int64_t x = a.N + bag;
    *gp(a.keys + x) = (n == 0 && col.default_row >= 0) ? col.row_base + (uint32_t)col.default_row
                                                       : a.total_rows;
    *gp(a.bags + x) = bag;
    if (a.pw_in) {
        *gp(a.bw + x) = make_uint2((uint32_t)bag, __float_as_uint(1.0f));
        *gp(a.posid + x) = (uint32_t)x;
    }
}

// 4 elements (q * 4 ...) of row r of the column's table as fp32
__device__ __forceinline__ float4 row_slice(const DevCol &col, int64_t r, int q)
{
    if (col.dtype == EMB_BF16) {
        const uint2 v = *gp(reinterpret_cast<const uint2 *>(
            static_cast<const uint16_t *>(col.weights) + r * col.dim + q * 4));
        return make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
    }
    return *gp(reinterpret_cast<const float4 *>(static_cast<const float *>(col.weights) + r * col.dim + q * 4));
}

// V: elements per lane (4, or 8 for bf16 rows whose dim is a multiple of 8)
template <int V, bool EXT>
__device__ __forceinline__ void bag_out(const FwdArgs &a, const DevCol &col, int c, int bag,
                                        const float (&acc)[V], int n, int q, bool qa,
                                        int32_t &zero_bags)
{
    static_assert(V == 4 || V == 8, "one or two 4-element slices per lane");
    const int s = bag - c * a.B;
    if (qa) {
        float o[V];
        const float sc = n == 0 ? 0.f : (col.pool == EMB_POOL_MEAN ? __builtin_amdgcn_rcpf((float)n) : 1.0f);
#pragma unroll
        for (int v = 0; v < V; v++) o[v] = acc[v] * sc;
        if (EXT && n == 0 && col.default_row >= 0) {
#pragma unroll
            for (int v = 0; v < V; v += 4) {
                const float4 d = row_slice(col, col.default_row, q * (V / 4) + v / 4);
                o[v] = d.x; o[v + 1] = d.y; o[v + 2] = d.z; o[v + 3] = d.w;
            }
        }
        EMB_GLOBAL float4 *y = gp(reinterpret_cast<float4 *>(a.Y + (int64_t)s * a.sumD + col.out_off + q * V));
#pragma unroll
        for (int v = 0; v < V; v += 4) y[v / 4] = make_float4(o[v], o[v + 1], o[v + 2], o[v + 3]);
    }
    if (q == 0) {
        if (a.training) *gp(a.bag_n + bag) = n;
        if (EXT && a.training && a.has_default) default_entry(a, col, bag, n);
        zero_bags += (n == 0);
    }
}

// a piece of a bag that crosses a tile boundary: publish it, and if this is the
// last piece to arrive, sum all pieces in tile order and write the bag
template <int V, bool W, bool EXT, class LT>
__device__ __forceinline__ void tile_piece(const FwdArgs &a, const LT &L, const TileCtx &t,
                                           const DevCol &col, int c, int side, int bag,
                                           const float (&sum)[V], int n, int leader, int q, bool qa,
                                           int32_t &zero_bags)
{
    const int64_t T = a.T;
    const int bs = offw<W>(a, L, t, bag), be = offw<W>(a, L, t, bag + 1);
    const int64_t k0 = bs / T, k1 = (be - 1) / T;
    const int64_t slot = t.k * 2 + side;
    float *pp = a.part + slot * a.maxD + q * V;
    if (qa) {
#pragma unroll
        for (int v = 0; v < V; v++) st_agent(pp + v, sum[v]);
    }
    if (q == 0) st_agent(a.pcnt + slot, n);
    wait_vm();                                   // the piece is visible before the ticket
    uint32_t old = 0;
    if (q == 0) old = ticket_add(&a.tick[k0]);
    old = __shfl(old, leader, kWave);
    if (old == (uint32_t)(k1 - k0)) {
        float tot[V];
        const float *p0 = a.part + (k0 * 2 + 1) * a.maxD + q * V;
        int tn = ld_agent(a.pcnt + k0 * 2 + 1);
#pragma unroll
        for (int v = 0; v < V; v++) tot[v] = qa ? ld_agent(p0 + v) : 0.f;
        // the incoming pieces of tiles k0+1 .. k1, four in flight at a time,
        // added in tile order
        constexpr int UP = 4;
        for (int64_t k2 = k0 + 1; k2 <= k1; k2 += UP) {
            float x[UP][V];
            int xn[UP];
#pragma unroll
            for (int r = 0; r < UP; r++) {
                const int64_t kk = min(k2 + r, k1);
                const float *pk = a.part + (kk * 2) * a.maxD + q * V;
                xn[r] = ld_agent(a.pcnt + kk * 2);
#pragma unroll
                for (int v = 0; v < V; v++) x[r][v] = qa ? ld_agent(pk + v) : 0.f;
            }
#pragma unroll
            for (int r = 0; r < UP; r++) {
                if (k2 + r > k1) break;
                tn += xn[r];
#pragma unroll
                for (int v = 0; v < V; v++) tot[v] += x[r][v];
            }
        }
        bag_out<V, EXT>(a, col, c, bag, tot, tn, q, qa, zero_bags);
        if (q == 0) st_agent(&a.tick[k0], 0u);   // ready for the next call
    }
}

// the V row elements of one lane as loaded: fp32 (V = 4), or bf16 pairs (V = 4 or 8)
template <bool BF, int V> struct RowRawT { using type = float4; };
template <> struct RowRawT<true, 4> { using type = uint2; };
template <> struct RowRawT<true, 8> { using type = uint4; };
template <bool BF, int V> using RowRaw = typename RowRawT<BF, V>::type;

__device__ __forceinline__ void row_f32(const float4 &v, float (&w)[4])
{
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
}
__device__ __forceinline__ void row_f32(const uint2 &v, float (&w)[4])
{
    w[0] = bf16_lo(v.x); w[1] = bf16_hi(v.x); w[2] = bf16_lo(v.y); w[3] = bf16_hi(v.y);
}
__device__ __forceinline__ void row_f32(const uint4 &v, float (&w)[8])
{
    w[0] = bf16_lo(v.x); w[1] = bf16_hi(v.x); w[2] = bf16_lo(v.y); w[3] = bf16_hi(v.y);
    w[4] = bf16_lo(v.z); w[5] = bf16_hi(v.z); w[6] = bf16_lo(v.w); w[7] = bf16_hi(v.w);
}

// one lane's slice of row r through a structured buffer descriptor over the
// table (r outside the table's rows: zeros)
template <bool BF, int V> __device__ __forceinline__ RowRaw<BF, V> row_load(__amdgpu_buffer_rsrc_t rs, int r, int off);
template <> __device__ __forceinline__ float4 row_load<false, 4>(__amdgpu_buffer_rsrc_t rs, int r, int off)
{
    const i32x4_t v = struct_buffer_load_x4(rs, r, off, 0, 0);
    return make_float4(__int_as_float(v.x), __int_as_float(v.y), __int_as_float(v.z), __int_as_float(v.w));
}
template <> __device__ __forceinline__ uint4 row_load<true, 8>(__amdgpu_buffer_rsrc_t rs, int r, int off)
{
    const i32x4_t v = struct_buffer_load_x4(rs, r, off, 0, 0);
    return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}
template <> __device__ __forceinline__ uint2 row_load<true, 4>(__amdgpu_buffer_rsrc_t rs, int r, int off)
{
    const i32x2_t v = struct_buffer_load_x2(rs, r, off, 0, 0);
    return make_uint2((uint32_t)v.x, (uint32_t)v.y);
}

// one column segment [s0, s1) of the tile.  A row is read by P lanes (a power
// of two), V elements per lane: 16-byte loads for fp32 rows (BF false, V = 4),
// 8-byte (V = 4) or 16-byte (V = 8) loads for bf16.  With 8 elements a lane
// group pays its per-position work (row address, bag checks, counts) for twice
// the elements.  Eight loads stay in flight per lane either way (with 8
// elements, four in flight made the long-sequence forward 6 % slower, and
// twelve gained nothing).
// SB: tables below 4 GB are read through a structured buffer descriptor (row
// index and lane offset go to the load as they are, and the dropped and default
// codes, negative, fall outside the descriptor's rows and read zeros); larger
// tables form each 64-bit row address in the loop.
template <bool BF, bool W, bool EXT, int V, bool SB, class LT>
__device__ __forceinline__ void fwd_walk(const FwdArgs &a, LT &L, const TileCtx &t,
                                         const DevCol &col, int c, int s0, int s1,
                                         int32_t &zero_bags)
{
    constexpr int U = 8;                       // row loads in flight per lane
    constexpr int esz = BF ? 2 : 4;
    const int P = col.lanes, lp = __ffs(P) - 1;
    const int G = kWave >> lp;
    const int lane = lane_id(), g = lane >> lp, q = lane & (P - 1);
    const int D = col.dim;
    const bool qa = q < D / V;
    const int len = s1 - s0, Lg = (len + G - 1) / G;
    const int ga = min(s0 + g * Lg, s1), ge = min(ga + Lg, s1);
    // lanes past the row's end read lane 0's slice and ignore it
    const int64_t loff = (int64_t)(qa ? q : 0) * V * esz;
    const char *wptr = static_cast<const char *>(col.weights);
    // without per-position weights, positions that add nothing (dropped, DEFAULT,
    // past the run) read zeros instead of row 0, so every loaded slice is added
    // as it is (no select per element); with weights the sum still selects, since
    // a weight may be infinite (those positions read zeros through the buffer
    // descriptor, row 0 otherwise)
    const int64_t rstride = (int64_t)D * esz;
    const __amdgpu_buffer_rsrc_t rsrc = row_buffer(col.weights, SB ? (int)rstride : 0,
                                                   SB ? (int32_t)col.rows : 0);

    float acc[V], hacc[V];
#pragma unroll
    for (int v = 0; v < V; v++) acc[v] = hacc[v] = 0.f;
    int cnt = 0, hcnt = 0, hbag = -1, tbag = -1;
    bool hpass = false;

    if (ga < ge) {
        int b = bag_of<W>(a, L, t, ga);
        int bend = offw<W>(a, L, t, b + 1);
        bool before = offw<W>(a, L, t, b) < ga;
        for (int p = ga; p < ge; p += U) {
            // every load is issued (dropped / default / past-the-run positions read
            // row 0), so that the single wait below covers exactly these loads
            int r[U];
            RowRaw<BF, V> h[U];
            // unconditional LDS reads from one base (immediate offsets): a read past
            // the run's end (at most U - 1 past the tile span) stays inside the wave's
            // LDS (pbag follows rows) and its value is replaced below
            const int32_t *rp = L.rows + (p - t.t0);
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int x = rp[u];
                r[u] = (p + u < ge) ? x : -1;
            }
#pragma unroll
            for (int u = 0; u < U; u++) {
                if (SB) h[u] = row_load<BF, V>(rsrc, r[u], (int)loff);
                else h[u] = *gp(reinterpret_cast<const RowRaw<BF, V> *>(
                         ((!EXT && r[u] < 0) ? a.zrow : wptr) + loff +
                         (uint64_t)(uint32_t)max(r[u], 0) * (uint32_t)rstride));
            }
#pragma unroll
            for (int u = 0; u < U; u++) landed(h[u]);   // before the bag-end stores below
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int pp = p + u;
                if (pp < ge && pp == bend) {       // bag b ended just before pp
                    if (before) {
#pragma unroll
                        for (int v = 0; v < V; v++) hacc[v] = acc[v];
                        hcnt = cnt; hbag = b; hpass = false;
                    } else {
                        bag_out<V, EXT>(a, col, c, b, acc, cnt, q, qa, zero_bags);
                    }
#pragma unroll
                    for (int v = 0; v < V; v++) acc[v] = 0.f;
                    cnt = 0;
                    b = next_bag<W>(a, L, t, b);
                    bend = offw<W>(a, L, t, b + 1);
                    before = false;
                }
                // every loaded row is consumed here, outside any branch: a load
                // whose result is never read would make the next batch wait for
                // every outstanding load and store before reusing its registers
                float w[V];
                row_f32(h[u], w);
                const bool use = pp < ge && r[u] >= 0;
                if (EXT) {
                    // the weight is read here, not with the batch: registers are
                    // short in this loop
                    const float vw = L.wt[min(pp, ge - 1) - t.t0];
#pragma unroll
                    for (int v = 0; v < V; v++) acc[v] += use ? vw * w[v] : 0.f;
                } else {
#pragma unroll
                    for (int v = 0; v < V; v++) acc[v] += w[v];   // zeros where !use
                }
                if (pp < ge) {
                    cnt += (r[u] != -1);
                    if (q == 0) L.pbag[pp - t.t0] = b;
                }
            }
        }
        // the piece holding the run's last position
        if (bend == ge) {
            if (before) {
#pragma unroll
                for (int v = 0; v < V; v++) hacc[v] = acc[v];
                hcnt = cnt; hbag = b; hpass = false;
            } else {
                bag_out<V, EXT>(a, col, c, b, acc, cnt, q, qa, zero_bags);
            }
        } else if (before) {
#pragma unroll
            for (int v = 0; v < V; v++) hacc[v] = acc[v];
            hcnt = cnt; hbag = b; hpass = true;
        } else {
            tbag = b;
        }
    }

    // publish the run's boundary pieces
#pragma unroll
    for (int v = 0; v < V; v++) {
        L.x.part[lane][v] = hacc[v];
    }
    if (q == 0) {
        L.hbag[g] = hbag; L.hcnt[g] = hcnt; L.hpass[g] = hpass;
    }
    wave_sync();

    // bags that start in this run and continue into the next runs
    if (tbag >= 0) {
        float sum[V];
#pragma unroll
        for (int v = 0; v < V; v++) sum[v] = acc[v];
        int n = cnt;
        bool ended = false;
        for (int g2 = g + 1; g2 < G; g2++) {
            if (L.hbag[g2] != tbag) break;
#pragma unroll
            for (int v = 0; v < V; v++) sum[v] += L.x.part[g2 * P + q][v];
            n += L.hcnt[g2];
            if (!L.hpass[g2]) { ended = true; break; }
        }
        if (ended) bag_out<V, EXT>(a, col, c, tbag, sum, n, q, qa, zero_bags);
        else tile_piece<V, W, EXT>(a, L, t, col, c, 1, tbag, sum, n, g * P, q, qa, zero_bags);
    }
    // the bag that came in from the previous tile
    if (g == 0 && hbag >= 0) {
        float sum[V];
#pragma unroll
        for (int v = 0; v < V; v++) sum[v] = hacc[v];
        int n = hcnt;
        bool pass = hpass;
        for (int g2 = 1; pass && g2 < G; g2++) {
            if (L.hbag[g2] != hbag) break;
#pragma unroll
            for (int v = 0; v < V; v++) sum[v] += L.x.part[g2 * P + q][v];
            n += L.hcnt[g2];
            pass = L.hpass[g2];
        }
        tile_piece<V, W, EXT>(a, L, t, col, c, 0, hbag, sum, n, 0, q, qa, zero_bags);
    }
    wave_sync();
}

template <bool BF, bool W, bool EXT, int V, class LT>
__device__ __forceinline__ void fwd_segment(const FwdArgs &a, LT &L, const TileCtx &t,
                                            const DevCol &col, int c, int s0, int s1,
                                            int32_t &zero_bags)
{
    const uint64_t bytes = (uint64_t)col.rows * (uint64_t)(col.dim * (BF ? 2 : 4));
    if (bytes <= 0xFFFFFFFFull && col.rows <= INT32_MAX && col.dim * (BF ? 2 : 4) <= kBufStrideMax)
        fwd_walk<BF, W, EXT, V, true>(a, L, t, col, c, s0, s1, zero_bags);
    else
        fwd_walk<BF, W, EXT, V, false>(a, L, t, col, c, s0, s1, zero_bags);
}

// #{j : b[j] <= x} for sorted b, by binary lifting (B is an LDS or a global array)
template <typename B>
__device__ __forceinline__ int bucket_count(B b, int nb, float x)
{
    int k = 0;
    int step = nb ? (1 << (31 - __clz(nb))) : 0;
    for (; step > 0; step >>= 1)
        if (k + step <= nb && b[k + step - 1] <= x) k += step;
    return k;
}

constexpr int kMargin = 64;             // offsets staged before the tile's first bag

// The raw inputs of the tile's positions, loaded once at the start of the tile so
// that they arrive while the offsets are searched.
template <int TM>
struct TileIn {
    static constexpr int kPL = (TM + kShort) / kWave;   // per lane: p0 + lane + 64 i
    int64_t id[kPL];
    float fv[kPL];
    int32_t kr[kPL];
};

// Sequence truncation and masking remove raw positions before the transform
// (RecIS Sec. 3.1 / Figure 2: SeqTrunc precedes Hash).  A removed position
// becomes a dropped one (-1): no row, not counted in a mean, no gradient.
template <class LT>
__device__ __forceinline__ bool position_kept(const FwdArgs &a, const LT &L,
                                              const TileCtx &t, const DevCol &col, int p)
{
    bool keep = true;
    if (a.mask) keep = *gp(a.mask + p) != 0;
    if (col.seq_max > 0) {
        const int b = bag_of<false>(a, L, t, p);
        const int bs = offat(a, L, t, b), be = offat(a, L, t, b + 1);
        const int j = p - bs;
        keep = keep && (col.seq_keep_last ? j >= be - bs - col.seq_max : j < col.seq_max);
    }
    return keep;
}

// FEAT: the extended forward's parts this launch needs, kFeatFilter (truncation
// or the mask) and kFeatWeights (per-position weights or default rows)
template <int FEAT, int MODE, int TM, bool WT>
__device__ __forceinline__ void fwd_transform(const FwdArgs &a, WaveLds<TM, WT> &L, const TileCtx &t,
                                              const DevCol &col, int s0, int s1,
                                              const TileIn<TM> &in, int32_t (&cnt)[5])
{
    constexpr int kPL = TileIn<TM>::kPL;
    const int lane = lane_id();
    const int nbd = col.n_bnd;
    const bool staged = col.kind == EMB_COL_BUCKET && nbd <= kBndCap;
    if (staged) {
        for (int i = lane; i < nbd; i += kWave) L.x.bnd[i] = *gp(col.boundaries + i);
        wave_sync();
    }
    const uint64_t rows = (uint64_t)col.rows;
#pragma unroll
    for (int i = 0; i < kPL; i++) {
        const int p = t.p0 + lane + kWave * i;
        if (p < s0 || p >= s1) continue;
        int r;
        if (MODE == kFromRows) {
            // row codes from a transform-only launch, checked like keyed rows
            const int kr = in.kr[i];
            r = kr == -2 ? -2 : ((kr >= 0 && (uint64_t)kr < rows) ? kr : -1);
        } else if (col.kind == EMB_COL_HASH) {
            const int64_t id = in.id[i];
            r = (id >= col.id_lo && id < col.id_hi)
                    ? (int)mod_magic(splitmix64((uint64_t)id), rows, col.magic) : -1;
        } else if (col.kind == EMB_COL_IDENTITY) {
            const int64_t id = in.id[i];
            r = (id >= 0 && (uint64_t)id < rows) ? (int)id : -1;
        } else if (col.kind == EMB_COL_BUCKET) {
            const float x = in.fv[i];
            r = (x != x) ? -1 : (staged ? bucket_count(L.x.bnd, nbd, x)
                                        : bucket_count(gp(col.boundaries), nbd, x));
        } else {
            const int kr = in.kr[i];
            r = kr == EMB_ROW_DEFAULT ? -2 : ((kr >= 0 && (uint64_t)kr < rows) ? kr : -1);
        }
        // removed positions are counted apart from the transform's drops
        const bool removed = (FEAT & kFeatFilter) && MODE != kFromRows && !position_kept(a, L, t, col, p);
        cnt[2] += (r == -1 && !removed);
        cnt[4] += removed;
        if (removed) r = -1;
        L.rows[p - t.t0] = r;
        if (FEAT & kFeatWeights) {
            const float v = a.pw_in ? *gp(a.pw_in + p) : 1.0f;
            L.wt[p - t.t0] = v;
            if (a.training && a.pw_in) *gp(a.posid + p) = (uint32_t)p;
        }
        cnt[0] += 1;
        cnt[1] += (r >= 0);
        cnt[3] += (r == -2);
        if (a.training)
            *gp(a.keys + p) = r >= 0 ? col.row_base + (uint32_t)r
                                     : (r == -2 ? a.total_rows + 1u : a.total_rows);
    }
    wave_sync();
}

// Positions of column c inside the tile.  The first column starts at or before
// t0 and the last ends at or after t1; the other boundaries are bags bf+1 .. bl,
// inside the LDS window when it covers the walk (win).
template <class LT>
__device__ __forceinline__ int col_lo(const FwdArgs &a, const LT &L, const TileCtx &t, int c,
                                      int c_first, bool win)
{
    if (c == c_first) return t.t0;
    return max(t.t0, win ? offw<true>(a, L, t, c * a.B) : offat(a, L, t, c * a.B));
}

template <class LT>
__device__ __forceinline__ int col_hi(const FwdArgs &a, const LT &L, const TileCtx &t, int c,
                                      int c_last, bool win)
{
    if (c == c_last) return t.t1;
    return min(t.t1, win ? offw<true>(a, L, t, (c + 1) * a.B) : offat(a, L, t, (c + 1) * a.B));
}

// FEAT: the parts of the extended forward this launch needs (kFeatFilter: a
// column truncates or the call has a mask; kFeatWeights: per-position weights or
// a column with a default row), each a separate instance so that the plain
// forward carries none of that code.  MODE: FwdMode.  TM: the tile capacity, T <= TM
// (the larger one holds more inputs per lane in registers: three waves per SIMD
// instead of four; four waves at the larger capacity spill in every tile's set-up:
// long sequences 234 against 208 us).  Only the weighted instances keep per-position
// weights in LDS.
template <int FEAT, int MODE, int TM>
__global__ __launch_bounds__(kTileBlock, TM > kTileMax ? 3 : 4) void fwd_kernel(FwdArgs a)
{
    constexpr bool EXT = (FEAT & kFeatWeights) != 0;
    using Lds = WaveLds<TM, EXT>;
    constexpr int kPL = TileIn<TM>::kPL, kOff = Lds::kOff;
    __shared__ Lds lds[kTileWaves];
    const int w = threadIdx.x / kWave, lane = lane_id();
    Lds &L = lds[w];
    TileCtx t;
    t.k = xcd_block(blockIdx.x, gridDim.x, 0) * kTileWaves + w;
    if (t.k >= a.ntiles) return;
    const int N = (int)a.N, T = a.T, nbag = a.C * a.B;
    // nominal range [k T, (k+1) T); the real one moves each end to the end of a
    // short bag that the nominal boundary cuts
    const int x0 = (int)min<int64_t>(t.k * T, N), x1 = (int)min<int64_t>((t.k + 1) * T, N);
    t.p0 = x0;
    const bool last = t.k == a.ntiles - 1;
    TileIn<TM> in;
#pragma unroll
    for (int i = 0; i < kPL; i++) {
        const int p = x0 + lane + kWave * i;
        const bool ok = p < N;
        in.id[i] = (MODE != kFromRows && a.ids && ok) ? *gp(a.ids + p) : 0;
        in.fv[i] = (MODE != kFromRows && a.fvals && ok) ? *gp(a.fvals + p) : 0.f;
        in.kr[i] = (a.krows && ok) ? *gp(a.krows + p) : 0;
    }

    // the bags this tile touches: one global search for the first, then the
    // offsets window in LDS answers the rest
    int own_lo, own_hi;
    int b0 = nbag;
    if (x0 < x1) {
        // bag holding x0; the search starts at the bag a uniform spread of the
        // positions would put there
        b0 = (int)wave_upper_bound_near(a.off, (int64_t)nbag + 1, x0,
                                        (int64_t)x0 * nbag / max(N, 1)) - 1;
        t.wb = max(0, b0 - kMargin);
    } else {
        t.wb = 0;
    }
    t.wn = min(nbag + 1 - t.wb, kOff);
    {
        // all window loads in flight at once
        int o[kOff / kWave];
#pragma unroll
        for (int j = 0; j < kOff / kWave; j++) {
            const int i = lane + kWave * j;
            o[j] = i < t.wn ? *gp(a.off + t.wb + i) : 0;
        }
#pragma unroll
        for (int j = 0; j < kOff / kWave; j++) {
            const int i = lane + kWave * j;
            if (i < t.wn) L.off[i] = o[j];
        }
    }
    wave_sync();
    t.t0 = x0;
    t.t1 = x1;
    if (x0 < x1) {
        // start: a short bag begun before x0 belongs to the previous tile (which
        // ends at its end); the same rule, applied there, gives that tile's end
        t.bf = b0;
        t.bl = b0;                     // provisional, for offat's window checks
        if (x0 > 0) {
            const int bs = offat(a, L, t, b0), be = offat(a, L, t, b0 + 1);
            if (bs < x0 && be - bs <= kShort && be < min(x0 + T, N)) {
                t.t0 = be;
                int nb = b0 + 1;
                while (offat(a, L, t, nb + 1) == be) nb++;
                t.bf = nb;
            }
        }
        // end: the bag holding x1, finished here if short
        int b1 = -1;
        if (x1 < N) {
            const int f = b0 - t.wb;
            b1 = (L.off[t.wn - 1] > x1)
                     ? b0 + (int)wave_upper_bound(L.off + f, (int64_t)(t.wn - f), x1) - 1
                     : (int)wave_upper_bound(a.off, (int64_t)nbag + 1, x1) - 1;
            const int bs = offat(a, L, t, b1), be = offat(a, L, t, b1 + 1);
            if (bs < x1 && be - bs <= kShort && be < min(x1 + T, N)) t.t1 = be;
        }
        if (t.t1 != x1) {
            t.bl = b1;                 // the short bag finished here
        } else {
            const int f = b0 - t.wb;
            t.bl = (L.off[t.wn - 1] > t.t1 - 1)
                       ? b0 + (int)wave_upper_bound(L.off + f, (int64_t)(t.wn - f), t.t1 - 1) - 1
                       : (int)wave_upper_bound(a.off, (int64_t)nbag + 1, t.t1 - 1) - 1;
        }
        // owned bags start in [t0, t1): empty bags sitting exactly at t0 come first
        own_lo = t.bf + 1;
        if (offat(a, L, t, t.bf) == t.t0) {
            own_lo = t.bf;
            while (own_lo > 0 && offat(a, L, t, own_lo - 1) == t.t0) own_lo--;
        }
        own_hi = last ? nbag : t.bl + 1;
    } else {
        t.bf = nbag;
        t.bl = nbag - 1;
        own_lo = 0;
        own_hi = nbag;
    }
    if (a.training) {
        // every bag is owned by exactly one tile: the owner of a column's first bag
        // records where the column starts (for the backward's column sort)
        for (int c = (own_lo + a.B - 1) / a.B + lane; c * a.B < own_hi; c += kWave) {
            const unsigned i = (unsigned)(c * a.B - t.wb);
            *gp(a.cstart + c) = (uint32_t)(i < (unsigned)t.wn ? L.off[i] : *gp(a.off + c * a.B));
        }
        if (last && lane == 0) *gp(a.cstart + a.C) = (uint32_t)N;
    }

    int32_t cnt[5] = {0, 0, 0, 0, 0};   // per lane: at most kPL positions, kWave bags
    int32_t zero_bags = 0;
    if (t.t0 < t.t1) {
        const int c_first = t.bf / a.B, c_last = t.bl / a.B;
        const bool win = t.bl + 1 < t.wb + t.wn;   // the window covers every bag the walk reads
        // transform every position of the tile, then walk each column segment
        for (int c = c_first; c <= c_last; c++) {
            const int cu = uniform(c);
            if (cu - c_first < kColCache && lane == 0) {
                L.cout[cu - c_first] = a.cols[cu].out_off;
                L.cdim[cu - c_first] = a.cols[cu].dim;
            }
            const int s0 = col_lo(a, L, t, cu, c_first, win), s1 = col_hi(a, L, t, cu, c_last, win);
            if (s0 >= s1) continue;
            const DevCol col = a.cols[cu];
            fwd_transform<FEAT, MODE>(a, L, t, col, s0, s1, in, cnt);
        }
        if (MODE == kTransform) {
#pragma unroll
            for (int i = 0; i < kPL; i++) {
                const int p = t.p0 + lane + kWave * i;
                if (p >= t.t0 && p < t.t1) *gp(a.rows_out + p) = L.rows[p - t.t0];
            }
        }
        for (int c = c_first; c <= c_last && MODE != kTransform; c++) {
            const int cu = uniform(c);
            const int s0 = col_lo(a, L, t, cu, c_first, win), s1 = col_hi(a, L, t, cu, c_last, win);
            if (s0 >= s1) continue;
            const DevCol col = a.cols[cu];
            if (win) {
                if (col.dtype == EMB_BF16 && col.vec == 8) fwd_segment<true, true, EXT, 8>(a, L, t, col, cu, s0, s1, zero_bags);
                else if (col.dtype == EMB_BF16) fwd_segment<true, true, EXT, 4>(a, L, t, col, cu, s0, s1, zero_bags);
                else fwd_segment<false, true, EXT, 4>(a, L, t, col, cu, s0, s1, zero_bags);
            } else {
                if (col.dtype == EMB_BF16 && col.vec == 8) fwd_segment<true, false, EXT, 8>(a, L, t, col, cu, s0, s1, zero_bags);
                else if (col.dtype == EMB_BF16) fwd_segment<true, false, EXT, 4>(a, L, t, col, cu, s0, s1, zero_bags);
                else fwd_segment<false, false, EXT, 4>(a, L, t, col, cu, s0, s1, zero_bags);
            }
        }
        if (a.training) {
#pragma unroll
            for (int i = 0; i < kPL; i++) {
                const int p = t.p0 + lane + kWave * i;
                if (p >= t.t0 && p < t.t1) {
                    *gp(a.bags + p) = L.pbag[p - t.t0];
                    // the weighted backward reads bag and weight in one load
                    if (EXT && a.pw_in)
                        *gp(a.bw + p) = make_uint2((uint32_t)L.pbag[p - t.t0], __float_as_uint(L.wt[p - t.t0]));
                }
            }
        }
    }

    // bags with no position that this tile owns: the zero default.  Usually their
    // offsets are in the LDS window and their columns were cached by the
    // transform: then the loop reads LDS only (a global read in it would wait
    // for every Y store issued so far)
    if (MODE == kTransform) own_hi = own_lo;   // outputs are the forward's
    const int c_base = t.t0 < t.t1 ? t.bf / a.B : 0;
    const bool zfast = t.t0 < t.t1 && own_lo >= t.wb && own_hi < t.wb + t.wn &&
                       own_lo / a.B >= c_base && (own_hi - 1) / a.B <= t.bl / a.B &&
                       (own_hi - 1) / a.B - c_base < kColCache;
    if (zfast && !(EXT && a.has_default)) {
        for (int b = own_lo + lane; b < own_hi; b += kWave) {
            if (L.off[b - t.wb] != L.off[b + 1 - t.wb]) continue;
            const int c = b / a.B;
            const int dim = L.cdim[c - c_base];
            EMB_GLOBAL float4 *y = gp(reinterpret_cast<float4 *>(
                a.Y + (int64_t)(b - c * a.B) * a.sumD + L.cout[c - c_base]));
            for (int d = 0; d < dim / 4; d++) y[d] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (a.training) *gp(a.bag_n + b) = 0;
            zero_bags++;
        }
    } else {
        for (int b = own_lo + lane; b < own_hi; b += kWave) {
            if (offat(a, L, t, b) != offat(a, L, t, b + 1)) continue;
            const int c = b / a.B;
            EMB_GLOBAL float4 *y = gp(reinterpret_cast<float4 *>(
                a.Y + (int64_t)(b - c * a.B) * a.sumD + *gp(&a.cols[c].out_off)));
            const int dim = *gp(&a.cols[c].dim);
            const int64_t dr = EXT ? *gp(&a.cols[c].default_row) : -1;
            if (EXT && dr >= 0) {
                const DevCol col = a.cols[c];
                for (int d = 0; d < dim / 4; d++) y[d] = row_slice(col, dr, d);
            } else {
                for (int d = 0; d < dim / 4; d++) y[d] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
            if (a.training) *gp(a.bag_n + b) = 0;
            if (EXT && a.training && a.has_default) default_entry(a, a.cols[c], b, 0);
            zero_bags++;
        }
    }

    // per-position counts come from the launch that transforms (a kFromRows
    // launch counts only its bags)
    if (MODE == kFromRows) cnt[0] = cnt[1] = cnt[2] = cnt[3] = cnt[4] = 0;
    if (a.stats) {
        const uint32_t s0 = wave_sum_u32(cnt[0]), s1 = wave_sum_u32(cnt[1]);
        const uint32_t s2 = wave_sum_u32(cnt[2]), s3 = wave_sum_u32(cnt[3]);
        const uint32_t s4 = wave_sum_u32(zero_bags), s5 = wave_sum_u32(cnt[4]);
        if (a.fstat) {
            // this tile's record; fwd_stats adds all of them afterwards (same-address
            // atomics from every tile serialized the forward)
            if (lane == 0) {
                uint4 *r = reinterpret_cast<uint4 *>(a.fstat + t.k * kFStat);
                r[0] = make_uint4(s0, s1, s2, s3);
                r[1] = make_uint4(s4, s5, 0u, 0u);
            }
        } else if (lane == 0) {
            if (s0) atomicAdd((unsigned long long *)&a.stats[EMB_STAT_IDS], (unsigned long long)s0);
            if (s1) atomicAdd((unsigned long long *)&a.stats[EMB_STAT_VALID], (unsigned long long)s1);
            if (s2) atomicAdd((unsigned long long *)&a.stats[EMB_STAT_DROPPED], (unsigned long long)s2);
            if (s3) atomicAdd((unsigned long long *)&a.stats[EMB_STAT_DEFAULT], (unsigned long long)s3);
            if (s4) atomicAdd((unsigned long long *)&a.stats[EMB_STAT_ZERO_BAGS], (unsigned long long)s4);
            if (s5) atomicAdd((unsigned long long *)&a.stats[EMB_STAT_FILTERED], (unsigned long long)s5);
        }
    }
}

// The forward's counters: the sum of every tile's record, added to stats.
__global__ __launch_bounds__(kBlock) void fwd_stats(const int32_t *__restrict__ fstat, int64_t ntiles,
                                                   int64_t *__restrict__ stats)
{
    __shared__ uint32_t part[kWavesPerBlock][6];
    uint32_t acc[6] = {0u, 0u, 0u, 0u, 0u, 0u};
    for (int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x; k < ntiles; k += (int64_t)gridDim.x * kBlock) {
        const uint4 r0 = *gp(reinterpret_cast<const uint4 *>(fstat + k * kFStat));
        const uint4 r1 = *gp(reinterpret_cast<const uint4 *>(fstat + k * kFStat + 4));
        acc[0] += r0.x; acc[1] += r0.y; acc[2] += r0.z; acc[3] += r0.w; acc[4] += r1.x; acc[5] += r1.y;
    }
    const int w = threadIdx.x / kWave;
#pragma unroll
    for (int i = 0; i < 6; i++) {
        const uint32_t s = wave_sum_u32(acc[i]);
        if (lane_id() == 0) part[w][i] = s;
    }
    __syncthreads();
    if (threadIdx.x < 6) {
        unsigned long long s = 0;
        for (int k = 0; k < kWavesPerBlock; k++) s += part[k][threadIdx.x];
        const int idx[6] = {EMB_STAT_IDS, EMB_STAT_VALID, EMB_STAT_DROPPED, EMB_STAT_DEFAULT,
                            EMB_STAT_ZERO_BAGS, EMB_STAT_FILTERED};
        if (s) atomicAdd((unsigned long long *)&stats[idx[threadIdx.x]], s);
    }
}

}  // namespace emb

using namespace emb;

template <int FEAT, int MODE>
static void launch_one(int64_t blocks, const FwdArgs &a, void *stream)
{
    if (a.T > kTileMax)
        hipLaunchKernelGGL((fwd_kernel<FEAT, MODE, kFwdTileMax>), dim3((unsigned)blocks), dim3(kTileBlock),
                           0, static_cast<hipStream_t>(stream), a);
    else
        hipLaunchKernelGGL((fwd_kernel<FEAT, MODE, kTileMax>), dim3((unsigned)blocks), dim3(kTileBlock),
                           0, static_cast<hipStream_t>(stream), a);
}

// sc: the split-bag partials and tickets of an inference call come from there
// instead of a workspace (emb_forward_noalloc); workspace is then NULL
static emb_status forward_impl(int mode, emb_plan *plan, const int32_t *offsets, const int64_t *ids,
                               const float *fvals, const int32_t *keyed_rows, const float *pweights,
                               const uint8_t *mask, int32_t *rows_out, int64_t n_ids, float *out,
                               void *workspace, int32_t training, int64_t *stats, void *stream,
                               const FwdScratch *sc = nullptr)
{
    if (!plan) return fail(EMB_ERR_INVALID_ARG, "plan is NULL");
    if (!offsets) return fail(EMB_ERR_INVALID_ARG, "offsets are required");
    if (sc && (mode != kFused || training || workspace))
        return fail(EMB_ERR_INVALID_ARG, "the fixed scratch serves the inference forward only");
    if (mode != kTransform && (!out || (!workspace && !sc)))
        return fail(EMB_ERR_INVALID_ARG, "out and workspace are required");
    if (n_ids < 0 || n_ids > plan->max_ids)
        return fail(EMB_ERR_WORKSPACE, "n_ids exceeds the plan's max_ids");
    if (mode == kFromRows) {
        if (n_ids > 0 && !keyed_rows) return fail(EMB_ERR_INVALID_ARG, "rows required");
    } else {
        if (plan->has_hash && n_ids > 0 && !ids) return fail(EMB_ERR_INVALID_ARG, "ids required (hash/identity columns)");
        if (plan->has_bucket && n_ids > 0 && !fvals) return fail(EMB_ERR_INVALID_ARG, "fvals required (bucket columns)");
        if (plan->has_keyed && n_ids > 0 && !keyed_rows) return fail(EMB_ERR_INVALID_ARG, "keyed_rows required (keyed columns)");
    }
    if (mode == kTransform && n_ids > 0 && !rows_out) return fail(EMB_ERR_INVALID_ARG, "rows_out required");
    if (mode != kTransform && !aligned(out, 16)) return fail(EMB_ERR_INVALID_ARG, "out must be 16-byte aligned");
    if (mode != kTransform && !sc && !aligned(workspace, 256))
        return fail(EMB_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    if (mode == kTransform) training = 0;      // writes nothing but rows_out (and stats)
    FwdArgs a{};
    char *ws = static_cast<char *>(workspace);
    a.cols = plan->dcols;
    a.C = plan->n_cols;
    a.B = plan->batch;
    a.sumD = plan->sum_dim;
    a.maxD = plan->max_dim;
    a.T = fwd_tile_for(plan, n_ids);
    a.training = training ? 1 : 0;
    a.N = n_ids;
    a.ntiles = std::max<int64_t>(1, (n_ids + a.T - 1) / a.T);
    a.off = offsets;
    a.ids = ids;
    a.fvals = fvals;
    a.krows = keyed_rows;
    a.mask = mask;
    a.pw_in = pweights;
    a.has_default = plan->has_default ? 1 : 0;
    a.rows_out = rows_out;
    a.Y = out;
    if (ws) {
        a.bw = reinterpret_cast<uint2 *>(ws + plan->ws.bw);
        a.posid = reinterpret_cast<uint32_t *>(ws + plan->ws.posid);
        a.keys = reinterpret_cast<uint32_t *>(ws + plan->ws.keys);
        a.bags = reinterpret_cast<int32_t *>(ws + plan->ws.bags);
        a.bag_n = reinterpret_cast<int32_t *>(ws + plan->ws.bag_n);
        a.part = reinterpret_cast<float *>(ws + plan->ws.fpart);
        a.pcnt = reinterpret_cast<int32_t *>(ws + plan->ws.fcnt);
        a.tick = reinterpret_cast<uint32_t *>(ws + plan->ws.ftick);
        a.cstart = reinterpret_cast<uint32_t *>(ws + plan->ws.cstart);
        a.zrow = ws + plan->ws.zrow;
    }
    if (ws) a.fstat = reinterpret_cast<int32_t *>(ws + plan->ws.fstat);
    if (sc) {
        a.zrow = sc->zrow;
        a.part = sc->part;
        a.pcnt = sc->pcnt;
        a.tick = sc->tick;
        a.fstat = sc->fstat;
    }
    a.stats = stats;
    a.total_rows = plan->total_rows;
    if (training) {
        plan->last_n = n_ids;
        plan->last_weighted = pweights != nullptr;
    }
    // contiguous tile ranges per XCD: each L2 caches the rows of fewer columns
    const int64_t blocks = xcd_grid((a.ntiles + kTileWaves - 1) / kTileWaves, 0);
    const bool filt = mask || plan->has_trunc, wts = pweights || plan->has_default;
    if (mode == kTransform) {
        if (filt) launch_one<kFeatFilter, kTransform>(blocks, a, stream);
        else launch_one<0, kTransform>(blocks, a, stream);
    } else if (mode == kFromRows) {
        a.mask = nullptr;                      // applied by the transform
        if (wts) launch_one<kFeatWeights, kFromRows>(blocks, a, stream);
        else launch_one<0, kFromRows>(blocks, a, stream);
    } else if (filt && wts) {
        launch_one<kFeatFilter | kFeatWeights, kFused>(blocks, a, stream);
    } else if (filt) {
        launch_one<kFeatFilter, kFused>(blocks, a, stream);
    } else if (wts) {
        launch_one<kFeatWeights, kFused>(blocks, a, stream);
    } else {
        launch_one<0, kFused>(blocks, a, stream);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(EMB_ERR_HIP, std::string("fwd_kernel launch: ") + hipGetErrorString(e));
    if (stats && a.fstat) {
        const int64_t sb = std::min<int64_t>(64, (a.ntiles + kBlock - 1) / kBlock);
        hipLaunchKernelGGL(fwd_stats, dim3((unsigned)sb), dim3(kBlock), 0, static_cast<hipStream_t>(stream),
                           a.fstat, a.ntiles, stats);
        e = hipGetLastError();
        if (e != hipSuccess) return fail(EMB_ERR_HIP, std::string("fwd_stats launch: ") + hipGetErrorString(e));
    }
    return EMB_OK;
}

extern "C" emb_status emb_forward(emb_plan *plan, const int32_t *offsets, const int64_t *ids,
                                  const float *fvals, const int32_t *keyed_rows, int64_t n_ids,
                                  float *out, void *workspace, int32_t training, int64_t *stats,
                                  void *stream)
{
    return forward_impl(kFused, plan, offsets, ids, fvals, keyed_rows, nullptr, nullptr, nullptr,
                        n_ids, out, workspace, training, stats, stream);
}

extern "C" emb_status emb_forward_ex(emb_plan *plan, const int32_t *offsets, const int64_t *ids,
                                     const float *fvals, const int32_t *keyed_rows,
                                     const float *pweights, const uint8_t *mask, int64_t n_ids,
                                     float *out, void *workspace, int32_t training, int64_t *stats,
                                     void *stream)
{
    return forward_impl(kFused, plan, offsets, ids, fvals, keyed_rows, pweights, mask, nullptr,
                        n_ids, out, workspace, training, stats, stream);
}

extern "C" emb_status emb_transform(emb_plan *plan, const int32_t *offsets, const int64_t *ids,
                                    const float *fvals, const int32_t *keyed_rows,
                                    const uint8_t *mask, int64_t n_ids, int32_t *rows_out,
                                    int64_t *stats, void *stream)
{
    return forward_impl(kTransform, plan, offsets, ids, fvals, keyed_rows, nullptr, mask, rows_out,
                        n_ids, nullptr, nullptr, 0, stats, stream);
}

extern "C" emb_status emb_forward_rows(emb_plan *plan, const int32_t *offsets, const int32_t *rows,
                                       const float *pweights, int64_t n_ids, float *out,
                                       void *workspace, int32_t training, int64_t *stats,
                                       void *stream)
{
    return forward_impl(kFromRows, plan, offsets, nullptr, nullptr, rows, pweights, nullptr, nullptr,
                        n_ids, out, workspace, training, stats, stream);
}

namespace emb {
size_t fwd_scratch_bytes(const emb_plan *plan, int64_t n_ids, FwdScratch *layout, void *base)
{
    const int32_t T = fwd_tile_for(plan, n_ids);
    const int64_t tiles = std::max<int64_t>(1, (n_ids + T - 1) / T);
    auto a256 = [](size_t x) { return (x + 255) & ~size_t(255); };
    const size_t part = a256(sizeof(float) * 2 * (size_t)tiles * (size_t)plan->max_dim);
    const size_t pcnt = a256(sizeof(int32_t) * 2 * (size_t)tiles);
    const size_t tick = a256(sizeof(uint32_t) * (size_t)tiles);
    const size_t fst = a256(sizeof(int32_t) * kFStat * (size_t)tiles);
    if (layout) {
        // the zero row first: it sits at the same place for every batch size
        char *b = static_cast<char *>(base);
        layout->zrow = b;
        b += kZeroRow;
        layout->part = reinterpret_cast<float *>(b);
        layout->pcnt = reinterpret_cast<int32_t *>(b + part);
        layout->tick = reinterpret_cast<uint32_t *>(b + part + pcnt);
        layout->fstat = reinterpret_cast<int32_t *>(b + part + pcnt + tick);
        layout->tiles = tiles;
    }
    return kZeroRow + part + pcnt + tick + fst;
}

emb_status forward_with_scratch(emb_plan *plan, const int32_t *offsets, const int64_t *ids,
                                const float *fvals, const int32_t *keyed_rows, int64_t n_ids,
                                float *out, int64_t *stats, void *stream, const FwdScratch &sc)
{
    return forward_impl(kFused, plan, offsets, ids, fvals, keyed_rows, nullptr, nullptr, nullptr,
                        n_ids, out, nullptr, 0, stats, stream, &sc);
}
}  // namespace emb
