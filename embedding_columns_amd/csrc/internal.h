// internal.h -- layouts shared by the host entry points and the gfx950 kernels.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "emb.h"

namespace emb {

constexpr int kWave = 64;            // CDNA wavefront
constexpr int kWavesPerBlock = 4;    // each wavefront owns one tile; no block-wide barriers
constexpr int kBlock = kWave * kWavesPerBlock;
// The tile kernels (forward, segment apply) launch one wavefront per workgroup:
// their tiles take very different times, and a single-wave workgroup frees its
// slot as soon as its tile is done.
#ifndef EMB_TILE_WAVES
#define EMB_TILE_WAVES 1
#endif
constexpr int kTileWaves = EMB_TILE_WAVES;
constexpr int kTileBlock = kWave * kTileWaves;
constexpr int kTileMax = 256;        // positions (or sorted contributors) per wavefront tile
constexpr int kTileDefault = 256;
constexpr int kFwdTileMax = 512;     // forward tiles of a batch of long bags (a second instance)
constexpr int kLongBag = 64;         // mean positions per bag from which a batch counts as long
// ... and the long tiles a batch must fill: twice the waves of that instance the
// chip holds at once (3 per SIMD, 1024 SIMDs).  Fewer tiles leave SIMDs idle, and
// there shorter tiles, more of them, finish sooner.
constexpr int64_t kLongTilesMin = 2 * 3 * 1024;
constexpr int kOffCap = kTileMax + 128;  // LDS window of segment offsets per wavefront
constexpr int kBndCap = 256;             // bucket boundaries staged in LDS (more: read from memory)
constexpr int kMaxDimF32 = 256;
constexpr int kMaxDimBF16 = 512;

// radix sort of (key, value) pairs
constexpr int kRadixBits = 9;                      // 3 passes for keys of <= 27 bits
constexpr int kRadix = 1 << kRadixBits;
constexpr int kSortItems = 16;                       // keys per thread
constexpr int kSortTile = kBlock * kSortItems;       // 4096 keys per block
constexpr int kUqItems = 8;                          // unique-row kernels: keys per thread
constexpr int kUqTile = kBlock * kUqItems;           // 2048 keys per block

// One column as the kernels read it (plan device memory), 96 bytes.
struct DevCol {
    int32_t kind, pool, dtype, dim;
    int64_t rows;
    int64_t id_lo, id_hi;
    uint64_t magic;          // floor((2^64 - 1) / rows): exact 64-bit remainder by multiply-high
    void *weights;
    float *state;
    const float *boundaries;
    int32_t n_bnd;
    int32_t out_off;         // first output column of this embedding column
    uint32_t row_base;       // sum of rows of the columns before this one
    int32_t lanes;           // forward lanes per row, vec elements each: pow2 >= dim / vec
    int32_t vec;             // forward elements per lane: 8 for bf16 rows with dim % 8 == 0, else 4
    int32_t glanes;          // lanes per gradient row (same as lanes)
    int32_t seq_max;         // keep at most this many positions per bag (0: all)
    int32_t seq_keep_last;   // ... the last seq_max (1) or the first (0)
    int64_t default_row;     // row read by a bag with no valid position, or -1 (zero vector)
};
static_assert(sizeof(DevCol) == 112, "DevCol layout");
static_assert(kOffCap % kWave == 0, "window loads are unrolled per lane");

// Byte offsets of the workspace regions (each 256-byte aligned).
struct WsLayout {
    size_t keys, bags, bag_n;                 // forward -> backward
    size_t fpart, fcnt, ftick;                // forward split-bag partials and tickets
    size_t keys2, vals2;                      // radix sort ping-pong
    size_t hist, dtot;                        // radix histograms, digit totals
    size_t seg, ukeys, ucnt, uscan, misc;     // unique rows: segment starts, keys, block counts
    size_t bpart, bcnt, btick;                // backward split-segment partials and tickets
    size_t cstart;                            // first position of each column [C + 1] (forward -> backward)
    size_t bw, posid;                         // weighted forward -> backward: (bag, weight) and index per position
    size_t ccnt;                              // column sort -> compaction: valid keys per column, their
                                              //   prefix [2 (C + 1)], and the ticket of the last column
    size_t fstat;                             // forward counters, one 8-word record per tile
    size_t zrow;                              // 1 KB never written: stays zero (the workspace is
                                              //   zero-filled once); the plain forward's masked
                                              //   positions load it
    size_t pairs;                             // radix passes between the first and the last:
    size_t pairs_n;                           //   (key, value) pairs, two buffers of pairs_n
    size_t total;
};

}  // namespace emb

struct emb_plan {
    int32_t n_cols = 0, batch = 0;
    int64_t max_ids = 0;
    int32_t sum_dim = 0, max_dim = 0;
    int32_t tile = emb::kTileDefault;
    int32_t fwd_tile = 0;          // positions per forward tile; 0: chosen per batch (fwd_tile_for)
    int32_t opt = EMB_OPT_EMIT;
    float lr = 0.f, eps = 0.f;
    uint32_t total_rows = 0;       // sum of rows: keys >= this are sentinels
    int32_t key_bits = 0;          // bits needed for keys up to total_rows + 1
    int64_t max_tiles = 0;         // tiles of the largest batch
    int64_t sort_blocks = 0;       // radix blocks of the largest batch
    int64_t uq_blocks = 0;         // unique-row blocks of the largest batch
    bool has_hash = false, has_bucket = false, has_keyed = false, any_mean = false;
    bool all_mean = true;          // every column pools by mean
    bool has_trunc = false;        // some column truncates its bags
    bool last_weighted = false;    // the last training forward had per-position weights
    bool has_default = false;      // some column has a default row: the forward adds one
                                   // sort entry per bag after the N positions
    int64_t last_n = -1;           // positions of the last training forward (read by the backward)
    bool seg_from_keys = false;    // the last dedup skipped the unique list (see emb_backward_dedup)
    emb::DevCol *dcols = nullptr;  // device copy of the column metadata
    uint32_t *drow_base = nullptr; // device [n_cols + 1] row bases (after dcols)
    uint32_t *hrow_base = nullptr; // host copy
    emb::DevCol *hcols = nullptr;  // host copy
    emb::WsLayout ws{};
};

struct emb_table {
    int64_t capacity = 0, row_capacity = 0;
    int32_t dim = 0, threshold = 0;
    float init_a = 0.f;            // fp32(init_std * sqrt(3)); 0 = zero rows
    int64_t *slot_keys = nullptr;  // [capacity], 0 = empty
    int32_t *slot_count = nullptr; // [capacity]
    int32_t *slot_seen = nullptr;  // [capacity], table step that last saw the key
    int32_t *slot_row = nullptr;   // [capacity], -1 = not admitted
    float *pool = nullptr;         // [row_capacity, dim]
    int32_t *next_row = nullptr;   // device counters: [0] rows taken from the pool's end,
                                   // [1] rows on the free list, [2] live keys, [3] evicted
    int32_t *free_rows = nullptr;  // [row_capacity], rows freed by eviction (a stack)
    int64_t *tmp_keys = nullptr;   // [capacity] eviction: the live slots, compacted
    int32_t *tmp_count = nullptr, *tmp_row = nullptr, *tmp_seen = nullptr;
    int64_t step = 0;              // lookups so far: the step the next lookup records
    bool track_seen = false;       // lookups record last-seen steps
    int32_t *sketch = nullptr;     // count-min admission counters [cm_depth][cm_width], or NULL
    int32_t cm_depth = 0;
    int64_t cm_width = 0;
    size_t bytes = 0;
};

namespace emb {
// Split-bag partials and tickets of an inference forward held outside a workspace
struct FwdScratch {
    const char *zrow;    // kZeroRow bytes that hold zero
    float *part;
    int32_t *pcnt;
    uint32_t *tick;
    int32_t *fstat;
    int64_t tiles;
};
constexpr size_t kZeroRow = 1024;   // the widest row a lane group reads: 256 fp32
// bytes an inference forward of n_ids positions needs for them; with layout, the
// regions placed from base (forward.hip)
size_t fwd_scratch_bytes(const emb_plan *plan, int64_t n_ids, FwdScratch *layout, void *base);
// Positions per forward tile for a batch of n_ids positions: the plan's fixed size,
// else kFwdTileMax when the batch's mean bag has kLongBag positions or more (bags
// are then cut by tiles; a longer tile cuts fewer) and the batch makes at least
// kLongTilesMin such tiles, else the plan's tile.
int32_t fwd_tile_for(const emb_plan *plan, int64_t n_ids);
emb_status forward_with_scratch(emb_plan *plan, const int32_t *offsets, const int64_t *ids,
                                const float *fvals, const int32_t *keyed_rows, int64_t n_ids,
                                float *out, int64_t *stats, void *stream, const FwdScratch &sc);
// host helpers (plan.cpp)
emb_status fail(emb_status s, const std::string &msg);
emb_status ok();
bool aligned(const void *p, size_t a);
emb_status plan_validate(const emb_column_desc *cols, int32_t n_cols, int32_t batch,
                         int64_t max_ids, const emb_plan_opts *opts);
void plan_layout(emb_plan &P);
}  // namespace emb
