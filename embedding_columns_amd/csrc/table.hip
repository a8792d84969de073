// table.hip -- collisionless int64-keyed embedding table with a frequency filter.
//
// Monolith (Sec. 2.1 "Hash Table") keeps every distinct ID in its own slot (no two
// IDs share an embedding) and admits an ID only once its occurrence count reaches
// a tunable threshold.  Here the table is GPU open addressing over a power-of-two
// slot array (buckets of 16 slots probed with a per-key odd stride from
// splitmix64(key), insertion by 64-bit compare-and-swap on the slot key) instead
// of Monolith's CPU cuckoo table; slot placement never shows in results.
//
// One lookup-or-insert step is three launches so that admission is decided on
// the whole batch's counts (every occurrence of a key in the step sees the same
// outcome, whatever the thread order):
//   ht_count    probe / insert every occurrence, count it in its slot
//   ht_admit    a slot whose count reached the threshold and has no row claims
//               one (CAS on the row field), takes a pool row and initializes it
//   ht_resolve  every occurrence reads its slot's row, or DEFAULT
//
// Lifecycle: each slot also keeps the table step that last saw its key; eviction
// (ht_evict_scan, ht_clear, ht_reinsert) frees the rows of keys unseen since a
// given step onto a free list and rebuilds the slot array from the live keys.
#include <algorithm>
#include <cmath>
#include <string>

#include "device.h"

namespace emb {

constexpr int32_t kSlotNoRow = -1;
constexpr int32_t kSlotClaim = -3;     // row being allocated by one thread
constexpr int32_t kPosRefused = -3;    // per-position code between the launches
constexpr int32_t kPosPending = -4;    // count-min: absent key, counted in the sketch

// Count-min cell of sketch row j for a key: output j of a SplitMix64 generator
// seeded with the key (splitmix64(key + j * gamma)), modulo the power-of-two width.
__device__ __forceinline__ uint64_t cm_cell(uint64_t key, int j, uint64_t wmask)
{
    return splitmix64(key + (uint64_t)j * 0x9E3779B97F4A7C15ull) & wmask;
}

// device counters (emb_table::next_row)
constexpr int kCtrBump = 0;    // rows taken from the unused end of the pool
constexpr int kCtrFree = 1;    // rows on the free list (below zero after failed pops: empty)
constexpr int kCtrLive = 2;    // eviction: live keys compacted so far
constexpr int kCtrEvicted = 3; // eviction: keys removed

struct TabArgs {
    unsigned long long *keys;   // slot keys (0 = empty)
    int32_t *count;
    int32_t *row;
    int32_t *seen;              // last-seen table step (written only when tracking)
    float *pool;
    int32_t *next_row;          // the counters above
    int32_t *free_rows;
    int64_t cap, row_cap;
    int32_t dim, threshold;
    float init_a;
    int32_t step;
    int32_t track;              // record last-seen steps in lookups (emb_table_track_seen)
    int32_t *sketch;            // count-min admission: [depth][width] counters, or NULL
    int32_t depth;
    uint64_t wmask;             // width - 1 (width a power of two)
};

static TabArgs tab_args(const emb_table &t)
{
    TabArgs a;
    a.keys = reinterpret_cast<unsigned long long *>(t.slot_keys);
    a.count = t.slot_count;
    a.seen = t.slot_seen;
    a.row = t.slot_row;
    a.pool = t.pool;
    a.next_row = t.next_row;
    a.free_rows = t.free_rows;
    a.step = (int32_t)t.step;
    a.track = t.track_seen ? 1 : 0;
    a.sketch = t.sketch;
    a.depth = t.cm_depth;
    a.wmask = (uint64_t)t.cm_width - 1;
    a.cap = t.capacity;
    a.row_cap = t.row_capacity;
    a.dim = t.dim;
    a.threshold = t.threshold;
    a.init_a = t.init_a;
    return a;
}

// probe for `key`, inserting it into the first empty slot on the way; returns
// the slot, or -1 if all capacity slots hold other keys.  `inserted` tells
// whether this thread placed the key.  Slot by slot (small tables).
__device__ __forceinline__ int64_t probe_insert_slots(const TabArgs &a, unsigned long long key,
                                                      bool &inserted, int64_t &probes)
{
    const uint64_t mask = (uint64_t)a.cap - 1;
    uint64_t h = splitmix64(key) & mask;
    inserted = false;
    for (int64_t i = 0; i < a.cap; i++) {
        unsigned long long k = __hip_atomic_load(&a.keys[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (k == 0ull) {
            k = atomicCAS(&a.keys[h], 0ull, key);
            if (k == 0ull) {
                inserted = true;
                probes = i + 1;
                return (int64_t)h;
            }
        }
        if (k == key) {
            probes = i + 1;
            return (int64_t)h;
        }
        h = (h + 1) & mask;
    }
    probes = a.cap;
    return -1;
}

// Tables of at least kBucketSlots slots probe whole buckets of 16 slots (128
// bytes of keys, read as eight 16-byte loads in flight): the home bucket
// b0 = splitmix64(key) mod nb, then b0 + i * step with an odd step taken from the
// hash's high bits, so every bucket is visited once in nb steps.  Linear probing
// from a home slot builds long runs of full slots at the 0.75-0.8 load of a
// prepopulated table, and the slowest probe of a step set its time; stepping
// over buckets by a per-key stride keeps every probe sequence short.  Within a
// bucket the first empty slot takes the key by compare-and-swap; plain loads may
// see a slot empty that another thread has just filled, and the CAS then returns
// the real key.  Keys never change once placed, so a key is never placed twice.
constexpr int kBucketSlots = 16;

__device__ __forceinline__ void bucket_start(const TabArgs &a, unsigned long long key, uint64_t &b,
                                             uint64_t &step, uint64_t &nbm)
{
    const uint64_t h = splitmix64(key);
    nbm = (uint64_t)a.cap / kBucketSlots - 1;
    b = h & nbm;
    step = ((h >> 32) & nbm) | 1u;
}

__device__ __forceinline__ void bucket_keys(const TabArgs &a, uint64_t b, unsigned long long (&kk)[kBucketSlots])
{
    const uint4 *q = reinterpret_cast<const uint4 *>(a.keys + b * kBucketSlots);
    uint4 v[kBucketSlots / 2];
#pragma unroll
    for (int j = 0; j < kBucketSlots / 2; j++) v[j] = *gp(q + j);
#pragma unroll
    for (int j = 0; j < kBucketSlots / 2; j++) {
        kk[2 * j] = ((unsigned long long)v[j].y << 32) | v[j].x;
        kk[2 * j + 1] = ((unsigned long long)v[j].w << 32) | v[j].z;
    }
}

__device__ __forceinline__ int64_t probe_insert(const TabArgs &a, unsigned long long key,
                                                bool &inserted, int64_t &probes)
{
    if (a.cap < kBucketSlots) return probe_insert_slots(a, key, inserted, probes);
    uint64_t b, step, nbm;
    bucket_start(a, key, b, step, nbm);
    inserted = false;
    for (uint64_t i = 0; i <= nbm; i++) {
        unsigned long long kk[kBucketSlots];
        bucket_keys(a, b, kk);
#pragma unroll
        for (int j = 0; j < kBucketSlots; j++) {
            const uint64_t s = b * kBucketSlots + j;
            unsigned long long k = kk[j];
            if (k == 0ull) {
                k = atomicCAS(&a.keys[s], 0ull, key);
                if (k == 0ull) {
                    inserted = true;
                    probes = (int64_t)(i * kBucketSlots + j + 1);
                    return (int64_t)s;
                }
            }
            if (k == key) {
                probes = (int64_t)(i * kBucketSlots + j + 1);
                return (int64_t)s;
            }
        }
        b = (b + step) & nbm;
    }
    probes = a.cap;
    return -1;
}

// read-only probe: slot of key, or -1 (the same sequence; the first empty slot
// ends it)
__device__ __forceinline__ int64_t probe_find(const TabArgs &a, unsigned long long key)
{
    if (a.cap < kBucketSlots) {
        const uint64_t mask = (uint64_t)a.cap - 1;
        uint64_t h = splitmix64(key) & mask;
        for (int64_t i = 0; i < a.cap; i++) {
            const unsigned long long k = __hip_atomic_load(&a.keys[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (k == key) return (int64_t)h;
            if (k == 0ull) return -1;
            h = (h + 1) & mask;
        }
        return -1;
    }
    uint64_t b, step, nbm;
    bucket_start(a, key, b, step, nbm);
    for (uint64_t i = 0; i <= nbm; i++) {
        unsigned long long kk[kBucketSlots];
        bucket_keys(a, b, kk);
#pragma unroll
        for (int j = 0; j < kBucketSlots; j++) {
            if (kk[j] == key) return (int64_t)(b * kBucketSlots + j);
            if (kk[j] == 0ull) return -1;
        }
        b = (b + step) & nbm;
    }
    return -1;
}

// initial value of element d of a new row: a * (2u - 1), u = top 24 bits of
// splitmix64(splitmix64(key) + d) / 2^24 -- exact up to the one final rounding
__device__ __forceinline__ void init_row(const TabArgs &a, int64_t r, unsigned long long key)
{
    float *dst = a.pool + r * a.dim;
    const uint64_t h = splitmix64(key);
    for (int d = 0; d < a.dim; d += 4) {
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint64_t z = splitmix64(h + (uint64_t)(d + j));
            const float u = __fmul_rn((float)(uint32_t)(z >> 40), 0x1p-24f);
            const float s = __fsub_rn(__fmul_rn(2.0f, u), 1.0f);
            v[j] = __fmul_rn(a.init_a, s);
        }
        *reinterpret_cast<float4 *>(dst + d) = make_float4(v[0], v[1], v[2], v[3]);
    }
}

// A row for a newly admitted key: one from the free list if any, else the next
// unused one; -1 if the pool is exhausted.  Pops happen only in admission
// kernels and pushes only in eviction, which never overlap: the first F pops of
// a launch (F = the list's size) get distinct entries, later ones see an empty
// list.  The load before the decrement keeps the counter from drifting far
// below zero; eviction clamps it back to zero before pushing.
__device__ __forceinline__ int32_t alloc_row(const TabArgs &a)
{
    if (__hip_atomic_load(&a.next_row[kCtrFree], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) > 0) {
        const int32_t f = atomicSub(&a.next_row[kCtrFree], 1) - 1;
        if (f >= 0) return __hip_atomic_load(&a.free_rows[f], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const int32_t r = atomicAdd(&a.next_row[kCtrBump], 1);
    return (int64_t)r < a.row_cap ? r : -1;
}

__device__ __forceinline__ void stat_add(int64_t *stats, int idx, int64_t v)
{
    const uint32_t s = wave_sum_u32((uint32_t)v);     // v is a 0 / 1 flag
    if (stats && lane_id() == 0 && s) atomicAdd((unsigned long long *)&stats[idx], (unsigned long long)s);
}

__device__ __forceinline__ void stat_max(int64_t *stats, int idx, int64_t v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, (int64_t)__shfl_xor(v, o, 64));
    if (stats && lane_id() == 0 && v) atomicMax((unsigned long long *)&stats[idx], (unsigned long long)v);
}

// Counting under a skewed key stream: one block takes 512 occurrences, adds them
// up per slot in an LDS hash (each hot key is counted once per block instead
// of once per occurrence), then adds each distinct slot's count to the table.
// 512 occurrences per block put every block of a 819,200-key step on the chip
// at once (1024: two rounds, lookup 122 us against 118; 256: more count
// updates on the hottest slots, 120 us).
constexpr int kCountTile = 512;                // occurrences per block, one per thread
constexpr int kLdsSlots = 2 * kCountTile;      // load factor <= 1/2: every insert finds room
constexpr int kLdsSlotBits = 10;
static_assert((1 << kLdsSlotBits) == kLdsSlots, "LDS hash size");

// CM: count-min admission (absent keys go to the sketch), a separate instance so
// that exact counting carries none of its code
template <bool CM>
__global__ __launch_bounds__(kCountTile) void ht_count(TabArgs a, const int64_t *__restrict__ keys,
                                                      int64_t n, int32_t *__restrict__ pos,
                                                      int64_t *stats)
{
    __shared__ int32_t lslot[kLdsSlots];
    __shared__ int32_t lcnt[kLdsSlots];
    __shared__ unsigned long long lstat[3];
    for (int i = threadIdx.x; i < kLdsSlots; i += kCountTile) {
        lslot[i] = -1;
        lcnt[i] = 0;
    }
    if (threadIdx.x < 3) lstat[threadIdx.x] = 0;
    __syncthreads();
    const int64_t p = (int64_t)blockIdx.x * kCountTile + threadIdx.x;
    int64_t ins = 0, full = 0, probes = 0;
    const int64_t key = p < n ? *gp(keys + p) : 0;
    if (p < n && key < 1) *gp(pos + p) = EMB_ROW_DROPPED;
    if (key >= 1) {
        bool inserted = false;
        int64_t s;
        if (CM) {
            // count-min admission: a key in the table counts in its slot; an absent
            // one adds to its sketch cells and waits for cm_enter
            s = probe_find(a, (unsigned long long)key);
            if (s < 0) {
                *gp(pos + p) = kPosPending;
                for (int j = 0; j < a.depth; j++)
                    atomicAdd(&a.sketch[(int64_t)j * (int64_t)(a.wmask + 1) +
                                        (int64_t)cm_cell((uint64_t)key, j, a.wmask)], 1);
            }
        } else {
            s = probe_insert(a, (unsigned long long)key, inserted, probes);
            if (s < 0) {
                *gp(pos + p) = kPosRefused;
                full = 1;
            }
        }
        if (s >= 0) {
            *gp(pos + p) = (int32_t)s;
            ins = inserted;
            // count this occurrence in the block's LDS hash
            uint32_t h = ((uint32_t)s * 2654435761u) >> (32 - kLdsSlotBits);
            while (true) {
                const int32_t cur = atomicCAS(&lslot[h], -1, (int32_t)s);
                if (cur == -1 || cur == (int32_t)s) break;
                h = (h + 1) & (kLdsSlots - 1);
            }
            atomicAdd(&lcnt[h], 1);
        }
    }
    if (stats) {
        // one LDS update per wavefront
        const uint32_t si = wave_sum_u32((uint32_t)ins), sf = wave_sum_u32((uint32_t)full);
        int64_t mp = probes;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) mp = max(mp, (int64_t)__shfl_xor(mp, o, 64));
        if (lane_id() == 0) {
            if (si) atomicAdd(&lstat[0], (unsigned long long)si);
            if (sf) atomicAdd(&lstat[1], (unsigned long long)sf);
            if (mp) atomicMax(&lstat[2], (unsigned long long)mp);
        }
    }
    __syncthreads();
    // each distinct slot once per block: its count, and (when tracking) this step as
    // its last-seen step (every block stores the same value)
    for (int i = threadIdx.x; i < kLdsSlots; i += kCountTile) {
        if (lslot[i] >= 0) {
            atomicAdd(&a.count[lslot[i]], lcnt[i]);
            if (a.track) a.seen[lslot[i]] = a.step;
        }
    }
    if (stats && threadIdx.x == 0) {
        if (lstat[0]) atomicAdd((unsigned long long *)&stats[EMB_STAT_TABLE_INSERTED], lstat[0]);
        if (lstat[1]) atomicAdd((unsigned long long *)&stats[EMB_STAT_TABLE_FULL], lstat[1]);
        if (lstat[2]) atomicMax((unsigned long long *)&stats[EMB_STAT_MAX_PROBE], lstat[2]);
    }
}

// count-min admission, after every occurrence of the step reached the sketch: an
// absent key whose estimate (the least of its cells) reached the threshold enters
// the table with that count; ht_admit then gives it a row.  All occurrences of a
// key compute the same estimate; the one whose insert lands sets the count.
__global__ __launch_bounds__(kBlock) void cm_enter(TabArgs a, const int64_t *__restrict__ keys,
                                                  int64_t n, int32_t *__restrict__ pos,
                                                  int64_t *stats)
{
    const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    int64_t ins = 0, full = 0, probes = 0;
    if (p < n && pos[p] == kPosPending) {
        const uint64_t key = (uint64_t)keys[p];
        int32_t est = INT32_MAX;
        for (int j = 0; j < a.depth; j++)
            est = min(est, a.sketch[(int64_t)j * (int64_t)(a.wmask + 1) + (int64_t)cm_cell(key, j, a.wmask)]);
        if (est >= a.threshold) {
            bool inserted;
            const int64_t s = probe_insert(a, (unsigned long long)key, inserted, probes);
            if (s < 0) {
                full = 1;                      // stays pending: reads DEFAULT
            } else {
                if (inserted) {
                    a.count[s] = est;
                    if (a.track) a.seen[s] = a.step;
                    ins = 1;
                }
                pos[p] = (int32_t)s;
            }
        }
    }
    stat_add(stats, EMB_STAT_TABLE_INSERTED, ins);
    stat_add(stats, EMB_STAT_TABLE_FULL, full);
    stat_max(stats, EMB_STAT_MAX_PROBE, probes);
}

__global__ __launch_bounds__(kBlock) void ht_admit(TabArgs a, const int64_t *__restrict__ keys,
                                                  int64_t n, const int32_t *__restrict__ pos,
                                                  int64_t *stats)
{
    const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    int64_t adm = 0, full = 0;
    if (p < n) {
        const int32_t s = pos[p];
        if (s >= 0 && __hip_atomic_load(&a.row[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == kSlotNoRow &&
            a.count[s] >= a.threshold) {
            if (atomicCAS(&a.row[s], kSlotNoRow, kSlotClaim) == kSlotNoRow) {
                const int32_t r = alloc_row(a);
                if (r >= 0) {
                    init_row(a, r, (unsigned long long)keys[p]);
                    atomicExch(&a.row[s], r);
                    adm = 1;
                } else {
                    atomicExch(&a.row[s], kSlotNoRow);   // row pool full: stays not admitted
                    full = 1;
                }
            }
        }
    }
    stat_add(stats, EMB_STAT_TABLE_ADMITTED, adm);
    stat_add(stats, EMB_STAT_TABLE_FULL, full);
}

__global__ __launch_bounds__(kBlock) void ht_resolve(TabArgs a, int64_t n, int32_t *__restrict__ pos)
{
    const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (p >= n) return;
    const int32_t s = pos[p];
    if (s == EMB_ROW_DROPPED) return;
    if (s < 0) {
        pos[p] = EMB_ROW_DEFAULT;
        return;
    }
    const int32_t r = a.row[s];
    pos[p] = r >= 0 ? r : EMB_ROW_DEFAULT;
}

__global__ __launch_bounds__(kBlock) void ht_bulk(TabArgs a, const int64_t *__restrict__ keys,
                                                 const float *__restrict__ rows, int64_t n,
                                                 int64_t *stats)
{
    const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    int64_t ins = 0, adm = 0, full = 0, probes = 0;
    if (p < n) {
        const int64_t key = keys[p];
        if (key >= 1) {
            bool inserted;
            const int64_t s = probe_insert(a, (unsigned long long)key, inserted, probes);
            if (s < 0) {
                full = 1;
            } else if (inserted) {
                ins = 1;
                a.seen[s] = a.step;
                const int32_t r = alloc_row(a);
                if (r >= 0) {
                    adm = 1;
                    if (rows) {
                        const float4 *src = reinterpret_cast<const float4 *>(rows + p * a.dim);
                        float4 *dst = reinterpret_cast<float4 *>(a.pool + (int64_t)r * a.dim);
                        for (int d = 0; d < a.dim / 4; d++) dst[d] = src[d];
                    } else {
                        init_row(a, r, (unsigned long long)key);
                    }
                    a.row[s] = r;
                } else {
                    full = 1;
                }
            }
        }
    }
    stat_add(stats, EMB_STAT_TABLE_INSERTED, ins);
    stat_add(stats, EMB_STAT_TABLE_ADMITTED, adm);
    stat_add(stats, EMB_STAT_TABLE_FULL, full);
    stat_max(stats, EMB_STAT_MAX_PROBE, probes);
}

__global__ __launch_bounds__(kBlock) void ht_find(TabArgs a, const int64_t *__restrict__ keys,
                                                 int64_t n, int32_t *__restrict__ rows_out,
                                                 int32_t *__restrict__ counts_out)
{
    const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (p >= n) return;
    const int64_t key = keys[p];
    const int64_t s = key >= 1 ? probe_find(a, (unsigned long long)key) : -1;
    if (s < 0) {
        rows_out[p] = EMB_ROW_DROPPED;
        if (counts_out) counts_out[p] = 0;
        return;
    }
    const int32_t r = a.row[s];
    rows_out[p] = r >= 0 ? r : EMB_ROW_DEFAULT;
    if (counts_out) counts_out[p] = a.count[s];
}

__global__ __launch_bounds__(kBlock) void ht_export(TabArgs a, int64_t *__restrict__ keys,
                                                   int32_t *__restrict__ counts,
                                                   int32_t *__restrict__ rows,
                                                   unsigned long long *n_out)
{
    const int64_t s = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const bool occ = s < a.cap && a.keys[s] != 0ull;
    const uint64_t m = __ballot(occ);
    if (!m) return;
    unsigned long long base = 0;
    const int lane = lane_id();
    const int leader = __ffsll((long long)m) - 1;
    if (lane == leader) base = atomicAdd(n_out, (unsigned long long)__popcll(m));
    base = __shfl(base, leader, kWave);
    if (occ) {
        const uint64_t below = m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane)));
        const int64_t i = (int64_t)base + __popcll(below);
        keys[i] = (int64_t)a.keys[s];
        counts[i] = a.count[s];
        rows[i] = a.row[s];
    }
}

// ---------------------------------------------------------------- lifecycle

__global__ void ht_evict_prep(TabArgs a)
{
    if (threadIdx.x == 0) {
        a.next_row[kCtrFree] = max(a.next_row[kCtrFree], 0);
        a.next_row[kCtrLive] = 0;
        a.next_row[kCtrEvicted] = 0;
    }
}

// one slot per thread: an expired key's row goes to the free list, a live key is
// appended (with its count, row and step) to the compaction buffers
__global__ __launch_bounds__(kBlock) void ht_evict_scan(TabArgs a, int32_t min_seen,
                                                       float *__restrict__ opt_state,
                                                       int64_t *__restrict__ tkeys,
                                                       int32_t *__restrict__ tcount,
                                                       int32_t *__restrict__ trow,
                                                       int32_t *__restrict__ tseen)
{
    const int64_t s = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const unsigned long long key = s < a.cap ? a.keys[s] : 0ull;
    const bool occ = key != 0ull;
    const bool live = occ && a.seen[s] >= min_seen;
    if (occ && !live) {
        const int32_t r = a.row[s];
        if (r >= 0) {
            const int32_t i = atomicAdd(&a.next_row[kCtrFree], 1);
            a.free_rows[i] = r;
            if (opt_state) {         // the next key to get this row starts from zero state
                float4 *z = reinterpret_cast<float4 *>(opt_state + (int64_t)r * a.dim);
                for (int d = 0; d < a.dim / 4; d++) z[d] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    }
    const uint64_t m = __ballot(live);
    const int lane = lane_id();
    const uint32_t ev = wave_sum_u32(occ && !live ? 1u : 0u);
    if (lane == 0 && ev) atomicAdd(&a.next_row[kCtrEvicted], (int32_t)ev);
    if (!m) return;
    const int leader = __ffsll((long long)m) - 1;
    int32_t base = 0;
    if (lane == leader) base = atomicAdd(&a.next_row[kCtrLive], __popcll(m));
    base = __shfl(base, leader, kWave);
    if (live) {
        const int32_t i = base + __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
        tkeys[i] = (int64_t)key;
        tcount[i] = a.count[s];
        trow[i] = a.row[s];
        tseen[i] = a.seen[s];
    }
}

__global__ __launch_bounds__(kBlock) void ht_clear(TabArgs a)
{
    const int64_t s = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (s >= a.cap) return;
    a.keys[s] = 0ull;
    a.count[s] = 0;
    a.row[s] = kSlotNoRow;
    a.seen[s] = 0;
}

// the live keys back into the cleared slots (all distinct, at most cap of them,
// so every insert finds a slot)
__global__ __launch_bounds__(kBlock) void ht_reinsert(TabArgs a, const int64_t *__restrict__ tkeys,
                                                     const int32_t *__restrict__ tcount,
                                                     const int32_t *__restrict__ trow,
                                                     const int32_t *__restrict__ tseen,
                                                     int64_t *n_live, int64_t *stats)
{
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int32_t live = a.next_row[kCtrLive];
    if (i == 0) {
        if (n_live) *n_live = live;
        if (stats && a.next_row[kCtrEvicted])
            atomicAdd((unsigned long long *)&stats[EMB_STAT_TABLE_EVICTED],
                      (unsigned long long)a.next_row[kCtrEvicted]);
    }
    if (i >= live) return;
    bool inserted;
    int64_t probes;
    const int64_t s = probe_insert(a, (unsigned long long)tkeys[i], inserted, probes);
    if (s < 0) return;                  // cannot happen: live <= cap distinct keys
    a.count[s] = tcount[i];
    a.row[s] = trow[i];
    a.seen[s] = tseen[i];
}

// checkpoint: every occupied slot with its row values
__global__ __launch_bounds__(kBlock) void ht_save(TabArgs a, int64_t *__restrict__ keys,
                                                 int32_t *__restrict__ counts,
                                                 int32_t *__restrict__ seen,
                                                 uint8_t *__restrict__ admitted,
                                                 float *__restrict__ values,
                                                 unsigned long long *n_out)
{
    const int64_t s = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const bool occ = s < a.cap && a.keys[s] != 0ull;
    const uint64_t m = __ballot(occ);
    if (!m) return;
    unsigned long long base = 0;
    const int lane = lane_id();
    const int leader = __ffsll((long long)m) - 1;
    if (lane == leader) base = atomicAdd(n_out, (unsigned long long)__popcll(m));
    base = __shfl(base, leader, kWave);
    if (occ) {
        const uint64_t below = m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane)));
        const int64_t i = (int64_t)base + __popcll(below);
        const int32_t r = a.row[s];
        keys[i] = (int64_t)a.keys[s];
        counts[i] = a.count[s];
        seen[i] = a.seen[s];
        admitted[i] = r >= 0;
        float4 *dst = reinterpret_cast<float4 *>(values + i * a.dim);
        const float4 *src = reinterpret_cast<const float4 *>(a.pool + (int64_t)max(r, 0) * a.dim);
        for (int d = 0; d < a.dim / 4; d++) dst[d] = r >= 0 ? src[d] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

__global__ __launch_bounds__(kBlock) void ht_load(TabArgs a, const int64_t *__restrict__ keys,
                                                 const int32_t *__restrict__ counts,
                                                 const int32_t *__restrict__ seen,
                                                 const uint8_t *__restrict__ admitted,
                                                 const float *__restrict__ values, int64_t n,
                                                 int64_t *stats)
{
    const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    int64_t ins = 0, adm = 0, full = 0, probes = 0;
    if (p < n && keys[p] >= 1) {
        bool inserted;
        const int64_t s = probe_insert(a, (unsigned long long)keys[p], inserted, probes);
        if (s < 0) {
            full = 1;
        } else if (inserted) {
            ins = 1;
            a.count[s] = counts[p];
            a.seen[s] = seen[p];
            if (admitted[p]) {
                const int32_t r = alloc_row(a);
                if (r >= 0) {
                    const float4 *src = reinterpret_cast<const float4 *>(values + p * a.dim);
                    float4 *dst = reinterpret_cast<float4 *>(a.pool + (int64_t)r * a.dim);
                    for (int d = 0; d < a.dim / 4; d++) dst[d] = src[d];
                    a.row[s] = r;
                    adm = 1;
                } else {
                    full = 1;
                }
            }
        }
    }
    stat_add(stats, EMB_STAT_TABLE_INSERTED, ins);
    stat_add(stats, EMB_STAT_TABLE_ADMITTED, adm);
    stat_add(stats, EMB_STAT_TABLE_FULL, full);
    stat_max(stats, EMB_STAT_MAX_PROBE, probes);
}

}  // namespace emb

using namespace emb;

static size_t a256(size_t x) { return (x + 255) & ~size_t(255); }

// device memory: slot keys, counts, rows, last-seen steps; the counters; the
// free list; the eviction's compaction buffers; the row pool
enum { kOffKeys, kOffCount, kOffSeen, kOffRow, kOffCtr, kOffFree, kOffTmpKeys, kOffTmpCount,
       kOffTmpRow, kOffTmpSeen, kOffPool, kNumOff };

static emb_status table_sizes(int64_t capacity, int64_t row_capacity, int32_t dim, size_t off[kNumOff])
{
    if (capacity < 2 || capacity > (int64_t(1) << 30) || (capacity & (capacity - 1)))
        return fail(EMB_ERR_INVALID_ARG, "capacity must be a power of two in [2, 2^30]");
    if (row_capacity < 1 || row_capacity > (int64_t(1) << 31) - 1)
        return fail(EMB_ERR_INVALID_ARG, "row_capacity must be in [1, 2^31-1]");
    if (dim <= 0 || dim % 4 || dim > kMaxDimF32)
        return fail(EMB_ERR_UNSUPPORTED, "table dim must be a multiple of 4 and <= 256");
    const size_t cap = (size_t)capacity;
    size_t o = 0;
    off[kOffKeys] = o; o = a256(o + 8 * cap);
    off[kOffCount] = o; o = a256(o + 4 * cap);
    off[kOffSeen] = o; o = a256(o + 4 * cap);
    off[kOffRow] = o; o = a256(o + 4 * cap);
    off[kOffCtr] = o; o = a256(o + 256);
    off[kOffFree] = o; o = a256(o + 4 * (size_t)row_capacity);
    off[kOffTmpKeys] = o; o = a256(o + 8 * cap);
    off[kOffTmpCount] = o; o = a256(o + 4 * cap);
    off[kOffTmpRow] = o; o = a256(o + 4 * cap);
    off[kOffTmpSeen] = o; o = a256(o + 4 * cap);
    off[kOffPool] = o;                                  // row pool [row_capacity, dim]
    return EMB_OK;
}

extern "C" {

emb_status emb_table_query(int64_t capacity, int64_t row_capacity, int32_t dim, size_t *table_bytes)
{
    if (!table_bytes) return fail(EMB_ERR_INVALID_ARG, "table_bytes is NULL");
    size_t off[kNumOff];
    emb_status s = table_sizes(capacity, row_capacity, dim, off);
    if (s != EMB_OK) return s;
    *table_bytes = off[kOffPool] + a256(4 * (size_t)row_capacity * (size_t)dim);
    return EMB_OK;
}

emb_status emb_table_create(int64_t capacity, int64_t row_capacity, int32_t dim, int32_t threshold,
                            float init_std, void *table_mem, void *stream, emb_table **out)
{
    if (!out) return fail(EMB_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    size_t off[kNumOff];
    emb_status s = table_sizes(capacity, row_capacity, dim, off);
    if (s != EMB_OK) return s;
    if (!table_mem || !aligned(table_mem, 256)) return fail(EMB_ERR_INVALID_ARG, "table_mem must be 256-byte aligned device memory");
    if (threshold < 1) return fail(EMB_ERR_INVALID_ARG, "threshold must be >= 1");
    if (!(init_std >= 0.f) || !std::isfinite(init_std)) return fail(EMB_ERR_INVALID_ARG, "init_std must be finite and >= 0");
    emb_table *T = new (std::nothrow) emb_table();
    if (!T) return fail(EMB_ERR_INVALID_ARG, "out of host memory");
    char *m = static_cast<char *>(table_mem);
    T->capacity = capacity;
    T->row_capacity = row_capacity;
    T->dim = dim;
    T->threshold = threshold;
    T->init_a = (float)((double)init_std * std::sqrt(3.0));
    T->slot_keys = reinterpret_cast<int64_t *>(m + off[kOffKeys]);
    T->slot_count = reinterpret_cast<int32_t *>(m + off[kOffCount]);
    T->slot_seen = reinterpret_cast<int32_t *>(m + off[kOffSeen]);
    T->slot_row = reinterpret_cast<int32_t *>(m + off[kOffRow]);
    T->next_row = reinterpret_cast<int32_t *>(m + off[kOffCtr]);
    T->free_rows = reinterpret_cast<int32_t *>(m + off[kOffFree]);
    T->tmp_keys = reinterpret_cast<int64_t *>(m + off[kOffTmpKeys]);
    T->tmp_count = reinterpret_cast<int32_t *>(m + off[kOffTmpCount]);
    T->tmp_row = reinterpret_cast<int32_t *>(m + off[kOffTmpRow]);
    T->tmp_seen = reinterpret_cast<int32_t *>(m + off[kOffTmpSeen]);
    T->pool = reinterpret_cast<float *>(m + off[kOffPool]);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemsetAsync(m, 0, off[kOffRow], st);                 // keys, counts, steps
    if (e == hipSuccess) e = hipMemsetAsync(T->slot_row, 0xFF, 4 * (size_t)capacity, st);   // rows = -1
    if (e == hipSuccess) e = hipMemsetAsync(T->next_row, 0, 256, st);
    if (e != hipSuccess) {
        delete T;
        return fail(EMB_ERR_HIP, std::string("table clear: ") + hipGetErrorString(e));
    }
    *out = T;
    return EMB_OK;
}

emb_status emb_table_destroy(emb_table *table)
{
    delete table;
    return EMB_OK;
}

float *emb_table_rows(emb_table *table) { return table ? table->pool : nullptr; }

static unsigned grid_of(int64_t n) { return (unsigned)std::max<int64_t>(1, (n + kBlock - 1) / kBlock); }

static emb_status launched(const char *what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(EMB_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
    return EMB_OK;
}

emb_status emb_table_bulk_insert(emb_table *table, const int64_t *keys, const float *rows, int64_t n,
                                 int64_t *stats, void *stream)
{
    if (!table || n < 0 || (n > 0 && !keys)) return fail(EMB_ERR_INVALID_ARG, "bad bulk insert arguments");
    if (rows && !aligned(rows, 16)) return fail(EMB_ERR_INVALID_ARG, "rows must be 16-byte aligned");
    if (n == 0) return EMB_OK;
    hipLaunchKernelGGL(ht_bulk, dim3(grid_of(n)), dim3(kBlock), 0, static_cast<hipStream_t>(stream),
                       tab_args(*table), keys, rows, n, stats);
    return launched("ht_bulk");
}

emb_status emb_table_lookup_or_insert(emb_table *table, const int64_t *keys, int64_t n,
                                      int32_t *rows_out, int64_t *stats, void *stream)
{
    if (!table || n < 0 || (n > 0 && (!keys || !rows_out)))
        return fail(EMB_ERR_INVALID_ARG, "bad lookup_or_insert arguments");
    if (n >= (int64_t(1) << 31)) return fail(EMB_ERR_UNSUPPORTED, "at most 2^31-1 keys per call");
    if (n == 0) return EMB_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const TabArgs a = tab_args(*table);
    const unsigned cgrid = (unsigned)std::max<int64_t>(1, (n + kCountTile - 1) / kCountTile);
    if (a.sketch) {
        hipLaunchKernelGGL(ht_count<true>, dim3(cgrid), dim3(kCountTile), 0, st, a, keys, n, rows_out, stats);
        hipLaunchKernelGGL(cm_enter, dim3(grid_of(n)), dim3(kBlock), 0, st, a, keys, n, rows_out, stats);
    } else {
        hipLaunchKernelGGL(ht_count<false>, dim3(cgrid), dim3(kCountTile), 0, st, a, keys, n, rows_out, stats);
    }
    hipLaunchKernelGGL(ht_admit, dim3(grid_of(n)), dim3(kBlock), 0, st, a, keys, n, rows_out, stats);
    hipLaunchKernelGGL(ht_resolve, dim3(grid_of(n)), dim3(kBlock), 0, st, a, n, rows_out);
    table->step++;
    return launched("lookup_or_insert");
}

emb_status emb_table_find(emb_table *table, const int64_t *keys, int64_t n, int32_t *rows_out,
                          int32_t *counts_out, void *stream)
{
    if (!table || n < 0 || (n > 0 && (!keys || !rows_out))) return fail(EMB_ERR_INVALID_ARG, "bad find arguments");
    if (n == 0) return EMB_OK;
    hipLaunchKernelGGL(ht_find, dim3(grid_of(n)), dim3(kBlock), 0, static_cast<hipStream_t>(stream),
                       tab_args(*table), keys, n, rows_out, counts_out);
    return launched("ht_find");
}

emb_status emb_table_export(emb_table *table, int64_t *keys, int32_t *counts, int32_t *rows,
                            int64_t *n_out, void *stream)
{
    if (!table || !keys || !counts || !rows || !n_out) return fail(EMB_ERR_INVALID_ARG, "bad export arguments");
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemsetAsync(n_out, 0, sizeof(int64_t), st);
    if (e != hipSuccess) return fail(EMB_ERR_HIP, std::string("export clear: ") + hipGetErrorString(e));
    hipLaunchKernelGGL(ht_export, dim3(grid_of(table->capacity)), dim3(kBlock), 0, st, tab_args(*table),
                       keys, counts, rows, reinterpret_cast<unsigned long long *>(n_out));
    return launched("ht_export");
}

int64_t emb_table_step(const emb_table *table) { return table ? table->step : -1; }

emb_status emb_table_use_count_min(emb_table *table, int32_t depth, int64_t width, int32_t *sketch)
{
    if (!table) return fail(EMB_ERR_INVALID_ARG, "table is NULL");
    if (!sketch) {
        table->sketch = nullptr;
        return EMB_OK;
    }
    if (depth < 1 || depth > 8) return fail(EMB_ERR_INVALID_ARG, "count-min depth must be in [1, 8]");
    if (width < 2 || width > (int64_t(1) << 30) || (width & (width - 1)))
        return fail(EMB_ERR_INVALID_ARG, "count-min width must be a power of two in [2, 2^30]");
    if (!aligned(sketch, 4)) return fail(EMB_ERR_INVALID_ARG, "sketch must be 4-byte aligned");
    table->sketch = sketch;
    table->cm_depth = depth;
    table->cm_width = width;
    return EMB_OK;
}

emb_status emb_table_track_seen(emb_table *table, int32_t on)
{
    if (!table) return fail(EMB_ERR_INVALID_ARG, "table is NULL");
    table->track_seen = on != 0;
    return EMB_OK;
}

emb_status emb_table_set_step(emb_table *table, int64_t step)
{
    if (!table || step < 0 || step > INT32_MAX) return fail(EMB_ERR_INVALID_ARG, "bad table step");
    table->step = step;
    return EMB_OK;
}

emb_status emb_table_evict(emb_table *table, int64_t min_seen, float *opt_state, int64_t *n_live,
                           int64_t *stats, void *stream)
{
    if (!table) return fail(EMB_ERR_INVALID_ARG, "table is NULL");
    if (opt_state && !aligned(opt_state, 16)) return fail(EMB_ERR_INVALID_ARG, "opt_state must be 16-byte aligned");
    const int32_t ms = (int32_t)std::min<int64_t>(std::max<int64_t>(min_seen, INT32_MIN), INT32_MAX);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const TabArgs a = tab_args(*table);
    const unsigned g = grid_of(table->capacity);
    hipLaunchKernelGGL(ht_evict_prep, dim3(1), dim3(kWave), 0, st, a);
    hipLaunchKernelGGL(ht_evict_scan, dim3(g), dim3(kBlock), 0, st, a, ms, opt_state, table->tmp_keys,
                       table->tmp_count, table->tmp_row, table->tmp_seen);
    hipLaunchKernelGGL(ht_clear, dim3(g), dim3(kBlock), 0, st, a);
    hipLaunchKernelGGL(ht_reinsert, dim3(g), dim3(kBlock), 0, st, a, table->tmp_keys,
                       table->tmp_count, table->tmp_row, table->tmp_seen, n_live, stats);
    return launched("emb_table_evict");
}

emb_status emb_table_save(emb_table *table, int64_t *keys, int32_t *counts, int32_t *seen,
                          uint8_t *admitted, float *values, int64_t *n_out, void *stream)
{
    if (!table || !keys || !counts || !seen || !admitted || !values || !n_out)
        return fail(EMB_ERR_INVALID_ARG, "bad save arguments");
    if (!aligned(values, 16)) return fail(EMB_ERR_INVALID_ARG, "values must be 16-byte aligned");
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemsetAsync(n_out, 0, sizeof(int64_t), st);
    if (e != hipSuccess) return fail(EMB_ERR_HIP, std::string("save clear: ") + hipGetErrorString(e));
    hipLaunchKernelGGL(ht_save, dim3(grid_of(table->capacity)), dim3(kBlock), 0, st, tab_args(*table),
                       keys, counts, seen, admitted, values, reinterpret_cast<unsigned long long *>(n_out));
    return launched("ht_save");
}

emb_status emb_table_load(emb_table *table, const int64_t *keys, const int32_t *counts,
                          const int32_t *seen, const uint8_t *admitted, const float *values,
                          int64_t n, int64_t *stats, void *stream)
{
    if (!table || n < 0 || (n > 0 && (!keys || !counts || !seen || !admitted || !values)))
        return fail(EMB_ERR_INVALID_ARG, "bad load arguments");
    if (values && !aligned(values, 16)) return fail(EMB_ERR_INVALID_ARG, "values must be 16-byte aligned");
    if (n == 0) return EMB_OK;
    hipLaunchKernelGGL(ht_load, dim3(grid_of(n)), dim3(kBlock), 0, static_cast<hipStream_t>(stream),
                       tab_args(*table), keys, counts, seen, admitted, values, n, stats);
    return launched("ht_load");
}

}  // extern "C"
