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
#include <algorithm>
#include <cmath>
#include <string>

#include "device.h"

namespace emb {

constexpr int32_t kSlotNoRow = -1;
constexpr int32_t kSlotClaim = -3;     // row being allocated by one thread
constexpr int32_t kPosRefused = -3;    // per-position code between the launches

struct TabArgs {
    unsigned long long *keys;   // slot keys (0 = empty)
    int32_t *count;
    int32_t *row;
    float *pool;
    int32_t *next_row;
    int64_t cap, row_cap;
    int32_t dim, threshold;
    float init_a;
};

static TabArgs tab_args(const emb_table &t)
{
    TabArgs a;
    a.keys = reinterpret_cast<unsigned long long *>(t.slot_keys);
    a.count = t.slot_count;
    a.row = t.slot_row;
    a.pool = t.pool;
    a.next_row = t.next_row;
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

__device__ __forceinline__ void stat_add(int64_t *stats, int idx, int64_t v)
{
    const int64_t s = wave_sum_i64(v);
    if (stats && lane_id() == 0 && s) atomicAdd((unsigned long long *)&stats[idx], (unsigned long long)s);
}

__device__ __forceinline__ void stat_max(int64_t *stats, int idx, int64_t v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, (int64_t)__shfl_xor(v, o, 64));
    if (stats && lane_id() == 0 && v) atomicMax((unsigned long long *)&stats[idx], (unsigned long long)v);
}

// Counting under a skewed key stream: one block takes 1024 occurrences, adds them
// up per slot in an LDS hash (each hot key is counted once per block instead
// of once per occurrence), then adds each distinct slot's count to the table.
constexpr int kCountTile = 1024;               // occurrences per block, one per thread
constexpr int kLdsSlots = 2 * kCountTile;      // load factor <= 1/2: every insert finds room
constexpr int kLdsSlotBits = 11;
static_assert((1 << kLdsSlotBits) == kLdsSlots, "LDS hash size");

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
        bool inserted;
        const int64_t s = probe_insert(a, (unsigned long long)key, inserted, probes);
        if (s < 0) {
            *gp(pos + p) = kPosRefused;
            full = 1;
        } else {
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
        const int64_t si = wave_sum_i64(ins), sf = wave_sum_i64(full);
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
    for (int i = threadIdx.x; i < kLdsSlots; i += kCountTile)
        if (lslot[i] >= 0) atomicAdd(&a.count[lslot[i]], lcnt[i]);
    if (stats && threadIdx.x == 0) {
        if (lstat[0]) atomicAdd((unsigned long long *)&stats[EMB_STAT_TABLE_INSERTED], lstat[0]);
        if (lstat[1]) atomicAdd((unsigned long long *)&stats[EMB_STAT_TABLE_FULL], lstat[1]);
        if (lstat[2]) atomicMax((unsigned long long *)&stats[EMB_STAT_MAX_PROBE], lstat[2]);
    }
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
                const int32_t r = atomicAdd(a.next_row, 1);
                if ((int64_t)r < a.row_cap) {
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
                const int32_t r = atomicAdd(a.next_row, 1);
                if ((int64_t)r < a.row_cap) {
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

}  // namespace emb

using namespace emb;

static size_t a256(size_t x) { return (x + 255) & ~size_t(255); }

static emb_status table_sizes(int64_t capacity, int64_t row_capacity, int32_t dim, size_t off[5])
{
    if (capacity < 2 || capacity > (int64_t(1) << 30) || (capacity & (capacity - 1)))
        return fail(EMB_ERR_INVALID_ARG, "capacity must be a power of two in [2, 2^30]");
    if (row_capacity < 1 || row_capacity > (int64_t(1) << 31) - 1)
        return fail(EMB_ERR_INVALID_ARG, "row_capacity must be in [1, 2^31-1]");
    if (dim <= 0 || dim % 4 || dim > kMaxDimF32)
        return fail(EMB_ERR_UNSUPPORTED, "table dim must be a multiple of 4 and <= 256");
    size_t o = 0;
    off[0] = o; o = a256(o + 8 * (size_t)capacity);     // keys
    off[1] = o; o = a256(o + 4 * (size_t)capacity);     // counts
    off[2] = o; o = a256(o + 4 * (size_t)capacity);     // rows
    off[3] = o; o = a256(o + 256);                      // next_row
    off[4] = o;                                         // row pool [row_capacity, dim]
    return EMB_OK;
}

extern "C" {

emb_status emb_table_query(int64_t capacity, int64_t row_capacity, int32_t dim, size_t *table_bytes)
{
    if (!table_bytes) return fail(EMB_ERR_INVALID_ARG, "table_bytes is NULL");
    size_t off[5];
    emb_status s = table_sizes(capacity, row_capacity, dim, off);
    if (s != EMB_OK) return s;
    *table_bytes = off[4] + a256(4 * (size_t)row_capacity * (size_t)dim);
    return EMB_OK;
}

emb_status emb_table_create(int64_t capacity, int64_t row_capacity, int32_t dim, int32_t threshold,
                            float init_std, void *table_mem, void *stream, emb_table **out)
{
    if (!out) return fail(EMB_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    size_t off[5];
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
    T->slot_keys = reinterpret_cast<int64_t *>(m + off[0]);
    T->slot_count = reinterpret_cast<int32_t *>(m + off[1]);
    T->slot_row = reinterpret_cast<int32_t *>(m + off[2]);
    T->next_row = reinterpret_cast<int32_t *>(m + off[3]);
    T->pool = reinterpret_cast<float *>(m + off[4]);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemsetAsync(m, 0, off[2], st);                               // keys, counts
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
    hipLaunchKernelGGL(ht_count, dim3(cgrid), dim3(kCountTile), 0, st, a, keys, n, rows_out, stats);
    hipLaunchKernelGGL(ht_admit, dim3(grid_of(n)), dim3(kBlock), 0, st, a, keys, n, rows_out, stats);
    hipLaunchKernelGGL(ht_resolve, dim3(grid_of(n)), dim3(kBlock), 0, st, a, n, rows_out);
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

}  // extern "C"
