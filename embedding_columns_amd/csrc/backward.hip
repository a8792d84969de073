// backward.hip -- deduplicate touched rows, segment-sum their gradients, update rows.
//
// The gradient of the pooled output with respect to a table row u is the sum
// over the positions r that looked u up of w_r * G[s(r), :] (RecIS Sec. 3.2,
// Algorithm 1, backward half).  Instead of RecIS's wave-merge + global atomics,
// the contributions are grouped by a stable LSD radix sort of their 32-bit row
// keys (key = row_base_c + row), which yields the distinct touched rows (the
// "Reduce-ID" of RecIS Fig. 3) in ascending order and a fixed summation order,
// so gradients and updated weights are deterministic run to run.
//
//   pass p (ceil(key_bits / 9) passes of 9-bit digits):
//     rs_hist     per-block digit histograms
//     rs_scan     per-digit exclusive scan over blocks (+ digit totals)
//     rs_scatter  per-wavefront stable ranking by ballot matching, LDS-local
//                 digit sort, coalesced scatter of each digit run
//   (inputs whose columns fit a workgroup's LDS take the column sort instead)
//   uq_count / uq_scan / uq_write   segment heads -> unique keys + segment starts
//   seg_apply   one tile of sorted contributors per wavefront: gather fp32
//               G slices scaled by the pooling weight, sum per segment in
//               registers (split segments through LDS / last-arriver tickets
//               as in the forward), then EMIT, SGD or Adagrad on the row.
#include <algorithm>
#include <string>

#include "device.h"

namespace emb {

// ---------------------------------------------------------------- radix sort

// lanes of this wavefront whose digit equals mine (active lanes only), by one
// ballot per digit bit
template <int BITS = kRadixBits>
__device__ __forceinline__ uint64_t match_digit(uint32_t d, bool in)
{
    // per bit: m = lanes whose bit is set; a lane differs from me where m does
    // not equal my bit broadcast (bm, 0 or all ones); peers = lanes differing
    // in no bit
    uint32_t mis_lo = 0u, mis_hi = 0u;
#pragma unroll
    for (int b = 0; b < BITS; b++) {
        const uint32_t bm = (uint32_t)__builtin_amdgcn_sbfe((int)d, b, 1);
        const uint64_t m = __ballot(bm != 0u);
        mis_lo |= (uint32_t)m ^ bm;
        mis_hi |= (uint32_t)(m >> 32) ^ bm;
    }
    const uint64_t act = __ballot(in);
    return act & ~(((uint64_t)mis_hi << 32) | mis_lo);
}

// exclusive scan of one value per thread over a workgroup of NW wavefronts;
// returns the total
template <int NW = kWavesPerBlock>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *tmp, uint32_t &excl)
{
    const int t = threadIdx.x, lane = lane_id(), w = t / kWave;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
    if (lane == kWave - 1) tmp[w] = x;
    __syncthreads();
    uint32_t wpre = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; i++) {
        const uint32_t s = tmp[i];
        wpre += (i < w) ? s : 0u;
        tot += s;
    }
    excl = wpre + x - v;
    __syncthreads();
    return tot;
}

// exclusive scan of kRadix values, DPT = kRadix / (64 NW) consecutive ones per
// thread of a workgroup of NW wavefronts
template <int NW, int DPT>
__device__ __forceinline__ uint32_t digit_exclusive_scan(const uint32_t (&v)[DPT], uint32_t (&ex)[DPT],
                                                         uint32_t *tmp)
{
    static_assert(DPT * kWave * NW == kRadix, "digits per thread");
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < DPT; i++) sum += v[i];
    uint32_t base;
    const uint32_t tot = block_exclusive_scan<NW>(sum, tmp, base);
#pragma unroll
    for (int i = 0; i < DPT; i++) {
        ex[i] = base;
        base += v[i];
    }
    return tot;
}

// The histogram kernel's workgroup: HB threads, kSortTile / HB keys each, for one
// kSortTile tile.  512 threads in general; 1024 when every tile's workgroup is
// resident at once (at most 512 tiles: each workgroup is then the whole kernel's
// time, and fewer keys per thread shorten it).  Long sequences, 2,184 tiles: 512
// threads 180.8 us of dedup, 1024 190.5 us; the keyed step's 200 tiles: 62.7 ->
// 60.0 us with 1024.
constexpr int kHistBlock = 512;
constexpr int kHistBlockSmall = 1024;
constexpr int64_t kHistSmallTiles = 512;

// digit histogram of one tile of kSortTile keys.  PI: the keys are the first
// words of (key, value) pairs (the passes between the first and the last keep
// the pairs together, so that a scattered digit run is one contiguous write
// instead of two)
//
// ndev: the passes after a first pass that left keys out sort the *ndev keys it
// kept.  excl: the first pass leaves out keys >= excl (dropped and default-row
// sentinels when nothing needs them sorted), so the later passes move fewer.
template <bool PI, int HB>
__device__ __forceinline__ void hist_tile(const uint32_t *__restrict__ keys,
                                          const uint2 *__restrict__ pin, int64_t n,
                                          const uint32_t *__restrict__ ndev, uint32_t excl, int shift,
                                          uint32_t *__restrict__ hist, int64_t nblk,
                                          uint32_t *__restrict__ misc, int64_t tile, uint32_t *h)
{
    // the first pass starts the count of valid contributors at n; the last
    // pass lowers it to the position of the first sentinel key (or the first
    // pass's scatter sets it to the keys it kept)
    if (shift == 0 && tile == 0 && threadIdx.x == 0) *gp(misc) = (uint32_t)n;
    if (ndev) n = min<int64_t>(n, (int64_t)*gp(ndev));
    constexpr int kItems = kSortTile / HB;
    static_assert(kItems % 4 == 0, "keys are loaded four (or two pairs) at a time");
    const int t = threadIdx.x, lane = lane_id();
    for (int d = t; d < kRadix; d += HB) h[d] = 0;
    __syncthreads();
    const int64_t base = tile * kSortTile;
    // the tile's keys in 16-byte loads (4 keys, or 2 pairs, per load); a
    // histogram does not depend on which thread counts which key
    uint32_t k[kItems];
    bool kin[kItems];
    if (PI) {
#pragma unroll
        for (int i = 0; i < kItems / 2; i++) {
            const int64_t idx = base + 2 * ((int64_t)i * HB + t);   // first of two pairs
            const uint4 v = idx < n ? static_cast<uint4>(*gp(reinterpret_cast<const uint4 *>(pin + idx)))
                                    : make_uint4(0u, 0u, 0u, 0u);
            k[2 * i] = v.x;
            k[2 * i + 1] = v.z;
            kin[2 * i] = idx < n && v.x < excl;
            kin[2 * i + 1] = idx + 1 < n && v.z < excl;
        }
    } else {
#pragma unroll
        for (int i = 0; i < kItems / 4; i++) {
            const int64_t idx = base + 4 * ((int64_t)i * HB + t);
            const uint4 v = idx < n ? static_cast<uint4>(*gp(reinterpret_cast<const uint4 *>(keys + idx)))
                                    : make_uint4(0u, 0u, 0u, 0u);
            k[4 * i] = v.x; k[4 * i + 1] = v.y; k[4 * i + 2] = v.z; k[4 * i + 3] = v.w;
#pragma unroll
            for (int j = 0; j < 4; j++) kin[4 * i + j] = idx + j < n && k[4 * i + j] < excl;
        }
    }
    // LDS atomics.  Skewed keys put most of a wavefront's lanes on one digit (the
    // hot rows' digit in the high passes), and same-address atomics of one
    // instruction run one after another: the lanes that share the digit of the
    // first remaining lane are counted with one atomic, twice over, and only the
    // lanes left after that add one each.
#pragma unroll
    for (int i = 0; i < kItems; i++) {
        bool left = kin[i];
        const uint32_t d = (k[i] >> shift) & (kRadix - 1);
#pragma unroll
        for (int r = 0; r < 2; r++) {
            const uint64_t rem = __ballot(left);
            if (rem == 0) break;
            const int fl = __ffsll((long long)rem) - 1;
            const uint32_t dr = (uint32_t)__builtin_amdgcn_readlane((int)d, fl);
            const uint64_t m = __ballot(left && d == dr);
            if (lane == fl) atomicAdd(&h[dr], (uint32_t)__popcll(m));
            left = left && d != dr;
        }
        if (left) atomicAdd(&h[d], 1u);
    }
    __syncthreads();
    for (int d = t; d < kRadix; d += HB) hist[(int64_t)d * nblk + tile] = h[d];
    __syncthreads();
}

// Both per-tile kernels take their tiles in one contiguous range per XCD: the
// histogram words of neighbouring tiles (hist[d][b], hist[d][b + 1]) and the
// two halves of a digit run cut by a line boundary then meet in one L2 instead
// of reaching memory as partial lines from two XCDs.
template <bool PI, int HB>
__global__ __launch_bounds__(HB) void rs_hist(const uint32_t *__restrict__ keys,
                                                 const uint2 *__restrict__ pin, int64_t n,
                                                 const uint32_t *__restrict__ ndev, uint32_t excl,
                                                 int shift, uint32_t *__restrict__ hist,
                                                 int64_t nblk, uint32_t *__restrict__ misc)
{
    __shared__ uint32_t h[kRadix];
    hist_tile<PI, HB>(keys, pin, n, ndev, excl, shift, hist, nblk, misc, xcd_block(blockIdx.x, gridDim.x, 0), h);
}

// exclusive scan of one digit's block counts hist[d][0..nblk) in place, total ->
// dtot[d], one block per digit.  Per round of kScanChunk counts: coalesced loads
// into LDS, each thread sums a contiguous run of kScanRun counts there, one
// block-wide scan of the run sums, the run prefixes back through LDS, coalesced
// stores.  (Each thread loading its own run straight from memory put 64
// different lines behind every load instruction.)
constexpr int kScanRun = 16;
constexpr int kScanChunk = kBlock * kScanRun;     // 4096 blocks per round
__global__ __launch_bounds__(kBlock) void rs_scan(uint32_t *__restrict__ hist, int64_t nblk,
                                                 uint32_t *__restrict__ dtot)
{
    __shared__ uint32_t buf[kScanChunk];
    __shared__ uint32_t tmp[kWavesPerBlock];
    const int t = threadIdx.x;
    uint32_t *h = hist + (int64_t)blockIdx.x * nblk;
    uint32_t carry = 0;
    for (int64_t s0 = 0; s0 < nblk; s0 += kScanChunk) {
        const int m = (int)min<int64_t>(kScanChunk, nblk - s0);
        uint32_t v[kScanRun];
#pragma unroll
        for (int k = 0; k < kScanRun; k++) {
            const int i = k * kBlock + t;
            v[k] = i < m ? h[s0 + i] : 0u;
        }
#pragma unroll
        for (int k = 0; k < kScanRun; k++) buf[k * kBlock + t] = v[k];
        __syncthreads();
        uint32_t sum = 0;
#pragma unroll
        for (int k = 0; k < kScanRun; k++) {
            v[k] = buf[t * kScanRun + k];
            sum += v[k];
        }
        uint32_t ex;
        const uint32_t tot = block_exclusive_scan(sum, tmp, ex);   // ends with a barrier
        uint32_t run = carry + ex;
#pragma unroll
        for (int k = 0; k < kScanRun; k++) {
            buf[t * kScanRun + k] = run;
            run += v[k];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kScanRun; k++) {
            const int i = k * kBlock + t;
            if (i < m) h[s0 + i] = buf[i];
        }
        carry += tot;
        __syncthreads();
    }
    if (t == 0) dtot[blockIdx.x] = carry;
}

// The scatter kernel's workgroup: kScatWaves wavefronts over one kSortTile tile.
constexpr int kScatWaves = 4;
constexpr int kScatBlock = kWave * kScatWaves;
constexpr int kScatItems = kSortTile / kScatBlock;     // keys per lane
constexpr int kScatDigits = kRadix / kScatBlock;       // digits per thread in the offset scans

struct SortLds {
    uint32_t skey[kSortTile];
    uint32_t sval[kSortTile];
    uint16_t run[kScatWaves][kRadix];       // per-wave running digit counts (<= 4096)
    uint32_t gdst[kRadix];                  // global destination of digit d's run minus its LDS start
    uint32_t tmp[kScatWaves];
};

// PI / PO: the input / output is (key, value) pairs instead of two arrays
template <bool PI, bool PO>
__device__ __forceinline__ void scatter_tile(const uint32_t *__restrict__ kin,
                                             const uint32_t *__restrict__ vin,
                                             uint32_t *__restrict__ kout, uint32_t *__restrict__ vout,
                                             const uint2 *__restrict__ pin, uint2 *__restrict__ pout,
                                             int64_t n, const uint32_t *__restrict__ ndev, uint32_t excl,
                                             uint32_t *__restrict__ nkept, int shift,
                                             const uint32_t *__restrict__ hist,
                                             const uint32_t *__restrict__ dtot, int64_t nblk,
                                             uint32_t sentinel, uint32_t *__restrict__ misc,
                                             int64_t tile, SortLds &S)
{
    const int t = threadIdx.x, lane = lane_id(), w = t / kWave;
    const int64_t base = tile * kSortTile;
    if (ndev) n = min<int64_t>(n, (int64_t)*gp(ndev));
    const int cnt = (int)min<int64_t>(kSortTile, n - base);
    if (cnt <= 0) return;                     // past the keys an excluding first pass kept

    // each wavefront owns W = kSortTile / kScatWaves consecutive keys: item j of lane l
    // is wave*W + j*64 + l, so (wave, j, lane) order is index order and the ranking
    // below is stable.
    // All loads are issued first: the barriers and fences below would otherwise
    // hold each load behind the previous step.
    uint32_t key[kScatItems], val[kScatItems], rank[kScatItems];
    bool inc[kScatItems];                     // loaded and not left out
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int j = 0; j < kScatItems; j++) {
        const int li = w * (kSortTile / kScatWaves) + j * kWave + lane;
        const bool in = li < cnt;
        if (PI) {
            const uint2 pr = in ? static_cast<uint2>(*gp(pin + base + li)) : make_uint2(0u, 0u);
            key[j] = pr.x;
            val[j] = pr.y;
        } else {
            key[j] = in ? *gp(kin + base + li) : 0u;
            val[j] = in ? *gp(vin + base + li) : 0u;
        }
        inc[j] = in;
    }
#pragma unroll
    for (int j = 0; j < kScatItems; j++) inc[j] = inc[j] && key[j] < excl;

    // digit offsets: global prefix over digits + this block's offset within each
    // digit (kept by the thread that owns digits t * kScatDigits + i)
    uint32_t gbase[kScatDigits];
    {
        uint32_t v[kScatDigits];
#pragma unroll
        for (int i = 0; i < kScatDigits; i++) v[i] = dtot[t * kScatDigits + i];
        const uint32_t kept = digit_exclusive_scan<kScatWaves>(v, gbase, S.tmp);
        // an excluding first pass: the keys kept are the later passes' count
        if (nkept && tile == 0 && t == 0) *gp(nkept) = kept;
#pragma unroll
        for (int i = 0; i < kScatDigits; i++)
            gbase[i] += hist[(int64_t)(t * kScatDigits + i) * nblk + tile];
        for (int d = t; d < kRadix; d += kScatBlock)
            for (int i = 0; i < kScatWaves; i++) S.run[i][d] = 0;
    }
    __syncthreads();

#pragma unroll
    for (int j = 0; j < kScatItems; j++) {
        const bool in = inc[j];
        const uint32_t d = (key[j] >> shift) & (kRadix - 1);
        const uint64_t peers = match_digit(d, in);
        const uint32_t before = S.run[w][d];
        rank[j] = before + (uint32_t)__popcll(peers & lt_mask);
        const bool leader = in && (peers >> lane) == 1ull;   // highest lane of its digit group
        wave_sync();
        if (leader) S.run[w][d] = (uint16_t)(before + (uint32_t)__popcll(peers));
        wave_sync();
    }
    __syncthreads();
    // block-local digit histogram -> local prefix; per-wave offsets inside each digit
    int nloc;                                  // keys of this tile that are sorted
    {
        uint32_t tot[kScatDigits], lex[kScatDigits], woff[kScatDigits][kScatWaves];
#pragma unroll
        for (int i = 0; i < kScatDigits; i++) {
            const int d = t * kScatDigits + i;
            tot[i] = 0;
#pragma unroll
            for (int k = 0; k < kScatWaves; k++) {
                woff[i][k] = tot[i];
                tot[i] += S.run[k][d];
            }
        }
        nloc = (int)digit_exclusive_scan<kScatWaves>(tot, lex, S.tmp);
#pragma unroll
        for (int i = 0; i < kScatDigits; i++) {
            const int d = t * kScatDigits + i;
            S.gdst[d] = gbase[i] - lex[i];      // wraps; gdst + LDS position is the destination
#pragma unroll
            for (int k = 0; k < kScatWaves; k++) S.run[k][d] = (uint16_t)(lex[i] + woff[i][k]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kScatItems; j++) {
        if (inc[j]) {
            const uint32_t d = (key[j] >> shift) & (kRadix - 1);
            const uint32_t lp = S.run[w][d] + rank[j];
            S.skey[lp] = key[j];
            S.sval[lp] = val[j];
        }
    }
    __syncthreads();
    // write each digit run contiguously
    uint32_t first_sentinel = 0xFFFFFFFFu;
    for (int lp = t; lp < nloc; lp += kScatBlock) {
        const uint32_t k = S.skey[lp];
        const uint32_t d = (k >> shift) & (kRadix - 1);
        const uint32_t dst = S.gdst[d] + (uint32_t)lp;
        if (PO) {
            *gp(pout + dst) = make_uint2(k, S.sval[lp]);
        } else {
            *gp(kout + dst) = k;
            *gp(vout + dst) = S.sval[lp];
        }
        if (k >= sentinel) first_sentinel = min(first_sentinel, dst);
    }
    // last pass: every key >= sentinel (dropped / default rows) sorts after the
    // valid ones, so the smallest destination of such a key is their count
    if (misc) {
        for (int o = 1; o < kWave; o <<= 1) first_sentinel = min(first_sentinel, (uint32_t)__shfl_xor((int)first_sentinel, o, kWave));
        if (lane == 0 && first_sentinel != 0xFFFFFFFFu) atomicMin(misc, first_sentinel);
    }
    __syncthreads();
}

template <bool PI, bool PO>
__global__ __launch_bounds__(kScatBlock) void rs_scatter(const uint32_t *__restrict__ kin,
                                                    const uint32_t *__restrict__ vin,
                                                    uint32_t *__restrict__ kout,
                                                    uint32_t *__restrict__ vout,
                                                    const uint2 *__restrict__ pin,
                                                    uint2 *__restrict__ pout, int64_t n,
                                                    const uint32_t *__restrict__ ndev, uint32_t excl,
                                                    uint32_t *__restrict__ nkept, int shift,
                                                    const uint32_t *__restrict__ hist,
                                                    const uint32_t *__restrict__ dtot, int64_t nblk,
                                                    uint32_t sentinel, uint32_t *__restrict__ misc)
{
    __shared__ SortLds S;
    scatter_tile<PI, PO>(kin, vin, kout, vout, pin, pout, n, ndev, excl, nkept, shift, hist, dtot, nblk,
                         sentinel, misc,
                         xcd_block(blockIdx.x, gridDim.x, 0), S);
}

// ------------------------------------------------ column-local sort in LDS
//
// Positions are column-major and a column's keys (row_base_c + row) lie in its
// own key range, so sorting all keys equals sorting each column's positions in
// place.  One workgroup per column sorts a column of at most kColCap positions
// entirely in LDS (a stable LSD radix sort on the row within the column, 7-bit
// digits), with dropped / DEFAULT keys last inside the column instead of at the
// end of the array; a larger column goes through global memory in chunks.

constexpr int kCSWaves = 16;
constexpr int kCSBlock = kCSWaves * kWave;
constexpr int kCSBits = 7;
constexpr int kCSRadix = 1 << kCSBits;
constexpr int kColCap = 12288;
constexpr int kCSItems = kColCap / kCSBlock;            // items per thread
static_assert(kColCap % (kCSBlock) == 0, "column capacity");
static_assert(kCSRadix == 2 * kWave, "the digit scan spans two wavefronts");

struct ColSortLds {
    uint32_t key[2][kColCap];          // local keys, ping-pong
    uint16_t idx[2][kColCap];          // position within the column
    uint32_t run[kCSWaves][kCSRadix];  // per-wave digit counts, then destinations
    uint32_t dpre[kCSRadix + 1];       // digit offsets (chunked sort); [kCSRadix]: a scan carry
};

// Digit-major destinations of one ranking round: thread d < kCSRadix reads
// digit d's per-wave counts S.run[k][d], and S.run[k][d] becomes base[d] plus
// the counts of digit d in waves before k (base: the digit starts).  Returns
// digit d's total to thread d.
__device__ __forceinline__ uint32_t cs_digit_bases(ColSortLds &S, bool chunk_bases)
{
    const int t = threadIdx.x, lane = lane_id();
    uint32_t cw[kCSWaves], incl = 0, tot = 0;
    if (t < kCSRadix) {
#pragma unroll
        for (int k = 0; k < kCSWaves; k++) {
            cw[k] = S.run[k][t];
            tot += cw[k];
        }
        incl = tot;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const uint32_t y = __shfl_up(incl, o, kWave);
            if (lane >= o) incl += y;
        }
        incl -= tot;                                   // exclusive within the wave
        if (t == kWave - 1) S.dpre[kCSRadix] = incl + tot;   // digits 0..63 in total
    }
    __syncthreads();
    if (t < kCSRadix) {
        // in-LDS sort: digit starts from the scan; chunked sort: running
        // per-digit offsets of the column, kept in S.dpre
        uint32_t base = chunk_bases ? S.dpre[t] : incl + (t >= kWave ? S.dpre[kCSRadix] : 0u);
#pragma unroll
        for (int k = 0; k < kCSWaves; k++) {
            S.run[k][t] = base;
            base += cw[k];
        }
    }
    __syncthreads();
    return tot;
}

// A column of more than kColCap positions, sorted by its workgroup through
// global memory: per pass (7-bit digit of the local key) a digit histogram of
// the column, then chunks of kColCap keys ranked stably in LDS and scattered to
// running per-digit offsets, ping-ponging between the column's ranges of the
// two key / bag arrays (A holds the input).  The result ends in kout / vout.
__device__ void col_sort_big(ColSortLds &S, uint32_t *kA, uint32_t *vA, uint32_t *kB, uint32_t *vB,
                             uint32_t *kout, uint32_t *vout, int P0, int cnt, uint32_t rb,
                             uint32_t rows, uint32_t total_rows, int passes)
{
    const int t = threadIdx.x, lane = lane_id(), w = t / kWave;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    auto lkey = [&](uint32_t k) { return k < total_rows ? k - rb : rows + (k - total_rows); };
    for (int pass = 0; pass < passes; pass++) {
        const int shift = pass * kCSBits;
        uint32_t *ks = (pass & 1) ? kB : kA, *vs = (pass & 1) ? vB : vA;
        uint32_t *kd = (pass & 1) ? kA : kB, *vd = (pass & 1) ? vA : vB;
        // digit histogram of the whole column -> running offsets S.dpre[d]
        if (t < kCSRadix) S.dpre[t] = 0u;
        __syncthreads();
        for (int i = t; i < cnt; i += kCSBlock)
            atomicAdd(&S.dpre[(lkey(*gp(ks + P0 + i)) >> shift) & (kCSRadix - 1)], 1u);
        __syncthreads();
        if (t < kCSRadix) {
            const uint32_t v = S.dpre[t];
            uint32_t incl = v;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const uint32_t y = __shfl_up(incl, o, kWave);
                if (lane >= o) incl += y;
            }
            if (t == kWave - 1) S.dpre[kCSRadix] = incl;
            S.run[0][t] = incl - v;
        }
        __syncthreads();
        if (t < kCSRadix) S.dpre[t] = S.run[0][t] + (t >= kWave ? S.dpre[kCSRadix] : 0u);
        __syncthreads();
        for (int c0 = 0; c0 < cnt; c0 += kColCap) {
            const int m = min(kColCap, cnt - c0);
            const int per = ((m + kCSWaves * kWave - 1) / (kCSWaves * kWave)) * kWave;
            for (int d = lane; d < kCSRadix; d += kWave) S.run[w][d] = 0;
            wave_sync();
            uint32_t rank[kCSItems], dig[kCSItems], prev[kCSItems], key[kCSItems];
            int lead[kCSItems];
#pragma unroll
            for (int j = 0; j < kCSItems; j++) {
                const int i = w * per + j * kWave + lane;
                key[j] = (j * kWave < per && i < m) ? *gp(ks + P0 + c0 + i) : 0u;
            }
#pragma unroll
            for (int j = 0; j < kCSItems; j++) {
                const int i = w * per + j * kWave + lane;
                const bool in = j * kWave < per && i < m;
                const uint32_t d = in ? (lkey(key[j]) >> shift) & (kCSRadix - 1) : 0u;
                const uint64_t peers = match_digit<kCSBits>(d, in);
                lead[j] = in ? __ffsll((unsigned long long)peers) - 1 : lane;
                rank[j] = (uint32_t)__popcll(peers & lt_mask);
                dig[j] = d;
                prev[j] = 0u;
                if (in && lead[j] == lane) prev[j] = atomicAdd(&S.run[w][d], (uint32_t)__popcll(peers));
            }
#pragma unroll
            for (int j = 0; j < kCSItems; j++) rank[j] += (uint32_t)__shfl((int)prev[j], lead[j], kWave);
            __syncthreads();
            const uint32_t tot = cs_digit_bases(S, true);
#pragma unroll
            for (int j = 0; j < kCSItems; j++) {
                const int i = w * per + j * kWave + lane;
                if (j * kWave < per && i < m) {
                    const uint32_t o = S.run[w][dig[j]] + rank[j];
                    *gp(kd + P0 + o) = key[j];
                    *gp(vd + P0 + o) = *gp(vs + P0 + c0 + i);
                }
            }
            if (t < kCSRadix) S.dpre[t] += tot;
            __syncthreads();
        }
    }
    uint32_t *kr = (passes & 1) ? kB : kA, *vr = (passes & 1) ? vB : vA;
    if (kr != kout) {
        for (int i = t; i < cnt; i += kCSBlock) {
            *gp(kout + P0 + i) = *gp(kr + P0 + i);
            *gp(vout + P0 + i) = *gp(vr + P0 + i);
        }
    }
}

// Columns whose local keys fit 20 bits (tables below 2^20 - 2 rows) sort in at
// most two passes of 10-bit digits.  Pass 1 ranks the keys straight from
// registers and writes (key >> 10, position) packed in 24 bits; pass 2 ranks
// those by their high digit.  Per-wave counts are 16-bit halves of 32-bit
// words (a count or offset never exceeds kColCap), which keeps 1024 digits per
// wave inside the LDS the 7-bit sort uses.  At the end the keys and values go
// into the two buffers by position and are gathered in sorted order.
constexpr int kC2Bits = 10;
constexpr int kC2Radix = 1 << kC2Bits;
constexpr int kC2PosBits = 14;
static_assert(kColCap <= (1 << kC2PosBits), "positions fit the packed item");
static_assert(kCSBlock == kC2Radix, "one thread per digit in the digit scan");

struct ColSort2Lds {
    uint32_t b1[kColCap];                  // pass 1 output: (key >> 10) << 14 | position
    uint32_t b2[kColCap];                  // pass 2 output, same packing
    uint32_t run[kCSWaves][kC2Radix / 2];  // per-wave counts, then offsets: digit d in half d & 1 of word d / 2
    uint32_t wsum[kCSWaves];
};

union ColSortShared {
    ColSortLds s7;
    ColSort2Lds s10;
};

// One stable ranking pass over the items of a column in wave-contiguous order
// (wave w holds items w*per .. w*per+per-1, lane-fastest): item j of this lane
// has value item[j] and digit (PASS 1) key[j] & 1023 of its local key, or
// (PASS 2) item[j] >> 14; the values land in `out` in digit order.
template <int PASS>
__device__ __forceinline__ uint32_t c2_digit(uint32_t key, uint32_t item)
{
    return PASS == 1 ? (key & (kC2Radix - 1)) : (item >> kC2PosBits);
}

template <int PASS>
__device__ __forceinline__ void c2_pass(ColSort2Lds &S, const uint32_t (&key)[kCSItems],
                                        const uint32_t (&item)[kCSItems], int per, int cnt,
                                        uint32_t *out)
{
    const int t = threadIdx.x, lane = lane_id(), w = t / kWave;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int k = lane; k < kC2Radix / 2; k += kWave) S.run[w][k] = 0u;
    wave_sync();
    // rank within this wave's earlier items of the digit: lower lanes now, plus
    // the count before this round, which the group's lowest lane gets back from
    // its LDS add (taken at once: registers are short here)
    uint32_t rk[kCSItems];
#pragma unroll
    for (int j = 0; j < kCSItems; j++) {
        const int i = w * per + j * kWave + lane;
        const bool in = j * kWave < per && i < cnt;
        const uint32_t d = in ? c2_digit<PASS>(key[j], item[j]) : 0u;
        const uint64_t peers = match_digit<kC2Bits>(d, in);
        const int lead = in ? __ffsll((unsigned long long)peers) - 1 : lane;
        uint32_t prev = 0u;
        if (in && lead == lane) {
            const uint32_t sh = (d & 1u) * 16u;
            prev = (atomicAdd(&S.run[w][d >> 1], (uint32_t)__popcll(peers) << sh) >> sh) & 0xFFFFu;
        }
        rk[j] = (uint32_t)__popcll(peers & lt_mask) + (uint32_t)__shfl((int)prev, lead, kWave);
    }
    __syncthreads();
    // offsets: thread t < 512 takes digits 2t and 2t+1; an exclusive scan of the
    // pair totals over those threads gives the digit starts, then each wave's
    // offset within a digit adds the counts of the waves before it
    uint32_t tlo = 0, thi = 0, incl = 0;
    if (t < kC2Radix / 2) {
#pragma unroll
        for (int k = 0; k < kCSWaves; k++) {
            const uint32_t v = S.run[k][t];
            tlo += v & 0xFFFFu;
            thi += v >> 16;
        }
        incl = tlo + thi;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const uint32_t y = __shfl_up(incl, o, kWave);
            if (lane >= o) incl += y;
        }
        if (lane == kWave - 1) S.wsum[w] = incl;
    }
    __syncthreads();
    if (t < kC2Radix / 2) {
        uint32_t carry = 0;
        for (int k = 0; k < w; k++) carry += S.wsum[k];
        uint32_t blo = carry + incl - (tlo + thi), bhi = blo + tlo;
#pragma unroll
        for (int k = 0; k < kCSWaves; k++) {
            const uint32_t v = S.run[k][t];
            S.run[k][t] = blo | (bhi << 16);
            blo += v & 0xFFFFu;
            bhi += v >> 16;
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kCSItems; j++) {
        const int i = w * per + j * kWave + lane;
        if (j * kWave < per && i < cnt) {
            const uint32_t d = c2_digit<PASS>(key[j], item[j]);
            const uint32_t o = ((S.run[w][d >> 1] >> ((d & 1u) * 16u)) & 0xFFFFu) + rk[j];
            out[o] = item[j];
        }
    }
    __syncthreads();
}

__device__ __forceinline__ void col_sort_2pass(ColSort2Lds &S, const uint32_t *kin, const uint32_t *vin,
                                               uint32_t *kout, uint32_t *vout, int P0, int cnt,
                                               uint32_t rb, uint32_t rows, uint32_t total_rows,
                                               int bits)
{
    const int t = threadIdx.x, lane = lane_id(), w = t / kWave;
    const int per = ((cnt + kCSBlock - 1) / kCSBlock) * kWave;
    // keys and values of this thread's items, wave-contiguous, all loads at once
    uint32_t kv[kCSItems], vv[kCSItems], item[kCSItems];
#pragma unroll
    for (int j = 0; j < kCSItems; j++) {
        const int i = w * per + j * kWave + lane;
        const bool in = j * kWave < per && i < cnt;
        kv[j] = in ? *gp(kin + P0 + i) : 0u;
        vv[j] = in ? *gp(vin + P0 + i) : 0u;
    }
    // pass 1: the low digit of the local key (the row, or rows / rows + 1 for
    // dropped / DEFAULT); kv holds local keys until the end
#pragma unroll
    for (int j = 0; j < kCSItems; j++) {
        const int i = w * per + j * kWave + lane;
        kv[j] = kv[j] < total_rows ? kv[j] - rb : rows + (kv[j] - total_rows);
        item[j] = ((kv[j] >> kC2Bits) << kC2PosBits) | (uint32_t)i;
    }
    c2_pass<1>(S, kv, item, per, cnt, S.b1);
    uint32_t *res = S.b1;
    if (bits > kC2Bits) {
        // pass 2: the high digit, in the pass 1 order
#pragma unroll
        for (int j = 0; j < kCSItems; j++) {
            const int i = w * per + j * kWave + lane;
            item[j] = (j * kWave < per && i < cnt) ? S.b1[i] : 0u;
        }
        c2_pass<2>(S, kv, item, per, cnt, S.b2);
        res = S.b2;
    }
    // sorted order -> positions; then keys and values by position into the two
    // buffers, gathered in sorted order
#pragma unroll
    for (int j = 0; j < kCSItems; j++) {
        const int i = w * per + j * kWave + lane;
        item[j] = (j * kWave < per && i < cnt) ? (res[i] & ((1u << kC2PosBits) - 1u)) : 0u;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kCSItems; j++) {
        const int i = w * per + j * kWave + lane;
        if (j * kWave < per && i < cnt) {
            S.b1[i] = kv[j] < rows ? kv[j] + rb : total_rows + (kv[j] - rows);
            S.b2[i] = vv[j];
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kCSItems; j++) {
        const int i = w * per + j * kWave + lane;
        if (j * kWave < per && i < cnt) {
            *gp(kout + P0 + i) = S.b1[item[j]];
            *gp(vout + P0 + i) = S.b2[item[j]];
        }
    }
}

__device__ __forceinline__ void col_sort_column(ColSortShared &SU, uint32_t *kin, uint32_t *vin,
                                                uint32_t *kspare, uint32_t *vspare, uint32_t *kout,
                                                uint32_t *vout, int64_t n,
                                                const uint32_t *__restrict__ cstart,
                                                const uint32_t *__restrict__ row_base,
                                                uint32_t total_rows, uint32_t *misc)
{
    ColSortLds &S = SU.s7;
    const int t = threadIdx.x, lane = lane_id(), w = t / kWave;
    const int c = blockIdx.x;
    if (c == 0 && t == 0) *gp(misc) = (uint32_t)n;   // every position is a contributor slot
    // the column's positions, recorded by the forward
    const int P0 = (int)cstart[c], cnt = (int)cstart[c + 1] - P0;
    if (cnt == 0) return;
    const uint32_t rb = row_base[c], rows = row_base[c + 1] - rb;
    const int bits = 32 - __clz((int)(rows + 1));
    const int passes = (bits + kCSBits - 1) / kCSBits;
    if (cnt > kColCap) {
        col_sort_big(S, kin, vin, kspare, vspare, kout, vout, P0, cnt, rb, rows, total_rows, passes);
        return;
    }
    if (bits <= 2 * kC2Bits) {
        col_sort_2pass(SU.s10, kin, vin, kout, vout, P0, cnt, rb, rows, total_rows, bits);
        return;
    }

    // local key: the row, or rows / rows + 1 for dropped / DEFAULT.  The values
    // are read now too, with the keys, and wait in registers: at the end they go
    // through the free LDS key buffer instead of a second round of global reads.
    uint32_t vv[kCSItems];
    {
        uint32_t kv[kCSItems];
#pragma unroll
        for (int j = 0; j < kCSItems; j++) {
            const int i = j * kCSBlock + t;
            kv[j] = i < cnt ? *gp(kin + P0 + i) : 0u;
            vv[j] = i < cnt ? *gp(vin + P0 + i) : 0u;
        }
#pragma unroll
        for (int j = 0; j < kCSItems; j++) {
            const int i = j * kCSBlock + t;
            if (i < cnt) {
                S.key[0][i] = kv[j] < total_rows ? kv[j] - rb : rows + (kv[j] - total_rows);
                S.idx[0][i] = (uint16_t)i;
            }
        }
    }
    __syncthreads();

    // wave w ranks items w*per .. (w+1)*per-1 in (j, lane) order: stable
    const int per = ((cnt + kCSWaves * kWave - 1) / (kCSWaves * kWave)) * kWave;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int pass = 0; pass < passes; pass++) {
        const int src = pass & 1, dst = src ^ 1, shift = pass * kCSBits;
        for (int d = lane; d < kCSRadix; d += kWave) S.run[w][d] = 0;
        wave_sync();
        // rank = items of the same digit in earlier rounds of this wave (the
        // value the group's lowest lane gets back from its LDS add: one wave's
        // LDS operations run in order) + lower lanes of this round
        uint32_t rank[kCSItems], dig[kCSItems], prev[kCSItems];
        int lead[kCSItems];
#pragma unroll
        for (int j = 0; j < kCSItems; j++) {         // all key reads first
            const int i = w * per + j * kWave + lane;
            dig[j] = (j * kWave < per && i < cnt) ? S.key[src][i] : 0u;
        }
#pragma unroll
        for (int j = 0; j < kCSItems; j++) {
            const int i = w * per + j * kWave + lane;
            const bool in = j * kWave < per && i < cnt;
            const uint32_t d = in ? (dig[j] >> shift) & (kCSRadix - 1) : 0u;
            const uint64_t peers = match_digit<kCSBits>(d, in);
            lead[j] = in ? __ffsll((unsigned long long)peers) - 1 : lane;
            rank[j] = (uint32_t)__popcll(peers & lt_mask);
            dig[j] = d;
            prev[j] = 0u;
            if (in && lead[j] == lane) prev[j] = atomicAdd(&S.run[w][d], (uint32_t)__popcll(peers));
        }
#pragma unroll
        for (int j = 0; j < kCSItems; j++) rank[j] += (uint32_t)__shfl((int)prev[j], lead[j], kWave);
        __syncthreads();
        // destinations, digit-major over (digit, wave)
        cs_digit_bases(S, false);
#pragma unroll
        for (int j = 0; j < kCSItems; j++) {
            const int i = w * per + j * kWave + lane;
            if (j * kWave < per && i < cnt) {
                const uint32_t o = S.run[w][dig[j]] + rank[j];
                S.key[dst][o] = S.key[src][i];
                S.idx[dst][o] = S.idx[src][i];
            }
        }
        __syncthreads();
    }

    // back to global keys; each value is gathered from the other key buffer
    // (free now), where the values were put in position order
    const int fin = passes & 1;
#pragma unroll
    for (int j = 0; j < kCSItems; j++) {
        const int i = j * kCSBlock + t;
        if (i < cnt) S.key[fin ^ 1][i] = vv[j];
    }
    __syncthreads();
    uint32_t ko[kCSItems], vo[kCSItems];
#pragma unroll
    for (int j = 0; j < kCSItems; j++) {
        const int i = j * kCSBlock + t;
        if (i < cnt) {
            const uint32_t k = S.key[fin][i];
            ko[j] = k < rows ? k + rb : total_rows + (k - rows);
            vo[j] = S.key[fin ^ 1][S.idx[fin][i]];
        }
    }
#pragma unroll
    for (int j = 0; j < kCSItems; j++) {
        const int i = j * kCSBlock + t;
        if (i < cnt) {
            *gp(kout + P0 + i) = ko[j];
            *gp(vout + P0 + i) = vo[j];
        }
    }
}

// Valid keys (below total_rows) of column blockIdx.x, counted in its sorted keys:
// the dropped ones sort after the column's rows.
// Each column's count of valid keys into vcnt[c]; the workgroup whose column
// finishes last (a ticket) then writes their exclusive prefix vbase[0 .. C]
// (vbase[C]: all valid keys) and resets the ticket for the next call.
__device__ __forceinline__ void col_valid_count(const uint32_t *kout, const uint32_t *cstart,
                                                uint32_t total_rows, uint32_t *vcnt, int C)
{
    __syncthreads();   // every wave's sorted keys are written
    if (threadIdx.x >= kWave) return;
    const int c = blockIdx.x, lane = lane_id();
    uint32_t *vbase = vcnt + C + 1, *vtick = vbase + C + 1;
    const int64_t P0 = cstart[c], cnt = (int64_t)cstart[c + 1] - P0;
    const int64_t nv = (cnt > 0 && total_rows > 0) ? wave_upper_bound(kout + P0, cnt, total_rows - 1u) : 0;
    if (lane == 0) st_agent(vcnt + c, (uint32_t)nv);
    wait_vm();                                   // the count is visible before the ticket
    uint32_t old = 0;
    if (lane == 0) old = ticket_add(vtick);
    old = (uint32_t)__shfl((int)old, 0, kWave);
    if (old != (uint32_t)(C - 1)) return;
    uint32_t carry = 0;
    for (int s = 0; s < C; s += kWave) {
        const int i = s + lane;
        const uint32_t v = i < C ? ld_agent(vcnt + i) : 0u;
        uint32_t x = v;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const uint32_t y = __shfl_up(x, o, kWave);
            if (lane >= o) x += y;
        }
        if (i < C) vbase[i] = carry + x - v;
        carry += (uint32_t)__shfl((int)x, kWave - 1, kWave);
    }
    if (lane == 0) {
        vbase[C] = carry;
        st_agent(vtick, 0u);                     // ready for the next call
    }
}

// One workgroup per column.  With vcnt, it also records the column's number of
// valid keys, for the compaction that turns the column runs into one sorted run.
__global__ __launch_bounds__(kCSBlock) void col_sort(uint32_t *kin, uint32_t *vin, uint32_t *kspare,
                                                    uint32_t *vspare, uint32_t *kout, uint32_t *vout,
                                                    int64_t n, const uint32_t *__restrict__ cstart,
                                                    const uint32_t *__restrict__ row_base,
                                                    uint32_t total_rows, uint32_t *misc, uint32_t *vcnt)
{
    __shared__ ColSortShared SU;
    col_sort_column(SU, kin, vin, kspare, vspare, kout, vout, n, cstart, row_base, total_rows, misc);
    if (vcnt) col_valid_count(kout, cstart, total_rows, vcnt, (int)gridDim.x);
}

// exclusive prefix of the columns' valid counts: vbase[c]; vbase[C] = all valid keys
// The column-sorted keys and values, moved so that the valid keys of all columns
// come first, column after column (one ascending run: columns own disjoint,
// increasing key ranges), then every column's dropped keys: the layout one
// global sort gives, which the unique-row kernels read.
__global__ __launch_bounds__(kBlock) void cs_compact(const uint32_t *__restrict__ kin,
                                                    const uint32_t *__restrict__ vin,
                                                    uint32_t *__restrict__ kout,
                                                    uint32_t *__restrict__ vout, int64_t n,
                                                    const uint32_t *__restrict__ cstart, int C,
                                                    const uint32_t *__restrict__ vcnt,
                                                    const uint32_t *__restrict__ vbase)
{
    const int64_t p = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (p >= n) return;
    // the column holding p: cstart[lo] <= p < cstart[lo + 1] (an empty column
    // shares its start with the next one, so the last such lo is not empty)
    int lo = 0, hi = C;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)cstart[mid] <= p) lo = mid; else hi = mid;
    }
    const uint32_t c0 = cstart[lo], i = (uint32_t)p - c0, v = vcnt[lo], vb = vbase[lo];
    // dropped keys: after all valid ones, behind the c0 - vb dropped keys of earlier columns
    const uint32_t d = i < v ? vb + i : vbase[C] + (c0 - vb) + (i - v);
    kout[d] = kin[p];
    vout[d] = vin[p];
}

// -------------------------------------------------------------- unique rows

// keys of one 2048-key block, read coalesced into LDS; key[-1] = the key before the block
struct UqLds {
    uint32_t key[kUqTile + 1];
    uint32_t tmp[kWavesPerBlock];
};

__device__ __forceinline__ int uq_stage(UqLds &S, const uint32_t *k, int64_t n,
                                        int64_t base = (int64_t)blockIdx.x * kUqTile)
{
    const int cnt = (int)min<int64_t>(kUqTile, n - base);
    uint32_t x[kUqTile / kBlock];
#pragma unroll
    for (int j = 0; j < kUqTile / kBlock; j++) {
        const int i = j * kBlock + threadIdx.x;
        x[j] = i < cnt ? *gp(k + base + i) : 0u;
    }
    if (threadIdx.x == 0) S.key[0] = base > 0 ? *gp(k + base - 1) : 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < kUqTile / kBlock; j++) {
        const int i = j * kBlock + threadIdx.x;
        if (i < cnt) S.key[i + 1] = x[j];
    }
    __syncthreads();
    return cnt;
}

// a segment head: a valid key that differs from its predecessor
__device__ __forceinline__ bool uq_head(const UqLds &S, int i, uint32_t total_rows, bool first)
{
    const uint32_t x = S.key[i + 1];
    return x < total_rows && (first || S.key[i] != x);
}

__global__ __launch_bounds__(kBlock) void uq_count(const uint32_t *__restrict__ k, int64_t n,
                                                  uint32_t total_rows, uint32_t *__restrict__ ucnt,
                                                  uint32_t *__restrict__ misc)
{
    __shared__ UqLds S;
    const int cnt = uq_stage(S, k, n);
    const int64_t base = (int64_t)blockIdx.x * kUqTile;
    uint32_t c = 0;
    for (int i = threadIdx.x; i < cnt; i += kBlock) {
        const bool first = base + i == 0;
        c += uq_head(S, i, total_rows, first);
        const uint32_t x = S.key[i + 1];
        // the first sentinel key marks the end of the valid contributors
        if (x >= total_rows && (first || S.key[i] < total_rows)) *gp(misc) = (uint32_t)(base + i);
        if (base + i == n - 1 && x < total_rows) *gp(misc) = (uint32_t)n;
    }
    uint32_t ex;
    const uint32_t tot = block_exclusive_scan(c, S.tmp, ex);
    if (threadIdx.x == 0) ucnt[blockIdx.x] = tot;
}

__global__ __launch_bounds__(kBlock) void uq_scan(const uint32_t *__restrict__ ucnt, int64_t nblk,
                                                 uint32_t *__restrict__ uscan,
                                                 uint32_t *__restrict__ misc, int64_t *n_uniq,
                                                 int64_t *stats)
{
    __shared__ uint32_t tmp[kWavesPerBlock];
    uint32_t carry = 0;
    for (int64_t s = 0; s < nblk; s += kBlock) {
        const int64_t i = s + threadIdx.x;
        const uint32_t v = i < nblk ? ucnt[i] : 0u;
        uint32_t ex;
        const uint32_t tot = block_exclusive_scan(v, tmp, ex);
        if (i < nblk) uscan[i] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0) {
        misc[1] = carry;
        if (n_uniq) *n_uniq = carry;
        if (stats) atomicAdd((unsigned long long *)&stats[EMB_STAT_UNIQUE], (unsigned long long)carry);
    }
}

__global__ __launch_bounds__(kBlock) void uq_write(const uint32_t *__restrict__ k, int64_t n,
                                                  uint32_t total_rows,
                                                  const uint32_t *__restrict__ uscan,
                                                  const uint32_t *__restrict__ misc,
                                                  uint32_t *__restrict__ seg,
                                                  uint32_t *__restrict__ ukeys,
                                                  uint32_t *__restrict__ user_keys)
{
    __shared__ UqLds S;
    const int cnt = uq_stage(S, k, n);
    const int64_t base = (int64_t)blockIdx.x * kUqTile;
    // each thread owns kUqItems consecutive keys, so ranks follow key order
    const int i0 = threadIdx.x * kUqItems;
    uint32_t c = 0;
    for (int j = 0; j < kUqItems; j++) {
        const int i = i0 + j;
        if (i < cnt) c += uq_head(S, i, total_rows, base + i == 0);
    }
    uint32_t ex;
    block_exclusive_scan(c, S.tmp, ex);
    uint32_t u = *gp(uscan + blockIdx.x) + ex;
    for (int j = 0; j < kUqItems; j++) {
        const int i = i0 + j;
        if (i < cnt && uq_head(S, i, total_rows, base + i == 0)) {
            const uint32_t x = S.key[i + 1];
            *gp(seg + u) = (uint32_t)(base + i);
            *gp(ukeys + u) = x;
            if (user_keys) *gp(user_keys + u) = x;
            u++;
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) seg[misc[1]] = misc[0];   // seg[U] = valid contributors
}

// The three kernels above in one workgroup, for inputs of at most kUqSmall keys
// (the tiny EMIT step): rounds of kUqTile keys, a running count of heads, and the
// valid count (the first sentinel position, or n) by a block minimum.
constexpr int64_t kUqSmall = 4 * kUqTile;
__global__ __launch_bounds__(kBlock) void uq_small(const uint32_t *__restrict__ k, int64_t n,
                                                  uint32_t total_rows, uint32_t *__restrict__ misc,
                                                  uint32_t *__restrict__ seg,
                                                  uint32_t *__restrict__ ukeys,
                                                  uint32_t *__restrict__ user_keys, int64_t *n_uniq,
                                                  int64_t *stats)
{
    __shared__ UqLds S;
    __shared__ uint32_t first_sent;
    if (threadIdx.x == 0) first_sent = (uint32_t)n;
    uint32_t carry = 0;
    const int i0 = threadIdx.x * kUqItems;
    for (int64_t base = 0; base < n; base += kUqTile) {
        const int cnt = uq_stage(S, k, n, base);
        uint32_t c = 0;
        for (int j = 0; j < kUqItems; j++) {
            const int i = i0 + j;
            if (i < cnt) {
                c += uq_head(S, i, total_rows, base + i == 0);
                const uint32_t x = S.key[i + 1];
                if (x >= total_rows && (base + i == 0 || S.key[i] < total_rows))
                    atomicMin(&first_sent, (uint32_t)(base + i));
            }
        }
        uint32_t ex;
        const uint32_t tot = block_exclusive_scan(c, S.tmp, ex);   // ends with a barrier
        uint32_t u = carry + ex;
        for (int j = 0; j < kUqItems; j++) {
            const int i = i0 + j;
            if (i < cnt && uq_head(S, i, total_rows, base + i == 0)) {
                const uint32_t x = S.key[i + 1];
                *gp(seg + u) = (uint32_t)(base + i);
                *gp(ukeys + u) = x;
                if (user_keys) *gp(user_keys + u) = x;
                u++;
            }
        }
        carry += tot;
        __syncthreads();                         // the staged keys are reused next round
    }
    if (threadIdx.x == 0) {
        misc[0] = first_sent;
        misc[1] = carry;
        seg[carry] = first_sent;                 // seg[U] = valid contributors
        if (n_uniq) *n_uniq = carry;
        if (stats) atomicAdd((unsigned long long *)&stats[EMB_STAT_UNIQUE], (unsigned long long)carry);
    }
}

// ------------------------------------------------------- segment-sum + apply

struct BwdArgs {
    const DevCol *cols;
    const uint32_t *row_base;   // [C + 1]
    int32_t C, B, sumD, maxD, T, opt;
    float lr, eps;
    int64_t ntiles;
    const float *G;
    const uint32_t *sval;       // sorted bags (PW: sorted positions)
    const uint2 *bw;            // PW: (bag, weight bits) of each position
    const int32_t *bag_n;
    const uint32_t *seg;        // [U + 1]
    const uint32_t *ukeys;      // [U]
    const uint32_t *skeys;      // sorted keys (segments found from them when seg is not built)
    const uint32_t *misc;       // [0] = valid contributors, [1] = U
    float *ugrads;              // EMIT output or NULL
    float *part;
    int32_t *pcnt;
    uint32_t *tick;
    int32_t any_mean;           // some column pools by mean
    int32_t all_mean;           // every column pools by mean
    int32_t zero;               // 0, unknown to the compiler: keeps repeated row loads distinct
    uint32_t total_rows;        // keys >= this are dropped / DEFAULT contributors: no row
    int32_t xcd_chunk;          // tile order over the XCDs (0: contiguous ranges)
};

// A segment of at most kSegShort contributors is never cut by a tile boundary:
// the tile holding its start finishes it.  Tiles span at most
// kTileMax + kSegShort - 1 contributors; the sorted keys around the nominal
// range (kKeyWin of them) are staged in LDS to place the boundaries.
constexpr int kSegShort = 64;
constexpr int kSegSpan = kTileMax + kSegShort;
constexpr int kKeyWin = kSegShort + kTileMax + 2 * kSegShort;   // keys [x0 - 64, x0 + 384)
static_assert(kKeyWin % kWave == 0, "key window loads are unrolled per lane");
static_assert(kWave * 4 * sizeof(float) + kOffCap * sizeof(int16_t) <= kKeyWin * sizeof(uint32_t),
              "the pieces and the entries' segment starts fit the key window's space");

struct BwdLds {
    int32_t bag[kSegSpan];      // bag of each contributor of the tile, then of each entry
    float wt[kSegSpan];         // pooling weight of each contributor, then each entry's sum
    union {                     // the keys are read only until the entries are built,
                                // the pieces and the entries' segment starts only after:
                                // sharing keeps a wave at 8 KB of LDS (room for five waves
                                // per SIMD; its registers allow four)
        uint32_t kw[kKeyWin];   // sorted keys x0 - 64 .. x0 + 383 (sentinels outside [0, nv))
        struct {
            float part[kWave][4];
            int16_t eseg[kOffCap];  // first entry of each of the tile's segments (compact_entries)
        };
    };
    uint32_t seg[kOffCap];      // window of segment starts
    uint32_t ukey[kOffCap];     // unique keys of the same segments
    int32_t hseg[kWave], hpass[kWave];
    int32_t njob;                  // segments whose last piece arrived here: summed by the
    int32_t job_u[4], job_c[4];    //   whole wavefront once the walk is done
    int64_t job_k0[4], job_k1[4];
};

struct BTile {
    int64_t k;
    int t0, t1, uf, ul, wb, wn, U;
};

// Segment starts and keys of the segments a tile touches, from its LDS window.
// The window always covers them: it starts at the tile's first segment uf and
// holds kOffCap > kSegSpan entries (or all up to U), while every later
// segment of the tile starts at a distinct contributor inside the tile, so the
// tile needs entries uf .. uf + kSegSpan - 1 at most.  Reading LDS only keeps
// global loads (and the waits they bring) out of the walk.
__device__ __forceinline__ int segat(const BwdArgs &, const BwdLds &L, const BTile &t, int u)
{
    return (int)L.seg[u - t.wb];
}

__device__ __forceinline__ uint32_t ukeyat(const BwdArgs &, const BwdLds &L, const BTile &t, int u)
{
    return L.ukey[u - t.wb];
}

// The walk runs over entries (compact_entries): segment u's first entry in the
// tile, and the segment holding entry e.
__device__ __forceinline__ int esegat(const BwdLds &L, const BTile &t, int u)
{
    return (int)L.eseg[u - t.uf];
}

__device__ __forceinline__ int eseg_of(const BwdLds &L, const BTile &t, int e)
{
    int lo = t.uf, hi = t.ul + 1;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (esegat(L, t, mid) <= e) lo = mid; else hi = mid;
    }
    return lo;
}

// A table row slice (4 elements per lane, raw bits: fp32, or bf16 pairs in w[0..1])
// and its Adagrad accumulator, read when a segment starts so that the update at
// its end does not wait.  Decoding waits for the load, so it happens at the update.
struct RowPre {
    uint32_t w[4];
    float s[4];
};

template <int OPT, bool BF>
__device__ __forceinline__ void row_load(const BwdArgs &a, const DevCol &col, int64_t e, RowPre &r)
{
    if (OPT == EMB_OPT_EMIT) return;
    if (BF) {
        const uint2 raw = *gp(reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(col.weights) + e));
        r.w[0] = raw.x; r.w[1] = raw.y;
    } else {
        const uint4 raw = *gp(reinterpret_cast<const uint4 *>(static_cast<const float *>(col.weights) + e));
        r.w[0] = raw.x; r.w[1] = raw.y; r.w[2] = raw.z; r.w[3] = raw.w;
    }
    if (OPT == EMB_OPT_ADAGRAD) {
        const float4 sv = *gp(reinterpret_cast<const float4 *>(col.state + e));
        r.s[0] = sv.x; r.s[1] = sv.y; r.s[2] = sv.z; r.s[3] = sv.w;
    }
}

template <int OPT, bool BF>
__device__ __forceinline__ void row_landed(const RowPre &r)
{
    if (OPT == EMB_OPT_EMIT) return;
    landed(r.w[0]);
    landed(r.w[1]);
    if (!BF) {
        landed(r.w[2]);
        landed(r.w[3]);
    }
    if (OPT == EMB_OPT_ADAGRAD) landed(make_float4(r.s[0], r.s[1], r.s[2], r.s[3]));
}

// the finished gradient g of unique row u (4 fp32 per lane): emit it, or
// update the row whose old values are in `r`
template <int OPT, bool BF>
__device__ __forceinline__ void row_apply(const BwdArgs &a, const DevCol &col, int u, int64_t e,
                                          const float (&g)[4], RowPre &r, int q)
{
    if (OPT == EMB_OPT_EMIT) {
        if (a.ugrads)
            *gp(reinterpret_cast<float4 *>(a.ugrads + (int64_t)u * a.maxD + q * 4)) =
                make_float4(g[0], g[1], g[2], g[3]);
        return;
    }
    float w[4];
    if (BF) {
        w[0] = bf16_lo(r.w[0]); w[1] = bf16_hi(r.w[0]); w[2] = bf16_lo(r.w[1]); w[3] = bf16_hi(r.w[1]);
    } else {
#pragma unroll
        for (int v = 0; v < 4; v++) w[v] = __uint_as_float(r.w[v]);
    }
    if (OPT == EMB_OPT_SGD) {
#pragma unroll
        for (int v = 0; v < 4; v++) w[v] = w[v] - a.lr * g[v];
    } else {
#pragma unroll
        for (int v = 0; v < 4; v++) {
            r.s[v] = r.s[v] + g[v] * g[v];
            // hardware square root and reciprocal (about 1 ulp each)
            w[v] = w[v] - a.lr * g[v] * __builtin_amdgcn_rcpf(__builtin_amdgcn_sqrtf(r.s[v]) + a.eps);
        }
        *gp(reinterpret_cast<float4 *>(col.state + e)) = make_float4(r.s[0], r.s[1], r.s[2], r.s[3]);
    }
    if (BF) {
        const uint64_t o = (uint64_t)bf16x2_rne(w[0], w[1]) | ((uint64_t)bf16x2_rne(w[2], w[3]) << 32);
        *gp(reinterpret_cast<uint64_t *>(static_cast<uint16_t *>(col.weights) + e)) = o;
    } else {
        *gp(reinterpret_cast<float4 *>(static_cast<float *>(col.weights) + e)) = make_float4(w[0], w[1], w[2], w[3]);
    }
}

// first element of lane slice q of unique row u; the dropped / DEFAULT keys that
// the column sort leaves inside a column point at row 0 (read, never written)
__device__ __forceinline__ int64_t row_elem(const BwdArgs &a, const BwdLds &L, const BTile &t,
                                            const DevCol &col, int u, int q)
{
    const uint32_t k = ukeyat(a, L, t, u);
    return (int64_t)(k < a.total_rows ? k - col.row_base : 0u) * col.dim + q * 4;
}

__device__ __forceinline__ bool seg_live(const BwdArgs &a, const BwdLds &L, const BTile &t, int u)
{
    return ukeyat(a, L, t, u) < a.total_rows;
}

// a segment that finished in another place than where it started: load its
// row now and apply
template <int OPT, bool BF>
__device__ __forceinline__ void seg_out(const BwdArgs &a, const BwdLds &L, const BTile &t,
                                       const DevCol &col, int u, const float (&g)[4], int q, bool qa)
{
    if (!qa) return;
    const int64_t e = row_elem(a, L, t, col, u, q);
    RowPre r;
    row_load<OPT, BF>(a, col, e, r);
    row_apply<OPT, BF>(a, col, u, e, g, r, q);
}

// a piece of a segment that crosses a tile boundary: publish it; the tile whose
// piece arrives last queues the segment for the wavefront-wide combine
__device__ __forceinline__ void bwd_piece(const BwdArgs &a, BwdLds &L, const BTile &t, int c,
                                          int side, int u, const float (&sum)[4], int leader,
                                          int q, bool qa)
{
    const int64_t T = a.T;
    const int ss = segat(a, L, t, u), se = segat(a, L, t, u + 1);
    const int64_t k0 = ss / T, k1 = (se - 1) / T;
    const int64_t slot = t.k * 2 + side;
    if (qa) {
#pragma unroll
        for (int v = 0; v < 4; v++) st_agent(a.part + slot * a.maxD + q * 4 + v, sum[v]);
    }
    wait_vm();                                 // the piece is visible before the ticket
    uint32_t old = 0;
    if (q == 0) old = ticket_add(&a.tick[k0]);
    old = __shfl(old, leader, kWave);
    if (old == (uint32_t)(k1 - k0) && q == 0) {
        const int j = atomicAdd(&L.njob, 1);   // at most two per tile (its first and last segment)
        L.job_u[j] = u;
        L.job_c[j] = c;
        L.job_k0[j] = k0;
        L.job_k1[j] = k1;
    }
}

// Sum the pieces of a queued segment in a fixed order with all 64 lanes: lane
// slice j = lane / P takes pieces j, j + 64/P, ... (several loads in flight per
// lane), then the slices are added by a butterfly over the slice bits.
template <int OPT>
__device__ __forceinline__ void bwd_job(const BwdArgs &a, const BwdLds &L, const BTile &t, int j)
{
    const int u = L.job_u[j], c = uniform(L.job_c[j]);
    const int64_t k0 = L.job_k0[j], k1 = L.job_k1[j];
    const DevCol col = a.cols[c];
    const int P = col.glanes, lp = __ffs(P) - 1;
    const int lane = lane_id(), sl = lane >> lp, q = lane & (P - 1), nsl = kWave >> lp;
    const bool qa = q < col.dim / 4;
    constexpr int UJ = 4;
    float tot[4] = {0.f, 0.f, 0.f, 0.f};
    // piece i = 0 is tile k0's outgoing slot, piece i >= 1 is tile k0+i's incoming slot
    const int64_t npc = k1 - k0 + 1;
    for (int64_t i0 = 0; i0 < npc; i0 += (int64_t)nsl * UJ) {
        float x[UJ][4];
#pragma unroll
        for (int r = 0; r < UJ; r++) {
            const int64_t i = i0 + (int64_t)r * nsl + sl;
            const int64_t slot = i == 0 ? k0 * 2 + 1 : (k0 + i) * 2;
            const bool ok = qa && i < npc;
#pragma unroll
            for (int v = 0; v < 4; v++) x[r][v] = ok ? ld_agent(a.part + slot * a.maxD + q * 4 + v) : 0.f;
        }
#pragma unroll
        for (int r = 0; r < UJ; r++)
#pragma unroll
            for (int v = 0; v < 4; v++) tot[v] += x[r][v];
    }
    for (int o = P; o < kWave; o <<= 1)
#pragma unroll
        for (int v = 0; v < 4; v++) tot[v] += __shfl_xor(tot[v], o, kWave);
    if (sl == 0) {
        if (col.dtype == EMB_BF16) seg_out<OPT, true>(a, L, t, col, u, tot, q, qa);
        else seg_out<OPT, false>(a, L, t, col, u, tot, q, qa);
    }
    if (lane == 0) st_agent(&a.tick[k0], 0u);  // ready for the next call
}

// one column run [s0, s1) of the tile's entries; P lanes per gradient row.
// DENSE (most entries start a segment): the rows of the entries' segments are
// loaded with the gradient slices.  Otherwise (long segments, the hot rows of a
// skewed column) the walk loads gradient slices only, and a segment that ends
// inside the run loads its row when it ends (a wait, but a rare one).
template <int OPT, bool BF, bool DENSE>
__device__ __forceinline__ void bwd_segment(const BwdArgs &a, BwdLds &L, const BTile &t,
                                            const DevCol &col, int c, int s0, int s1)
{
    constexpr int U = 4;
    const int P = col.glanes, lp = __ffs(P) - 1;
    const int G = kWave >> lp;
    const int lane = lane_id(), g = lane >> lp, q = lane & (P - 1);
    const bool qa = q < col.dim / 4;
    const int len = s1 - s0, Lg = (len + G - 1) / G;
    const int ga = min(s0 + g * Lg, s1), ge = min(ga + Lg, s1);
    const int cB = c * a.B;

    float acc[4] = {0.f, 0.f, 0.f, 0.f}, hacc[4] = {0.f, 0.f, 0.f, 0.f};
    int hseg = -1, tseg = -1;
    bool hpass = false;
    if (ga < ge) {
        int u = eseg_of(L, t, ga);
        int uend = esegat(L, t, u + 1);
        bool before = esegat(L, t, u) < ga;
        // Row loads are issued for every entry, unconditionally: the row of the
        // segment holding it (lanes past the row's end read lane 0's slice), used
        // only where a segment starts.  Loads that are always issued keep the
        // compiler's wait counts exact; conditional ones made it wait for every
        // earlier load before issuing the next.  Repeats of a row hit in cache.
        const int qq = qa ? q : 0;
        RowPre cur;
        if (DENSE) row_load<OPT, BF>(a, col, row_elem(a, L, t, col, u, qq), cur);
        int64_t e = row_elem(a, L, t, col, u, qq);
        const float *gq = a.G + col.out_off + qq * 4;
        for (int p = ga; p < ge; p += U) {
            // one batch: the rows of its contributors' segments, then U gradient
            // slices, all in flight together
            float4 x[U];
            float wt[U];
            bool st[U];
            RowPre pre[U];
            int ue = uend, ns = 0;
#pragma unroll
            for (int j = 0; j < U; j++) {
                st[j] = p + j < ge && p + j == ue;
                if (st[j]) {
                    ns++;
                    ue = esegat(L, t, u + ns + 1);   // end of segment u + ns
                }
                // a.zero stops the compiler from merging repeats of one row into
                // register copies, which would wait for the load
                if (DENSE)
                    row_load<OPT, BF>(a, col, row_elem(a, L, t, col, u + ns, qq) + (int64_t)j * a.zero, pre[j]);
            }
#pragma unroll
            for (int j = 0; j < U; j++) {
                const int pl = min(p + j, ge - 1);
                wt[j] = p + j < ge ? L.wt[pl] : 0.f;
                x[j] = *gp(reinterpret_cast<const float4 *>(gq + (int64_t)(L.bag[pl] - cB) * a.sumD));
            }
            // every load of the batch lands before the row stores below
            if (DENSE) {
#pragma unroll
                for (int j = 0; j < U; j++) row_landed<OPT, BF>(pre[j]);
            }
#pragma unroll
            for (int j = 0; j < U; j++) landed(x[j]);
#pragma unroll
            for (int j = 0; j < U; j++) {
                if (p + j < ge) {
                    if (st[j]) {                   // segment u ended just before p + j
                        if (before) {
#pragma unroll
                            for (int v = 0; v < 4; v++) hacc[v] = acc[v];
                            hseg = u; hpass = false;
                        } else if (qa && seg_live(a, L, t, u)) {
                            if (DENSE) row_apply<OPT, BF>(a, col, u, e, acc, cur, q);
                            else seg_out<OPT, BF>(a, L, t, col, u, acc, q, qa);
                        }
#pragma unroll
                        for (int v = 0; v < 4; v++) acc[v] = 0.f;
                        u++;
                        before = false;
                        if (DENSE) cur = pre[j];
                        e = row_elem(a, L, t, col, u, qq);
                    }
                    acc[0] += wt[j] * x[j].x;
                    acc[1] += wt[j] * x[j].y;
                    acc[2] += wt[j] * x[j].z;
                    acc[3] += wt[j] * x[j].w;
                }
            }
            uend = ue;
        }
        if (uend == ge) {
            if (before) {
#pragma unroll
                for (int v = 0; v < 4; v++) hacc[v] = acc[v];
                hseg = u; hpass = false;
            } else if (qa && seg_live(a, L, t, u)) {
                if (DENSE) row_apply<OPT, BF>(a, col, u, e, acc, cur, q);
                else seg_out<OPT, BF>(a, L, t, col, u, acc, q, qa);
            }
        } else if (before) {
#pragma unroll
            for (int v = 0; v < 4; v++) hacc[v] = acc[v];
            hseg = u; hpass = true;
        } else {
            tseg = u;
        }
    }
#pragma unroll
    for (int v = 0; v < 4; v++) L.part[lane][v] = hacc[v];
    if (q == 0) {
        L.hseg[g] = hseg; L.hpass[g] = hpass;
    }
    wave_sync();
    if (tseg >= 0) {
        float sum[4] = {acc[0], acc[1], acc[2], acc[3]};
        bool ended = false;
        for (int g2 = g + 1; g2 < G; g2++) {
            if (L.hseg[g2] != tseg) break;
#pragma unroll
            for (int v = 0; v < 4; v++) sum[v] += L.part[g2 * P + q][v];
            if (!L.hpass[g2]) { ended = true; break; }
        }
        if (!seg_live(a, L, t, tseg)) {
            // dropped / DEFAULT contributors: nothing to update
        } else if (ended) {
            seg_out<OPT, BF>(a, L, t, col, tseg, sum, q, qa);
        } else {
            bwd_piece(a, L, t, c, 1, tseg, sum, g * P, q, qa);
        }
    }
    if (g == 0 && hseg >= 0) {
        float sum[4] = {hacc[0], hacc[1], hacc[2], hacc[3]};
        bool pass = hpass;
        for (int g2 = 1; pass && g2 < G; g2++) {
            if (L.hseg[g2] != hseg) break;
#pragma unroll
            for (int v = 0; v < 4; v++) sum[v] += L.part[g2 * P + q][v];
            pass = L.hpass[g2];
        }
        if (seg_live(a, L, t, hseg)) bwd_piece(a, L, t, c, 0, hseg, sum, 0, q, qa);
    }
    wave_sync();
}

// The two ends of the runs that cross a tile's edges, searched together: the
// start of the run of k0 that holds t0 - 1 (the keys before the run are smaller,
// or at least hi: dropped / DEFAULT keys the column sort left at the end of
// earlier columns) and the end of the run of kl that holds t1 (the keys after it
// are larger).  Each search first gallops away from the tile over multiples of
// the step, 64 probes per round, the step starting at the nominal tile size T
// and growing 64-fold while all 64 probes stay in the run; then 64-ary rounds
// narrow the bracket that the gallop found (at most one step wide) down to the
// answer.  The gallop's probes are multiples of T, so every tile of a long run
// reads the same few lines, and the narrowing rounds read the lines around the
// run's ends, again shared by those tiles.  (A 64-ary search over the whole key
// range put every round's probes on different lines for every tile: about
// 0.24 GB of reads per long-sequence apply.)  Both searches advance together, so
// a tile waits for the longer one only.
__device__ __forceinline__ void run_bounds(const uint32_t *key, bool need_s, int64_t t0, uint32_t k0,
                                           uint32_t hi, bool need_e, int64_t t1, int64_t nv,
                                           uint32_t kl, int64_t T, int64_t &start, int64_t &end)
{
    const int l = lane_id();
    // phase per side: 0 gallop, 1 narrow, 2 done
    int pa = need_s ? 0 : 2, pb = need_e ? 0 : 2;
    // A: while galloping, inA holds k0; then the start is in [loA, upA]
    int64_t inA = t0 - 1, sA = T, loA = 0, upA = 0;
    // B: while galloping, inB holds kl; then the end (first index past the run) is in [loB, upB]
    int64_t inB = t1, sB = T, loB = t1, upB = t1;
    start = t0;
    end = t1;
    while (pa < 2 || pb < 2) {
        int64_t iA = -1, iB = nv, stA = 1, stB = 1, baseA = 0, baseB = 0;
        if (pa == 0) {
            baseA = inA / sA * sA;
            iA = baseA - (int64_t)l * sA;
        } else if (pa == 1) {
            stA = upA - loA > 64 ? (upA - loA + 63) / 64 : 1;
            iA = loA + (int64_t)l * stA;
        }
        if (pb == 0) {
            baseB = (inB / sB + 1) * sB;
            iB = baseB + (int64_t)l * sB;
        } else if (pb == 1) {
            stB = upB - loB > 64 ? (upB - loB + 63) / 64 : 1;
            iB = loB + (int64_t)l * stB;
        }
        const bool okA = (pa == 0 && iA >= 0) || (pa == 1 && iA < upA);
        const bool okB = (pb == 0 && iB < nv) || (pb == 1 && iB < upB);
        const uint32_t vA = okA ? *gp(key + iA) : 0u;
        const uint32_t vB = okB ? *gp(key + iB) : 0xFFFFFFFFu;
        const bool runA = okA && vA >= k0 && vA < hi;      // holds k0
        const bool runB = okB && vB <= kl;                 // holds kl
        const int inRunA = __popcll(__ballot(runA));       // a prefix of the lanes while galloping
        const int outA = __popcll(__ballot(okA && !runA)); // a prefix of the lanes while narrowing
        const int inRunB = __popcll(__ballot(runB));       // a prefix of the lanes in both phases
        if (pa == 0) {
            if (inRunA == kWave) {
                inA = baseA - (int64_t)(kWave - 1) * sA;
                sA *= kWave;
            } else {
                upA = inRunA > 0 ? baseA - (int64_t)(inRunA - 1) * sA : inA;
                const int64_t out = baseA - (int64_t)inRunA * sA;     // outside the run, or < 0
                loA = out + 1 > 0 ? out + 1 : 0;
                pa = 1;
            }
        } else if (pa == 1) {
            if (stA == 1 || outA == 0) {
                start = loA + (stA == 1 ? outA : 0);
                pa = 2;
            } else {
                const int64_t nu = loA + (int64_t)outA * stA < upA ? loA + (int64_t)outA * stA : upA;
                loA = loA + (int64_t)(outA - 1) * stA + 1;
                upA = nu;
            }
        }
        if (pb == 0) {
            if (inRunB == kWave) {
                inB = baseB + (int64_t)(kWave - 1) * sB;
                sB *= kWave;
            } else {
                loB = (inRunB > 0 ? baseB + (int64_t)(inRunB - 1) * sB : inB) + 1;
                const int64_t out = baseB + (int64_t)inRunB * sB;     // outside the run, or >= nv
                upB = out < nv ? out : nv;
                pb = 1;
            }
        } else if (pb == 1) {
            if (stB == 1 || inRunB == 0) {
                end = loB + (stB == 1 ? inRunB : 0);
                pb = 2;
            } else {
                const int64_t nu = loB + (int64_t)inRunB * stB < upB ? loB + (int64_t)inRunB * stB : upB;
                loB = loB + (int64_t)(inRunB - 1) * stB + 1;
                upB = nu;
            }
        }
    }
}

// The segments of tile t from the sorted keys, without a unique list: heads
// (positions whose key differs from the previous one) are compacted into the
// window in position order; a first segment that began in an earlier tile, or
// a last one that goes on into a later tile, gets its true start / end from a
// search of the sorted keys.  Window indices are then local (wb = 0).
__device__ __forceinline__ void seg_window_from_keys(const BwdArgs &a, BwdLds &L, BTile &t, int nv, int x0)
{
    constexpr int kPL = kSegSpan / kWave;
    const int lane = lane_id();
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int kb = x0 - kSegShort;                 // position of L.kw[0]
    int base = 0;
#pragma unroll
    for (int i = 0; i < kPL; i++) {
        const int p = t.t0 + lane + kWave * i;
        const bool head = p < t.t1 && (p == t.t0 || L.kw[p - 1 - kb] != L.kw[p - kb]);
        const uint64_t m = __ballot(head);
        if (head) {
            const int j = base + __popcll(m & lt_mask);
            L.seg[j] = (uint32_t)p;
            L.ukey[j] = L.kw[p - kb];
        }
        base += __popcll(m);
    }
    wave_sync();
    const int nseg = base;
    const uint32_t k0 = L.ukey[0], kl = L.ukey[nseg - 1];
    const uint32_t kprev = t.t0 > 0 ? L.kw[t.t0 - 1 - kb] : 0xFFFFFFFFu;
    const uint32_t knext = t.t1 < nv ? L.kw[t.t1 - kb] : 0xFFFFFFFFu;
    int start = t.t0, end = t.t1;
    // only a long segment crosses a tile boundary: its ends come from a search.
    // Keys before the run are smaller, or dropped / DEFAULT keys (>= total_rows)
    // that the column sort left at the end of earlier columns.
    if (kprev == k0 || knext == kl) {
        int64_t s64, e64;
        run_bounds(a.skeys, kprev == k0, (int64_t)t.t0, k0, a.total_rows, knext == kl, (int64_t)t.t1,
                   (int64_t)nv, kl, (int64_t)a.T, s64, e64);
        if (kprev == k0) start = (int)s64;
        if (knext == kl) end = (int)e64;
    }
    if (lane == 0) {
        L.seg[0] = (uint32_t)start;
        L.seg[nseg] = (uint32_t)end;
    }
    wave_sync();
    t.wb = 0;
    t.wn = nseg + 1;
    t.uf = 0;
    t.ul = nseg - 1;
}

// Entries: the tile's contributors [t0, t1) merged into maximal runs of one
// segment (one row) and one bag.  The stable sort keeps such runs together,
// and every contribution in one carries the same gradient slice G[bag], so the
// walk reads that slice once, times the run's summed weight (w times the run
// length when the weight is the bag's pooling weight; the sum of the
// per-position weights otherwise, added in contributor order).  In a long
// sequence a hot row repeats inside a bag many times over.  L.bag / L.wt are
// rewritten in place with the entries, and L.eseg[s] gets the first entry of the
// tile's s-th segment (t.uf + s): -1 when that segment began before the tile,
// and at s = nseg the entry count E, or E + 1 when the last segment goes on past
// the tile (so the walk does not take it as finished).  Returns E.
template <bool PW>
__device__ __forceinline__ int compact_entries(BwdLds &L, const BTile &t, int x0)
{
    constexpr int kPL = kSegSpan / kWave;
    const int lane = lane_id();
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int kb = x0 - kSegShort;                 // position of L.kw[0]
    const int len = t.t1 - t.t0;                   // 1 .. kSegSpan
    int bg[kPL];
    float ws[kPL];
    uint64_t hm[kPL], sm[kPL];
    // heads of entries (hm) and of segments (sm), by ballot
#pragma unroll
    for (int i = 0; i < kPL; i++) {
        const int idx = lane + kWave * i;
        const bool in = idx < len;
        const int j = min(idx, len - 1);
        const int p = t.t0 + j;
        bg[i] = L.bag[j];
        const bool sf = in && (idx == 0 || L.kw[p - kb] != L.kw[p - 1 - kb]);
        const bool hd = in && (sf || bg[i] != L.bag[max(j - 1, 0)]);
        hm[i] = __ballot(hd);
        sm[i] = __ballot(sf);
    }
    // each head's summed weight, up to the next head (the masks are uniform)
#pragma unroll
    for (int i = 0; i < kPL; i++) {
        const int idx = lane + kWave * i;
        ws[i] = 0.f;
        if ((hm[i] >> lane) & 1ull) {
            const uint64_t rest = lane < kWave - 1 ? hm[i] >> (lane + 1) : 0ull;
            int nxt = len;
            if (rest) {
                nxt = idx + __ffsll((unsigned long long)rest);
            } else {
#pragma unroll
                for (int k = kPL - 1; k > i; k--)
                    if (hm[k]) nxt = kWave * k + __ffsll((unsigned long long)hm[k]) - 1;
            }
            if (PW) {
                float w = 0.f;
                for (int k = idx; k < nxt; k++) w += L.wt[k];
                ws[i] = w;
            } else {
                ws[i] = L.wt[idx] * (float)(nxt - idx);
            }
        }
    }
    wave_sync();                                   // every read above precedes the writes
    int E = 0, S = 0;
#pragma unroll
    for (int i = 0; i < kPL; i++) {
        const int e = E + __popcll(hm[i] & lt_mask), sl = S + __popcll(sm[i] & lt_mask);
        if ((hm[i] >> lane) & 1ull) {
            L.bag[e] = bg[i];
            L.wt[e] = ws[i];
        }
        if ((sm[i] >> lane) & 1ull) L.eseg[sl] = (int16_t)e;
        E += __popcll(hm[i]);
        S += __popcll(sm[i]);
    }
    wave_sync();
    if (lane == 0) {
        if ((int)L.seg[t.uf - t.wb] < t.t0) L.eseg[0] = -1;
        L.eseg[S] = (int16_t)((int)L.seg[t.ul + 1 - t.wb] == t.t1 ? E : E + 1);
    }
    wave_sync();
    return E;
}

// Where a tile boundary lands: the nominal boundary x, or the end of the short
// segment (run of equal sorted keys) that x cuts.  The run is measured inside
// the staged keys x - 64 .. x + 63; a run reaching either edge counts as long.
// Tiles on both sides of x evaluate this on the same keys, so they agree.
__device__ __forceinline__ int seg_boundary(const BwdLds &L, int x, int x0, int nv, int T)
{
    if (x <= 0 || x >= nv) return x;
    const int lane = lane_id();
    const int kb = x0 - kSegShort;
    const uint32_t kx = L.kw[x - kb];
    const uint32_t lo = L.kw[x - kSegShort + lane - kb];   // keys x-64 .. x-1
    const uint32_t hi = L.kw[x + lane - kb];               // keys x .. x+63
    const bool lo_in = x - kSegShort + lane >= 0;
    // equal keys are adjacent: the run is a suffix of the keys below x and a
    // prefix of those from x
    const int before = __popcll(__ballot(lo_in && lo == kx));
    const int same = __popcll(__ballot(x + lane < nv && hi == kx));
    const int ss = x - before, se = x + same;
    const bool touches = (before == kSegShort) || same == kSegShort;
    if (ss < x && !touches && se - ss <= kSegShort && se < min(x + T, nv)) return se;
    return x;
}

// PW: the forward had per-position weights; the sort then carried positions, and
// each contributor's bag and weight are read through its position
template <int OPT, bool KM, bool PW>
__global__ __launch_bounds__(kTileBlock, 4) void seg_apply(BwdArgs a)
{
    __shared__ BwdLds lds[kTileWaves];
    const int w = threadIdx.x / kWave, lane = lane_id();
    BwdLds &L = lds[w];
    BTile t;
    t.k = xcd_block(blockIdx.x, gridDim.x, a.xcd_chunk) * kTileWaves + w;
    if (t.k >= a.ntiles) return;
    const int nv = (int)*gp(a.misc);
    const int x0 = (int)min<int64_t>(t.k * a.T, nv), x1 = (int)min<int64_t>((t.k + 1) * a.T, nv);
    if (x0 >= x1) return;

    // the sorted keys around the nominal range, and the bags of its contributors
    // and of the short segment that may extend it, all loaded in one round
    constexpr int kPL = kSegSpan / kWave;
    int bagr[kPL], nr[kPL];
    // (loads at clamped indices, issued by every lane: a load inside a per-lane
    // branch makes the compiler wait for it before the next one)
#pragma unroll
    for (int i = 0; i < kPL; i++) {
        const int p = x0 + lane + kWave * i;
        const int v = (int)*gp(a.sval + min(p, nv - 1));
        bagr[i] = p < nv ? v : 0;
    }
    {
        uint32_t kv[kKeyWin / kWave];
#pragma unroll
        for (int j = 0; j < kKeyWin / kWave; j++) {
            const int p = x0 - kSegShort + lane + kWave * j;
            const uint32_t v = *gp(a.skeys + min(max(p, 0), nv - 1));
            kv[j] = (p >= 0 && p < nv) ? v : (p < 0 ? 0u : 0xFFFFFFFFu);
        }
#pragma unroll
        for (int j = 0; j < kKeyWin / kWave; j++) L.kw[lane + kWave * j] = kv[j];
    }
    float vw[kPL];
    if (PW) {
        // bagr holds positions here (< N: the sorted entries are positions)
#pragma unroll
        for (int i = 0; i < kPL; i++) {
            const uint2 r = *gp(a.bw + bagr[i]);
            bagr[i] = (int)r.x;
            vw[i] = __uint_as_float(r.y);
        }
        // the mean weight is folded in here, per contributor's column (a lookup
        // of its pooling only when the plan mixes sum and mean columns)
#pragma unroll
        for (int i = 0; i < kPL; i++) {
            const bool mean = a.all_mean ? true : (a.any_mean ? *gp(&a.cols[bagr[i] / a.B].pool) == EMB_POOL_MEAN : false);
            nr[i] = mean ? max(*gp(a.bag_n + bagr[i]), 1) : 1;
        }
    } else if (a.any_mean) {
        // the mean weight of each contributor's bag; a plan that mixes sum and
        // mean columns looks up the pooling of the contributor's column (both
        // loads depend only on the bag, so they go out together).  A bag with no
        // valid position reaches here only through its default row's entry,
        // whose weight is 1.
#pragma unroll
        for (int i = 0; i < kPL; i++) {
            const bool mean = a.all_mean ? true : *gp(&a.cols[bagr[i] / a.B].pool) == EMB_POOL_MEAN;
            nr[i] = mean ? max(*gp(a.bag_n + bagr[i]), 1) : 1;
        }
    } else {
#pragma unroll
        for (int i = 0; i < kPL; i++) nr[i] = 1;
    }
    wave_sync();
    t.t0 = seg_boundary(L, x0, x0, nv, a.T);
    t.t1 = seg_boundary(L, x1, x0, nv, a.T);

    if (KM) {
        seg_window_from_keys(a, L, t, nv, x0);
    } else {
        const int U = (int)*gp(a.misc + 1);
        t.U = U;
        t.uf = (int)wave_upper_bound(a.seg, (int64_t)U + 1, (uint32_t)t.t0) - 1;
        t.wb = t.uf;
        t.wn = min(U + 1 - t.uf, kOffCap);
        {
            // all window loads in flight at once
            uint32_t sg[kOffCap / kWave], uk[kOffCap / kWave];
#pragma unroll
            for (int j = 0; j < kOffCap / kWave; j++) {
                const int i = lane + kWave * j;
                sg[j] = i < t.wn ? *gp(a.seg + t.wb + i) : 0u;
                uk[j] = (i < t.wn && t.wb + i < U) ? *gp(a.ukeys + t.wb + i) : 0xFFFFFFFFu;
            }
#pragma unroll
            for (int j = 0; j < kOffCap / kWave; j++) {
                const int i = lane + kWave * j;
                if (i < t.wn) {
                    L.seg[i] = sg[j];
                    L.ukey[i] = uk[j];
                }
            }
        }
        wave_sync();
        if (L.seg[t.wn - 1] > (uint32_t)(t.t1 - 1))
            t.ul = t.uf + (int)wave_upper_bound(L.seg, (int64_t)t.wn, (uint32_t)(t.t1 - 1)) - 1;
        else
            t.ul = (int)wave_upper_bound(a.seg, (int64_t)U + 1, (uint32_t)(t.t1 - 1)) - 1;
    }
#pragma unroll
    for (int i = 0; i < kPL; i++) {
        const int p = x0 + lane + kWave * i;
        if (p >= t.t0 && p < t.t1) {
            L.bag[p - t.t0] = bagr[i];
            // pooling weight: 1 / n for a mean bag, 1 for a sum bag (PW: times the
            // contributor's own weight)
            L.wt[p - t.t0] = PW ? vw[i] * __builtin_amdgcn_rcpf((float)nr[i])
                                : __builtin_amdgcn_rcpf((float)nr[i]);
        }
    }
    if (lane == 0) L.njob = 0;
    wave_sync();
    const int ne = compact_entries<PW>(L, t, x0);
    // column runs: entries are sorted by (column, row), and bag / B is the column
    int p = 0;
    while (p < ne) {
        const int c = uniform(L.bag[p] / a.B);
        const int lim = (c + 1) * a.B;
        int lo = p, hi = ne;            // first entry of a later column
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (L.bag[mid] < lim) lo = mid + 1; else hi = mid;
        }
        const int s1 = uniform(lo);
        const DevCol col = a.cols[c];
        // the dense walk where segments average fewer than 8 entries (measured:
        // with 4, short-segment runs of the training front end lost 6 % to the
        // waits of the gradient-only walk; always dense, long sequences lost 6 %)
        const bool dense = s1 - p < 8 * (eseg_of(L, t, s1 - 1) - eseg_of(L, t, p) + 1);
        if (col.dtype == EMB_BF16) {
            if (dense) bwd_segment<OPT, true, true>(a, L, t, col, c, p, s1);
            else bwd_segment<OPT, true, false>(a, L, t, col, c, p, s1);
        } else {
            if (dense) bwd_segment<OPT, false, true>(a, L, t, col, c, p, s1);
            else bwd_segment<OPT, false, false>(a, L, t, col, c, p, s1);
        }
        p = s1;
    }
    wave_sync();
    const int nj = uniform(L.njob);
    for (int j = 0; j < nj; j++) bwd_job<OPT>(a, L, t, j);
}

// ------------------------------------------ atomic scatter (RecIS's backward)
//
// The pages' own backward (RecIS Sec. 3.2, Algorithm 1, backward half) sends
// each contribution w_r G[s(r), :] to its row with atomic adds instead of
// grouping contributors by a sort.  For SGD the update is linear, so every
// contribution can be applied to the row directly: E[u] -= lr w_r G[s(r), :].
// Positions are taken in forward order (so G slices are read nearly in order),
// 4 per lane group in flight; contributions of the same row within one batch of
// a group are merged first.  The rounding depends on the order of the atomic
// adds, so results are not bit-reproducible (they agree within the sum of
// |terms| bound used for the sorted path).
struct AtomArgs {
    const DevCol *cols;
    int32_t C, B, sumD, T;
    float lr;
    int64_t n, ntiles;
    const float *G;
    const uint32_t *keys;       // forward: row key per position (>= total_rows: no row)
    const int32_t *bags;        // forward: bag per position
    const int32_t *bag_n;
    const uint32_t *cstart;     // forward: first position of each column [C + 1]
    const uint2 *bw;            // forward: (bag, weight bits) of each position, or NULL
    uint32_t total_rows;
};

__global__ __launch_bounds__(kTileBlock, 4) void atomic_apply(AtomArgs a)
{
    const int lane = lane_id();
    const int64_t k = (int64_t)blockIdx.x;
    if (k >= a.ntiles) return;
    const int x0 = (int)(k * a.T), x1 = (int)min<int64_t>((k + 1) * a.T, a.n);
    // the columns of this tile: the last column starting at or before x0, then on
    int c = (int)wave_upper_bound(a.cstart, (int64_t)a.C + 1, (uint32_t)x0) - 1;
    int p = x0;
    while (p < x1) {
        c = uniform(c);
        const int cend = min(x1, (int)*gp(a.cstart + c + 1));
        if (cend <= p) { c++; continue; }
        const DevCol col = a.cols[c];
        const int P = col.glanes, lp = __ffs(P) - 1, G = kWave >> lp;
        const int g = lane >> lp, q = lane & (P - 1);
        const bool qa = q < col.dim / 4;
        const int qq = qa ? q : 0;
        const bool mean = col.pool == EMB_POOL_MEAN;
        float *w = static_cast<float *>(col.weights);
        const float *gq = a.G + col.out_off + qq * 4;
        const int cB = c * a.B;
        constexpr int U = 4;
        // group g takes positions p + g, p + g + G, ...: consecutive groups read
        // consecutive keys and bags
        for (int b0 = p; b0 < cend; b0 += G * U) {
            uint32_t key[U];
            int bag[U], nb[U];
            float4 x[U];
            float vw[U];
#pragma unroll
            for (int j = 0; j < U; j++) {
                const int pp = min(b0 + j * G + g, cend - 1);
                key[j] = b0 + j * G + g < cend ? *gp(a.keys + pp) : a.total_rows;
                bag[j] = *gp(a.bags + pp);
                vw[j] = a.bw ? __uint_as_float((*gp(a.bw + pp)).y) : 1.0f;
            }
#pragma unroll
            for (int j = 0; j < U; j++) {
                nb[j] = mean ? *gp(a.bag_n + bag[j]) : 1;
                x[j] = *gp(reinterpret_cast<const float4 *>(gq + (int64_t)(bag[j] - cB) * a.sumD));
            }
            // merge repeats of one row inside the lane group's batch
            float s[U][4];
#pragma unroll
            for (int j = 0; j < U; j++) {
                const float wt = (mean ? __builtin_amdgcn_rcpf((float)nb[j]) : 1.0f) * vw[j] * -a.lr;
                s[j][0] = wt * x[j].x; s[j][1] = wt * x[j].y; s[j][2] = wt * x[j].z; s[j][3] = wt * x[j].w;
            }
#pragma unroll
            for (int j = 1; j < U; j++) {
#pragma unroll
                for (int i = 0; i < j; i++) {
                    if (key[i] == key[j]) {
#pragma unroll
                        for (int v = 0; v < 4; v++) { s[i][v] += s[j][v]; s[j][v] = 0.f; }
                        key[j] = a.total_rows;     // merged: nothing left to send
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < U; j++) {
                if (qa && key[j] < a.total_rows) {
                    float *dst = w + (int64_t)(key[j] - col.row_base) * col.dim + q * 4;
#pragma unroll
                    for (int v = 0; v < 4; v++) __builtin_amdgcn_global_atomic_fadd_f32(gp(dst + v), s[j][v]);
                }
            }
        }
        p = cend;
        c++;
    }
}

}  // namespace emb

using namespace emb;

static emb_status bwd_check(emb_plan *plan, void *workspace)
{
    if (!plan || !workspace) return fail(EMB_ERR_INVALID_ARG, "plan and workspace are required");
    if (!aligned(workspace, 256)) return fail(EMB_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    if (plan->last_n < 0) return fail(EMB_ERR_INVALID_ARG, "no training forward ran on this plan");
    return EMB_OK;
}

template <bool PW>
static void launch_apply(const emb_plan *plan, const BwdArgs &a, dim3 grid, dim3 block, hipStream_t st)
{
    if (a.opt == EMB_OPT_EMIT)
        hipLaunchKernelGGL((seg_apply<EMB_OPT_EMIT, false, PW>), grid, block, 0, st, a);
    else if (a.opt == EMB_OPT_SGD && plan->seg_from_keys)
        hipLaunchKernelGGL((seg_apply<EMB_OPT_SGD, true, PW>), grid, block, 0, st, a);
    else if (a.opt == EMB_OPT_SGD)
        hipLaunchKernelGGL((seg_apply<EMB_OPT_SGD, false, PW>), grid, block, 0, st, a);
    else if (plan->seg_from_keys)
        hipLaunchKernelGGL((seg_apply<EMB_OPT_ADAGRAD, true, PW>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((seg_apply<EMB_OPT_ADAGRAD, false, PW>), grid, block, 0, st, a);
}

// entries the backward sorts: the positions of the last training forward, plus
// one per bag when a column has a default row
static int64_t sort_n(const emb_plan *plan)
{
    return plan->last_n + (plan->has_default ? (int64_t)plan->n_cols * plan->batch : 0);
}

static int sort_passes(const emb_plan *plan) { return (plan->key_bits + kRadixBits - 1) / kRadixBits; }

extern "C" emb_status emb_backward_dedup(emb_plan *plan, void *workspace, uint32_t *uniq_keys,
                                         int64_t *n_uniq, int64_t *stats, void *stream)
{
    emb_status s = bwd_check(plan, workspace);
    if (s != EMB_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    const int64_t n = sort_n(plan);
    const WsLayout &W = plan->ws;
    uint32_t *k0 = reinterpret_cast<uint32_t *>(ws + W.keys);
    // the sort's values: the bag of each position, or with per-position weights
    // the position itself (the apply then reads bag and weight through it)
    uint32_t *v0 = reinterpret_cast<uint32_t *>(ws + (plan->last_weighted ? W.posid : W.bags));
    uint32_t *k1 = reinterpret_cast<uint32_t *>(ws + W.keys2);
    uint32_t *v1 = reinterpret_cast<uint32_t *>(ws + W.vals2);
    uint32_t *hist = reinterpret_cast<uint32_t *>(ws + W.hist);
    uint32_t *dtot = reinterpret_cast<uint32_t *>(ws + W.dtot);
    uint32_t *misc = reinterpret_cast<uint32_t *>(ws + W.misc);
    uint32_t *ucnt = reinterpret_cast<uint32_t *>(ws + W.ucnt);
    uint32_t *uscan = reinterpret_cast<uint32_t *>(ws + W.uscan);
    uint32_t *seg = reinterpret_cast<uint32_t *>(ws + W.seg);
    uint32_t *ukeys = reinterpret_cast<uint32_t *>(ws + W.ukeys);
    const int64_t nblk = std::max<int64_t>(1, (n + kSortTile - 1) / kSortTile);
    const int64_t ublk = std::max<int64_t>(1, (n + kUqTile - 1) / kUqTile);
    if (n == 0) {
        hipError_t e = n_uniq ? hipMemsetAsync(n_uniq, 0, sizeof(int64_t), st) : hipSuccess;
        if (e != hipSuccess) return fail(EMB_ERR_HIP, std::string("backward: ") + hipGetErrorString(e));
        return EMB_OK;
    }
    // Without an EMIT optimizer and with nothing asked about the unique rows, the
    // apply kernel finds segments in the sorted keys itself and the unique-list
    // kernels are skipped.
    const bool from_keys = plan->opt != EMB_OPT_EMIT && !uniq_keys && !n_uniq && !stats;
    plan->seg_from_keys = from_keys;
    const int passes = sort_passes(plan);
    // the sorted keys and values end in the buffers the apply reads them from
    uint32_t *kf = (passes % 2) ? k1 : k0, *vf = (passes % 2) ? v1 : v0;
    // The column sort runs when the average column fits its LDS (n <= C * kColCap;
    // a larger column is sorted by its workgroup through global memory); it
    // leaves dropped keys inside each column.  Segments found from the keys take
    // that as it is.  The unique list needs one sorted run of valid keys: the
    // columns are then sorted into the other buffers and compacted into kf / vf.
    // Otherwise the global radix passes sort everything; they also take the
    // default-row entries, which sit after the N positions.
    if (!plan->has_default && n <= (int64_t)plan->n_cols * kColCap) {
        const uint32_t *cst = reinterpret_cast<const uint32_t *>(ws + W.cstart);
        uint32_t *kc = from_keys ? kf : (kf == k0 ? k1 : k0);
        uint32_t *vc = from_keys ? vf : (vf == v0 ? v1 : v0);
        // valid counts [C + 1], their prefix [C + 1] (written by col_sort's last column), a ticket
        uint32_t *vcnt = reinterpret_cast<uint32_t *>(ws + W.ccnt), *vbase = vcnt + plan->n_cols + 1;
        hipLaunchKernelGGL(col_sort, dim3((unsigned)plan->n_cols), dim3(kCSBlock), 0, st, k0, v0, k1, v1,
                           kc, vc, n, cst, plan->drow_base, plan->total_rows, misc,
                           from_keys ? nullptr : vcnt);
        if (!from_keys) {
            hipLaunchKernelGGL(cs_compact, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock), 0, st,
                               kc, vc, kf, vf, n, cst, plan->n_cols, vcnt, vbase);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(EMB_ERR_HIP, std::string("col_sort launch: ") + hipGetErrorString(e));
        if (from_keys) return EMB_OK;
    } else {
        // the first pass reads the forward's keys and values, the last writes the
        // sorted keys and values into kf / vf; the passes between keep (key, value)
        // pairs together in two ping-pong buffers
        uint2 *pairs[2] = {reinterpret_cast<uint2 *>(ws + W.pairs),
                           reinterpret_cast<uint2 *>(ws + W.pairs) + (W.pairs_n)};
        const dim3 grid((unsigned)nblk);
        // Segments found from the keys need only the valid keys sorted: the first
        // pass leaves out the dropped and default-row sentinels and the later
        // passes sort the keys it kept (their count, in misc[0], is the apply's).
        const bool excl = from_keys;
        for (int p = 0; p < passes; p++) {
            const int shift = p * kRadixBits;
            const bool pi = p > 0, po = p < passes - 1;
            const uint2 *pin = pi ? pairs[(p - 1) & 1] : nullptr;
            uint2 *pout = po ? pairs[p & 1] : nullptr;
            uint32_t *lm = (from_keys && !excl && p == passes - 1) ? misc : nullptr;
            const uint32_t *ndev = (excl && p > 0) ? misc : nullptr;
            const uint32_t lim = (excl && p == 0) ? plan->total_rows : 0xFFFFFFFFu;
            uint32_t *nkept = (excl && p == 0) ? misc : nullptr;
            if (nblk <= kHistSmallTiles) {
                if (pi) hipLaunchKernelGGL((rs_hist<true, kHistBlockSmall>), grid, dim3(kHistBlockSmall), 0, st,
                                           nullptr, pin, n, ndev, lim, shift, hist, nblk, misc);
                else hipLaunchKernelGGL((rs_hist<false, kHistBlockSmall>), grid, dim3(kHistBlockSmall), 0, st,
                                        k0, nullptr, n, ndev, lim, shift, hist, nblk, misc);
            } else {
                if (pi) hipLaunchKernelGGL((rs_hist<true, kHistBlock>), grid, dim3(kHistBlock), 0, st, nullptr,
                                           pin, n, ndev, lim, shift, hist, nblk, misc);
                else hipLaunchKernelGGL((rs_hist<false, kHistBlock>), grid, dim3(kHistBlock), 0, st, k0, nullptr,
                                        n, ndev, lim, shift, hist, nblk, misc);
            }
            hipLaunchKernelGGL(rs_scan, dim3(kRadix), dim3(kBlock), 0, st, hist, nblk, dtot);
            if (pi && po)
                hipLaunchKernelGGL((rs_scatter<true, true>), grid, dim3(kScatBlock), 0, st, nullptr, nullptr,
                                   nullptr, nullptr, pin, pout, n, ndev, lim, nkept, shift, hist, dtot, nblk,
                                   plan->total_rows, lm);
            else if (pi)
                hipLaunchKernelGGL((rs_scatter<true, false>), grid, dim3(kScatBlock), 0, st, nullptr, nullptr,
                                   kf, vf, pin, nullptr, n, ndev, lim, nkept, shift, hist, dtot, nblk,
                                   plan->total_rows, lm);
            else if (po)
                hipLaunchKernelGGL((rs_scatter<false, true>), grid, dim3(kScatBlock), 0, st, k0, v0, nullptr,
                                   nullptr, nullptr, pout, n, ndev, lim, nkept, shift, hist, dtot, nblk,
                                   plan->total_rows, lm);
            else
                hipLaunchKernelGGL((rs_scatter<false, false>), grid, dim3(kScatBlock), 0, st, k0, v0, kf, vf,
                                   nullptr, nullptr, n, ndev, lim, nkept, shift, hist, dtot, nblk,
                                   plan->total_rows, lm);
        }
        if (from_keys) {
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return fail(EMB_ERR_HIP, std::string("backward dedup launch: ") + hipGetErrorString(e));
            return EMB_OK;
        }
    }
    if (n <= kUqSmall) {
        hipLaunchKernelGGL(uq_small, dim3(1), dim3(kBlock), 0, st, kf, n, plan->total_rows, misc, seg, ukeys,
                           uniq_keys, n_uniq, stats);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(EMB_ERR_HIP, std::string("backward dedup launch: ") + hipGetErrorString(e));
        return EMB_OK;
    }
    hipLaunchKernelGGL(uq_count, dim3((unsigned)ublk), dim3(kBlock), 0, st, kf, n, plan->total_rows, ucnt, misc);
    hipLaunchKernelGGL(uq_scan, dim3(1), dim3(kBlock), 0, st, ucnt, ublk, uscan, misc, n_uniq, stats);
    hipLaunchKernelGGL(uq_write, dim3((unsigned)ublk), dim3(kBlock), 0, st, kf, n, plan->total_rows,
                       uscan, misc, seg, ukeys, uniq_keys);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(EMB_ERR_HIP, std::string("backward dedup launch: ") + hipGetErrorString(e));
    return EMB_OK;
}

extern "C" emb_status emb_backward_apply(emb_plan *plan, const float *grad_out, void *workspace,
                                         float *uniq_grads, void *stream)
{
    emb_status s = bwd_check(plan, workspace);
    if (s != EMB_OK) return s;
    if (!grad_out || !aligned(grad_out, 16)) return fail(EMB_ERR_INVALID_ARG, "grad_out must be 16-byte aligned device memory");
    if (uniq_grads && (plan->opt != EMB_OPT_EMIT || !aligned(uniq_grads, 16)))
        return fail(EMB_ERR_INVALID_ARG, "uniq_grads needs the EMIT optimizer and 16-byte alignment");
    const int64_t n = sort_n(plan);
    if (n == 0) return EMB_OK;
    char *ws = static_cast<char *>(workspace);
    const WsLayout &W = plan->ws;
    BwdArgs a{};
    a.cols = plan->dcols;
    a.row_base = plan->drow_base;
    a.C = plan->n_cols;
    a.B = plan->batch;
    a.sumD = plan->sum_dim;
    a.maxD = plan->max_dim;
    a.T = plan->tile;
    a.opt = plan->opt;
    a.lr = plan->lr;
    a.eps = plan->eps;
    a.ntiles = std::max<int64_t>(1, (n + plan->tile - 1) / plan->tile);
    a.G = grad_out;
    // the sorted bags sit in the buffer the last radix pass wrote
    a.sval = reinterpret_cast<const uint32_t *>(
        ws + (sort_passes(plan) % 2 ? W.vals2 : (plan->last_weighted ? W.posid : W.bags)));
    a.bw = reinterpret_cast<const uint2 *>(ws + W.bw);
    a.skeys = reinterpret_cast<const uint32_t *>(ws + (sort_passes(plan) % 2 ? W.keys2 : W.keys));
    a.bag_n = reinterpret_cast<const int32_t *>(ws + W.bag_n);
    a.seg = reinterpret_cast<const uint32_t *>(ws + W.seg);
    a.ukeys = reinterpret_cast<const uint32_t *>(ws + W.ukeys);
    a.misc = reinterpret_cast<const uint32_t *>(ws + W.misc);
    a.ugrads = uniq_grads;
    a.part = reinterpret_cast<float *>(ws + W.bpart);
    a.pcnt = reinterpret_cast<int32_t *>(ws + W.bcnt);
    a.tick = reinterpret_cast<uint32_t *>(ws + W.btick);
    a.any_mean = plan->any_mean ? 1 : 0;
    a.all_mean = plan->all_mean ? 1 : 0;
    a.zero = 0;
    a.total_rows = plan->total_rows;
    // Sorted segments of a few long columns change cost along the tile range
    // (hot rows: few segments; the cold tail: one row update per contributor):
    // chunks spread them over the XCDs.  With many columns each contiguous XCD
    // range mixes enough of them, and keeps one column's rows and gradient
    // slices in one L2.
    a.xcd_chunk = plan->n_cols >= 32 ? 0 : 16;
    const int64_t blocks = xcd_grid((a.ntiles + kTileWaves - 1) / kTileWaves, a.xcd_chunk);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)blocks), block(kTileBlock);
    if (plan->last_weighted) launch_apply<true>(plan, a, grid, block, st);
    else launch_apply<false>(plan, a, grid, block, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(EMB_ERR_HIP, std::string("seg_apply launch: ") + hipGetErrorString(e));
    return EMB_OK;
}

extern "C" emb_status emb_backward(emb_plan *plan, const float *grad_out, void *workspace,
                                   uint32_t *uniq_keys, float *uniq_grads, int64_t *n_uniq,
                                   int64_t *stats, void *stream)
{
    emb_status s = bwd_check(plan, workspace);
    if (s != EMB_OK) return s;
    if (!grad_out || !aligned(grad_out, 16)) return fail(EMB_ERR_INVALID_ARG, "grad_out must be 16-byte aligned device memory");
    if (uniq_grads && (!plan || plan->opt != EMB_OPT_EMIT || !aligned(uniq_grads, 16)))
        return fail(EMB_ERR_INVALID_ARG, "uniq_grads needs the EMIT optimizer and 16-byte alignment");
    s = emb_backward_dedup(plan, workspace, uniq_keys, n_uniq, stats, stream);
    if (s != EMB_OK) return s;
    return emb_backward_apply(plan, grad_out, workspace, uniq_grads, stream);
}

extern "C" emb_status emb_backward_atomic(emb_plan *plan, const float *grad_out, void *workspace,
                                          void *stream)
{
    emb_status s = bwd_check(plan, workspace);
    if (s != EMB_OK) return s;
    if (plan->opt != EMB_OPT_SGD) return fail(EMB_ERR_UNSUPPORTED, "the atomic backward is for SGD only");
    if (plan->has_default) return fail(EMB_ERR_UNSUPPORTED, "the atomic backward has no default rows");
    for (int32_t c = 0; c < plan->n_cols; c++)
        if (plan->hcols[c].dtype != EMB_F32) return fail(EMB_ERR_UNSUPPORTED, "the atomic backward needs fp32 tables");
    if (!grad_out || !aligned(grad_out, 16)) return fail(EMB_ERR_INVALID_ARG, "grad_out must be 16-byte aligned device memory");
    const int64_t n = plan->last_n;
    if (n == 0) return EMB_OK;
    char *ws = static_cast<char *>(workspace);
    AtomArgs a{};
    a.cols = plan->dcols;
    a.C = plan->n_cols;
    a.B = plan->batch;
    a.sumD = plan->sum_dim;
    a.T = plan->tile;
    a.lr = plan->lr;
    a.n = n;
    a.ntiles = (n + plan->tile - 1) / plan->tile;
    a.G = grad_out;
    a.keys = reinterpret_cast<const uint32_t *>(ws + plan->ws.keys);
    a.bags = reinterpret_cast<const int32_t *>(ws + plan->ws.bags);
    a.bag_n = reinterpret_cast<const int32_t *>(ws + plan->ws.bag_n);
    a.cstart = reinterpret_cast<const uint32_t *>(ws + plan->ws.cstart);
    a.bw = plan->last_weighted ? reinterpret_cast<const uint2 *>(ws + plan->ws.bw) : nullptr;
    a.total_rows = plan->total_rows;
    hipLaunchKernelGGL(atomic_apply, dim3((unsigned)a.ntiles), dim3(kTileBlock), 0,
                       static_cast<hipStream_t>(stream), a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(EMB_ERR_HIP, std::string("atomic_apply launch: ") + hipGetErrorString(e));
    return EMB_OK;
}
