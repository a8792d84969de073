// device.h -- gfx950 device helpers: ID hashing, exact 64-bit remainder, wavefront
// searches and reductions, bf16 conversion.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace emb {

// SplitMix64 output function of x + golden gamma (the first output of a SplitMix64
// generator seeded with x; Steele, Lea & Flood 2014).
__device__ __forceinline__ uint64_t splitmix64(uint64_t x)
{
    uint64_t z = x + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// h mod d for any 64-bit h and d >= 1, with magic = floor((2^64-1)/d): the
// multiply-high quotient is q or q-1, so one conditional subtraction is exact
// (the second is a guard).  CDNA has no 64-bit integer divide.
__device__ __forceinline__ uint64_t mod_magic(uint64_t h, uint64_t d, uint64_t magic)
{
    uint64_t q = __umul64hi(h, magic);
    uint64_t r = h - q * d;
    if (r >= d) r -= d;
    if (r >= d) r -= d;
    return r;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Pointers read from memory (column metadata) have no known address space, so
// the compiler would emit flat loads, which also count against the LDS wait
// counter and stall every later LDS access; these casts make them global.
#if defined(__HIP_DEVICE_COMPILE__)
#define EMB_GLOBAL __attribute__((address_space(1)))
#else
#define EMB_GLOBAL   /* the host pass only type-checks device code */
#endif
template <typename T>
__device__ __forceinline__ const EMB_GLOBAL T *gp(const T *p)
{
    return (const EMB_GLOBAL T *)p;
}
template <typename T>
__device__ __forceinline__ EMB_GLOBAL T *gp(T *p)
{
    return (EMB_GLOBAL T *)p;
}

// Cross-workgroup exchange without cache flushes.  Stores and loads at agent
// scope go to the device-coherent level (past the per-XCD L2) for these words
// only; a full __threadfence() would write back and invalidate the whole L2.
__device__ __forceinline__ void st_agent(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int32_t *p, int32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float *p)
{
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_agent(const int32_t *p)
{
    return __hip_atomic_load(const_cast<int32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent(const uint32_t *p)
{
    return __hip_atomic_load(const_cast<uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait until this wavefront's outstanding memory operations (stores included)
// have completed, i.e. reached their coherence point
__device__ __forceinline__ void wait_vm()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ uint32_t ticket_add(uint32_t *p)
{
    return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Wavefront-level fence + barrier: makes one wavefront's LDS writes visible to
// all its lanes (all waves of a block run independent tiles, so no s_barrier).
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// First index i in [0, n) with a[i] > x (a non-decreasing), n if none, searched
// by the whole wavefront: 64 probes per step, so ~log64(n) dependent loads.
template <typename T>
__device__ __forceinline__ int64_t wave_upper_bound(const T *a, int64_t n, T x)
{
    int64_t lo = 0, hi = n;   // answer in [lo, hi]
    const int l = lane_id();
    while (hi - lo > 64) {
        const int64_t step = (hi - lo + 63) / 64;
        const int64_t i = lo + (int64_t)l * step;
        const bool le = (i < hi) ? (a[i] <= x) : false;
        const uint64_t m = __ballot(le);
        const int cnt = __popcll(m);          // probes with a[i] <= x (a prefix of lanes)
        if (cnt == 0) { hi = lo; break; }     // a[lo] > x
        const int64_t nlo = lo + (int64_t)(cnt - 1) * step + 1;   // a[nlo-1] <= x
        const int64_t nhi = (lo + (int64_t)cnt * step < hi) ? lo + (int64_t)cnt * step : hi;
        lo = nlo;
        hi = nhi;
    }
    if (hi > lo) {
        const int64_t i = lo + l;
        const bool le = (i < hi) ? (a[i] <= x) : false;
        lo += __popcll(__ballot(le));
    }
    return lo;
}

// wave_upper_bound started from a guess: one round of 64 probes 64 apart around
// `guess` brackets the answer when it lies within 2048 entries of the guess (one
// more round then finds it); otherwise the full search runs.  Same result.
template <typename T>
__device__ __forceinline__ int64_t wave_upper_bound_near(const T *a, int64_t n, T x, int64_t guess)
{
    const int l = lane_id();
    const int64_t lo = min(max(guess - 2048, (int64_t)0), max(n - 4096, (int64_t)0));
    const int64_t i = lo + (int64_t)l * 64;
    const bool le = (i < n) ? (a[i] <= x) : false;
    const int cnt = __popcll(__ballot(le));
    if (cnt == 0) {
        if (lo == 0) return 0;                       // a[0] > x
        return wave_upper_bound(a, n, x);
    }
    const int64_t i0 = lo + (int64_t)(cnt - 1) * 64;  // a[i0] <= x
    if (cnt == 64 && i0 + 64 < n) return wave_upper_bound(a, n, x);
    // the answer is in (i0, min(i0 + 64, n)]
    const int64_t j = i0 + 1 + l;
    const bool le2 = (l < 63 && j < n) ? (a[j] <= x) : false;
    return i0 + 1 + __popcll(__ballot(le2));
}

// First index i in [0, n) with a[i] >= x, n if none.
template <typename T>
__device__ __forceinline__ int64_t wave_lower_bound(const T *a, int64_t n, T x)
{
    int64_t lo = 0, hi = n;
    const int l = lane_id();
    while (hi - lo > 64) {
        const int64_t step = (hi - lo + 63) / 64;
        const int64_t i = lo + (int64_t)l * step;
        const bool lt = (i < hi) ? (a[i] < x) : false;
        const int cnt = __popcll(__ballot(lt));
        if (cnt == 0) { hi = lo; break; }
        const int64_t nlo = lo + (int64_t)(cnt - 1) * step + 1;
        const int64_t nhi = (lo + (int64_t)cnt * step < hi) ? lo + (int64_t)cnt * step : hi;
        lo = nlo;
        hi = nhi;
    }
    if (hi > lo) {
        const int64_t i = lo + l;
        const bool lt = (i < hi) ? (a[i] < x) : false;
        lo += __popcll(__ballot(lt));
    }
    return lo;
}

// Sum over the 64 lanes of a wavefront with DPP moves (gfx9 controls): swaps
// inside quads, the half-row and row mirrors, then the row broadcasts of lanes 15
// and 31 into the odd rows and the upper half; the total ends in lane 63 and is
// read out as a uniform value.  Every lane of the wavefront must be active.  The
// per-lane values are counts small enough that the total fits 32 bits.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v)
{
    int x = (int)v;
    x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);   // quad_perm [1, 0, 3, 2]
    x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);   // quad_perm [2, 3, 0, 1]
    x += __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);  // row_half_mirror
    x += __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false);  // row_mirror
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
    return (uint32_t)__builtin_amdgcn_readlane(x, 63);
}

// Wait here for loaded values (an empty asm that reads them and orders memory).
// A loop that issues a batch of loads and then stores results in divergent
// branches should let every load land before its first store: the one vector
// memory counter retires loads and stores in order, so a load consumed after a
// store would also wait for that store.
__device__ __forceinline__ void landed(const float4 &v)
{
    asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w) : "memory");
}
__device__ __forceinline__ void landed(const uint4 &v)
{
    asm volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w) : "memory");
}
__device__ __forceinline__ void landed(const uint2 &v)
{
    asm volatile("" ::"v"(v.x), "v"(v.y) : "memory");
}
__device__ __forceinline__ void landed(uint32_t v)
{
    asm volatile("" ::"v"(v) : "memory");
}
__device__ __forceinline__ void landed(float v)
{
    asm volatile("" ::"v"(v) : "memory");
}

// Structured buffer loads (the buffer_load "idxen offen" form): the address is
// base + index * stride + offset, formed by the load itself, and an index at or
// past the descriptor's record count reads zeros without touching memory.  The
// compiler has builtins for the raw form only, so the intrinsic is named
// directly.  Flags word: a 32-bit data format, as gfx9 buffer loads need.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x2_t __attribute__((ext_vector_type(2)));
__device__ i32x4_t struct_buffer_load_x4(__amdgpu_buffer_rsrc_t rsrc, int32_t vindex, int32_t voffset,
                                         int32_t soffset, int32_t aux)
    __asm("llvm.amdgcn.struct.ptr.buffer.load.v4i32");
__device__ i32x2_t struct_buffer_load_x2(__amdgpu_buffer_rsrc_t rsrc, int32_t vindex, int32_t voffset,
                                         int32_t soffset, int32_t aux)
    __asm("llvm.amdgcn.struct.ptr.buffer.load.v2i32");
constexpr int32_t kBufFlags = 0x00020000;
constexpr int kBufStrideMax = 16383;          // the descriptor's 14-bit stride field

// A descriptor over `rows` records of `stride` bytes at `base`; the arguments
// are the same in every lane, and are read from the first so that the
// descriptor sits in scalar registers (a descriptor the compiler must assume
// to vary is looped over lane by lane at every load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_buffer(const void *base, int stride, int32_t rows)
{
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    void *p = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)__builtin_amdgcn_readfirstlane(stride),
                                             __builtin_amdgcn_readfirstlane(rows), kBufFlags);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Block order over the 8 XCDs.  Hardware block b runs on XCD b mod 8, and each
// XCD starts its blocks in order.
//   chunk == 0: XCD x takes one contiguous range of tiles (x * nb / 8 ...).  Its
//     L2 then holds the rows, offsets and gradient slices of few columns.
//   chunk > 0: the i-th block of XCD x takes tile
//     ((i / chunk) * 8 + x) * chunk + i mod chunk.  All XCDs move through the
//     tile range together, so tiles whose cost changes along the range (hot
//     and cold rows of a few long columns) are spread evenly over them.  The
//     grid is padded to a multiple of 8 * chunk blocks; blocks past the last
//     tile exit at once.
__host__ __device__ __forceinline__ int64_t xcd_grid(int64_t ntiles, int chunk)
{
    const int64_t g = chunk ? 8 * (int64_t)chunk : 1;
    return (ntiles + g - 1) / g * g;
}

__device__ __forceinline__ int64_t xcd_block(int64_t b, int64_t nb, int chunk)
{
    const int64_t x = b & 7, i = b >> 3;
    if (chunk == 0) {
        const int64_t base = nb >> 3, rem = nb & 7;
        return x * base + (x < rem ? x : rem) + i;
    }
    return ((i / chunk) * 8 + x) * chunk + i % chunk;
}

// fp32 pair -> packed bf16 pair (lo in the low half), round to nearest even
// (one v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

}  // namespace emb
