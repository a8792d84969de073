// noalloc.hip -- the inference forward for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).
//
// The only device memory emb_forward needs beyond its inputs and outputs at
// inference is the split-bag scratch: fp32 partials of bags cut by tile
// boundaries, their counts, and one ticket per tile.  Here that scratch is a
// file-scope device array of kScratchBytes, one copy per GPU, held until the
// process exits.  Its device address is looked up once per device (with that
// device current) and kept; host code never passes the array's own name to a
// kernel, since in host code that name is a host-side stand-in.
//
// Every call on one GPU shares that GPU's array.  Tickets must start at zero,
// and the forward's zero row must hold zeros: each call clears both with one
// fill kernel before the forward (no memset node, so the pair can be captured
// into a graph).  Two calls that
// overlap on one GPU (different streams, no ordering) race on the array.
#include <mutex>
#include <string>

#include "device.h"

namespace emb {

constexpr size_t kScratchBytes = size_t(32) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kMaxDevices];

// clears n0 words at p0 and n1 words at p1
__global__ __launch_bounds__(kBlock) void zero_words(uint32_t *__restrict__ p0, int64_t n0,
                                                     uint32_t *__restrict__ p1, int64_t n1)
{
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < n0) p0[i] = 0u;
    else if (i < n0 + n1) p1[i - n0] = 0u;
}

// the device address of this GPU's array, looked up on the first call here
static emb_status scratch_ptr(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(EMB_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(EMB_ERR_UNSUPPORTED, "device index beyond 63");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(EMB_ERR_HIP, std::string("hipGetSymbolAddress: ") + hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return EMB_OK;
}

}  // namespace emb

using namespace emb;

extern "C" emb_status emb_forward_noalloc(emb_plan *plan, const int32_t *offsets, const int64_t *ids,
                                          const float *fvals, const int32_t *keyed_rows,
                                          int64_t n_ids, float *out, int64_t *stats, void *stream)
{
    if (!plan) return fail(EMB_ERR_INVALID_ARG, "plan is NULL");
    if (n_ids < 0 || n_ids > plan->max_ids)
        return fail(EMB_ERR_WORKSPACE, "n_ids exceeds the plan's max_ids");
    const size_t need = fwd_scratch_bytes(plan, n_ids, nullptr, nullptr);
    if (need > kScratchBytes)
        return fail(EMB_ERR_WORKSPACE, "the batch needs " + std::to_string(need) +
                                           " bytes of split-bag scratch; the fixed array holds " +
                                           std::to_string(kScratchBytes));
    void *base = nullptr;
    emb_status s = scratch_ptr(&base);
    if (s != EMB_OK) return s;
    FwdScratch sc{};
    fwd_scratch_bytes(plan, n_ids, &sc, base);
    // the tickets, and the zero row (the forward only reads it; cleared anyway,
    // the array's contents before the first call being the loader's)
    const int64_t zw = (int64_t)(kZeroRow / 4);
    hipLaunchKernelGGL(zero_words, dim3((unsigned)((sc.tiles + zw + kBlock - 1) / kBlock)), dim3(kBlock), 0,
                       static_cast<hipStream_t>(stream), sc.tick, sc.tiles,
                       reinterpret_cast<uint32_t *>(const_cast<char *>(sc.zrow)), zw);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(EMB_ERR_HIP, std::string("zero_words launch: ") + hipGetErrorString(e));
    return forward_with_scratch(plan, offsets, ids, fvals, keyed_rows, n_ids, out, stats, stream, sc);
}
