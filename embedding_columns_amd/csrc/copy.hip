// copy.hip -- a plain streaming device copy: the bandwidth a kernel that only
// reads and writes contiguous memory reaches on this GPU, measured next to the
// stage's own kernels (their achieved GB/s is reported against it as well as
// against the specified peak).
#include <string>

#include "device.h"

namespace emb {

constexpr int kCopyBlock = 256;
constexpr int kCopyUnroll = 4;                            // 16-byte loads in flight per lane
constexpr int64_t kCopyChunk = kCopyBlock * kCopyUnroll;  // 16-byte words per workgroup

// Each workgroup copies one contiguous chunk of kCopyChunk words: every lane
// issues its kCopyUnroll loads (lane-adjacent words, so each load instruction is
// one contiguous kilobyte) before its stores.  One chunk per workgroup over a
// large grid measured faster on this GPU than grid-stride loops over a
// resident grid (5.5-5.8 against 4.1-4.5 TB/s for 1 GiB).
__global__ __launch_bounds__(kCopyBlock) void stream_copy(uint4 *__restrict__ dst,
                                                          const uint4 *__restrict__ src, int64_t n)
{
    const int64_t b0 = (int64_t)blockIdx.x * kCopyChunk + threadIdx.x;
    uint4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; u++) {
        const int64_t i = b0 + u * kCopyBlock;
        if (i < n) v[u] = src[i];
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; u++) {
        const int64_t i = b0 + u * kCopyBlock;
        if (i < n) dst[i] = v[u];
    }
}

}  // namespace emb

using namespace emb;

extern "C" emb_status emb_stream_copy(void *dst, const void *src, int64_t bytes, void *stream)
{
    if (bytes < 0 || (bytes > 0 && (!dst || !src))) return fail(EMB_ERR_INVALID_ARG, "copy: bad buffers");
    if (bytes % 16 || !aligned(dst, 16) || !aligned(src, 16))
        return fail(EMB_ERR_INVALID_ARG, "copy: 16-byte aligned buffers and a multiple of 16 bytes");
    if (bytes == 0) return EMB_OK;
    const int64_t n = bytes / 16;
    const int64_t blocks = (n + kCopyChunk - 1) / kCopyChunk;
    if (blocks > 0x7FFFFFFF) return fail(EMB_ERR_UNSUPPORTED, "copy: more than 2^31 - 1 chunks");
    const unsigned grid = (unsigned)blocks;
    hipLaunchKernelGGL(stream_copy, dim3(grid), dim3(kCopyBlock), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint4 *>(dst), static_cast<const uint4 *>(src), n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(EMB_ERR_HIP, std::string("stream_copy launch: ") + hipGetErrorString(e));
    return EMB_OK;
}
