// copy.hip -- a plain streaming device copy: the bandwidth a kernel that only
// reads and writes contiguous memory reaches on this GPU, measured next to the
// stage's own kernels (their achieved GB/s is reported against it as well as
// against the specified peak).
#include <string>

#include "device.h"

namespace emb {

constexpr int kCopyBlock = 256;
constexpr int kCopyUnroll = 4;       // 16-byte loads in flight per lane

// Grid-stride over 16-byte words; each lane issues kCopyUnroll loads before its
// stores, and neighbouring lanes touch neighbouring words (coalesced).
__global__ __launch_bounds__(kCopyBlock) void stream_copy(uint4 *__restrict__ dst,
                                                          const uint4 *__restrict__ src, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * kCopyBlock;
    int64_t i = (int64_t)blockIdx.x * kCopyBlock + threadIdx.x;
    for (; i + (kCopyUnroll - 1) * stride < n; i += kCopyUnroll * stride) {
        uint4 v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; u++) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; u++) dst[i + u * stride] = v[u];
    }
    for (; i < n; i += stride) dst[i] = src[i];
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
    // 256 CUs x 8 workgroups of 256 lanes, each lane 4 words per round
    const int64_t want = (n + kCopyBlock * kCopyUnroll - 1) / (kCopyBlock * kCopyUnroll);
    const unsigned grid = (unsigned)std::min<int64_t>(want, 256 * 8);
    hipLaunchKernelGGL(stream_copy, dim3(grid), dim3(kCopyBlock), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint4 *>(dst), static_cast<const uint4 *>(src), n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(EMB_ERR_HIP, std::string("stream_copy launch: ") + hipGetErrorString(e));
    return EMB_OK;
}
