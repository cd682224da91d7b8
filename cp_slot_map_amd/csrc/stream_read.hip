// Streaming-read reference kernel (measurement support): reads a buffer once with 16-byte coalesced nontemporal loads
// and nothing else, so its rate is the read bandwidth this device reaches on a plain sequential stream (measured on
// gfx950: ~7.0 TB/s with the nontemporal hint, ~6.3 TB/s without, over 1024 to 16384 workgroups). Benchmarks report
// the attention kernels' KV rate against it as a second, achievable denominator next to the nominal HBM peak.
#include <algorithm>

#include "common.h"

namespace cpattn {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;     // loads each lane has in flight before it uses any

// Block i reads the contiguous range [i * per_block, min((i + 1) * per_block, n)) of 16-byte words: each pass issues
// kStreamUnroll loads per lane (256 lanes x 16 B = 4 KB per load instruction of the block), then folds them into an
// XOR. Each block writes one word, the XOR of everything it read, so no load can be dropped.
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4_t* __restrict__ src, int64_t n,
                                                                     int64_t per_block, uint32_t* __restrict__ sink) {
    const int64_t lo = int64_t(blockIdx.x) * per_block;
    const int64_t hi = std::min<int64_t>(lo + per_block, n);
    u32x4_t acc = {0u, 0u, 0u, 0u};
    int64_t i = lo + threadIdx.x;
    constexpr int64_t kPass = int64_t(kStreamThreads) * kStreamUnroll;
    for (; i + (kStreamUnroll - 1) * kStreamThreads < hi; i += kPass) {
        u32x4_t v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kStreamThreads);
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u];
    }
    for (; i < hi; i += kStreamThreads) acc ^= __builtin_nontemporal_load(src + i);
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m);
    __shared__ uint32_t s_x[kStreamThreads / 64];
    if ((threadIdx.x & 63) == 0) s_x[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t y = 0;
#pragma unroll
        for (int w = 0; w < kStreamThreads / 64; ++w) y ^= s_x[w];
        sink[blockIdx.x] = y;
    }
}

}  // namespace cpattn

using namespace cpattn;

extern "C" int32_t cp_debug_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t sink_words,
                                        hipStream_t stream) {
    if (bytes < 0 || sink_words < 1) return fail(CPATTN_EINVAL, "cp_debug_stream_read: negative size or empty sink");
    if (bytes % 16) return fail(CPATTN_EINVAL, "cp_debug_stream_read: %lld bytes is not a multiple of 16",
                                static_cast<long long>(bytes));
    if (bytes == 0) return CPATTN_OK;
    if (!src || !sink) return fail(CPATTN_EINVAL, "cp_debug_stream_read: null pointer");
    if (reinterpret_cast<uintptr_t>(src) % 16) return fail(CPATTN_EINVAL, "cp_debug_stream_read: src not 16-byte aligned");
    const int64_t n = bytes / 16;
    // Blocks: as many as the sink holds, at most one per 4 KB pass of work; each block's range a whole number of
    // passes where the buffer allows.
    constexpr int64_t kPass = int64_t(kStreamThreads) * kStreamUnroll;
    const int64_t blocks_wanted = std::max<int64_t>(1, std::min<int64_t>(sink_words, (n + kPass - 1) / kPass));
    const int64_t per_block = ((n + blocks_wanted - 1) / blocks_wanted + kPass - 1) / kPass * kPass;
    const int64_t blocks = (n + per_block - 1) / per_block;
    hipLaunchKernelGGL(stream_read_kernel, dim3(uint32_t(blocks)), dim3(kStreamThreads), 0, stream,
                       static_cast<const u32x4_t*>(src), n, per_block, sink);
    return check_launch("cp_debug_stream_read");
}
