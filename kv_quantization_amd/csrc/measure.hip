// Measurement helper, not part of the method: a plain streaming read, the
// empirical HBM ceiling against which the kernels' bandwidth is reported.
// 256-thread workgroups read 16-byte words, four per thread per pass, over a
// grid-strided range; the loaded words are folded into one value that is
// stored only if it matches an impossible pattern, so the loads cannot be
// removed and almost nothing is written.
#include "kvq_common.h"

namespace kvq {
namespace {

constexpr int kBlock = 256;
constexpr int kUnroll = 4;
constexpr uint32_t kMaxBlocks = 8192;

__global__ __launch_bounds__(kBlock) void stream_read(const u32x4 *__restrict__ src, uint64_t n16,
                                                      uint32_t *__restrict__ sink) {
    const uint64_t stride = (uint64_t)gridDim.x * kBlock;
    uint64_t i = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(&src[i + u * stride]);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(&src[i]);
    const uint32_t f = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (f == 0x9E3779B9u && (acc.x & acc.y) == 0x7F4A7C15u) sink[0] = f;
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" int kvq_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream) {
    const char *fn = "kvq_stream_read";
    if (!src || !sink) return fail(KVQ_E_INVALID, "%s: null pointer argument", fn);
    if (!aligned16(src) || bytes % 16 || bytes == 0)
        return fail(KVQ_E_INVALID, "%s: src must be 16-byte aligned and bytes a positive multiple of 16", fn);
    const uint64_t n16 = bytes / 16;
    uint64_t blocks = (n16 + kBlock * kUnroll - 1) / (kBlock * kUnroll);
    if (blocks > kMaxBlocks) blocks = kMaxBlocks;
    stream_read<<<(unsigned)blocks, kBlock, 0, as_stream(stream)>>>(static_cast<const u32x4 *>(src), n16, sink);
    return launch_status(fn);
}
