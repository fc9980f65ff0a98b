// Streaming read of device memory: the practical HBM read bandwidth that the
// decode kernels are measured against, next to the published peak.  Not part
// of the attention method; a measurement aid.
//
// One single-wave workgroup per contiguous chunk (the layout that streamed
// fastest on MI355X: each wave walks its own range with non-temporal 16-byte
// loads, four per lane in flight, so every load instruction covers 1 KiB of
// consecutive bytes).  Each workgroup writes the XOR of its chunk's 32-bit
// words to sink[workgroup], so the loads cannot be dropped and the result can
// be checked exactly.
#include "common.h"

namespace da {
namespace {

using namespace dev;

constexpr int kReadUnroll = 4;

__global__ __launch_bounds__(64) void read_stream_kernel(const u32x4 *__restrict__ p, int64_t n16, int64_t per,
                                                         uint32_t *__restrict__ sink) {
    const int lane = threadIdx.x;
    const int64_t c0 = (int64_t)blockIdx.x * per;
    const int64_t c1 = blockIdx.x + 1 == gridDim.x ? n16 : min(n16, c0 + per);   // last chunk takes the rest
    uint32_t acc = 0;
    int64_t i = c0 + lane;
    for (; i + 64 * (kReadUnroll - 1) < c1; i += 64 * kReadUnroll) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + 64 * u);
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < c1; i += 64) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) acc ^= __shfl_xor(acc, o, 64);
    if (lane == 0) sink[blockIdx.x] = acc;
}

}  // namespace

hipError_t launch_read_stream(const void *buf, int64_t n16, int32_t n_groups, uint32_t *sink, hipStream_t stream) {
    if (n16 <= 0 || n_groups < 1 || n_groups > 65535 || n_groups > n16) return hipErrorInvalidValue;
    const int64_t per = n16 / n_groups;
    hipLaunchKernelGGL(read_stream_kernel, dim3((unsigned)n_groups), dim3(64), 0, stream, (const u32x4 *)buf, n16,
                       per, sink);
    return hipGetLastError();
}

}  // namespace da
