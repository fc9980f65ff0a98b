// Per-step append of head-wise streaming: the device-side half, shared by
// the C-ABI (stream.cpp) and the kernel (kernels/append.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace da {

// Append of one token's K and V rows to host caches (the per-step append of
// head-wise streaming).  Heads head0 .. head0 + n_heads - 1 (global index
// l * Hkv + h) of k_new / v_new [L][batch][Hkv][row bytes] go to row `len` of
// their caches [batch][cap][row bytes], whose device-visible addresses (of
// page-locked host memory) are k_dst[i] / v_dst[i].
constexpr int kAppendMaxHeads = 32;
struct AppendArgs {
    const uint8_t *k_new = nullptr, *v_new = nullptr;
    uint8_t *k_dst[kAppendMaxHeads] = {}, *v_dst[kAppendMaxHeads] = {};
    int32_t head0 = 0, n_heads = 0, Hkv = 0, batch = 0;
    int64_t row = 0;            // bytes per row, a multiple of 16, <= 1024
    int64_t dst_off = 0;        // len * row
    int64_t dst_bstride = 0;    // cap * row
};
hipError_t launch_append(const AppendArgs &a, hipStream_t stream);

}  // namespace da
