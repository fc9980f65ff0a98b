// Per-step append of the new token for head-wise streaming (HeadInfer,
// section "核心 idea": the whole cache lives in host memory, so each decode
// step's key and value rows must reach it).
//
// One 64-lane workgroup per (head, batch row) copies the row's bytes in
// 16-byte pieces from the device array of new rows straight into row `len`
// of the head's page-locked host cache, through the cache's device-visible
// address: one launch covers up to kAppendMaxHeads heads, instead of one
// small device-to-host copy per (head, K or V).
#include "append.h"
#include "common.h"

namespace da {
namespace {

using namespace dev;

__global__ __launch_bounds__(64) void append_kernel(AppendArgs a) {
    const int lane = threadIdx.x;
    const int i = blockIdx.x / a.batch;                  // head within this launch
    const int b = blockIdx.x - i * a.batch;              // batch row
    if (i >= a.n_heads || (int64_t)lane * 16 >= a.row) return;
    const int gh = a.head0 + i;
    const int l = gh / a.Hkv, h = gh - l * a.Hkv;
    const int64_t src = (((int64_t)l * a.batch + b) * a.Hkv + h) * a.row + 16 * lane;
    const int64_t dst = b * a.dst_bstride + a.dst_off + 16 * lane;
    *(u32x4 *)(a.k_dst[i] + dst) = *(const u32x4 *)(a.k_new + src);
    *(u32x4 *)(a.v_dst[i] + dst) = *(const u32x4 *)(a.v_new + src);
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, hipStream_t stream) {
    if (a.n_heads < 1 || a.n_heads > kAppendMaxHeads || a.batch < 1 || a.row < 16 || a.row > 1024 || a.row % 16)
        return hipErrorInvalidValue;
    const int64_t blocks = (int64_t)a.n_heads * a.batch;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace da
