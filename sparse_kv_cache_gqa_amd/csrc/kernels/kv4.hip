// uint4 group quantization of a KV cache for gfx950 (FlexGen digest, section
// "方法细节": groups of 64 along the hidden dimension, min/max, 4-bit codes,
// dequantized back to FP16 before compute).
//
// Eight lanes share one group of 64 fp16 values (16 bytes each).  min and max
// are exact; the scale is the exact (max - min) / 15 rounded once to binary16
// (fp64 quotient, then a single fp64 -> fp16 rounding from the bits); each
// code is round-half-even of (x - min) / scale computed in fp64.  fp16 values
// are multiples of 2^-24 below 2^16, so both quotients are correctly rounded
// fp64 values that cannot sit on, or cross, a rounding tie unless the exact
// value does: the codes equal the exact-rational definition.
#include "common.h"
#include "f16_round.h"

namespace da {
namespace {

using namespace dev;

__global__ __launch_bounds__(256) void quantize_kv4_kernel(int64_t n_groups, const u32x4 *__restrict__ x,
                                                           uint32_t *__restrict__ codes,
                                                           uint16_t *__restrict__ gmin,
                                                           uint16_t *__restrict__ gscale) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t grp = t >> 3;
    const int part = (int)(t & 7);
    const bool ok = grp < n_groups;
    const u32x4 v = ok ? x[t] : (u32x4){0u, 0u, 0u, 0u};
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = f16_to_f32(v[e] & 0xFFFFu);
        f[2 * e + 1] = f16_to_f32(v[e] >> 16);
    }
    float mn = f[0], mx = f[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) { mn = fminf(mn, f[e]); mx = fmaxf(mx, f[e]); }
    mn = xor_reduce<1, 8>(mn, OpMin{});
    mx = xor_reduce<1, 8>(mx, OpMax{});
    const double dmn = (double)mn;
    const uint16_t s16 = f64_to_f16_rne(((double)mx - dmn) / 15.0);
    const double s = (double)f16_to_f32(s16);
    uint32_t packed = 0;
    if (s != 0.0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            double c = rint(((double)f[e] - dmn) / s);
            c = c < 0.0 ? 0.0 : (c > 15.0 ? 15.0 : c);
            packed |= (uint32_t)c << (4 * e);
        }
    }
    if (ok) {
        codes[t] = packed;
        if (part == 0) {
            gmin[grp] = (uint16_t)f32_to_f16(mn);
            gscale[grp] = s16;
        }
    }
}

__global__ __launch_bounds__(256) void dequantize_kv4_kernel(int64_t n_words, const uint32_t *__restrict__ codes,
                                                             const uint16_t *__restrict__ gmin,
                                                             const uint16_t *__restrict__ gscale,
                                                             u32x4 *__restrict__ x) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_words) return;
    const int64_t grp = t >> 3;
    const uint32_t c = codes[t];
    const double mn = (double)f16_to_f32(gmin[grp]);
    const double s = (double)f16_to_f32(gscale[grp]);
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = f64_to_f16_rne(mn + (double)((c >> (4 * e)) & 15u) * s);
    u32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = h[2 * e] | (h[2 * e + 1] << 16);
    x[t] = out;
}

}  // namespace

hipError_t launch_quantize_kv4(int64_t n_groups, const void *x, uint8_t *codes, void *gmin, void *gscale,
                               hipStream_t stream) {
    const int64_t threads = n_groups * 8;
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quantize_kv4_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, n_groups,
                       (const u32x4 *)x, (uint32_t *)codes, (uint16_t *)gmin, (uint16_t *)gscale);
    return hipGetLastError();
}

hipError_t launch_dequantize_kv4(int64_t n_groups, const uint8_t *codes, const void *gmin, const void *gscale,
                                 void *x, hipStream_t stream) {
    const int64_t words = n_groups * 8;
    const int64_t blocks = (words + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(dequantize_kv4_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, words,
                       (const uint32_t *)codes, (const uint16_t *)gmin, (const uint16_t *)gscale, (u32x4 *)x);
    return hipGetLastError();
}

}  // namespace da
