// Split-K decode attention for gfx950 (CDNA4): the fp32/fp16/bf16 instances
// of the partial pass (attn_split.h), the cross-split merges, the launch
// code and the allocation-free scratch array.
#include "attn_split.h"

#include <mutex>

namespace da {
namespace {

using namespace dev;

// Merge of the split partials of query-head rows: two rows per block, D
// threads per row (one per output channel).  Partial row: [u(D), m, l, pad,
// pad].  Weights 2^(m_s - M) are computed once per split into LDS, then every
// thread sums its channel over the splits.  (Two rows per block rather than
// one: measured on MI355X at 256 rows x 16 splits, the partial pass that
// follows the merge in the next decode step ran 166 us after this shape and
// 172-175 us after one-row blocks of the same arithmetic, or after an empty
// kernel of that grid -- the grid of the preceding kernel changes how the
// next one's single-wave workgroups land on the SIMDs.)
constexpr int kMergeRowsPerBlock = 2;
constexpr int kMergeMaxLds = 4096;       // weights per row kept in LDS

__global__ __launch_bounds__(256) void attn_reduce_kernel(const float *__restrict__ ws, float *__restrict__ o,
                                                          int n_split, int D, int HG, int64_t o_bstride,
                                                          int64_t rows) {
    __shared__ float w_all[kMergeRowsPerBlock][kMergeMaxLds];
    __shared__ float red_all[kMergeRowsPerBlock][4];
    const int half = threadIdx.x / D;              // row of this block
    const int tid = threadIdx.x - half * D, nt = D;
    const int64_t row = (int64_t)blockIdx.x * kMergeRowsPerBlock + half;   // b * HG + hq
    const bool live = row < rows;
    const int64_t b = row / HG, hq = row - b * HG;
    const int PSTR = D + 4;
    const float *p = ws + row * n_split * PSTR;
    float *w_lds = w_all[half];
    float *red = red_all[half];
    const int wv = tid >> 6;                       // wave within the row

    float M = neg_inf();
    if (live)
        for (int s = tid; s < n_split; s += nt) M = fmaxf(M, p[(int64_t)s * PSTR + D]);
    M = xor_reduce<1, 64>(M, OpMax{});
    if ((tid & 63) == 0) red[wv] = M;
    __syncthreads();
    M = red[0];
    for (int w = 1; w < (nt + 63) / 64; ++w) M = fmaxf(M, red[w]);
    __syncthreads();

    const bool use_lds = n_split <= kMergeMaxLds;
    float L = 0.f;
    if (live)
        for (int s = tid; s < n_split; s += nt) {
            const float m = p[(int64_t)s * PSTR + D];
            const float f = (m == neg_inf()) ? 0.f : fast_exp2(m - M);
            if (use_lds) w_lds[s] = f;
            L = fmaf(f, p[(int64_t)s * PSTR + D + 1], L);
        }
    L = xor_reduce<1, 64>(L, OpAdd{});
    if ((tid & 63) == 0) red[wv] = L;
    __syncthreads();
    L = red[0];
    for (int w = 1; w < (nt + 63) / 64; ++w) L += red[w];

    __syncthreads();   // w_lds complete
    if (!live) return;
    for (int d = tid; d < D; d += nt) {
        float O0 = 0.f, O1 = 0.f, O2 = 0.f, O3 = 0.f;
        int s = 0;
        if (use_lds) {
            // 16 independent loads in flight per batch
            for (; s + 16 <= n_split; s += 16) {
                float x[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) x[j] = p[(int64_t)(s + j) * PSTR + d];
#pragma unroll
                for (int j = 0; j < 16; j += 4) {
                    O0 = fmaf(w_lds[s + j], x[j], O0);
                    O1 = fmaf(w_lds[s + j + 1], x[j + 1], O1);
                    O2 = fmaf(w_lds[s + j + 2], x[j + 2], O2);
                    O3 = fmaf(w_lds[s + j + 3], x[j + 3], O3);
                }
            }
            for (; s < n_split; ++s) O0 = fmaf(w_lds[s], p[(int64_t)s * PSTR + d], O0);
        } else {
            for (; s < n_split; ++s) {
                const float m = p[(int64_t)s * PSTR + D];
                const float f = (m == neg_inf()) ? 0.f : fast_exp2(m - M);
                O0 = fmaf(f, p[(int64_t)s * PSTR + d], O0);
            }
        }
        o[b * o_bstride + hq * D + d] = L > 0.f ? ((O0 + O1) + (O2 + O3)) / L : 0.f;
    }
}

// Merge for n_split <= 4: one thread per output element, no LDS and no
// barriers (measured on MI355X: 3584 rows x 2 splits in a third of the time
// of the block-per-row kernel; with 16 splits over 256 rows the block-per-row
// kernel stays faster).  Bit for bit the result of attn_reduce_kernel: M is
// a max; L = (w0 l0 + w1 l1) + (w2 l2 + w3 l3), the tree its shuffle
// butterfly forms for n_split <= 4 (empty slots add 0); O is one fma chain.
constexpr int kMergeSmall = 4;

__global__ __launch_bounds__(256) void attn_reduce_small_kernel(const float *__restrict__ ws, float *__restrict__ o,
                                                                int n_split, int D, int HG, int64_t o_bstride,
                                                                int64_t total) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total) return;
    const int64_t row = t / D;
    const int d = (int)(t - row * D);
    const int64_t b = row / HG, hq = row - b * HG;
    const int PSTR = D + 4;
    const float *p = ws + row * n_split * PSTR;
    float M = neg_inf();
    for (int s = 0; s < n_split; ++s) M = fmaxf(M, p[s * PSTR + D]);
    float w[kMergeSmall], pl[kMergeSmall];
#pragma unroll
    for (int s = 0; s < kMergeSmall; ++s) {
        w[s] = 0.f;
        pl[s] = 0.f;
        if (s < n_split) {
            const float m = p[s * PSTR + D];
            w[s] = (m == neg_inf()) ? 0.f : fast_exp2(m - M);
            pl[s] = fmaf(w[s], p[s * PSTR + D + 1], 0.f);
        }
    }
#pragma unroll
    for (int half = kMergeSmall / 2; half >= 1; half >>= 1)
#pragma unroll
        for (int i = 0; i < half; ++i) pl[i] = pl[2 * i] + pl[2 * i + 1];
    const float L = pl[0];
    float O0 = 0.f;
    const float O1 = 0.f, O2 = 0.f, O3 = 0.f;
#pragma unroll
    for (int j = 0; j < kMergeSmall; ++j)
        if (j < n_split) O0 = fmaf(w[j], p[j * PSTR + d], O0);
    o[b * o_bstride + hq * D + d] = L > 0.f ? ((O0 + O1) + (O2 + O3)) / L : 0.f;
}

// Merge for 4 < n_split <= 32: one thread per output element, every split's
// m, l and this channel's u loaded in one round (attn_reduce_kernel takes
// three dependent rounds of loads with barriers between them).  Measured on
// MI355X, the Llama-3-8B decode step (256 rows x 16 splits) went from 168.44
// to 168.13 us: most of the merge's time is its launch and ramp, not its
// loads.  The arithmetic, and its order, is attn_reduce_kernel's, so the
// bits are the same (checked bitwise for 5..33 splits): M is a max; w_s =
// 2^(m_s - M); L is the pairwise tree that its lane butterfly forms over
// w_s l_s (slots past n_split add 0); O runs four fma chains over s in
// batches of 16, the remainder on the first.
constexpr int kMergeMid = 32;

__global__ __launch_bounds__(256) void attn_reduce_mid_kernel(const float *__restrict__ ws, float *__restrict__ o,
                                                              int n_split, int D, int HG, int64_t o_bstride,
                                                              int64_t total) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total) return;
    const int64_t row = t / D;
    const int d = (int)(t - row * D);
    const int64_t b = row / HG, hq = row - b * HG;
    const int PSTR = D + 4;
    const float *p = ws + row * n_split * PSTR;
    float w[kMergeMid], pl[kMergeMid], x[kMergeMid];
#pragma unroll
    for (int s = 0; s < kMergeMid; ++s) {
        w[s] = neg_inf();
        pl[s] = 0.f;
        x[s] = 0.f;
        if (s < n_split) {
            w[s] = p[s * PSTR + D];
            pl[s] = p[s * PSTR + D + 1];
            x[s] = p[s * PSTR + d];
        }
    }
    float M = neg_inf();
#pragma unroll
    for (int s = 0; s < kMergeMid; ++s) M = fmaxf(M, w[s]);
#pragma unroll
    for (int s = 0; s < kMergeMid; ++s) {
        const float f = (w[s] == neg_inf()) ? 0.f : fast_exp2(w[s] - M);
        w[s] = f;
        pl[s] = s < n_split ? fmaf(f, pl[s], 0.f) : 0.f;
    }
#pragma unroll
    for (int half = kMergeMid / 2; half >= 1; half >>= 1)
#pragma unroll
        for (int i = 0; i < half; ++i) pl[i] = pl[2 * i] + pl[2 * i + 1];
    const float L = pl[0];
    float O0 = 0.f, O1 = 0.f, O2 = 0.f, O3 = 0.f;
#pragma unroll
    for (int s0 = 0; s0 + 16 <= kMergeMid; s0 += 16) {
        if (s0 + 16 <= n_split) {
#pragma unroll
            for (int j = 0; j < 16; j += 4) {
                O0 = fmaf(w[s0 + j], x[s0 + j], O0);
                O1 = fmaf(w[s0 + j + 1], x[s0 + j + 1], O1);
                O2 = fmaf(w[s0 + j + 2], x[s0 + j + 2], O2);
                O3 = fmaf(w[s0 + j + 3], x[s0 + j + 3], O3);
            }
        }
    }
    const int rem0 = n_split & ~15;
#pragma unroll
    for (int s = 0; s < kMergeMid; ++s)
        if (s >= rem0 && s < n_split) O0 = fmaf(w[s], x[s], O0);
    o[b * o_bstride + hq * D + d] = L > 0.f ? ((O0 + O1) + (O2 + O3)) / L : 0.f;
}

using SplitFn = void (*)(AttnLaunch);

struct SplitKernel {
    SplitFn fn = nullptr;
    explicit operator bool() const { return fn != nullptr; }
};

template <int KF, int QF, int D, int G, bool PAGED, int SV = 0>
SplitKernel pick_one() {
    using C = Cfg<KF, QF, D, G>;
    if constexpr (C::ok) return {attn_split_kernel<KF, QF, D, G, PAGED, SV>};
    else return {};
}

template <int KF, int QF, int D, bool PAGED>
SplitKernel pick_g(int G) {
    if constexpr (PAGED) {
        return G == 1 ? pick_one<KF, QF, D, 1, PAGED>() : SplitKernel{};
    } else {
        switch (G) {
        case 1: return pick_one<KF, QF, D, 1, PAGED>();
        case 2: return pick_one<KF, QF, D, 2, PAGED>();
        case 4: return pick_one<KF, QF, D, 4, PAGED>();
        case 8: return pick_one<KF, QF, D, 8, PAGED>();
        default: return {};
        }
    }
}

template <int KF, int QF, bool PAGED>
SplitKernel pick_d(int D, int G) {
    if (D == 64) return pick_g<KF, QF, 64, PAGED>(G);
    if (D == 128) return pick_g<KF, QF, 128, PAGED>(G);
    return {};
}

// `waves`: the launch's wave count (0 when only asking whether a kernel
// exists); it picks between the two one-head uint4 forms.
SplitKernel pick(int kv, int qf, int D, int G, bool paged, int64_t waves = 0) {
    if (paged) {
        if (G != 1) return {};
        switch (kv) {
        case FMT_F32: return qf == FMT_F32 ? pick_d<FMT_F32, FMT_F32, true>(D, G) : SplitKernel{};
        case FMT_F16:
            if (qf == FMT_F16) return pick_d<FMT_F16, FMT_F16, true>(D, G);
            if (qf == FMT_F32) return pick_d<FMT_F16, FMT_F32, true>(D, G);
            return {};
        case FMT_BF16:
            if (qf == FMT_BF16) return pick_d<FMT_BF16, FMT_BF16, true>(D, G);
            if (qf == FMT_F32) return pick_d<FMT_BF16, FMT_F32, true>(D, G);
            return {};
        default: return {};
        }
    }
    switch (kv) {
    case FMT_F32: return qf == FMT_F32 ? pick_d<FMT_F32, FMT_F32, false>(D, G) : SplitKernel{};
    case FMT_F16:
        if (qf == FMT_F16) return pick_d<FMT_F16, FMT_F16, false>(D, G);
        if (qf == FMT_F32) return pick_d<FMT_F16, FMT_F32, false>(D, G);
        return {};
    case FMT_BF16:
        if (qf == FMT_BF16) return pick_d<FMT_BF16, FMT_BF16, false>(D, G);
        if (qf == FMT_F32) return pick_d<FMT_BF16, FMT_F32, false>(D, G);
        return {};
    case FMT_U4:
        // one query head per KV head: this unit (its accumulators are few);
        // grouped query heads: attn_u4.hip
        if (G != 1) return {pick_split_u4(qf, D, G)};
        if (D != 128) return {};
        {
            // int8 score products for grids of three or more waves per SIMD
            // (MI355X: 256 CUs x 4 SIMDs), where more waves cover their
            // longer chain; fp16 products below that
            const bool q8 = waves >= 3 * 1024;
            if (qf == FMT_F16) return q8 ? pick_one<FMT_U4, FMT_F16, 128, 1, false, 1>()
                                         : pick_one<FMT_U4, FMT_F16, 128, 1, false>();
            if (qf == FMT_F32) return q8 ? pick_one<FMT_U4, FMT_F32, 128, 1, false, 1>()
                                         : pick_one<FMT_U4, FMT_F32, 128, 1, false>();
        }
        return {};
    default: return {};
    }
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

// Split-K partials of the allocation-free entry point: a fixed device array
// (one per GPU the library runs on, held until the process ends) instead of
// a caller workspace.  Host code never passes `scratch` itself to a kernel --
// in host code the name stands for a host-side shadow, not a device address;
// it passes the device address that hipGetSymbolAddress returns for the
// current GPU, looked up once per device.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

hipError_t noalloc_scratch(float **out) {
    *out = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));      // this device's copy
        if (e != hipSuccess) return e;
        if (!p || ((uintptr_t)p & 255u) != 0) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = (float *)p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

int32_t default_split_dense(int64_t n_ctx) {
    int64_t want = (n_ctx + 15) / 16;
    int32_t s = kDefaultSplitDenseMin;
    while (s < kDefaultSplitDense && s < want) s <<= 1;
    return s;
}

// uint4: the longest split (from 256 tokens, doubling) that still gives at
// least kU4MinWaves waves over the units (batch rows x KV heads); measured on
// MI355X at B64 H56 N1024: one 1024-token split per head (no merge) 92 us,
// 512 (two splits and a merge) 99 us, 256 105 us.
int32_t default_split_u4(int64_t n_ctx, int64_t units) {
    int32_t s = kDefaultSplitU4Min;
    while (s < n_ctx && s < 65536 && units * ((n_ctx + 2 * (int64_t)s - 1) / (2 * (int64_t)s)) >= kU4MinWaves) s <<= 1;
    return s;
}

int32_t attn_n_split(int64_t n_ctx, int32_t split_tokens, bool paged, int32_t top_k, int32_t log2_page) {
    if (split_tokens <= 0) split_tokens = paged ? kDefaultSplitPaged : default_split_dense(n_ctx);
    if (paged) {
        int pps = split_tokens >> log2_page;
        if (pps < 1) pps = 1;
        if (pps > kMaxPagesPerSplit) pps = kMaxPagesPerSplit;
        return (top_k + pps - 1) / pps;
    }
    return (int32_t)((n_ctx + split_tokens - 1) / split_tokens);
}

size_t attn_ws_bytes(int64_t rows, int32_t n_split, int32_t D) {
    return (size_t)rows * (size_t)n_split * (size_t)(D + 4) * sizeof(float);
}

bool attn_supported(int kv_fmt, int q_fmt, int D, int G, bool paged) {
    return static_cast<bool>(pick(kv_fmt, q_fmt, D, G, paged));
}

hipError_t launch_split(const AttnLaunch &a, hipStream_t stream) {
    const bool paged = a.page_idx != nullptr;
    const SplitKernel k = pick(a.kv_fmt, a.q_fmt, a.D, a.G, paged, (int64_t)a.B * a.Hkv * a.n_split);
    if (!k) return hipErrorInvalidValue;
    if (a.wpb < 1 || a.wpb > kMaxWavesPerBlock || a.n_split < 1) return hipErrorInvalidValue;
    if (a.fused && a.n_split > a.wpb) return hipErrorInvalidValue;
    // uint4 with grouped query heads (P.V on the matrix cores): each wave's
    // LDS tiles follow the merge slots
    constexpr int kU4Tile = Cfg<FMT_U4, FMT_F16, 128, 2>::TILE;
    static_assert(Cfg<FMT_U4, FMT_F16, 128, 8>::TILE == kU4Tile && Cfg<FMT_U4, FMT_F32, 128, 4>::TILE == kU4Tile,
                  "one stage size for every grouped-query uint4 instance");
    const bool pvm = a.kv_fmt == FMT_U4 && a.G > 1;
    const size_t lds = (a.fused ? merge_lds_bytes(a.wpb, a.G, a.D) : 0) + (pvm ? a.wpb * kPvmWaveBytes<kU4Tile> : 0);
    dim3 grid((a.n_split + a.wpb - 1) / a.wpb, a.B * a.Hkv);
    hipLaunchKernelGGL(k.fn, grid, dim3(64 * a.wpb), lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_merge(int64_t rows, int32_t heads_per_row, int32_t n_split, int32_t D, const float *ws, float *o,
                        int64_t o_bstride, hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    if (rows > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (n_split <= kMergeSmall) {
        const int64_t total = rows * D;
        const int64_t blocks = (total + 255) / 256;
        if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
        hipLaunchKernelGGL(attn_reduce_small_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ws, o, n_split,
                           D, heads_per_row, o_bstride, total);
        return hipGetLastError();
    }
    if (n_split <= kMergeMid) {
        const int64_t total = rows * D;
        const int64_t blocks = (total + 255) / 256;
        if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
        hipLaunchKernelGGL(attn_reduce_mid_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ws, o, n_split, D,
                           heads_per_row, o_bstride, total);
        return hipGetLastError();
    }
    const int64_t blocks = (rows + kMergeRowsPerBlock - 1) / kMergeRowsPerBlock;
    hipLaunchKernelGGL(attn_reduce_kernel, dim3((unsigned)blocks), dim3(kMergeRowsPerBlock * D), 0, stream, ws, o,
                       n_split, D, heads_per_row, o_bstride, rows);
    return hipGetLastError();
}

// When to merge in the workgroup (measured on MI355X).  A single split
// always does (nothing to wait for).  Several splits do when there are at
// least as many (b, h) units as compute units (fewer would leave CUs idle)
// and the whole grid is at most 4 waves per SIMD: with more waves queued the
// separate merge costs little and 1-wave workgroups schedule more freely.
constexpr int64_t kFuseMinUnits = 256;
constexpr int64_t kFuseMaxWaves = 4096;

hipError_t launch_attention(const AttnLaunch &a, hipStream_t stream) {
    AttnLaunch f = a;
    f.wpb = 1;
    f.fused = 0;
    const int64_t units = (int64_t)a.B * a.Hkv;
    if (a.n_split == 1 || (a.n_split <= kMaxWavesPerBlock && units >= kFuseMinUnits &&
                           units * a.n_split <= kFuseMaxWaves)) {
        f.wpb = a.n_split;
        f.fused = 1;
    }
    hipError_t e = launch_split(f, stream);
    if (e != hipSuccess || f.fused) return e;
    return launch_merge((int64_t)a.B * a.Hkv * a.G, a.Hkv * a.G, a.n_split, a.D, a.ws, a.o, a.o_bstride, stream);
}

}  // namespace da
