// Query-aware page selection for gfx950 (TinyServe, section "方法细节" and
// Algorithm 1 steps 1-2).
//
// page_meta_kernel: per page of S = 2^log2S tokens and per channel, the min
//   and max of the keys (the page's bounding box).  Exact: min/max of values
//   of the storage type are values of that type.
//
// select_kernel: one 1024-thread workgroup per (batch row, head).
//   1. Bound score r_j = sum_d (q_d M_{j,d} if q_d >= 0 else q_d m_{j,d}),
//      written as q+ . M_j + q- . m_j with q+ = max(q, 0), q- = min(q, 0), so
//      it is a dense contraction: two 16x16x32 MFMAs per 32 channels take 16
//      pages as the N dimension, loading each page's M and m rows straight
//      from HBM into the B operand.  Products of 16-bit values are exact in
//      fp32; q in fp32 is split into 16-bit terms on the A rows.  Scores stay
//      in LDS (and optionally go to page_score).
//      With EXACT the key rows themselves are read once and scored against q
//      (q . k_i, one MFMA per 32 channels): token-level selection (FlexGen's
//      top-10% sparse attention, section "方法细节").
//   2. Top-K by a most-significant-digit radix select (4 passes of 8 bits)
//      over an order-preserving uint32 image of the fp32 scores, one shared
//      LDS histogram per pass.  Ties at the K-th score go to the lower page
//      index: the equal keys are ranked by a block-wide prefix count in index
//      order (skipped when every key equal to the K-th is kept).  The kept
//      indices are compacted in index order, so they come out ascending.
#include "common.h"

namespace da {
namespace {

using namespace dev;

template <int F>
struct Elem;
template <> struct Elem<FMT_F32> { static constexpr int size = 4; };
template <> struct Elem<FMT_F16> { static constexpr int size = 2; };
template <> struct Elem<FMT_BF16> { static constexpr int size = 2; };

template <int F>
__device__ __forceinline__ void unpack16(const u32x4 &x, float (&f)[16 / Elem<F>::size]) {
    if constexpr (F == FMT_F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(x[e]);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (F == FMT_BF16) {
                f[2 * e] = __uint_as_float(x[e] << 16);
                f[2 * e + 1] = __uint_as_float(x[e] & 0xFFFF0000u);
            } else {
                f[2 * e] = f16_to_f32(x[e] & 0xFFFFu);
                f[2 * e + 1] = f16_to_f32(x[e] >> 16);
            }
        }
    }
}

template <int F>
__device__ __forceinline__ u32x4 pack16(const float (&f)[16 / Elem<F>::size]) {
    u32x4 x;
    if constexpr (F == FMT_F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = __float_as_uint(f[e]);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint32_t lo, hi;
            if constexpr (F == FMT_BF16) {            // exact: the values are bf16 values
                lo = __float_as_uint(f[2 * e]) >> 16;
                hi = __float_as_uint(f[2 * e + 1]) >> 16;
            } else {
                lo = f32_to_f16(f[2 * e]);
                hi = f32_to_f16(f[2 * e + 1]);
            }
            x[e] = lo | (hi << 16);
        }
    }
    return x;
}

// One thread per (row block, page, 16-byte column chunk).
template <int F>
__global__ __launch_bounds__(256) void page_meta_kernel(int64_t BH, int64_t N, int D, int log2S, int64_t P,
                                                        const uint8_t *__restrict__ k, uint8_t *__restrict__ kmin,
                                                        uint8_t *__restrict__ kmax) {
    constexpr int EPC = 16 / Elem<F>::size;
    const int R = D * Elem<F>::size;
    const int CPR = R / 16;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t items = BH * P * CPR;
    if (t >= items) return;
    const int chunk = (int)(t % CPR);
    const int64_t pg = (t / CPR) % P;
    const int64_t bh = t / ((int64_t)CPR * P);
    const int64_t t0 = pg << log2S;
    const int64_t t1 = min(t0 + ((int64_t)1 << log2S), N);
    const uint8_t *src = k + (bh * N + t0) * R + 16 * chunk;
    float mn[EPC], mx[EPC];
    unpack16<F>(*(const u32x4 *)src, mn);
#pragma unroll
    for (int e = 0; e < EPC; ++e) mx[e] = mn[e];
    for (int64_t r = t0 + 1; r < t1; ++r) {
        src += R;
        float f[EPC];
        unpack16<F>(*(const u32x4 *)src, f);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
            mn[e] = fminf(mn[e], f[e]);
            mx[e] = fmaxf(mx[e], f[e]);
        }
    }
    const int64_t dst = (bh * P + pg) * R + 16 * chunk;
    *(u32x4 *)(kmin + dst) = pack16<F>(mn);
    *(u32x4 *)(kmax + dst) = pack16<F>(mx);
}

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

__device__ __forceinline__ uint32_t order_key(float f) {
    if (f == 0.f) f = 0.f;                        // -0 and +0 are one score
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of `v` over the workgroup (thread order); returns the
// total through *total.  Uses `buf` (kSelWaves + 1 entries).
__device__ __forceinline__ uint32_t block_exscan(uint32_t v, uint32_t *buf, uint32_t *total) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) buf[w] = x;
    __syncthreads();
    if (w == 0) {
        uint32_t s = lane < kSelWaves ? buf[lane] : 0u;
#pragma unroll
        for (int o = 1; o < kSelWaves; o <<= 1) {
            const uint32_t y = __shfl_up(s, o, 64);
            if (lane >= o) s += y;
        }
        if (lane < kSelWaves) buf[lane] = s;       // inclusive over waves
    }
    __syncthreads();
    const uint32_t before = (w ? buf[w - 1] : 0u) + x - v;
    *total = buf[kSelWaves - 1];
    __syncthreads();
    return before;
}

template <int KF, int QF, int D, bool EXACT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(int64_t P, int top_k, const void *__restrict__ q,
                                                             const uint8_t *__restrict__ kmin,
                                                             const uint8_t *__restrict__ kmax,
                                                             int32_t *__restrict__ page_idx,
                                                             float *__restrict__ page_score) {
    constexpr int R = D * Elem<KF>::size;
    constexpr int NCH = R / 64;
    constexpr int NMF = KF == FMT_F32 ? 4 * NCH : NCH;
    constexpr int SPL = (KF == FMT_F32 || QF == KF) ? 1 : (KF == FMT_BF16 ? 3 : 2);

    extern __shared__ float sc_lds[];              // [P]
    __shared__ uint32_t hist[256];
    __shared__ uint32_t scan_buf[kSelWaves + 1];
    __shared__ uint32_t pick_digit, pick_need, pick_count;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g4 = lane >> 4, n16 = lane & 15;
    const int64_t bh = blockIdx.x;

    // A operands: row s holds the s-th split term of q+ (pos) or q- (neg);
    // EXACT: of q itself (pos only)
    u32x4 Apos[KF == FMT_F32 ? 1 : NMF], Aneg[KF == FMT_F32 ? 1 : NMF];
    float Fpos[KF == FMT_F32 ? NMF : 1], Fneg[KF == FMT_F32 ? NMF : 1];
    {
        const int s = n16;
        const bool rowok = s < SPL;
        const int64_t qoff = bh * D;
#pragma unroll
        for (int mf = 0; mf < NMF; ++mf) {
            if constexpr (KF == FMT_F32) {
                const float x = rowok ? load_scalar<QF>(q, qoff + qk_dim<KF>(mf, g4, 0)) : 0.f;
                Fpos[mf] = EXACT ? x : fmaxf(x, 0.f);
                Fneg[mf] = fminf(x, 0.f);
            } else {
                uint32_t hp[8], hn[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = rowok ? load_scalar<QF>(q, qoff + qk_dim<KF>(mf, g4, e)) : 0.f;
                    hp[e] = rowok ? split_term<KF>(EXACT ? x : fmaxf(x, 0.f), s) : 0u;
                    hn[e] = rowok ? split_term<KF>(fminf(x, 0.f), s) : 0u;
                }
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    Apos[mf][e2] = hp[2 * e2] | (hp[2 * e2 + 1] << 16);
                    Aneg[mf][e2] = hn[2 * e2] | (hn[2 * e2 + 1] << 16);
                }
            }
        }
    }

    // ---- 1. bound scores --------------------------------------------------
    const uint8_t *mxb = kmax + bh * P * R + 16 * g4;
    const uint8_t *mnb = kmin + bh * P * R + 16 * g4;
    for (int64_t base = (int64_t)w * 16; base < P; base += 16 * kSelWaves) {
        const int64_t pg = base + n16;
        const bool ok = pg < P;
        u32x4 Kx[NCH], Kn[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            Kx[c] = ok ? *(const u32x4 *)(mxb + pg * R + 64 * c) : (u32x4){0u, 0u, 0u, 0u};
            if constexpr (!EXACT) Kn[c] = ok ? *(const u32x4 *)(mnb + pg * R + 64 * c) : (u32x4){0u, 0u, 0u, 0u};
        }
        f32x4 cc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            if constexpr (KF == FMT_F32) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    cc = __builtin_amdgcn_mfma_f32_16x16x4f32(Fpos[4 * c + e], __uint_as_float(Kx[c][e]), cc, 0, 0, 0);
                    if constexpr (!EXACT)
                        cc = __builtin_amdgcn_mfma_f32_16x16x4f32(Fneg[4 * c + e], __uint_as_float(Kn[c][e]), cc, 0, 0, 0);
                }
            } else if constexpr (KF == FMT_BF16) {
                cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, Apos[c]),
                                                             __builtin_bit_cast(bf16x8, Kx[c]), cc, 0, 0, 0);
                if constexpr (!EXACT)
                    cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, Aneg[c]),
                                                                 __builtin_bit_cast(bf16x8, Kn[c]), cc, 0, 0, 0);
            } else {
                cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, Apos[c]),
                                                            __builtin_bit_cast(f16x8, Kx[c]), cc, 0, 0, 0);
                if constexpr (!EXACT)
                    cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, Aneg[c]),
                                                                __builtin_bit_cast(f16x8, Kn[c]), cc, 0, 0, 0);
            }
        }
        if (g4 == 0 && ok) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < SPL; ++i) s += cc[i];
            if (s == 0.f) s = 0.f;
            sc_lds[pg] = s;
            if (page_score) page_score[bh * P + pg] = s;
        }
    }
    __syncthreads();

    // ---- 2. radix select of the top_k largest keys -------------------------
    // MSB-first, 8 bits per pass, one shared 256-bin histogram per pass.
    uint32_t prefix = 0, pmask = 0;
    uint32_t need = (uint32_t)top_k;
    uint32_t eq_count = 0;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        if (tid < 256) hist[tid] = 0u;
        __syncthreads();
        for (int64_t i = tid; i < P; i += kSelThreads) {
            const uint32_t key = order_key(sc_lds[i]);
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (w == 0) {
            uint32_t c[4], loc = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c[j] = hist[lane * 4 + j];
                loc += c[j];
            }
            // candidates in bins above this lane's four bins
            uint32_t suf = loc;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_down(suf, o, 64);
                if (lane + o < 64) suf += y;
            }
            uint32_t cum = suf - loc;
#pragma unroll
            for (int j = 3; j >= 0; --j) {
                if (cum < need && cum + c[j] >= need) {
                    pick_digit = (uint32_t)(lane * 4 + j);
                    pick_need = need - cum;
                    pick_count = c[j];
                }
                cum += c[j];
            }
        }
        __syncthreads();
        prefix |= pick_digit << shift;
        pmask |= 0xFFu << shift;
        need = pick_need;
        eq_count = pick_count;
    }
    const uint32_t T = prefix;              // key of the top_k-th largest score

    // ---- 3. ties by lower index; compact in index order --------------------
    // Keep every key > T and the `need` lowest-indexed keys == T.  When all
    // eq_count keys equal to T are kept (need == eq_count) that is key >= T.
    const int64_t E = (P + kSelThreads - 1) / kSelThreads;
    const int64_t i0 = (int64_t)tid * E, i1 = min(i0 + E, P);
    uint32_t tot;
    uint32_t eq_before = 0;
    const bool all_ties = need == eq_count;
    if (!all_ties) {
        uint32_t n_eq = 0;
        for (int64_t i = i0; i < i1; ++i) n_eq += order_key(sc_lds[i]) == T;
        eq_before = block_exscan(n_eq, scan_buf, &tot);
    }
    uint32_t n_sel = 0;
    {
        uint32_t r = eq_before;
        for (int64_t i = i0; i < i1; ++i) {
            const uint32_t key = order_key(sc_lds[i]);
            if (key > T) ++n_sel;
            else if (key == T) { if (all_ties || r < need) ++n_sel; ++r; }
        }
    }
    uint32_t pos = block_exscan(n_sel, scan_buf, &tot);
    int32_t *out = page_idx + bh * top_k;
    {
        uint32_t r = eq_before;
        for (int64_t i = i0; i < i1; ++i) {
            const uint32_t key = order_key(sc_lds[i]);
            bool sel = key > T;
            if (key == T) { sel = all_ties || r < need; ++r; }
            if (sel && pos < (uint32_t)top_k) out[pos++] = (int32_t)i;
        }
    }
}

using SelFn = void (*)(int64_t, int, const void *, const uint8_t *, const uint8_t *, int32_t *, float *);

template <int KF, int QF, bool EXACT>
SelFn sel_d(int D) {
    if (D == 64) return select_kernel<KF, QF, 64, EXACT>;
    if (D == 128) return select_kernel<KF, QF, 128, EXACT>;
    return nullptr;
}

template <bool EXACT>
SelFn sel_pick(int kv, int qf, int D) {
    switch (kv) {
    case FMT_F32: return qf == FMT_F32 ? sel_d<FMT_F32, FMT_F32, EXACT>(D) : nullptr;
    case FMT_F16:
        if (qf == FMT_F16) return sel_d<FMT_F16, FMT_F16, EXACT>(D);
        if (qf == FMT_F32) return sel_d<FMT_F16, FMT_F32, EXACT>(D);
        return nullptr;
    case FMT_BF16:
        if (qf == FMT_BF16) return sel_d<FMT_BF16, FMT_BF16, EXACT>(D);
        if (qf == FMT_F32) return sel_d<FMT_BF16, FMT_F32, EXACT>(D);
        return nullptr;
    default: return nullptr;
    }
}

}  // namespace

hipError_t launch_page_meta(int kv_fmt, int64_t BH, int64_t N, int D, int log2_page, const void *k, void *kmin,
                            void *kmax, hipStream_t stream) {
    const int64_t P = (N + (1ll << log2_page) - 1) >> log2_page;
    const int esz = kv_fmt == FMT_F32 ? 4 : 2;
    const int64_t items = BH * P * (D * esz / 16);
    const int64_t blocks = (items + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    auto *kk = (const uint8_t *)k;
    auto *mn = (uint8_t *)kmin;
    auto *mx = (uint8_t *)kmax;
    switch (kv_fmt) {
    case FMT_F32: hipLaunchKernelGGL(page_meta_kernel<FMT_F32>, dim3((unsigned)blocks), dim3(256), 0, stream, BH, N, D, log2_page, P, kk, mn, mx); break;
    case FMT_F16: hipLaunchKernelGGL(page_meta_kernel<FMT_F16>, dim3((unsigned)blocks), dim3(256), 0, stream, BH, N, D, log2_page, P, kk, mn, mx); break;
    case FMT_BF16: hipLaunchKernelGGL(page_meta_kernel<FMT_BF16>, dim3((unsigned)blocks), dim3(256), 0, stream, BH, N, D, log2_page, P, kk, mn, mx); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

bool select_supported(int kv_fmt, int q_fmt, int D) { return sel_pick<false>(kv_fmt, q_fmt, D) != nullptr; }

hipError_t launch_select(int kv_fmt, int q_fmt, int64_t BH, int64_t P, int D, int top_k, const void *q,
                         const void *kmin, const void *kmax, int32_t *page_idx, float *page_score,
                         hipStream_t stream, bool exact) {
    SelFn fn = exact ? sel_pick<true>(kv_fmt, q_fmt, D) : sel_pick<false>(kv_fmt, q_fmt, D);
    if (!fn) return hipErrorInvalidValue;
    const size_t lds = (size_t)P * sizeof(float);
    hipLaunchKernelGGL(fn, dim3((unsigned)BH), dim3(kSelThreads), lds, stream, P, top_k, q,
                       (const uint8_t *)kmin, (const uint8_t *)kmax, page_idx, page_score);
    return hipGetLastError();
}

}  // namespace da
