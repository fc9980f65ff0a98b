// Chunked prefill attention for gfx950 (HeadInfer, section "chunked prefill
// 与 adaptive head grouping"; per-head equation of section "核心 idea" with the
// causal mask of prefill).
//
// A chunk of C queries at positions prefix .. prefix + C - 1 attends to the
// cache rows 0 .. prefix + i (the earlier chunks and the chunk itself).
// Unlike decode this is a dense contraction with reuse (each K/V tile serves
// 128 queries), so both products run on the matrix cores:
//
//   * One 256-thread workgroup per (b, query head, 128 queries); wave w owns
//     queries 32w .. 32w + 31 (two blocks of 16).  K/V tiles of 64 keys are
//     staged in LDS, V transposed while it is stored; the next tile's global
//     loads are issued before the current tile is computed.
//   * S^T = K Q^T on v_mfma_f32_16x16x32_{bf16,f16}: A = 16 keys of the K
//     tile (LDS), B = 16 queries (registers, loaded once).  In the output
//     layout a lane holds 4 keys of one query, so the softmax is per lane
//     plus two shuffles, and the probabilities already sit where the B
//     operand of the next product wants them.
//   * O^T += V^T P^T on the same MFMA: A = 16 channels of V^T (LDS), B = P^T
//     straight from the S^T registers (lane k-slots 0-3 / 4-7 = keys
//     4g .. 4g + 3 of the two 16-key halves of a 32-key step; the V^T reads
//     use the same key order).  P is split into two 16-bit terms (hi + lo),
//     so the product is accurate to about 2^-16 of each weight.
//   * Online softmax in base 2 per query; rows past the causal limit get -inf.
#include "common.h"

namespace da {
namespace {

using namespace dev;

constexpr int kPreQ = 128;          // queries per workgroup
constexpr int kPreKeys = 64;        // keys per tile
constexpr int kPreThreads = 256;

template <int F>
__device__ __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
    if constexpr (F == FMT_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
}

template <int F>
__device__ __forceinline__ uint32_t to16(float x) {
    if constexpr (F == FMT_BF16) return f32_to_bf16(x);
    else return f32_to_f16(x);
}
template <int F>
__device__ __forceinline__ float from16(uint32_t b) {
    if constexpr (F == FMT_BF16) return bf16_to_f32(b);
    else return f16_to_f32(b);
}

struct PrefillArgs {
    const void *q;          // [B][Hq][C][D]
    const void *k, *v;      // [B][Hkv][T][D], T = prefix + C
    float *o;               // [B][Hq][C][D]
    int32_t Hq, G;
    int64_t C, T, prefix;
    float scale_log2;
};

template <int F, int D>
__global__ __launch_bounds__(kPreThreads) void prefill_kernel(PrefillArgs a) {
    constexpr int KSTR = D + 8;                 // K tile row stride (elements)
    constexpr int VSTR = kPreKeys + 8;          // V^T row stride (elements)
    constexpr int NKS = D / 32;                 // 32-channel steps of S
    constexpr int NCB = D / 16;                 // 16-channel blocks of O
    constexpr int CPR = D / 8;                  // 16-byte chunks per row
    constexpr int NLD = kPreKeys * CPR / kPreThreads;   // chunks per thread per tile
    static_assert(NLD * kPreThreads == kPreKeys * CPR, "tile split");

    __shared__ uint16_t k_lds[kPreKeys * KSTR];
    __shared__ uint16_t vt_lds[D * VSTR];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, n = lane & 15;
    const int64_t bh = blockIdx.y;                      // b * Hq + hq
    const int64_t b = bh / a.Hq, hq = bh - b * a.Hq;
    const int64_t hkv = hq / a.G;
    const int64_t q0 = (int64_t)blockIdx.x * kPreQ;     // first query of the workgroup (chunk-relative)
    const int64_t qw = q0 + wave * 32;                  // first query of this wave

    const uint8_t *kbase = (const uint8_t *)a.k + (b * (a.Hq / a.G) + hkv) * a.T * D * 2;
    const uint8_t *vbase = (const uint8_t *)a.v + (b * (a.Hq / a.G) + hkv) * a.T * D * 2;
    const uint32_t kv_bytes = (uint32_t)(a.T * D * 2);
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, kv_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, kv_bytes);

    // keys this workgroup needs: 0 .. min(prefix + q0 + kPreQ, T) - 1
    const int64_t kend = min(a.prefix + q0 + kPreQ, a.T);
    const int ntiles = (int)((kend + kPreKeys - 1) / kPreKeys);

    // ---- Q^T operands (B of S^T): query qw + 16 qb + n, channels 32 ks + 8 g ..
    u32x4 Qb[2][NKS];
    {
        const uint8_t *qbase = (const uint8_t *)a.q + bh * a.C * D * 2;
        const uint32_t q_bytes = (uint32_t)(a.C * D * 2);
        const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qbase, q_bytes);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                Qb[qb][ks] = buf_load16(qrs, (uint32_t)((qw + 16 * qb + n) * D + 32 * ks + 8 * g) * 2);
    }

    // ---- staging of one K/V tile: thread chunks c = tid + 256 j -> (key, 8 channels)
    u32x4 kreg[NLD], vreg[NLD];
    auto load_tile = [&](int t) {
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int c = tid + kPreThreads * j;
            const int key = c / CPR, col = (c % CPR) * 8;
            const uint32_t off = (uint32_t)(((int64_t)t * kPreKeys + key) * D + col) * 2;
            kreg[j] = buf_load16(krs, off);          // rows past T read as zeros
            vreg[j] = buf_load16(vrs, off);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int c = tid + kPreThreads * j;
            const int key = c / CPR, col = (c % CPR) * 8;
            *(u32x4 *)&k_lds[key * KSTR + col] = kreg[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vt_lds[(col + 2 * e) * VSTR + key] = (uint16_t)(vreg[j][e] & 0xFFFFu);
                vt_lds[(col + 2 * e + 1) * VSTR + key] = (uint16_t)(vreg[j][e] >> 16);
            }
        }
    };

    // ---- running state per query (lane n of each block) ---------------------
    float m_run[2] = {neg_inf(), neg_inf()};
    float l_run[2] = {0.f, 0.f};                  // this lane's keys only; summed over g at the end
    f32x4 acc[2][NCB];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[qb][cb] = (f32x4){0.f, 0.f, 0.f, 0.f};

    const float sl2 = a.scale_log2;
    if (ntiles > 0) load_tile(0);
    for (int t = 0; t < ntiles; ++t) {
        __syncthreads();                      // every wave is done reading the previous tile
        store_tile();
        __syncthreads();
        if (t + 1 < ntiles) load_tile(t + 1);

        const int64_t t0 = (int64_t)t * kPreKeys;
        // S^T blocks: keys 16 kb + 4 g + i of this tile, query n of block qb
        f32x4 st[2][4];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) st[qb][kb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const u32x4 ka = *(const u32x4 *)&k_lds[(16 * kb + n) * KSTR + 32 * ks + 8 * g];
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) st[qb][kb] = mfma16<F>(ka, Qb[qb][ks], st[qb][kb]);
            }

        // online softmax per query; build P^T operands (hi and lo terms)
        u32x4 ph[2][2], pl[2][2];                     // [qb][32-key step]
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int64_t qpos = a.prefix + qw + 16 * qb + n;
            float s[4][4];
            float mx = neg_inf();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t kpos = t0 + 16 * kb + 4 * g + i;
                    s[kb][i] = (kpos <= qpos) ? st[qb][kb][i] * sl2 : neg_inf();
                    mx = fmaxf(mx, s[kb][i]);
                }
            mx = fmaxf(mx, shfl_xor(mx, 16));
            mx = fmaxf(mx, shfl_xor(mx, 32));
            const float mnew = fmaxf(m_run[qb], mx);
            const float alpha = (mnew == m_run[qb]) ? 1.f : fast_exp2(m_run[qb] - mnew);
            m_run[qb] = mnew;
            float lsum = 0.f;
            uint32_t hb[4][4], lb[4][4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = (s[kb][i] == neg_inf()) ? 0.f : fast_exp2(s[kb][i] - mnew);
                    lsum += p;
                    const uint32_t h = to16<F>(p);
                    hb[kb][i] = h;
                    lb[kb][i] = to16<F>(p - from16<F>(h));
                }
            l_run[qb] = l_run[qb] * alpha + lsum;
            if (alpha != 1.f) {
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) acc[qb][cb] *= alpha;
            }
            // step s2 covers keys 32 s2 .. 32 s2 + 31: slots 0-3 <- block 2 s2, 4-7 <- block 2 s2 + 1
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                ph[qb][s2] = (u32x4){hb[2 * s2][0] | (hb[2 * s2][1] << 16), hb[2 * s2][2] | (hb[2 * s2][3] << 16),
                                     hb[2 * s2 + 1][0] | (hb[2 * s2 + 1][1] << 16),
                                     hb[2 * s2 + 1][2] | (hb[2 * s2 + 1][3] << 16)};
                pl[qb][s2] = (u32x4){lb[2 * s2][0] | (lb[2 * s2][1] << 16), lb[2 * s2][2] | (lb[2 * s2][3] << 16),
                                     lb[2 * s2 + 1][0] | (lb[2 * s2 + 1][1] << 16),
                                     lb[2 * s2 + 1][2] | (lb[2 * s2 + 1][3] << 16)};
            }
        }

        // O^T += V^T P^T: A = channels 16 cb + m, keys in the P^T slot order
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const uint16_t *vr = &vt_lds[(16 * cb + n) * VSTR + 32 * s2 + 4 * g];
                const uint2 lo4 = *(const uint2 *)vr;           // keys 32 s2 + 4 g .. + 3
                const uint2 hi4 = *(const uint2 *)(vr + 16);    // keys 32 s2 + 16 + 4 g .. + 3
                const u32x4 va = (u32x4){lo4.x, lo4.y, hi4.x, hi4.y};
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    acc[qb][cb] = mfma16<F>(va, ph[qb][s2], acc[qb][cb]);
                    acc[qb][cb] = mfma16<F>(va, pl[qb][s2], acc[qb][cb]);
                }
            }
    }

    // ---- normalise and store: lane holds channels 16 cb + 4 g .. + 3 of query n
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        float l = l_run[qb];
        l += shfl_xor(l, 16);
        l += shfl_xor(l, 32);
        const int64_t qi = qw + 16 * qb + n;
        if (qi < a.C) {
            float *dst = a.o + (bh * a.C + qi) * D;
            const float inv = 1.f / l;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                f32x4 r = acc[qb][cb];
#pragma unroll
                for (int e = 0; e < 4; ++e) r[e] = r[e] * inv;
                *(f32x4 *)(dst + 16 * cb + 4 * g) = r;
            }
        }
    }
}

using PrefillFn = void (*)(PrefillArgs);

PrefillFn prefill_pick(int fmt, int D) {
    if (fmt == FMT_BF16) return D == 64 ? prefill_kernel<FMT_BF16, 64> : (D == 128 ? prefill_kernel<FMT_BF16, 128> : nullptr);
    if (fmt == FMT_F16) return D == 64 ? prefill_kernel<FMT_F16, 64> : (D == 128 ? prefill_kernel<FMT_F16, 128> : nullptr);
    return nullptr;
}

}  // namespace

bool prefill_supported(int fmt, int D) { return prefill_pick(fmt, D) != nullptr; }

hipError_t launch_prefill(int fmt, int64_t B, int32_t Hq, int32_t Hkv, int D, int64_t C, int64_t T, float scale_log2,
                          const void *q, const void *k, const void *v, float *o, hipStream_t stream) {
    PrefillFn fn = prefill_pick(fmt, D);
    if (!fn) return hipErrorInvalidValue;
    PrefillArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.Hq = Hq;
    a.G = Hq / Hkv;
    a.C = C;
    a.T = T;
    a.prefix = T - C;
    a.scale_log2 = scale_log2;
    const int64_t qblocks = (C + kPreQ - 1) / kPreQ;
    if (qblocks > 0x7FFFFFFF || B * Hq > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3((unsigned)qblocks, (unsigned)(B * Hq)), dim3(kPreThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace da
