// Chunked prefill attention for gfx950 (HeadInfer, section "chunked prefill
// 与 adaptive head grouping"; per-head equation of section "核心 idea" with the
// causal mask of prefill).
//
// A chunk of C queries at positions prefix .. prefix + C - 1 attends to the
// cache rows 0 .. prefix + i (the earlier chunks and the chunk itself).
// Unlike decode this is a dense contraction with reuse (each K/V tile serves
// 128 queries), so both products run on the matrix cores:
//
//   * One 512-thread workgroup per (b, query head, 256 queries); wave w owns
//     two blocks of 16 queries, 32w .. 32w + 31, so every K and V^T operand
//     it reads from LDS feeds two MFMAs.  K/V tiles of 64 keys are staged in
//     LDS, V transposed while it is stored (two keys per dword, in the key
//     order of the P^T operand, so each V^T operand is one 16-byte read); the
//     next tile's global loads are issued before the current tile is
//     computed.  The workgroups of one (b, KV head) share a die (its L2 holds
//     their K/V tiles), latest blocks first.
//   * S^T = K Q^T on v_mfma_f32_16x16x32_{bf16,f16}: A = 16 keys of the K
//     tile (LDS), B = 16 queries of a block (registers, loaded once).  In the output
//     layout a lane holds 4 keys of one query, so the softmax is per lane
//     plus two shuffles, and the probabilities already sit where the B
//     operand of the next product wants them.
//   * O^T += V^T P^T on the same MFMA: A = 16 channels of V^T (LDS), B = P^T
//     straight from the S^T registers (lane k-slots 0-3 / 4-7 = keys
//     4g .. 4g + 3 of the two 16-key halves of a 32-key step; V^T rows hold
//     those eight keys contiguously).  P is split into two 16-bit terms (hi +
//     lo), so the product is accurate to about 2^-16 of each weight.
//   * Only tiles that reach the diagonal run the causal mask (a wave-uniform
//     branch); the first product of each S^T chain starts from a zero
//     accumulator operand.
//   * Within a tile the softmax of query block 1 is independent of the P.V
//     products of block 0; scheduling-group hints interleave the two, so the
//     VALU and the matrix cores work at the same time within a wave.
//   * Online softmax in base 2 per query, the scale folded into the exp2
//     argument; rows past the causal limit get -inf; the running max is
//     raised lazily (see below).
#include "common.h"

namespace da {
namespace {

using namespace dev;

constexpr int kPreQ = 256;          // queries per workgroup
constexpr int kPreKeys = 64;        // keys per tile

template <int F>
__device__ __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
    if constexpr (F == FMT_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats rounded (nearest, ties to even) to the 16-bit type, packed low
// then high; bf16 uses the packed hardware conversion.
template <int F>
__device__ __forceinline__ uint32_t pack16(float a, float b) {
    if constexpr (F == FMT_BF16) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
    } else {
        return f32_to_f16(a) | (f32_to_f16(b) << 16);
    }
}
template <int F>
__device__ __forceinline__ float lo16(uint32_t w) {
    if constexpr (F == FMT_BF16) return __uint_as_float(w << 16);
    else return f16_to_f32(w & 0xFFFFu);
}
template <int F>
__device__ __forceinline__ float hi16(uint32_t w) {
    if constexpr (F == FMT_BF16) return __uint_as_float(w & 0xFFFF0000u);
    else return f16_to_f32(w >> 16);
}

// Position of key k (0..63 of a tile) inside a V^T row: within each 32-key
// step, the eight keys that one lane's P^T operand slots hold (keys 4 g .. +3
// and 16 + 4 g .. +3) are stored contiguously at 8 g, so the A operand is a
// single 16-byte read.  Keys 2 j and 2 j + 1 stay adjacent.
__device__ __forceinline__ int vt_pos(int k) {
    return (k & ~31) | (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}

constexpr int kSgVa = 14, kSgVb = 3;   // scheduling groups, VALU counts (measured on MI355X)
constexpr float kLazy = 8.f;        // log2 headroom before the running max is raised

struct PrefillArgs {
    const void *q;          // [B][Hq][C][D]
    const void *k, *v;      // [B][Hkv][T][D], T = prefix + C
    float *o;               // [B][Hq][C][D]
    int32_t Hq, G;
    int64_t C, T, prefix;
    float scale_log2;
    int32_t nqb;            // query blocks per head
    int32_t xcd_map;        // 1: workgroups of one KV head share an XCD (see below)
};

constexpr int kXcds = 8;    // MI355X: 8 accelerator dies; workgroup i starts on die i mod 8

// QB blocks of 16 queries per wave; kPreQ / (16 QB) waves per workgroup.
template <int QB>
constexpr int pre_threads() { return 64 * (kPreQ / (16 * QB)); }

template <int F, int D, int QB>
__global__ __launch_bounds__(pre_threads<QB>()) void prefill_kernel(PrefillArgs a) {
    constexpr int kPreThreads = pre_threads<QB>();
    constexpr int KSTR = D + 8;                 // K tile row stride (elements)
    constexpr int VSTR = kPreKeys + 8;          // V^T row stride (elements; 16-byte aligned rows)
    constexpr int NKS = D / 32;                 // 32-channel steps of S
    constexpr int NCB = D / 16;                 // 16-channel blocks of O
    constexpr int NKB = kPreKeys / 16;          // 16-key blocks of a tile
    constexpr int NS2 = kPreKeys / 32;          // 32-key steps of a tile
    constexpr int CPR = D / 8;                  // 16-byte chunks per row
    constexpr int NKA = kPreKeys * CPR;                            // K (key, chunk) assignments
    constexpr int NLD = NKA >= kPreThreads ? NKA / kPreThreads : 1; // per thread
    static_assert(NKA % kPreThreads == 0 || NKA < kPreThreads, "K split");
    constexpr int NVA = kPreKeys / 2 * CPR;                        // V (key pair, chunk) assignments
    constexpr int NV = NVA >= kPreThreads ? NVA / kPreThreads : 1; // per thread
    static_assert(NVA % kPreThreads == 0 || NVA < kPreThreads, "V split");

    __shared__ __attribute__((aligned(16))) uint16_t k_lds[kPreKeys * KSTR];
    __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * VSTR];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, n = lane & 15;
    // Workgroup -> (batch row, query head, query block).  With xcd_map, the
    // workgroups of one (batch row, KV head) all sit on one die, so its L2
    // serves their shared K/V tiles: die = unit mod 8; inside a unit the G
    // query heads of one query block are consecutive (they read the same
    // tiles at the same time) and the blocks run latest first (the longest
    // first, for a shorter tail).  Otherwise: x = query block, y = b * Hq + hq.
    int64_t bh, qblk;
    if (a.xcd_map) {
        const int64_t L = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
        const int64_t per_unit = (int64_t)a.G * a.nqb;
        const int64_t kk = L / kXcds;
        const int64_t unit = (L % kXcds) + kXcds * (kk / per_unit);   // b * Hkv + hkv
        const int64_t r = kk % per_unit;
        const int64_t Hkv = a.Hq / a.G;
        const int64_t ub = unit / Hkv, uh = unit - ub * Hkv;
        bh = ub * a.Hq + uh * a.G + r % a.G;
        qblk = a.nqb - 1 - r / a.G;
    } else {
        bh = blockIdx.y;
        qblk = blockIdx.x;
    }
    const int64_t b = bh / a.Hq, hq = bh - b * a.Hq;
    const int64_t hkv = hq / a.G;
    const int64_t q0 = qblk * kPreQ;                    // first query of the workgroup (chunk-relative)
    const int64_t qw = q0 + wave * 16 * QB;             // first query of this wave

    const uint8_t *kbase = (const uint8_t *)a.k + (b * (a.Hq / a.G) + hkv) * a.T * D * 2;
    const uint8_t *vbase = (const uint8_t *)a.v + (b * (a.Hq / a.G) + hkv) * a.T * D * 2;
    const uint32_t kv_bytes = (uint32_t)(a.T * D * 2);
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, kv_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, kv_bytes);

    // keys this workgroup needs: 0 .. min(prefix + q0 + kPreQ, T) - 1
    const int64_t kend = min(a.prefix + q0 + kPreQ, a.T);
    const int ntiles = (int)((kend + kPreKeys - 1) / kPreKeys);

    // ---- Q^T operands (B of S^T): query qw + 16 qb + n, channels 32 ks + 8 g ..
    u32x4 Qb[QB][NKS];
    {
        const uint8_t *qbase = (const uint8_t *)a.q + bh * a.C * D * 2;
        const uint32_t q_bytes = (uint32_t)(a.C * D * 2);
        const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qbase, q_bytes);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                Qb[qb][ks] = buf_load16(qrs, (uint32_t)((qw + 16 * qb + n) * D + 32 * ks + 8 * g) * 2);
    }

    // ---- staging of one K/V tile ------------------------------------------
    // K: thread chunk c = tid + 256 j -> (key c / CPR, 8 channels), stored as is.
    // V: thread (pair c % 32, channel chunk c / 32) loads keys 2 pair and
    // 2 pair + 1 of one 8-channel chunk and stores each channel's two keys as
    // one dword of V^T: consecutive lanes write consecutive dwords.
    u32x4 kreg[NLD], vreg[NV][2];
    auto load_tile = [&](int t) {
        const int64_t r0 = (int64_t)t * kPreKeys;
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int c = tid + kPreThreads * j;
            if (c < NKA) {
                const int key = c / CPR, col = (c % CPR) * 8;
                kreg[j] = buf_load16(krs, (uint32_t)((r0 + key) * D + col) * 2);   // rows past T read as zeros
            }
        }
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int c = tid + kPreThreads * j;
            if (c < NVA) {
                const int pair = c % (kPreKeys / 2), col = (c / (kPreKeys / 2)) * 8;
                vreg[j][0] = buf_load16(vrs, (uint32_t)((r0 + 2 * pair) * D + col) * 2);
                vreg[j][1] = buf_load16(vrs, (uint32_t)((r0 + 2 * pair + 1) * D + col) * 2);
            }
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int c = tid + kPreThreads * j;
            if (c >= NKA) continue;
            const int key = c / CPR, col = (c % CPR) * 8;
            *(u32x4 *)&k_lds[key * KSTR + col] = kreg[j];
        }
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int c = tid + kPreThreads * j;
            if (c >= NVA) continue;
            const int pair = c % (kPreKeys / 2), col = (c / (kPreKeys / 2)) * 8;
            const int kp = vt_pos(2 * pair);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t a0 = vreg[j][0][e], a1 = vreg[j][1][e];
                *(uint32_t *)&vt_lds[(col + 2 * e) * VSTR + kp] = (a0 & 0xFFFFu) | (a1 << 16);
                *(uint32_t *)&vt_lds[(col + 2 * e + 1) * VSTR + kp] = (a0 >> 16) | (a1 & 0xFFFF0000u);
            }
        }
    };

    // ---- running state per query (lane n of each block) ---------------------
    float m_run[QB], l_run[QB];                   // l: this lane's keys only; summed over g at the end
    f32x4 acc[QB][NCB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = neg_inf();
        l_run[qb] = 0.f;
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
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
        // (the first step of each chain starts from a zero accumulator operand)
        f32x4 st[QB][NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const u32x4 ka = *(const u32x4 *)&k_lds[(16 * kb + n) * KSTR + 32 * ks + 8 * g];
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    st[qb][kb] = mfma16<F>(ka, Qb[qb][ks], ks == 0 ? (f32x4){0.f, 0.f, 0.f, 0.f} : st[qb][kb]);
            }

        // online softmax per query; build P^T operands (hi and lo terms).
        // The causal mask only matters on tiles that reach past the wave's
        // first query (a wave-uniform test).  The running max is raised
        // lazily: only when some query of the wave sees a score more than
        // kLazy above its current max are that wave's accumulators rescaled;
        // otherwise p = 2^(s - m) may reach 2^kLazy, which fp32 sums and the
        // two 16-bit terms carry without loss.
        const bool diag = t0 + kPreKeys - 1 > a.prefix + qw;
        u32x4 ph[QB][NS2], pl[QB][NS2];               // [qb][32-key step]
        float mx[QB];                                 // raw (unscaled) tile max per query
        bool up = false;
        if (diag) {                                   // wave-uniform: only tiles on the diagonal
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int rel = (int)(a.prefix + qw - t0) + 16 * qb + n - 4 * g;   // qpos - (t0 + 4 g)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (16 * kb + i > rel) st[qb][kb][i] = neg_inf();
            }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float m = neg_inf();
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) m = fmaxf(m, st[qb][kb][i]);
            // LDS lane shuffles here: this loop is bound by its VALU issue,
            // and the VALU butterfly (permlane swaps) measured slower
            m = fmaxf(m, __shfl_xor(m, 16, 64));
            mx[qb] = fmaxf(m, __shfl_xor(m, 32, 64));
            up |= mx[qb] * sl2 > m_run[qb] + kLazy;
        }
        if (__builtin_amdgcn_ballot_w64(up) != 0) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float mnew = fmaxf(m_run[qb], mx[qb] * sl2);
                const float alpha = (mnew == m_run[qb]) ? 1.f : fast_exp2(m_run[qb] - mnew);
                m_run[qb] = mnew;
                l_run[qb] *= alpha;
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) acc[qb][cb] *= alpha;
            }
        }
        // softmax of block qb: P^T operands (hi and lo terms) and the row sum
        auto softmax_block = [&](int qb) {
            const float nm = -m_run[qb];
            float lsum = 0.f;
            uint32_t hw[NKB][2], lw[NKB][2];              // [kb][pair of keys]
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int i2 = 0; i2 < 2; ++i2) {
                    // 2^(s scale log2e - m); a masked s = -inf gives 0
                    const float p0 = fast_exp2(fmaf(st[qb][kb][2 * i2], sl2, nm));
                    const float p1 = fast_exp2(fmaf(st[qb][kb][2 * i2 + 1], sl2, nm));
                    lsum += p0 + p1;
                    const uint32_t h = pack16<F>(p0, p1);
                    hw[kb][i2] = h;
                    lw[kb][i2] = pack16<F>(p0 - lo16<F>(h), p1 - hi16<F>(h));
                }
            l_run[qb] += lsum;
            // step s2 covers keys 32 s2 .. 32 s2 + 31: slots 0-3 <- block 2 s2, 4-7 <- block 2 s2 + 1
#pragma unroll
            for (int s2 = 0; s2 < NS2; ++s2) {
                ph[qb][s2] = (u32x4){hw[2 * s2][0], hw[2 * s2][1], hw[2 * s2 + 1][0], hw[2 * s2 + 1][1]};
                pl[qb][s2] = (u32x4){lw[2 * s2][0], lw[2 * s2][1], lw[2 * s2 + 1][0], lw[2 * s2 + 1][1]};
            }
        };
        // O^T += V^T P^T of block qb: A = channels 16 cb + m, keys in the P^T slot order
        auto pv_block = [&](int qb) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int s2 = 0; s2 < NS2; ++s2) {
                    // slots 0-3: keys 32 s2 + 4 g .. + 3; 4-7: keys 32 s2 + 16 + 4 g .. + 3
                    const u32x4 va = *(const u32x4 *)&vt_lds[(16 * cb + n) * VSTR + 32 * s2 + 8 * g];
                    acc[qb][cb] = mfma16<F>(va, ph[qb][s2], acc[qb][cb]);
                    acc[qb][cb] = mfma16<F>(va, pl[qb][s2], acc[qb][cb]);
                }
        };
        // the products of block qb and the softmax of block qb + 1 are
        // independent, so the matrix cores and the VALU can work side by side
        softmax_block(0);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            pv_block(qb);
            if (qb + 1 < QB) softmax_block(qb + 1);
        }
        if constexpr (QB == 2) {
            // instruction order for the scheduler: block 0's softmax, then
            // block 0's products each followed by a few VALU instructions of
            // block 1's softmax, then block 1's products
#pragma unroll
            for (int i = 0; i < kSgVa; ++i) __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
#pragma unroll
            for (int i = 0; i < 2 * NCB * NS2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, kSgVb, 0);
            }
#pragma unroll
            for (int i = 0; i < 2 * NCB * NS2; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
    }

    // ---- normalise and store: lane holds channels 16 cb + 4 g .. + 3 of query n
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        float l = l_run[qb];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
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

constexpr int kPreQB = 2;           // query blocks per wave (measured on MI355X)

PrefillFn prefill_pick(int fmt, int D) {
    if (fmt == FMT_BF16)
        return D == 64 ? prefill_kernel<FMT_BF16, 64, kPreQB> : (D == 128 ? prefill_kernel<FMT_BF16, 128, kPreQB> : nullptr);
    if (fmt == FMT_F16)
        return D == 64 ? prefill_kernel<FMT_F16, 64, kPreQB> : (D == 128 ? prefill_kernel<FMT_F16, 128, kPreQB> : nullptr);
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
    a.nqb = (int32_t)qblocks;
    a.xcd_map = (B * Hkv) % kXcds == 0;
    hipLaunchKernelGGL(fn, dim3((unsigned)qblocks, (unsigned)(B * Hq)), dim3(pre_threads<kPreQB>()), 0, stream, a);
    return hipGetLastError();
}

}  // namespace da
