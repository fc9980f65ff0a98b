// The split-K partial pass of decode attention (attn_split_kernel) and its
// helpers, shared by the two units that instantiate it: attn.hip (fp32,
// fp16 and bf16 caches, the merges and the launch code) and attn_u4.hip
// (uint4 caches, compiled with the MFMA accumulators kept in VGPRs).
//
// Split-K decode attention for gfx950 (CDNA4).
//
// Computes, per (batch row b, KV head h) and each of its G query heads, the
// decode-attention output softmax(scale * q . k_i) v_i over a token range
// (HeadInfer, section "核心 idea", per-head equation; TinyServe, section
// "方法细节", Attn and SparseAttn).  One wave reduces one split of the range
// to a partial (running max, running sum, unnormalised output); a second
// kernel merges the splits, unless all splits of a (b, h) fit in one
// workgroup, whose waves then merge them through LDS.
//
// Mapping to the hardware
//   * q.K^T runs on the matrix cores.  A 16x16x32 MFMA takes 16 tokens as its
//     N dimension; every lane loads 16 bytes of one token's key row straight
//     from HBM into the B operand (no LDS round trip).  The 16 rows of the A
//     operand hold the G query heads, each split into several bf16/fp16 terms
//     (hi + mid + lo) when q is fp32, so the products are exact and the sum is
//     fp32-accurate; for a uint4 cache the rows also separate the two
//     64-channel quantization groups so their scales can be applied after,
//     and the codes enter as the exact fp16 values 1 + c/16.  With grouped
//     query heads and a uint4 cache the products are int8 instead: the codes
//     as bytes, q of each (head, group) as a 22-bit fixed-point integer in
//     three int8 digits (A rows), so q . c comes out exact per digit.  With
//     one query head per KV head (uint4, MHA) q fills all 16 rows, so every
//     lane group receives scores and each lane scores the token whose
//     min/scale words it loaded itself (no metadata shuffles; the tile max by
//     DPP).
//   * P.V runs on the VALU in fp32: each lane owns a fixed set of channels and
//     accumulates them over the tokens it loads (16-byte coalesced loads).
//     For a uint4 cache with grouped query heads it runs on the matrix cores
//     instead (bf16 weights in two terms, the codes as bf16 1 + c/16, staged
//     through LDS; see pv_mma).
//   * Online softmax per 32- or 64-token tile in base 2 (exp2 with log2(e) folded
//     into the scale); the per-head tile max is reduced with lane shuffles
//     and broadcast with readlane; accumulators are rescaled only when a max
//     changes (uint4 with grouped query heads: only when it grows by more
//     than 2^8, kLazyMax).
//   * A workgroup holds 1..4 waves, one split each.  Partials go to the
//     workspace and attn_reduce combines the splits of each query head; or,
//     when the workgroup holds every split of its (b, h), the partials go to
//     LDS and the workgroup merges them itself, in the same order as
//     attn_reduce (so both routes give identical bits).
#pragma once

#include "common.h"

#include <math.h>

namespace da {
namespace {

using namespace dev;


constexpr int kSub = 16;               // tokens per MFMA (its N dimension)
// uint4 with grouped query heads: a head's running max moves only when a
// tile's max passes it by more than this (base-2 logits), so p <= 2^8 and
// most tiles skip the accumulator rescale
constexpr float kLazyMax = 8.f;
constexpr int kMaxPagesPerSplit = 1024;

// Pages per split of a paged launch.
__host__ __device__ inline int pages_per_split(int split_tokens, int log2_page) {
    const int pps = split_tokens >> log2_page;
    return pps < 1 ? 1 : (pps > kMaxPagesPerSplit ? kMaxPagesPerSplit : pps);
}

// Dynamic LDS of the in-workgroup merge: one partial [G][D + 4] per wave.
__host__ __device__ inline size_t merge_lds_bytes(int wpb, int G, int D) {
    return (size_t)wpb * G * (D + 4) * sizeof(float);
}
// Dynamic LDS per wave of uint4 P.V on the matrix cores (stage of TILE
// tokens): the V codes (TILE x 64 B), then the bf16 weights (2 x 16 x TILE).
template <int TILE> constexpr size_t kPvvBytes = (size_t)TILE * 64;
template <int TILE> constexpr size_t kPvmWaveBytes = kPvvBytes<TILE> + (size_t)2 * 16 * TILE * 2;

// Compile-time layout of one kernel instance.
template <int KF, int QF, int D, int G>
struct Cfg {
    static constexpr bool U4 = KF == FMT_U4;
    static constexpr int R = KF == FMT_F32 ? 4 * D : (U4 ? D / 2 : 2 * D);   // row bytes
    static constexpr int NGRP = U4 ? D / 64 : 1;        // quantization groups per row
    // number of terms q is split into for the MFMA input type (uint4 with
    // grouped query heads: one, q enters the int8 products as digits)
    static constexpr int SPL = (KF == FMT_F32) ? 1
                             : (QF == KF || (U4 && (QF == FMT_F16 || G > 1))) ? 1
                             : (KF == FMT_BF16 ? (G <= 4 ? 3 : 2) : 2);
    static constexpr int RPH0 = SPL * NGRP;            // A rows used per head
    // uint4 with 2 or 4 query heads: four rows per head (the int8 scores'
    // three digits and a zero row), so each lane group scores one head and
    // the per-head work after the scores (softmax, P.V weights) spreads over
    // the lane groups; with 8 heads, two blocks of A rows, and lane group g
    // scores heads g and g + 4 (HPL = 2)
    static constexpr int RPH = RPH0 <= 1 ? 1 : (RPH0 <= 2 ? ((U4 && G > 1 && G <= 4) ? 4 : 2) : 4);
    static constexpr int HPL = 4 / RPH;                 // heads per 16-lane group
    static constexpr int NCH = R / 64;                  // 16-byte K chunks per lane per sub-tile
    static constexpr int NMF = KF == FMT_F32 ? 4 * NCH : (U4 ? 4 * NCH : NCH);
    static constexpr int VP = R / 64;                   // 16-byte V pieces per lane per sub-tile
    static constexpr int TPP = 1024 / R;                // token stride between V pieces
    static constexpr int CPL = KF == FMT_F32 ? 4 : (U4 ? 32 : 8);   // V channels per lane
    static constexpr int CH_LANES = R / 16;             // lanes covering one row (V side)
    // sub-tiles per pipeline stage (measured on MI355X): 4 for 128-byte rows
    // and for uint4 with grouped query heads (half the per-stage fixed work);
    // 2 otherwise -- the one-head uint4 layout assumes 32-token stages, and
    // deeper stages cost the other layouts occupancy
    static constexpr int TS = (R == 128 || (U4 && G > 1)) ? 4 : 2;
    static constexpr int TILE = kSub * TS;              // tokens per stage
    // uint4 with grouped query heads: q.K^T on the int8 matrix cores
    // (measured on MI355X, uint4 K/V of 8 rows x 8 KV heads x 32768 tokens:
    // G = 4 / 8 took 60.5-60.9 / 72.5 us against 63.3-63.7 / 75.6 us with
    // the fp16 products, G = 2 unchanged at 61.9; the codes need 3 VALU
    // instructions per 8 instead of 9)
    static constexpr bool I8S = U4 && G > 1;
    // minimum waves per SIMD the register allocation must leave room for:
    // four for the one-head uint4 layout (its 3584-wave grid at the FlexGen
    // shape then runs in one round), no constraint otherwise
    static constexpr int WPE = (U4 && G == 1) ? 4 : 1;
    // 16 MFMA rows must hold every (head, group, split term); rows fit 64..1024 bytes
    static constexpr bool ok = RPH0 <= 4 && G * RPH <= 16 && R >= 64 && R <= 1024;
};

typedef int i32x4v __attribute__((ext_vector_type(4)));

// K/V rows are read once per call: load them non-temporally (streaming).
__device__ __forceinline__ u32x4 ld_stream(const char *p) {
    return __builtin_nontemporal_load((const u32x4 *)p);
}

// One dword of 8 codes -> 8 fp16 values 1 + c/16 (exact) in the order of
// qk_dim(): output k moves nibbles k and k + 4 (bits 4k, 4k + 16) to mantissa
// bits 6..9 of its two halves, under the exponent of 1.0.  A dot product with
// them is sum(q) + sum(q c)/16, so sum(q c) = 16 (dot - sum(q)).
// (m << SH) | one in one VALU instruction: the shift is an inline constant
// and `one` a scalar register, so no vector register holds a constant
template <int SH>
__device__ __forceinline__ uint32_t lshl_or(uint32_t m, uint32_t one) {
    uint32_t r;
    asm("v_lshl_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "n"(SH), "s"(one));
    return r;
}
__device__ __forceinline__ u32x4 u4_to_f16x8(uint32_t x) {
    constexpr uint32_t kLo = 0x000F000Fu, kHi = 0x00F000F0u;
    const uint32_t one = __builtin_amdgcn_readfirstlane(0x3C003C00u);
    const uint32_t y = x >> 8;
    u32x4 r;
    r[0] = lshl_or<6>(x & kLo, one);     // nibbles 0, 4
    r[1] = lshl_or<2>(x & kHi, one);     // nibbles 1, 5
    r[2] = lshl_or<6>(y & kLo, one);     // nibbles 2, 6
    r[3] = lshl_or<2>(y & kHi, one);     // nibbles 3, 7
    return r;
}

// (x shifted) & mask | one in two VALU instructions: the shift, then
// v_and_or_b32 with the exponent bits in a scalar register
__device__ __forceinline__ uint32_t and_or(uint32_t m, uint32_t mask, uint32_t one) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(mask), "s"(one));
    return r;
}

// One dword of 8 codes -> 8 bf16 values 1 + c/16 (exact; bf16 keeps 7
// mantissa bits) as the pairs (nibble k, nibble k + 4), k = 0..3: output k
// puts nibbles k and k + 4 at mantissa bits 3..6 of its two halves.
__device__ __forceinline__ u32x4 u4_to_bf16x8(uint32_t x) {
    const uint32_t one = __builtin_amdgcn_readfirstlane(0x3F803F80u);
    const uint32_t mask = 0x00780078u;        // mantissa bits 3..6 of both halves
    u32x4 r;
    r[0] = and_or(x << 3, mask, one);
    r[1] = and_or(x >> 1, mask, one);
    r[2] = and_or(x >> 5, mask, one);
    r[3] = and_or(x >> 9, mask, one);
    return r;
}

typedef int v2i32 __attribute__((ext_vector_type(2)));
#define DA_LDS __attribute__((address_space(3)))

// gfx950 LDS transpose read of 4-bit elements: within each group of 16
// lanes, every lane reads 8 bytes (16 nibbles) at its own address, and lane d
// receives nibble d of lane s's 8 bytes in nibble slot s (bits 4s .. 4s + 3
// of the 64-bit result), s = 0..15 (lane layout measured on MI355X).
__device__ __forceinline__ v2i32 lds_read_tr4(const uint32_t *lds, int byte_off) {
    return __builtin_amdgcn_ds_read_tr4_b64_v2i32((DA_LDS v2i32 *)((DA_LDS char *)lds + byte_off));
}

// gfx950 LDS transpose read of 16-bit elements: within each group of 16
// lanes, every lane reads 4 elements at its own address, and lane d receives
// element d mod 4 of lane 4 j + d / 4 in slot j, j = 0..3 (measured on
// MI355X).
typedef short v4i16 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t *lds, int half_off) {
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DA_LDS v4i16 *)((DA_LDS char *)lds + 2 * half_off));
    return make_uint2((uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16),
                      (uint16_t)r[2] | ((uint32_t)(uint16_t)r[3] << 16));
}

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
// two floats rounded to bf16 (nearest, ties to even) in one instruction, low then high
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){a, b}, bf16x2v));
}

// Registers of one pipeline stage: the K and V of TS sub-tiles of 16 tokens.
template <int KF, int QF, int D, int G>
struct Stage {
    using C = Cfg<KF, QF, D, G>;
    u32x4 K[C::TS][C::NCH];
    u32x4 V[C::TS][C::VP];
    bool kok[C::TS];
    // uint4: the fp16 (min, min) / (scale, scale) pairs of both groups of the
    // K and V rows of stage token (lane mod tile), one coalesced dword each;
    // with several query heads the lanes that use a token's pair fetch it
    // with a lane shuffle, with one head each lane scores its own token
    uint32_t mk, sk, mv, sv;
    // uint4 with 2 or 4 query heads: the pairs of the tokens this lane
    // scores (ts * 16 + lane mod 16), loaded directly instead of fetched
    // with lane shuffles (measured on MI355X, uint4 K/V of 8 rows x 8 KV
    // heads x 32768 tokens: G = 2 / 4 59.9-60.5 / 61.5-61.7 us against
    // 62.1-62.2 / 61.9-62.6; 24 more VGPRs, so G = 8 keeps the shuffles)
    static constexpr bool DM = C::I8S && G <= 4;
    uint32_t mk4[DM ? C::TS : 1], sk4[DM ? C::TS : 1], mv4[DM ? C::TS : 1], sv4[DM ? C::TS : 1];
};

// In-workgroup merge of the n_split (<= waves) partials in `mrg` ([wave][G]
// [D + 4] fp32) into o.  The operations and their order are those of
// attn_reduce_kernel for n_split <= 4: max; weights 2^(m_s - M); L = (w0 l0 +
// w1 l1) + (w2 l2 + w3 l3) (its shuffle tree; adding to a +0 start is exact,
// the terms are >= 0); O = fma chain over s; o = O / L.
template <int G, int D>
__device__ __forceinline__ void merge_in_workgroup(const AttnLaunch &a, const float *mrg, int b, int hkv, int wave,
                                                   int lane) {
    constexpr int PSTR = D + 4;
    __syncthreads();
    const int ns = a.n_split;
    const int slot = G * PSTR;
    float *ob = a.o + (int64_t)b * a.o_bstride + (int64_t)hkv * G * D;
#pragma unroll 1
    for (int idx = wave * 64 + lane; idx < G * D; idx += a.wpb * 64) {
        const int h = idx / D, d = idx - h * D;
        const float *ps = mrg + h * PSTR;
        float M = neg_inf();
#pragma unroll 1
        for (int s = 0; s < ns; ++s) M = fmaxf(M, ps[s * slot + D]);
        float L01 = 0.f, L23 = 0.f, O0 = 0.f;
        const float O1 = 0.f, O2 = 0.f, O3 = 0.f;
#pragma unroll 1
        for (int s = 0; s < ns; ++s) {
            const float m = ps[s * slot + D];
            const float w = (m == neg_inf()) ? 0.f : fast_exp2(m - M);
            const float pl = fmaf(w, ps[s * slot + D + 1], 0.f);
            if (s < 2) L01 += pl;
            else L23 += pl;
            O0 = fmaf(w, ps[s * slot + d], O0);
        }
        const float L = L01 + L23;
        // L == 0: no split saw a token (every listed page out of range)
        ob[h * D + d] = L > 0.f ? ((O0 + O1) + (O2 + O3)) / L : 0.f;
    }
}

// Each wave reduces one split of one (batch row, KV head) to a partial per
// query head.  Loads of the next tile are issued before the current tile is
// computed (two register stages).  SV = 1 selects int8 score products for the
// one-head uint4 layout (see compute_tile_solo); 0 everywhere else.
template <int KF, int QF, int D, int G, bool PAGED, int SV = 0>
__global__ __launch_bounds__(64 * kMaxWavesPerBlock) __attribute__((amdgpu_waves_per_eu(Cfg<KF, QF, D, G>::WPE))) void attn_split_kernel(AttnLaunch a) {
    using C = Cfg<KF, QF, D, G>;
    static_assert(C::ok, "unsupported layout");
    static_assert(!(PAGED && C::U4), "no paged uint4 cache");
    static_assert(!C::U4 || (C::NGRP == 2 && C::VP == 1 && C::TILE <= 64), "uint4 layout");
    using St = Stage<KF, QF, D, G>;
    constexpr int R = C::R, RPH = C::RPH, HPL = C::HPL, SPL = C::SPL, NGRP = C::NGRP;
    constexpr int NCH = C::NCH, NMF = C::NMF, VP = C::VP, TPP = C::TPP, CPL = C::CPL;
    constexpr int MT = C::U4 ? FMT_F16 : KF;
    constexpr int PSTR = D + 4;        // floats per partial row: u[D], m, l, pad, pad
    constexpr int kTS = C::TS, kTile = C::TILE;
    // uint4 with one query head per KV head: q fills every MFMA row, so every
    // lane group receives scores; group g scores sub-tile g mod 2, and lane l
    // holds stage token l mod 32, whose metadata it loaded itself
    constexpr bool SOLO = C::U4 && G == 1;
    static_assert(!SOLO || (kTS == 2 && kTile == 32), "one-head uint4 layout");
    constexpr bool SOLO8 = SOLO && SV == 1;      // one head, int8 score products
    static_assert(SV == 0 || SOLO, "int8 one-head scores are a one-head uint4 form");

    // uint4 with grouped query heads: P.V runs on the matrix cores (see
    // pv_store and pv_mma below); with one query head per KV head it stays on
    // the VALU, where the one-head layout needs fewer registers (measured on
    // MI355X)
    constexpr bool PVM = C::U4 && G > 1;
    __shared__ float p_all[kMaxWavesPerBlock][(G > 1 && !PVM) ? kTile * G : 1];   // p exchange
    __shared__ int32_t pg_all[kMaxWavesPerBlock][PAGED ? kMaxPagesPerSplit : 1];  // page lists
    // Dynamic LDS: the merge slots (fused launches), then, for uint4 with
    // grouped query heads, per wave a stage's V codes [32 tokens][64 B] and
    // its P.V weights as bf16 [V group][32 tokens][A row = 2 head + term].
    // Sized per launch (pvm_lds_bytes), so single-wave workgroups hold only
    // their own wave's tiles and more of them fit on a CU.
    extern __shared__ float mrg_lds[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int g4 = lane >> 4;          // lane group (MFMA k-chunk / C row block)
    const int n16 = lane & 15;         // token within sub-tile (K side)
    const int split = blockIdx.x * a.wpb + wave;
    const int unit = blockIdx.y;       // b * Hkv + h
    const int b = unit / a.Hkv;
    const int hkv = unit - b * a.Hkv;
    const int pps = PAGED ? pages_per_split(a.split_tokens, a.log2_page) : 0;

    // the score lanes: lane group g4 holds heads hd(g4, 0..HPL-1); with int8
    // scores (I8S) A-row block hh carries heads 4 hh .. 4 hh + 3
    auto hd = [](int g, int hh) { return C::I8S ? g + 4 * hh : g * HPL + hh; };
    auto grp_of = [](int h) { return C::I8S ? h % 4 : h / HPL; };
    auto slot_of = [](int h) { return C::I8S ? h / 4 : h % HPL; };

    float *const p_lds = p_all[wave];
    int32_t *const pg_lds = pg_all[wave];
    uint32_t *pvv = nullptr;
    uint16_t *pvp = nullptr;
    if constexpr (PVM) {
        char *const dyn = (char *)mrg_lds + (a.fused ? merge_lds_bytes(a.wpb, G, D) : 0) +
                          (size_t)wave * kPvmWaveBytes<kTile>;
        pvv = (uint32_t *)dyn;
        pvp = (uint16_t *)(dyn + kPvvBytes<kTile>);
    }

    // ---- token range of this split (empty past the last split) ----------
    int64_t s0 = 0;
    int ntok;
    int pg_mask = 0;
    if constexpr (PAGED) {
        const int p0 = split * pps;
        const int np = max(0, min(pps, a.top_k - p0));
        const int32_t *lst = a.page_idx + (int64_t)unit * a.top_k + p0;
        for (int i = lane; i < np; i += 64) pg_lds[i] = lst[i];
        ntok = np << a.log2_page;
        pg_mask = (1 << a.log2_page) - 1;
        wave_lds_sync();
    } else {
        s0 = (int64_t)split * a.split_tokens;
        ntok = (int)max((int64_t)0, min((int64_t)a.split_tokens, a.N - s0));
    }

    const int64_t kvoff = (int64_t)b * a.kv_bstride + (int64_t)(hkv / a.kv_group) * a.kv_hstride;
    const char *kbase = (const char *)a.k + kvoff * R;
    const char *vbase = (const char *)a.v + kvoff * R;
    const uint16_t *kmn = nullptr, *ksc = nullptr, *vmn = nullptr, *vsc = nullptr;
    if constexpr (C::U4) {
        kmn = (const uint16_t *)a.kmin + kvoff * NGRP;
        ksc = (const uint16_t *)a.kscale + kvoff * NGRP;
        vmn = (const uint16_t *)a.vmin + kvoff * NGRP;
        vsc = (const uint16_t *)a.vscale + kvoff * NGRP;
    }
    const int64_t qoff = (int64_t)b * a.q_bstride + (int64_t)hkv * G * D;

    const int vcol = (lane * 16) % R;            // V byte column of this lane
    const int vtok = (lane * 16) / R;            // V token within a piece

    auto row_of = [&](int pos, bool &ok) -> int64_t {
        if constexpr (PAGED) {
            ok = pos < ntok;
            if (!ok) return 0;
            const int32_t pg = pg_lds[pos >> a.log2_page];
            const int64_t r = ((int64_t)pg << a.log2_page) + (pos & pg_mask);
            ok = pg >= 0 && r < a.N;
            return ok ? r : 0;
        } else {
            ok = pos < ntok;
            return ok ? s0 + pos : 0;
        }
    };

    // ---- issue the loads of one tile ---------------------------------------
    // dense: buffer resources over this split's rows (rows past the split
    // read as zeros, so the last tile needs no per-lane masks)
    // (unused in paged mode, where they cover nothing)
    const uint32_t kv_bytes = PAGED ? 0u : (uint32_t)ntok * R;
    const uint32_t ms_bytes = (PAGED || !C::U4) ? 0u : (uint32_t)ntok * NGRP * 2;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase + s0 * R, kv_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase + s0 * R, kv_bytes);
    const __amdgpu_buffer_rsrc_t kmrs = make_rsrc(kmn + s0 * NGRP, ms_bytes);
    const __amdgpu_buffer_rsrc_t ksrs = make_rsrc(ksc + s0 * NGRP, ms_bytes);
    const __amdgpu_buffer_rsrc_t vmrs = make_rsrc(vmn + s0 * NGRP, ms_bytes);
    const __amdgpu_buffer_rsrc_t vsrs = make_rsrc(vsc + s0 * NGRP, ms_bytes);

    auto load_tile = [&](St &st, int t0) {
        if constexpr (!PAGED) {
#pragma unroll
            for (int ts = 0; ts < kTS; ++ts) {
                const int rk = t0 + ts * kSub + n16;          // row within the split
                st.kok[ts] = rk < ntok;
#pragma unroll
                for (int c = 0; c < NCH; ++c)
                    st.K[ts][c] = buf_load16(krs, (uint32_t)rk * R + 16 * g4 + 64 * c);
#pragma unroll
                for (int p = 0; p < VP; ++p)
                    st.V[ts][p] = buf_load16(vrs, (uint32_t)(t0 + ts * kSub + p * TPP + vtok) * R + vcol);
            }
            if constexpr (C::U4) {
                if constexpr (St::DM) {
#pragma unroll
                    for (int ts = 0; ts < kTS; ++ts) {
                        const uint32_t o4 = (uint32_t)(t0 + ts * kSub + n16) * NGRP * 2;
                        st.mk4[ts] = buf_load4(kmrs, o4);
                        st.sk4[ts] = buf_load4(ksrs, o4);
                        st.mv4[ts] = buf_load4(vmrs, o4);
                        st.sv4[ts] = buf_load4(vsrs, o4);
                    }
                } else {
                const uint32_t off = (uint32_t)(t0 + lane % kTile) * NGRP * 2;
                st.mk = buf_load4(kmrs, off);
                st.sk = buf_load4(ksrs, off);
                st.mv = buf_load4(vmrs, off);
                st.sv = buf_load4(vsrs, off);
                }
            }
            return;
        }
#pragma unroll
        for (int ts = 0; ts < kTS; ++ts) {
            bool ok;
            const int64_t r = row_of(t0 + ts * kSub + n16, ok);
            st.kok[ts] = ok;
            const char *p = kbase + r * R + 16 * g4;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
                st.K[ts][c] = ok ? ld_stream(p + 64 * c) : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
            for (int p2 = 0; p2 < VP; ++p2) {
                bool okv;
                const int64_t rv = row_of(t0 + ts * kSub + p2 * TPP + vtok, okv);
                st.V[ts][p2] = okv ? ld_stream(vbase + rv * R + vcol) : (u32x4){0u, 0u, 0u, 0u};
            }
        }
    };

    // The two halves of load_tile (fp16 / bf16 caches, and uint4 with up to
    // 4 query heads per KV head, with the minima and scales of each side):
    // the keys of a tile, which the scores consume first, and its values.
    auto load_k = [&](St &st, int t0) {
        if constexpr (St::DM && !PAGED) {
#pragma unroll
            for (int ts = 0; ts < kTS; ++ts) {
                const uint32_t o4 = (uint32_t)(t0 + ts * kSub + n16) * NGRP * 2;
                st.mk4[ts] = buf_load4(kmrs, o4);
                st.sk4[ts] = buf_load4(ksrs, o4);
            }
        }
        if constexpr (SOLO && !PAGED) {
            const uint32_t off = (uint32_t)(t0 + lane % kTile) * NGRP * 2;
            st.mk = buf_load4(kmrs, off);
            st.sk = buf_load4(ksrs, off);
        }
#pragma unroll
        for (int ts = 0; ts < kTS; ++ts) {
            if constexpr (!PAGED) {
                const int rk = t0 + ts * kSub + n16;
                st.kok[ts] = rk < ntok;
#pragma unroll
                for (int c = 0; c < NCH; ++c)
                    st.K[ts][c] = buf_load16(krs, (uint32_t)rk * R + 16 * g4 + 64 * c);
            } else {
                bool ok;
                const int64_t r = row_of(t0 + ts * kSub + n16, ok);
                st.kok[ts] = ok;
                const char *p = kbase + r * R + 16 * g4;
#pragma unroll
                for (int c = 0; c < NCH; ++c)
                    st.K[ts][c] = ok ? ld_stream(p + 64 * c) : (u32x4){0u, 0u, 0u, 0u};
            }
        }
    };
    auto load_v = [&](St &st, int t0) {
        if constexpr (St::DM && !PAGED) {
#pragma unroll
            for (int ts = 0; ts < kTS; ++ts) {
                const uint32_t o4 = (uint32_t)(t0 + ts * kSub + n16) * NGRP * 2;
                st.mv4[ts] = buf_load4(vmrs, o4);
                st.sv4[ts] = buf_load4(vsrs, o4);
            }
        }
        if constexpr (SOLO && !PAGED) {
            const uint32_t off = (uint32_t)(t0 + lane % kTile) * NGRP * 2;
            st.mv = buf_load4(vmrs, off);
            st.sv = buf_load4(vsrs, off);
        }
#pragma unroll
        for (int ts = 0; ts < kTS; ++ts) {
#pragma unroll
            for (int p2 = 0; p2 < VP; ++p2) {
                if constexpr (!PAGED) {
                    st.V[ts][p2] = buf_load16(vrs, (uint32_t)(t0 + ts * kSub + p2 * TPP + vtok) * R + vcol);
                } else {
                    bool okv;
                    const int64_t rv = row_of(t0 + ts * kSub + p2 * TPP + vtok, okv);
                    st.V[ts][p2] = okv ? ld_stream(vbase + rv * R + vcol) : (u32x4){0u, 0u, 0u, 0u};
                }
            }
        }
    };

    // issue the first tile before the q set-up below, so its latency overlaps
    St sa, sb;
    if (ntok > 0) load_tile(sa, 0);

    // ---- A operand: query rows, split into MFMA-type terms -------------------
    // Every lane issues every q load (a row or channel that holds no value
    // reads head 0 and drops it): with no load behind a branch they all go
    // out before the first wait, where conditional loads had cost one
    // memory round trip each (measured on MI355X, see the uint4 one-head
    // pass).
    u32x4 Aq[KF == FMT_F32 ? 1 : NMF];
    float Af[KF == FMT_F32 ? NMF : 1];
    {
        const int m = n16;
        const int h = SOLO ? 0 : m / RPH, within = m % RPH;
        const int grp = within / SPL, s = within % SPL;
        const bool rowok = h < G && within < SPL * NGRP;
#pragma unroll
        for (int mf = 0; mf < NMF; ++mf) {
            if constexpr (KF == FMT_F32) {
                const int d = qk_dim<KF>(mf, g4, 0);
                const float v = load_scalar<QF>(a.q, qoff + (rowok ? h : 0) * D + d);
                Af[mf] = rowok ? v : 0.f;
            } else {
                uint32_t hv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int d = qk_dim<KF>(mf, g4, e);
                    const bool ok = rowok && (!C::U4 || d / 64 == grp);
                    const float v = load_scalar<QF>(a.q, qoff + (ok ? h : 0) * D + d);
                    const float x = ok ? v : 0.f;
                    hv[e] = split_term<MT>(x, s);
                }
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) Aq[mf][e2] = hv[2 * e2] | (hv[2 * e2 + 1] << 16);
            }
        }
    }

    // uint4 with grouped query heads: q of (head h, group gr) as the integer
    // rint(q * 2^e), e from the group's largest |q| so that |q| 2^e < 2^22,
    // in three signed int8 digits d0 2^16 + d1 2^8 + d2 (A row 4 (h mod 4) +
    // digit of block h / 4; row 4 h' + 3 stays zero).  After the key codes
    // are regrouped (see the scores), k-slot byte j of lane group g4 is
    // channel 64 gr + base(g4) + 8 (j / 8) + 2 (j mod 4) + (j / 4) mod 2,
    // base = 0, 32, 16, 48 for g4 = 0..3: the order in which a dword of
    // codes splits into its low and high nibbles.  The rounding of q to 22
    // bits of its group's largest value is below fp32 accumulation error.
    // (one-head layout with SOLO8: head 0's digits in all four row blocks)
    constexpr bool Q8 = C::I8S || SOLO8;
    constexpr int NB8 = C::I8S ? HPL : 1;
    u32x4 Aq8[Q8 ? 2 : 1][NB8];
    float ek[Q8 ? 2 : 1][NB8][3];
    if constexpr (Q8) {
#pragma unroll
        for (int hb = 0; hb < NB8; ++hb) {
        const int m = n16, h = SOLO ? 0 : 4 * hb + (m >> 2), t = m & 3;
#pragma unroll
        for (int gr = 0; gr < 2; ++gr) {
            float qv[16];
            float mx = 0.f;
            int bad = 0;                         // a NaN or an infinity in the group
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int ch = 64 * gr + 32 * (g4 & 1) + 16 * (g4 >> 1) + 8 * (j >> 3) + 2 * (j & 3) + ((j >> 2) & 1);
                const float v = load_scalar<QF>(a.q, qoff + (h < G ? h : 0) * D + ch);
                qv[j] = h < G ? v : 0.f;
                mx = fmaxf(mx, fabsf(qv[j]));
                bad |= !(fabsf(qv[j]) <= 3.402823466e38f);
            }
            mx = xor_reduce<16, 64>(mx, OpMax{});
            bad = xor_reduce<16, 64>(bad, OpOr{});
            int ex;
            (void)frexpf(mx, &ex);
            const int e = 22 - ex;               // |q| 2^e < 2^22
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t dw = 0;
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const int qi = (int)rintf(ldexpf(qv[4 * w + bb], e));
                    const int d2 = (int)(int8_t)(qi & 0xFF);
                    const int q1 = (qi - d2) >> 8;
                    const int d1 = (int)(int8_t)(q1 & 0xFF);
                    const int d0 = (q1 - d1) >> 8;
                    const int dig = (h >= G || t == 3) ? 0 : (t == 0 ? d0 : (t == 1 ? d1 : d2));
                    dw |= (uint32_t)(dig & 0xFF) << (8 * bb);
                }
                Aq8[gr][hb][w] = dw;
            }
            // the score lanes of head hd(g4, hb) take its exponent from row 4 g4;
            // a group holding a NaN or an infinity gets NaN scales, so that
            // head's scores and output are NaN, as the arithmetic would give
            const int es = SOLO ? e : __shfl(e, 4 * g4, 64);
            const int bs = SOLO ? bad : __shfl(bad, 4 * g4, 64);
            const float sc = bs ? __builtin_nanf("") : ldexpf(1.f, -es);
            ek[gr][hb][0] = 65536.f * sc;
            ek[gr][hb][1] = 256.f * sc;
            ek[gr][hb][2] = sc;
        }
        }
    }

    // uint4: per (head, group) sum of q, for the min term of the folded dequantization
    float qs[HPL][NGRP];
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh)
#pragma unroll
        for (int gr = 0; gr < NGRP; ++gr) qs[hh][gr] = 0.f;
    if constexpr (C::U4) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int gr = 0; gr < NGRP; ++gr) {
                float x = load_scalar<QF>(a.q, qoff + h * D + gr * 64 + lane);
                x = xor_reduce<1, 64>(x, OpAdd{});
                if (SOLO || grp_of(h) == g4) qs[slot_of(h)][gr] = x;
            }
    }

    // ---- running state ----------------------------------------------------
    float m_run[G];
#pragma unroll
    for (int h = 0; h < G; ++h) m_run[h] = neg_inf();
    float l_part[HPL];
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh) l_part[hh] = 0.f;
    float acc[PVM ? 1 : G][PVM ? 1 : CPL];
    float amin[G];
#pragma unroll
    for (int h = 0; h < G; ++h) amin[h] = 0.f;
    if constexpr (!PVM) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[h][c] = 0.f;
    }
    // uint4: P.V accumulators, one 16x16 MFMA output per 16-channel block:
    // lane (g4, n) holds rows 4 g4 + i = (head 2 g4 + i / 2, bf16 term i mod 2)
    // of channel 16 nb + n; amg[hh][g]: sum of p * (V group minimum) of head
    // hd(g4, hh) over this lane's tokens (one-head layout: am below)
    f32x4 acc2[PVM ? 8 : 1];
#pragma unroll
    for (int nb = 0; nb < (PVM ? 8 : 1); ++nb) acc2[nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    // and -sum W per V group (the same for all 16-channel blocks of a group)
    f32x4 accn[PVM ? 2 : 1];
#pragma unroll
    for (int g = 0; g < (PVM ? 2 : 1); ++g) accn[g] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float amg[HPL][2];
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh) amg[hh][0] = amg[hh][1] = 0.f;
    if constexpr (PVM) {
        // rows of the weights that no head writes stay zero for the whole call
        u32x4 *z = (u32x4 *)pvp;
        for (int i = lane; i < 2 * 16 * kTile / 8; i += 64) z[i] = (u32x4){0u, 0u, 0u, 0u};
        wave_lds_sync();
    }
    // P.V of one stage on the matrix cores: O += P V over the stage's
    // tokens, per 16-channel block nb (V group nb / 4), as
    //   C += W (1 + c/16)  and, once per V group,  N += W (-1),
    // W = p * (V group scale) as two bf16 terms (A rows 2 h, 2 h + 1), the
    // codes as the exact bf16 values 1 + c/16 (B); the offset product is
    // the same for every channel of a group, so one product per group
    // carries it and C + N = sum W c / 16 at the end (measured on MI355X:
    // 4-5% faster at G = 8 than taking it out per block and stage).  The
    // codes reach the B layout (8 tokens of one channel per lane) through
    // LDS: stored as loaded, read back transposed.
    // The products of a stage run one stage late, after the next stage's
    // scores (pv_store at the end of a stage, pv_mma in the next): the LDS
    // round trip of the weights and codes then overlaps independent work.
    bool pv_pend = false;    // a stage's weights and codes wait in LDS for their products
    auto pv_store = [&](St &st) {
      if constexpr (PVM) {
        uint32_t *vl = pvv;
#pragma unroll
        for (int ts = 0; ts < kTS; ++ts)
            *(u32x4 *)&vl[(ts * kSub + vtok) * 16 + 4 * (lane & 3)] = st.V[ts][0];
      }
    };
    auto pv_mma = [&]() {
      if constexpr (PVM) {
        const uint32_t *vl = pvv;
        wave_lds_sync();    // this wave's weights and codes of the stage are written
        // A operands, rows = (head, term), in the B operand's token order:
        // k-slots 0..7 of lane group g4 hold tokens 8 g4 + {0,4,1,5,2,6,3,7};
        // source lane 4 j + r of a transposed read supplies token slot j, rows
        // 4 r .. 4 r + 3
        const uint16_t *pl = pvp;
        const int jr = n16 >> 2, rr = n16 & 3;
        const int t_lo = 8 * g4 + (jr >> 1) + 4 * (jr & 1);       // slots 0..3: tokens 0, 4, 1, 5
        const u32x4 mones = {0xBF80BF80u, 0xBF80BF80u, 0xBF80BF80u, 0xBF80BF80u};   // bf16 -1
        // source lane (g4, s) of a code read: token 8 g4 + s mod 8, 16-channel
        // chunk 2 j + s / 8 (blocks 2 j and 2 j + 1, V group j / 2)
#pragma unroll
        for (int hf = 0; hf < kTile / 32; ++hf) {      // 32-token halves of the stage
        const int tok = 32 * hf + 8 * g4 + (n16 & 7);
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const uint2 x0 = lds_read_tr16(pl, (g * kTile + 32 * hf + t_lo) * 16 + 4 * rr);
            const uint2 x1 = lds_read_tr16(pl, (g * kTile + 32 * hf + t_lo + 2) * 16 + 4 * rr);   // 2, 6, 3, 7
            const u32x4 Aw = {x0.x, x0.y, x1.x, x1.y};
#pragma unroll
            for (int j = 2 * g; j < 2 * g + 2; ++j) {
                const v2i32 r = lds_read_tr4(vl, tok * 64 + 8 * (2 * j + (n16 >> 3)));
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const int nb = 2 * j + h2;
                    const u32x4 bv = u4_to_bf16x8((uint32_t)r[h2]);
                    acc2[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, Aw),
                                                                       __builtin_bit_cast(bf16x8, bv), acc2[nb], 0, 0, 0);
                }
            }
            accn[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, Aw),
                                                              __builtin_bit_cast(bf16x8, mones), accn[g], 0, 0, 0);
        }
        }
        wave_lds_sync();    // read before the next stage rewrites both tiles
      }
    };
    // W = p * scale of both V groups of one (head h, stage token t): two
    // bf16 terms each (hi, lo = the rest) into rows 2 h and 2 h + 1 of the
    // weights, one dword per group
    auto pv_put2 = [&](int h, int t, float w0, float w1) {
      if constexpr (PVM) {
        const uint32_t hi = pack_bf16(w0, w1);
        const uint32_t lo = pack_bf16(w0 - __uint_as_float(hi << 16), w1 - __uint_as_float(hi & 0xFFFF0000u));
        *(uint32_t *)&pvp[t * 16 + 2 * h] = __builtin_amdgcn_perm(lo, hi, 0x05040100u);
        *(uint32_t *)&pvp[(kTile + t) * 16 + 2 * h] = __builtin_amdgcn_perm(lo, hi, 0x07060302u);
      }
    };
    // rescale the P.V accumulators of this lane's rows (heads 2 g4, 2 g4 + 1)
    auto pv_rescale = [&](const float *alpha) {
      if constexpr (PVM) {
        float aA = 1.f, aB = 1.f;
#pragma unroll
        for (int h2 = 0; h2 < G; ++h2) {
            if (h2 == 2 * g4) aA = alpha[h2];
            if (h2 == 2 * g4 + 1) aB = alpha[h2];
        }
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
            acc2[nb][0] *= aA;
            acc2[nb][1] *= aA;
            acc2[nb][2] *= aB;
            acc2[nb][3] *= aB;
        }
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            accn[g][0] *= aA;
            accn[g][1] *= aA;
            accn[g][2] *= aB;
            accn[g][3] *= aB;
        }
      }
    };

    const float sl2 = a.scale_log2;

    // ---- scores, online softmax and P.V of one loaded tile ---------------------
    auto compute_tile = [&](St &st, auto &&after_scores) {
        float sc[kTS][HPL];

#pragma unroll
        for (int ts = 0; ts < kTS; ++ts) {
          if constexpr (C::I8S) {
            // q . c per group, exact in int32 per digit, then
            // raw = sum_gr min sum(q) + scale (q . c)
            uint32_t kmn2, ksc2;
            if constexpr (St::DM) {
                kmn2 = st.mk4[ts];
                ksc2 = st.sk4[ts];
            } else {
                kmn2 = __shfl(st.mk, ts * kSub + n16, 64);
                ksc2 = __shfl(st.sk, ts * kSub + n16, 64);
            }
            float raw[HPL];
#pragma unroll
            for (int hb = 0; hb < HPL; ++hb) raw[hb] = 0.f;
            // lanes 0..31 keep their first 16 codes (group 0) and take the
            // first 16 of lane + 32 (group 1); lanes 32..63 take the last 16
            // of lane - 32 (group 0) and keep their last 16 (group 1)
            const auto s0 = __builtin_amdgcn_permlane32_swap(st.K[ts][0][0], st.K[ts][0][2], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(st.K[ts][0][1], st.K[ts][0][3], false, false);
            const uint32_t kw[4] = {s0[0], s1[0], s0[1], s1[1]};
#pragma unroll
            for (int gr = 0; gr < 2; ++gr) {
                const uint32_t x0 = kw[2 * gr], x1 = kw[2 * gr + 1];
                const u32x4 bv = {x0 & 0x0F0F0F0Fu, (x0 >> 4) & 0x0F0F0F0Fu, x1 & 0x0F0F0F0Fu, (x1 >> 4) & 0x0F0F0F0Fu};
                const i32x4v z = {0, 0, 0, 0};
                const float mn = f16_to_f32((kmn2 >> (16 * gr)) & 0xFFFFu);
                const float sg = f16_to_f32((ksc2 >> (16 * gr)) & 0xFFFFu);
#pragma unroll
                for (int hb = 0; hb < HPL; ++hb) {
                    const i32x4v tt = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4v, Aq8[gr][hb]),
                                                                            __builtin_bit_cast(i32x4v, bv), z, 0, 0, 0);
                    const float dq = fmaf((float)tt[0], ek[gr][hb][0],
                                          fmaf((float)tt[1], ek[gr][hb][1], (float)tt[2] * ek[gr][hb][2]));
                    raw[hb] += fmaf(mn, qs[hb][gr], sg * dq);
                }
            }
#pragma unroll
            for (int hb = 0; hb < HPL; ++hb)
                sc[ts][hb] = (hd(g4, hb) < G && st.kok[ts]) ? raw[hb] * sl2 : neg_inf();
          } else {
            f32x4 cc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                if constexpr (KF == FMT_F32) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        cc = __builtin_amdgcn_mfma_f32_16x16x4f32(Af[4 * c + e], __uint_as_float(st.K[ts][c][e]), cc, 0, 0, 0);
                } else if constexpr (KF == FMT_BF16) {
                    cc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, Aq[c]),
                                                                 __builtin_bit_cast(bf16x8, st.K[ts][c]), cc, 0, 0, 0);
                } else if constexpr (KF == FMT_F16) {
                    cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, Aq[c]),
                                                                __builtin_bit_cast(f16x8, st.K[ts][c]), cc, 0, 0, 0);
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, Aq[4 * c + u]),
                                                                    __builtin_bit_cast(f16x8, u4_to_f16x8(st.K[ts][c][u])), cc, 0, 0, 0);
                }
            }
#pragma unroll
            for (int hh = 0; hh < HPL; ++hh) {
                const int h = hd(g4, hh);
                float raw = 0.f;
                if constexpr (C::U4) {
                    // this lane's K token (ts, n16): its (min, min) and (scale, scale) pairs
                    const uint32_t kmn2 = __shfl(st.mk, ts * kSub + n16, 64);
                    const uint32_t ksc2 = __shfl(st.sk, ts * kSub + n16, 64);
#pragma unroll
                    for (int gr = 0; gr < NGRP; ++gr) {
                        float dot = 0.f;
#pragma unroll
                        for (int s = 0; s < SPL; ++s) dot += cc[hh * RPH + gr * SPL + s];
                        const float mn = f16_to_f32((kmn2 >> (16 * gr)) & 0xFFFFu);
                        const float sg = f16_to_f32((ksc2 >> (16 * gr)) & 0xFFFFu);
                        // q . (mn + c sg) = mn sum(q) + 16 sg (dot - sum(q))
                        raw += mn * qs[hh][gr] + (16.f * sg) * (dot - qs[hh][gr]);
                    }
                } else {
#pragma unroll
                    for (int s = 0; s < SPL; ++s) raw += cc[hh * RPH + s];
                }
                sc[ts][hh] = (h < G && st.kok[ts]) ? raw * sl2 : neg_inf();
            }
          }
        }

        // the scores are done with st.K (and st.kok)
        after_scores();

        // the previous stage's products, before its accumulators are rescaled below
        if constexpr (PVM) {
            if (pv_pend) pv_mma();
        }

        // online softmax (base 2): per-head tile max over the 16 lanes of a group
        float mt[HPL];
#pragma unroll
        for (int hh = 0; hh < HPL; ++hh) {
            float x = sc[0][hh];
#pragma unroll
            for (int ts = 1; ts < kTS; ++ts) x = fmaxf(x, sc[ts][hh]);
            x = xor_reduce<1, 16>(x, OpMax{});
            mt[hh] = x;
        }
        float alpha[G];
        bool changed = false;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float tmax = readlane_f(mt[slot_of(h)], grp_of(h) * 16);
            float mn = fmaxf(m_run[h], tmax);
            if constexpr (PVM) mn = (tmax > m_run[h] + kLazyMax) ? tmax : m_run[h];
            alpha[h] = (mn == m_run[h]) ? 1.f : fast_exp2(m_run[h] - mn);
            changed |= (mn != m_run[h]);
            m_run[h] = mn;
        }
        if (changed) {
            if constexpr (PVM) {
                pv_rescale(alpha);
            } else {
#pragma unroll
                for (int h = 0; h < G; ++h)
#pragma unroll
                    for (int c = 0; c < CPL; ++c) acc[h][c] *= alpha[h];
            }
#pragma unroll
            for (int hh = 0; hh < HPL; ++hh) {
                const int h = hd(g4, hh);
                float al = 1.f;
#pragma unroll
                for (int h2 = 0; h2 < G; ++h2) if (h2 == h) al = alpha[h2];
                l_part[hh] *= al;
                if constexpr (PVM) {
                    amg[hh][0] *= al;
                    amg[hh][1] *= al;
                }
            }
        }
        // G == 1: head 0's p of token (ts, n16) stays in lane n16 and the P.V
        // lanes fetch it with a lane shuffle; otherwise p goes through LDS.
        // uint4: each lane turns its p into the P.V weights of both V groups
        // (the token's V scale and minimum fetched from the lane that loaded
        // them)
        float p0[kTS];
        uint32_t sv2[kTS], mv2[kTS];
        if constexpr (PVM) {
#pragma unroll
            for (int ts = 0; ts < kTS; ++ts) {
                if constexpr (St::DM) {
                    sv2[ts] = st.sv4[ts];
                    mv2[ts] = st.mv4[ts];
                } else {
                    sv2[ts] = __shfl(st.sv, ts * kSub + n16, 64);
                    mv2[ts] = __shfl(st.mv, ts * kSub + n16, 64);
                }
            }
        }
#pragma unroll
        for (int hh = 0; hh < HPL; ++hh) {
            const int h = hd(g4, hh);
            float mh = 0.f;
#pragma unroll
            for (int h2 = 0; h2 < G; ++h2) if (h2 == h) mh = m_run[h2];
#pragma unroll
            for (int ts = 0; ts < kTS; ++ts) {
                const float p = (sc[ts][hh] == neg_inf()) ? 0.f : fast_exp2(sc[ts][hh] - mh);
                l_part[hh] += p;
                if constexpr (PVM) {
                    if (h < G) {
                        pv_put2(h, ts * kSub + n16, p * f16_to_f32(sv2[ts] & 0xFFFFu), p * f16_to_f32(sv2[ts] >> 16));
#pragma unroll
                        for (int g = 0; g < 2; ++g)
                            amg[hh][g] = fmaf(p, f16_to_f32((mv2[ts] >> (16 * g)) & 0xFFFFu), amg[hh][g]);
                    }
                } else if constexpr (G == 1) {
                    if (hh == 0) p0[ts] = p;
                } else {
                    if (h < G) p_lds[(ts * kSub + n16) * G + h] = p;
                }
            }
        }
        if constexpr (PVM) {
            pv_store(st);
            pv_pend = true;
            return;
        }
        if constexpr (G > 1) wave_lds_sync();

        // P.V on the VALU
        if constexpr (!PVM) {
#pragma unroll
        for (int ts = 0; ts < kTS; ++ts) {
#pragma unroll
            for (int p = 0; p < VP; ++p) {
                const int t = ts * kSub + p * TPP + vtok;
                float pv[G];
                if constexpr (G == 1) {
                    pv[0] = __shfl(p0[ts], p * TPP + vtok, 64);     // lane = token in the sub-tile
                } else {
#pragma unroll
                    for (int h = 0; h < G; ++h) pv[h] = p_lds[t * G + h];
                }
                const u32x4 x = st.V[ts][p];
                if constexpr (KF == FMT_F32) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float xv = __uint_as_float(x[e]);
#pragma unroll
                        for (int h = 0; h < G; ++h) acc[h][e] = fmaf(pv[h], xv, acc[h][e]);
                    }
                } else {
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        float x0, x1;
                        if constexpr (KF == FMT_BF16) {
                            x0 = __uint_as_float(x[e2] << 16);
                            x1 = __uint_as_float(x[e2] & 0xFFFF0000u);
                        } else {
                            x0 = f16_to_f32(x[e2] & 0xFFFFu);
                            x1 = f16_to_f32(x[e2] >> 16);
                        }
#pragma unroll
                        for (int h = 0; h < G; ++h) {
                            acc[h][2 * e2] = fmaf(pv[h], x0, acc[h][2 * e2]);
                            acc[h][2 * e2 + 1] = fmaf(pv[h], x1, acc[h][2 * e2 + 1]);
                        }
                    }
                }
            }
        }
        if constexpr (G > 1) wave_lds_sync();
        }
    };

    // ---- uint4, one query head: each lane scores stage token lane mod 32 ----
    // am: sum of p * (V group minimum) over this lane's tokens, for V group
    // lane / 32 (lanes 32..63 repeat the tokens of lanes 0..31)
    float am = 0.f;
    auto compute_tile_solo = [&](St &st, auto &&after_scores) {
        const bool odd = (g4 & 1) != 0;          // this lane group's sub-tile
        float raw = 0.f;
        if constexpr (SOLO8) {
            // int8 products as with grouped heads (the A rows repeat head 0's
            // three digits four times, so every lane group receives them):
            // fewer VALU instructions and products, a longer chain per stage
            // (measured on MI355X: 86.1 against 86.9 us at the FlexGen shape,
            // 3584 waves; 56.5 against 55.0 us with 8 rows x 8 KV heads x
            // 32768 tokens, 2048 waves); the host picks it for grids of three
            // or more waves per SIMD
            uint32_t kw[kTS][4];
#pragma unroll
            for (int ts = 0; ts < kTS; ++ts) {
                const auto s0 = __builtin_amdgcn_permlane32_swap(st.K[ts][0][0], st.K[ts][0][2], false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(st.K[ts][0][1], st.K[ts][0][3], false, false);
                kw[ts][0] = s0[0];
                kw[ts][1] = s1[0];
                kw[ts][2] = s0[1];
                kw[ts][3] = s1[1];
            }
#pragma unroll
            for (int gr = 0; gr < NGRP; ++gr) {
                i32x4v tt[kTS];
#pragma unroll
                for (int ts = 0; ts < kTS; ++ts) {
                    const uint32_t x0 = kw[ts][2 * gr], x1 = kw[ts][2 * gr + 1];
                    const u32x4 bv = {x0 & 0x0F0F0F0Fu, (x0 >> 4) & 0x0F0F0F0Fu, x1 & 0x0F0F0F0Fu, (x1 >> 4) & 0x0F0F0F0Fu};
                    const i32x4v z = {0, 0, 0, 0};
                    tt[ts] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4v, Aq8[gr][0]),
                                                                   __builtin_bit_cast(i32x4v, bv), z, 0, 0, 0);
                }
                const int d0 = odd ? tt[1][0] : tt[0][0];
                const int d1 = odd ? tt[1][1] : tt[0][1];
                const int d2 = odd ? tt[1][2] : tt[0][2];
                const float dq = fmaf((float)d0, ek[gr][0][0], fmaf((float)d1, ek[gr][0][1], (float)d2 * ek[gr][0][2]));
                const float mn = f16_to_f32((st.mk >> (16 * gr)) & 0xFFFFu);
                const float sg = f16_to_f32((st.sk >> (16 * gr)) & 0xFFFFu);
                raw += fmaf(mn, qs[0][gr], sg * dq);
            }
        } else {
        f32x4 cc[kTS];
#pragma unroll
        for (int ts = 0; ts < kTS; ++ts) {
            cc[ts] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 4; ++u)
                cc[ts] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, Aq[u]),
                                                                __builtin_bit_cast(f16x8, u4_to_f16x8(st.K[ts][0][u])),
                                                                cc[ts], 0, 0, 0);
        }
#pragma unroll
        for (int gr = 0; gr < NGRP; ++gr) {
            float dot = 0.f;
#pragma unroll
            for (int s = 0; s < SPL; ++s) dot += odd ? cc[1][gr * SPL + s] : cc[0][gr * SPL + s];
            const float mn = f16_to_f32((st.mk >> (16 * gr)) & 0xFFFFu);
            const float sg = f16_to_f32((st.sk >> (16 * gr)) & 0xFFFFu);
            raw += mn * qs[0][gr] + (16.f * sg) * (dot - qs[0][gr]);
        }
        }
        const float sc = (odd ? st.kok[1] : st.kok[0]) ? raw * sl2 : neg_inf();
        after_scores();
        const float rmax = row16_max(sc);
        const float mn = fmaxf(m_run[0], fmaxf(readlane_f(rmax, 0), readlane_f(rmax, 16)));
        if (mn != m_run[0]) {
            const float alpha = fast_exp2(m_run[0] - mn);
            am *= alpha;
            l_part[0] *= alpha;
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[0][c] *= alpha;
            m_run[0] = mn;
        }
        const float p = (sc == neg_inf()) ? 0.f : fast_exp2(sc - m_run[0]);
        if (lane < 32) l_part[0] += p;
        // this lane's V group (lane / 32): its minimum and scale for the token
        const int gsh = lane < 32 ? 0 : 16;
        const float vmn1 = f16_to_f32((st.mv >> gsh) & 0xFFFFu);
        const float vsc1 = f16_to_f32((st.sv >> gsh) & 0xFFFFu);
        am = fmaf(p, vmn1, am);
        const float pw = p * vsc1;
        // P.V: the V lanes take p * scale of their token and group from the
        // lane that scored it (lane = token + 32 * group)
#pragma unroll
        for (int ts = 0; ts < kTS; ++ts) {
            const float wv = __shfl(pw, ts * kSub + vtok + 32 * (vcol / 32), 64);
            const float wv16 = wv * 0.0625f;
            const u32x4 x = st.V[ts][0];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t lo = opaque(x[u] & 0x0F0F0F0Fu);
                const uint32_t hi = opaque(x[u] & 0xF0F0F0F0u);
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    acc[0][8 * u + 2 * bb] = fmaf(wv, ubyte_f32(lo, bb), acc[0][8 * u + 2 * bb]);
                    acc[0][8 * u + 2 * bb + 1] = fmaf(wv16, ubyte_f32(hi, bb), acc[0][8 * u + 2 * bb + 1]);
                }
            }
        }
    };
    auto compute = [&](St &st) {
        if constexpr (SOLO) compute_tile_solo(st, [] {});
        else compute_tile(st, [] {});
    };

    // ---- main loop: two register stages -------------------------------------
    // Early refill (below) on dense fp16 / bf16 caches with up to 4 query
    // heads per KV head (measured on MI355X: the Llama-3-8B step about 0.5%
    // faster), in the one-head uint4 layout (the key codes and their minima
    // and scales refilled after the scores, the value side after the P.V;
    // 128 VGPRs at four waves per SIMD; the FlexGen step about 1.2 us
    // faster) and for uint4 with 2 or 4 query heads per KV head (each lane's
    // own metadata words; 8 x 8 KV heads x 32768 tokens: G = 4 61.6 -> 58.4
    // us, G = 2 58.9 -> 57.4 us).  Elsewhere it needed more registers than
    // the file holds (spills, AGPR copies), cost occupancy, or measured
    // slower (the paged gather; uint4 with 8 query heads, 72.6 -> 74.4 us).
    constexpr bool EARLYK = (!C::U4 && !PAGED && KF != FMT_F32 && G <= 4) || (SOLO && !PAGED) || (St::DM && !PAGED);
    if constexpr (!EARLYK) {
        for (int t0 = 0; t0 < ntok; t0 += 2 * kTile) {
            const bool more = t0 + kTile < ntok;
            if (more) load_tile(sb, t0 + kTile);
            compute(sa);
            if (!more) break;
            if (t0 + 2 * kTile < ntok) load_tile(sa, t0 + 2 * kTile);
            compute(sb);
        }
    } else {
        // a stage's registers are refilled with the tile two ahead as soon as
        // they are free: its keys right after the scores, its values after
        // the P.V, so more loads stay in flight while a stage computes
        if (kTile < ntok) load_tile(sb, kTile);
        for (int t0 = 0; t0 < ntok; t0 += 2 * kTile) {
            const int n2 = t0 + 2 * kTile, n3 = t0 + 3 * kTile;
            auto hook_a = [&] {
                if (n2 < ntok) load_k(sa, n2);
            };
            if constexpr (SOLO) compute_tile_solo(sa, hook_a);
            else compute_tile(sa, hook_a);
            if (n2 < ntok) load_v(sa, n2);
            if (t0 + kTile >= ntok) break;
            auto hook_b = [&] {
                if (n3 < ntok) load_k(sb, n3);
            };
            if constexpr (SOLO) compute_tile_solo(sb, hook_b);
            else compute_tile(sb, hook_b);
            if (n3 < ntok) load_v(sb, n3);
        }
    }

    if constexpr (PVM) {
        if (pv_pend) pv_mma();     // the last stage's products
    }

    // ---- partial of this split ------------------------------------------------
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh) {
        float x = l_part[hh];
        x = xor_reduce<1, SOLO ? 32 : 16>(x, OpAdd{});
        l_part[hh] = x;
    }
    // uint4: the minimum term of each (head, V group), for the lanes whose
    // P.V rows hold that head: amr[a][g] for head 2 g4 + a
    float amr[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
    if constexpr (SOLO) {
        // per V group: lanes 0..31 sum group 0, lanes 32..63 group 1; the V
        // lanes of channel group vcol / 32 add it to their channels
        am = xor_reduce<1, 32>(am, OpAdd{});
        amin[0] = __shfl(am, 32 * (vcol / 32), 64);
    } else if constexpr (PVM) {
#pragma unroll
        for (int hh = 0; hh < HPL; ++hh)
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                float x = amg[hh][g];
                x = xor_reduce<1, 16>(x, OpAdd{});
                amg[hh][g] = x;
            }
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const float x = readlane_f(amg[slot_of(h)][g], 16 * grp_of(h));
                if (h == 2 * g4) amr[0][g] = x;
                if (h == 2 * g4 + 1) amr[1][g] = x;
            }
    }
    if constexpr (SOLO) {
        // one-head uint4: lane l holds 32 channels 32 (l mod 4) + k summed
        // over token slot l / 4; reduce over the slots as a reduce-scatter:
        // at each step over lane bit b a lane keeps half of its values, adds
        // its partner's copies of them and passes on the other half, so the
        // lane ends with the two channels 32 (l mod 4) + 2 (l / 4) + {0, 1}
        // (30 exchanges and 30 additions instead of 128 each)
        float *v = acc[0];
#pragma unroll
        for (int j = 0; j < 16; ++j) {       // bit 5: keep j (bit clear) or j + 16
            const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[j]), __float_as_uint(v[j + 16]), false, false);
            v[j] = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {        // bit 4: keep j or j + 8
            const auto pr = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[j]), __float_as_uint(v[j + 8]), false, false);
            v[j] = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
        }
        const bool b3 = (lane & 8) != 0, b2 = (lane & 4) != 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {        // bit 3: keep j or j + 4
            const float send = b3 ? v[j] : v[j + 4], keep = b3 ? v[j + 4] : v[j];
            v[j] = keep + lane_xor<8>(send);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {        // bit 2: keep j or j + 2
            const float send = b2 ? v[j] : v[j + 2], keep = b2 ? v[j + 2] : v[j];
            v[j] = keep + lane_xor<4>(send);
        }
    } else if constexpr (!PVM) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[h][c] = xor_reduce<C::CH_LANES, 64>(acc[h][c], OpAdd{});
        }
    }
    // to the workspace, or to this wave's LDS slot [G][PSTR] for the merge
    // below (two separate store paths, so each keeps its own address space)
    const bool fused = a.fused != 0;
    auto emit = [&](float *dst0, int64_t hstride) {
        if (lane == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) dst0[h * hstride + D] = m_run[h];
        }
        if (n16 == 0) {
#pragma unroll
            for (int hh = 0; hh < HPL; ++hh) {
                const int h = hd(g4, hh);
                if (h < G) dst0[h * hstride + D + 1] = l_part[hh];
            }
        }
        if constexpr (PVM) {
            // u = min term + sum W c = am + 16 (C + N) over both terms, channel 16 nb + n16
#pragma unroll
            for (int a2 = 0; a2 < 2; ++a2) {
                const int h = 2 * g4 + a2;
                if (h < G) {
#pragma unroll
                    for (int nb = 0; nb < 8; ++nb)
                        dst0[h * hstride + 16 * nb + n16] =
                            fmaf(16.f, (acc2[nb][2 * a2] + accn[nb >> 2][2 * a2]) +
                                           (acc2[nb][2 * a2 + 1] + accn[nb >> 2][2 * a2 + 1]),
                                 amr[a2][nb >> 2]);
                }
            }
        } else if constexpr (SOLO) {
            const int ch = 32 * (lane & 3) + 2 * (lane >> 2);
            *(float2 *)(dst0 + ch) = make_float2(acc[0][0] + amin[0], acc[0][1] + amin[0]);
        } else if (lane < C::CH_LANES) {
            const int c0 = KF == FMT_F32 ? vcol / 4 : (C::U4 ? vcol * 2 : vcol / 2);
#pragma unroll
            for (int h = 0; h < G; ++h) {
#pragma unroll
                for (int c = 0; c < CPL; c += 4) {
                    f32x4 v4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v4[e] = acc[h][c + e] + (C::U4 ? amin[h] : 0.f);
                    *(f32x4 *)(dst0 + h * hstride + c0 + c) = v4;
                }
            }
        }
    };
    if (fused) emit(mrg_lds + wave * G * PSTR, PSTR);
    else if (split < a.n_split)
        emit(a.ws + ((int64_t)unit * G * a.n_split + split) * PSTR, (int64_t)a.n_split * PSTR);

    if (fused) merge_in_workgroup<G, D>(a, mrg_lds, b, hkv, wave, lane);
}

}  // namespace

// The uint4 instance for (q format, D, G), or nullptr (attn_u4.hip).
using SplitFnPtr = void (*)(AttnLaunch);
SplitFnPtr pick_split_u4(int qf, int D, int G);

}  // namespace da
