// Query-aware page selection for gfx950 (TinyServe, section "方法细节" and
// Algorithm 1 steps 1-2).
//
// page_meta_kernel: per page of S = 2^log2S tokens and per channel, the min
//   and max of the keys (the page's bounding box).  Exact: min/max of values
//   of the storage type are values of that type.
//
// select_kernel: one workgroup per (batch row, head).
//   1. Bound score r_j = sum_d (q_d M_{j,d} if q_d >= 0 else q_d m_{j,d}),
//      written as q+ . M_j + q- . m_j with q+ = max(q, 0), q- = min(q, 0).
//      The scan reads each page's M and m rows once; it is bound by HBM, so
//      it runs on the VALU with whole-row loads: every lane owns a 16-byte
//      piece of a row, accumulates its exact products (fma) and the lanes of
//      a row add up by shuffles.  Scores stay in LDS (and optionally go to
//      page_score).
//      With EXACT the key rows themselves are read once and scored against q
//      (q . k_i): token-level selection (FlexGen's top-10% sparse attention,
//      section "方法细节").
//   2. Top-K by a most-significant-digit radix select (3 passes: digits of 11,
//      11 and 10 bits) over an order-preserving uint32 image of the fp32
//      scores, one shared LDS histogram per pass (two buffers, so the next
//      pass's is cleared while the current one counts: two barriers a
//      pass; the passes stop once every key left in the chosen bin is kept,
//      usually after the second).  Ties at the K-th score go to the lower
//      page index: the equal keys are ranked by a block-wide prefix count in
//      index order (skipped when every key equal to the K-th is kept).  The kept indices are
//      compacted in index order, so they come out ascending.
//   3. Attend modes continue in the same workgroup: token mode weights the
//      kept tokens' value rows by the softmax of their exact scores, still in
//      LDS; page mode first scores the tokens of the kept pages exactly (the
//      same lane layout), then does the same over them -- TinyServe's whole
//      decode step (Algorithm 1) in one kernel, the kept set and every
//      intermediate in LDS.
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

// Selection modes: bound scores over pages; exact scores over tokens; exact
// scores over tokens followed by attention over the kept tokens.
// SEL_PAGES: bound scores + top-K pages.  SEL_TOKENS: exact scores + top-K
// tokens.  SEL_ATTEND: SEL_TOKENS, then attention over the kept tokens.
// SEL_PAGE_ATTEND: SEL_PAGES, then attention over the tokens of the kept
// pages (TinyServe's whole decode step for one head in one workgroup).
enum SelMode : int { SEL_PAGES = 0, SEL_TOKENS = 1, SEL_ATTEND = 2, SEL_PAGE_ATTEND = 3 };

constexpr bool sel_paged(int mode) { return mode == SEL_PAGES || mode == SEL_PAGE_ATTEND; }
// Threads per workgroup (measured on MI355X): 1024 for pages (P = 2048 at
// the TinyServe shape), 512 for tokens (P = 1024 at the FlexGen shape).
constexpr int sel_threads(int mode) { return sel_paged(mode) ? 1024 : 512; }
// 16-byte loads per lane and array in flight per scoring trip (measured on
// MI355X): 2 for pages (two arrays; more costs the 1024-thread workgroups
// their second slot per CU), 4 for tokens.
constexpr int sel_loads(int mode) { return sel_paged(mode) ? 2 : 4; }

struct SelArgs {
    int64_t P = 0;                 // pages (or tokens) per (b, h)
    int32_t top_k = 0;
    const void *q = nullptr;
    const uint8_t *kmin = nullptr, *kmax = nullptr;   // tokens: kmax = the key rows
    int32_t *page_idx = nullptr;   // may be NULL in SEL_ATTEND
    float *page_score = nullptr;   // optional
    const uint8_t *v = nullptr;    // SEL_ATTEND: value rows, laid out as the keys
    float *o = nullptr;            // SEL_ATTEND: [BH][D] fp32
    float scale_log2 = 0.f;        // SEL_ATTEND: softmax scale * log2(e)
    const uint8_t *k = nullptr;    // SEL_PAGE_ATTEND: key rows [BH][N][D] (v likewise)
    int64_t N = 0;                 // SEL_PAGE_ATTEND: tokens per head
    int32_t log2_page = 0;         // SEL_PAGE_ATTEND: page = 2^log2_page tokens
    // grouped-query heads: workgroup bh = b * Hq + j serves query head j; its
    // metadata, key and value rows are those of KV head b * (Hq / G) + j / G
    int32_t Hq = 1, G = 1;
};

__device__ __forceinline__ uint32_t order_key(float f) {
    if (f == 0.f) f = 0.f;                        // -0 and +0 are one score
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of `v` over the workgroup of NW waves (thread order);
// returns the total through *total.  Uses `buf` (NW + 1 entries).
template <int NW>
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
        uint32_t s = lane < NW ? buf[lane] : 0u;
#pragma unroll
        for (int o = 1; o < NW; o <<= 1) {
            const uint32_t y = __shfl_up(s, o, 64);
            if (lane >= o) s += y;
        }
        if (lane < NW) buf[lane] = s;              // inclusive over waves
    }
    __syncthreads();
    const uint32_t before = (w ? buf[w - 1] : 0u) + x - v;
    *total = buf[NW - 1];
    __syncthreads();
    return before;
}

// Float reduction over the workgroup (NW waves); every thread gets the result.
template <int NW, bool MAX>
__device__ __forceinline__ float block_reduce(float x, float *buf) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if constexpr (MAX) x = xor_reduce<1, 64>(x, OpMax{});
    else x = xor_reduce<1, 64>(x, OpAdd{});
    if (lane == 0) buf[w] = x;
    __syncthreads();
    float r = buf[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) r = MAX ? fmaxf(r, buf[i]) : r + buf[i];
    __syncthreads();
    return r;
}

// Attention of one (b, h) over n selected items: item i has its score
// score(i) in LDS (the raw q . k; -inf for a slot that holds no token) and
// its value row row_of(i).  With M the maximum score,
// w_i = 2^((s_i - M) * scale * log2 e), o = sum_i w_i v_i / sum_i w_i (FlexGen's
// top-k sparse attention, section "方法细节": only the kept tokens' V rows are
// read; TinyServe, section "方法细节", SparseAttn over the selected pages).
// Threads own 16-byte column chunks of the value rows; workgroup slots of CH
// lanes walk the items, four loads in flight per slot (the items of a slot in
// ascending order, one fma chain per channel); the slots are summed by lane
// shuffles within a wave and through LDS across waves.
template <int KF, int D, int NW, typename ScoreF, typename RowF>
__device__ __forceinline__ void attend_items(const SelArgs &args, int64_t bh, int64_t kvh, int n,
                                             int64_t rows_per_head,
                                             ScoreF score, RowF row_of, float *wl, float *red,
                                             uint32_t *scan_buf) {
    constexpr int R = D * Elem<KF>::size;
    constexpr int EPC = 16 / Elem<KF>::size;    // values per 16-byte chunk
    constexpr int CH = R / 16;                  // chunks (lanes) per row
    constexpr int NT = NW * 64;
    constexpr int SLOTS = NT / CH;
    constexpr int UNR = 4;
    const int tid = threadIdx.x;
    float *fbuf = (float *)scan_buf;
    __syncthreads();                            // the items and their scores are complete

    float m = -__builtin_inff();
    for (int i = tid; i < n; i += NT) m = fmaxf(m, score(i));
    const float M = block_reduce<NW, true>(m, fbuf);
    float lsum = 0.f;
    for (int i = tid; i < n; i += NT) {
        const float w = exp2f((score(i) - M) * args.scale_log2);
        wl[i] = w;
        lsum += w;
    }
    const float L = block_reduce<NW, false>(lsum, fbuf);   // also orders wl[] before use

    const int ch = tid % CH, slot = tid / CH;
    const uint8_t *vb = args.v + kvh * rows_per_head * R + 16 * ch;
    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
    for (int i0 = slot; i0 < n; i0 += SLOTS * UNR) {
        u32x4 x[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int i = i0 + u * SLOTS;
            x[u] = i < n ? __builtin_nontemporal_load((const u32x4 *)(vb + row_of(i) * R)) : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int i = i0 + u * SLOTS;
            if (i < n) {
                float f[EPC];
                unpack16<KF>(x[u], f);
                const float w = wl[i];
#pragma unroll
                for (int e = 0; e < EPC; ++e) acc[e] = fmaf(w, f[e], acc[e]);
            }
        }
    }
    // sum the slots of each wave (lanes with the same chunk), then the waves
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = xor_reduce<CH, 64>(acc[e], OpAdd{});
    const int lane = tid & 63, w = tid >> 6;
    if (lane < CH) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) red[w * D + ch * EPC + e] = acc[e];
    }
    __syncthreads();
    for (int d = tid; d < D; d += NT) {
        float sum = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) sum += red[ww * D + d];
        args.o[bh * D + d] = sum / L;
    }
}

template <int KF, int QF, int D, int MODE>
__global__ __launch_bounds__(sel_threads(MODE)) void select_kernel(SelArgs args) {
    constexpr bool EXACT = !sel_paged(MODE);
    constexpr int kSelThreads = sel_threads(MODE);
    constexpr int kSelWaves = kSelThreads / 64;
    const int64_t P = args.P;
    const int top_k = args.top_k;
    const void *__restrict__ q = args.q;
    const uint8_t *__restrict__ kmin = args.kmin;
    const uint8_t *__restrict__ kmax = args.kmax;
    int32_t *__restrict__ page_idx = args.page_idx;
    float *__restrict__ page_score = args.page_score;
    constexpr int R = D * Elem<KF>::size;

    extern __shared__ float sc_lds[];              // [P] (SEL_ATTEND: then kept[top_k], w[top_k])
    // radix histograms: 2048 bins (11-bit digits), two buffers so that a pass
    // can clear the next pass's while it counts; one pad word per 32 bins
    // keeps the scan's reads (lane L: bins 32 L .. 32 L + 31) conflict-free
    constexpr int kBins = 2048, kHist = kBins + kBins / 32;
    __shared__ uint32_t hist[2][kHist];
    __shared__ uint32_t scan_buf[kSelWaves + 1];
    __shared__ uint32_t pick_digit, pick_need, pick_count;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t bh = blockIdx.x;                 // (batch row, query head)
    const int64_t kvh = (bh / args.Hq) * (args.Hq / args.G) + (bh % args.Hq) / args.G;   // its KV head

    // ---- 1. scores ----------------------------------------------------------
    // Lanes own 16-byte pieces of a row: piece = lane mod PCS of row lane / PCS,
    // so one load instruction covers TPI whole rows (whole 128-byte lines;
    // measured on MI355X: non-temporal loads of whole lines stream ~15% faster
    // than the 64-byte halves an MFMA operand layout would need).  Each lane
    // keeps q+ and q- (EXACT: q) for its EPC channels, sums its exact products
    // in two fma chains, and the PCS lanes of a row add up by lane shuffles.
    constexpr int EPC = 16 / Elem<KF>::size;   // channels per piece
    constexpr int PCS = R / 16;                // pieces per row
    constexpr int TPI = 64 / PCS;              // rows per load instruction
    constexpr int NI = sel_loads(MODE);            // load instructions per array per trip
    constexpr int TPT = NI * TPI;              // rows per trip of one wave
    static_assert(PCS >= 4 && PCS <= 64, "row layout");
    const int piece = lane % PCS, rin = lane / PCS;
    float qp[EPC], qn[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
        const float x = load_scalar<QF>(q, bh * D + piece * EPC + e);
        qp[e] = EXACT ? x : fmaxf(x, 0.f);
        qn[e] = fminf(x, 0.f);
    }
    // buffer resources over this head's rows: rows at or past P read as zeros
    const uint32_t head_bytes = (uint32_t)(P * R);
    const __amdgpu_buffer_rsrc_t mxr = make_rsrc(kmax + kvh * P * R, head_bytes);
    const __amdgpu_buffer_rsrc_t mnr = make_rsrc((EXACT ? kmax : kmin) + kvh * P * R, head_bytes);
    {
        const int64_t step = (int64_t)TPT * kSelWaves;
        u32x4 X[NI], Nn[NI];
        for (int64_t base = (int64_t)w * TPT; base < P; base += step) {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const uint32_t off = (uint32_t)(base + i * TPI + rin) * R + 16 * piece;
                X[i] = buf_load16(mxr, off);
                if constexpr (!EXACT) Nn[i] = buf_load16(mnr, off);
            }
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                float fx[EPC];
                unpack16<KF>(X[i], fx);
                float sp = 0.f, sn = 0.f;
#pragma unroll
                for (int e = 0; e < EPC; ++e) sp = fmaf(qp[e], fx[e], sp);
                if constexpr (!EXACT) {
                    float fn[EPC];
                    unpack16<KF>(Nn[i], fn);
#pragma unroll
                    for (int e = 0; e < EPC; ++e) sn = fmaf(qn[e], fn[e], sn);
                }
                float s = EXACT ? sp : sp + sn;
                // LDS lane shuffles in this VALU-heavy scan: the VALU
                // butterfly measured slower here
#pragma unroll
                for (int o = 1; o < PCS; o <<= 1) s += __shfl_xor(s, o, 64);
                const int64_t row = base + i * TPI + rin;
                if (piece == 0 && row < P) {
                    if (s == 0.f) s = 0.f;
                    sc_lds[row] = s;
                    if (page_score) page_score[bh * P + row] = s;
                }
            }
        }
    }
    for (int i = tid; i < kHist; i += kSelThreads) hist[0][i] = 0u;
    __syncthreads();
    // ---- 2. radix select of the top_k largest keys -------------------------
    // MSB-first, digits of 11, 11 and 10 bits, one shared histogram per pass.
    uint32_t prefix = 0, pmask = 0;
    uint32_t need = (uint32_t)top_k;
    uint32_t eq_count = 0;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const uint32_t dmask = pass < 2 ? 0x7FFu : 0x3FFu;
        uint32_t *const h = hist[pass & 1];
        // the other buffer's last reader was the previous pass's scan, which
        // finished before the barrier that ended that pass
        if (pass < 2)
            for (int i = tid; i < kHist; i += kSelThreads) hist[(pass + 1) & 1][i] = 0u;
        for (int64_t i = tid; i < P; i += kSelThreads) {
            const uint32_t key = order_key(sc_lds[i]);
            if ((key & pmask) == prefix) {
                const uint32_t bin = (key >> shift) & dmask;
                atomicAdd(&h[bin + (bin >> 5)], 1u);
            }
        }
        __syncthreads();
        if (w == 0) {
            // lane L holds bins 32 L .. 32 L + 31; candidates in the bins above
            // its range by a suffix sum over the lanes; the 32 bins of the one
            // range that holds the need-th largest key are then scanned by 32
            // lanes at once
            const uint32_t *hl = h + 33 * lane;
            uint32_t loc = 0;
#pragma unroll
            for (int j = 0; j < 32; ++j) loc += hl[j];
            uint32_t suf = loc;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_down(suf, o, 64);
                if (lane + o < 64) suf += y;
            }
            const uint32_t cum = suf - loc;
            const uint64_t hit = __builtin_amdgcn_ballot_w64(cum < need && cum + loc >= need);
            const int lc = __builtin_ctzll(hit);                       // the lane whose range holds it
            const uint32_t base = __builtin_amdgcn_readlane(cum, lc);  // candidates above that range
            // lanes 0..31 take its bins 31 - lane (descending), prefix sums in that order
            const uint32_t cb = lane < 32 ? h[33 * lc + 31 - lane] : 0u;
            uint32_t pre = cb;
#pragma unroll
            for (int o = 1; o < 32; o <<= 1) {
                const uint32_t y = __shfl_up(pre, o, 64);
                if ((lane & 31) >= o) pre += y;
            }
            const uint32_t above = base + pre - cb;
            if (lane < 32 && above < need && above + cb >= need) {
                pick_digit = (uint32_t)(32 * lc + 31 - lane);
                pick_need = need - above;
                pick_count = cb;
            }
        }
        __syncthreads();
        prefix |= pick_digit << shift;
        pmask |= dmask << shift;
        need = pick_need;
        eq_count = pick_count;
        // every key left in the chosen bin is kept: the later digits would
        // only order keys that are all selected anyway
        if (need == eq_count) break;
    }
    // the leading digits (pmask) of the top_k-th largest key; all 32 bits
    // unless the passes stopped early
    const uint32_t T = prefix;

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
        for (int64_t i = i0; i < i1; ++i) n_eq += (order_key(sc_lds[i]) & pmask) == T;
        eq_before = block_exscan<kSelWaves>(n_eq, scan_buf, &tot);
    }
    uint32_t n_sel = 0;
    {
        uint32_t r = eq_before;
        for (int64_t i = i0; i < i1; ++i) {
            const uint32_t key = order_key(sc_lds[i]) & pmask;
            if (key > T) ++n_sel;
            else if (key == T) { if (all_ties || r < need) ++n_sel; ++r; }
        }
    }
    uint32_t pos = block_exscan<kSelWaves>(n_sel, scan_buf, &tot);
    int32_t *out = page_idx ? page_idx + bh * top_k : nullptr;
    int32_t *kept = (int32_t *)(sc_lds + P);       // SEL_ATTEND: kept indices, ascending
    {
        uint32_t r = eq_before;
        for (int64_t i = i0; i < i1; ++i) {
            const uint32_t key = order_key(sc_lds[i]) & pmask;
            bool sel = key > T;
            if (key == T) { sel = all_ties || r < need; ++r; }
            if (sel && pos < (uint32_t)top_k) {
                if (out) out[pos] = (int32_t)i;
                if constexpr (MODE == SEL_ATTEND || MODE == SEL_PAGE_ATTEND) kept[pos] = (int32_t)i;
                ++pos;
            }
        }
    }
    if constexpr (MODE == SEL_ATTEND) {
        // kept[] holds exactly top_k indices in [0, P); the clamp only guards memory
        auto row = [&](int i) -> int64_t {
            const int32_t t = kept[i];
            return (t >= 0 && t < P) ? t : 0;
        };
        float *wl = (float *)(kept + top_k);
        attend_items<KF, D, kSelWaves>(args, bh, kvh, top_k, P, [&](int i) { return sc_lds[row(i)]; }, row, wl,
                                       wl + top_k, scan_buf);
    }
    if constexpr (MODE == SEL_PAGE_ATTEND) {
        // ---- 4. exact scores of the kept pages' tokens ---------------------
        // slot t holds token kept[t / S] * S + t mod S; slots past n_ctx (the
        // last page's tail) score -inf.  Same lane layout as the bound scan,
        // with q itself (q+ + q-, one of them zero).
        __syncthreads();                             // kept[] complete
        const int lg = args.log2_page;
        const int T = top_k << lg;
        const int64_t N = args.N;
        float *tsc = (float *)(kept + top_k);        // [T]
        float qe[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) qe[e] = qp[e] + qn[e];
        auto tok = [&](int t) -> int64_t {
            const int32_t pg = kept[t >> lg];
            const int64_t r = ((int64_t)(pg >= 0 && pg < P ? pg : 0) << lg) + (t & ((1 << lg) - 1));
            return r < N ? r : -1;
        };
        // one array here (the bound scan reads two): twice the loads per trip
        constexpr int NI4 = 2 * NI, TPT4 = NI4 * TPI;
        const uint8_t *kb = args.k + kvh * N * R + 16 * piece;
        for (int base = w * TPT4; base < T; base += TPT4 * kSelWaves) {
            u32x4 X[NI4];
            int64_t rr[NI4];
#pragma unroll
            for (int i = 0; i < NI4; ++i) {
                const int t = base + i * TPI + rin;
                rr[i] = t < T ? tok(t) : -1;
                X[i] = rr[i] >= 0 ? __builtin_nontemporal_load((const u32x4 *)(kb + rr[i] * R)) : (u32x4){0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int i = 0; i < NI4; ++i) {
                float fx[EPC];
                unpack16<KF>(X[i], fx);
                float s = 0.f;
#pragma unroll
                for (int e = 0; e < EPC; ++e) s = fmaf(qe[e], fx[e], s);
                s = xor_reduce<1, PCS>(s, OpAdd{});
                const int t = base + i * TPI + rin;
                if (piece == 0 && t < T) tsc[t] = rr[i] >= 0 ? s : -__builtin_inff();
            }
        }
        // ---- 5. attention over them ----------------------------------------
        float *wl = tsc + T;
        attend_items<KF, D, kSelWaves>(args, bh, kvh, T, N, [&](int i) { return tsc[i]; },
                                       [&](int i) -> int64_t { const int64_t r = tok(i); return r >= 0 ? r : 0; },
                                       wl, wl + T, scan_buf);
    }
}

using SelFn = void (*)(SelArgs);

template <int KF, int QF, int MODE>
SelFn sel_d(int D) {
    if (D == 64) return select_kernel<KF, QF, 64, MODE>;
    if (D == 128) return select_kernel<KF, QF, 128, MODE>;
    return nullptr;
}

template <int MODE>
SelFn sel_pick(int kv, int qf, int D) {
    switch (kv) {
    case FMT_F32: return qf == FMT_F32 ? sel_d<FMT_F32, FMT_F32, MODE>(D) : nullptr;
    case FMT_F16:
        if (qf == FMT_F16) return sel_d<FMT_F16, FMT_F16, MODE>(D);
        if (qf == FMT_F32) return sel_d<FMT_F16, FMT_F32, MODE>(D);
        return nullptr;
    case FMT_BF16:
        if (qf == FMT_BF16) return sel_d<FMT_BF16, FMT_BF16, MODE>(D);
        if (qf == FMT_F32) return sel_d<FMT_BF16, FMT_F32, MODE>(D);
        return nullptr;
    default: return nullptr;
    }
}

SelFn sel_for(int mode, int kv, int qf, int D) {
    switch (mode) {
    case SEL_PAGES: return sel_pick<SEL_PAGES>(kv, qf, D);
    case SEL_TOKENS: return sel_pick<SEL_TOKENS>(kv, qf, D);
    case SEL_ATTEND: return sel_pick<SEL_ATTEND>(kv, qf, D);
    case SEL_PAGE_ATTEND: return sel_pick<SEL_PAGE_ATTEND>(kv, qf, D);
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

bool select_supported(int kv_fmt, int q_fmt, int D) { return sel_for(SEL_PAGES, kv_fmt, q_fmt, D) != nullptr; }

hipError_t launch_select(int kv_fmt, int q_fmt, int64_t BH, int32_t Hq, int32_t G, int64_t P, int D, int top_k,
                         const void *q, const void *kmin, const void *kmax, int32_t *page_idx, float *page_score,
                         hipStream_t stream, bool exact) {
    const int mode = exact ? SEL_TOKENS : SEL_PAGES;
    SelFn fn = sel_for(mode, kv_fmt, q_fmt, D);
    if (!fn) return hipErrorInvalidValue;
    SelArgs a;
    a.P = P;
    a.top_k = top_k;
    a.q = q;
    a.kmin = (const uint8_t *)kmin;
    a.kmax = (const uint8_t *)kmax;
    a.page_idx = page_idx;
    a.page_score = page_score;
    a.Hq = Hq;
    a.G = G;
    const size_t lds = (size_t)P * sizeof(float);
    hipLaunchKernelGGL(fn, dim3((unsigned)BH), dim3(sel_threads(mode)), lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_topk_attention(int kv_fmt, int q_fmt, int64_t BH, int32_t Hq, int32_t G, int64_t N, int D,
                                 int top_k, float scale_log2, const void *q, const void *k, const void *v, float *o,
                                 int32_t *token_idx, hipStream_t stream) {
    SelFn fn = sel_for(SEL_ATTEND, kv_fmt, q_fmt, D);
    if (!fn) return hipErrorInvalidValue;
    SelArgs a;
    a.P = N;
    a.top_k = top_k;
    a.q = q;
    a.kmin = (const uint8_t *)k;
    a.kmax = (const uint8_t *)k;
    a.page_idx = token_idx;
    a.v = (const uint8_t *)v;
    a.o = o;
    a.scale_log2 = scale_log2;
    a.Hq = Hq;
    a.G = G;
    const int nw = sel_threads(SEL_ATTEND) / 64;
    const size_t lds = ((size_t)N + 2 * (size_t)top_k + (size_t)nw * D) * sizeof(float);
    hipLaunchKernelGGL(fn, dim3((unsigned)BH), dim3(sel_threads(SEL_ATTEND)), lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_page_attention(int kv_fmt, int q_fmt, int64_t BH, int32_t Hq, int32_t G, int64_t N, int64_t P,
                                 int D, int log2_page, int top_k, float scale_log2, const void *q, const void *kmin,
                                 const void *kmax, const void *k, const void *v, float *o, int32_t *page_idx,
                                 hipStream_t stream) {
    SelFn fn = sel_for(SEL_PAGE_ATTEND, kv_fmt, q_fmt, D);
    if (!fn) return hipErrorInvalidValue;
    SelArgs a;
    a.P = P;
    a.top_k = top_k;
    a.q = q;
    a.kmin = (const uint8_t *)kmin;
    a.kmax = (const uint8_t *)kmax;
    a.page_idx = page_idx;
    a.k = (const uint8_t *)k;
    a.v = (const uint8_t *)v;
    a.o = o;
    a.N = N;
    a.log2_page = log2_page;
    a.scale_log2 = scale_log2;
    a.Hq = Hq;
    a.G = G;
    const int nw = sel_threads(SEL_PAGE_ATTEND) / 64;
    const size_t lds = page_attention_lds_floats(P, top_k, log2_page, D, nw) * sizeof(float);
    hipLaunchKernelGGL(fn, dim3((unsigned)BH), dim3(sel_threads(SEL_PAGE_ATTEND)), lds, stream, a);
    return hipGetLastError();
}

}  // namespace da
