// Internal interface between the C-ABI layer (api.cpp, stream.cpp) and the
// HIP kernels.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

// Storage formats of q and of the KV cache.  Values 0..2 equal da_dtype.
enum Fmt : int { FMT_F32 = 0, FMT_F16 = 1, FMT_BF16 = 2, FMT_U4 = 3 };

// Default tokens (dense) or selected positions (paged) per split.  They depend
// only on the entry point and the context length, never on batch or head
// counts.  Dense: the power of two nearest above n_ctx / 16, within
// [256, 2048] (long splits amortise each wave's set-up and keep the partials
// small); uint4 and paged: fixed.
constexpr int kDefaultSplitDenseMin = 256;
constexpr int kDefaultSplitDense = 2048;
constexpr int kDefaultSplitU4Min = 256;
constexpr int64_t kU4MinWaves = 2048;    // two waves per SIMD
constexpr int kDefaultSplitPaged = 512;

// One attention launch (split-K partial pass + cross-split merge).
// The KV cache is addressed by rows (tokens): row r of (batch b, KV head h)
// starts at base + ((b * kv_bstride + h * kv_hstride) + r) * row_bytes.
struct AttnLaunch {
    int32_t B = 0, Hkv = 0, G = 0, D = 0;
    int64_t N = 0;                 // valid tokens per (b, h)
    float scale_log2 = 0.f;        // softmax scale * log2(e)
    int32_t q_fmt = 0, kv_fmt = 0;

    const void *q = nullptr;       // head (h*G + g) of row b at q + b*q_bstride + (h*G+g)*D
    int64_t q_bstride = 0;         // elements
    float *o = nullptr;            // same indexing as q, fp32
    int64_t o_bstride = 0;         // floats

    const void *k = nullptr, *v = nullptr;
    int64_t kv_bstride = 0, kv_hstride = 0;   // rows
    // uint4 cache: per-row fp16 min and scale arrays, D/64 per row
    const void *kmin = nullptr, *kscale = nullptr, *vmin = nullptr, *vscale = nullptr;

    // page-sparse: page list [B][Hkv][top_k], page = 2^log2_page tokens.
    // Grouped-query heads run one unit per query head (Hkv = query heads,
    // G = 1) with kv_group = query heads per KV head: unit h reads the rows of
    // KV head h / kv_group.
    const int32_t *page_idx = nullptr;
    int32_t top_k = 0, log2_page = 0;
    int32_t kv_group = 1;

    int32_t split_tokens = kDefaultSplitDense;
    int32_t n_split = 0;
    float *ws = nullptr;           // [B*Hkv*G][n_split][D+4]

    // Waves per workgroup (1..kMaxWavesPerBlock); wave w of workgroup x
    // reduces split x * wpb + w.  With `fused` set, one workgroup holds every
    // split of its (b, h) (n_split <= wpb) and merges them through LDS into
    // o; the workspace is then not touched and no merge kernel runs.
    int32_t wpb = 1;
    int32_t fused = 0;
};

constexpr int kMaxWavesPerBlock = 4;

int32_t default_split_dense(int64_t n_ctx);
int32_t default_split_u4(int64_t n_ctx, int64_t units);

// Number of splits and workspace bytes for a launch description.
int32_t attn_n_split(int64_t n_ctx, int32_t split_tokens, bool paged,
                     int32_t top_k, int32_t log2_page);
size_t attn_ws_bytes(int64_t rows, int32_t n_split, int32_t D);

// True if a kernel is built for this combination.
bool attn_supported(int kv_fmt, int q_fmt, int D, int G, bool paged);

// Split-K partial pass + cross-split merge.  When a (b, h) has at most
// kMaxWavesPerBlock splits they run as the waves of one workgroup and merge
// in LDS (same arithmetic, in the same order, as the merge kernel).
hipError_t launch_attention(const AttnLaunch &a, hipStream_t stream);
// The two halves on their own.  Partials: [rows][n_split][D + 4] fp32 holding
// (unnormalised output u[D], max m of the base-2 logits, sum l of
// 2^(logit - m), two pad words).
// Merge: row r = b * heads_per_row + j goes to o + b * o_bstride + j * D.
hipError_t launch_split(const AttnLaunch &a, hipStream_t stream);
hipError_t launch_merge(int64_t rows, int32_t heads_per_row, int32_t n_split, int32_t D, const float *ws, float *o,
                        int64_t o_bstride, hipStream_t stream);

// Page metadata: kmin/kmax [B*H][P][D] from k [B*H][N][D].
hipError_t launch_page_meta(int kv_fmt, int64_t BH, int64_t N, int D,
                            int log2_page, const void *k, void *kmin, void *kmax,
                            hipStream_t stream);

// Bound score + top-K per (b, h).  With `exact`, kmax holds the key rows
// themselves (P = N tokens, kmin unused) and the score is q . k.
bool select_supported(int kv_fmt, int q_fmt, int D);
hipError_t launch_select(int kv_fmt, int q_fmt, int64_t BH, int32_t Hq, int32_t G, int64_t P, int D,
                         int top_k, const void *q, const void *kmin,
                         const void *kmax, int32_t *page_idx, float *page_score,
                         hipStream_t stream, bool exact = false);

// Exact-score token selection fused with attention over the kept tokens:
// one workgroup per (b, h); o [BH][D] fp32; token_idx optional.  Dynamic
// LDS holds N + 2 * top_k + 8 * D floats.
hipError_t launch_topk_attention(int kv_fmt, int q_fmt, int64_t BH, int32_t Hq, int32_t G, int64_t N, int D,
                                 int top_k, float scale_log2, const void *q, const void *k, const void *v, float *o,
                                 int32_t *token_idx, hipStream_t stream);

// Page selection fused with attention over the kept pages' tokens (one
// 1024-thread workgroup per (b, h)): bound scores, top-K pages, exact scores
// of their K * 2^log2_page token slots, softmax and the value rows; o
// [BH][D] fp32; page_idx optional.  Dynamic LDS: P page scores, K page
// indices, two floats per token slot, 16 * D partial sums.
inline int64_t page_attention_lds_floats(int64_t P, int64_t top_k, int log2_page, int D, int n_waves) {
    return P + top_k + 2 * (top_k << log2_page) + (int64_t)n_waves * D;
}
constexpr int64_t kPageAttnLdsFloats = 16384;   // 64 KiB of dynamic LDS
hipError_t launch_page_attention(int kv_fmt, int q_fmt, int64_t BH, int32_t Hq, int32_t G, int64_t N, int64_t P,
                                 int D, int log2_page, int top_k, float scale_log2, const void *q, const void *kmin,
                                 const void *kmax, const void *k, const void *v, float *o, int32_t *page_idx,
                                 hipStream_t stream);

// Chunked prefill attention: q [B][Hq][C][D], k/v [B][Hkv][T][D] (T = prefix
// + C), o [B][Hq][C][D] fp32; q, k and v in `fmt` (bf16 or fp16).
bool prefill_supported(int fmt, int D);
hipError_t launch_prefill(int fmt, int64_t B, int32_t Hq, int32_t Hkv, int D, int64_t C, int64_t T,
                          float scale_log2, const void *q, const void *k, const void *v, float *o,
                          hipStream_t stream);

// Allocation-free decode attention: the split-K partials go to a fixed
// device array of kNoAllocScratchBytes per GPU.  noalloc_scratch returns its
// device address on the current GPU (looked up with hipGetSymbolAddress on
// the first call on each device; later calls allocate and look up nothing).
constexpr size_t kNoAllocScratchBytes = 16u << 20;
hipError_t noalloc_scratch(float **out);

// uint4 group quantization.
hipError_t launch_read_stream(const void *buf, int64_t n16, int32_t n_groups, uint32_t *sink, hipStream_t stream);
hipError_t launch_quantize_kv4(int64_t n_groups, const void *x, uint8_t *codes,
                               void *gmin, void *gscale, hipStream_t stream);
hipError_t launch_dequantize_kv4(int64_t n_groups, const uint8_t *codes,
                                 const void *gmin, const void *gscale, void *x,
                                 hipStream_t stream);

}  // namespace da
