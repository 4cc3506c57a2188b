// Internal launch interface between the C ABI (abi.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace orthrus {

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (expcnt and lgkmcnt left at their maxima), gfx9 encoding.
constexpr int vmcnt_encode(int n) {
    return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8);
}

// Largest key range of one split in the paged layout (page ids staged in LDS).
constexpr int kMaxSplitKeysPaged = 8192;
constexpr int kMaxSplitPages = kMaxSplitKeysPaged / 16;

struct AttnParams {
    const void *q, *kb, *vb;          // [B][K][Hq|Hkv][D]
    const void *kc, *vc;              // cache (layout)
    const int32_t *page_table;        // paged: [B][maxp]
    const int32_t *lens;              // [B]
    void *out;                        // [B][K][Hq][D]
    float *lse;                       // [B][Hq][K] or null
    void *ws_o;                       // split partials [B*Hkv][S_grid][Mpad x D] fragment order
    float *ws_lse;                    // [B*Hkv][S_grid][Mpad] (base-2 units)
    int B, K, Hq, Hkv, G, M, Mpad, D;   // Mpad = M rounded up to 32
    int64_t cap, maxp;
    int layout, mask;
    int SL, S_grid;                   // keys per split (multiple of 64), grid splits
    int rows_per_wg, row_blocks;
    float c;                          // scale * log2(e)
    int lpt;                          // paged, B <= 64: blockIdx.x walks a longest-first
                                      // list of (request, split) work items
    int nbps;                         // requests per cache sequence: request b reads the
                                      // contiguous cache of sequence b / nbps (1 = its own)
    int reverse;                      // dispatch requests from the last one (longest first
                                      // when lengths grow with the request index)
    int kv8;                          // cache holds e4m3 codes (kc, vc) with per-row scales
    const float *ks, *vs;             // kv8: scale of each cache row, laid out like the rows
};

int attn_rows_per_wg(int dtype, int M);
hipError_t launch_block_attn(const AttnParams &p, int dtype, hipStream_t st);

// Consensus / argmax
constexpr int kArgmaxChunkBytes = 16384;   // bytes of one row handled by one work-group
hipError_t launch_argmax_partial(const void *logits0, const void *logits1, int64_t rows0,
                                 int64_t rows1, int V, int dtype, uint64_t *ws, int chunks,
                                 hipStream_t st);
hipError_t launch_argmax_finalize(const uint64_t *ws, int64_t rows, int chunks, int32_t *idx,
                                  hipStream_t st);
hipError_t launch_consensus_tokens(const int32_t *diff_tok, const int32_t *ar_tok, int B, int K,
                                  int32_t *n_match, int32_t *n_emit, int32_t *emit_off,
                                  int32_t *emitted, int32_t *next_anchor, hipStream_t st);
hipError_t launch_consensus_finalize(const uint64_t *ws, int B, int K, int chunks,
                                     int32_t *diff_tok, int32_t *ar_tok, int32_t *n_match,
                                     int32_t *n_emit, int32_t *emit_off, int32_t *emitted,
                                     int32_t *next_anchor, hipStream_t st);

// KV append
struct AppendParams {
    void *kc, *vc;
    const void *kb, *vb;
    const int32_t *page_table, *lens, *n_emit;
    int32_t *lens_out;
    int B, K, Hkv, D, esize, layers, layout;
    int64_t cap, maxp, cache_layer_stride, blk_layer_stride;   // elements
    int lens_in_place;                // lens_out == lens: a second launch advances lens
    int kv8;                          // the cache holds e4m3 codes: quantize the rows
    float *ks, *vs;                   // kv8: per-row scales (layer l at + l * scale_layer_stride)
    int64_t scale_layer_stride;
};
hipError_t launch_kv_append(const AppendParams &p, hipStream_t st);

}  // namespace orthrus
