// C ABI of the Orthrus decode-step library: argument validation (host only,
// never touches the device), split-KV planning, workspace sizing, launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/orthrus.h"
#include "kernels.hpp"

using namespace orthrus;

namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;
// Attention work-groups the automatic split plan aims at: about 80% of the
// 256 CUs.  Longer splits amortize each work-group's ~5 us of start-up and
// drain and shrink the partials' round trip: at 8,192 keys x 8 KV heads, 26
// splits of 320 keys took 16.4 us per layer pass against 17.35 us with 32
// splits of 256 (and 16.65 with 22 of 384).
constexpr int kTargetWorkGroups = 208;
constexpr int kMinKeysPerSplit = 128;     // bf16 (MFMA) path: two tiles per split at least
constexpr int kMinKeysPerSplitF32 = 64;   // fp32 (vector ALU) path: compute-bound per tile
// Paged work-list items (see plan_block_attn).  32 requests of 512..8,192
// keys, A/B on one box: 2,560-key items 176 us per layer pass, 3,072: 152,
// 3,584: 152, 4,096: 164 (items per CU decide: about two, paired long with
// short, pack best).
constexpr int kLptSplitKeys = 3584;
constexpr int64_t kMaxGrid = 2147483647;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct AttnPlan {
    int status;
    int M, G, rows_per_wg, row_blocks, SL, S_grid;
    size_t ws_bytes, ws_lse_offset;
};

// Shape/dtype checks shared by the workspace query and the launch.
AttnPlan plan_block_attn(const orthrus_cache *c, int B, int K, int Hq, int Hkv, int D, int dtype,
                         int num_splits)
{
    AttnPlan pl{};
    if (!c) { pl.status = ORTHRUS_ERR_NULL; return pl; }
    if (dtype != ORTHRUS_F32 && dtype != ORTHRUS_BF16) { pl.status = ORTHRUS_ERR_DTYPE; return pl; }
    if (c->layout != ORTHRUS_LAYOUT_CONTIGUOUS && c->layout != ORTHRUS_LAYOUT_PAGED) {
        pl.status = ORTHRUS_ERR_DTYPE;
        return pl;
    }
    if (B < 1 || K < 1 || Hq < 1 || Hkv < 1 || D < 1 || num_splits < 0 || Hq % Hkv != 0 ||
        c->max_len < 0) {
        pl.status = ORTHRUS_ERR_SHAPE;
        return pl;
    }
    if (K > 64 || (D != 64 && D != 128) || Hq / Hkv > 16) { pl.status = ORTHRUS_ERR_UNSUPPORTED; return pl; }
    if (c->kv_dtype != 0 && c->kv_dtype != ORTHRUS_FP8_E4M3) { pl.status = ORTHRUS_ERR_DTYPE; return pl; }
    if (c->kv_dtype == ORTHRUS_FP8_E4M3 && (dtype != ORTHRUS_BF16 || D != 128)) {
        pl.status = ORTHRUS_ERR_UNSUPPORTED;
        return pl;
    }
    int64_t lmax;
    if (c->layout == ORTHRUS_LAYOUT_CONTIGUOUS) {
        if (c->capacity < 0 || c->max_len > c->capacity) { pl.status = ORTHRUS_ERR_SHAPE; return pl; }
        lmax = c->max_len > 0 ? c->max_len : c->capacity;
    } else {
        if (c->page_size != 16) { pl.status = ORTHRUS_ERR_UNSUPPORTED; return pl; }
        if (c->num_pages < 1 || c->max_pages_per_req < 1 ||
            c->max_len > c->max_pages_per_req * (int64_t)c->page_size) {
            pl.status = ORTHRUS_ERR_SHAPE;
            return pl;
        }
        lmax = c->max_len > 0 ? c->max_len : c->max_pages_per_req * (int64_t)c->page_size;
    }
    if (lmax > (int64_t)1 << 30) { pl.status = ORTHRUS_ERR_UNSUPPORTED; return pl; }
    pl.G = Hq / Hkv;
    pl.M = pl.G * K;
    pl.rows_per_wg = attn_rows_per_wg(dtype, pl.M);
    pl.row_blocks = (int)ceil_div(pl.M, pl.rows_per_wg);
    int64_t S;
    if (num_splits > 0) {
        S = num_splits;
    } else {
        S = ceil_div(kTargetWorkGroups, (int64_t)B * Hkv * pl.row_blocks);
        const int64_t cap_s =
            ceil_div(lmax, dtype == ORTHRUS_F32 ? kMinKeysPerSplitF32 : kMinKeysPerSplit);
        if (S > cap_s) S = cap_s;
        // ragged paged batches are scheduled longest-first (the kernel's
        // work list): items of at most kLptSplitKeys keys pack the CUs evenly
        if (c->layout == ORTHRUS_LAYOUT_PAGED && dtype == ORTHRUS_BF16 && B <= 64 &&
            S < ceil_div(lmax, kLptSplitKeys))
            S = ceil_div(lmax, kLptSplitKeys);
    }
    if (S < 1) S = 1;
    if (c->layout == ORTHRUS_LAYOUT_PAGED && S < ceil_div(lmax, kMaxSplitKeysPaged))
        S = ceil_div(lmax, kMaxSplitKeysPaged);
    int64_t SL = 64 * ceil_div(ceil_div(lmax > 0 ? lmax : 1, S), 64);
    int64_t S_grid = lmax > 0 ? ceil_div(lmax, SL) : 1;
    if (c->layout == ORTHRUS_LAYOUT_PAGED) {
        // The kernel stages one split's page ids in LDS, so no split may
        // exceed kMaxSplitKeysPaged keys even if the hint is too small: size
        // the grid for the largest length the page table can describe.
        if (SL > kMaxSplitKeysPaged) SL = kMaxSplitKeysPaged;
        S_grid = ceil_div(c->max_pages_per_req * (int64_t)c->page_size, SL);
    }
    if (S_grid < 1) S_grid = 1;
    if ((int64_t)B * Hkv * S_grid > kMaxGrid || pl.row_blocks > 65535) {
        pl.status = ORTHRUS_ERR_UNSUPPORTED;
        return pl;
    }
    pl.SL = (int)SL;
    pl.S_grid = (int)S_grid;
    // partials in the path's dtype (bf16 or fp32), then the fp32 base-2 lse
    const size_t esz = dtype == ORTHRUS_BF16 ? 2 : 4;
    const size_t mpad = (size_t)(pl.M + 31) / 32 * 32;
    const size_t rows = (size_t)B * Hkv * S_grid * mpad;
    pl.ws_lse_offset = ((size_t)B * Hkv * S_grid * mpad * D * esz + 255) / 256 * 256;
    pl.ws_bytes = S_grid > 1 ? pl.ws_lse_offset + rows * sizeof(float) : 0;
    pl.status = ORTHRUS_OK;
    return pl;
}

int argmax_chunks(int V, int dtype) {
    const int64_t bytes = (int64_t)V * (dtype == ORTHRUS_BF16 ? 2 : 4);
    return (int)ceil_div(bytes, kArgmaxChunkBytes);
}

int map_err(hipError_t e) { return e == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char *orthrus_status_string(int status)
{
    switch (status) {
        case ORTHRUS_OK: return "ok";
        case ORTHRUS_ERR_NULL: return "null pointer";
        case ORTHRUS_ERR_SHAPE: return "bad shape";
        case ORTHRUS_ERR_DTYPE: return "bad dtype, layout or mask";
        case ORTHRUS_ERR_UNSUPPORTED: return "unsupported configuration";
        case ORTHRUS_ERR_WORKSPACE: return "workspace missing or too small";
        case ORTHRUS_ERR_LAUNCH: return "HIP launch error";
        default: return "unknown status";
    }
}

int orthrus_version(void) { return kVersion; }

size_t orthrus_block_attn_workspace_bytes(const orthrus_cache *cache, int B, int K, int Hq,
                                          int Hkv, int D, int dtype, int num_splits)
{
    AttnPlan pl = plan_block_attn(cache, B, K, Hq, Hkv, D, dtype, num_splits);
    return pl.status == ORTHRUS_OK ? pl.ws_bytes : 0;
}

}  // extern "C"

namespace {

// The block attention launch shared by the decode step (nbps = 1: request b
// reads its own cache) and the training-time block mask (nbps = blocks per
// sequence: block b reads the context of sequence b / nbps).
int block_attn_impl(const orthrus_cache *cache, const void *q, const void *k_blk,
                    const void *v_blk, void *out, float *lse, int B, int K, int Hq, int Hkv,
                    int D, int dtype, int mask, float scale, int num_splits, void *workspace,
                    size_t workspace_bytes, hipStream_t stream, int nbps, int reverse)
{
    if (!cache || !q || !k_blk || !v_blk || !out) return ORTHRUS_ERR_NULL;
    if (!cache->k || !cache->v || !cache->lens) return ORTHRUS_ERR_NULL;
    if (cache->layout == ORTHRUS_LAYOUT_PAGED && !cache->page_table) return ORTHRUS_ERR_NULL;
    if (cache->kv_dtype == ORTHRUS_FP8_E4M3 && (!cache->k_scale || !cache->v_scale))
        return ORTHRUS_ERR_NULL;
    if (mask != ORTHRUS_MASK_BIDIR && mask != ORTHRUS_MASK_CAUSAL) return ORTHRUS_ERR_DTYPE;
    AttnPlan pl = plan_block_attn(cache, B, K, Hq, Hkv, D, dtype, num_splits);
    if (pl.status != ORTHRUS_OK) return pl.status;
    if (!std::isfinite(scale)) return ORTHRUS_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(out) ||
        !aligned16(cache->k) || !aligned16(cache->v))
        return ORTHRUS_ERR_UNSUPPORTED;
    if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes || !aligned16(workspace)))
        return ORTHRUS_ERR_WORKSPACE;

    AttnParams p{};
    p.q = q;
    p.kb = k_blk;
    p.vb = v_blk;
    p.kc = cache->k;
    p.vc = cache->v;
    p.page_table = cache->page_table;
    p.lens = cache->lens;
    p.out = out;
    p.lse = lse;
    p.B = B;
    p.K = K;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.G = pl.G;
    p.M = pl.M;
    p.Mpad = (pl.M + 31) / 32 * 32;
    p.D = D;
    p.cap = cache->capacity;
    p.maxp = cache->max_pages_per_req;
    p.layout = cache->layout;
    p.mask = mask;
    p.SL = pl.SL;
    p.S_grid = pl.S_grid;
    p.rows_per_wg = pl.rows_per_wg;
    p.row_blocks = pl.row_blocks;
    p.c = scale * 1.4426950408889634f;
    p.lpt = (cache->layout == ORTHRUS_LAYOUT_PAGED && dtype == ORTHRUS_BF16 && B <= 64 &&
             pl.S_grid > 1) ? 1 : 0;
    p.nbps = nbps;
    p.reverse = reverse;
    p.kv8 = cache->kv_dtype == ORTHRUS_FP8_E4M3 ? 1 : 0;
    p.ks = cache->k_scale;
    p.vs = cache->v_scale;
    if (pl.S_grid > 1) {
        p.ws_o = workspace;
        p.ws_lse = reinterpret_cast<float *>(static_cast<char *>(workspace) + pl.ws_lse_offset);
    }
    return map_err(launch_block_attn(p, dtype, stream));
}

// The context of a training-time block-mask call as a contiguous cache of
// B*NB requests (the anchors are the lengths).
bool mdiff_cache(orthrus_cache *c, const void *k_ctx, const void *v_ctx, int64_t ctx_capacity,
                 const int32_t *anchors, int64_t max_anchor, int B, int NB)
{
    if (B < 1 || NB < 1 || ctx_capacity < 0 || max_anchor < 0 || max_anchor > ctx_capacity ||
        (int64_t)B * NB > (int64_t)1 << 24)
        return false;
    *c = orthrus_cache{};
    c->layout = ORTHRUS_LAYOUT_CONTIGUOUS;
    c->page_size = 16;
    c->k = const_cast<void *>(k_ctx);
    c->v = const_cast<void *>(v_ctx);
    c->capacity = ctx_capacity;
    c->lens = anchors;
    c->max_len = max_anchor;
    return true;
}

}  // namespace

extern "C" {

int orthrus_block_attn(const orthrus_cache *cache, const void *q, const void *k_blk,
                       const void *v_blk, void *out, float *lse, int B, int K, int Hq, int Hkv,
                       int D, int dtype, int mask, float scale, int num_splits, void *workspace,
                       size_t workspace_bytes, hipStream_t stream)
{
    return block_attn_impl(cache, q, k_blk, v_blk, out, lse, B, K, Hq, Hkv, D, dtype, mask, scale,
                           num_splits, workspace, workspace_bytes, stream, 1, 0);
}

size_t orthrus_mdiff_attn_workspace_bytes(int64_t ctx_capacity, int64_t max_anchor, int B, int NB,
                                          int K, int Hq, int Hkv, int D, int dtype,
                                          int num_splits)
{
    orthrus_cache c;
    if (!mdiff_cache(&c, nullptr, nullptr, ctx_capacity, nullptr, max_anchor, B, NB)) return 0;
    AttnPlan pl = plan_block_attn(&c, B * NB, K, Hq, Hkv, D, dtype, num_splits);
    return pl.status == ORTHRUS_OK ? pl.ws_bytes : 0;
}

int orthrus_mdiff_attn(const void *k_ctx, const void *v_ctx, int64_t ctx_capacity,
                       const int32_t *anchors, int64_t max_anchor, const void *q,
                       const void *k_blk, const void *v_blk, void *out, float *lse, int B, int NB,
                       int K, int Hq, int Hkv, int D, int dtype, float scale, int num_splits,
                       void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!k_ctx || !v_ctx || !anchors) return ORTHRUS_ERR_NULL;
    orthrus_cache c;
    if (!mdiff_cache(&c, k_ctx, v_ctx, ctx_capacity, anchors, max_anchor, B, NB))
        return ORTHRUS_ERR_SHAPE;
    // blocks are dispatched from the last one: with anchors growing along the
    // sequence that is longest first, so the long blocks do not start last
    return block_attn_impl(&c, q, k_blk, v_blk, out, lse, B * NB, K, Hq, Hkv, D, dtype,
                           ORTHRUS_MASK_BIDIR, scale, num_splits, workspace, workspace_bytes,
                           stream, NB, 1);
}

size_t orthrus_consensus_workspace_bytes(int B, int K, int V, int dtype)
{
    if (B < 1 || K < 1 || K > 64 || V < 1 || (int64_t)B * K > 65536) return 0;
    if (dtype != ORTHRUS_F32 && dtype != ORTHRUS_BF16) return 0;
    return (size_t)2 * B * K * argmax_chunks(V, dtype) * sizeof(uint64_t);
}

int orthrus_consensus(const void *diff_logits, const void *ar_logits, int B, int K, int V,
                      int dtype, int32_t *diff_tok, int32_t *ar_tok, int32_t *n_match,
                      int32_t *n_emit, int32_t *emit_off, int32_t *emitted,
                      int32_t *next_anchor, void *workspace, size_t workspace_bytes,
                      hipStream_t stream)
{
    if (!diff_logits || !ar_logits || !diff_tok || !ar_tok || !n_match || !n_emit || !emit_off ||
        !emitted || !next_anchor)
        return ORTHRUS_ERR_NULL;
    if (dtype != ORTHRUS_F32 && dtype != ORTHRUS_BF16) return ORTHRUS_ERR_DTYPE;
    if (B < 1 || K < 1 || V < 1) return ORTHRUS_ERR_SHAPE;
    if (K > 64 || (int64_t)B * K > 65536) return ORTHRUS_ERR_UNSUPPORTED;
    const int chunks = argmax_chunks(V, dtype);
    const int64_t rows = (int64_t)2 * B * K;
    if (rows * chunks > kMaxGrid) return ORTHRUS_ERR_UNSUPPORTED;
    const size_t need = (size_t)rows * chunks * sizeof(uint64_t);
    if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 7u))
        return ORTHRUS_ERR_WORKSPACE;
    uint64_t *ws = static_cast<uint64_t *>(workspace);
    hipError_t e = launch_argmax_partial(diff_logits, ar_logits, (int64_t)B * K, (int64_t)B * K, V,
                                         dtype, ws, chunks, stream);
    if (e != hipSuccess) return ORTHRUS_ERR_LAUNCH;
    return map_err(launch_consensus_finalize(ws, B, K, chunks, diff_tok, ar_tok, n_match, n_emit,
                                             emit_off, emitted, next_anchor, stream));
}

int orthrus_consensus_tokens(const int32_t *diff_tok, const int32_t *ar_tok, int B, int K,
                             int32_t *n_match, int32_t *n_emit, int32_t *emit_off,
                             int32_t *emitted, int32_t *next_anchor, hipStream_t stream)
{
    if (!diff_tok || !ar_tok || !n_match || !n_emit || !emit_off || !emitted || !next_anchor)
        return ORTHRUS_ERR_NULL;
    if (B < 1 || K < 1) return ORTHRUS_ERR_SHAPE;
    if (K > 64 || (int64_t)B * K > 65536) return ORTHRUS_ERR_UNSUPPORTED;
    return map_err(launch_consensus_tokens(diff_tok, ar_tok, B, K, n_match, n_emit, emit_off,
                                           emitted, next_anchor, stream));
}

size_t orthrus_argmax_workspace_bytes(int64_t rows, int V, int dtype)
{
    if (rows < 1 || rows > 131072 || V < 1) return 0;
    if (dtype != ORTHRUS_F32 && dtype != ORTHRUS_BF16) return 0;
    return (size_t)rows * argmax_chunks(V, dtype) * sizeof(uint64_t);
}

int orthrus_argmax(const void *logits, int64_t rows, int V, int dtype, int32_t *idx,
                   void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!logits || !idx) return ORTHRUS_ERR_NULL;
    if (dtype != ORTHRUS_F32 && dtype != ORTHRUS_BF16) return ORTHRUS_ERR_DTYPE;
    if (rows < 1 || V < 1) return ORTHRUS_ERR_SHAPE;
    if (rows > 131072) return ORTHRUS_ERR_UNSUPPORTED;
    const int chunks = argmax_chunks(V, dtype);
    if (rows * chunks > kMaxGrid) return ORTHRUS_ERR_UNSUPPORTED;
    const size_t need = (size_t)rows * chunks * sizeof(uint64_t);
    if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 7u))
        return ORTHRUS_ERR_WORKSPACE;
    uint64_t *ws = static_cast<uint64_t *>(workspace);
    hipError_t e = launch_argmax_partial(logits, logits, rows, 0, V, dtype, ws, chunks, stream);
    if (e != hipSuccess) return ORTHRUS_ERR_LAUNCH;
    return map_err(launch_argmax_finalize(ws, rows, chunks, idx, stream));
}

int orthrus_kv_append(const orthrus_cache *cache, const void *k_blk, const void *v_blk,
                      const int32_t *n_emit, int32_t *lens_out, int B, int K, int Hkv, int D,
                      int dtype, int num_layers, int64_t cache_layer_stride,
                      int64_t blk_layer_stride, hipStream_t stream)
{
    if (!cache || !k_blk || !v_blk || !n_emit || !lens_out) return ORTHRUS_ERR_NULL;
    if (!cache->k || !cache->v || !cache->lens) return ORTHRUS_ERR_NULL;
    if (cache->layout == ORTHRUS_LAYOUT_PAGED && !cache->page_table) return ORTHRUS_ERR_NULL;
    if (dtype != ORTHRUS_F32 && dtype != ORTHRUS_BF16) return ORTHRUS_ERR_DTYPE;
    if (cache->layout != ORTHRUS_LAYOUT_CONTIGUOUS && cache->layout != ORTHRUS_LAYOUT_PAGED)
        return ORTHRUS_ERR_DTYPE;
    if (B < 1 || K < 1 || Hkv < 1 || D < 1 || num_layers < 1 || cache_layer_stride < 0 ||
        blk_layer_stride < 0)
        return ORTHRUS_ERR_SHAPE;
    if (K > 64 || (D != 64 && D != 128) || B > 8192) return ORTHRUS_ERR_UNSUPPORTED;
    if (cache->kv_dtype != 0 && cache->kv_dtype != ORTHRUS_FP8_E4M3) return ORTHRUS_ERR_DTYPE;
    const bool kv8 = cache->kv_dtype == ORTHRUS_FP8_E4M3;
    if (kv8) {
        if (!cache->k_scale || !cache->v_scale) return ORTHRUS_ERR_NULL;
        if (dtype != ORTHRUS_BF16 || D != 128) return ORTHRUS_ERR_UNSUPPORTED;
        if (num_layers > 1 && (cache_layer_stride % D)) return ORTHRUS_ERR_UNSUPPORTED;
    }
    const int esize = dtype == ORTHRUS_BF16 ? 2 : 4;
    if (cache->layout == ORTHRUS_LAYOUT_CONTIGUOUS) {
        if (cache->capacity < 1) return ORTHRUS_ERR_SHAPE;
    } else {
        if (cache->page_size != 16) return ORTHRUS_ERR_UNSUPPORTED;
        if (cache->num_pages < 1 || cache->max_pages_per_req < 1) return ORTHRUS_ERR_SHAPE;
    }
    const int cache_esize = kv8 ? 1 : esize;
    if (num_layers > 1 &&
        (((cache_layer_stride * cache_esize) & 15) || ((blk_layer_stride * esize) & 15)))
        return ORTHRUS_ERR_UNSUPPORTED;
    if (!aligned16(k_blk) || !aligned16(v_blk) || !aligned16(cache->k) || !aligned16(cache->v))
        return ORTHRUS_ERR_UNSUPPORTED;
    if ((int64_t)ceil_div((int64_t)B * K, 4) * num_layers > kMaxGrid) return ORTHRUS_ERR_UNSUPPORTED;
    AppendParams p{};
    p.kc = cache->k;
    p.vc = cache->v;
    p.kb = k_blk;
    p.vb = v_blk;
    p.page_table = cache->page_table;
    p.lens = cache->lens;
    p.n_emit = n_emit;
    p.lens_out = lens_out;
    p.B = B;
    p.K = K;
    p.Hkv = Hkv;
    p.D = D;
    p.esize = esize;
    p.layers = num_layers;
    p.layout = cache->layout;
    p.cap = cache->capacity;
    p.maxp = cache->max_pages_per_req;
    p.cache_layer_stride = cache_layer_stride;
    p.blk_layer_stride = blk_layer_stride;
    p.lens_in_place = lens_out == cache->lens ? 1 : 0;
    p.kv8 = kv8 ? 1 : 0;
    p.ks = cache->k_scale;
    p.vs = cache->v_scale;
    p.scale_layer_stride = kv8 ? cache_layer_stride / D : 0;
    return map_err(launch_kv_append(p, stream));
}

}  // extern "C"
