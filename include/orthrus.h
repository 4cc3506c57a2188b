/*
 * orthrus.h -- C ABI of the Orthrus decode-step library for MI355X (gfx950).
 *
 * One Orthrus decode step (see "Orthrus: Memory-Efficient Parallel Token
 * Generation via Dual-View Diffusion", gist.science technical summary,
 * §2.1-§2.3; the paper's abstract on chatpaper.ai; the agents-report.net
 * commentary, core-design section) is:
 *
 *   1. the diffusion view's block attention (bidirectional inside the block)
 *      and the AR view's verification attention (causal inside the block),
 *      both over ONE shared, prefilled KV cache          -> orthrus_block_attn
 *   2. greedy prediction of both views, left-to-right exact consensus
 *                                                        -> orthrus_consensus
 *   3. the commit: the accepted positions' AR-view KV rows are appended to
 *      the shared cache                                  -> orthrus_kv_append
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor argument is a DEVICE pointer owned by the caller.  The
 *    library never allocates, frees or synchronises; scratch memory comes in
 *    through (workspace, workspace_bytes).  Work is enqueued on `stream`
 *    (0 = the null stream) and is ordered with the caller's other work.
 *  - Arguments are validated on the host before anything is enqueued; on a
 *    validation error nothing is launched and outputs are untouched.
 *    Validation never touches the device.  Device-side contents (page ids,
 *    lens, token counts) are caller contracts listed per function.
 *  - Return value: ORTHRUS_OK or an orthrus_status code;
 *    orthrus_status_string() names it.  ORTHRUS_ERR_LAUNCH reports a HIP
 *    launch error (hipGetLastError after the launch).
 *  - No global mutable state: concurrent calls on different streams are
 *    safe as long as their outputs and workspaces do not overlap.
 *  - Tensors are dense, row-major, in the shapes given below; element type
 *    `dtype` is ORTHRUS_F32 (float) or ORTHRUS_BF16 (bfloat16).
 */
#ifndef ORTHRUS_H
#define ORTHRUS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ORTHRUS_OK = 0,
    ORTHRUS_ERR_NULL = 1,        /* a required pointer is NULL             */
    ORTHRUS_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
    ORTHRUS_ERR_DTYPE = 3,       /* unknown dtype / layout / mask value    */
    ORTHRUS_ERR_UNSUPPORTED = 4, /* valid but not implemented (e.g. D=96)  */
    ORTHRUS_ERR_WORKSPACE = 5,   /* workspace missing or too small         */
    ORTHRUS_ERR_LAUNCH = 6       /* the HIP runtime reported an error      */
} orthrus_status;

typedef enum { ORTHRUS_F32 = 0, ORTHRUS_BF16 = 1 } orthrus_dtype;

/* In-block visibility of the block rows:
 *   BIDIR  -- every block row sees every block row (the diffusion view's
 *             parallel projection; summary §2.2 and §2.3 step 1)
 *   CAUSAL -- block row i sees block rows 0..i (the frozen AR view's
 *             verification pass; summary §2.3 step 2)
 * Every block row always sees all lens[b] cache rows.                      */
typedef enum { ORTHRUS_MASK_BIDIR = 0, ORTHRUS_MASK_CAUSAL = 1 } orthrus_mask;

typedef enum { ORTHRUS_LAYOUT_CONTIGUOUS = 0, ORTHRUS_LAYOUT_PAGED = 1 } orthrus_layout;

/*
 * The shared KV cache of ONE layer (summary §2.1: both views read the same
 * cache; the history is never copied).
 *
 *  layout = CONTIGUOUS: k, v are [B][Hkv][capacity][D]; row t of request b,
 *           KV head g is at ((b*Hkv + g)*capacity + t)*D.
 *  layout = PAGED:      k, v are [num_pages][Hkv][page_size][D]; logical row
 *           t of request b lives in physical page
 *           page_table[b*max_pages_per_req + t/page_size], slot t%page_size.
 *           page_size must be 16.
 *  lens      device int32 [B]: number of valid cache rows of each request.
 *  max_len   host-side upper bound on lens[b] used to size the split-KV grid
 *            (0 = derive it from capacity or max_pages_per_req*page_size).
 *            A wrong hint costs speed, never correctness.
 * Caller contracts (not checked on the device): 0 <= lens[b]; for
 * CONTIGUOUS lens[b] <= capacity; for PAGED every page id the rows
 * 0..lens[b]-1 (and, for an append, the appended rows) map to is in
 * [0, num_pages).
 */
typedef struct orthrus_cache {
    int32_t layout;              /* orthrus_layout                          */
    int32_t page_size;           /* PAGED: tokens per page (16)             */
    void *k;                     /* device                                  */
    void *v;                     /* device                                  */
    int64_t capacity;            /* CONTIGUOUS: rows per (request, head)    */
    int64_t num_pages;           /* PAGED: physical pages                   */
    const int32_t *page_table;   /* PAGED: device int32 [B][max_pages_per_req] */
    int64_t max_pages_per_req;   /* PAGED                                   */
    const int32_t *lens;         /* device int32 [B]                        */
    int64_t max_len;             /* host hint, see above                    */
} orthrus_cache;

/*
 * orthrus_block_attn -- shared-KV block attention of one layer, one view.
 * (summary §2.1-§2.3; agents-report core design: the block attends to the
 * shared cache and, bidirectionally, to itself; the AR view verifies the
 * whole block in one causal pass.)
 *
 * For request b, query head h (KV head g = h / (Hq/Hkv), contiguous GQA
 * groups) and block row i:
 *   keys    = cache rows 0..lens[b]-1 of head g, then block rows j of k_blk
 *             with j < K (BIDIR) or j <= i (CAUSAL)
 *   s_t     = scale * <q[b,i,h,:], key_t>
 *   out     = sum_t softmax(s)_t * value_t      (fp32 accumulation)
 *   lse     = log(sum_t exp(s_t))               (natural log, fp32)
 *
 *  q         [B][K][Hq][D]   dtype, block row 0 is the anchor (post-RoPE)
 *  k_blk     [B][K][Hkv][D]  dtype, the view's own block keys (post-RoPE)
 *  v_blk     [B][K][Hkv][D]  dtype
 *  out       [B][K][Hq][D]   dtype (bf16 outputs are rounded to nearest even)
 *  lse       [B][Hq][K]      float, may be NULL
 *  K         1..64; D in {64, 128}; Hq % Hkv == 0; Hq/Hkv <= 16
 *  scale     softmax scale (1/sqrt(D) for Qwen3)
 *  num_splits  0 = automatic; otherwise the largest number of key-range
 *            partitions per (request, KV head) -- split-KV partial results
 *            are merged by a second log-sum-exp pass
 *  workspace >= orthrus_block_attn_workspace_bytes(...) bytes of device
 *            memory (may be NULL when that function returns 0); contents on
 *            entry are ignored.
 * The block K/V are scratch: nothing is written to the cache.
 */
int orthrus_block_attn(const orthrus_cache *cache, const void *q,
                       const void *k_blk, const void *v_blk, void *out,
                       float *lse, int B, int K, int Hq, int Hkv, int D,
                       int dtype, int mask, float scale, int num_splits,
                       void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* Workspace bytes orthrus_block_attn needs for these arguments (0 if none).
 * Depends only on host-side values; returns 0 on invalid arguments too. */
size_t orthrus_block_attn_workspace_bytes(const orthrus_cache *cache, int B,
                                          int K, int Hq, int Hkv, int D,
                                          int dtype, int num_splits);

/*
 * orthrus_consensus -- greedy prediction of both views and exact
 * left-to-right consensus (summary §2.3 step 3).
 *
 *  diff_logits, ar_logits  [B][K][V] dtype: row i of both views predicts the
 *            same position (the token after block input i).
 *  diff_tok, ar_tok   out int32 [B][K]: row argmax, lowest index on ties,
 *            -0.0 == +0.0.  (NaN logits: result unspecified.)
 *  n_match   out int32 [B]: j = first i with diff_tok != ar_tok (K if none)
 *  n_emit    out int32 [B]: n = min(j + 1, K) tokens emitted this step
 *  emit_off  out int32 [B+1]: exclusive prefix sum of n_emit (emit_off[B] =
 *            total)
 *  emitted   out int32 [B*K] (capacity): ar_tok[b][0..n-1] packed at
 *            emit_off[b]; entries past emit_off[B] are not written
 *  next_anchor out int32 [B]: ar_tok[b][n-1], the next block's anchor
 *  workspace >= orthrus_consensus_workspace_bytes(B, K, V, dtype) bytes.
 *  B >= 1, 1 <= K <= 64, 1 <= V < 2^31, B*K <= 65536.
 */
int orthrus_consensus(const void *diff_logits, const void *ar_logits, int B,
                      int K, int V, int dtype, int32_t *diff_tok,
                      int32_t *ar_tok, int32_t *n_match, int32_t *n_emit,
                      int32_t *emit_off, int32_t *emitted,
                      int32_t *next_anchor, void *workspace,
                      size_t workspace_bytes, hipStream_t stream);

size_t orthrus_consensus_workspace_bytes(int B, int K, int V, int dtype);

/*
 * orthrus_argmax -- the greedy-prediction half of orthrus_consensus on its
 * own (a pipeline needs the diffusion view's candidates before the AR pass;
 * summary §2.3 steps 1-2): idx[r] = argmax_v logits[r][v], lowest index on
 * ties, for r < rows.  Same kernels and workspace formula as consensus with
 * rows = 2*B*K.  rows >= 1, rows <= 131072.
 */
int orthrus_argmax(const void *logits, int64_t rows, int V, int dtype,
                   int32_t *idx, void *workspace, size_t workspace_bytes,
                   hipStream_t stream);

size_t orthrus_argmax_workspace_bytes(int64_t rows, int V, int dtype);

/*
 * orthrus_lmhead_argmax -- greedy prediction straight from hidden states
 * (summary §2.3: both views predict greedily; the consensus compares their
 * argmax tokens): idx[r] = argmax_v sum_k hidden[r][k] * weight[v][k], lowest
 * index on ties, without materialising the R x V logits.  bf16 inputs, fp32
 * accumulation.
 *
 *  hidden    [R][H] bf16, 16-byte aligned (final hidden states of R rows,
 *            e.g. the B*K block rows of one view)
 *  weight    [V][H] bf16, 16-byte aligned (the LM head, one row per token)
 *  idx       out int32 [R]
 *  workspace >= orthrus_lmhead_argmax_workspace_bytes(R, H, V, dtype) bytes
 *            (8-byte aligned); contents on entry are ignored.
 *  dtype must be BF16 (F32 -> ORTHRUS_ERR_UNSUPPORTED); H a multiple of 64,
 *  64 <= H <= 65536; 1 <= R <= 2,097,120; V >= 1.  The weight matrix is read
 *  once for R <= 256 (once per 256 rows beyond), so the call suits decode and
 *  serving batches; large R is bound by the matrix cores.  The argmax decision
 *  is taken on the fp32 accumulations: logits within a few fp32 ulps of each
 *  other may resolve differently from an exact evaluation.  Equal fp32
 *  logits go to the lowest index; the accumulation order over H is the same
 *  within each block of 128 vocabulary rows and rotates from block to block,
 *  so equal weight rows give bitwise-equal logits only inside one block.
 */
int orthrus_lmhead_argmax(const void *hidden, const void *weight, int R, int H,
                          int V, int dtype, int32_t *idx, void *workspace,
                          size_t workspace_bytes, hipStream_t stream);

size_t orthrus_lmhead_argmax_workspace_bytes(int R, int H, int V, int dtype);

/*
 * orthrus_kv_append -- commit (summary §2.3 step 3; agents-report core
 * design: accepted tokens' KV state is appended to the shared cache).
 *
 * For every layer l < num_layers, request b and i < n_emit[b], copies the AR
 * view's block row i (all Hkv heads, K and V) to cache row lens[b] + i, and
 * writes lens_out[b] = lens[b] + n_emit[b].  Rows are copied bit-exactly;
 * no other cache byte is written.  Work is distributed over the compacted
 * list of accepted rows (exclusive prefix sum of n_emit).
 *
 *  cache     layer 0's cache; layer l's k/v are at cache->k/v + l *
 *            cache_layer_stride ELEMENTS (paged: one page table for all
 *            layers).  cache->lens is read, never written.
 *  k_blk, v_blk  layer 0's AR-view block rows [B][K][Hkv][D]; layer l at
 *            + l * blk_layer_stride elements
 *  n_emit    device int32 [B], each in 0..K (e.g. orthrus_consensus output)
 *  lens_out  device int32 [B]; must not alias cache->lens
 * Caller contracts: lens[b] + n_emit[b] <= capacity (CONTIGUOUS) or the
 * pages for those rows exist (PAGED).
 */
int orthrus_kv_append(const orthrus_cache *cache, const void *k_blk,
                      const void *v_blk, const int32_t *n_emit,
                      int32_t *lens_out, int B, int K, int Hkv, int D,
                      int dtype, int num_layers, int64_t cache_layer_stride,
                      int64_t blk_layer_stride, hipStream_t stream);

/* Static string naming a status code ("ok", "null pointer", ...). */
const char *orthrus_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int orthrus_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ORTHRUS_H */
