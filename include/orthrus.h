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
 *  - No global mutable state (but for the static scratch array of
 *    orthrus_block_attn_noalloc): concurrent calls on different streams are
 *    safe as long as their outputs and workspaces do not overlap.
 *  - Tensors are dense, row-major, in the shapes given below, except the
 *    weight matrices of the projections and the LM head, which are read in
 *    the packed tile layout of orthrus_pack_weight; element type `dtype` is
 *    ORTHRUS_F32 (float) or ORTHRUS_BF16 (bfloat16).
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

typedef enum { ORTHRUS_F32 = 0, ORTHRUS_BF16 = 1, ORTHRUS_FP8_E4M3 = 2 } orthrus_dtype;

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
 *  kv_dtype  element type of k and v: 0 (the call's dtype) or ORTHRUS_FP8_E4M3.
 *            FP8_E4M3 (bf16 calls, D = 128): k and v hold OCP FP8 E4M3 codes
 *            (1 byte per element: sign, 4 exponent bits with bias 7, 3
 *            mantissa bits; no infinities; S.1111.111 is NaN; largest finite
 *            448) laid out as above, and k_scale / v_scale hold one fp32 scale
 *            per cache row and KV head, laid out like the rows without D
 *            ([B][Hkv][capacity], or [num_pages][Hkv][page_size]).  A row's
 *            values are code * scale.  Scales are powers of two (so that
 *            code * scale is exact in bf16); orthrus_kv_append writes
 *            2^e with e the smallest integer such that 448 * 2^e >= the
 *            row's largest |value| (e >= -120; an all-zero row gets 1).
 *            This is the "low-precision kernels" direction of the
 *            agents-report outlook: the cache streams half the bytes.
 * Caller contracts (not checked on the device): 0 <= lens[b]; for
 * CONTIGUOUS lens[b] <= capacity; for PAGED every page id the rows
 * 0..lens[b]-1 (and, for an append, the appended rows) map to is in
 * [0, num_pages); FP8 scales are finite powers of two.
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
    int32_t kv_dtype;            /* 0 or ORTHRUS_FP8_E4M3                   */
    int32_t reserved;            /* 0                                       */
    float *k_scale;              /* FP8: device fp32 scale per row and head */
    float *v_scale;              /* FP8: device fp32 scale per row and head */
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
 * orthrus_block_attn_noalloc -- orthrus_block_attn for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments and results, without
 * the workspace: the split partials go to a fixed array of
 * orthrus_block_attn_noalloc_max_workspace() bytes (64 MiB) that the library
 * holds on each GPU it runs on until the process ends.  A call whose
 * orthrus_block_attn_workspace_bytes(...) exceeds that size returns
 * ORTHRUS_ERR_WORKSPACE and launches nothing.  The array is looked up for
 * the current device (hipGetDevice) on its first call there; `stream` must
 * belong to that device.  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (other streams, other threads) race
 * on it; calls ordered on one stream do not.  Nothing in it needs clearing
 * between calls (every partial read is written by the same call first).
 */
int orthrus_block_attn_noalloc(const orthrus_cache *cache, const void *q,
                               const void *k_blk, const void *v_blk, void *out,
                               float *lse, int B, int K, int Hq, int Hkv,
                               int D, int dtype, int mask, float scale,
                               int num_splits, hipStream_t stream);

size_t orthrus_block_attn_noalloc_max_workspace(void);

/*
 * orthrus_mdiff_attn -- the diffusion view's attention under the training
 * block mask M_diff, forward only (summary §2.2).  A sequence carries NB
 * blocks; block j is an anchor followed by K-1 <mask> positions.  The mask
 * has two rules: the positions of block j see the clean AR context that
 * precedes the block's anchor (context rows t < anchors[b][j]), and the
 * positions of one block see each other bidirectionally (all K block rows,
 * no other block's).
 *
 * For sequence b, block j, block row i, query head h (KV head g = h/(Hq/Hkv)):
 *   keys = k_ctx rows 0..anchors[b][j]-1 of head g, then k_blk rows 0..K-1 of
 *          block (b, j);   out, lse as in orthrus_block_attn.
 *
 *  k_ctx, v_ctx [B][Hkv][ctx_capacity][D] dtype: each sequence's clean context
 *               (the AR view's keys/values, post-RoPE), read, never written
 *  anchors      device int32 [B][NB]: 0 <= anchors[b][j] <= ctx_capacity
 *               (caller contract, not checked on the device)
 *  max_anchor   host upper bound on the anchors (0 = ctx_capacity); sizes the
 *               split plan only: a wrong hint costs speed, never correctness
 *  q, out       [B][NB][K][Hq][D] dtype
 *  k_blk, v_blk [B][NB][K][Hkv][D] dtype: the diffusion view's block keys/values
 *  lse          [B][NB][Hq][K] float, may be NULL
 *  Same limits as orthrus_block_attn (K <= 64, D in {64, 128}, ...), and
 *  B*NB <= 2^24.  workspace >= orthrus_mdiff_attn_workspace_bytes(...).
 * Blocks are the requests of the block attention kernels, each reading its
 * sequence's context through a shared base (no copy); they are dispatched
 * from the last block of the last sequence, longest first when anchors grow
 * along a sequence.
 */
int orthrus_mdiff_attn(const void *k_ctx, const void *v_ctx,
                       int64_t ctx_capacity, const int32_t *anchors,
                       int64_t max_anchor, const void *q, const void *k_blk,
                       const void *v_blk, void *out, float *lse, int B, int NB,
                       int K, int Hq, int Hkv, int D, int dtype, float scale,
                       int num_splits, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

size_t orthrus_mdiff_attn_workspace_bytes(int64_t ctx_capacity,
                                          int64_t max_anchor, int B, int NB,
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
 * orthrus_consensus_tokens -- the consensus of orthrus_consensus from the two
 * views' greedy tokens themselves (e.g. from orthrus_lmhead_argmax, which
 * never writes logits): diff_tok, ar_tok device int32 [B][K] (read only);
 * the other outputs and limits as in orthrus_consensus.  No workspace.
 */
int orthrus_consensus_tokens(const int32_t *diff_tok, const int32_t *ar_tok,
                             int B, int K, int32_t *n_match, int32_t *n_emit,
                             int32_t *emit_off, int32_t *emitted,
                             int32_t *next_anchor, hipStream_t stream);

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
 *  weight    the LM head ([V][H] bf16, one row per token) in the packed tile
 *            layout of orthrus_pack_weight(weight, V, H, ...), 16-byte aligned
 *  idx       out int32 [R]
 *  workspace >= orthrus_lmhead_argmax_workspace_bytes(R, H, V, dtype) bytes
 *            (8-byte aligned); contents on entry are ignored.
 *  dtype must be BF16 (F32 -> ORTHRUS_ERR_UNSUPPORTED); H a multiple of 64,
 *  64 <= H <= 65536; 1 <= R <= 2,097,120; V >= 1.  The weight matrix is read
 *  once for R <= 256 (once per 256 rows beyond), so the call suits decode and
 *  serving batches; large R is bound by the matrix cores.  The argmax decision
 *  is taken on the fp32 accumulations: logits within a few fp32 ulps of each
 *  other may resolve differently from an exact evaluation.  Every vocabulary
 *  row goes through the same fp32 operations, so equal weight rows give
 *  bitwise-equal logits wherever they are in V, and equal fp32 logits go to
 *  the lowest index.
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
 *            layers).  cache->lens is read, never written.  An FP8_E4M3
 *            cache (bf16 rows, D = 128) quantizes each appended row and head:
 *            scale 2^e as described at orthrus_cache, code = value / 2^e
 *            rounded to nearest even; layer l's scales are at k_scale /
 *            v_scale + l * cache_layer_stride / D (the stride counts codes).
 *  k_blk, v_blk  layer 0's AR-view block rows [B][K][Hkv][D]; layer l at
 *            + l * blk_layer_stride elements
 *  n_emit    device int32 [B], each in 0..K (e.g. orthrus_consensus output)
 *  lens_out  device int32 [B]; may be cache->lens itself (an in-place
 *            advance: the rows are placed first, then a second launch writes
 *            lens_out), or any other buffer that overlaps nothing else
 * Caller contracts: lens[b] + n_emit[b] <= capacity (CONTIGUOUS) or the
 * pages for those rows exist (PAGED).
 */
int orthrus_kv_append(const orthrus_cache *cache, const void *k_blk,
                      const void *v_blk, const int32_t *n_emit,
                      int32_t *lens_out, int B, int K, int Hkv, int D,
                      int dtype, int num_layers, int64_t cache_layer_stride,
                      int64_t blk_layer_stride, hipStream_t stream);

/*
 * orthrus_stream_read -- a measurement aid, not part of the decode step: reads
 * `bytes` of device memory at `src` once, with `work_groups` work-groups each
 * streaming one contiguous share (16-byte loads, several in flight per lane),
 * and writes one folded word per work-group to sink[0..work_groups-1].  The
 * time of one launch is the streaming ceiling of a read of that size with
 * that many work-groups, on this chip, with nothing else to do: the yardstick
 * next to which the block attention's bytes per second are read (the
 * summary's §1 frames decoding as bound by memory bandwidth).
 *  bytes a positive multiple of 16; src 16-byte aligned; 1 <= work_groups
 *  <= 65535; sink device uint32 [work_groups].
 */
int orthrus_stream_read(const void *src, size_t bytes, int work_groups,
                        uint32_t *sink, hipStream_t stream);

/*
 * The decode step around the Orthrus kernels (summary §2.3 steps 1-2: the
 * diffusion view projects K candidates in one forward pass over its block,
 * the frozen AR view verifies the block in one forward pass; each pass runs
 * the model's layers on the block's B*K rows).  A Qwen3-style layer:
 *   x = rmsnorm(h) -> qkv = x Wqkv^T -> q, k = rmsnorm_head(q, k) then rotary
 *   embedding, v copied -> o = block attention -> h += o Wo^T ->
 *   x = rmsnorm(h) -> h += swiglu(x Wgu^T) Wdown^T
 * with an fp32 residual stream h and bf16 weights and projection inputs.
 * The views differ only in their attention weights (the diffusion module's
 * own Wqkv, Wo) and the block mask.  Rows are [R][...] row-major.
 */

/*
 * orthrus_pack_weight -- lays a weight out for the projections and the LM
 * head: w bf16 [N][Kin] row-major (16-byte aligned) is written to packed as
 * tiles of 128 rows x 64 columns (16 KiB each, rows in order, 128 bytes per
 * row); the tiles of one 128-row block follow each other in column order, and
 * the blocks follow each other: element (n, k) lands at bf16 index
 * ((n / 128) * (Kin / 64) + k / 64) * 8192 + (n % 128) * 64 + k % 64.  The
 * rows of the last block past N are zero.  Each work-group of a projection
 * or of the LM head then reads its weight as one contiguous run instead of
 * rows 2*Kin bytes apart that keep landing on the same HBM channels.  A
 * load-time step: weights are packed once and used by every decode step.
 *  Kin a multiple of 64; packed (16-byte aligned, not overlapping w) holds
 *  orthrus_packed_weight_bytes(N, Kin) bytes, else ORTHRUS_ERR_WORKSPACE.
 */
int orthrus_pack_weight(const void *w, int N, int Kin, void *packed,
                        size_t packed_bytes, hipStream_t stream);
/* ceil(N / 128) * 128 * Kin * 2 bytes; 0 if N < 1 or Kin is not a positive
 * multiple of 64. */
size_t orthrus_packed_weight_bytes(int N, int Kin);

/* orthrus_pack_weight_gate_up -- the MLP's gate/up weight w bf16 [2I][Kin]
 * (the I gate rows, then the I up rows) packed for orthrus_gemm_swiglu: as
 * orthrus_pack_weight of the 2I rows reordered so that every 8 rows are gate
 * rows 4g..4g+3 and then up rows I+4g..I+4g+3 (g = row / 8).  Each 128-row
 * block then holds 64 outputs' gate and up rows, and an unsplit projection
 * applies SwiGLU in its own epilogue.  I a multiple of 4; packed holds
 * orthrus_packed_weight_bytes(2I, Kin) bytes. */
int orthrus_pack_weight_gate_up(const void *w, int I, int Kin, void *packed,
                                size_t packed_bytes, hipStream_t stream);

/*
 * orthrus_gemm -- y = x W^T (+ residual): x bf16 [R][Kin], W bf16 [N][Kin]
 * (a linear layer's weight, one row per output) in the packed tile layout of
 * orthrus_pack_weight, residual fp32 [R][N] or NULL, y [R][N] in out_dtype
 * (F32 or BF16; y may be the residual itself).
 * fp32 accumulation in a fixed order per output that does not depend on R
 * (the input dimension is split S ways by N and Kin only; the partial sums
 * are added in split order).  Kin a multiple of 64, N a multiple of 4,
 * pointers 16-byte aligned.  workspace >= orthrus_gemm_workspace_bytes.
 */
int orthrus_gemm(const void *x, const void *w, const float *residual, void *y,
                 int R, int N, int Kin, int out_dtype, void *workspace,
                 size_t workspace_bytes, hipStream_t stream);
size_t orthrus_gemm_workspace_bytes(int R, int N, int Kin);

/* orthrus_rmsnorm -- y[r] = x[r] / sqrt(mean_k x[r][k]^2 + eps) * weight:
 * x fp32 [R][H], weight bf16 [H], y bf16 [R][H].  The sum of squares of a
 * row is formed in one fixed order that depends on H only.  H a multiple of
 * 4 and at most 16384; x 16-byte, weight and y 8-byte aligned. */
int orthrus_rmsnorm(const float *x, const void *weight, void *y, int R, int H,
                    float eps, hipStream_t stream);

/*
 * The projections with the operation that follows each of them in the layer,
 * fused into the second pass that adds the partial sums of the split input
 * dimension.  Each gives, bit for bit, what orthrus_gemm (fp32 output)
 * followed by the separate kernel gives: the partial sums are added in split
 * order and the epilogue's arithmetic is the separate kernel's.  They may
 * write partial sums also when the input dimension is not split, so
 * workspace >= orthrus_gemm_epilogue_workspace_bytes(R, N, Kin) bytes,
 * 16-byte aligned, with N the projection's output width.  Same x / W
 * contract as orthrus_gemm (W packed by orthrus_pack_weight, Kin a multiple
 * of 64, 16-byte aligned).
 */
size_t orthrus_gemm_epilogue_workspace_bytes(int R, int N, int Kin);

/* orthrus_gemm_rmsnorm -- the output (or down) projection with the residual
 * and the next RMSNorm: h += x W^T in place (fp32 [R][H], W bf16 [H][Kin]),
 * then xn = rmsnorm(h) * norm_weight (bf16 [R][H]).  = orthrus_gemm(x, W, h,
 * h, R, H, Kin, F32) then orthrus_rmsnorm(h, norm_weight, xn, R, H, eps).
 * H as for orthrus_rmsnorm; h 16-byte, norm_weight and xn 8-byte aligned. */
int orthrus_gemm_rmsnorm(const void *x, const void *w, float *h,
                         const void *norm_weight, void *xn, int R, int H,
                         int Kin, float eps, void *workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* orthrus_gemm_swiglu -- the MLP's gate/up projection and SwiGLU: W bf16
 * [2I][Kin] (the I gate rows, then the I up rows) packed by
 * orthrus_pack_weight_gate_up, act bf16 [R][I] = orthrus_gemm(x, W, NULL, gu,
 * R, 2I, Kin, F32) (W packed by orthrus_pack_weight) then orthrus_swiglu(gu,
 * act, R, I), without the fp32 gu ever being written.  When the input
 * dimension is not split (the Qwen3-8B MLP: 2I = 24,576 rows) it is one
 * launch that applies SwiGLU in its epilogue.  I a multiple of 4; act 8-byte
 * aligned. */
int orthrus_gemm_swiglu(const void *x, const void *w_gate_up, void *act, int R,
                        int I, int Kin, void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* orthrus_gemm_qk_norm_rope -- the QKV projection (W bf16 [(Hq+2Hkv)*D][Kin])
 * and orthrus_qk_norm_rope on its output, without the fp32 projection ever
 * being written: = orthrus_gemm(x, W, NULL, qkv, R, (Hq+2Hkv)*D, Kin, F32)
 * then orthrus_qk_norm_rope(qkv, ...).  Arguments as for those two. */
int orthrus_gemm_qk_norm_rope(const void *x, const void *w_qkv,
                              const void *q_norm, const void *k_norm,
                              const int32_t *lens, int K, void *q, void *k,
                              void *v, int R, int Hq, int Hkv, int D, int Kin,
                              float eps, float rope_theta, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* orthrus_qk_norm_rope -- from the fp32 projection qkv [R][(Hq+2Hkv)*D]
 * (q heads, then k heads, then v heads) of a block's rows (row r is block
 * row r % K of request r / K, at position lens[r / K] + r % K; lens device
 * int32): q and k heads are normalised by RMSNorm over D (weights q_norm,
 * k_norm bf16 [D]) and rotated by the rotary embedding (pairs (d, d + D/2),
 * angle position * rope_theta^(-2d/D), computed in fp64); v is copied.
 * Outputs bf16 q [R][Hq][D], k [R][Hkv][D], v [R][Hkv][D] -- the block
 * attention's q, k_blk, v_blk.  D = 128, R a multiple of K. */
int orthrus_qk_norm_rope(const float *qkv, const void *q_norm,
                         const void *k_norm, const int32_t *lens, int K,
                         void *q, void *k, void *v, int R, int Hq, int Hkv,
                         int D, float eps, float rope_theta, hipStream_t stream);

/* orthrus_block_tokens -- a view's block input tokens: out[b][0] = anchor[b]
 * and out[b][i] = cand[b][i-1] for i >= 1 (the AR view: anchor, then the
 * first K-1 candidates), or = fill when cand is NULL (the diffusion view:
 * anchor, then <mask>).  Device int32: anchor [B], cand [B][K], out [B][K]. */
int orthrus_block_tokens(const int32_t *anchor, const int32_t *cand,
                         int32_t fill, int32_t *out, int B, int K,
                         hipStream_t stream);

/* orthrus_swiglu -- act[r][i] = silu(gate_up[r][i]) * gate_up[r][I + i],
 * silu(g) = g / (1 + e^-g): gate_up fp32 [R][2I], act bf16 [R][I].  I a
 * multiple of 4; gate_up 16-byte, act 8-byte aligned. */
int orthrus_swiglu(const float *gate_up, void *act, int R, int I,
                   hipStream_t stream);

/* orthrus_embed -- h[r] = table[tokens[r]] (bf16 -> fp32): tokens device int32
 * [R] (caller contract: valid rows of table), table bf16 [rows][H], h fp32
 * [R][H]. */
int orthrus_embed(const int32_t *tokens, const void *table, float *h, int R,
                  int H, hipStream_t stream);

/* Static string naming a status code ("ok", "null pointer", ...). */
const char *orthrus_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int orthrus_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ORTHRUS_H */
