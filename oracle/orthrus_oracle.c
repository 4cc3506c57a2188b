/*
 * Orthrus decode-step oracle: a plain, slow fp64 CPU implementation.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header or table with the HIP
 * library.
 *
 * Sources (the pages the method is described on):
 *   [SUM]  "Orthrus: Memory-Efficient Parallel Token Generation via
 *          Dual-View Diffusion", gist.science technical summary:
 *          §2.1 dual-view attention over one shared KV cache,
 *          §2.2 block masking (anchor + K-1 mask slots, bidirectional block),
 *          §2.3 inference: parallel projection, AR verification, left-to-right
 *               consensus and commit.
 *   [ABS]  the paper's abstract (chatpaper.ai page): both views read the same
 *          KV cache; exact consensus makes inference lossless.
 *   [REP]  agents-report.net commentary, section on the core design: accepted
 *          tokens' KV state is appended to the shared cache.
 *
 * Every floating-point step is fp64 on the exact input values (bf16 and fp32
 * inputs convert to fp64 without rounding).  No blocking, fusion or
 * reordering: each output is its definition written out.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { O_CONTIGUOUS = 0, O_PAGED = 1 };
enum { O_BIDIR = 0, O_CAUSAL = 1 };

/* Address of cache row t of request b, KV head g.
 * Contiguous layout [B][Hkv][cap][D]; paged layout [num_pages][Hkv][page][D]
 * where logical token t of request b lives in page page_table[b][t / page],
 * slot t % page.  Returns NULL if the page table points out of range. */
static const double *cache_row(const double *base, int layout, long cap,
                               int page_size, const int32_t *page_table,
                               int max_pages, int num_pages, int Hkv, int D,
                               int b, int g, long t)
{
    if (layout == O_CONTIGUOUS)
        return base + (((long)b * Hkv + g) * cap + t) * D;
    long lp = t / page_size;
    if (lp >= max_pages) return NULL;
    int32_t page = page_table[(long)b * max_pages + lp];
    if (page < 0 || page >= num_pages) return NULL;
    return base + (((long)page * Hkv + g) * page_size + t % page_size) * D;
}

/*
 * Shared-KV block attention for one layer.  [SUM] §2.1-§2.3, [REP].
 *
 * For request b, query head h (KV head g = h / (Hq/Hkv)) and block row i, the
 * key set is every cache row 0..lens[b]-1 of head g, plus block rows
 *   j = 0..K-1  (mask BIDIR, the diffusion view: the block attends to itself
 *                bidirectionally)
 *   j = 0..i    (mask CAUSAL, the AR verification view: causal, row i sees
 *                itself)
 * Scores s_t = scale * <q, k_t>; out = sum_t exp(s_t - m) v_t / sum_t
 * exp(s_t - m) with m = max_t s_t; lse = m + log(sum_t exp(s_t - m)).
 *
 * q, k_blk, v_blk, out: [B][K][H][D]; lse: [B][Hq][K] (may be NULL).
 * Returns 0, or -1 on a bad argument / page index.
 */
int oracle_block_attn(const double *q, const double *k_cache,
                      const double *v_cache, int layout, long cap,
                      int page_size, const int32_t *page_table, int max_pages,
                      int num_pages, const int32_t *lens, const double *k_blk,
                      const double *v_blk, int B, int K, int Hq, int Hkv,
                      int D, int mask, double scale, double *out, double *lse)
{
    if (B < 1 || K < 1 || Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv) return -1;
    const int G = Hq / Hkv;
    int bad = 0;
    long nrows = (long)B * Hq * K;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (long row = 0; row < nrows; ++row) {
        const int b = (int)(row / ((long)Hq * K));
        const int h = (int)((row / K) % Hq);
        const int i = (int)(row % K);
        const int g = h / G;
        const long L = lens[b];
        const int nblk = (mask == O_BIDIR) ? K : i + 1;
        const long n = L + nblk;
        const double *qv = q + (((long)b * K + i) * Hq + h) * D;
        double *s = (double *)malloc(sizeof(double) * (size_t)n);
        const double **vrow = (const double **)malloc(sizeof(double *) * (size_t)n);
        if (!s || !vrow) { bad = 1; free(s); free(vrow); continue; }
        for (long t = 0; t < n; ++t) {
            const double *kr, *vr;
            if (t < L) {
                kr = cache_row(k_cache, layout, cap, page_size, page_table,
                               max_pages, num_pages, Hkv, D, b, g, t);
                vr = cache_row(v_cache, layout, cap, page_size, page_table,
                               max_pages, num_pages, Hkv, D, b, g, t);
            } else {
                long j = t - L;
                kr = k_blk + (((long)b * K + j) * Hkv + g) * D;
                vr = v_blk + (((long)b * K + j) * Hkv + g) * D;
            }
            if (!kr || !vr) { bad = 1; break; }
            double dot = 0.0;
            for (int d = 0; d < D; ++d) dot += qv[d] * kr[d];
            s[t] = scale * dot;
            vrow[t] = vr;
        }
        if (!bad) {
            double m = -INFINITY;
            for (long t = 0; t < n; ++t) if (s[t] > m) m = s[t];
            double denom = 0.0;
            for (long t = 0; t < n; ++t) {
                s[t] = exp(s[t] - m);            /* s now holds the weight w_t */
                denom += s[t];
            }
            double *o = out + (((long)b * K + i) * Hq + h) * D;
            for (int d = 0; d < D; ++d) {
                double acc = 0.0;
                for (long t = 0; t < n; ++t) acc += s[t] * vrow[t][d];
                o[d] = acc / denom;
            }
            if (lse) lse[((long)b * Hq + h) * K + i] = m + log(denom);
        }
        free(s);
        free(vrow);
    }
    return bad ? -1 : 0;
}

/*
 * Greedy prediction of one row: the smallest index v with x[v] >= x[u] for
 * every u (numeric comparison, so -0.0 equals +0.0).  [SUM] §2.3 step 3: a
 * candidate is judged against the frozen AR view's greedy choice; both views'
 * candidates are row argmaxes of their logits.  Returns -1 if a row holds a
 * NaN (no greedy choice is defined then).
 */
int oracle_argmax_rows(const double *x, long rows, long V, int32_t *idx)
{
    if (rows < 0 || V < 1) return -1;
    for (long r = 0; r < rows; ++r) {
        const double *row = x + r * V;
        long best = 0;
        for (long v = 0; v < V; ++v) {
            if (isnan(row[v])) return -1;
            if (row[v] > row[best]) best = v;
        }
        idx[r] = (int32_t)best;
    }
    return 0;
}

/*
 * Exact left-to-right consensus.  [SUM] §2.3 step 3.
 *
 * Block row i of both views predicts the same position (the token after the
 * i-th block input).  Scan i = 0, 1, ...: the first i with d[i] != a[i] is
 * the divergence index j (K if none).  The tokens a[0..j-1] equal the
 * accepted candidates d[0..j-1]; a[j] is the AR correction.  So the step
 * emits n = min(j + 1, K) tokens a[0..n-1]; the last emitted token becomes
 * the next block's anchor.  emit_off is the exclusive prefix sum of n over
 * the batch (emit_off[B] = total) and emitted packs the tokens at those
 * offsets.
 */
void oracle_consensus(const int32_t *d, const int32_t *a, int B, int K,
                      int32_t *j_out, int32_t *n_out, int32_t *emit_off,
                      int32_t *emitted, int32_t *next_anchor)
{
    int32_t off = 0;
    for (int b = 0; b < B; ++b) {
        const int32_t *db = d + (long)b * K;
        const int32_t *ab = a + (long)b * K;
        int j = 0;
        while (j < K && db[j] == ab[j]) ++j;      /* strict left-to-right */
        int n = (j < K) ? j + 1 : K;
        j_out[b] = j;
        n_out[b] = n;
        emit_off[b] = off;
        for (int i = 0; i < n; ++i) emitted[off + i] = ab[i];
        next_anchor[b] = ab[n - 1];
        off += n;
    }
    emit_off[B] = off;
}

/*
 * Commit: append the accepted positions' KV to the shared cache.  [SUM] §2.3
 * step 3 (commit the agreed prefix) and [REP] (the accepted tokens' KV state
 * is appended to the shared cache).
 *
 * The rows appended are the AR view's block rows 0..n[b]-1 (the anchor and
 * the n-1 accepted inputs after it), written at cache positions lens[b]+i
 * for every layer and KV head.  Every other cache byte is left unchanged;
 * lens_out[b] = lens[b] + n[b].  Elements are copied as opaque bytes.
 *
 * k_cache/v_cache: per layer (stride cache_layer_stride elements) the cache
 * layout of oracle_block_attn; k_blk/v_blk: per layer (stride
 * blk_layer_stride) [B][K][Hkv][D].  Returns -1 on a bad argument, a page
 * index out of range or a row beyond the capacity.
 */
int oracle_kv_append(unsigned char *k_cache, unsigned char *v_cache,
                     int layout, long cap, int page_size,
                     const int32_t *page_table, int max_pages, int num_pages,
                     const int32_t *lens, const unsigned char *k_blk,
                     const unsigned char *v_blk, const int32_t *n,
                     int32_t *lens_out, int B, int K, int Hkv, int D,
                     int elem_bytes, int layers, long cache_layer_stride,
                     long blk_layer_stride)
{
    const long row_bytes = (long)D * elem_bytes;
    for (int b = 0; b < B; ++b)
        if (n[b] < 0 || n[b] > K) return -1;
    for (int l = 0; l < layers; ++l) {
        for (int b = 0; b < B; ++b) {
            for (int i = 0; i < n[b]; ++i) {
                long t = (long)lens[b] + i;
                for (int g = 0; g < Hkv; ++g) {
                    long dst;
                    if (layout == O_CONTIGUOUS) {
                        if (t >= cap) return -1;
                        dst = ((long)b * Hkv + g) * cap + t;
                    } else {
                        long lp = t / page_size;
                        if (lp >= max_pages) return -1;
                        int32_t page = page_table[(long)b * max_pages + lp];
                        if (page < 0 || page >= num_pages) return -1;
                        dst = ((long)page * Hkv + g) * page_size + t % page_size;
                    }
                    long src = ((long)b * K + i) * Hkv + g;
                    long cdst = (l * cache_layer_stride + dst * D) * elem_bytes;
                    long csrc = (l * blk_layer_stride + src * D) * elem_bytes;
                    memcpy(k_cache + cdst, k_blk + csrc, (size_t)row_bytes);
                    memcpy(v_cache + cdst, v_blk + csrc, (size_t)row_bytes);
                }
            }
        }
    }
    for (int b = 0; b < B; ++b) lens_out[b] = lens[b] + n[b];
    return 0;
}

/* Number of OpenMP threads the oracle runs with (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the number of OpenMP threads later calls use (no effect without
 * OpenMP); the benchmark times the oracle at one thread and at all. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Training-time diffusion-view attention under the block mask M_diff, forward
 * only.  [SUM] §2.2: a sequence carries several blocks; each block is an
 * anchor (kept visible) followed by K-1 <mask> positions.  The diffusion head
 * reads the blocks under a mask with two rules:
 *   1. causal context: every position of block j sees the clean AR context
 *      that precedes the block's anchor, i.e. context rows t < anchor[j];
 *   2. bidirectional block: the positions of one block see each other, all
 *      K of them; positions of other blocks are never seen.
 *
 * For sequence b, block j, block row i and query head h (KV head
 * g = h / (Hq/Hkv)): keys = k_ctx rows 0..anchor[b][j]-1 of head g, then
 * k_blk rows 0..K-1 of block (b, j).  s_t = scale * <q, k_t>; out = softmax
 * weighted sum of the values; lse = log sum_t exp(s_t).
 *
 *  k_ctx, v_ctx  [B][Hkv][cap][D]   the clean context (AR view), per sequence
 *  anchors       [B][NB]            anchor position of each block, 0..cap
 *  q, out        [B][NB][K][Hq][D]
 *  k_blk, v_blk  [B][NB][K][Hkv][D] the diffusion view's own block K/V
 *  lse           [B][NB][Hq][K]     may be NULL
 * Returns 0, or -1 on a bad argument (an anchor outside 0..cap).
 */
int oracle_mdiff_attn(const double *q, const double *k_ctx, const double *v_ctx,
                      long cap, const int32_t *anchors, const double *k_blk,
                      const double *v_blk, int B, int NB, int K, int Hq,
                      int Hkv, int D, double scale, double *out, double *lse)
{
    if (B < 1 || NB < 1 || K < 1 || Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv) return -1;
    for (long x = 0; x < (long)B * NB; ++x)
        if (anchors[x] < 0 || anchors[x] > cap) return -1;
    const int G = Hq / Hkv;
    const long nrows = (long)B * NB * K * Hq;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (long row = 0; row < nrows; ++row) {
        const long blk = row / ((long)K * Hq);          /* b * NB + j */
        const int i = (int)((row / Hq) % K);
        const int h = (int)(row % Hq);
        const int b = (int)(blk / NB);
        const int g = h / G;
        const long A = anchors[blk];
        const long n = A + K;
        const double *qv = q + ((blk * K + i) * Hq + h) * D;
        double *w = (double *)malloc(sizeof(double) * (size_t)n);
        if (!w) { bad = 1; continue; }
        /* scores: the context rows before the anchor, then the whole block */
        for (long t = 0; t < n; ++t) {
            const double *kr = t < A ? k_ctx + (((long)b * Hkv + g) * cap + t) * D
                                     : k_blk + ((blk * K + (t - A)) * Hkv + g) * D;
            double dot = 0.0;
            for (int d = 0; d < D; ++d) dot += qv[d] * kr[d];
            w[t] = scale * dot;
        }
        double m = -INFINITY;
        for (long t = 0; t < n; ++t) if (w[t] > m) m = w[t];
        double denom = 0.0;
        for (long t = 0; t < n; ++t) { w[t] = exp(w[t] - m); denom += w[t]; }
        double *o = out + ((blk * K + i) * Hq + h) * D;
        for (int d = 0; d < D; ++d) {
            double acc = 0.0;
            for (long t = 0; t < n; ++t) {
                const double *vr = t < A ? v_ctx + (((long)b * Hkv + g) * cap + t) * D
                                         : v_blk + ((blk * K + (t - A)) * Hkv + g) * D;
                acc += w[t] * vr[d];
            }
            o[d] = acc / denom;
        }
        if (lse) lse[(blk * Hq + h) * K + i] = m + log(denom);
        free(w);
    }
    return bad ? -1 : 0;
}

/*
 * FP8 KV cache (the agents-report outlook names low-precision kernels as the
 * direction; the format is the OCP 8-bit floating point E4M3 of the OCP
 * "OFP8" specification): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
 * bits.  Exponent field 0 holds the subnormals m * 2^-9 (m = 0..7); fields
 * 1..15 hold (1 + m/8) * 2^(field-7); the code S.1111.111 is NaN and there
 * are no infinities, so the largest finite magnitude is 1.75 * 2^8 = 448.
 */

/* Value of one code (NaN for S.1111.111). */
double oracle_e4m3_decode(int code)
{
    const int sign = (code >> 7) & 1;
    const int field = (code >> 3) & 15;
    const int m = code & 7;
    double v;
    if (field == 15 && m == 7) return NAN;
    if (field == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, field - 7);
    return sign ? -v : v;
}

/* Nearest code to x, ties to the even code (the one whose mantissa is even);
 * |x| must not exceed 448.  Returns -1 otherwise. */
int oracle_e4m3_encode(double x)
{
    if (isnan(x) || fabs(x) > 448.0) return -1;
    const int sign = signbit(x) ? 1 : 0;
    double a = fabs(x);
    /* candidates: the representable magnitudes are k * 2^(E-3) on the
     * binade [2^E, 2^(E+1)) for E >= -6, and k * 2^-9 below 2^-6 */
    int field;
    double step;
    if (a < ldexp(1.0, -6)) {
        field = 0;
        step = ldexp(1.0, -9);
    } else {
        int E;
        frexp(a, &E);          /* a = f * 2^E, f in [0.5, 1): binade [2^(E-1), 2^E) */
        E -= 1;
        field = E + 7;
        step = ldexp(1.0, E - 3);
    }
    double q = a / step;       /* exact: a and step are dyadic */
    double lo = floor(q);
    double r = q - lo;
    double k = (r > 0.5 || (r == 0.5 && fmod(lo, 2.0) != 0.0)) ? lo + 1.0 : lo;
    /* k counts steps of this binade: field 0 codes k = 0..8 (8 = 2^-6, the
     * smallest normal, whose code is 0.0001.000 = 8); normal binades k =
     * 8..16 (16 = the next binade's 1.000) */
    int code;
    if (field == 0) {
        code = (int)k;
    } else {
        int m = (int)k - 8;
        int f = field;
        if (m == 8) { m = 0; f += 1; }
        code = (f << 3) | m;
    }
    if (code > 0x7e) return -1;           /* beyond 448 */
    return (sign << 7) | code;
}

/* Scale exponent of a row whose largest magnitude is amax: the smallest
 * integer e >= -120 with 448 * 2^e >= amax (so every value / 2^e fits the
 * format); 0 for amax = 0.  Written as the search it defines. */
int oracle_fp8_scale_exp(double amax)
{
    if (amax == 0.0) return 0;
    int e = -120;
    while (448.0 * ldexp(1.0, e) < amax) ++e;
    return e;
}

/*
 * Commit into an FP8 cache: the accepted AR rows of oracle_kv_append, each
 * (row, KV head) of D values quantized on the way.  Scale s = 2^e with
 * e = oracle_fp8_scale_exp(max |value|); code = encode(value / s).  Codes go
 * where oracle_kv_append puts elements (one byte each); the scale goes to
 * the same row index of k_scale / v_scale (the row layout without D).
 * k_blk/v_blk are fp64 values (exact copies of the bf16 rows).  Returns -1 on
 * a bad argument or page.
 */
int oracle_kv_append_fp8(unsigned char *k_cache, unsigned char *v_cache, float *k_scale,
                         float *v_scale, int layout, long cap, int page_size,
                         const int32_t *page_table, int max_pages, int num_pages,
                         const int32_t *lens, const double *k_blk, const double *v_blk,
                         const int32_t *n, int32_t *lens_out, int B, int K, int Hkv, int D,
                         int layers, long cache_layer_stride, long blk_layer_stride)
{
    for (int b = 0; b < B; ++b)
        if (n[b] < 0 || n[b] > K) return -1;
    for (int l = 0; l < layers; ++l) {
        for (int b = 0; b < B; ++b) {
            for (int i = 0; i < n[b]; ++i) {
                long t = (long)lens[b] + i;
                for (int g = 0; g < Hkv; ++g) {
                    long dst;
                    if (layout == O_CONTIGUOUS) {
                        if (t >= cap) return -1;
                        dst = ((long)b * Hkv + g) * cap + t;
                    } else {
                        long lp = t / page_size;
                        if (lp >= max_pages) return -1;
                        int32_t page = page_table[(long)b * max_pages + lp];
                        if (page < 0 || page >= num_pages) return -1;
                        dst = ((long)page * Hkv + g) * page_size + t % page_size;
                    }
                    for (int which = 0; which < 2; ++which) {
                        const double *src = (which ? v_blk : k_blk) + l * blk_layer_stride +
                                            (((long)b * K + i) * Hkv + g) * D;
                        unsigned char *cc = (which ? v_cache : k_cache) + l * cache_layer_stride;
                        float *sc = (which ? v_scale : k_scale) + l * (cache_layer_stride / D);
                        double amax = 0.0;
                        for (int d = 0; d < D; ++d)
                            if (fabs(src[d]) > amax) amax = fabs(src[d]);
                        const int e = oracle_fp8_scale_exp(amax);
                        for (int d = 0; d < D; ++d) {
                            const int code = oracle_e4m3_encode(ldexp(src[d], -e));
                            if (code < 0) return -1;
                            cc[dst * D + d] = (unsigned char)code;
                        }
                        sc[dst] = (float)ldexp(1.0, e);
                    }
                }
            }
        }
    }
    for (int b = 0; b < B; ++b) lens_out[b] = lens[b] + n[b];
    return 0;
}

/* oracle_e4m3_decode over an array. */
void oracle_e4m3_decode_array(const unsigned char *codes, long n, double *out)
{
    for (long i = 0; i < n; ++i) out[i] = oracle_e4m3_decode(codes[i]);
}
