// Greedy prediction (row argmax) and exact left-to-right consensus, gfx950.
//
// Operation (Orthrus summary on gist.science, §2.3 step 3): a diffusion
// candidate is accepted iff it equals the frozen AR view's greedy choice,
// scanning the block left to right; at the first divergence j the agreed
// prefix is kept and the AR view's token at j is added.  Rows i of both
// views predict the same position, so the step emits n = min(j+1, K) tokens
// ar[0..n-1] and the last one is the next anchor.
//
// Design: the logits are streamed once (HBM-bound).  Each row of V entries
// is cut into 16 KiB chunks, one work-group per (row, chunk), coalesced
// 16-byte loads, a per-thread running (max, first index) in increasing index
// order, then a wave/work-group reduction of 64-bit keys whose maximum is the
// largest value with the lowest index (-0.0 and +0.0 compare equal).  A
// single work-group then reduces the chunk keys, runs the consensus scan per
// request and an exclusive prefix sum over the batch for the packed output.
#include "common.hpp"
#include "kernels.hpp"

namespace orthrus {

template <bool BF16>
__global__ void __launch_bounds__(256)
argmax_partial_kernel(const void *l0, const void *l1, int64_t rows0, int V, uint64_t *ws,
                      int chunks)
{
    constexpr int ES = BF16 ? 2 : 4;
    constexpr int E = kArgmaxChunkBytes / ES;   // elements per chunk
    constexpr int VE = 16 / ES;                 // elements per 16-byte vector
    constexpr int NV = E / VE / 256;            // vectors per thread (4)
    __shared__ uint64_t red[4];

    const int64_t row = blockIdx.x / chunks;
    const int chunk = blockIdx.x % chunks;
    const int tid = threadIdx.x;
    const char *base = row < rows0 ? (const char *)l0 + row * (int64_t)V * ES
                                   : (const char *)l1 + (row - rows0) * (int64_t)V * ES;
    const int beg = chunk * E;
    const int end = (beg + E < V) ? beg + E : V;

    float best = -INFINITY;
    uint32_t bi = 0;
    bool has = false;
    auto consider = [&](float v, uint32_t idx) {
        if (!has || v > best) { best = v; bi = idx; has = true; }
    };

    int scalar_from = beg;
    if ((((uintptr_t)base) & 15) == 0) {
        const int nvec = (end - beg) / VE;
        u32x4 buf[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int vi = tid + 256 * k;
            if (vi < nvec) buf[k] = *(const u32x4 *)(base + (int64_t)(beg + vi * VE) * ES);
        }
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int vi = tid + 256 * k;
            if (vi < nvec) {
                const uint32_t i0 = beg + vi * VE;
                if (BF16) {
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        consider(__uint_as_float(buf[k][w] << 16), i0 + 2 * w);
                        consider(__uint_as_float(buf[k][w] & 0xffff0000u), i0 + 2 * w + 1);
                    }
                } else {
#pragma unroll
                    for (int w = 0; w < 4; ++w) consider(__uint_as_float(buf[k][w]), i0 + w);
                }
            }
        }
        scalar_from = beg + nvec * VE;
    }
    for (int i = scalar_from + tid; i < end; i += 256) {
        float v;
        if (BF16) v = bf16_bits_to_f32(((const uint16_t *)base)[i]);
        else v = ((const float *)base)[i];
        consider(v, (uint32_t)i);
    }

    uint64_t key = has ? argmax_key(best, bi) : 0ull;
    key = wave_max_u64(key);
    if ((tid & 63) == 0) red[tid >> 6] = key;
    __syncthreads();
    if (tid == 0) {
        uint64_t k = red[0];
#pragma unroll
        for (int w = 1; w < 4; ++w) k = red[w] > k ? red[w] : k;
        ws[row * chunks + chunk] = k;
    }
}

// Keys of rows r0..r0+3 (chunk keys ws[row][0..chunks)), reduced over the
// wave: lanes load chunks lane, lane+64, ...; all four rows' loads are issued
// before the reductions.  Rows past `rows` give 0.
__device__ __forceinline__ void reduce_rows4(const uint64_t *ws, int64_t rows, int chunks,
                                             int64_t r0, int lane, uint64_t (&k)[4])
{
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        k[u] = 0;
        if (r0 + u < rows && lane < chunks) k[u] = ws[(r0 + u) * chunks + lane];
    }
    for (int c = lane + 64; c < chunks; c += 64)
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (r0 + u < rows) {
                const uint64_t v = ws[(r0 + u) * chunks + c];
                k[u] = v > k[u] ? v : k[u];
            }
#pragma unroll
    for (int u = 0; u < 4; ++u) k[u] = wave_max_u64(k[u]);
}

__global__ void __launch_bounds__(256)
argmax_finalize_kernel(const uint64_t *ws, int64_t rows, int chunks, int32_t *idx0, int64_t rows0,
                       int32_t *idx1)
{
    // one wave per 4 rows: lanes take the chunk keys, a wave reduction each;
    // rows below rows0 go to idx0, the rest to idx1
    const int lane = threadIdx.x & 63;
    const int64_t r0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4;
    uint64_t k[4];
    reduce_rows4(ws, rows, chunks, r0, lane, k);
    if (lane == 0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t row = r0 + u;
            if (row >= rows) break;
            const int32_t tok = (int32_t)argmax_key_index(k[u]);
            if (row < rows0) idx0[row] = tok;
            else idx1[row - rows0] = tok;
        }
    }
}

// One work-group: per-request consensus and the packed emission with an
// exclusive prefix sum over the batch.  TOKENS: it first reduces the chunk
// keys to the tokens of both views itself (small batches, 2*B*K <= 1024:
// saves a launch); otherwise argmax_finalize_kernel did.  Requests are taken
// one per wave (lane i = block position i, K <= 64), so every step is one
// memory round trip, not K.
template <bool TOKENS>
__global__ void __launch_bounds__(1024)
consensus_finalize_kernel(const uint64_t *ws, int chunks, int B, int K, int32_t *diff_tok,
                          int32_t *ar_tok, int32_t *n_match, int32_t *n_emit, int32_t *emit_off,
                          int32_t *emitted, int32_t *next_anchor)
{
    __shared__ int part[1024];
    // small batches (TOKENS, 2*B*K <= 1024): tokens and counts stay in LDS
    __shared__ int s_tok[TOKENS ? 1024 : 1];
    __shared__ int s_n[TOKENS ? 513 : 1];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    constexpr int NWAVE = 16;
    const int BK = B * K;
    if (TOKENS) {
        for (int r0 = wave * 4; r0 < 2 * BK; r0 += NWAVE * 4) {
            uint64_t k[4];
            reduce_rows4(ws, 2 * BK, chunks, r0, lane, k);
            if (lane == 0) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int row = r0 + u;
                    if (row >= 2 * BK) break;
                    const int32_t tok = (int32_t)argmax_key_index(k[u]);
                    s_tok[row] = tok;
                    if (row < BK) diff_tok[row] = tok;
                    else ar_tok[row - BK] = tok;
                }
            }
        }
        __syncthreads();
    }
    auto dtok = [&](int i) { return TOKENS ? s_tok[i] : diff_tok[i]; };
    auto atok = [&](int i) { return TOKENS ? s_tok[BK + i] : ar_tok[i]; };
    // per request (one wave): first divergence j, emitted count n, next anchor
    for (int b = wave; b < B; b += NWAVE) {
        const int d = lane < K ? dtok(b * K + lane) : 0;
        const int a = lane < K ? atok(b * K + lane) : 0;
        const uint64_t mism = __ballot(lane < K && d != a);
        const int j = mism ? __builtin_ctzll(mism) : K;
        const int n = (j < K) ? j + 1 : K;
        const int anchor = __shfl(a, n - 1, 64);
        if (lane == 0) {
            n_match[b] = j;
            n_emit[b] = n;
            next_anchor[b] = anchor;
            if (TOKENS) s_n[b] = n;
        }
    }
    __syncthreads();
    auto nof = [&](int b) { return TOKENS ? s_n[b] : n_emit[b]; };
    if (B <= 64) {
        // exclusive prefix sum of n on one wave (lane = request)
        __shared__ int s_off[64];
        if (wave == 0) {
            const int n = lane < B ? nof(lane) : 0;
            int incl = n;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int v = __shfl_up(incl, d, 64);
                if (lane >= d) incl += v;
            }
            if (lane < B) {
                emit_off[lane] = incl - n;
                s_off[lane] = incl - n;
            }
            if (lane == B - 1) emit_off[B] = incl;
        }
        __syncthreads();
        for (int b = wave; b < B; b += NWAVE) {
            const int n = nof(b);
            if (lane < n) emitted[s_off[b] + lane] = atok(b * K + lane);
        }
        return;
    }
    // exclusive prefix sum of n: each thread owns a contiguous run of
    // requests (two-level)
    const int per = (B + 1023) / 1024;
    const int b0 = tid * per;
    const int b1 = (b0 + per < B) ? b0 + per : B;
    int local = 0;
    for (int b = b0; b < b1; ++b) local += nof(b);
    part[tid] = local;
    __syncthreads();
    // inclusive scan of the 1024 partial sums (Hillis-Steele)
    for (int off = 1; off < 1024; off <<= 1) {
        const int v = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int run = part[tid] - local;   // exclusive prefix of this thread's run
    for (int b = b0; b < b1; ++b) {
        emit_off[b] = run;
        run += nof(b);
    }
    if (tid == 1023) emit_off[B] = part[1023];
    // packed emission: request b's tokens a_0..a_{n-1} at its offset, one
    // wave each (the offset is the inclusive scan of the owning thread's run,
    // read back from LDS)
    __syncthreads();
    for (int b = wave; b < B; b += NWAVE) {
        const int owner = b / per;
        int off = part[owner];
        // part[owner] is the inclusive prefix through owner's run; step back
        // over the requests of that run from b on
        for (int bb = owner * per + per - 1; bb >= b; --bb)
            if (bb < B) off -= nof(bb);
        const int n = nof(b);
        if (lane < n) emitted[off + lane] = atok(b * K + lane);
    }
}

hipError_t launch_argmax_partial(const void *logits0, const void *logits1, int64_t rows0,
                                 int64_t rows1, int V, int dtype, uint64_t *ws, int chunks,
                                 hipStream_t st)
{
    const int64_t nblk = (rows0 + rows1) * chunks;
    if (dtype == 1)
        hipLaunchKernelGGL(argmax_partial_kernel<true>, dim3((unsigned)nblk), dim3(256), 0, st,
                           logits0, logits1, rows0, V, ws, chunks);
    else
        hipLaunchKernelGGL(argmax_partial_kernel<false>, dim3((unsigned)nblk), dim3(256), 0, st,
                           logits0, logits1, rows0, V, ws, chunks);
    return hipGetLastError();
}

hipError_t launch_argmax_finalize(const uint64_t *ws, int64_t rows, int chunks, int32_t *idx,
                                  hipStream_t st)
{
    hipLaunchKernelGGL(argmax_finalize_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0,
                       st, ws, rows, chunks, idx, rows, idx);
    return hipGetLastError();
}

hipError_t launch_consensus_tokens(const int32_t *diff_tok, const int32_t *ar_tok, int B, int K,
                                  int32_t *n_match, int32_t *n_emit, int32_t *emit_off,
                                  int32_t *emitted, int32_t *next_anchor, hipStream_t st)
{
    // the tokens are given: only the consensus pass (which reads, never
    // writes, diff_tok and ar_tok when its TOKENS flag is off)
    hipLaunchKernelGGL(consensus_finalize_kernel<false>, dim3(1), dim3(1024), 0, st,
                       (const uint64_t *)nullptr, 0, B, K, const_cast<int32_t *>(diff_tok),
                       const_cast<int32_t *>(ar_tok), n_match, n_emit, emit_off, emitted,
                       next_anchor);
    return hipGetLastError();
}

hipError_t launch_consensus_finalize(const uint64_t *ws, int B, int K, int chunks,
                                     int32_t *diff_tok, int32_t *ar_tok, int32_t *n_match,
                                     int32_t *n_emit, int32_t *emit_off, int32_t *emitted,
                                     int32_t *next_anchor, hipStream_t st)
{
    // tokens of both views (rows 0..BK-1: diffusion, BK..2BK-1: AR), then the
    // consensus over them
    const int64_t rows = 2 * (int64_t)B * K;
    if (rows <= 1024) {
        hipLaunchKernelGGL(consensus_finalize_kernel<true>, dim3(1), dim3(1024), 0, st, ws, chunks,
                           B, K, diff_tok, ar_tok, n_match, n_emit, emit_off, emitted, next_anchor);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(argmax_finalize_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0,
                       st, ws, rows, chunks, diff_tok, (int64_t)B * K, ar_tok);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(consensus_finalize_kernel<false>, dim3(1), dim3(1024), 0, st, ws, chunks,
                       B, K, diff_tok, ar_tok, n_match, n_emit, emit_off, emitted, next_anchor);
    return hipGetLastError();
}

}  // namespace orthrus
