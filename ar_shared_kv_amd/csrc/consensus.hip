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

__global__ void __launch_bounds__(256)
argmax_finalize_kernel(const uint64_t *ws, int64_t rows, int chunks, int32_t *idx)
{
    const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (row >= rows) return;
    uint64_t k = 0;
    for (int c = 0; c < chunks; ++c) {
        const uint64_t v = ws[row * chunks + c];
        k = v > k ? v : k;
    }
    idx[row] = (int32_t)argmax_key_index(k);
}

// One work-group: tokens of both views, then per-request consensus and the
// packed emission with an exclusive prefix sum over the batch.
__global__ void __launch_bounds__(1024)
consensus_finalize_kernel(const uint64_t *ws, int B, int K, int chunks, int32_t *diff_tok,
                          int32_t *ar_tok, int32_t *n_match, int32_t *n_emit, int32_t *emit_off,
                          int32_t *emitted, int32_t *next_anchor)
{
    __shared__ int part[1024];
    const int tid = threadIdx.x;
    const int BK = B * K;
    for (int row = tid; row < 2 * BK; row += 1024) {
        uint64_t k = 0;
        for (int c = 0; c < chunks; ++c) {
            const uint64_t v = ws[(int64_t)row * chunks + c];
            k = v > k ? v : k;
        }
        const int32_t tok = (int32_t)argmax_key_index(k);
        if (row < BK) diff_tok[row] = tok;
        else ar_tok[row - BK] = tok;
    }
    __syncthreads();
    // per request: divergence index and emitted count; each thread owns a
    // contiguous run of requests so the prefix sum is two-level
    const int per = (B + 1023) / 1024;
    const int b0 = tid * per;
    const int b1 = (b0 + per < B) ? b0 + per : B;
    int local = 0;
    for (int b = b0; b < b1; ++b) {
        int j = 0;
        while (j < K && diff_tok[b * K + j] == ar_tok[b * K + j]) ++j;
        const int n = (j < K) ? j + 1 : K;
        n_match[b] = j;
        n_emit[b] = n;
        next_anchor[b] = ar_tok[b * K + n - 1];
        local += n;
    }
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
        const int n = n_emit[b];
        emit_off[b] = run;
        for (int i = 0; i < n; ++i) emitted[run + i] = ar_tok[b * K + i];
        run += n;
    }
    if (tid == 1023) emit_off[B] = part[1023];
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
    hipLaunchKernelGGL(argmax_finalize_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0,
                       st, ws, rows, chunks, idx);
    return hipGetLastError();
}

hipError_t launch_consensus_finalize(const uint64_t *ws, int B, int K, int chunks,
                                     int32_t *diff_tok, int32_t *ar_tok, int32_t *n_match,
                                     int32_t *n_emit, int32_t *emit_off, int32_t *emitted,
                                     int32_t *next_anchor, hipStream_t st)
{
    hipLaunchKernelGGL(consensus_finalize_kernel, dim3(1), dim3(1024), 0, st, ws, B, K, chunks,
                       diff_tok, ar_tok, n_match, n_emit, emit_off, emitted, next_anchor);
    return hipGetLastError();
}

}  // namespace orthrus
