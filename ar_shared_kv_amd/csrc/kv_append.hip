// Commit of the accepted positions' KV into the shared cache, gfx950.
//
// Operation (Orthrus summary on gist.science, §2.3 step 3: commit the agreed
// prefix; agents-report core design: the accepted tokens' KV state is
// appended to the shared cache): for every layer, request b and i < n[b],
// the AR view's block row i (all KV heads, K and V) is copied bit-exactly to
// cache row lens[b] + i; lens_out[b] = lens[b] + n[b].
//
// Design: the accepted rows form a compacted list, indexed through the
// exclusive prefix sum of n over the batch (recomputed in LDS by every
// work-group: B is small next to the copy).  Each work-group copies a few
// compacted rows of one layer with 16-byte loads/stores, so the grid work is
// proportional to the accepted rows, not to B*K.
#include "common.hpp"
#include "kernels.hpp"

namespace orthrus {

constexpr int kAppendRowsPerWG = 4;
constexpr int kAppendMaxB = 8192;

__global__ void __launch_bounds__(256) kv_append_kernel(AppendParams p, int chunks_per_layer)
{
    __shared__ int off[kAppendMaxB + 1];
    __shared__ int part[256];
    const int tid = threadIdx.x;
    const int layer = blockIdx.x / chunks_per_layer;
    const int chunk = blockIdx.x % chunks_per_layer;

    // exclusive prefix sum of n over the batch (contiguous runs per thread)
    const int per = (p.B + 255) / 256;
    const int b0 = tid * per;
    const int b1 = (b0 + per < p.B) ? b0 + per : p.B;
    int local = 0;
    for (int b = b0; b < b1; ++b) {
        int n = p.n_emit[b];
        n = n < 0 ? 0 : (n > p.K ? p.K : n);
        off[b] = n;          // temporarily the count
        local += n;
    }
    part[tid] = local;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        const int v = tid >= o ? part[tid - o] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int run = part[tid] - local;
    for (int b = b0; b < b1; ++b) {
        const int n = off[b];
        off[b] = run;
        run += n;
    }
    if (tid == 255) off[p.B] = part[255];
    __syncthreads();
    if (layer == 0 && chunk == 0 && !p.lens_in_place) {
        for (int b = tid; b < p.B; b += 256) p.lens_out[b] = p.lens[b] + (off[b + 1] - off[b]);
    }

    const int total = off[p.B];
    const int gpr = p.D * p.esize / 16;             // 16-byte granules per head row
    const int per_row = 2 * p.Hkv * gpr;            // K and V granules of one block row
    const char *kb = (const char *)p.kb + (int64_t)layer * p.blk_layer_stride * p.esize;
    const char *vb = (const char *)p.vb + (int64_t)layer * p.blk_layer_stride * p.esize;
    char *kc = (char *)p.kc + (int64_t)layer * p.cache_layer_stride * p.esize;
    char *vc = (char *)p.vc + (int64_t)layer * p.cache_layer_stride * p.esize;
    const int64_t row_bytes = (int64_t)p.D * p.esize;

    for (int rr = 0; rr < kAppendRowsPerWG; ++rr) {
        const int cidx = chunk * kAppendRowsPerWG + rr;
        if (cidx >= total) break;
        // request owning compacted row cidx: last b with off[b] <= cidx
        int lo = 0, hi = p.B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (off[mid] <= cidx) lo = mid;
            else hi = mid - 1;
        }
        const int b = lo;
        const int i = cidx - off[b];
        const int64_t t = (int64_t)p.lens[b] + i;
        for (int x = tid; x < per_row; x += 256) {
            const bool isv = x >= p.Hkv * gpr;
            const int y = isv ? x - p.Hkv * gpr : x;
            const int g = y / gpr;
            const int q = y % gpr;
            int64_t dst_row;
            if (p.layout == 0) {
                dst_row = ((int64_t)b * p.Hkv + g) * p.cap + t;
            } else {
                const int page = p.page_table[(int64_t)b * p.maxp + (t >> 4)];
                dst_row = ((int64_t)page * p.Hkv + g) * 16 + (t & 15);
            }
            const int64_t src_row = ((int64_t)b * p.K + i) * p.Hkv + g;
            const u32x4 v = *(const u32x4 *)((isv ? vb : kb) + src_row * row_bytes + q * 16);
            *(u32x4 *)((isv ? vc : kc) + dst_row * row_bytes + q * 16) = v;
        }
    }
}

// Power-of-two scale exponent of a row whose largest magnitude is amax: the
// smallest e >= -120 with 448 * 2^e >= amax (448 is the largest e4m3 value),
// read off amax's bits: amax = 1.f * 2^E needs e = E - 8 when 1.f <= 1.75
// (448 = 1.75 * 2^8) and E - 7 above; 0 for an all-zero row.
__device__ __forceinline__ int e4m3_scale_exp(float amax)
{
    if (amax == 0.f) return 0;
    const uint32_t u = __float_as_uint(amax);
    const int be = (int)(u >> 23);
    const int e = be - 135 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
    return e < -120 ? -120 : e;
}

// Commit into an e4m3 cache: as kv_append_kernel, but every appended (row,
// head) of K and V is quantized on the way: scale s = 2^e from the row's
// largest |value| (e4m3_scale_exp), code = x / s rounded to nearest even
// (exact division; |x / s| <= 448), and s stored beside the row.  Sixteen
// lanes share one (row, head) of D = 128 bf16 values, 8 each.
__global__ void __launch_bounds__(256) kv_append_fp8_kernel(AppendParams p, int chunks_per_layer)
{
    __shared__ int off[kAppendMaxB + 1];
    __shared__ int part[256];
    const int tid = threadIdx.x;
    const int layer = blockIdx.x / chunks_per_layer;
    const int chunk = blockIdx.x % chunks_per_layer;
    const int per = (p.B + 255) / 256;
    const int b0 = tid * per;
    const int b1 = (b0 + per < p.B) ? b0 + per : p.B;
    int local = 0;
    for (int b = b0; b < b1; ++b) {
        int n = p.n_emit[b];
        n = n < 0 ? 0 : (n > p.K ? p.K : n);
        off[b] = n;
        local += n;
    }
    part[tid] = local;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        const int v = tid >= o ? part[tid - o] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int run = part[tid] - local;
    for (int b = b0; b < b1; ++b) {
        const int n = off[b];
        off[b] = run;
        run += n;
    }
    if (tid == 255) off[p.B] = part[255];
    __syncthreads();
    if (layer == 0 && chunk == 0 && !p.lens_in_place) {
        for (int b = tid; b < p.B; b += 256) p.lens_out[b] = p.lens[b] + (off[b + 1] - off[b]);
    }
    const int total = off[p.B];
    const uint16_t *kb = (const uint16_t *)p.kb + (int64_t)layer * p.blk_layer_stride;
    const uint16_t *vb = (const uint16_t *)p.vb + (int64_t)layer * p.blk_layer_stride;
    uint8_t *kc = (uint8_t *)p.kc + (int64_t)layer * p.cache_layer_stride;
    uint8_t *vc = (uint8_t *)p.vc + (int64_t)layer * p.cache_layer_stride;
    float *ks = p.ks + (int64_t)layer * p.scale_layer_stride;
    float *vs = p.vs + (int64_t)layer * p.scale_layer_stride;
    const int sub = tid & 15;                  // 8 of the row's 128 values
    for (int rr = 0; rr < kAppendRowsPerWG; ++rr) {
        const int cidx = chunk * kAppendRowsPerWG + rr;
        if (cidx >= total) break;
        int lo = 0, hi = p.B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (off[mid] <= cidx) lo = mid;
            else hi = mid - 1;
        }
        const int b = lo;
        const int i = cidx - off[b];
        const int64_t t = (int64_t)p.lens[b] + i;
        for (int item = tid >> 4; item < 2 * p.Hkv; item += 16) {
            const bool isv = item >= p.Hkv;
            const int g = isv ? item - p.Hkv : item;
            int64_t dst_row;
            if (p.layout == 0) {
                dst_row = ((int64_t)b * p.Hkv + g) * p.cap + t;
            } else {
                const int page = p.page_table[(int64_t)b * p.maxp + (t >> 4)];
                dst_row = ((int64_t)page * p.Hkv + g) * 16 + (t & 15);
            }
            const int64_t src_row = ((int64_t)b * p.K + i) * p.Hkv + g;
            const u32x4 v = *(const u32x4 *)((isv ? vb : kb) + src_row * 128 + sub * 8);
            float x[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                x[2 * k] = __uint_as_float(v[k] << 16);
                x[2 * k + 1] = __uint_as_float(v[k] & 0xffff0000u);
            }
            float amax = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
#pragma unroll
            for (int m = 8; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 16));
            const int e = e4m3_scale_exp(amax);
            const float inv = __builtin_ldexpf(1.f, -e);
            uint32_t w0 = 0, w1 = 0;
            w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] * inv, x[1] * inv, w0, false);
            w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] * inv, x[3] * inv, w0, true);
            w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[4] * inv, x[5] * inv, w1, false);
            w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[6] * inv, x[7] * inv, w1, true);
            *(u32x2 *)((isv ? vc : kc) + dst_row * 128 + sub * 8) = u32x2{w0, w1};
            if (sub == 0) (isv ? vs : ks)[dst_row] = __builtin_ldexpf(1.f, e);
        }
    }
}

// lens_out = lens + n, one thread per request: the second launch of an
// in-place append (lens_out aliases lens), which must follow every read of
// lens by the copy launch.
__global__ void __launch_bounds__(256) lens_advance_kernel(const int32_t *lens,
                                                           const int32_t *n_emit, int32_t *lens_out,
                                                           int B, int K)
{
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b >= B) return;
    int n = n_emit[b];
    n = n < 0 ? 0 : (n > K ? K : n);
    lens_out[b] = lens[b] + n;
}

hipError_t launch_kv_append(const AppendParams &p, hipStream_t st)
{
    const int chunks = (p.B * p.K + kAppendRowsPerWG - 1) / kAppendRowsPerWG;
    if (p.kv8)
        hipLaunchKernelGGL(kv_append_fp8_kernel, dim3((unsigned)(chunks * p.layers)), dim3(256), 0,
                           st, p, chunks);
    else
        hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)(chunks * p.layers)), dim3(256), 0, st,
                           p, chunks);
    if (!p.lens_in_place) return hipGetLastError();
    // every work-group of the copy reads lens[b] to place its rows, so an
    // update in place waits for the whole copy: stream order does that
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lens_advance_kernel, dim3((unsigned)((p.B + 255) / 256)), dim3(256), 0, st,
                       p.lens, p.n_emit, p.lens_out, p.B, p.K);
    return hipGetLastError();
}

}  // namespace orthrus
