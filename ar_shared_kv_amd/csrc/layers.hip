// The decode step around the Orthrus kernels: the Transformer layers that
// produce the block attention's inputs and consume its output, for one block
// of rows of either view (summary §2.3 steps 1-2: the diffusion head projects
// K candidates in one pass, the frozen AR head verifies them in one pass).
// A Qwen3-style layer: RMSNorm -> QKV projection -> per-head RMSNorm on q and
// k -> rotary position embedding -> block attention -> output projection +
// residual -> RMSNorm -> SwiGLU MLP + residual.  The residual stream is fp32;
// the matrices and the projections' inputs are bf16.
//
// gemm_kernel: y[r][n] = sum_k x[r][k] * w[n][k] for the few rows of a
// decode block (R = B*K) against a weight of N rows: HBM-bound (the weight
// is read once), so the weight streams HBM -> LDS with global_load_lds
// through a ring (4 slots at 32 rows, 3 at 64, 2 at 128), like the LM head.  A work-group covers 128 weight
// rows and RB hidden rows; when the N/128 blocks cannot fill the chip the
// input dimension is split S ways (S depends on N and the input size only)
// and a second launch adds the fp32 partial sums in split order.  Every
// output element thus goes through the same operations whatever R is: a row
// computed in a block of 32 equals the same row computed alone.
//
// Weights are stored packed (pack_weight_kernel): 128 rows x 64 columns per
// 16 KiB tile, the tiles of one 128-row block in column order, block after
// block, rows past N zero.  A work-group's weight is then one contiguous run
// read front to back.  Row-major rows are 2*Kin bytes apart, so every
// work-group reading the same column chunk at once kept hitting the same HBM
// channels: the Qwen3-8B gate/up projection (N = 24,576, Kin = 4,096) took
// 48 us row-major and 39 us packed.
#include "common.hpp"
#include "kernels.hpp"
#include "wtile.hpp"

#include "../../include/orthrus.h"

namespace orthrus {
namespace {

constexpr int kGemmNB = kWTileRows;           // weight rows per work-group
constexpr int kGemmHC = kWTileCols;           // input columns per chunk (one packed tile)
// Split-K aims at about one work-group per CU: at the Qwen3-8B layer (R = 32)
// the four projections took 114 us with 512 (S = 8, 16, 2, 16), 102 with 256
// (S = 4, 8, 1, 8), 109 with 192 and 108 with 384 -- fewer partial sums and
// longer runs per work-group win until the chip is no longer filled.
constexpr int kGemmTargetWG = 256;

__device__ __forceinline__ void g_dma16(const void* gptr, uint32_t lds_addr) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "s"(m0)
                 : "memory", "m0");
}

// silu(g) * u with silu(g) = g / (1 + e^-g): the one SwiGLU expression of
// every kernel below that applies it.
__device__ __forceinline__ float swiglu1(float g, float u) { return g / (1.f + expf(-g)) * u; }

// out_mode: 0 fp32 partial (split s of S) to part[s][R][N]; 1 fp32 y (+ res);
// 2 bf16 y (+ res); 3 SwiGLU of a paired gate/up weight (S = 1): every 8
// weight rows are 4 gate rows then the 4 matching up rows (pack_weight_kernel
// with pair_I), y = act bf16 [R][N / 2]
template <int NSTAGE, int RB>
__global__ void __launch_bounds__(256, 2)
gemm_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int R, int N, int Kin,
            int cps, int out_mode, float* __restrict__ part, void* __restrict__ y,
            const float* __restrict__ res)
{
    constexpr int HC = kGemmHC;
    constexpr int WB = kGemmNB * HC * 2;
    constexpr int XB = RB * HC * 2;
    constexpr int NB = RB / 32;
    constexpr int SLOT = WB + XB;
    constexpr int GR = HC / 8;
    constexpr int RPP = 1024 / (HC * 2);
    constexpr int LOADS = SLOT / 4096;
    constexpr int NPRE = NSTAGE - 1;
    static_assert(SLOT % 4096 == 0 && LOADS * NSTAGE <= 63, "ring");
    __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * SLOT];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int n0 = blockIdx.x * kGemmNB;
    const int r0 = blockIdx.y * RB;
    const int sp = blockIdx.z;
    const int c_lo = sp * cps;
    const uint32_t lds_base = (uint32_t)(uintptr_t)(ORTHRUS_LDS void*)&smem[0];

    auto issue = [&](int c) __attribute__((always_inline)) {
        const uint32_t slot = lds_base + (uint32_t)((c % NSTAGE) * SLOT);
        const int col = (c_lo + c) * HC;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int k = i * 4 + wave;
            const bool isx = k >= WB / 1024;
            const int row = (isx ? k - WB / 1024 : k) * RPP + lane / GR;
            const int gsrc = (lane % GR) ^ (row % GR);
            const uint16_t* src;
            if (isx) {
                const int rr = r0 + row < R ? r0 + row : R - 1;
                src = x + (int64_t)rr * Kin + col + gsrc * 8;
            } else {
                // tile (block, chunk) of the packed weight; its rows past N are zero
                src = w + ((int64_t)blockIdx.x * (Kin / HC) + (c_lo + c)) * (kGemmNB * HC) +
                      row * HC + gsrc * 8;
            }
            g_dma16(src, slot + (uint32_t)(k * 1024));
        }
    };
    auto wait_chunk = [&](int c) __attribute__((always_inline)) {
        const int later = cps - 1 - c;
        const int pend = later < NPRE - 1 ? later : NPRE - 1;
        switch (pend) {
            case 0: __builtin_amdgcn_s_waitcnt(vmcnt_encode(0)); break;
            case 1: __builtin_amdgcn_s_waitcnt(vmcnt_encode(LOADS)); break;
            default: __builtin_amdgcn_s_waitcnt(vmcnt_encode(2 * LOADS)); break;
        }
    };
    static_assert(NPRE - 1 <= 2, "wait_chunk covers up to 2 later chunks");

    f32x16 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j] = f32x16{};
    const int wrow = wave * 32 + (lane & 31);
    for (int c = 0; c < NPRE && c < cps; ++c) issue(c);
    for (int c = 0; c < cps; ++c) {
        wait_chunk(c);
        __syncthreads();
        if (c + NPRE < cps) issue(c + NPRE);
        const char* Ws = smem + (c % NSTAGE) * SLOT;
        const char* Xs = Ws + WB;
        u32x4 af[HC / 16], bfr[NB][HC / 16];
#pragma unroll
        for (int ds = 0; ds < HC / 16; ++ds) {
            const int g = 2 * ds + half;
            af[ds] = *(const u32x4*)(Ws + wrow * (HC * 2) + ((g ^ (wrow % GR)) * 16));
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int xrow = 32 * j + (lane & 31);
                bfr[j][ds] = *(const u32x4*)(Xs + xrow * (HC * 2) + ((g ^ (xrow % GR)) * 16));
            }
        }
#pragma unroll
        for (int ds = 0; ds < HC / 16; ++ds)
#pragma unroll
            for (int j = 0; j < NB; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, af[ds]), __builtin_bit_cast(bf16x8, bfr[j][ds]),
                    acc[j], 0, 0, 0);
    }
    // acc[j][i]: weight row n0 + 32*wave + 8*(i/4) + 4*half + i%4, hidden row
    // r0 + 32*j + lane%32; four consecutive outputs per store
    if (out_mode == 3) {
        // the block's RB x 128 fp32 results through LDS (the ring is free once
        // every wave is past its last chunk), then one thread per (hidden row,
        // 4 outputs): gate at paired columns 8g..8g+3, up at 8g+4..8g+7
        __syncthreads();
        float* buf = reinterpret_cast<float*>(smem);
        static_assert(RB * kGemmNB * 4 <= NSTAGE * SLOT, "epilogue buffer fits in the ring");
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *(f32x4*)(buf + (32 * j + (lane & 31)) * kGemmNB + wave * 32 + 8 * q4 + 4 * half) =
                    f32x4{acc[j][4 * q4], acc[j][4 * q4 + 1], acc[j][4 * q4 + 2], acc[j][4 * q4 + 3]};
        __syncthreads();
        const int I = N / 2;
        for (int it = tid; it < RB * (kGemmNB / 8); it += 256) {
            const int rr = it / (kGemmNB / 8), g = it % (kGemmNB / 8);
            const int r = r0 + rr, i = blockIdx.x * (kGemmNB / 2) + 4 * g;
            if (r >= R || i >= I) continue;
            const f32x4 gv = *(const f32x4*)(buf + rr * kGemmNB + 8 * g);
            const f32x4 uv = *(const f32x4*)(buf + rr * kGemmNB + 8 * g + 4);
            *(u32x2*)((uint16_t*)y + (int64_t)r * I + i) =
                u32x2{pack_bf16x2(swiglu1(gv[0], uv[0]), swiglu1(gv[1], uv[1])),
                      pack_bf16x2(swiglu1(gv[2], uv[2]), swiglu1(gv[3], uv[3]))};
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int r = r0 + 32 * j + (lane & 31);
        if (r >= R) continue;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int n = n0 + wave * 32 + 8 * q4 + 4 * half;
            if (n >= N) continue;
            f32x4 v = {acc[j][4 * q4], acc[j][4 * q4 + 1], acc[j][4 * q4 + 2], acc[j][4 * q4 + 3]};
            const int64_t o = (int64_t)r * N + n;
            if (out_mode == 0) {
                *(f32x4*)(part + (int64_t)sp * R * N + o) = v;
            } else {
                if (res) v += *(const f32x4*)(res + o);
                if (out_mode == 1) *(f32x4*)((float*)y + o) = v;
                else *(u32x2*)((uint16_t*)y + o) = u32x2{pack_bf16x2(v[0], v[1]),
                                                          pack_bf16x2(v[2], v[3])};
            }
        }
    }
}

// The partial sums of the split input dimension are always added in split
// order, v = ((p0 + p1) + p2) + ..., and a residual last (res + v), by every
// kernel below that reads them: a fused epilogue gives the same bits as the
// plain reduction followed by the separate kernel.
__device__ __forceinline__ f32x4 sum_splits(const float* __restrict__ part, int S, int64_t stride,
                                            int64_t i)
{
    f32x4 v = *(const f32x4*)(part + i);
#pragma unroll 8
    for (int s = 1; s < S; ++s) v += *(const f32x4*)(part + (int64_t)s * stride + i);
    return v;
}

// y = (res +) sum of the S partials; fp32 or bf16.
__global__ void __launch_bounds__(256)
gemm_reduce_kernel(const float* __restrict__ part, int S, int64_t RN4, int out_bf16,
                   void* __restrict__ y, const float* __restrict__ res)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= RN4) return;
    f32x4 v = sum_splits(part, S, RN4 * 4, i * 4);
    if (res) v = ((const f32x4*)res)[i] + v;
    if (out_bf16) ((u32x2*)y)[i] = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    else ((f32x4*)y)[i] = v;
}

int gemm_splits(int N, int Kin)
{
    const int nblk = (N + kGemmNB - 1) / kGemmNB;
    const int chunks = Kin / kGemmHC;
    int S = 1;
    while ((int64_t)nblk * S * 2 <= kGemmTargetWG && chunks % (S * 2) == 0 && chunks / (S * 2) >= 4)
        S *= 2;
    return S;
}

// ---------------------------------------------------------------- RMSNorm
// y[r] = x[r] / sqrt(mean(x[r]^2) + eps) * w.  One work-group of 1024
// threads per row; thread t holds the float4 groups t, t + 1024, ... (NG of
// them) in registers.  The sum of squares has one fixed order: each thread
// over its groups and their four values in turn, then the 64 lanes of a wave
// (xor butterfly: every lane ends with the same bits), then the 16 waves in
// index order.  So a row's result depends neither on R nor on which kernel
// (the plain norm or a projection's fused epilogue) formed its input.
constexpr int kNormThreads = 1024;
constexpr int kNormMaxGroups = 4;             // H <= 4 * 4 * 1024

template <int NG>
__device__ __forceinline__ void rmsnorm_row(const f32x4 (&v)[NG], int H, const uint16_t* __restrict__ w,
                                            uint16_t* __restrict__ yr, float eps)
{
    __shared__ float red[kNormThreads / 64];
    const int tid = threadIdx.x;
    const int H4 = H / 4;
    float ss = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        if (tid + g * kNormThreads < H4) {
            ss += v[g][0] * v[g][0];
            ss += v[g][1] * v[g][1];
            ss += v[g][2] * v[g][2];
            ss += v[g][3] * v[g][3];
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    float tot = red[0];
#pragma unroll
    for (int i = 1; i < kNormThreads / 64; ++i) tot += red[i];
    const float inv = 1.f / sqrtf(tot / (float)H + eps);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int j = tid + g * kNormThreads;
        if (j < H4) {
            const u32x2 wb = *(const u32x2*)(w + 4 * j);
            const float y0 = v[g][0] * inv * bf16_bits_to_f32((uint16_t)(wb[0] & 0xffffu));
            const float y1 = v[g][1] * inv * bf16_bits_to_f32((uint16_t)(wb[0] >> 16));
            const float y2 = v[g][2] * inv * bf16_bits_to_f32((uint16_t)(wb[1] & 0xffffu));
            const float y3 = v[g][3] * inv * bf16_bits_to_f32((uint16_t)(wb[1] >> 16));
            *(u32x2*)(yr + 4 * j) = u32x2{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
        }
    }
}

template <int NG>
__global__ void __launch_bounds__(kNormThreads)
rmsnorm_kernel(const float* __restrict__ x, const uint16_t* __restrict__ w, uint16_t* __restrict__ y,
               int H, float eps)
{
    const int64_t row = blockIdx.x;
    const float* xr = x + row * H;
    f32x4 v[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int j = threadIdx.x + g * kNormThreads;
        v[g] = j < H / 4 ? *(const f32x4*)(xr + 4 * j) : f32x4{};
    }
    rmsnorm_row<NG>(v, H, w, y + row * H, eps);
}

// The output (or down) projection's epilogue: h = res + sum of the partials
// (stored, fp32), then the RMSNorm of h into y.  Bit for bit the plain
// reduction followed by rmsnorm_kernel.
template <int NG>
__global__ void __launch_bounds__(kNormThreads)
reduce_rmsnorm_kernel(const float* __restrict__ part, int S, int64_t RN, const float* res,
                      float* h, const uint16_t* __restrict__ w, uint16_t* __restrict__ y, int H,
                      float eps)
{
    const int64_t row = blockIdx.x;
    f32x4 v[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int j = threadIdx.x + g * kNormThreads;
        if (j < H / 4) {
            const int64_t i = row * H + 4 * j;
            v[g] = sum_splits(part, S, RN, i);
            if (res) v[g] = *(const f32x4*)(res + i) + v[g];
            *(f32x4*)(h + i) = v[g];
        } else {
            v[g] = f32x4{};
        }
    }
    rmsnorm_row<NG>(v, H, w, y + row * H, eps);
}

// ------------------------------------------------------ QK norm + rotary
// From the fp32 QKV projection [R][(Hq + 2 Hkv) * D] of the block rows (row
// r is row r % K of request r / K, at position lens[r / K] + r % K): q and k
// heads get RMSNorm over D (weights wq / wk), then the rotary
// embedding with pairs (d, d + D/2) rotated by pos * theta^(-2d/D); v heads
// are copied.  One wave per (row, head), D = 128 (lane l holds d = l and
// l + 64).  Angles in fp64.
__device__ __forceinline__ void qk_norm_rope_item(float x0, float x1, int r, int h, int lane,
                                                  const uint16_t* __restrict__ wq,
                                                  const uint16_t* __restrict__ wk,
                                                  const int32_t* __restrict__ lens, int K,
                                                  uint16_t* __restrict__ q,
                                                  uint16_t* __restrict__ k,
                                                  uint16_t* __restrict__ v, int Hq, int Hkv,
                                                  float eps, double log_theta)
{
    constexpr int D = 128;
    if (h >= Hq + Hkv) {                              // v: a copy
        uint16_t* dst = v + ((int64_t)r * Hkv + (h - Hq - Hkv)) * D;
        dst[lane] = (uint16_t)(pack_bf16x2(x0, 0.f) & 0xffffu);
        dst[lane + 64] = (uint16_t)(pack_bf16x2(x1, 0.f) & 0xffffu);
        return;
    }
    float ss = x0 * x0 + x1 * x1;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float inv = 1.f / sqrtf(ss / (float)D + eps);
    const uint16_t* wn = h < Hq ? wq : wk;
    const float n0 = x0 * inv * bf16_bits_to_f32(wn[lane]);
    const float n1 = x1 * inv * bf16_bits_to_f32(wn[lane + 64]);
    const double freq = exp(-(2.0 * lane / D) * log_theta);
    double sn, cs;
    const int pos = lens[r / K] + r % K;
    sincos((double)pos * freq, &sn, &cs);
    const float c = (float)cs, s = (float)sn;
    const float o0 = n0 * c - n1 * s;
    const float o1 = n1 * c + n0 * s;
    uint16_t* dst = h < Hq ? q + ((int64_t)r * Hq + h) * D : k + ((int64_t)r * Hkv + (h - Hq)) * D;
    dst[lane] = (uint16_t)(pack_bf16x2(o0, 0.f) & 0xffffu);
    dst[lane + 64] = (uint16_t)(pack_bf16x2(o1, 0.f) & 0xffffu);
}

// qkv holds S >= 1 partial sums [S][R][heads*D] of the projection (S = 1:
// the projection itself), added in split order first.
__global__ void __launch_bounds__(256)
qk_norm_rope_kernel(const float* __restrict__ qkv, int S, const uint16_t* __restrict__ wq,
                    const uint16_t* __restrict__ wk, const int32_t* __restrict__ lens, int K,
                    uint16_t* __restrict__ q, uint16_t* __restrict__ k, uint16_t* __restrict__ v,
                    int R, int Hq, int Hkv, float eps, double log_theta)
{
    constexpr int D = 128;
    const int heads = Hq + 2 * Hkv;
    const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= R * heads) return;
    const int lane = threadIdx.x & 63;
    const int r = item / heads;
    const int h = item % heads;
    const int64_t i = (int64_t)r * heads * D + (int64_t)h * D + lane;
    float x0 = qkv[i], x1 = qkv[i + 64];
    const int64_t stride = (int64_t)R * heads * D;
#pragma unroll 8
    for (int s = 1; s < S; ++s) {
        x0 += qkv[s * stride + i];
        x1 += qkv[s * stride + i + 64];
    }
    qk_norm_rope_item(x0, x1, r, h, lane, wq, wk, lens, K, q, k, v, Hq, Hkv, eps, log_theta);
}

// ---------------------------------------------------------------- SwiGLU
// act[r][i] = silu(g) * u, g = gu[r][i], u = gu[r][I + i], silu(g) =
// g / (1 + e^-g); gu holds S >= 1 partial sums [S][R][2I] of the gate/up
// projection (S = 1: the projection itself), added in split order first.
// paired: the columns come from a paired weight (4 gate columns, then their 4
// up columns), so g = gu[r][8(i/4) + i%4] and u = gu[r][8(i/4) + 4 + i%4].
// One thread per four consecutive i (I a multiple of 4).
__global__ void __launch_bounds__(256)
swiglu_kernel(const float* __restrict__ gu, int S, uint16_t* __restrict__ act, int R, int I,
              int paired)
{
    const int I4 = I / 4;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (int64_t)R * I4) return;
    const int64_t r = t / I4;
    const int i = (int)(t % I4) * 4;
    const int64_t stride = (int64_t)R * 2 * I;
    const int64_t go = r * 2 * I + (paired ? 2 * i : i);
    const int64_t uo = paired ? go + 4 : go + I;
    const f32x4 g = sum_splits(gu, S, stride, go);
    const f32x4 u = sum_splits(gu, S, stride, uo);
    *(u32x2*)(act + r * I + i) = u32x2{pack_bf16x2(swiglu1(g[0], u[0]), swiglu1(g[1], u[1])),
                                       pack_bf16x2(swiglu1(g[2], u[2]), swiglu1(g[3], u[3]))};
}

// ----------------------------------------------------- block input tokens
// out[b][0] = anchor[b]; out[b][i] = cand[b][i-1] (the AR view's block: the
// anchor then the first K-1 candidates) or, with no cand, the fill token
// (the diffusion view's block: the anchor then <mask> tokens).
__global__ void __launch_bounds__(256)
block_tokens_kernel(const int32_t* __restrict__ anchor, const int32_t* __restrict__ cand,
                    int32_t fill, int32_t* __restrict__ out, int B, int K)
{
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= B * K) return;
    const int b = t / K, i = t % K;
    out[t] = i == 0 ? anchor[b] : (cand ? cand[b * K + i - 1] : fill);
}

// ------------------------------------------------------------- embedding
__global__ void __launch_bounds__(256)
embed_kernel(const int32_t* __restrict__ tok, const uint16_t* __restrict__ table,
             float* __restrict__ h, int H)
{
    const uint16_t* row = table + (int64_t)tok[blockIdx.x] * H;
    float* out = h + (int64_t)blockIdx.x * H;
    for (int i = threadIdx.x; i < H; i += 256) out[i] = bf16_bits_to_f32(row[i]);
}

// ---------------------------------------------------------- weight packing
// One thread per 16 bytes of the packed weight (8 columns of one row of one
// tile): a coalesced write, a 16-byte read of the row-major weight, zeros for
// the rows past N that fill the last block.  pair_I > 0: the weight is a
// gate/up pair [2I][Kin] (gate rows, then up rows) and packed row n holds, in
// every group of 8, gate rows 4(n/8)..+3 and then the matching up rows.
__global__ void __launch_bounds__(256)
pack_weight_kernel(const uint16_t* __restrict__ w, int N, int Kin, int64_t pieces,
                   int pair_I, uint16_t* __restrict__ out)
{
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (p >= pieces) return;
    constexpr int PPT = kWTileRows * kWTileCols / 8;          // 16-byte pieces per tile
    const int64_t tile = p / PPT;
    const int q = (int)(p % PPT);
    const int cpb = Kin / kWTileCols;                          // tiles per 128-row block
    const int64_t n = (tile / cpb) * kWTileRows + q / (kWTileCols / 8);
    const int64_t k = (tile % cpb) * kWTileCols + (q % (kWTileCols / 8)) * 8;
    const int64_t src = pair_I > 0 ? (n % 8 < 4 ? 4 * (n / 8) + n % 8 : pair_I + 4 * (n / 8) + n % 8 - 4)
                                   : n;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (n < N) v = *(const u32x4*)(w + src * Kin + k);
    *(u32x4*)(out + p * 8) = v;
}

}  // namespace
}  // namespace orthrus

using namespace orthrus;

extern "C" {

size_t orthrus_packed_weight_bytes(int N, int Kin)
{
    if (N < 1 || Kin < kWTileCols || Kin % kWTileCols) return 0;
    const int64_t blocks = ((int64_t)N + kWTileRows - 1) / kWTileRows;
    return (size_t)blocks * kWTileRows * (size_t)Kin * sizeof(uint16_t);
}

namespace {

int pack(const void *w, int N, int Kin, int pair_I, void *packed, size_t packed_bytes,
         hipStream_t stream)
{
    if (!w || !packed) return ORTHRUS_ERR_NULL;
    if (N < 1 || Kin < 1) return ORTHRUS_ERR_SHAPE;
    const size_t need = orthrus_packed_weight_bytes(N, Kin);
    if (!need) return ORTHRUS_ERR_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(w) & 15u) || (reinterpret_cast<uintptr_t>(packed) & 15u))
        return ORTHRUS_ERR_UNSUPPORTED;
    if (packed_bytes < need) return ORTHRUS_ERR_WORKSPACE;
    const int64_t pieces = (int64_t)(need / 16);
    hipLaunchKernelGGL(pack_weight_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0,
                       stream, static_cast<const uint16_t *>(w), N, Kin, pieces, pair_I,
                       static_cast<uint16_t *>(packed));
    return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

}  // namespace

int orthrus_pack_weight(const void *w, int N, int Kin, void *packed, size_t packed_bytes,
                        hipStream_t stream)
{
    return pack(w, N, Kin, 0, packed, packed_bytes, stream);
}

int orthrus_pack_weight_gate_up(const void *w, int I, int Kin, void *packed,
                                size_t packed_bytes, hipStream_t stream)
{
    if (!w || !packed) return ORTHRUS_ERR_NULL;
    if (I < 1 || I > INT32_MAX / 2) return ORTHRUS_ERR_SHAPE;      // 2I rows must fit an int
    if (I % 4) return ORTHRUS_ERR_UNSUPPORTED;
    return pack(w, 2 * I, Kin, I, packed, packed_bytes, stream);
}

namespace {

bool mis16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }
bool mis8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) != 0; }

// Shape checks shared by the projections.
int gemm_check(const void* x, const void* w, int R, int N, int Kin)
{
    if (!x || !w) return ORTHRUS_ERR_NULL;
    if (R < 1 || N < 1 || Kin < 1) return ORTHRUS_ERR_SHAPE;
    if (Kin % kGemmHC || N % 4 || R > 65535 * 128) return ORTHRUS_ERR_UNSUPPORTED;
    if (mis16(x) || mis16(w)) return ORTHRUS_ERR_UNSUPPORTED;
    return ORTHRUS_OK;
}

// The projection's main launch: out_mode 0 writes the S partial sums to
// part, 1 / 2 write y (fp32 / bf16, + res) directly (S = 1 only).
int gemm_main(const void* x, const void* w, int R, int N, int Kin, int S, int mode, float* part,
              void* y, const float* res, hipStream_t stream)
{
    const int cps = Kin / kGemmHC / S;
    const uint16_t *xp = static_cast<const uint16_t*>(x), *wp = static_cast<const uint16_t*>(w);
    const unsigned gx = (unsigned)((N + kGemmNB - 1) / kGemmNB);
    if (R <= 32)   // three chunks in flight: the Qwen3-8B layer's projections 94.4 against
                   // 96.3 us with two (a work-group streams only 8 to 64 chunks), 97.1 with five
        hipLaunchKernelGGL((gemm_kernel<4, 32>), dim3(gx, 1, S), dim3(256), 0, stream, xp, wp, R,
                           N, Kin, cps, mode, part, y, res);
    else if (R <= 64)
        hipLaunchKernelGGL((gemm_kernel<3, 64>), dim3(gx, 1, S), dim3(256), 0, stream, xp, wp, R,
                           N, Kin, cps, mode, part, y, res);
    else
        hipLaunchKernelGGL((gemm_kernel<2, 128>), dim3(gx, (unsigned)((R + 127) / 128), S),
                           dim3(256), 0, stream, xp, wp, R, N, Kin, cps, mode, part, y, res);
    return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

// The partial sums of a fused projection: always written, even with S = 1.
size_t partial_bytes(int R, int N, int Kin)
{
    return (size_t)gemm_splits(N, Kin) * (size_t)R * (size_t)N * sizeof(float);
}

int partial_check(void* ws, size_t ws_bytes, int R, int N, int Kin)
{
    if (!ws || ws_bytes < partial_bytes(R, N, Kin) || mis16(ws)) return ORTHRUS_ERR_WORKSPACE;
    return ORTHRUS_OK;
}

int norm_groups(int H) { return (H / 4 + kNormThreads - 1) / kNormThreads; }

int launch_norm(const float* part, int S, int64_t RN, const float* res, float* h,
                const uint16_t* w, uint16_t* y, int R, int H, float eps, hipStream_t stream)
{
    const int ng = norm_groups(H);
    const dim3 grid((unsigned)R), block(kNormThreads);
#define ORTHRUS_NORM(NG)                                                                        \
    if (part)                                                                                   \
        hipLaunchKernelGGL((reduce_rmsnorm_kernel<NG>), grid, block, 0, stream, part, S, RN,   \
                           res, h, w, y, H, eps);                                               \
    else                                                                                        \
        hipLaunchKernelGGL((rmsnorm_kernel<NG>), grid, block, 0, stream, h, w, y, H, eps);
    if (ng <= 1) { ORTHRUS_NORM(1) }
    else if (ng <= 2) { ORTHRUS_NORM(2) }
    else { ORTHRUS_NORM(4) }
#undef ORTHRUS_NORM
    return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

int norm_check(int H, float eps)
{
    if (H < 4 || !(eps > 0.f)) return ORTHRUS_ERR_SHAPE;
    if (H % 4 || H / 4 > kNormMaxGroups * kNormThreads) return ORTHRUS_ERR_UNSUPPORTED;
    return ORTHRUS_OK;
}

}  // namespace

size_t orthrus_gemm_workspace_bytes(int R, int N, int Kin)
{
    if (R < 1 || N < 1 || Kin < kGemmHC || Kin % kGemmHC || N % 4) return 0;
    const int S = gemm_splits(N, Kin);
    return S > 1 ? (size_t)S * R * N * sizeof(float) : 0;
}

size_t orthrus_gemm_epilogue_workspace_bytes(int R, int N, int Kin)
{
    if (R < 1 || N < 1 || Kin < kGemmHC || Kin % kGemmHC || N % 4) return 0;
    return partial_bytes(R, N, Kin);
}

int orthrus_gemm(const void *x, const void *w, const float *residual, void *y, int R, int N,
                 int Kin, int out_dtype, void *workspace, size_t workspace_bytes,
                 hipStream_t stream)
{
    if (!y) return ORTHRUS_ERR_NULL;
    int st = gemm_check(x, w, R, N, Kin);
    if (st != ORTHRUS_OK) return st;
    if (out_dtype != ORTHRUS_F32 && out_dtype != ORTHRUS_BF16) return ORTHRUS_ERR_DTYPE;
    if (mis16(y) || mis16(residual)) return ORTHRUS_ERR_UNSUPPORTED;
    const int S = gemm_splits(N, Kin);
    const size_t need = S > 1 ? (size_t)S * R * N * sizeof(float) : 0;
    if (need && (!workspace || workspace_bytes < need || mis16(workspace)))
        return ORTHRUS_ERR_WORKSPACE;
    const int mode = S > 1 ? 0 : (out_dtype == ORTHRUS_F32 ? 1 : 2);
    float *part = static_cast<float *>(workspace);
    st = gemm_main(x, w, R, N, Kin, S, mode, part, y, residual, stream);
    if (st != ORTHRUS_OK || S == 1) return st;
    const int64_t rn4 = (int64_t)R * N / 4;
    hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)((rn4 + 255) / 256)), dim3(256), 0,
                       stream, part, S, rn4, out_dtype == ORTHRUS_BF16 ? 1 : 0, y, residual);
    return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

int orthrus_rmsnorm(const float *x, const void *weight, void *y, int R, int H, float eps,
                    hipStream_t stream)
{
    if (!x || !weight || !y) return ORTHRUS_ERR_NULL;
    if (R < 1) return ORTHRUS_ERR_SHAPE;
    const int st = norm_check(H, eps);
    if (st != ORTHRUS_OK) return st;
    if (mis16(x) || mis8(weight) || mis8(y)) return ORTHRUS_ERR_UNSUPPORTED;
    return launch_norm(nullptr, 0, 0, nullptr, const_cast<float *>(x),
                       static_cast<const uint16_t *>(weight), static_cast<uint16_t *>(y), R, H,
                       eps, stream);
}

int orthrus_gemm_rmsnorm(const void *x, const void *w, float *h, const void *norm_weight,
                         void *xn, int R, int H, int Kin, float eps, void *workspace,
                         size_t workspace_bytes, hipStream_t stream)
{
    if (!h || !norm_weight || !xn) return ORTHRUS_ERR_NULL;
    int st = gemm_check(x, w, R, H, Kin);
    if (st != ORTHRUS_OK) return st;
    if ((st = norm_check(H, eps)) != ORTHRUS_OK) return st;
    if (mis16(h) || mis8(norm_weight) || mis8(xn)) return ORTHRUS_ERR_UNSUPPORTED;
    if ((st = partial_check(workspace, workspace_bytes, R, H, Kin)) != ORTHRUS_OK) return st;
    const int S = gemm_splits(H, Kin);
    float *part = static_cast<float *>(workspace);
    if ((st = gemm_main(x, w, R, H, Kin, S, 0, part, nullptr, nullptr, stream)) != ORTHRUS_OK)
        return st;
    return launch_norm(part, S, (int64_t)R * H, h, h, static_cast<const uint16_t *>(norm_weight),
                       static_cast<uint16_t *>(xn), R, H, eps, stream);
}

namespace {

int qk_check(const void *q_norm, const void *k_norm, const int32_t *lens, int K, const void *q,
             const void *k, const void *v, int R, int Hq, int Hkv, int D, float eps,
             float rope_theta)
{
    if (!q_norm || !k_norm || !lens || !q || !k || !v) return ORTHRUS_ERR_NULL;
    if (R < 1 || K < 1 || R % K || Hq < 1 || Hkv < 1 || !(eps > 0.f) || !(rope_theta > 1.f))
        return ORTHRUS_ERR_SHAPE;
    if (D != 128 || Hq > 65536 || Hkv > 65536) return ORTHRUS_ERR_UNSUPPORTED;
    return ORTHRUS_OK;
}

int launch_qk(const float *qkv, int S, const void *q_norm, const void *k_norm,
              const int32_t *lens, int K, void *q, void *k, void *v, int R, int Hq, int Hkv,
              float eps, float rope_theta, hipStream_t stream)
{
    const int64_t items = (int64_t)R * (Hq + 2 * Hkv);
    hipLaunchKernelGGL(qk_norm_rope_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, stream,
                       qkv, S, static_cast<const uint16_t *>(q_norm),
                       static_cast<const uint16_t *>(k_norm), lens, K,
                       static_cast<uint16_t *>(q), static_cast<uint16_t *>(k),
                       static_cast<uint16_t *>(v), R, Hq, Hkv, eps, std::log((double)rope_theta));
    return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

int launch_swiglu(const float *gu, int S, void *act, int R, int I, int paired,
                  hipStream_t stream)
{
    const int64_t total = (int64_t)R * (I / 4);
    hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       gu, S, static_cast<uint16_t *>(act), R, I, paired);
    return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

}  // namespace

int orthrus_qk_norm_rope(const float *qkv, const void *q_norm, const void *k_norm,
                         const int32_t *lens, int K, void *q, void *k, void *v, int R, int Hq,
                         int Hkv, int D, float eps, float rope_theta, hipStream_t stream)
{
    if (!qkv) return ORTHRUS_ERR_NULL;
    const int st = qk_check(q_norm, k_norm, lens, K, q, k, v, R, Hq, Hkv, D, eps, rope_theta);
    if (st != ORTHRUS_OK) return st;
    return launch_qk(qkv, 1, q_norm, k_norm, lens, K, q, k, v, R, Hq, Hkv, eps, rope_theta,
                     stream);
}

int orthrus_gemm_qk_norm_rope(const void *x, const void *w_qkv, const void *q_norm,
                              const void *k_norm, const int32_t *lens, int K, void *q, void *k,
                              void *v, int R, int Hq, int Hkv, int D, int Kin, float eps,
                              float rope_theta, void *workspace, size_t workspace_bytes,
                              hipStream_t stream)
{
    int st = qk_check(q_norm, k_norm, lens, K, q, k, v, R, Hq, Hkv, D, eps, rope_theta);
    if (st != ORTHRUS_OK) return st;
    const int N = (Hq + 2 * Hkv) * D;
    if ((st = gemm_check(x, w_qkv, R, N, Kin)) != ORTHRUS_OK) return st;
    if ((st = partial_check(workspace, workspace_bytes, R, N, Kin)) != ORTHRUS_OK) return st;
    const int S = gemm_splits(N, Kin);
    float *part = static_cast<float *>(workspace);
    if ((st = gemm_main(x, w_qkv, R, N, Kin, S, 0, part, nullptr, nullptr, stream)) != ORTHRUS_OK)
        return st;
    return launch_qk(part, S, q_norm, k_norm, lens, K, q, k, v, R, Hq, Hkv, eps, rope_theta,
                     stream);
}

int orthrus_swiglu(const float *gate_up, void *act, int R, int I, hipStream_t stream)
{
    if (!gate_up || !act) return ORTHRUS_ERR_NULL;
    if (R < 1 || I < 1 || I > INT32_MAX / 2) return ORTHRUS_ERR_SHAPE;
    if (I % 4 || mis16(gate_up) || mis8(act)) return ORTHRUS_ERR_UNSUPPORTED;
    if ((int64_t)R * (I / 4) > (int64_t)INT32_MAX * 256) return ORTHRUS_ERR_UNSUPPORTED;
    return launch_swiglu(gate_up, 1, act, R, I, 0, stream);
}

int orthrus_gemm_swiglu(const void *x, const void *w_gate_up, void *act, int R, int I, int Kin,
                        void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!act) return ORTHRUS_ERR_NULL;
    if (I < 1 || I > INT32_MAX / 2) return ORTHRUS_ERR_SHAPE;     // 2I rows must fit an int
    int st = gemm_check(x, w_gate_up, R, 2 * I, Kin);
    if (st != ORTHRUS_OK) return st;
    if (I % 4 || mis8(act)) return ORTHRUS_ERR_UNSUPPORTED;
    if ((st = partial_check(workspace, workspace_bytes, R, 2 * I, Kin)) != ORTHRUS_OK) return st;
    const int S = gemm_splits(2 * I, Kin);
    float *part = static_cast<float *>(workspace);
    // not split: SwiGLU in the projection's own epilogue, no partial sums
    if (S == 1) return gemm_main(x, w_gate_up, R, 2 * I, Kin, 1, 3, nullptr, act, nullptr, stream);
    if ((st = gemm_main(x, w_gate_up, R, 2 * I, Kin, S, 0, part, nullptr, nullptr, stream)) !=
        ORTHRUS_OK)
        return st;
    return launch_swiglu(part, S, act, R, I, 1, stream);
}

int orthrus_block_tokens(const int32_t *anchor, const int32_t *cand, int32_t fill,
                         int32_t *out, int B, int K, hipStream_t stream)
{
    if (!anchor || !out) return ORTHRUS_ERR_NULL;
    if (B < 1 || K < 1) return ORTHRUS_ERR_SHAPE;
    hipLaunchKernelGGL(block_tokens_kernel, dim3((unsigned)((B * K + 255) / 256)), dim3(256), 0,
                       stream, anchor, cand, fill, out, B, K);
    return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

int orthrus_embed(const int32_t *tokens, const void *table, float *h, int R, int H,
                  hipStream_t stream)
{
    if (!tokens || !table || !h) return ORTHRUS_ERR_NULL;
    if (R < 1 || H < 1) return ORTHRUS_ERR_SHAPE;
    hipLaunchKernelGGL(embed_kernel, dim3((unsigned)R), dim3(256), 0, stream, tokens,
                       static_cast<const uint16_t *>(table), h, H);
    return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

}  // extern "C"
