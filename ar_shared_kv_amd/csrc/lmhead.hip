// Greedy prediction straight from the hidden states: the LM head's logits
// row . W^T and their row argmax in one pass, without writing the logits.
//
// Operation (Orthrus summary on gist.science, §2.3: both views predict
// greedily from their final hidden states; the consensus compares the two
// argmax tokens): idx[r] = argmax_v sum_k x[r][k] * w[v][k], lowest index on
// ties, for R rows of H hidden values and a V x H weight matrix.
//
// Design (MI355X): decode has few rows (R = B*K, 32 at the Qwen3-8B shape)
// against V = 151,936 vocabulary rows, so the weight matrix is read once and
// the work is HBM-bound.  One work-group per (128 vocabulary rows, RB hidden
// rows; RB = 32, 64, 128 or 256 by R, so that serving batches read the weight
// once per 256 rows): 128 x 64 weight chunks and the matching RB x 64 hidden chunk
// stream HBM -> LDS with global_load_lds (16-byte granules XOR-swizzled per
// row) through a ring (3 slots at RB <= 64: two chunks in flight while one is
// computed; 2 slots at RB >= 128); two work-groups share a CU at RB <= 128.  Each wave owns 32 vocabulary rows:
// logits^T = W x^T on the matrix cores (v_mfma_f32_32x32x16_bf16, fp32
// accumulation over H), then a (value, lowest index) key per hidden row is
// reduced over the lanes, the waves and, in a second launch with one
// work-group per row, over the vocabulary blocks.
//
// The weight is stored packed (orthrus_pack_weight: 128 x 64 tiles, a block's
// tiles in column order, block after block), so each work-group streams one
// contiguous 1 MiB run (H = 4,096).  Row-major rows are H*2 bytes apart and
// work-groups reading the same column chunk at once kept hitting the same HBM
// channels: at the Qwen3-8B head (32 rows) 268 us per call row-major, 228 us
// with row-major walks started at nine different places (and a bookkeeping of
// segment sums to keep one summation order), 215 us packed.  Every block
// walks H from column 0 in order, so every vocabulary row goes through the
// same fp32 operations: equal weight rows give bitwise-equal logits anywhere
// in V, and ties go to the lowest index.
#include "common.hpp"
#include "kernels.hpp"
#include "wtile.hpp"

#include "../../include/orthrus.h"

namespace orthrus {

namespace {

constexpr int kLmVB = 128;                    // vocabulary rows per work-group
constexpr int kLmHC = 64;                     // hidden columns per chunk (the H granularity)
constexpr int kLmStages = 3;                  // ring slots at RB <= 64: two chunks in flight

// 16-byte global -> LDS copy per lane (lane l lands at lds + 16*l); the waits
// are the explicit s_waitcnt of the chunk loop.
__device__ __forceinline__ void lm_dma16(const void* gptr, uint32_t lds_addr) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "s"(m0)
                 : "memory", "m0");
}

// HC hidden columns per chunk (one packed tile), NSTAGE ring slots (NSTAGE - 1
// chunks in flight while one is computed), RB hidden rows per work-group (32,
// 64, 128 or 256: the weight is read once per RB rows).
template <int HC, int NSTAGE, int RB>
__global__ void __launch_bounds__(256, 2)
lmhead_argmax_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int R, int H,
                     int V, int nvb, uint64_t* __restrict__ ws)
{
    constexpr int WB = kLmVB * HC * 2;          // weight bytes per chunk
    constexpr int XB = RB * HC * 2;             // hidden bytes per chunk
    constexpr int NB = RB / 32;                 // 32-row MFMA column blocks per wave
    constexpr int SLOT = WB + XB;
    constexpr int GR = HC / 8;                  // 16-byte granules per row
    constexpr int RPP = 1024 / (HC * 2);        // rows per 1 KiB wave load
    constexpr int LOADS = SLOT / 4096;          // loads per lane per chunk
    constexpr int NPRE = NSTAGE - 1;
    static_assert(HC == kWTileCols && kLmVB == kWTileRows, "one packed tile per chunk");
    static_assert(SLOT % 4096 == 0 && WB % 1024 == 0, "whole wave loads per chunk");
    static_assert(LOADS * NSTAGE <= 63, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * SLOT];
    __shared__ uint64_t red[4][RB];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int vb = blockIdx.x;
    const int v0 = vb * kLmVB;
    const int r0 = blockIdx.y * RB;
    const int nchunk = H / HC;
    const uint16_t* wblk = w + (int64_t)vb * nchunk * (kLmVB * HC);   // this block's tiles
    const uint32_t lds_base = (uint32_t)(uintptr_t)(ORTHRUS_LDS void*)&smem[0];

    // DMA of chunk c into slot c % NSTAGE.  A 1 KiB wave load covers RPP rows
    // of GR granules; lane l writes LDS granule l % GR of its row with the
    // global granule (l % GR) ^ (row % GR), so that granule g of a row sits at
    // g ^ (row % GR) and the fragment reads below spread over the banks.
    auto issue = [&](int c) __attribute__((always_inline)) {
        const uint32_t slot = lds_base + (uint32_t)((c % NSTAGE) * SLOT);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int k = i * 4 + wave;                  // 1 KiB piece of the slot
            const bool isx = k >= WB / 1024;
            const int row = (isx ? k - WB / 1024 : k) * RPP + lane / GR;
            const int gsrc = (lane % GR) ^ (row % GR);
            const uint16_t* src;
            if (isx) {
                const int rr = r0 + row < R ? r0 + row : R - 1;
                src = x + (int64_t)rr * H + c * HC + gsrc * 8;
            } else {
                src = wblk + (int64_t)c * (kLmVB * HC) + row * HC + gsrc * 8;
            }
            lm_dma16(src, slot + (uint32_t)(k * 1024));
        }
    };
    // wait until chunk c has landed: at most min(NPRE - 1, chunks after c)
    // later chunks of this lane may still fly
    auto wait_chunk = [&](int c) __attribute__((always_inline)) {
        const int later = nchunk - 1 - c;
        const int pend = later < NPRE - 1 ? later : NPRE - 1;
        switch (pend) {
            case 0: __builtin_amdgcn_s_waitcnt(vmcnt_encode(0)); break;
            case 1: __builtin_amdgcn_s_waitcnt(vmcnt_encode(LOADS)); break;
            case 2: __builtin_amdgcn_s_waitcnt(vmcnt_encode(2 * LOADS)); break;
            default: __builtin_amdgcn_s_waitcnt(vmcnt_encode(3 * LOADS)); break;
        }
    };
    static_assert(NPRE - 1 <= 3, "wait_chunk covers up to 3 later chunks");

    f32x16 tot[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) tot[j] = f32x16{};
    const int vrow = wave * 32 + (lane & 31);            // this lane's vocabulary row (A operand)
    for (int c = 0; c < NPRE && c < nchunk; ++c) issue(c);
    for (int c = 0; c < nchunk; ++c) {
        wait_chunk(c);
        __syncthreads();                 // everyone's part landed; slot (c-1) % NSTAGE is free
        if (c + NPRE < nchunk) issue(c + NPRE);
        const char* Ws = smem + (c % NSTAGE) * SLOT;
        const char* Xs = Ws + WB;
        u32x4 af[HC / 16], bfr[NB][HC / 16];
#pragma unroll
        for (int ds = 0; ds < HC / 16; ++ds) {
            const int g = 2 * ds + half;
            af[ds] = *(const u32x4*)(Ws + vrow * (HC * 2) + ((g ^ (vrow % GR)) * 16));
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int xrow = 32 * j + (lane & 31);   // hidden row of block j (B operand)
                bfr[j][ds] = *(const u32x4*)(Xs + xrow * (HC * 2) + ((g ^ (xrow % GR)) * 16));
            }
        }
#pragma unroll
        for (int ds = 0; ds < HC / 16; ++ds)
#pragma unroll
            for (int j = 0; j < NB; ++j)
                tot[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, af[ds]), __builtin_bit_cast(bf16x8, bfr[j][ds]),
                    tot[j], 0, 0, 0);
    }

    // tot[j][i] = logit of vocabulary row v0 + 32*wave + 8*(i/4) + 4*half + i%4
    // for hidden row r0 + 32*j + lane%32
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        uint64_t key = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int v = v0 + wave * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
            if (v < V) {
                const uint64_t k = argmax_key(tot[j][i], (uint32_t)v);
                key = k > key ? k : key;
            }
        }
        const uint64_t o = shfl_xor_u64(key, 32);
        key = o > key ? o : key;
        if (lane < 32) red[wave][32 * j + lane] = key;
    }
    __syncthreads();
    if (tid < RB) {
        uint64_t k = red[0][tid];
#pragma unroll
        for (int q = 1; q < 4; ++q) k = red[q][tid] > k ? red[q][tid] : k;
        if (r0 + tid < R) ws[(int64_t)(r0 + tid) * nvb + vb] = k;
    }
}

// Second pass: one work-group per hidden row reduces that row's per-block
// keys.  Every lane issues all its loads before the first comparison, so the
// pass costs one memory round trip for up to 2048 vocabulary blocks.
__global__ void __launch_bounds__(256)
lmhead_finalize_kernel(const uint64_t* __restrict__ ws, int nvb, int32_t* __restrict__ idx)
{
    __shared__ uint64_t part[4];
    const uint64_t* p = ws + (int64_t)blockIdx.x * nvb;
    uint64_t key = 0;
    for (int c0 = threadIdx.x; c0 < nvb; c0 += 256 * 8) {
        uint64_t v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = c0 + 256 * j < nvb ? p[c0 + 256 * j] : 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) key = v[j] > key ? v[j] : key;
    }
    key = wave_max_u64(key);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = key;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t k = part[0];
#pragma unroll
        for (int q = 1; q < 4; ++q) k = part[q] > k ? part[q] : k;
        idx[blockIdx.x] = (int32_t)argmax_key_index(k);
    }
}

int64_t lm_blocks(int V) { return ((int64_t)V + kLmVB - 1) / kLmVB; }

bool lm_shape_ok(int R, int H, int V) {
    return R >= 1 && R <= 65535 * 32 && H >= kLmHC && H % kLmHC == 0 && H <= 65536 &&
           V >= 1;
}

}  // namespace

}  // namespace orthrus

using namespace orthrus;

extern "C" {

size_t orthrus_lmhead_argmax_workspace_bytes(int R, int H, int V, int dtype)
{
    if (dtype != ORTHRUS_BF16 || !lm_shape_ok(R, H, V)) return 0;
    return (size_t)R * (size_t)lm_blocks(V) * sizeof(uint64_t);
}

int orthrus_lmhead_argmax(const void *hidden, const void *weight, int R, int H, int V, int dtype,
                          int32_t *idx, void *workspace, size_t workspace_bytes,
                          hipStream_t stream)
{
    if (!hidden || !weight || !idx) return ORTHRUS_ERR_NULL;
    if (dtype != ORTHRUS_BF16 && dtype != ORTHRUS_F32) return ORTHRUS_ERR_DTYPE;
    if (R < 1 || H < 1 || V < 1) return ORTHRUS_ERR_SHAPE;
    if (dtype != ORTHRUS_BF16 || !lm_shape_ok(R, H, V)) return ORTHRUS_ERR_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(hidden) & 15u) || (reinterpret_cast<uintptr_t>(weight) & 15u))
        return ORTHRUS_ERR_UNSUPPORTED;
    const int64_t nvb = lm_blocks(V);
    const size_t need = (size_t)R * (size_t)nvb * sizeof(uint64_t);
    if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 7u))
        return ORTHRUS_ERR_WORKSPACE;
    uint64_t *ws = static_cast<uint64_t *>(workspace);
    // hidden rows per work-group: the weight is read ceil(R / RB) times
    const uint16_t *xp = static_cast<const uint16_t *>(hidden);
    const uint16_t *wp = static_cast<const uint16_t *>(weight);
    const dim3 g1((unsigned)nvb, 1);
    if (R <= 32) {
        hipLaunchKernelGGL((lmhead_argmax_kernel<kLmHC, kLmStages, 32>), g1, dim3(256), 0, stream,
                           xp, wp, R, H, V, (int)nvb, ws);
    } else if (R <= 64) {
        hipLaunchKernelGGL((lmhead_argmax_kernel<kLmHC, kLmStages, 64>), g1, dim3(256), 0, stream,
                           xp, wp, R, H, V, (int)nvb, ws);
    } else if (R > 128) {
        // one work-group per CU (104 KiB of LDS), half the weight reads of
        // 128-row blocks (R = 1024: 1.70 vs 1.91 ms per call, row-major weight)
        hipLaunchKernelGGL((lmhead_argmax_kernel<kLmHC, 2, 256>),
                           dim3((unsigned)nvb, (unsigned)((R + 255) / 256)), dim3(256), 0, stream,
                           xp, wp, R, H, V, (int)nvb, ws);
    } else {
        // two slots: two work-groups per CU (68 KiB of LDS each) beat one with
        // three slots (R = 1024: 1.90 vs 2.13 ms per call, row-major weight)
        hipLaunchKernelGGL((lmhead_argmax_kernel<kLmHC, 2, 128>),
                           dim3((unsigned)nvb, (unsigned)((R + 127) / 128)), dim3(256), 0, stream,
                           xp, wp, R, H, V, (int)nvb, ws);
    }
    if (hipGetLastError() != hipSuccess) return ORTHRUS_ERR_LAUNCH;
    hipLaunchKernelGGL(lmhead_finalize_kernel, dim3((unsigned)R), dim3(256), 0, stream,
                       static_cast<const uint64_t *>(ws), (int)nvb, idx);
    return hipGetLastError() == hipSuccess ? ORTHRUS_OK : ORTHRUS_ERR_LAUNCH;
}

}  // extern "C"
