// Shared-KV block attention for the Orthrus decode step, gfx950.
//
// Operation (Orthrus summary on gist.science, §2.1-§2.3; agents-report core
// design): a block of K query rows (anchor + K-1 mask slots) attends to the
// prefilled cache rows 0..lens[b]-1 of its KV head and to the block's own K
// rows -- all of them (diffusion view, BIDIR) or rows 0..i (AR verification
// view, CAUSAL).  One shared cache, no copy of the history.
//
// Design (MI355X):
//  * One work-group per (request b, KV head g, key split s, row block).  All
//    G*K query rows of a KV head share every K/V byte read from HBM, so the
//    contraction is dense: bf16 MFMA 32x32x16 for S^T = K Q^T and
//    O^T += V^T P^T with fp32 accumulation.
//  * K/V tiles of 64 keys stream HBM -> LDS with global_load_lds (16 B per
//    lane, no VGPR staging) through an NSTAGE-deep ring, so several tiles are
//    in flight per CU.  K is XOR-swizzled per row for conflict-free 16-byte
//    reads; V is read transposed with ds_read_b64_tr_b16 straight into the
//    MFMA A operand.
//  * S^T puts one query per lane column, so the softmax row max/sum over keys
//    is in-lane plus one permlane32 swap.  exp2 with log2(e) folded into the
//    scale.
//  * Split-KV: each split writes a normalised fp32 partial O and its base-2
//    log-sum-exp; a second pass merges them (attn_merge_kernel).  The block
//    rows are processed by the last split of each request.
//  * blockIdx.x = split * (B*Hkv) + (b*Hkv + g): with B*Hkv a multiple of 8
//    every split of one KV head lands on the same XCD (work-groups are dealt
//    round-robin over the 8 XCDs), sharing that XCD's L2 for the query tile.
#include "common.hpp"
#include "kernels.hpp"

namespace orthrus {

namespace {

constexpr int TK = 64;  // keys per tile

// 16-byte global -> LDS copy per lane (lane l lands at lds + 16*l).  Issued
// from inline asm so that the compiler does not guard every later LDS read
// with a full vmcnt(0) wait; the ring's waits are explicit s_waitcnt below.
__device__ __forceinline__ void lds_dma16(const void *gptr, uint32_t lds_addr) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "s"(m0)
                 : "memory", "m0");
}

}  // namespace

// --------------------------------------------------------------------------
// bf16 MFMA kernel
// --------------------------------------------------------------------------
// NR: 32-row query groups per work-group; KS: waves sharing one row group,
// each taking a 64/KS-key slice of every tile.  Waves = NR*KS.
template <int D, int NR, int KS, int NSTAGE, bool PAGED>
__global__ void __launch_bounds__(64 * NR * KS)
attn_bf16_kernel(AttnParams p)
{
    constexpr int NW = NR * KS;
    constexpr int GPR = D / 8;                 // 16-byte granules per row
    constexpr int RPC = 64 / GPR;              // rows per 1 KiB chunk
    constexpr int CPT = TK / RPC;              // chunks per K (or V) tile
    constexpr int TILE_ELEMS = TK * D;         // per K or V tile
    constexpr int TILE_BYTES = TILE_ELEMS * 2;
    constexpr int KPW = TK / KS;               // keys per wave per tile
    constexpr int NBLK = KPW / 32;             // S^T 32x32 blocks per wave
    constexpr int NDT = D / 32;                // O^T tiles
    static_assert(KPW % 32 == 0, "each wave needs whole 32-key blocks");
    static_assert((2 * CPT) % NW == 0, "chunks must split evenly over waves");
    constexpr int LPT = 2 * CPT / NW;          // loads per tile per lane
    constexpr int HALF = LPT / 2;              // loads [0,HALF) K, [HALF,LPT) V
    // Lazy rescaling: the running max only moves when a tile's max exceeds
    // it by more than 2^kLazy in exp2 units (weights stay <= 2^kLazy).
    constexpr float kLazy = 8.0f;

    __shared__ __attribute__((aligned(1024))) uint16_t smem[NSTAGE][2][TILE_ELEMS];
    __shared__ int s_pages[PAGED ? kMaxSplitPages : 1];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int rg = wave % NR;      // row group
    const int kg = wave / NR;      // key slice
    const int BH = p.B * p.Hkv;
    const int bh = blockIdx.x % BH;
    const int s = blockIdx.x / BH;
    const int b = bh / p.Hkv;
    const int g = bh % p.Hkv;

    // ---- key range of this split (same rule as attn_merge_kernel) ----
    const int L = p.lens[b];
    int S_b = (L + p.SL - 1) / p.SL;
    S_b = S_b < 1 ? 1 : (S_b > p.S_grid ? p.S_grid : S_b);
    if (s >= S_b) return;
    const bool last = (s == S_b - 1);
    const int kbeg = s * p.SL;
    const int kend = last ? L : kbeg + p.SL;
    const int n_cache_tiles = (kend - kbeg + TK - 1) / TK;
    const int n_tiles = n_cache_tiles + (last ? 1 : 0);   // K <= 64 = TK

    // ---- page ids of this split (paged layout) ----
    if constexpr (PAGED) {
        const int pg0 = kbeg / 16;
        const int npg = (kend - kbeg + 15) / 16;
        for (int i = tid; i < npg; i += 64 * NW)
            s_pages[i] = p.page_table[(int64_t)b * p.maxp + pg0 + i];
        __syncthreads();
    }

    // ---- query rows of this lane: B operand Q^T[d][q], q = lane % 32 ----
    const int half = lane >> 5;
    const int r = blockIdx.y * (32 * NR) + rg * 32 + (lane & 31);
    const bool row_ok = r < p.M;
    const int hl = row_ok ? r / p.K : 0;
    const int qi = row_ok ? r % p.K : 0;
    const int h = g * p.G + hl;
    bf16x8 qreg[D / 16];
    {
        const uint16_t* qp = (const uint16_t*)p.q + (((int64_t)b * p.K + qi) * p.Hq + h) * D
                             + 8 * half;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
            u32x4 v = row_ok ? *(const u32x4*)(qp + 16 * ds) : u32x4{0, 0, 0, 0};
            qreg[ds] = __builtin_bit_cast(bf16x8, v);
        }
        // Make the query loads complete here, before the LDS ring starts: the
        // compiler does not see the ring's loads, so a wait it placed later
        // for these would become a full drain of the ring.
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) asm volatile("" ::"v"(qreg[ds]));
    }

    // ---- load geometry: lane -> (row, granule) of each 1 KiB chunk ----
    // K rows are XOR-swizzled by (row & (GPR-1)) for conflict-free 16-byte
    // reads; V rows by 2*(row & 3) for the transposed 8-byte reads.
    const char* kc = (const char*)p.kc;
    const char* vc = (const char*)p.vc;
    const int64_t cont_base = ((int64_t)b * p.Hkv + g) * p.cap * D * 2;    // bytes
    const int64_t blk_base = ((int64_t)b * p.K * p.Hkv + g) * D * 2;
    const int blk_stride = p.Hkv * D * 2;
    const int prow = lane / GPR;
    const int pgr = lane % GPR;
    int lrow[LPT];                 // tile row loaded by this lane for load i
    uint32_t lgoff[LPT];           // swizzled granule byte offset within the row
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
        const bool isv = i >= HALF;
        const int cc = (isv ? i - HALF : i) * NW + wave;
        lrow[i] = cc * RPC + prow;
        lgoff[i] = 16u * (uint32_t)(isv ? (pgr ^ (2 * (lrow[i] & 3))) : (pgr ^ (lrow[i] & (GPR - 1))));
    }
    const uint32_t lds_base = (uint32_t)(uintptr_t)(ORTHRUS_LDS void*)&smem[0][0][0];

    // issue the global->LDS loads of tile t into ring slot t % NSTAGE
    auto issue = [&](int t) {
        const uint32_t slot_lds = lds_base + (uint32_t)((t % NSTAGE) * 2 * TILE_BYTES);
        const bool is_blk = t >= n_cache_tiles;
        const int start = is_blk ? 0 : kbeg + t * TK;
        const int count = is_blk ? p.K : (kend - start < TK ? kend - start : TK);
        if (!is_blk && !PAGED && count == TK) {
            // fast path: a full contiguous tile, rows D*2 bytes apart
            const char* kt = kc + cont_base + (int64_t)start * D * 2;
            const char* vt = vc + cont_base + (int64_t)start * D * 2;
#pragma unroll
            for (int i = 0; i < LPT; ++i) {
                const bool isv = i >= HALF;
                const int cc = (isv ? i - HALF : i) * NW + wave;
                lds_dma16((isv ? vt : kt) + (uint32_t)(lrow[i] * D * 2) + lgoff[i],
                          slot_lds + (isv ? TILE_BYTES : 0) + cc * 1024);
            }
        } else if (!is_blk && PAGED && count == TK) {
            // full paged tile: 4 pages of 16 rows
            const int pidx = (start - kbeg) >> 4;
#pragma unroll
            for (int i = 0; i < LPT; ++i) {
                const bool isv = i >= HALF;
                const int cc = (isv ? i - HALF : i) * NW + wave;
                const int page = s_pages[pidx + (lrow[i] >> 4)];
                const char* base = (isv ? vc : kc) +
                    ((int64_t)page * p.Hkv + g) * (16 * D * 2);
                lds_dma16(base + (uint32_t)((lrow[i] & 15) * D * 2) + lgoff[i],
                          slot_lds + (isv ? TILE_BYTES : 0) + cc * 1024);
            }
        } else {
            // partial cache tile or the block tile: clamp rows to count-1
#pragma unroll
            for (int i = 0; i < LPT; ++i) {
                const bool isv = i >= HALF;
                const int cc = (isv ? i - HALF : i) * NW + wave;
                const int rowc = lrow[i] < count ? lrow[i] : count - 1;
                const char* src;
                if (is_blk) {
                    src = (isv ? (const char*)p.vb : (const char*)p.kb) + blk_base +
                          (int64_t)rowc * blk_stride;
                } else if (PAGED) {
                    const int key = start + rowc;
                    const int page = s_pages[(key - kbeg) >> 4];
                    src = (isv ? vc : kc) + (((int64_t)page * p.Hkv + g) * 16 + (key & 15)) * D * 2;
                } else {
                    src = (isv ? vc : kc) + cont_base + (int64_t)(start + rowc) * D * 2;
                }
                lds_dma16(src + lgoff[i], slot_lds + (isv ? TILE_BYTES : 0) + cc * 1024);
            }
        }
    };

    f32x16 oacc[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY;   // running max of raw scores (this lane's query)
    float l_run = 0.f;         // running sum of this lane-half's weights
    const float c = p.c;       // scale * log2(e)
    const float lazy_raw = kLazy / c;

    // prologue
#pragma unroll
    for (int t = 0; t < NSTAGE - 1; ++t)
        if (t < n_tiles) issue(t);

    for (int t = 0; t < n_tiles; ++t) {
        // wait for this lane's loads of tile t, then make everyone's visible
        if (t + NSTAGE - 2 < n_tiles)
            __builtin_amdgcn_s_waitcnt(vmcnt_encode((NSTAGE - 2) * LPT));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_encode(0));
        __syncthreads();
        if (t + NSTAGE - 1 < n_tiles) issue(t + NSTAGE - 1);

        const int slot = t % NSTAGE;
        const uint16_t* Ks = smem[slot][0];
        const uint16_t* Vs = smem[slot][1];
        const bool is_blk = t >= n_cache_tiles;
        const int start = is_blk ? 0 : kbeg + t * TK;
        const int count = is_blk ? p.K : (kend - start < TK ? kend - start : TK);

        // ---- S^T = K Q^T for this wave's key slice ----
        f32x16 sacc[NBLK];
#pragma unroll
        for (int kb = 0; kb < NBLK; ++kb) {
            const int krow = kg * KPW + kb * 32 + (lane & 31);
            u32x4 kf[D / 16];   // all operand reads of the block first, then the MFMAs
#pragma unroll
            for (int ds = 0; ds < D / 16; ++ds) {
                const int lgr = (2 * ds + half) ^ (krow & (GPR - 1));
                kf[ds] = *(const u32x4*)(Ks + krow * D + lgr * 8);
            }
            sacc[kb] = f32x16{};
#pragma unroll
            for (int ds = 0; ds < D / 16; ++ds)
                sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, kf[ds]), qreg[ds], sacc[kb], 0, 0, 0);
        }

        // ---- mask (partial cache tile, or the block tile) ----
        const bool need_mask = is_blk ? (p.mask == 1 || count < TK) : (count < TK);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < NBLK; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = kg * KPW + kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                    bool ok = key < count;
                    if (is_blk && p.mask == 1) ok = ok && key <= qi;
                    if (!ok) sacc[kb][i] = -INFINITY;
                }
        }

        // ---- online softmax (row = this lane's query column) ----
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NBLK; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
        {
            auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        if (__any(mx > m_run + lazy_raw)) {
            const float m_new = fmaxf(m_run, mx);
            const float corr = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * c);
            m_run = m_new;
            l_run *= corr;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= corr;
        }
        const float mc = (m_run == -INFINITY) ? 0.f : m_run * c;
        float psum = 0.f;
        bf16x8 pb[NBLK][2];
#pragma unroll
        for (int kb = 0; kb < NBLK; ++kb)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                f32x2 pv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pv[j][0] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * hh + 2 * j], c, -mc));
                    pv[j][1] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * hh + 2 * j + 1], c, -mc));
                }
                uint32_t w[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    w[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pv[j], bf16x2));
                    // the denominator sums the same rounded weights that enter P V,
                    // so the output stays an exact convex combination of V rows
                    psum += __uint_as_float(w[j] << 16) + __uint_as_float(w[j] & 0xffff0000u);
                }
                pb[kb][hh] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
            }
        l_run += psum;

        // ---- O^T += V^T P^T ----
        const int G16 = lane >> 4;
        const int sl = lane & 15;
#pragma unroll
        for (int kb = 0; kb < NBLK; ++kb)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int rowbase = kg * KPW + kb * 32 + 16 * hh + 4 * (G16 >> 1) + (sl >> 2);
                u32x4 vf[NDT];   // all transposed reads of this k-step first
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const int col = 32 * dt + 16 * (G16 & 1) + 4 * (sl & 3);
                    u32x2 vv[2];
#pragma unroll
                    for (int ins = 0; ins < 2; ++ins) {
                        const int row = rowbase + 8 * ins;
                        const int gr = (col >> 3) ^ (2 * (row & 3));
                        const uint16_t* a = Vs + row * D + gr * 8 + (col & 7);
                        vv[ins] = __builtin_bit_cast(
                            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((ORTHRUS_LDS s16x4*)a));
                    }
                    vf[dt] = u32x4{vv[0][0], vv[0][1], vv[1][0], vv[1][1]};
                }
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, vf[dt]), pb[kb][hh], oacc[dt], 0, 0, 0);
            }
    }

    // ---- merge the key slices of one row group (KS > 1) ----
    if constexpr (KS > 1) {
        __syncthreads();   // all waves are done with the ring; reuse it
        float* red = reinterpret_cast<float*>(&smem[0][0][0]);
        // per row group: [KS-1][NDT*16 + 2][64] floats (accumulators, m, l)
        constexpr int ACC = NDT * 16;
        float* base = red + rg * (KS - 1) * (ACC + 2) * 64;
        if (kg > 0) {
            float* mine = base + (kg - 1) * (ACC + 2) * 64;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) mine[(dt * 16 + i) * 64 + lane] = oacc[dt][i];
            mine[ACC * 64 + lane] = m_run;
            mine[(ACC + 1) * 64 + lane] = l_run;
        }
        __syncthreads();
        if (kg > 0) return;
#pragma unroll
        for (int o = 0; o < KS - 1; ++o) {
            const float* other = base + o * (ACC + 2) * 64;
            const float m_o = other[ACC * 64 + lane];
            const float l_o = other[(ACC + 1) * 64 + lane];
            const float m_t = fmaxf(m_run, m_o);
            const float a0 = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_run - m_t) * c);
            const float a1 = (m_o == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_o - m_t) * c);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    oacc[dt][i] = oacc[dt][i] * a0 + other[(dt * 16 + i) * 64 + lane] * a1;
            l_run = l_run * a0 + l_o * a1;
            m_run = m_t;
        }
    }

    // ---- finalize: this lane owns query row r, d = 32dt + 8(i/4) + 4*half + i%4 ----
    {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run),
                                                   false, false);
        l_run = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if (!row_ok) return;
    const float inv = 1.f / l_run;
    const float lse2 = m_run * c + __builtin_log2f(l_run);
    if (p.S_grid == 1) {
        uint16_t* op = (uint16_t*)p.out + (((int64_t)b * p.K + qi) * p.Hq + h) * D + 4 * half;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int i0 = 4 * q4;
                const bf16x2 lo = __builtin_convertvector(
                    (f32x2{oacc[dt][i0] * inv, oacc[dt][i0 + 1] * inv}), bf16x2);
                const bf16x2 hi = __builtin_convertvector(
                    (f32x2{oacc[dt][i0 + 2] * inv, oacc[dt][i0 + 3] * inv}), bf16x2);
                *(u32x2*)(op + 32 * dt + 8 * q4) =
                    u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
            }
        if (p.lse && half == 0) p.lse[((int64_t)b * p.Hq + h) * p.K + qi] = lse2 * kLn2;
    } else {
        const int64_t prow = ((int64_t)bh * p.M + r) * p.S_grid + s;
        float* op = p.ws_o + prow * D + 4 * half;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int i0 = 4 * q4;
                f32x4 v = {oacc[dt][i0] * inv, oacc[dt][i0 + 1] * inv, oacc[dt][i0 + 2] * inv,
                           oacc[dt][i0 + 3] * inv};
                *(f32x4*)(op + 32 * dt + 8 * q4) = v;
            }
        if (half == 0) p.ws_lse[prow] = lse2;
    }
}

// --------------------------------------------------------------------------
// fp32 kernel (VALU, exact-ish fp32 arithmetic; small problems)
// --------------------------------------------------------------------------
// 4 waves; each wave owns 4 query rows of the work-group's 16; a lane is a
// key for scores and an output column for P V.
template <int D>
__global__ void __launch_bounds__(256) attn_f32_kernel(AttnParams p)
{
    constexpr int RW = 4;                 // rows per wave
    constexpr int ROWS = 16;
    constexpr int DC = D / 64;            // output columns per lane
    __shared__ float Ks[TK][D + 1];
    __shared__ float Vs[TK][D];
    __shared__ float Qs[ROWS][D];
    __shared__ float Ps[4][TK];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int BH = p.B * p.Hkv;
    const int bh = blockIdx.x % BH;
    const int s = blockIdx.x / BH;
    const int b = bh / p.Hkv;
    const int g = bh % p.Hkv;
    const int L = p.lens[b];
    int S_b = (L + p.SL - 1) / p.SL;
    S_b = S_b < 1 ? 1 : (S_b > p.S_grid ? p.S_grid : S_b);
    if (s >= S_b) return;
    const bool last = (s == S_b - 1);
    const int kbeg = s * p.SL;
    const int kend = last ? L : kbeg + p.SL;
    const int n_cache_tiles = (kend - kbeg + TK - 1) / TK;
    const int n_tiles = n_cache_tiles + (last ? 1 : 0);
    const float* q = (const float*)p.q;
    const float* kc = (const float*)p.kc;
    const float* vc = (const float*)p.vc;
    const float* kbk = (const float*)p.kb;
    const float* vbk = (const float*)p.vb;

    const int row0 = blockIdx.y * ROWS;
    for (int i = tid; i < ROWS * D; i += 256) {
        const int rr = row0 + i / D;
        float v = 0.f;
        if (rr < p.M) {
            const int hl = rr / p.K, qi = rr % p.K;
            v = q[(((int64_t)b * p.K + qi) * p.Hq + g * p.G + hl) * D + i % D];
        }
        Qs[i / D][i % D] = v;
    }
    float m_run[RW], l_run[RW], o[RW][DC];
#pragma unroll
    for (int j = 0; j < RW; ++j) {
        m_run[j] = -INFINITY;
        l_run[j] = 0.f;
#pragma unroll
        for (int k = 0; k < DC; ++k) o[j][k] = 0.f;
    }
    const float c = p.c;
    for (int t = 0; t < n_tiles; ++t) {
        const bool is_blk = t >= n_cache_tiles;
        const int start = is_blk ? 0 : kbeg + t * TK;
        const int count = is_blk ? p.K : (kend - start < TK ? kend - start : TK);
        __syncthreads();
        for (int i = tid; i < TK * D; i += 256) {
            const int row = i / D, d = i % D;
            float kv = 0.f, vv = 0.f;
            if (row < count) {
                int64_t off;
                if (is_blk) {
                    off = (((int64_t)b * p.K + row) * p.Hkv + g) * D + d;
                    kv = kbk[off];
                    vv = vbk[off];
                } else {
                    const int key = start + row;
                    if (p.layout == 0) {
                        off = (((int64_t)b * p.Hkv + g) * p.cap + key) * D + d;
                    } else {
                        const int page = p.page_table[(int64_t)b * p.maxp + (key >> 4)];
                        off = (((int64_t)page * p.Hkv + g) * 16 + (key & 15)) * D + d;
                    }
                    kv = kc[off];
                    vv = vc[off];
                }
            }
            Ks[row][d] = kv;
            Vs[row][d] = vv;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            const int lr = wave * RW + j;
            const int rr = row0 + lr;
            const int qi = rr < p.M ? rr % p.K : 0;
            float sc = 0.f;
#pragma unroll 8
            for (int d = 0; d < D; ++d) sc = __builtin_fmaf(Qs[lr][d], Ks[lane][d], sc);
            bool ok = lane < count;
            if (is_blk && p.mask == 1) ok = ok && lane <= qi;
            sc = ok ? sc : -INFINITY;
            float mx = sc;
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
            const float m_new = fmaxf(m_run[j], mx);
            const float corr = (m_run[j] == -INFINITY) ? 0.f : exp2f((m_run[j] - m_new) * c);
            const float pv = ok ? exp2f((sc - m_new) * c) : 0.f;
            m_run[j] = m_new;
            float ps = pv;
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) ps += __shfl_xor(ps, m, 64);
            l_run[j] = l_run[j] * corr + ps;
            Ps[wave][lane] = pv;
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int k = 0; k < DC; ++k) {
                float acc = o[j][k] * corr;
                for (int key = 0; key < TK; ++key)
                    acc = __builtin_fmaf(Ps[wave][key], Vs[key][lane + 64 * k], acc);
                o[j][k] = acc;
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
#pragma unroll
    for (int j = 0; j < RW; ++j) {
        const int rr = row0 + wave * RW + j;
        if (rr >= p.M) continue;
        const int hl = rr / p.K, qi = rr % p.K;
        const int h = g * p.G + hl;
        const float inv = 1.f / l_run[j];
        const float lse2 = m_run[j] * c + log2f(l_run[j]);
        if (p.S_grid == 1) {
            float* op = (float*)p.out + (((int64_t)b * p.K + qi) * p.Hq + h) * D;
#pragma unroll
            for (int k = 0; k < DC; ++k) op[lane + 64 * k] = o[j][k] * inv;
            if (p.lse && lane == 0) p.lse[((int64_t)b * p.Hq + h) * p.K + qi] = lse2 * kLn2;
        } else {
            const int64_t prow = ((int64_t)bh * p.M + rr) * p.S_grid + s;
#pragma unroll
            for (int k = 0; k < DC; ++k) p.ws_o[prow * D + lane + 64 * k] = o[j][k] * inv;
            if (lane == 0) p.ws_lse[prow] = lse2;
        }
    }
}

// --------------------------------------------------------------------------
// split-KV merge: lse = log sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s
// --------------------------------------------------------------------------
// Partials are [B*Hkv][M][S_grid][D] (one row's splits contiguous) with base-2
// lse [B*Hkv][M][S_grid].  A work-group of 128 threads merges 128/(D/4) rows;
// each thread owns 4 columns of one row and keeps 8 split loads in flight.
template <int D, bool BF16>
__global__ void __launch_bounds__(128) attn_merge_kernel(AttnParams p)
{
    constexpr int TPR = D / 4;          // threads per row (4 floats each)
    constexpr int RPB = 128 / TPR;      // rows per block
    constexpr int UNROLL = 8;
    const int bh = blockIdx.x;
    const int b = bh / p.Hkv;
    const int g = bh % p.Hkv;
    const int r = blockIdx.y * RPB + threadIdx.x / TPR;
    const int d = (threadIdx.x % TPR) * 4;
    if (r >= p.M) return;
    const int L = p.lens[b];
    int S_b = (L + p.SL - 1) / p.SL;
    S_b = S_b < 1 ? 1 : (S_b > p.S_grid ? p.S_grid : S_b);
    const int64_t row = (int64_t)bh * p.M + r;
    const float* lse_r = p.ws_lse + row * p.S_grid;
    const float* o_r = p.ws_o + row * p.S_grid * D + d;
    float mx = -INFINITY;
    for (int s = 0; s < S_b; ++s) mx = fmaxf(mx, lse_r[s]);
    float W = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int s = 0;
    for (; s + UNROLL <= S_b; s += UNROLL) {
        f32x4 v[UNROLL];
        float w[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = *(const f32x4*)(o_r + (int64_t)(s + u) * D);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) w[u] = __builtin_amdgcn_exp2f(lse_r[s + u] - mx);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            W += w[u];
            acc += w[u] * v[u];
        }
    }
    for (; s < S_b; ++s) {
        const float w = __builtin_amdgcn_exp2f(lse_r[s] - mx);
        W += w;
        acc += w * *(const f32x4*)(o_r + (int64_t)s * D);
    }
    const float inv = 1.f / W;
    const int hl = r / p.K, qi = r % p.K;
    const int h = g * p.G + hl;
    const int64_t oo = (((int64_t)b * p.K + qi) * p.Hq + h) * D + d;
    if (BF16) {
        u32x2 v = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
        *(u32x2*)((uint16_t*)p.out + oo) = v;
    } else {
        *(f32x4*)((float*)p.out + oo) = acc * inv;
    }
    if (p.lse && d == 0) p.lse[((int64_t)b * p.Hq + h) * p.K + qi] = (mx + __builtin_log2f(W)) * kLn2;
}

// --------------------------------------------------------------------------
// launch
// --------------------------------------------------------------------------
template <int D, int NR, int KS>
static hipError_t launch_bf16(const AttnParams& p, hipStream_t st) {
    dim3 grid(p.S_grid * p.B * p.Hkv, p.row_blocks);
    constexpr int NSTAGE = 4;
    if (p.layout == 1)
        hipLaunchKernelGGL((attn_bf16_kernel<D, NR, KS, NSTAGE, true>), grid, dim3(64 * NR * KS), 0, st, p);
    else
        hipLaunchKernelGGL((attn_bf16_kernel<D, NR, KS, NSTAGE, false>), grid, dim3(64 * NR * KS), 0, st, p);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_bf16_d(const AttnParams& p, hipStream_t st) {
    switch (p.rows_per_wg) {
        case 32: return launch_bf16<D, 1, 2>(p, st);
        case 64: return launch_bf16<D, 2, 2>(p, st);
        case 128: return launch_bf16<D, 4, 2>(p, st);
        default: return launch_bf16<D, 8, 1>(p, st);
    }
}

int attn_rows_per_wg(int dtype, int M) {
    if (dtype == 0) return 16;
    if (M <= 32) return 32;
    if (M <= 64) return 64;
    if (M <= 128) return 128;
    return 256;
}

hipError_t launch_block_attn(const AttnParams& p, int dtype, hipStream_t st) {
    hipError_t e;
    dim3 grid(p.S_grid * p.B * p.Hkv, p.row_blocks);
    if (dtype == 1) {
        e = (p.D == 128) ? launch_bf16_d<128>(p, st) : launch_bf16_d<64>(p, st);
    } else {
        if (p.D == 128) hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(256), 0, st, p);
        else hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(256), 0, st, p);
        e = hipGetLastError();
    }
    if (e != hipSuccess || p.S_grid == 1) return e;
    const int rpb = 128 / (p.D / 4);
    dim3 mgrid(p.B * p.Hkv, (p.M + rpb - 1) / rpb);
    if (p.D == 128) {
        if (dtype == 1) hipLaunchKernelGGL((attn_merge_kernel<128, true>), mgrid, dim3(128), 0, st, p);
        else hipLaunchKernelGGL((attn_merge_kernel<128, false>), mgrid, dim3(128), 0, st, p);
    } else {
        if (dtype == 1) hipLaunchKernelGGL((attn_merge_kernel<64, true>), mgrid, dim3(128), 0, st, p);
        else hipLaunchKernelGGL((attn_merge_kernel<64, false>), mgrid, dim3(128), 0, st, p);
    }
    return hipGetLastError();
}

}  // namespace orthrus
