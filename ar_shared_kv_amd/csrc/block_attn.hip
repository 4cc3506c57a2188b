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
//    lane, no VGPR staging) through an NSTAGE-deep ring, NPRE tiles ahead of
//    the one computed.  K is XOR-swizzled per row for conflict-free 16-byte
//    reads; V is read transposed with ds_read_b64_tr_b16 straight into the
//    MFMA A operand.
//  * S^T puts one query per lane column, so the softmax row max over keys is
//    in-lane plus one permlane32 swap; exp2 with log2(e) folded into the
//    scale; row sums of the bf16-rounded weights on the matrix cores.
//  * Split-KV: each split writes its normalised partial O (in the path's
//    dtype, in MFMA fragment order) and its base-2 log-sum-exp through the
//    L2; a second launch merges them (attn_merge_kernel).  The block rows are
//    processed by the last split of each request.
//  * blockIdx.x = split * (B*Hkv) + (b*Hkv + g): with B*Hkv a multiple of 8
//    every split of one KV head lands on the same XCD (work-groups are dealt
//    round-robin over the 8 XCDs), sharing that XCD's L2 for the query tile.
//    Ragged paged batches instead walk a longest-first list of (request,
//    split) items.
//  * Full tiles run in a steady loop with every per-tile test resolved;
//    work-groups of at most four waves (32 or 64 rows, or 128 rows in one key
//    slice when they outnumber the CUs) take a 2-slot ring so that two share
//    a CU.
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

// The same with a wave-uniform base in SGPRs and a 32-bit per-lane offset
// (the SADDR form): the per-lane 64-bit address adds drop out of the loop.
__device__ __forceinline__ void lds_dma16_s(const void *sbase, uint32_t voff, uint32_t lds_addr) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(m0)
                 : "memory", "m0");
}

// 4-byte global -> LDS copy per active lane (lane l lands at lds + 4*l).
__device__ __forceinline__ void lds_dma4(const void *gptr, uint32_t lds_addr) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(gptr), "s"(m0)
                 : "memory", "m0");
}

}  // namespace

// Element offset of (row r, column d) inside one split partial block of
// Mpad x D values, in the order the MFMA accumulators hold them: every store
// of four columns by a wave covers 512 contiguous bytes (bf16).
__device__ __forceinline__ int64_t frag_offset(int r, int d, int D) {
    return (((((int64_t)(r >> 5) * (D >> 5) + (d >> 5)) * 4 + ((d & 31) >> 3)) * 2 + ((d & 7) >> 2)) * 32
            + (r & 31)) * 4 + (d & 3);
}

// Work item of position `pos` in a longest-first list of (request, split)
// items, for ragged paged batches (B <= 64, one request per lane).  Every
// request's splits but its last have SL keys; those come first, in (request,
// split) order, then the last splits by decreasing length (ties by request).
// The hardware starts work-groups in index order as CUs free up, so this is
// list scheduling longest-first: the long items no longer start last and
// leave CUs idle at the end.  Computed by each wave from lens (no DMA is in
// flight yet, so the vector load does not wait behind one).  Returns false for
// positions past the last item.
__device__ __forceinline__ bool lpt_item(const AttnParams& p, int pos, int lane, int& b_out,
                                         int& s_out) {
    const bool in = lane < p.B;
    const int L = in ? p.lens[lane] : 0;
    int Sb = (L + p.SL - 1) / p.SL;
    Sb = Sb < 1 ? 1 : (Sb > p.S_grid ? p.S_grid : Sb);
    const int nfull = in ? Sb - 1 : 0;
    const int tail = in ? L - (Sb - 1) * p.SL : -1;
    int incl = nfull;                                  // inclusive scan of nfull
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    const int F = __shfl(incl, 63, 64);                // full splits in the batch
    const int excl = incl - nfull;
    if (pos < F) {
        const uint64_t m = __ballot(in && pos >= excl && pos < incl);
        const int b = __builtin_ctzll(m);
        b_out = __builtin_amdgcn_readfirstlane(b);
        s_out = __builtin_amdgcn_readfirstlane(pos - __shfl(excl, b, 64));
        return true;
    }
    const int want = pos - F;                          // rank among the last splits
    if (want >= p.B) return false;
    int rank = 0;
    for (int j = 0; j < p.B; ++j) {
        const int tj = __shfl(tail, j, 64);
        rank += (tj > tail || (tj == tail && j < lane)) ? 1 : 0;
    }
    const uint64_t m = __ballot(in && rank == want);
    const int b = __builtin_ctzll(m);
    b_out = __builtin_amdgcn_readfirstlane(b);
    s_out = __builtin_amdgcn_readfirstlane(__shfl(Sb, b, 64) - 1);
    return true;
}

// --------------------------------------------------------------------------
// bf16 MFMA kernel
// --------------------------------------------------------------------------
// NR: 32-row query groups per work-group; KS: waves sharing one row group,
// each taking a 64/KS-key slice of every tile (waves = NR*KS); NSTAGE: ring
// slots; NPRE: tiles kept in
// flight ahead of the one being computed; QLDS: the query tile is fetched by
// LDS DMA as part of the prologue instead of through VGPR loads.
// Two work-groups per CU (a 2-slot ring) keep four-wave work-groups (64 rows
// in two key slices, or 128 rows in one) within 256 registers per lane.
// FP8: the cache holds OCP e4m3 codes with one power-of-two scale per (row,
// KV head).  Cache tiles stream into the ring as codes and scales (half the
// bytes); once a tile has landed the work-group decodes it into a bf16 tile
// buffer (one of two; one alone with a 2-slot ring) -- code x scale is exact
// in bf16 -- and the tile is then computed exactly as a bf16 one.  The block
// rows arrive as bf16 and go straight into a tile buffer.
template <int D, int NR, int KS, int NSTAGE, int NPRE, bool PAGED, bool QLDS, bool FP8>
__global__ void __launch_bounds__(64 * NR * KS, (NR * KS == 4 && NSTAGE == 2) ? 2 : 1)
attn_bf16_kernel(AttnParams p)
{
    constexpr int NW = NR * KS;
    constexpr int GPR = D / 8;                 // 16-byte granules per K row
    constexpr int GPRV = D / 8;                // 16-byte granules per V row
    constexpr int RPCK = 64 / GPR;             // K rows per 1 KiB chunk
    constexpr int RPCV = 64 / GPRV;            // V rows per 1 KiB chunk
    constexpr int CK = TK / RPCK;              // K chunks per tile
    constexpr int CV = TK / RPCV;              // V chunks per tile
    constexpr int K_BYTES = TK * D * 2;
    constexpr int V_BYTES = TK * D * 2;
    constexpr int SLOT = K_BYTES + V_BYTES;
    constexpr int KPW = TK / KS;               // keys per wave per tile
    constexpr int NBLK = KPW / 32;             // S^T 32x32 blocks per wave
    constexpr int NDT = D / 32;                // O^T tiles
    constexpr int QROWS = 32 * NR;
    constexpr int Q_BYTES = QLDS ? QROWS * D * 2 : 0;
    constexpr int CQ = Q_BYTES / 1024;         // query chunks
    // paged: the query tile borrows ring slot NSTAGE-1 (the page ids take the
    // room a separate query buffer would need); contiguous: its own buffer
    constexpr bool QSLOT = QLDS && PAGED;
    constexpr int Q_EXTRA = QSLOT ? 0 : Q_BYTES;
    static_assert(!QSLOT || Q_BYTES <= SLOT, "the query tile fits one ring slot");
    static_assert(KPW % 32 == 0, "each wave needs whole 32-key blocks");
    static_assert(CK % NW == 0 && CV % NW == 0 && CQ % NW == 0, "chunks must split evenly");
    static_assert(NPRE >= 1 && NPRE < NSTAGE, "prefetch depth");
    constexpr int LK = CK / NW, LV = CV / NW, LQ = CQ / NW;
    // FP8 ring slots: K codes (TK x D bytes), V codes, then 64 K and 64 V
    // scales (fp32); each wave moves one share of the scales with 4-byte DMAs
    static_assert(!FP8 || (D == 128 && !QLDS && NSTAGE == NPRE + 1), "fp8 layout");
    constexpr int K8_BYTES = TK * D, V8_BYTES = TK * D;
    constexpr int SC_OFF = K8_BYTES + V8_BYTES;
    constexpr int SLOT8 = SC_OFF + 1024;                  // 512 B of scales, 1 KiB aligned
    constexpr int LK8 = K8_BYTES / 1024 / NW, LV8 = V8_BYTES / 1024 / NW;
    constexpr int SC_LANES = 2 * TK / NW;                 // scale dwords per wave
    static_assert(!FP8 || (LK8 * NW * 1024 == K8_BYTES && SC_LANES <= 64), "fp8 chunks");
    constexpr int LPT = FP8 ? LK8 + LV8 + 1 : LK + LV;   // DMA loads per cache tile per lane
    static_assert(LPT * (NPRE + 1) + LQ <= 63, "vmcnt range");
    // Lazy rescaling: the running max only moves when a tile's max exceeds
    // it by more than 2^kLazy in exp2 units (weights stay <= 2^kLazy).
    constexpr float kLazy = 8.0f;

    constexpr int PAGE_BYTES = PAGED ? kMaxSplitPages * 4 : 0;
    constexpr int RING = FP8 ? NSTAGE * SLOT8 : NSTAGE * SLOT;
    constexpr int BF_OFF = RING;                          // FP8: two bf16 tile buffers
    // FP8: two decoded tile buffers (decode of tile t+1 may start while other
    // waves still read tile t), or one with a 2-slot ring, so that two
    // work-groups of up to four waves share a CU (66 KiB each)
    constexpr int FP8_BUFS = NSTAGE == 2 ? 1 : 2;
    constexpr int BF_BYTES = FP8 ? FP8_BUFS * SLOT : 0;
    constexpr int LDS_TOTAL = RING + BF_BYTES + Q_EXTRA + PAGE_BYTES;
    __shared__ __attribute__((aligned(1024))) char smem[LDS_TOTAL];
    int* s_pages = reinterpret_cast<int*>(smem + RING + BF_BYTES + Q_EXTRA);   // PAGED only
    constexpr int Q_OFF = QSLOT ? (NSTAGE - 1) * SLOT : RING + BF_BYTES;
    // LDS of tile t's bf16 K and V (the ring slot, or FP8's decoded buffer)
    auto tile_lds = [&](int t) __attribute__((always_inline)) -> char* {
        return FP8 ? smem + BF_OFF + (FP8_BUFS == 2 ? (t & 1) * SLOT : 0)
                   : smem + (t % NSTAGE) * SLOT;
    };

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int rg = wave % NR;      // row group
    const int kg = wave / NR;      // key slice
    const int BH = p.B * p.Hkv;
    int bh = blockIdx.x % BH;
    int s = blockIdx.x / BH;
    if (!PAGED && p.reverse) bh = BH - 1 - bh;
    if (PAGED && p.lpt) {             // longest-first work list
        int bi, si;
        if (!lpt_item(p, blockIdx.x / p.Hkv, lane, bi, si)) return;
        bh = bi * p.Hkv + blockIdx.x % p.Hkv;
        s = si;
    }
    const int b = bh / p.Hkv;
    const int g = bh % p.Hkv;
    const int rb = blockIdx.y;        // row block
    const int kbeg = s * p.SL;

    // ---- query rows: lane column q = lane % 32 of row group rg ----
    const int half = lane >> 5;
    const int r = rb * QROWS + rg * 32 + (lane & 31);
    const bool row_ok = r < p.M;
    const int hl = row_ok ? r / p.K : 0;
    const int qi = row_ok ? r % p.K : 0;
    const int h = g * p.G + hl;
    const uint32_t lds_base = (uint32_t)(uintptr_t)(ORTHRUS_LDS void*)&smem[0];
    const uint32_t q_lds = lds_base + Q_OFF;
    bf16x8 qreg[D / 16];
    if constexpr (QLDS) {
        // DMA the query tile (rows XOR-swizzled like K) ahead of the K/V ring
#pragma unroll
        for (int i = 0; i < LQ; ++i) {
            const int cc = i * NW + wave;
            const int row = cc * RPCK + lane / GPR;
            const int rr = rb * QROWS + row;
            const int rq = rr < p.M ? rr : 0;
            const int gr = (lane % GPR) ^ (row & (GPR - 1));
            const char* src = (const char*)p.q +
                ((((int64_t)b * p.K + rq % p.K) * p.Hq + g * p.G + rq / p.K) * D + gr * 8) * 2;
            lds_dma16(src, q_lds + cc * 1024);
        }
    } else {
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
    constexpr int ESZ = FP8 ? 1 : 2;                      // bytes per cache element
    const int64_t cont_row0 = ((int64_t)(b / p.nbps) * p.Hkv + g) * p.cap;   // first cache row
    const int64_t cont_base = cont_row0 * D * ESZ;                          // bytes
    const int64_t blk_base = ((int64_t)b * p.K * p.Hkv + g) * D * 2;
    const int blk_stride = p.Hkv * D * 2;
    // Load i of a tile by this lane (K chunks first, then V): the tile row it
    // reads, the byte offset of its (swizzled) 16-byte granule in that row,
    // and the LDS byte offset of its 1 KiB chunk within a ring slot.
    // Recomputed where used (no per-lane arrays, which could land in scratch).
    auto lrow = [&](int i) __attribute__((always_inline)) {
        return i < LK ? (i * NW + wave) * RPCK + lane / GPR
                      : ((i - LK) * NW + wave) * RPCV + lane / GPRV;
    };
    auto loff = [&](int i) __attribute__((always_inline)) -> uint32_t {
        const int row = lrow(i);
        return i < LK ? 16u * (uint32_t)((lane % GPR) ^ (row & (GPR - 1)))
                      : 16u * (uint32_t)((lane % GPRV) ^ (2 * (row & 3)));
    };
    auto ldst = [&](int i) __attribute__((always_inline)) -> uint32_t {
        return i < LK ? (uint32_t)((i * NW + wave) * 1024)
                      : (uint32_t)(K_BYTES + ((i - LK) * NW + wave) * 1024);
    };

    // Key range of this split: needs lens[b], which is read after the first
    // loads are in flight (contiguous layout: the split's nominal tiles are
    // fetched speculatively, rows clamped to the capacity).
    int kend = kbeg + p.SL;
    int n_cache_tiles = 0;
    int last_issued = -1;      // highest tile index of the true sequence issued so far

    constexpr int LPT16 = LK + LV;              // DMA loads per bf16 tile per lane
    // FP8 cache tile t (rows start..start+count-1): codes and scales into ring
    // slot t % NSTAGE.  Chunk i of the codes: 8 rows of 128 bytes, lane l on
    // row 8*(i*NW + wave) + l/8, bytes 16*(l%8); scales: dword q = the wave's
    // share, K scales of keys 0..63 then V scales (rows clamped to count-1).
    auto issue_rows8 = [&](int t, int start, int count) __attribute__((always_inline)) {
        const uint32_t slot_lds = lds_base + (uint32_t)((t % NSTAGE) * SLOT8);
#pragma unroll
        for (int i = 0; i < LK8 + LV8; ++i) {
            const bool isv = i >= LK8;
            const int cc = (isv ? i - LK8 : i) * NW + wave;
            const int row = cc * 8 + lane / 8;
            const int rowc = row < count ? row : count - 1;
            const char* base = isv ? vc : kc;
            const char* src;
            if constexpr (PAGED) {
                const int key = start + rowc;
                const int page = s_pages[(key - kbeg) >> 4];
                src = base + (((int64_t)page * p.Hkv + g) * 16 + (key & 15)) * D;
            } else {
                src = base + cont_base + (int64_t)(start + rowc) * D;
            }
            lds_dma16(src + 16 * (lane % 8), slot_lds + (isv ? K8_BYTES : 0) + cc * 1024);
        }
        if (lane < SC_LANES) {
            const int q = wave * SC_LANES + lane;     // 0..127
            const int key = q & (TK - 1);
            const int rowc = key < count ? key : count - 1;
            const float* sc = q < TK ? p.ks : p.vs;
            int64_t e;
            if constexpr (PAGED) {
                const int kk = start + rowc;
                const int page = s_pages[(kk - kbeg) >> 4];
                e = ((int64_t)page * p.Hkv + g) * 16 + (kk & 15);
            } else {
                e = cont_row0 + start + rowc;
            }
            lds_dma4(sc + e, slot_lds + SC_OFF + (uint32_t)(wave * SC_LANES) * 4);
        }
    };
    // issue the global->LDS loads of tile t (rows start..start+count-1 of the
    // cache, or the block rows) into ring slot t % NSTAGE (FP8: cache tiles
    // as codes, the bf16 block rows into tile buffer t & 1)
    auto issue_rows = [&](int t, bool is_blk, int start, int count) __attribute__((always_inline)) {
        if constexpr (FP8) {
            if (!is_blk) {
                issue_rows8(t, start, count);
                return;
            }
        }
        const uint32_t slot_lds = lds_base + (uint32_t)(tile_lds(t) - smem);
        if (!is_blk && !PAGED && count == TK) {
            // fast path: a full contiguous tile, rows D*2 bytes apart
            const char* kt = kc + cont_base + (int64_t)start * D * 2;
            const char* vt = vc + cont_base + (int64_t)start * D * 2;
            // 256-row work-groups (at the register limit) take the SADDR form,
            // which needs no per-lane 64-bit address: 179-181 vs 184 us at
            // 131,072 keys, K = 64; the others were 1% faster without it
#pragma unroll
            for (int i = 0; i < LPT16; ++i) {
                if constexpr (NR * 32 > 128)
                    lds_dma16_s(i >= LK ? vt : kt, (uint32_t)(lrow(i) * D * 2) + loff(i),
                                slot_lds + ldst(i));
                else
                    lds_dma16((i >= LK ? vt : kt) + (uint32_t)(lrow(i) * D * 2) + loff(i),
                              slot_lds + ldst(i));
            }
        } else if (!is_blk && PAGED && count == TK) {
            // full paged tile: 4 pages of 16 rows
            const int pidx = (start - kbeg) >> 4;
#pragma unroll
            for (int i = 0; i < LPT16; ++i) {
                const int page = s_pages[pidx + (lrow(i) >> 4)];
                const char* base = (i >= LK ? vc : kc) + ((int64_t)page * p.Hkv + g) * (16 * D * 2);
                lds_dma16(base + (uint32_t)((lrow(i) & 15) * D * 2) + loff(i), slot_lds + ldst(i));
            }
        } else {
            // partial cache tile or the block tile: clamp rows to count-1
#pragma unroll
            for (int i = 0; i < LPT16; ++i) {
                const bool isv = i >= LK;
                const int rowc = lrow(i) < count ? lrow(i) : count - 1;
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
                lds_dma16(src + loff(i), slot_lds + ldst(i));
            }
        }
    };
    auto issue = [&](int t) __attribute__((always_inline)) {
        const bool is_blk = t >= n_cache_tiles;
        const int start = is_blk ? 0 : kbeg + t * TK;
        const int count = is_blk ? p.K : (kend - start < TK ? kend - start : TK);
        issue_rows(t, is_blk, start, count);
        last_issued = t > last_issued ? t : last_issued;
    };

    // wait until at most `pending` later tiles of this lane are in flight
    auto wait_tiles = [&](int pending) __attribute__((always_inline)) {
        switch (pending) {
            case 0: __builtin_amdgcn_s_waitcnt(vmcnt_encode(0)); break;
            case 1: __builtin_amdgcn_s_waitcnt(vmcnt_encode(LPT)); break;
            case 2: __builtin_amdgcn_s_waitcnt(vmcnt_encode(2 * LPT)); break;
            case 3: __builtin_amdgcn_s_waitcnt(vmcnt_encode(3 * LPT)); break;
            default: __builtin_amdgcn_s_waitcnt(vmcnt_encode(4 * LPT)); break;
        }
    };
    static_assert(NPRE <= 4, "wait_tiles covers up to 4 pending tiles");
    static_assert(!QSLOT || NPRE <= NSTAGE - 2, "the query slot must not be in the prologue");

    // ---- prologue: NPRE tiles in flight; iteration t issues tile t + NPRE
    // into the slot of an already consumed tile (NPRE < NSTAGE) ----
    int spec = 0;   // speculative cache tiles issued before lens[b] is known
    if constexpr (!PAGED) {
        const int64_t nominal_end = (int64_t)kbeg + p.SL < p.cap ? (int64_t)kbeg + p.SL : p.cap;
        const int nom = nominal_end > kbeg ? (int)((nominal_end - kbeg + TK - 1) / TK) : 0;
        spec = nom < NPRE ? nom : NPRE;
        for (int t = 0; t < spec; ++t) {
            const int start = kbeg + t * TK;
            const int64_t inb = p.cap - start;     // in-bounds rows of this tile
            issue_rows(t, false, start, inb < TK ? (int)inb : TK);
        }
    }
    // lens[b] through the scalar unit: a vector load would only return after
    // every DMA issued above (vector loads complete in order)
    const int L = ((const __attribute__((address_space(4))) int32_t*)p.lens)[b];
    int S_b = (L + p.SL - 1) / p.SL;
    S_b = S_b < 1 ? 1 : (S_b > p.S_grid ? p.S_grid : S_b);
    if (s >= S_b) {                       // no keys for this split: drain the DMA, exit
        __builtin_amdgcn_s_waitcnt(vmcnt_encode(0));
        return;
    }
    const bool last = (s == S_b - 1);
    kend = last ? L : kbeg + p.SL;
    n_cache_tiles = (kend - kbeg + TK - 1) / TK;
    const int n_tiles = n_cache_tiles + (last ? 1 : 0);   // K <= 64 = TK
    if (spec > n_cache_tiles) {
        // a short last split: speculative tiles past its end are discarded;
        // drain them before their slots take the block tile
        __builtin_amdgcn_s_waitcnt(vmcnt_encode(0));
        spec = n_cache_tiles;
    }
    last_issued = spec - 1;
    if constexpr (PAGED) {   // page ids of this split
        const int pg0 = kbeg / 16;
        const int npg = (kend - kbeg + 15) / 16;
        for (int i = tid; i < npg; i += 64 * NW)
            s_pages[i] = p.page_table[(int64_t)b * p.maxp + pg0 + i];
        __syncthreads();
    }
    // FP8: the prologue issues cache tiles only; the block tile follows the
    // last cache tile's arrival (its tile buffer is then free), or comes
    // first when the split has no cache rows
    const int n_pro = FP8 && n_cache_tiles > 0 ? n_cache_tiles : n_tiles;
    for (int t = spec; t < NPRE && t < n_pro; ++t) issue(t);

    f32x16 oacc[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) oacc[i] = f32x16{};
    f32x16 lacc = f32x16{};    // row sums of the bf16 weights (ones x P^T on the MFMA)
    float m_run = -INFINITY;   // running max of raw scores (this lane's query)
    const float c = p.c;       // scale * log2(e)
    const float lazy_raw = kLazy / c;
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});

    // Tile t's scores: S^T = K Q^T for this wave's key slice of ring slot t.
    auto qk = [&](int t, f32x16 (&sacc)[NBLK]) {
        const char* Ks = tile_lds(t);
        // operand reads first, then the MFMAs; with two 32-key blocks per wave
        // (64 keys) in halves of D, to stay within the register budget
        constexpr int KCH = NBLK > 1 ? 2 : 1;
        constexpr int DSC = D / 16 / KCH;
#pragma unroll
        for (int kb = 0; kb < NBLK; ++kb) {
            const int krow = kg * KPW + kb * 32 + (lane & 31);
            sacc[kb] = f32x16{};
#pragma unroll
            for (int ch = 0; ch < KCH; ++ch) {
                u32x4 kf[DSC];
#pragma unroll
                for (int j = 0; j < DSC; ++j) {
                    const int ds = ch * DSC + j;
                    const int lgr = (2 * ds + half) ^ (krow & (GPR - 1));
                    kf[j] = *(const u32x4*)(Ks + krow * D * 2 + lgr * 16);
                }
#pragma unroll
                for (int j = 0; j < DSC; ++j)
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, kf[j]), qreg[ch * DSC + j], sacc[kb], 0, 0, 0);
            }
        }
    };
    // wait for this lane's loads of tile t (and, for t = 0, the query tile
    // issued before it), make everyone's visible, and keep the ring full.
    // Tiles are issued in index order, so last_issued - t tiles may still
    // fly.  arrive(t) comes after every wave has issued its P V of tile t-1,
    // whose operands are then in registers, so the refill (tile t + NPRE)
    // may take the slot of tile t-1 (NSTAGE = NPRE + 1).
    static_assert(NSTAGE >= NPRE + 1, "ring slots for the tiles in flight");
    // FP8: decode cache tile t (landed in ring slot t % NSTAGE) into its bf16
    // tile buffer, in the swizzled layouts the K and V reads expect.  A job is
    // 16 codes of one row of K or V: two codes at a time to fp32 (exact,
    // subnormal codes included), times the row's power-of-two scale (exact),
    // to bf16 (exact: at most 4 significant bits).  The scaled fp8 -> bf16
    // conversion instruction would do it in one step, but on this chip it
    // loses the low mantissa bit of the code (odd codes decode as the even
    // code below them).
    auto decode = [&](int t) __attribute__((always_inline)) {
        if constexpr (FP8) {
            const char* src = smem + (t % NSTAGE) * SLOT8;
            char* dst = tile_lds(t);
            constexpr int JOBS = 2 * TK * (D / 16) / (64 * NW);
#pragma unroll
            for (int jj = 0; jj < JOBS; ++jj) {
                const int jb = tid + 64 * NW * jj;
                const int isv = jb / (TK * (D / 16));
                const int r = (jb / (D / 16)) % TK;
                const int u = jb % (D / 16);
                const u32x4 code = *(const u32x4*)(src + isv * K8_BYTES + r * D + 16 * u);
                const float sc = *(const float*)(src + SC_OFF + 4 * (isv * TK + r));
                u32x4 lo, hi;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const f32x2 fa = __builtin_amdgcn_cvt_pk_f32_fp8(code[w], false);
                    const f32x2 fb = __builtin_amdgcn_cvt_pk_f32_fp8(code[w], true);
                    const uint32_t a = pack_bf16x2(fa[0] * sc, fa[1] * sc);
                    const uint32_t bb = pack_bf16x2(fb[0] * sc, fb[1] * sc);
                    if (w < 2) { lo[2 * w] = a; lo[2 * w + 1] = bb; }
                    else { hi[2 * (w - 2)] = a; hi[2 * (w - 2) + 1] = bb; }
                }
                const int g0 = 2 * u, g1 = 2 * u + 1;
                const int s0 = isv ? g0 ^ (2 * (r & 3)) : g0 ^ (r & (GPR - 1));
                const int s1 = isv ? g1 ^ (2 * (r & 3)) : g1 ^ (r & (GPR - 1));
                char* row = dst + isv * K_BYTES + r * D * 2;
                *(u32x4*)(row + 16 * s0) = lo;
                *(u32x4*)(row + 16 * s1) = hi;
            }
        }
    };
    auto arrive = [&](int t) __attribute__((always_inline)) {
        wait_tiles(last_issued - t);
        __syncthreads();
        if constexpr (FP8) {
            if (t + NPRE < n_cache_tiles) issue(t + NPRE);
            if constexpr (FP8_BUFS == 2) {
                if (t + 1 == n_cache_tiles && t + 1 < n_tiles) issue(t + 1);   // the block tile
            } else if (t == n_cache_tiles && t > 0) {
                // one buffer: the block rows go in once the last cache tile
                // has been computed (every wave is past the barrier above)
                issue(t);
                __builtin_amdgcn_s_waitcnt(vmcnt_encode(0));
                __syncthreads();
            }
            if (t < n_cache_tiles) {
                decode(t);
                __syncthreads();
            }
        } else {
            if (t + NPRE < n_tiles) issue(t + NPRE);
        }
    };

    arrive(0);
    if constexpr (QLDS) {
        // in ring slot NSTAGE-1 it is first overwritten by tile NSTAGE-1, issued
        // after a barrier that every wave passes once it has read its query rows
        const char* Qs = smem + Q_OFF + rg * 32 * D * 2;
        const int qrow = lane & 31;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
            const int gr = (2 * ds + half) ^ ((rg * 32 + qrow) & (GPR - 1));
            u32x4 v = *(const u32x4*)(Qs + qrow * D * 2 + gr * 16);
            if (!row_ok) v = u32x4{0, 0, 0, 0};
            qreg[ds] = __builtin_bit_cast(bf16x8, v);
        }
    }
    f32x16 scur[NBLK];
    qk(0, scur);

    // A key slice that holds none of the K block rows (K <= 32 with two
    // slices) would only add zero weights for the block tile: its waves stop
    // before that tile (the last one; they still pass its arrival barrier),
    // which leaves the SIMD to the other slice on the last split's critical
    // path.
    // One tile: mask, online softmax, P V.  Force-inlined, so that the steady
    // loop below gets it with the full-tile arguments folded in.
    auto tile = [&](int t, const uint16_t* Vs, bool is_blk, int count)
        __attribute__((always_inline)) {
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
                    if (!ok) scur[kb][i] = -INFINITY;
                }
        }

        // ---- online softmax (row = this lane's query column) ----
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NBLK; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, scur[kb][i]);
        {
            auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        if (__any(mx > m_run + lazy_raw)) {
            const float m_new = fmaxf(m_run, mx);
            const float corr = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * c);
            m_run = m_new;
            lacc *= corr;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= corr;
        }
        const float mc = (m_run == -INFINITY) ? 0.f : m_run * c;
        bf16x8 pb[NBLK][2];
#pragma unroll
        for (int kb = 0; kb < NBLK; ++kb)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                f32x2 pv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pv[j][0] = __builtin_amdgcn_exp2f(__builtin_fmaf(scur[kb][8 * hh + 2 * j], c, -mc));
                    pv[j][1] = __builtin_amdgcn_exp2f(__builtin_fmaf(scur[kb][8 * hh + 2 * j + 1], c, -mc));
                }
                const bf16x2 q0 = __builtin_convertvector(pv[0], bf16x2);
                const bf16x2 q1 = __builtin_convertvector(pv[1], bf16x2);
                const bf16x2 q2 = __builtin_convertvector(pv[2], bf16x2);
                const bf16x2 q3 = __builtin_convertvector(pv[3], bf16x2);
                pb[kb][hh] = bf16x8{q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
            }

        // ---- O^T += V^T P^T; row sums: (ones) P^T, from the same bf16 weights,
        // so the output is an exact convex combination of V rows ----
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
                lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pb[kb][hh], lacc, 0, 0, 0);
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, vf[dt]), pb[kb][hh], oacc[dt], 0, 0, 0);
            }
    };

    const int n_loop = n_tiles - ((KS > 1 && last && kg * KPW >= p.K) ? 1 : 0);
    // Steady state first: full cache tiles whose refill is a full cache tile
    // too.  Every test of the general loop below (partial or block tile, mask,
    // tiles left to issue, how many may still fly) is then known, and its
    // scalar branches leave the per-tile instruction stream.
    const int n_full = (kend - kbeg) / TK;
    const int n_fast = n_full - 1 - NPRE > 0 ? n_full - 1 - NPRE : 0;
    int t = 0;
    for (; t < n_fast; ++t) {
        tile(t, (const uint16_t*)(tile_lds(t) + K_BYTES), false, TK);
        // arrive(t + 1): NPRE - 1 later tiles may fly; refill tile t + 1 + NPRE
        __builtin_amdgcn_s_waitcnt(vmcnt_encode((NPRE - 1) * LPT));
        __syncthreads();
        issue_rows(t + 1 + NPRE, false, kbeg + (t + 1 + NPRE) * TK, TK);
        last_issued = t + 1 + NPRE;
        if constexpr (FP8) {
            decode(t + 1);
            __syncthreads();
        }
        qk(t + 1, scur);
    }
    for (; t < n_loop; ++t) {

        const uint16_t* Vs = (const uint16_t*)(tile_lds(t) + K_BYTES);
        const bool is_blk = t >= n_cache_tiles;
        const int start = is_blk ? 0 : kbeg + t * TK;
        const int count = is_blk ? p.K : (kend - start < TK ? kend - start : TK);

        tile(t, Vs, is_blk, count);
        // Only now wait for the next tile: everything this tile allows is
        // issued, so after the last tile lands only its own work remains.  Its
        // scores go to the matrix cores behind this tile's P V.
        if (t + 1 < n_tiles) {
            arrive(t + 1);
            if (t + 1 < n_loop) qk(t + 1, scur);
        }
    }
    float l_run = lacc[0];     // every row of ones x P^T holds the query's sum

    // ---- merge the two key slices of one row group (KS = 2) ----
    // Each slice finalizes half of the D tiles: it hands the other half of
    // its accumulators (and its m, l) to the other slice through LDS and
    // takes the other slice's accumulators for its own half.
    constexpr int HALF_DT = KS > 1 ? NDT / 2 : NDT;
    // does this wave write D tile dt of the result?
    auto owns = [&](int dt) __attribute__((always_inline)) { return KS == 1 || ((dt < HALF_DT) == (kg == 0)); };
    if constexpr (KS > 1) {
        static_assert(KS == 2 && NDT % 2 == 0, "two key slices, even number of D tiles");
        constexpr int REC = HALF_DT * 16 + 4;             // floats per lane record
        static_assert(NR * 2 * 64 * REC * 4 <= RING + BF_BYTES, "merge buffer");
        __builtin_amdgcn_s_waitcnt(vmcnt_encode(0));
        __syncthreads();   // all waves are done with the ring; reuse it
        float* base = reinterpret_cast<float*>(smem) + rg * 2 * 64 * REC;
        float* mine = base + (kg * 64 + lane) * REC;
        const float* other = base + ((1 - kg) * 64 + lane) * REC;
        auto put = [&](int dt0) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < HALF_DT; ++j)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4)
                    *(f32x4*)(mine + j * 16 + 4 * i4) =
                        f32x4{oacc[dt0 + j][4 * i4], oacc[dt0 + j][4 * i4 + 1],
                              oacc[dt0 + j][4 * i4 + 2], oacc[dt0 + j][4 * i4 + 3]};
        };
        if (kg == 0) put(HALF_DT); else put(0);
        *(f32x4*)(mine + HALF_DT * 16) = f32x4{m_run, l_run, 0.f, 0.f};
        __syncthreads();
        const f32x4 ml = *(const f32x4*)(other + HALF_DT * 16);
        const float m_o = ml[0], l_o = ml[1];
        const float m_t = fmaxf(m_run, m_o);
        const float a0 = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_run - m_t) * c);
        const float a1 = (m_o == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_o - m_t) * c);
        auto take = [&](int dt0) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < HALF_DT; ++j)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const f32x4 v = *(const f32x4*)(other + j * 16 + 4 * i4);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        oacc[dt0 + j][4 * i4 + e] = oacc[dt0 + j][4 * i4 + e] * a0 + v[e] * a1;
                }
        };
        if (kg == 0) take(0); else take(HALF_DT);
        l_run = l_run * a0 + l_o * a1;
        m_run = m_t;
    }

    // ---- finalize: lane owns query row r, columns 32dt + 8(i/4) + 4*half + i%4 ----
    const float inv = 1.f / l_run;
    // Paged batches are ragged: a request with a single split writes its rows
    // directly (the merge skips it).  Contiguous launches keep one epilogue
    // per grid (measured faster at the benchmark shape).
    if (PAGED ? S_b > 1 : p.S_grid > 1) {
        // split partial, stored in fragment order: each store is 512
        // contiguous bytes per wave; base-2 lse per row.  Written through the
        // L2 (the merge launch reads them; 0.75 us less per layer pass at
        // 8,192 keys x 32 rows than stores left for the end-of-launch
        // write-back).  Row groups past Mpad (M not a multiple of the row
        // block) hold no rows.
        if (rb * QROWS + rg * 32 < p.Mpad) {
            uint16_t* blk = (uint16_t*)p.ws_o + ((int64_t)bh * p.S_grid + s) * p.Mpad * D;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                if (owns(dt))
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int i0 = 4 * q4;
                    const int64_t off = frag_offset(r, 32 * dt + 8 * q4 + 4 * half, D);
                    store_through(blk + off,
                        u32x2{pack_bf16x2(oacc[dt][i0] * inv, oacc[dt][i0 + 1] * inv),
                              pack_bf16x2(oacc[dt][i0 + 2] * inv, oacc[dt][i0 + 3] * inv)});
                }
            if (row_ok && half == 0 && kg == 0)
                store_through(p.ws_lse + ((int64_t)bh * p.S_grid + s) * p.Mpad + r,
                              m_run * c + __builtin_log2f(l_run));
        }
        return;
    }
    // No merge for these rows: stage them in
    // LDS ([row][D] with a 16-byte pad) so that the output stores are whole
    // 16-byte pieces of rows.
    constexpr int RSTR = D * 2 + 16;                        // staged row stride, bytes
    static_assert(QROWS * RSTR <= RING + BF_BYTES, "staging buffer");
    __builtin_amdgcn_s_waitcnt(vmcnt_encode(0));
    __syncthreads();                                        // ring (or merge buffer) free
    char* stage = smem;
    {
        char* my = stage + (rg * 32 + (lane & 31)) * RSTR + 8 * half;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
            if (owns(dt))
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int i0 = 4 * q4;
                *(u32x2*)(my + (32 * dt + 8 * q4) * 2) =
                    u32x2{pack_bf16x2(oacc[dt][i0] * inv, oacc[dt][i0 + 1] * inv),
                          pack_bf16x2(oacc[dt][i0 + 2] * inv, oacc[dt][i0 + 3] * inv)};
            }
        if (row_ok && half == 0 && kg == 0 && p.lse)
            p.lse[((int64_t)b * p.Hq + h) * p.K + qi] = (m_run * c + __builtin_log2f(l_run)) * kLn2;
    }
    __syncthreads();
    constexpr int PIECES = D * 2 / 16;                      // 16-byte pieces per row
    for (int idx = tid; idx < QROWS * PIECES; idx += 64 * NW) {
        const int row = idx / PIECES;
        const int pc = idx % PIECES;
        const int rr = rb * QROWS + row;
        if (rr >= p.M) continue;
        const u32x4 v = *(const u32x4*)(stage + row * RSTR + pc * 16);
        const int hh_ = g * p.G + rr / p.K;
        uint16_t* dst = (uint16_t*)p.out + (((int64_t)b * p.K + rr % p.K) * p.Hq + hh_) * D;
        *(u32x4*)(dst + pc * 8) = v;
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
    __shared__ __attribute__((aligned(16))) float Qs[ROWS][D];
    __shared__ __attribute__((aligned(16))) float Ps[4][RW][TK];   // per wave: the rows' weights of a tile

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int BH = p.B * p.Hkv;
    const int bh = p.reverse ? BH - 1 - (int)(blockIdx.x % BH) : (int)(blockIdx.x % BH);
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
    // tile t's K/V values of this thread (element i = tid + 256*e of the
    // 64 x D tile), loaded into registers one tile ahead of the compute
    constexpr int E = TK * D / 256;
    float kr[E], vr[E];
    auto load_tile = [&](int t) __attribute__((always_inline)) {
        const bool is_blk = t >= n_cache_tiles;
        const int start = is_blk ? 0 : kbeg + t * TK;
        const int count = is_blk ? p.K : (kend - start < TK ? kend - start : TK);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = tid + 256 * e;
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
                        off = (((int64_t)(b / p.nbps) * p.Hkv + g) * p.cap + key) * D + d;
                    } else {
                        const int page = p.page_table[(int64_t)b * p.maxp + (key >> 4)];
                        off = (((int64_t)page * p.Hkv + g) * 16 + (key & 15)) * D + d;
                    }
                    kv = kc[off];
                    vv = vc[off];
                }
            }
            kr[e] = kv;
            vr[e] = vv;
        }
    };
    load_tile(0);
    for (int t = 0; t < n_tiles; ++t) {
        const bool is_blk = t >= n_cache_tiles;
        const int start = is_blk ? 0 : kbeg + t * TK;
        const int count = is_blk ? p.K : (kend - start < TK ? kend - start : TK);
        __syncthreads();   // the previous tile's reads of Ks/Vs are done
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int i = tid + 256 * e;
            Ks[i / D][i % D] = kr[e];
            Vs[i / D][i % D] = vr[e];
        }
        if (t + 1 < n_tiles) load_tile(t + 1);   // in flight during this tile's compute
        __syncthreads();
        // scores of the wave's RW rows against key `lane`: one K read feeds
        // RW FMAs, the query values come as broadcast float4 reads
        float sc[RW];
#pragma unroll
        for (int j = 0; j < RW; ++j) sc[j] = 0.f;
#pragma unroll 4
        for (int d = 0; d < D; d += 4) {
            const float k0 = Ks[lane][d], k1 = Ks[lane][d + 1], k2 = Ks[lane][d + 2],
                        k3 = Ks[lane][d + 3];
#pragma unroll
            for (int j = 0; j < RW; ++j) {
                const f32x4 qv = *(const f32x4*)&Qs[wave * RW + j][d];
                sc[j] = __builtin_fmaf(qv[0], k0, sc[j]);
                sc[j] = __builtin_fmaf(qv[1], k1, sc[j]);
                sc[j] = __builtin_fmaf(qv[2], k2, sc[j]);
                sc[j] = __builtin_fmaf(qv[3], k3, sc[j]);
            }
        }
        float corr[RW];
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            const int rr = row0 + wave * RW + j;
            const int qi = rr < p.M ? rr % p.K : 0;
            bool ok = lane < count;
            if (is_blk && p.mask == 1) ok = ok && lane <= qi;
            const float sj = ok ? sc[j] : -INFINITY;
            float mx = sj;
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
            const float m_new = fmaxf(m_run[j], mx);
            corr[j] = (m_run[j] == -INFINITY) ? 0.f : exp2f((m_run[j] - m_new) * c);
            const float pv = ok ? exp2f((sj - m_new) * c) : 0.f;
            m_run[j] = m_new;
            float ps = pv;
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) ps += __shfl_xor(ps, m, 64);
            l_run[j] = l_run[j] * corr[j] + ps;
            Ps[wave][j][lane] = pv;
        }
        __builtin_amdgcn_wave_barrier();
        // O += P V: one V read feeds RW FMAs, the weights come as broadcast
        // float4 reads
#pragma unroll
        for (int k = 0; k < DC; ++k) {
            float acc[RW];
#pragma unroll
            for (int j = 0; j < RW; ++j) acc[j] = o[j][k] * corr[j];
#pragma unroll 4
            for (int key = 0; key < TK; key += 4) {
                const float v0 = Vs[key][lane + 64 * k], v1 = Vs[key + 1][lane + 64 * k],
                            v2 = Vs[key + 2][lane + 64 * k], v3 = Vs[key + 3][lane + 64 * k];
#pragma unroll
                for (int j = 0; j < RW; ++j) {
                    const f32x4 pw = *(const f32x4*)&Ps[wave][j][key];
                    acc[j] = __builtin_fmaf(pw[0], v0, acc[j]);
                    acc[j] = __builtin_fmaf(pw[1], v1, acc[j]);
                    acc[j] = __builtin_fmaf(pw[2], v2, acc[j]);
                    acc[j] = __builtin_fmaf(pw[3], v3, acc[j]);
                }
            }
#pragma unroll
            for (int j = 0; j < RW; ++j) o[j][k] = acc[j];
        }
        __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int j = 0; j < RW; ++j) {
        const int rr = row0 + wave * RW + j;
        if (rr >= p.M) continue;
        const int hl = rr / p.K, qi = rr % p.K;
        const int h = g * p.G + hl;
        const float inv = 1.f / l_run[j];
        const float lse2 = m_run[j] * c + log2f(l_run[j]);
        if (p.layout == 1 ? S_b == 1 : p.S_grid == 1) {   // no merge for these rows
            float* op = (float*)p.out + (((int64_t)b * p.K + qi) * p.Hq + h) * D;
#pragma unroll
            for (int k = 0; k < DC; ++k) op[lane + 64 * k] = o[j][k] * inv;
            if (p.lse && lane == 0) p.lse[((int64_t)b * p.Hq + h) * p.K + qi] = lse2 * kLn2;
        } else {
            float* blk = (float*)p.ws_o + ((int64_t)bh * p.S_grid + s) * p.Mpad * D;
#pragma unroll
            for (int k = 0; k < DC; ++k) store_through(blk + frag_offset(rr, lane + 64 * k, D), o[j][k] * inv);
            if (lane == 0) store_through(p.ws_lse + ((int64_t)bh * p.S_grid + s) * p.Mpad + rr, lse2);
        }
    }
}

// --------------------------------------------------------------------------
// split-KV merge: lse = log sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s
// --------------------------------------------------------------------------
// Partial blocks [B*Hkv][S_grid][Mpad x D] in fragment order (bf16 on the bf16
// path, fp32 on the fp32 path), base-2 lse [B*Hkv][S_grid][Mpad].  A work-group
// covers 32 rows x 16 columns with NG groups of 128 threads: in a group,
// thread = (row q, 4 columns), so 32 consecutive threads read one contiguous
// run of a partial block (and of the lse).  Group g merges its own range of
// about S_grid / NG splits (online log-sum-exp, up to UNROLL loads in flight
// per thread); the groups' (max, sum, O) are then combined through LDS.
// Splitting the splits keeps every SIMD busy and the serial weighting chain
// short when there are many (one group over all 32 splits of the Qwen3-8B
// shape spent 1.5 us in it, after a 2.5 us load round trip); with a few
// splits one group does it, and the grid's many small work-groups start
// sooner (NG = 4 over 3 splits took 18 us instead of 6 on a 32-request paged
// batch).
// SKIP1: paged launches, whose single-split requests were written by the
// attention kernel itself.
template <int D, bool BF16, int UNROLL, bool SKIP1, int NG>
__global__ void __launch_bounds__(128 * NG) attn_merge_kernel(AttnParams p)
{
    const int bh = blockIdx.x;
    const int b = bh / p.Hkv;
    const int g = bh % p.Hkv;
    const int rgrp = blockIdx.y / (D / 16);
    const int cgrp = blockIdx.y % (D / 16);
    const int grp = __builtin_amdgcn_readfirstlane(threadIdx.x >> 7);   // split group
    const int tg = threadIdx.x & 127;
    const int q = tg & 31;
    const int quad = tg >> 5;                          // 0..3: 4 columns each
    const int r = rgrp * 32 + q;
    const int d = cgrp * 16 + quad * 4;
    const bool row_ok = r < p.M;
    const int rr = row_ok ? r : 0;                     // rows past M: read row 0, store nothing
    const float* lse_r = p.ws_lse + (int64_t)bh * p.S_grid * p.Mpad + rr;   // split sp at + sp*Mpad
    const int64_t blk0 = (int64_t)bh * p.S_grid * p.Mpad * D + frag_offset(rr, d, D);
    const int64_t bstride = (int64_t)p.Mpad * D;
    const int spg = (p.S_grid + NG - 1) / NG;    // splits per group
    const int s_lo = grp * spg;
    auto part = [&](int sp) __attribute__((always_inline)) -> f32x4 {
        if (BF16) {
            const u32x2 v = *(const u32x2*)((const uint16_t*)p.ws_o + blk0 + sp * bstride);
            return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u),
                         __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xffff0000u)};
        }
        return *(const f32x4*)((const float*)p.ws_o + blk0 + sp * bstride);
    };
    f32x4 v[UNROLL];
    float l2[UNROLL];
    auto load = [&](int s0) __attribute__((always_inline)) {
        // splits s0.. (clamped into the grid; no branches, so that all loads
        // are in flight together)
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int sp = s0 + u < p.S_grid ? s0 + u : p.S_grid - 1;
            l2[u] = lse_r[(int64_t)sp * p.Mpad];
            v[u] = part(sp);
        }
    };
    // The first chunk does not depend on lens[b] (splits past S_b are read,
    // then discarded): issue it first so that its round trip and the one of
    // lens overlap.
    load(s_lo);
    asm volatile("" ::: "memory");
    const int L = ((const __attribute__((address_space(4))) int32_t*)p.lens)[b];
    int S_b = (L + p.SL - 1) / p.SL;
    S_b = S_b < 1 ? 1 : (S_b > p.S_grid ? p.S_grid : S_b);
    if (SKIP1 && S_b == 1) return;                     // uniform over the work-group
    const int s_hi = s_lo + spg < S_b ? s_lo + spg : S_b;
    float mx = -INFINITY;
    float W = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = s_lo; s0 < s_hi;) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            if (s0 + u >= s_hi) {    // another group's split, or past this request's (stale)
                l2[u] = -INFINITY;
                v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        float gm = l2[0];
#pragma unroll
        for (int u = 1; u < UNROLL; ++u) gm = fmaxf(gm, l2[u]);
        const float m_new = fmaxf(mx, gm);
        const float corr = (mx == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mx - m_new);
        W *= corr;
        acc *= corr;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const float w = __builtin_amdgcn_exp2f(l2[u] - m_new);   // 0 for padding
            W += w;
            acc += w * v[u];
        }
        mx = m_new;
        s0 += UNROLL;
        if (s0 >= s_hi) break;
        load(s0);
    }
    // combine the groups (group 0 holds at least split 0, so its max is finite)
    float mt = mx;
    if constexpr (NG > 1) {
        __shared__ f32x4 s_acc[NG - 1][128];
        __shared__ f32x2 s_mw[NG - 1][128];
        if (grp > 0) {
            s_acc[grp - 1][tg] = acc;
            s_mw[grp - 1][tg] = f32x2{mx, W};
        }
        __syncthreads();
        if (grp > 0) return;
#pragma unroll
        for (int k = 0; k < NG - 1; ++k) mt = fmaxf(mt, s_mw[k][tg][0]);
        const float c0 = __builtin_amdgcn_exp2f(mx - mt);
        W *= c0;
        acc *= c0;
#pragma unroll
        for (int k = 0; k < NG - 1; ++k) {
            const f32x2 mw = s_mw[k][tg];
            const float ck = (mw[0] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw[0] - mt);
            W += ck * mw[1];
            acc += ck * s_acc[k][tg];
        }
    }
    if (!row_ok) return;
    const float inv = 1.f / W;
    const int hl = r / p.K, qi = r % p.K;
    const int h = g * p.G + hl;
    const int64_t oo = (((int64_t)b * p.K + qi) * p.Hq + h) * D + d;
    if (BF16) {
        u32x2 o = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
        *(u32x2*)((uint16_t*)p.out + oo) = o;
    } else {
        *(f32x4*)((float*)p.out + oo) = acc * inv;
    }
    if (p.lse && d == 0) p.lse[((int64_t)b * p.Hq + h) * p.K + qi] = (mt + __builtin_log2f(W)) * kLn2;
}

// --------------------------------------------------------------------------
// launch
// --------------------------------------------------------------------------
// K/V ring slots: as many as fit the 160 KiB of LDS next to the page-id
// staging (paged) or the query tile (contiguous), at most 4.  Two tiles fly
// ahead of the one computed (below), so a third slot is all the ring needs;
// a power of two keeps the slot base a shift, which lets every LDS operand
// read be one lane offset plus an immediate.  With 5 slots the compiler kept
// one precomputed offset per read and two adds per read per tile (96 VALU
// instructions per tile in the 256-row work-group, 40 registers, and spills).
constexpr int ring_depth(int D, int NR, bool paged, bool qlds) {
    const int slot = 64 * D * 2 * 2;
    const int extra = paged ? kMaxSplitPages * 4 : (qlds ? 32 * NR * D * 2 : 0);
    const int n = (163840 - extra) / slot;
    return n > 4 ? 4 : n;
}
// Tiles in flight ahead of the one computed: 2 (with every CU streaming, a
// deeper queue delays the first tiles more than it speeds up the last),
// NSTAGE - 2 when the query tile sits in the last slot (it is read after the
// first refill could be issued otherwise), within the DMA counter range.
constexpr int prefetch_depth(int D, int NR, int KS, int nstage, bool qslot) {
    const int lpt = (D / 8 + D / 8) / (NR * KS);
    const int lq = 32 * NR * D * 2 / 1024 / (NR * KS);
    int np = qslot ? nstage - 2 : nstage - 1;
    np = np > 2 ? 2 : np;
    while (np > 1 && lpt * (np + 1) + lq > 63) --np;
    return np;
}

template <int D, int NR, int KS, bool QLDS>
static hipError_t launch_bf16(const AttnParams& p, hipStream_t st) {
    dim3 grid(p.S_grid * p.B * p.Hkv, p.row_blocks);
    dim3 block(64 * NR * KS);
    if (p.layout == 1) {
        constexpr int NS = ring_depth(D, NR, true, QLDS);
        constexpr int NP = prefetch_depth(D, NR, KS, NS, QLDS);
        hipLaunchKernelGGL((attn_bf16_kernel<D, NR, KS, NS, NP, true, QLDS, false>), grid, block, 0, st, p);
    } else if ((NR <= 2 && (NR == 2 || (int64_t)grid.x * grid.y > 256)) || (NR == 4 && KS == 1)) {
        // Contiguous 64-row work-groups, and 32-row ones when the grid has
        // more work-groups than CUs: a 2-slot ring, one tile in flight while
        // another is computed, so that two work-groups share a CU and one's
        // start-up and drain overlap the other's streaming (131,072 keys,
        // 64 splits, K = 4 / 8 / 16: 111 -> 98, 116 -> 97, 111 -> 99 us per
        // layer pass; 8,192 keys, K = 16: 15.5 -> 14.8 us).  With at most
        // one 32-row work-group per CU the deep ring is faster (32,768 keys,
        // K = 8: 32.0 vs 36.2 us).  128-row work-groups come here as four
        // waves (KS = 1) when they outnumber the CUs.
        if constexpr (NR <= 2 || (NR == 4 && KS == 1))
            hipLaunchKernelGGL((attn_bf16_kernel<D, NR, KS, 2, 1, false, QLDS, false>), grid, block, 0, st, p);
    } else {
        constexpr int NS = ring_depth(D, NR, false, QLDS);
        constexpr int NP = prefetch_depth(D, NR, KS, NS, false);
        hipLaunchKernelGGL((attn_bf16_kernel<D, NR, KS, NS, NP, false, QLDS, false>), grid, block, 0, st, p);
    }
    return hipGetLastError();
}

// fp8 cache (head_dim 128): the query in registers; the ring and decoded
// buffers by wave count (below)
template <int NR, int KS>
static hipError_t launch_fp8(const AttnParams& p, hipStream_t st) {
    dim3 grid(p.S_grid * p.B * p.Hkv, p.row_blocks);
    dim3 block(64 * NR * KS);
    // up to four waves: a 2-slot ring and one decoded buffer, two work-groups
    // per CU; eight waves: a 3-slot ring, two buffers, one per CU
    constexpr int NS = NR * KS <= 4 ? 2 : 3;
    if (p.layout == 1)
        hipLaunchKernelGGL((attn_bf16_kernel<128, NR, KS, NS, NS - 1, true, false, true>), grid, block, 0, st, p);
    else
        hipLaunchKernelGGL((attn_bf16_kernel<128, NR, KS, NS, NS - 1, false, false, true>), grid, block, 0, st, p);
    return hipGetLastError();
}

template <int D, bool BF16, bool SKIP1>
static void launch_merge_u(const AttnParams& p, dim3 grid, hipStream_t st) {
    if (p.S_grid <= 2)
        hipLaunchKernelGGL((attn_merge_kernel<D, BF16, 2, SKIP1, 1>), grid, dim3(128), 0, st, p);
    else if (p.S_grid <= 4)
        hipLaunchKernelGGL((attn_merge_kernel<D, BF16, 4, SKIP1, 1>), grid, dim3(128), 0, st, p);
    else if (p.S_grid <= 16)   // four groups of up to 4 splits
        hipLaunchKernelGGL((attn_merge_kernel<D, BF16, 4, SKIP1, 4>), grid, dim3(512), 0, st, p);
    else if (p.S_grid <= 32)
        hipLaunchKernelGGL((attn_merge_kernel<D, BF16, 8, SKIP1, 4>), grid, dim3(512), 0, st, p);
    else
        hipLaunchKernelGGL((attn_merge_kernel<D, BF16, 16, SKIP1, 4>), grid, dim3(512), 0, st, p);
}

template <int D, bool BF16>
static void launch_merge(const AttnParams& p, dim3 grid, hipStream_t st) {
    if (p.layout == 1) launch_merge_u<D, BF16, true>(p, grid, st);
    else launch_merge_u<D, BF16, false>(p, grid, st);
}

template <int D>
static hipError_t launch_bf16_d(const AttnParams& p, hipStream_t st) {
    if (p.kv8) {
        if constexpr (D == 128) {
            switch (p.rows_per_wg) {
                case 32: return launch_fp8<1, 2>(p, st);
                case 64: return launch_fp8<2, 2>(p, st);
                case 128:
                    // more contiguous work-groups than CUs: four waves, two per CU
                    if (p.layout == 0 && (int64_t)p.S_grid * p.B * p.Hkv * p.row_blocks > 256)
                        return launch_fp8<4, 1>(p, st);
                    return launch_fp8<4, 2>(p, st);
                default: return launch_fp8<8, 1>(p, st);
            }
        }
        return hipErrorInvalidValue;
    }
    switch (p.rows_per_wg) {
        case 32: return launch_bf16<D, 1, 2, true>(p, st);
        case 64: return launch_bf16<D, 2, 2, true>(p, st);
        case 128:
            // more contiguous work-groups than CUs: four waves each, so that
            // two share a CU (131,072 keys, K = 32, 64 splits: 263 -> 250 us
            // per step, 58 -> 60.5% of HBM peak); the query then lives in
            // VGPRs to leave the LDS to two 2-slot rings
            if (p.layout == 0 && (int64_t)p.S_grid * p.B * p.Hkv * p.row_blocks > 256)
                return launch_bf16<D, 4, 1, false>(p, st);
            return launch_bf16<D, 4, 2, true>(p, st);
        default: return launch_bf16<D, 8, 1, false>(p, st);
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
    dim3 mgrid(p.B * p.Hkv, (p.Mpad / 32) * (p.D / 16));
    if (p.D == 128) {
        if (dtype == 1) launch_merge<128, true>(p, mgrid, st);
        else launch_merge<128, false>(p, mgrid, st);
    } else {
        if (dtype == 1) launch_merge<64, true>(p, mgrid, st);
        else launch_merge<64, false>(p, mgrid, st);
    }
    return hipGetLastError();
}

}  // namespace orthrus
