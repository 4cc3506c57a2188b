// orthrus_block_attn_noalloc: the block attention for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  The split-KV partials live in a fixed
// array of this library on each GPU instead of a caller workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/orthrus.h"

namespace {

// Split partials of one call: 64 MiB covers the partials of every workload of
// the decode step (the largest, 131,072 keys in 64 splits with K = 64 and
// 32 query / 8 KV heads, needs 34 MB).  Each GPU the library runs on holds
// its own copy until the process ends.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_scratch[kMaxDevices];   // device address of `scratch` on each GPU

// The array's device address on the current GPU, looked up once per GPU
// (with that GPU current).  The host-side name `scratch` is not a device
// address; only this pointer is passed to kernels.
int scratch_on_current_device(void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return ORTHRUS_ERR_LAUNCH;
    std::lock_guard<std::mutex> g(g_lock);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return ORTHRUS_ERR_LAUNCH;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return ORTHRUS_OK;
}

}  // namespace

extern "C" {

size_t orthrus_block_attn_noalloc_max_workspace(void) { return kScratchBytes; }

int orthrus_block_attn_noalloc(const orthrus_cache *cache, const void *q, const void *k_blk,
                               const void *v_blk, void *out, float *lse, int B, int K, int Hq,
                               int Hkv, int D, int dtype, int mask, float scale, int num_splits,
                               hipStream_t stream)
{
    if (!cache) return ORTHRUS_ERR_NULL;
    const size_t need =
        orthrus_block_attn_workspace_bytes(cache, B, K, Hq, Hkv, D, dtype, num_splits);
    if (need > kScratchBytes) return ORTHRUS_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0) {
        const int st = scratch_on_current_device(&ws);
        if (st != ORTHRUS_OK) return st;
    }
    return orthrus_block_attn(cache, q, k_blk, v_blk, out, lse, B, K, Hq, Hkv, D, dtype, mask,
                              scale, num_splits, ws, need, stream);
}

}  // extern "C"
