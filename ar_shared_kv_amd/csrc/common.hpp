// Device helpers shared by the Orthrus HIP kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace orthrus {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;

#define ORTHRUS_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Two fp32 -> packed bf16 (hardware v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// Stores of data that the next launch reads.  A relaxed atomic store at agent
// scope is written through this XCD's L2 (global_store ... sc1), so the data is
// not left dirty there: the L2 write-back that ends a launch, and that the
// next launch waits for, then has little to do.
__device__ __forceinline__ void store_through(void* p, u32x2 v) {
    __hip_atomic_store((uint64_t*)p, __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_through(void* p, f32x4 v) {
    const u32x4 u = __builtin_bit_cast(u32x4, v);
    store_through(p, u32x2{u[0], u[1]});
    store_through((char*)p + 8, u32x2{u[2], u[3]});
}
__device__ __forceinline__ void store_through(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Order-preserving map of a float to uint32 (-0.0 and +0.0 map to the same key).
__device__ __forceinline__ uint32_t float_order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// (value, index) -> 64-bit key whose maximum is the largest value and, among
// equal values, the smallest index.
__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t idx) {
    return ((uint64_t)float_order_key(v) << 32) | (uint64_t)(0xffffffffu - idx);
}

__device__ __forceinline__ uint32_t argmax_key_index(uint64_t key) {
    return 0xffffffffu - (uint32_t)(key & 0xffffffffu);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
    uint32_t lo = __shfl_xor((uint32_t)v, mask, 64);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), mask, 64);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint64_t o = shfl_xor_u64(v, m);
        v = o > v ? o : v;
    }
    return v;
}

}  // namespace orthrus
