// Shared device helpers for libkvc's gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

constexpr int D = 128;          // head dimension
constexpr int WAVE = 64;        // CDNA wavefront width
constexpr int VT = 32;          // tokens per V tile

// Element offset of value V[t][d] inside one slab.  Values are stored in
// tiles of 32 tokens, each tile channel-major ([d][32]): the 32-token slice
// of all 128 channels is one contiguous 8 KB (bf16) block, and the
// token-contiguous operand of the P*V product is one 16-byte load per lane.
__host__ __device__ __forceinline__ size_t vt_off(int t, int d) {
    return (size_t)(t >> 5) * (D * VT) + (size_t)d * VT + (t & (VT - 1));
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

// bfloat16 bits -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(uint32_t(h) << 16);
}
// Low / high bfloat16 of a packed pair -> float (exact).
// Written as bfloat16 -> float conversions (a shift or a mask in the
// generated code), so the compiler knows the results are canonical floats and
// max / min on them need no extra quieting instruction.
__device__ __forceinline__ float bf16lo(uint32_t w) {
    return (float)__builtin_bit_cast(__bf16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float bf16hi(uint32_t w) {
    return (float)__builtin_bit_cast(__bf16, (uint16_t)(w >> 16));
}

// float -> bfloat16 bits, round to nearest even (hardware convert).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// Non-temporal 16-byte load for data streamed exactly once.
__device__ __forceinline__ u32x4 load_stream16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 load16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

}  // namespace kvc
