// Shared definitions of the gfx950 kernels: compiled shape, vector types,
// bf16/fp16 helpers, and the fixed permutation of K inside 8-element blocks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Compiled layer shape ("Config" table of the qwen35moe forward-pass page).
constexpr int D = 2048;   // n_embd
constexpr int E = 256;    // routed experts
constexpr int K = 8;      // experts used per token
constexpr int F = 512;    // routed expert FF
constexpr int FS = 512;   // shared expert FF
constexpr int G = 64;     // quantisation group
constexpr int WAVE = 64;

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// K order inside every 8-element block of an fp16 operand row.  Position p
// holds element kPerm8[p] = {0,4,1,5,2,6,3,7}[p]: the order in which one u32
// of eight nibbles unpacks into four fp16 pairs (nibbles j and j+4 land in
// one 32-bit lane).  Every fp16 GEMM operand (activations and dequantised
// weights) uses this order, so dot products over K are unchanged.
__host__ __device__ constexpr int perm8_pos(int j) { return j < 4 ? 2 * j : 2 * (j - 4) + 1; }

// Eight bf16 (natural order, 4 dwords) -> eight fp16 in perm8 order.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8_perm(u32x4 v) {
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        f[2 * i] = __uint_as_float(v[i] << 16);
        f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        f16x2 p = {(f16)f[j], (f16)f[j + 4]};
        o[j] = __builtin_bit_cast(uint32_t, p);
    }
    return o;
}

// One u32 of eight 4-bit codes -> eight fp16 weights s*q + b (one rounding,
// fused multiply-add) in perm8 order.  s2, b2 hold the group's scale and
// bias in both halves.
__device__ __forceinline__ u32x4 q4_word_to_f16x8(uint32_t w, f16x2 s2, f16x2 b2) {
    const f16x2 k1024 = {(f16)1024.0f, (f16)1024.0f};
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        // (1024 + q) in each fp16 half: 0x6400 is 1024.0 and the 10-bit
        // mantissa holds the nibble exactly
        uint32_t code = ((w >> (4 * j)) & 0x000f000fu) | 0x64006400u;
        f16x2 q = __builtin_bit_cast(f16x2, code) - k1024;  // exact
        f16x2 r = __builtin_elementwise_fma(q, s2, b2);
        o[j] = __builtin_bit_cast(uint32_t, r);
    }
    return o;
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace moe
