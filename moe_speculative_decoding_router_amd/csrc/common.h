// Device helpers shared by the kernels of libmoeverify (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Total order used for every selection: larger value first, then lower index.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// Butterfly reductions: every lane ends with the same bits (each step adds
// the same two operands in every lane of a pair).
__device__ __forceinline__ void wave_argmax(float &v, int &i) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(v, off);
        const int oi = __shfl_xor(i, off);
        if (better(ov, oi, v, i)) {
            v = ov;
            i = oi;
        }
    }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

// float32 -> bf16 bits, round to nearest even (finite input).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float a) {
    uint32_t u = __float_as_uint(a);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Position of activation element (k, column c) in the compact matrix-core
// B-operand layout: per k-step of 32, four lane groups of 8 consecutive k,
// `cols` columns of 8 bf16 (16 bytes) each.  For fp8 weights a 16-byte
// weight load covers 16 consecutive k, split into two k-steps, so k is
// permuted inside each 64-wide block to match.
__device__ __forceinline__ int b_index(int k, int c, int cols, bool fp8) {
    int ks, g;
    if (!fp8) {
        ks = k >> 5;
        g = (k >> 3) & 3;
    } else {
        ks = ((k >> 6) << 1) | ((k >> 3) & 1);
        g = (k >> 4) & 3;
    }
    return ((ks * 4 + g) * cols + c) * 8 + (k & 7);
}

}  // namespace moe
