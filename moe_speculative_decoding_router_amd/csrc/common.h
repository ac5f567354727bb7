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

// Wave-wide reductions.  Inside each row of 16 lanes the values are combined
// with DPP row rotations (v op= ror(v, 8), 4, 2, 1), which leaves every lane
// of the row with the row's result; the four row results are then read from
// lanes 0, 16, 32, 48 and combined in row order.  The result is uniform (the
// same bits in every lane) and independent of scheduling.
template <int N>
__device__ __forceinline__ int dpp_ror(int v) {
    return __builtin_amdgcn_update_dpp(0, v, 0x120 + N, 0xF, 0xF, false);
}
template <int N>
__device__ __forceinline__ float dpp_ror(float v) {
    return __int_as_float(dpp_ror<N>(__float_as_int(v)));
}

__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_ror<8>(v);
    v += dpp_ror<4>(v);
    v += dpp_ror<2>(v);
    v += dpp_ror<1>(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return ((r0 + r1) + r2) + r3;
}

__device__ __forceinline__ int wave_sum_int(int v) {
    v += dpp_ror<8>(v);
    v += dpp_ror<4>(v);
    v += dpp_ror<2>(v);
    v += dpp_ror<1>(v);
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
           __builtin_amdgcn_readlane(v, 48);
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_ror<8>(v));
    v = fmaxf(v, dpp_ror<4>(v));
    v = fmaxf(v, dpp_ror<2>(v));
    v = fmaxf(v, dpp_ror<1>(v));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(fmaxf(r0, r1), r2), r3);
}

template <int N>
__device__ __forceinline__ void argmax_step(float &v, int &i) {
    const float ov = dpp_ror<N>(v);
    const int oi = dpp_ror<N>(i);
    if (better(ov, oi, v, i)) {
        v = ov;
        i = oi;
    }
}

// Best (value, index) of the wave under `better`; uniform result.
__device__ __forceinline__ void wave_argmax(float &v, int &i) {
    argmax_step<8>(v, i);
    argmax_step<4>(v, i);
    argmax_step<2>(v, i);
    argmax_step<1>(v, i);
    float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
        const float ov = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r));
        const int oi = __builtin_amdgcn_readlane(i, 16 * r);
        if (better(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
        }
    }
    v = bv;
    i = bi;
}

// Inclusive prefix sum over the wave: DPP row shifts inside each row of 16
// lanes, then the totals of the preceding rows (read from lanes 15, 31, 47).
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
    const int r0 = __builtin_amdgcn_readlane(v, 15);
    const int r1 = __builtin_amdgcn_readlane(v, 31);
    const int r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = (threadIdx.x & 63) >> 4;
    return v + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane l of the wave writes lds_wave_base + 16 l;
// the base must be the same in every lane.  Completion is tracked by the
// vector memory counter, so a wait for it and a barrier precede any read.
__device__ __forceinline__ void load_lds16(const void *src, void *lds_wave_base) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds_wave_base, 16, 0, 0);
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS (and
// scalar) operations, not for its outstanding global loads, so direct
// global->LDS loads issued earlier stay in flight across it.  __syncthreads()
// carries a release fence that waits for every vector memory operation.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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
