// Grouped skinny SwiGLU FFN over the union experts only, and the combine.
//
// [EcoSpec] = review of "Less Experts, Faster Decoding" (§1-§2: at one MoE
// layer the verified tokens need the weights of the union of their experts;
// each unique expert is loaded once and applied to all of its tokens).
//
// Work decomposition (bf16 / fp8 weights):
//   gate-up : item = (union slot s, 16 intermediate rows i0..i0+15).  The 4
//             waves of a workgroup split the H contraction; each streams the
//             16 gate rows and 16 up rows of its K-quarter with 16-byte
//             non-temporal loads straight into the matrix-core A operand
//             (v_mfma_f32_16x16x32_bf16; fp8 is decoded exactly to bf16 in
//             registers and each 128-wide K block is scaled after its own
//             products).  The activations are the B operand: the T tokens as
//             columns (as a bf16 high/low pair when 2T <= 64), read from a
//             small L2-resident buffer.  Partial sums meet in LDS in a fixed
//             order; SiLU(gate) * up, times the token's gate weight, is
//             written in the B-operand layout of the down projection.
//   down    : item = (slot s, 16 output rows), one wave per item over the
//             full I contraction; per-(token, expert) rows of ydown.
//   combine : y[t] = sum over the token's k ranks of ydown (+ shared expert),
//             in rank order, so the output is reproducible.
// Float32 weights use plain VALU dot products (one wave per output row).
#include <math.h>

#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kFfnThreads = 256;

__device__ __forceinline__ u32x4 ld_nt(const uint8_t *ptr) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ptr));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16 OCP E4M3FN codes -> two bf16x8 operands (codes 0..7 and 8..15).  The
// hardware conversion yields exact float32 values with at most 4 significant
// bits, so taking their upper halves is an exact bf16 conversion.
__device__ __forceinline__ void fp8x16_to_bf16(u32x4 q, bf16x8 &lo, bf16x8 &hi) {
    u32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x2 f01 = __builtin_amdgcn_cvt_pk_f32_fp8(q[i], false);
        const f32x2 f23 = __builtin_amdgcn_cvt_pk_f32_fp8(q[i], true);
        const unsigned p0 = __builtin_amdgcn_perm(__float_as_uint(f01[1]), __float_as_uint(f01[0]), 0x07060302u);
        const unsigned p1 = __builtin_amdgcn_perm(__float_as_uint(f23[1]), __float_as_uint(f23[0]), 0x07060302u);
        if (i < 2) {
            a[2 * i] = p0;
            a[2 * i + 1] = p1;
        } else {
            b[2 * (i - 2)] = p0;
            b[2 * (i - 2) + 1] = p1;
        }
    }
    lo = as_bf16x8(a);
    hi = as_bf16x8(b);
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu(float z) { return z / (1.f + expf(-z)); }

// WT: 0 = bf16, 1 = fp8.  NT: 16-column tiles of the B operand.  SPLIT: the
// B columns are (hi of token t, lo of token t) pairs.  NKS: waves splitting
// the contraction of one item.  GU: gate-up (true) or down (false).
template <int WT, int NT, bool SPLIT, int NKS, bool GU>
__global__ __launch_bounds__(kFfnThreads) void ffn_mfma_kernel(VerifyParams p) {
    constexpr int IPW = 4 / NKS;
    constexpr int NACC = GU ? 2 : 1;
    constexpr int KU = NT == 1 ? 8 : (NT == 2 ? 4 : 2);  // bf16 k-steps per batch
    constexpr int KUB = NT == 1 ? 2 : 1;                  // fp8 128-blocks per batch
    constexpr size_t ESZ = WT == 1 ? 1 : 2;
    __shared__ f32x4 red[NKS > 1 ? 4 : 1][NACC * NT][64];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int sub = w / NKS, kpart = w % NKS;
    const int lr = lane & 15, g = lane >> 4;
    const int T = p.T, H = p.H, I = p.I, E = p.E, cols = p.cols;
    const int K = GU ? H : I;
    const int tiles = (GU ? I : H) / 16;
    const int items = min(p.meta[1], p.max_slots) * tiles;

    for (int base = blockIdx.x * IPW; base < items; base += gridDim.x * IPW) {
        const int item = base + sub;
        const bool active = item < items;
        f32x4 acc0[NT], acc1[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            acc0[n] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc1[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        int s = 0, r0 = 0;
        if (active) {
            s = item / tiles;
            r0 = (item - s * tiles) * 16;
            const int e = min(max(p.slot_expert[s], 0), p.has_shared ? E : E - 1);
            const bool shared = e == E && p.has_shared;
            const uint8_t *wbase;
            const float *sbase = nullptr;
            size_t mstride;  // bytes between the gate and up blocks
            int srow0 = 0, srow1 = 0, sld = 0;
            if (GU) {
                wbase = shared ? static_cast<const uint8_t *>(p.Wsh_gu)
                               : static_cast<const uint8_t *>(p.W_gu) + (size_t)e * 2 * I * H * ESZ;
                mstride = (size_t)I * H * ESZ;
                if (WT == 1) {
                    sld = H / 128;
                    sbase = shared ? p.ssh_gu : p.s_gu + (size_t)e * (2 * I / 128) * sld;
                    srow0 = (r0 / 128) * sld;
                    srow1 = ((I + r0) / 128) * sld;
                }
            } else {
                wbase = shared ? static_cast<const uint8_t *>(p.Wsh_d)
                               : static_cast<const uint8_t *>(p.W_d) + (size_t)e * H * I * ESZ;
                mstride = 0;
                if (WT == 1) {
                    sld = I / 128;
                    sbase = shared ? p.ssh_d : p.s_d + (size_t)e * (H / 128) * sld;
                    srow0 = (r0 / 128) * sld;
                }
            }
            const uint8_t *row0 = wbase + (size_t)(r0 + lr) * K * ESZ + g * 16;
            const uint8_t *row1 = row0 + mstride;
            const uint16_t *bbase = GU ? p.xB : p.hB + (size_t)s * I * cols;
            const uint16_t *bp[NT];
            bool bvalid[NT];
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const int c = n * 16 + lr;
                bvalid[n] = c < cols;
                bp[n] = bbase + (size_t)(g * cols + c) * 8;
            }
            const size_t bstep = (size_t)4 * cols * 8;  // elements per k-step
            const bf16x8 zero8 = as_bf16x8(u32x4{0u, 0u, 0u, 0u});

            if (WT == 0) {
                const int KS = K / 32;
                const int kb = (kpart * KS) / NKS, ke = ((kpart + 1) * KS) / NKS;
                for (int ks = kb; ks < ke; ks += KU) {
                    u32x4 a0[KU], a1[KU];
                    bf16x8 b[KU][NT];
#pragma unroll
                    for (int u = 0; u < KU; ++u) {
                        if (ks + u < ke) {
                            a0[u] = ld_nt(row0 + (size_t)(ks + u) * 64);
                            if (GU) a1[u] = ld_nt(row1 + (size_t)(ks + u) * 64);
#pragma unroll
                            for (int n = 0; n < NT; ++n)
                                b[u][n] = bvalid[n] ? as_bf16x8(*reinterpret_cast<const u32x4 *>(bp[n] + (ks + u) * bstep))
                                                    : zero8;
                        }
                    }
#pragma unroll
                    for (int u = 0; u < KU; ++u) {
                        if (ks + u < ke) {
#pragma unroll
                            for (int n = 0; n < NT; ++n) {
                                acc0[n] = mfma(as_bf16x8(a0[u]), b[u][n], acc0[n]);
                                if (GU) acc1[n] = mfma(as_bf16x8(a1[u]), b[u][n], acc1[n]);
                            }
                        }
                    }
                }
            } else {
                const int NB = K / 128;
                const int bb = (kpart * NB) / NKS, be = ((kpart + 1) * NB) / NKS;
                for (int kb = bb; kb < be; kb += KUB) {
                    u32x4 a0[KUB][2], a1[KUB][2];
                    bf16x8 b[KUB][4][NT];
                    float sc0[KUB], sc1[KUB];
#pragma unroll
                    for (int u = 0; u < KUB; ++u) {
                        if (kb + u < be) {
#pragma unroll
                            for (int h = 0; h < 2; ++h) {
                                a0[u][h] = ld_nt(row0 + (size_t)(kb + u) * 128 + h * 64);
                                if (GU) a1[u][h] = ld_nt(row1 + (size_t)(kb + u) * 128 + h * 64);
                            }
#pragma unroll
                            for (int q = 0; q < 4; ++q)
#pragma unroll
                                for (int n = 0; n < NT; ++n)
                                    b[u][q][n] = bvalid[n]
                                                     ? as_bf16x8(*reinterpret_cast<const u32x4 *>(
                                                           bp[n] + ((kb + u) * 4 + q) * bstep))
                                                     : zero8;
                            sc0[u] = sbase[srow0 + kb + u];
                            if (GU) sc1[u] = sbase[srow1 + kb + u];
                        }
                    }
#pragma unroll
                    for (int u = 0; u < KUB; ++u) {
                        if (kb + u < be) {
                            f32x4 t0[NT], t1[NT];
#pragma unroll
                            for (int n = 0; n < NT; ++n) {
                                t0[n] = f32x4{0.f, 0.f, 0.f, 0.f};
                                t1[n] = f32x4{0.f, 0.f, 0.f, 0.f};
                            }
#pragma unroll
                            for (int h = 0; h < 2; ++h) {
                                bf16x8 lo, hi;
                                fp8x16_to_bf16(a0[u][h], lo, hi);
#pragma unroll
                                for (int n = 0; n < NT; ++n) {
                                    t0[n] = mfma(lo, b[u][2 * h][n], t0[n]);
                                    t0[n] = mfma(hi, b[u][2 * h + 1][n], t0[n]);
                                }
                                if (GU) {
                                    fp8x16_to_bf16(a1[u][h], lo, hi);
#pragma unroll
                                    for (int n = 0; n < NT; ++n) {
                                        t1[n] = mfma(lo, b[u][2 * h][n], t1[n]);
                                        t1[n] = mfma(hi, b[u][2 * h + 1][n], t1[n]);
                                    }
                                }
                            }
#pragma unroll
                            for (int n = 0; n < NT; ++n) {
                                acc0[n] += sc0[u] * t0[n];
                                if (GU) acc1[n] += sc1[u] * t1[n];
                            }
                        }
                    }
                }
            }
        }

        if (NKS > 1) {
            if (active && kpart != 0) {
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    red[w][n][lane] = acc0[n];
                    if (GU) red[w][NT + n][lane] = acc1[n];
                }
            }
            __syncthreads();
            if (active && kpart == 0) {
#pragma unroll
                for (int q = 1; q < NKS; ++q) {
#pragma unroll
                    for (int n = 0; n < NT; ++n) {
                        acc0[n] += red[w + q][n][lane];
                        if (GU) acc1[n] += red[w + q][NT + n][lane];
                    }
                }
            }
        }

        if (active && kpart == 0) {
            const bool fp8 = WT == 1;
            // Column c of tile n is token n * 16 + lr.  In split mode the low
            // part of token t sits in column T + t (tile (T + t) / 16, lane
            // (T + t) % 16 of the same lane group) and is added here.
            float v0[NT][4], v1[NT][4];
#pragma unroll
            for (int n = 0; n < NT; ++n)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v0[n][j] = acc0[n][j];
                    v1[n][j] = acc1[n][j];
                }
            if (SPLIT) {
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    const int clo = T + n * 16 + lr;
                    const int nlo = clo >> 4;
                    const int src = (lane & ~15) | (clo & 15);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float lo0 = 0.f, lo1 = 0.f;
#pragma unroll
                        for (int q = 0; q < NT; ++q) {
                            const float a = __shfl(acc0[q][j], src);
                            const float b = GU ? __shfl(acc1[q][j], src) : 0.f;
                            if (q == nlo) {
                                lo0 = a;
                                lo1 = b;
                            }
                        }
                        v0[n][j] += lo0;
                        v1[n][j] += lo1;
                    }
                }
            }
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const int t = n * 16 + lr;
                if (t < T) {
                    if (GU) {
                        const float wt = p.tokw[(size_t)s * T + t];
                        float hv[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) hv[j] = wt * (silu(v0[n][j]) * v1[n][j]);
                        uint16_t hi[4], lo[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            hi[j] = f32_to_bf16_rne(hv[j]);
                            lo[j] = f32_to_bf16_rne(hv[j] - bf16_to_f32(hi[j]));
                        }
                        uint16_t *hb = p.hB + (size_t)s * I * cols;
                        const int i = r0 + 4 * g;
                        *reinterpret_cast<u32x2 *>(hb + b_index(i, t, cols, fp8)) =
                            u32x2{(unsigned)hi[0] | ((unsigned)hi[1] << 16), (unsigned)hi[2] | ((unsigned)hi[3] << 16)};
                        if (SPLIT)
                            *reinterpret_cast<u32x2 *>(hb + b_index(i, T + t, cols, fp8)) =
                                u32x2{(unsigned)lo[0] | ((unsigned)lo[1] << 16), (unsigned)lo[2] | ((unsigned)lo[3] << 16)};
                    } else {
                        const int pos = p.tokpos[(size_t)s * T + t];
                        if (pos >= 0 && pos < T * p.k + T)
                            *reinterpret_cast<float4 *>(p.ydown + (size_t)pos * H + r0 + 4 * g) =
                                make_float4(v0[n][0], v0[n][1], v0[n][2], v0[n][3]);
                    }
                }
            }
        }
        if (NKS > 1) __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Float32 weights: one wave per (slot, row), lanes over the contraction.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kFfnThreads) void gateup_f32_kernel(VerifyParams p) {
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6), nw = gridDim.x * 4;
    const int T = p.T, H = p.H, I = p.I;
    const int items = min(p.meta[1], p.max_slots) * I;
    for (int item = gw; item < items; item += nw) {
        const int s = item / I, i = item - s * I;
        const int e = min(max(p.slot_expert[s], 0), p.has_shared ? p.E : p.E - 1);
        const float *wg = (e == p.E && p.has_shared ? static_cast<const float *>(p.Wsh_gu)
                                    : static_cast<const float *>(p.W_gu) + (size_t)e * 2 * I * H) +
                          (size_t)i * H;
        const float *wu = wg + (size_t)I * H;
        for (int t0 = 0; t0 < T; t0 += 8) {
            float ag[8], au[8];
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) ag[tt] = au[tt] = 0.f;
            for (int h = lane; h < H; h += 64) {
                const float a = wg[h], b = wu[h];
#pragma unroll
                for (int tt = 0; tt < 8; ++tt) {
                    if (t0 + tt < T) {
                        const float xv = p.x[(size_t)(t0 + tt) * H + h];
                        ag[tt] += a * xv;
                        au[tt] += b * xv;
                    }
                }
            }
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                const float gs = wave_sum(ag[tt]), us = wave_sum(au[tt]);
                const int t = t0 + tt;
                if (lane == 0 && t < T)
                    p.h32[((size_t)s * T + t) * I + i] = p.tokw[(size_t)s * T + t] * (silu(gs) * us);
            }
        }
    }
}

__global__ __launch_bounds__(kFfnThreads) void down_f32_kernel(VerifyParams p) {
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6), nw = gridDim.x * 4;
    const int T = p.T, H = p.H, I = p.I;
    const int items = min(p.meta[1], p.max_slots) * H;
    for (int item = gw; item < items; item += nw) {
        const int s = item / H, r = item - s * H;
        const int e = min(max(p.slot_expert[s], 0), p.has_shared ? p.E : p.E - 1);
        const float *wd = (e == p.E && p.has_shared ? static_cast<const float *>(p.Wsh_d)
                                    : static_cast<const float *>(p.W_d) + (size_t)e * H * I) +
                          (size_t)r * I;
        for (int t0 = 0; t0 < T; t0 += 8) {
            float acc[8];
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) acc[tt] = 0.f;
            for (int i = lane; i < I; i += 64) {
                const float a = wd[i];
#pragma unroll
                for (int tt = 0; tt < 8; ++tt)
                    if (t0 + tt < T) acc[tt] += a * p.h32[((size_t)s * T + t0 + tt) * I + i];
            }
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                const float v = wave_sum(acc[tt]);
                const int t = t0 + tt;
                if (lane == 0 && t < T) {
                    const int pos = p.tokpos[(size_t)s * T + t];
                    if (pos >= 0 && pos < T * p.k + T) p.ydown[(size_t)pos * H + r] = v;
                }
            }
        }
    }
}

__global__ __launch_bounds__(256) void combine_kernel(VerifyParams p) {
    const int T = p.T, H = p.H, k = p.k;
    const int total = T * H;
    for (int idx = blockIdx.x * 256 + threadIdx.x; idx < total; idx += gridDim.x * 256) {
        const int t = idx / H, r = idx - t * H;
        float acc = 0.f;
        for (int j = 0; j < k; ++j) {
            const int pos = p.tpos[t * k + j];
            if (pos >= 0 && pos < T * k) acc += p.ydown[(size_t)pos * H + r];
        }
        if (p.has_shared) acc += p.ydown[(size_t)(T * k + t) * H + r];
        p.y[idx] = acc;
    }
}

// Persistent grid: as many workgroups as fit on the device at once.
template <typename K>
int resident_grid(K kernel, int n_cu) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kFfnThreads, 0) != hipSuccess || per_cu < 1)
        per_cu = 1;
    return per_cu * n_cu;
}

template <int WT, int NT, bool SPLIT, bool GU>
hipError_t launch_one(const VerifyParams &p, int n_cu, hipStream_t s) {
    constexpr int NKS = GU ? 4 : 1;
    auto kernel = ffn_mfma_kernel<WT, NT, SPLIT, NKS, GU>;
    static const int grid = resident_grid(kernel, n_cu);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kFfnThreads), 0, s, p);
    return hipGetLastError();
}

template <int WT, bool GU>
hipError_t launch_mfma(const VerifyParams &p, int n_cu, hipStream_t s) {
    const int nt = (p.cols + 15) / 16;
    if (p.split) {
        switch (nt) {
            case 1: return launch_one<WT, 1, true, GU>(p, n_cu, s);
            case 2: return launch_one<WT, 2, true, GU>(p, n_cu, s);
            case 3: return launch_one<WT, 3, true, GU>(p, n_cu, s);
            default: return launch_one<WT, 4, true, GU>(p, n_cu, s);
        }
    }
    switch (nt) {
        case 1: return launch_one<WT, 1, false, GU>(p, n_cu, s);
        case 2: return launch_one<WT, 2, false, GU>(p, n_cu, s);
        case 3: return launch_one<WT, 3, false, GU>(p, n_cu, s);
        default: return launch_one<WT, 4, false, GU>(p, n_cu, s);
    }
}

}  // namespace

hipError_t launch_gateup(const VerifyParams &p, int n_cu, hipStream_t s) {
    const int grid = n_cu * 4;
    if (p.wdtype == 0) {
        hipLaunchKernelGGL(gateup_f32_kernel, dim3(grid), dim3(kFfnThreads), 0, s, p);
        return hipGetLastError();
    }
    return p.wdtype == 1 ? launch_mfma<0, true>(p, n_cu, s) : launch_mfma<1, true>(p, n_cu, s);
}

hipError_t launch_down(const VerifyParams &p, int n_cu, hipStream_t s) {
    const int grid = n_cu * 4;
    if (p.wdtype == 0) {
        hipLaunchKernelGGL(down_f32_kernel, dim3(grid), dim3(kFfnThreads), 0, s, p);
        return hipGetLastError();
    }
    return p.wdtype == 1 ? launch_mfma<0, false>(p, n_cu, s) : launch_mfma<1, false>(p, n_cu, s);
}

hipError_t launch_combine(const VerifyParams &p, hipStream_t s) {
    int blocks = (p.T * p.H + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace moe
