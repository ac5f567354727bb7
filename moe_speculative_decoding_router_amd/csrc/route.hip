// Router GEMV, routing (top-k, optional reuse-aware bias), expert union and
// token-by-expert grouping.
//
// Pages: [EcoSpec] = review of "Less Experts, Faster Decoding: Cost-Aware
// Speculative Decoding for Mixture-of-Experts"; [S2-MoE] = walkthrough of
// S^2-MoE.  Routing follows [EcoSpec] §3.1 (logits -> softmax -> top-k); the
// union is the verify expert set of [EcoSpec] §2; the bias is [S2-MoE]
// component 2, steps 1-3 (Fig. 5).
#include <math.h>

#include "common.h"
#include "internal.h"
#include "route_block.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// Router GEMV: logits[t, e] = sum_h x[t, h] * Wr[e, h] in float32.
// One workgroup per expert; its 8 waves split H (at the Qwen3 and DeepSeek
// widths every load of a wave is issued before any is used: one memory round
// trip); the partial sums are added in a fixed order, so the result is
// reproducible.  The same kernel writes
// x as the bf16 matrix-core operand (high/low pair or single) for the FFN.
// ---------------------------------------------------------------------------
constexpr int kRouterThreads = 512;
constexpr int kRouterWaves = kRouterThreads / 64;

// TC: tokens per pass (T itself up to 8, so no row is loaded twice).
template <bool VEC4, int TC>
__global__ __launch_bounds__(kRouterThreads) void router_kernel(VerifyParams p) {
    __shared__ float red[kRouterWaves][8];
    const int e = blockIdx.x;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int H = p.H, T = p.T;
    const int total = T * H;
    const int gid = blockIdx.x * kRouterThreads + threadIdx.x, gstride = gridDim.x * kRouterThreads;
    // x element of the activation-operand conversion, loaded up front
    const bool conv = p.wdtype != 0;
    float xc = 0.f;
    if (conv && gid < total) xc = p.x[gid];
    if (p.tile_cnt)  // per-row-tile piece counters of the down kernel
        for (int i = gid; i < p.H / 16; i += gstride) p.tile_cnt[i] = 0;
    if (p.gu_ticket && gid == 0) p.gu_ticket[0] = 0;

    if (e < p.E) {
        const int n = VEC4 ? H / 4 : H;
        const int hb = (w * n) / kRouterWaves, he = ((w + 1) * n) / kRouterWaves;
        for (int t0 = 0; t0 < T; t0 += TC) {
            float acc[TC];
#pragma unroll
            for (int tt = 0; tt < TC; ++tt) acc[tt] = 0.f;
            if (VEC4) {
                // 4 float4 of Wr and of each token's x per lane per pass; all
                // loads (clamped into range) are issued before any is used
                const float4 *wr = reinterpret_cast<const float4 *>(p.Wr) + (size_t)e * n;
                const float4 *xv = reinterpret_cast<const float4 *>(p.x);
                const int nt = T - t0 < TC ? T - t0 : TC;
                for (int h0 = hb + lane; h0 < he; h0 += 256) {
                    float4 a[4], b[TC][4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) a[u] = wr[min(h0 + 64 * u, he - 1)];
#pragma unroll
                    for (int tt = 0; tt < TC; ++tt)
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            b[tt][u] = xv[(size_t)(t0 + min(tt, nt - 1)) * n + min(h0 + 64 * u, he - 1)];
#pragma unroll
                    for (int tt = 0; tt < TC; ++tt)
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            if (tt < nt && h0 + 64 * u < he)
                                acc[tt] += a[u].x * b[tt][u].x + a[u].y * b[tt][u].y + a[u].z * b[tt][u].z +
                                           a[u].w * b[tt][u].w;
                }
            } else {
                const float *wr = p.Wr + (size_t)e * H;
                for (int h = hb + lane; h < he; h += 64) {
                    const float a = wr[h];
#pragma unroll
                    for (int tt = 0; tt < TC; ++tt)
                        if (t0 + tt < T) acc[tt] += a * p.x[(size_t)(t0 + tt) * H + h];
                }
            }
            const int nt = T - t0 < TC ? T - t0 : TC;
#pragma unroll
            for (int tt = 0; tt < TC; ++tt) {
                if (tt < nt) {
                    const float v = wave_sum(acc[tt]);
                    if (lane == 0) red[w][tt] = v;
                }
            }
            __syncthreads();
            if (threadIdx.x < nt) {
                const int tt = threadIdx.x;
                float sum = red[0][tt];
#pragma unroll
                for (int q = 1; q < kRouterWaves; ++q) sum += red[q][tt];
                p.logits[(size_t)(t0 + tt) * p.E + e] = sum;
            }
            __syncthreads();
        }
    }

    if (conv) {
        // x -> bf16 operand columns: split mode stores hi = bf16(x) in
        // column t and lo = bf16(x - hi) in column T + t.
        const bool fp8 = p.wdtype == 2;
        for (int g = gid; g < total; g += gstride) {
            const int t = g / H, h = g - t * H;
            const float v = g == gid ? xc : p.x[g];
            const uint16_t hi = f32_to_bf16_rne(v);
            p.xB[b_index(h, t, p.cstride, fp8)] = hi;
            if (p.split) p.xB[b_index(h, T + t, p.cstride, fp8)] = f32_to_bf16_rne(v - bf16_to_f32(hi));
        }
    }
}

// ---------------------------------------------------------------------------
// Route as its own launch (one workgroup of 1024 threads); used when the
// gate-up kernel cannot hold the routing tables in LDS, and for float32
// weights.  The tables go to the workspace for the FFN kernels.
// ---------------------------------------------------------------------------
constexpr int kRouteThreads = 1024;

__global__ __launch_bounds__(kRouteThreads) void route_kernel(VerifyParams p) {
    extern __shared__ __align__(16) unsigned char dyn[];
    __shared__ int nslots;
    // the slot tables go straight to the workspace
    block_route<kRouteThreads>(p, dyn, p.slot_expert, p.tokw, &nslots, true);
}

}  // namespace

hipError_t launch_router(const VerifyParams &p, hipStream_t s, KernelEvents ev) {
    const dim3 g(p.E), b(kRouterThreads);
    if (p.H % 4 != 0) return launch_k(router_kernel<false, 8>, g, b, 0, s, ev, p);
    switch (p.T < 8 ? p.T : 8) {
        case 1: return launch_k(router_kernel<true, 1>, g, b, 0, s, ev, p);
        case 2: return launch_k(router_kernel<true, 2>, g, b, 0, s, ev, p);
        case 3: return launch_k(router_kernel<true, 3>, g, b, 0, s, ev, p);
        case 4: return launch_k(router_kernel<true, 4>, g, b, 0, s, ev, p);
        case 5: return launch_k(router_kernel<true, 5>, g, b, 0, s, ev, p);
        case 6: return launch_k(router_kernel<true, 6>, g, b, 0, s, ev, p);
        case 7: return launch_k(router_kernel<true, 7>, g, b, 0, s, ev, p);
        default: return launch_k(router_kernel<true, 8>, g, b, 0, s, ev, p);
    }
}

size_t route_lds_bytes(const VerifyParams &p) { return RouteScratch::bytes(p.T, p.k, p.E, kRouteThreads / 64); }

hipError_t launch_route(const VerifyParams &p, hipStream_t s, KernelEvents ev) {
    const size_t lds = route_lds_bytes(p);
    if (lds > 64 * 1024 &&
        hipFuncSetAttribute(reinterpret_cast<const void *>(route_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds) != hipSuccess)
        return hipErrorInvalidValue;
    return launch_k(route_kernel, dim3(1), dim3(kRouteThreads), lds, s, ev, p);
}

}  // namespace moe
