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
#include "launch.h"
#include "route_block.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// Router GEMV: logits[t, e] = sum_h x[t, h] * Wr[e, h] in float32.
// Workgroup (e, c) takes expert e and the c-th chunk of TC tokens (the
// tokens are split so that the grid covers every compute unit even with
// few experts); its 8 waves split H (every load of a wave is issued before
// any is used: one memory round trip); the partial sums are added in a
// fixed order, so the result is reproducible.  The same kernel writes x as
// the bf16 matrix-core operand (high/low pair or single) for the FFN.
// ---------------------------------------------------------------------------
constexpr int kRouterThreads = 512;
constexpr int kRouterWaves = kRouterThreads / 64;

// TC: tokens per pass (T itself when it fits, so no row is loaded twice and
// up to 20 tokens take one pass); UP: float4 of the row per lane and pass
// (2 covers H <= 4096 with 8 waves, 4 covers H <= 8192).
template <bool VEC4, int TC, int UP>
__global__ __launch_bounds__(kRouterThreads) void router_kernel(VerifyParams p) {
    __shared__ float red[kRouterWaves][TC];
    const int e = blockIdx.x;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int H = p.H, T = p.T;
    const int total = T * H;
    const int gid = (blockIdx.y * gridDim.x + blockIdx.x) * kRouterThreads + threadIdx.x;
    const int gstride = gridDim.x * gridDim.y * kRouterThreads;
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
        for (int t0 = blockIdx.y * TC; t0 < T; t0 += TC * gridDim.y) {
            float acc[TC];
#pragma unroll
            for (int tt = 0; tt < TC; ++tt) acc[tt] = 0.f;
            if (VEC4) {
                // UP float4 of Wr and of each token's x per lane per pass; all
                // loads (clamped into range) are issued before any is used
                const float4 *wr = reinterpret_cast<const float4 *>(p.Wr) + (size_t)e * n;
                const float4 *xv = reinterpret_cast<const float4 *>(p.x);
                const int nt = T - t0 < TC ? T - t0 : TC;
                for (int h0 = hb + lane; h0 < he; h0 += 64 * UP) {
                    float4 a[UP], b[TC][UP];
#pragma unroll
                    for (int u = 0; u < UP; ++u) a[u] = wr[min(h0 + 64 * u, he - 1)];
#pragma unroll
                    for (int tt = 0; tt < TC; ++tt)
#pragma unroll
                        for (int u = 0; u < UP; ++u)
                            b[tt][u] = xv[(size_t)(t0 + min(tt, nt - 1)) * n + min(h0 + 64 * u, he - 1)];
#pragma unroll
                    for (int tt = 0; tt < TC; ++tt)
#pragma unroll
                        for (int u = 0; u < UP; ++u)
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
            if ((int)threadIdx.x < nt) {
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
// Route as its own launch (one workgroup of 512 threads); used when the
// gate-up kernel cannot hold the routing tables in LDS, and for float32
// weights.  The tables go to the workspace for the FFN kernels.
// ---------------------------------------------------------------------------
constexpr int kRouteThreads = 512;  // one thread per expert at the most experts; 256 registers per lane

__global__ __launch_bounds__(kRouteThreads) void route_kernel(VerifyParams p) {
    extern __shared__ __align__(16) unsigned char dyn[];
    __shared__ int nslots;
    // The expert of each slot is written by wave 0 and read back by the other
    // waves after an LDS-only barrier, so it must live in LDS; the routing
    // writes the workspace copy (slot_expert) itself.  The gate weights per
    // (slot, token) are only written, each by one thread, and go straight to
    // the workspace.
    __shared__ int sexp[kMaxExperts + 1];
    block_route<kRouteThreads>(p, dyn, sexp, p.tokw, nullptr, &nslots, true);
}

// Token chunks per expert: enough workgroups for the 256 compute units.
int router_chunks(int E, int T) {
    const int c = (256 + E - 1) / E;
    return c < T ? c : T;
}

template <int UP>
hipError_t launch_router_up(const VerifyParams &p, hipStream_t s, KernelEvents ev) {
    // tokens per workgroup: up to 8 exactly, else 10 or (with 2 float4 per
    // lane) 20, keeping the operand registers of a pass near 160
    const int T = p.T, chunks = router_chunks(p.E, T);
    const int need = (T + chunks - 1) / chunks;
    const int tc = need <= 8 ? need : (need <= 10 || UP > 2 ? 10 : 20);
    const dim3 g(p.E, (T + tc - 1) / tc), b(kRouterThreads);
    switch (tc) {
        case 1: return launch_k(router_kernel<true, 1, UP>, g, b, 0, s, ev, p);
        case 2: return launch_k(router_kernel<true, 2, UP>, g, b, 0, s, ev, p);
        case 3: return launch_k(router_kernel<true, 3, UP>, g, b, 0, s, ev, p);
        case 4: return launch_k(router_kernel<true, 4, UP>, g, b, 0, s, ev, p);
        case 5: return launch_k(router_kernel<true, 5, UP>, g, b, 0, s, ev, p);
        case 6: return launch_k(router_kernel<true, 6, UP>, g, b, 0, s, ev, p);
        case 7: return launch_k(router_kernel<true, 7, UP>, g, b, 0, s, ev, p);
        case 8: return launch_k(router_kernel<true, 8, UP>, g, b, 0, s, ev, p);
        case 10: return launch_k(router_kernel<true, 10, UP>, g, b, 0, s, ev, p);
        default: return launch_k(router_kernel<true, 20, 2>, g, b, 0, s, ev, p);
    }
}

}  // namespace

hipError_t launch_router(const VerifyParams &p, hipStream_t s, KernelEvents ev) {
    if (p.H % 4 != 0)
        return launch_k(router_kernel<false, 8, 1>, dim3(p.E, (p.T + 7) / 8), dim3(kRouterThreads), 0, s, ev, p);
    // float4 of the row per wave: 2 per lane cover up to 128
    const int per_wave = (p.H / 4 + kRouterWaves - 1) / kRouterWaves;
    return per_wave <= 128 ? launch_router_up<2>(p, s, ev) : launch_router_up<4>(p, s, ev);
}

size_t route_lds_bytes(const VerifyParams &p) {
    return RouteScratch::bytes(p.T, p.k, p.E, kRouteThreads / 64, false, route_nseq(p));
}

hipError_t launch_route(const VerifyParams &p, hipStream_t s, KernelEvents ev) {
    const size_t lds = route_lds_bytes(p);
    if (lds > 64 * 1024 &&
        hipFuncSetAttribute(reinterpret_cast<const void *>(route_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds) != hipSuccess)
        return hipErrorInvalidValue;
    return launch_k(route_kernel, dim3(1), dim3(kRouteThreads), lds, s, ev, p);
}

}  // namespace moe
