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

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// Router GEMV: logits[t, e] = sum_h x[t, h] * Wr[e, h] in float32.
// One workgroup per expert; its 4 waves split H; the partial sums are added
// in a fixed order, so the result is reproducible.  The same kernel writes
// x as the bf16 matrix-core operand (high/low pair or single) for the FFN.
// ---------------------------------------------------------------------------
constexpr int kRouterThreads = 256;

template <bool VEC4>
__global__ __launch_bounds__(kRouterThreads) void router_kernel(VerifyParams p) {
    __shared__ float red[4][8];
    const int e = blockIdx.x;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int H = p.H, T = p.T;

    if (e < p.E) {
        const int n = VEC4 ? H / 4 : H;
        const int hb = (w * n) / 4, he = ((w + 1) * n) / 4;
        for (int t0 = 0; t0 < T; t0 += 8) {
            float acc[8];
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) acc[tt] = 0.f;
            if (VEC4) {
                const float4 *wr = reinterpret_cast<const float4 *>(p.Wr) + (size_t)e * n;
                const float4 *xv = reinterpret_cast<const float4 *>(p.x);
                for (int h = hb + lane; h < he; h += 64) {
                    const float4 a = wr[h];
#pragma unroll
                    for (int tt = 0; tt < 8; ++tt) {
                        if (t0 + tt < T) {
                            const float4 b = xv[(size_t)(t0 + tt) * n + h];
                            acc[tt] += a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
                        }
                    }
                }
            } else {
                const float *wr = p.Wr + (size_t)e * H;
                for (int h = hb + lane; h < he; h += 64) {
                    const float a = wr[h];
#pragma unroll
                    for (int tt = 0; tt < 8; ++tt)
                        if (t0 + tt < T) acc[tt] += a * p.x[(size_t)(t0 + tt) * H + h];
                }
            }
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                const float v = wave_sum(acc[tt]);
                if (lane == 0) red[w][tt] = v;
            }
            __syncthreads();
            if (threadIdx.x < 8 && t0 + (int)threadIdx.x < T) {
                const int tt = threadIdx.x;
                p.logits[(size_t)(t0 + tt) * p.E + e] = ((red[0][tt] + red[1][tt]) + red[2][tt]) + red[3][tt];
            }
            __syncthreads();
        }
    }

    if (p.wdtype != 0) {
        // x -> bf16 operand columns: split mode stores hi = bf16(x) in
        // column t and lo = bf16(x - hi) in column T + t.
        const bool fp8 = p.wdtype == 2;
        const int total = T * H;
        for (int g = blockIdx.x * kRouterThreads + threadIdx.x; g < total; g += gridDim.x * kRouterThreads) {
            const int t = g / H, h = g - t * H;
            const float v = p.x[g];
            const uint16_t hi = f32_to_bf16_rne(v);
            p.xB[b_index(h, t, p.cols, fp8)] = hi;
            if (p.split) p.xB[b_index(h, T + t, p.cols, fp8)] = f32_to_bf16_rne(v - bf16_to_f32(hi));
        }
    }
}

// ---------------------------------------------------------------------------
// Route: one workgroup of 1024 threads.  Each wave handles tokens w, w+16, ...
// Top-k is a sequence of wave-wide arg-max reductions under the total order
// (logit desc, index asc); NaN logits compare as -inf.
// ---------------------------------------------------------------------------
constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kNJ = kMaxExperts / 64;  // logits per lane

struct RouteShared {
    int sel_i[kMaxTokens][kMaxTopK + 1];    // first pass selection (k or k+1)
    float sel_v[kMaxTokens][kMaxTopK + 1];
    float cg[kMaxTokens][kMaxTopK];         // w_b * softmax(l_b)_e for selected e
    float lam[kMaxTokens];
    int fin_i[kMaxTokens][kMaxTopK];        // final selection
    float fin_w[kMaxTokens][kMaxTopK];
    unsigned long long tmask[kMaxExperts];  // tokens routed to each expert
    unsigned long long tmask0[kMaxExperts]; // first-pass membership (bias only)
    float g[kMaxExperts];
    int inP[kMaxExperts];
    int wtot_flag[kRouteWaves], wtot_cnt[kRouteWaves];
    int npstar;
};

__device__ inline float nan_to_ninf(float v) { return v != v ? -INFINITY : v; }

// Wave-wide selection of the best untaken entry.  v[j] holds expert
// lane + 64 j; `taken` marks entries already chosen by this lane.
__device__ inline void wave_select(const float (&v)[kNJ], unsigned &taken, int E, float &bv, int &bi) {
    const int lane = threadIdx.x & 63;
    bv = -INFINITY;
    bi = INT_MAX;
#pragma unroll
    for (int j = 0; j < kNJ; ++j) {
        const int e = lane + 64 * j;
        const float vj = v[j] != v[j] ? -INFINITY : v[j];
        if (e < E && !((taken >> j) & 1u) && better(vj, e, bv, bi)) {
            bv = vj;
            bi = e;
        }
    }
    wave_argmax(bv, bi);
    if (bi != INT_MAX && (bi & 63) == lane) taken |= 1u << (bi >> 6);
}

__global__ __launch_bounds__(kRouteThreads) void route_kernel(VerifyParams p) {
    __shared__ RouteShared sh;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int T = p.T, E = p.E, k = p.k;
    const bool bias = p.bias_on != 0;

    for (int e = tid; e < E; e += kRouteThreads) {
        sh.tmask[e] = 0ull;
        sh.tmask0[e] = 0ull;
        sh.inP[e] = 0;
    }
    __syncthreads();

    // ---- pass 1: top-k (k + 1 when the bias needs the (k+1)-th logit) ----
    // Lane r keeps the r-th choice in registers.
    const int R = (bias && k < E) ? k + 1 : k;
    for (int t = w; t < T; t += kRouteWaves) {
        float v[kNJ];
#pragma unroll
        for (int j = 0; j < kNJ; ++j) {
            const int e = lane + 64 * j;
            v[j] = e < E ? nan_to_ninf(p.logits[(size_t)t * E + e]) : -INFINITY;
        }
        unsigned taken = 0;
        float m = 0.f, vk1 = 0.f, my_v = -INFINITY;
        int my_i = 0;
        for (int r = 0; r < R; ++r) {
            float bv;
            int bi;
            wave_select(v, taken, E, bv, bi);
            if (r == 0) m = bv;
            if (r == k) vk1 = bv;
            if (lane == r) {
                my_v = bv;
                my_i = bi;
            }
        }
        const bool mine = lane < k;
        if (mine) sh.sel_i[t][lane] = my_i;
        if (!bias) {
            const float ex = mine ? expf(my_v - m) : 0.f;
            const float s = wave_sum(ex);
            if (mine) {
                sh.fin_i[t][lane] = my_i;
                sh.fin_w[t][lane] = ex / s;
            }
        } else {
            // softmax over all E for the importance aggregation (R4)
            float z = 0.f;
#pragma unroll
            for (int j = 0; j < kNJ; ++j)
                if (lane + 64 * j < E) z += expf(v[j] - m);
            z = wave_sum(z);
            if (mine) {
                sh.cg[t][lane] = p.w_conf[t] * (expf(my_v - m) / z);
                if (my_i >= 0 && my_i < E) atomicOr(&sh.tmask0[my_i], 1ull << t);
            }
            // lambda_b = alpha * (l_(1) - l_(k+1)), float32, no contraction (R6)
            if (lane == 0) sh.lam[t] = k < E ? __fmul_rn(p.alpha, __fsub_rn(m, vk1)) : 0.f;
        }
    }
    __syncthreads();

    if (bias) {
        // ---- importance g_e (R4), summed in token order ----
        for (int e = tid; e < E; e += kRouteThreads) {
            float g = 0.f;
            const unsigned long long m0 = sh.tmask0[e];
            for (int t = 0; t < T; ++t) {
                if ((m0 >> t) & 1ull) {
                    for (int j = 0; j < k; ++j)
                        if (sh.sel_i[t][j] == e) g += sh.cg[t][j];
                }
            }
            sh.g[e] = g;
        }
        __syncthreads();
        // ---- preferred set P*: top-cap by (g desc, index asc), g > 0 (R5) ----
        if (w == 0) {
            float gv[kNJ];
#pragma unroll
            for (int j = 0; j < kNJ; ++j) {
                const int e = lane + 64 * j;
                gv[j] = e < E ? sh.g[e] : -INFINITY;
            }
            unsigned taken = 0;
            int n = 0;
            for (; n < p.cap; ++n) {
                float bv;
                int bi;
                wave_select(gv, taken, E, bv, bi);
                if (bi < 0 || bi >= E || !(bv > 0.f)) break;
                if (lane == 0) {
                    sh.inP[bi] = 1;
                    p.pstar[n] = bi;
                }
            }
            if (lane == 0) {
                sh.npstar = n;
                p.meta[2] = n;
                if (p.pstar_size_out) p.pstar_size_out[0] = n;
            }
        }
        __syncthreads();
        // ---- re-select on the biased logits; weights from the original (R6, R7) ----
        for (int t = w; t < T; t += kRouteWaves) {
            float v[kNJ], vb[kNJ];
            const float lam = sh.lam[t];
#pragma unroll
            for (int j = 0; j < kNJ; ++j) {
                const int e = lane + 64 * j;
                v[j] = e < E ? nan_to_ninf(p.logits[(size_t)t * E + e]) : -INFINITY;
                vb[j] = (e < E && sh.inP[e]) ? __fadd_rn(v[j], lam) : v[j];
            }
            unsigned taken = 0;
            float my_ov = -INFINITY;
            int my_i = 0;
            for (int r = 0; r < k; ++r) {
                float bv;
                int bi;
                wave_select(vb, taken, E, bv, bi);
                float ov = -INFINITY;  // original logit of the chosen expert
#pragma unroll
                for (int j = 0; j < kNJ; ++j)
                    if (lane + 64 * j == bi) ov = v[j];
                ov = wave_max(ov);
                if (lane == r) {
                    my_ov = ov;
                    my_i = bi;
                }
            }
            const bool mine = lane < k;
            const float m = wave_max(mine ? my_ov : -INFINITY);
            const float ex = mine ? expf(my_ov - m) : 0.f;
            const float s = wave_sum(ex);
            if (mine) {
                sh.fin_i[t][lane] = my_i;
                sh.fin_w[t][lane] = ex / s;
            }
        }
        __syncthreads();
    }

    // ---- outputs per token and membership masks ----
    for (int i = tid; i < T * k; i += kRouteThreads) {
        const int t = i / k, j = i - t * k;
        const int e = sh.fin_i[t][j];
        p.topk_idx[i] = e;
        p.topk_w[i] = sh.fin_w[t][j];
        if (e >= 0 && e < E) atomicOr(&sh.tmask[e], 1ull << t);
    }
    __syncthreads();

    // ---- union (ascending) and CSR via a block scan over experts ----
    const int e = tid;
    const unsigned long long m = e < E ? sh.tmask[e] : 0ull;
    const int cnt = __popcll(m);
    const int flag = cnt > 0;
    const unsigned long long bal = __ballot(flag);
    const int rank_in_wave = __popcll(bal & ((1ull << lane) - 1ull));
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) {
        sh.wtot_flag[w] = __popcll(bal);
        sh.wtot_cnt[w] = incl;
    }
    __syncthreads();
    int base_flag = 0, base_cnt = 0, U = 0;
    for (int q = 0; q < kRouteWaves; ++q) {
        if (q < w) {
            base_flag += sh.wtot_flag[q];
            base_cnt += sh.wtot_cnt[q];
        }
        U += sh.wtot_flag[q];
    }
    if (flag) {
        const int rank = base_flag + rank_in_wave;
        const int off = base_cnt + incl - cnt;
        p.union_experts[rank] = e;
        p.csr_ptr[rank] = off;
        p.slot_expert[rank] = e;
        for (int t = 0; t < T; ++t) {
            float wt = 0.f;
            int pos = -1;
            if ((m >> t) & 1ull) {
                pos = off + __popcll(m & ((1ull << t) - 1ull));
                int jj = 0;
                for (int j = 0; j < k; ++j)
                    if (sh.fin_i[t][j] == e) jj = j;
                wt = sh.fin_w[t][jj];
                p.csr_tok[pos] = t;
                p.csr_w[pos] = wt;
                p.tpos[t * k + jj] = pos;
            }
            p.tokw[(size_t)rank * T + t] = wt;
            p.tokpos[(size_t)rank * T + t] = pos;
        }
    }
    if (tid == 0) {
        p.csr_ptr[U] = T * k;
        p.meta[0] = U;
        p.meta[1] = U + p.has_shared;
        if (p.union_size_out) p.union_size_out[0] = U;
        if (!bias) {
            p.meta[2] = 0;
            if (p.pstar_size_out) p.pstar_size_out[0] = 0;
        }
    }
    if (p.has_shared && tid < T) {
        if (tid == 0) p.slot_expert[U] = E;
        p.tokw[(size_t)U * T + tid] = 1.f;
        p.tokpos[(size_t)U * T + tid] = T * k + tid;
    }
}

}  // namespace

hipError_t launch_router(const VerifyParams &p, hipStream_t s) {
    if (p.H % 4 == 0)
        hipLaunchKernelGGL(router_kernel<true>, dim3(p.E), dim3(kRouterThreads), 0, s, p);
    else
        hipLaunchKernelGGL(router_kernel<false>, dim3(p.E), dim3(kRouterThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_route(const VerifyParams &p, hipStream_t s) {
    hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kRouteThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace moe
