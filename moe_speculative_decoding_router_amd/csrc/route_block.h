// Routing of one verify call by one workgroup: per-token top-k over the
// router logits (optionally with the reuse-aware soft bias), gate weights,
// expert union, token-by-expert grouping and the slot tables of the FFN.
//
// [EcoSpec] = review of "Less Experts, Faster Decoding": §3.1 (logits ->
// softmax -> top-k per layer), §2 (the verify expert set is the union of the
// tokens' experts).  [S2-MoE] = walkthrough of S^2-MoE, component 2 (reuse-
// aware expert gating: importance aggregation, TopCap preferred set, additive
// bias sized by the top-1 / (k+1)-th margin; Fig. 5).
//
// Its barriers order LDS only (global tables written here are read by later
// kernels), so global loads issued by the caller before it stay in flight.
// The function is deterministic: every workgroup that runs it on the same
// logits obtains bit-identical tables (selections are exact comparisons,
// sums run in fixed orders, LDS atomics are ORs), so the gate-up kernel runs
// it redundantly in every workgroup instead of paying for a separate launch.
#pragma once

#include <math.h>

#include "common.h"
#include "internal.h"

namespace moe {

constexpr int kRouteNJ = kMaxExperts / 64;  // logits per lane

__device__ __forceinline__ float nan_to_ninf(float v) { return v != v ? -INFINITY : v; }

// Row of E logits into registers, entry lane + 64 j in v[j]; entries past E
// read -inf.  Every load is issued (clamped to the row) before any is used,
// so the row costs one memory round trip.
__device__ __forceinline__ void load_logits(const float *row, int E, float (&v)[kRouteNJ]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < kRouteNJ; ++j) v[j] = row[min(lane + 64 * j, E - 1)];
#pragma unroll
    for (int j = 0; j < kRouteNJ; ++j) v[j] = lane + 64 * j < E ? nan_to_ninf(v[j]) : -INFINITY;
}

// Wave-wide selection of the best untaken entry under (value desc, index
// asc).  v[j] holds entry lane + 64 j; `taken` marks entries this lane has
// given out.  NaN compares as -inf; with k <= E an untaken entry always wins
// over the empty sentinel.
__device__ __forceinline__ void wave_select(const float (&v)[kRouteNJ], unsigned &taken, int E, float &bv, int &bi) {
    const int lane = threadIdx.x & 63;
    bv = -INFINITY;
    bi = INT_MAX;
#pragma unroll
    for (int j = 0; j < kRouteNJ; ++j) {
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

// LDS scratch of block_route, carved from a byte buffer for runtime T, k, E.
struct RouteScratch {
    int *sel_i;                 // [T * k] first-pass selection (bias only)
    float *cg;                  // [T * k] w_b * softmax(l_b)_e of the selected e
    float *lam;                 // [T]
    int *fin_i;                 // [T * k] final selection
    float *fin_w;               // [T * k]
    unsigned long long *tmask;  // [E] tokens routed to each expert
    unsigned long long *tmask0; // [E] first-pass membership (bias only)
    float *g;                   // [E]
    int *inP;                   // [E]
    int *wtot;                  // [2 * waves]
    int *misc;                  // [4]: U, |P*|

    __host__ __device__ static size_t bytes(int T, int k, int E, int waves) {
        return (size_t)E * 16 + (size_t)T * k * 16 + (size_t)E * 8 + (size_t)T * 4 + (size_t)(2 * waves + 4) * 4 + 64;
    }
    __device__ void carve(unsigned char *base, int T, int k, int E, int waves) {
        unsigned char *q = base;
        tmask = reinterpret_cast<unsigned long long *>(q);
        q += (size_t)E * 8;
        tmask0 = reinterpret_cast<unsigned long long *>(q);
        q += (size_t)E * 8;
        sel_i = reinterpret_cast<int *>(q);
        q += (size_t)T * k * 4;
        cg = reinterpret_cast<float *>(q);
        q += (size_t)T * k * 4;
        fin_i = reinterpret_cast<int *>(q);
        q += (size_t)T * k * 4;
        fin_w = reinterpret_cast<float *>(q);
        q += (size_t)T * k * 4;
        g = reinterpret_cast<float *>(q);
        q += (size_t)E * 4;
        inP = reinterpret_cast<int *>(q);
        q += (size_t)E * 4;
        lam = reinterpret_cast<float *>(q);
        q += (size_t)T * 4;
        wtot = reinterpret_cast<int *>(q);
        q += (size_t)2 * waves * 4;
        misc = reinterpret_cast<int *>(q);
    }
};

// Routes the call with NTHREADS threads (NTHREADS >= E).  Results:
//   LDS: sexp[s] expert of slot s (E = shared expert), tw[s * T + t] gate
//        weight of token t in slot s (0 if not routed), *nslots_lds.
//   global (when write_global): topk_idx, topk_w, union, CSR, P*, meta, the
//        slot tables (slot_expert, tokw, tokpos, tpos) of the FFN kernels.
template <int NTHREADS>
__device__ __forceinline__ void block_route(const VerifyParams &p, unsigned char *scratch, int *sexp, float *tw, int *nslots_lds,
                            bool write_global) {
    static_assert(NTHREADS >= kMaxExperts, "the union scan gives every expert one thread");
    constexpr int NW = NTHREADS / 64;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int T = p.T, E = p.E, k = p.k;
    const bool bias = p.bias_on != 0;
    RouteScratch sh;
    sh.carve(scratch, T, k, E, NW);

    for (int e = tid; e < E; e += NTHREADS) {
        sh.tmask[e] = 0ull;
        sh.tmask0[e] = 0ull;
        sh.inP[e] = 0;
    }
    lds_barrier();

    // ---- pass 1: top-k (k + 1 when the bias needs the (k+1)-th logit);
    //      lane r keeps the r-th choice in registers ----
    const int R = (bias && k < E) ? k + 1 : k;
    for (int t = w; t < T; t += NW) {
        float v[kRouteNJ];
        load_logits(p.logits + (size_t)t * E, E, v);
        const float wc = bias ? p.w_conf[t] : 0.f;
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
        if (!bias) {
            const float ex = mine ? expf(my_v - m) : 0.f;
            const float s = wave_sum(ex);
            if (mine) {
                sh.fin_i[t * k + lane] = my_i;
                sh.fin_w[t * k + lane] = ex / s;
            }
        } else {
            // softmax over all E for the importance aggregation (R4)
            float z = 0.f;
#pragma unroll
            for (int j = 0; j < kRouteNJ; ++j)
                if (lane + 64 * j < E) z += expf(v[j] - m);
            z = wave_sum(z);
            if (mine) {
                sh.sel_i[t * k + lane] = my_i;
                sh.cg[t * k + lane] = wc * (expf(my_v - m) / z);
                if (my_i >= 0 && my_i < E) atomicOr(&sh.tmask0[my_i], 1ull << t);
            }
            // lambda_b = alpha * (l_(1) - l_(k+1)), float32, no contraction (R6)
            if (lane == 0) sh.lam[t] = k < E ? __fmul_rn(p.alpha, __fsub_rn(m, vk1)) : 0.f;
        }
    }
    lds_barrier();

    if (bias) {
        // ---- importance g_e (R4), summed in token order ----
        for (int e = tid; e < E; e += NTHREADS) {
            float g = 0.f;
            const unsigned long long m0 = sh.tmask0[e];
            for (int t = 0; t < T; ++t)
                if ((m0 >> t) & 1ull)
                    for (int j = 0; j < k; ++j)
                        if (sh.sel_i[t * k + j] == e) g += sh.cg[t * k + j];
            sh.g[e] = g;
        }
        lds_barrier();
        // ---- preferred set P*: top-cap by (g desc, index asc), g > 0 (R5) ----
        if (w == 0) {
            float gv[kRouteNJ];
#pragma unroll
            for (int j = 0; j < kRouteNJ; ++j) {
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
                    if (write_global) p.pstar[n] = bi;
                }
            }
            if (lane == 0) sh.misc[1] = n;
        }
        lds_barrier();
        // ---- re-select on the biased logits; weights from the original (R6, R7) ----
        for (int t = w; t < T; t += NW) {
            float v[kRouteNJ], vb[kRouteNJ];
            load_logits(p.logits + (size_t)t * E, E, v);
            const float lam = sh.lam[t];
#pragma unroll
            for (int j = 0; j < kRouteNJ; ++j) {
                const int e = lane + 64 * j;
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
                for (int j = 0; j < kRouteNJ; ++j)
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
                sh.fin_i[t * k + lane] = my_i;
                sh.fin_w[t * k + lane] = ex / s;
            }
        }
        lds_barrier();
    }

    // ---- per-token outputs and membership masks ----
    for (int i = tid; i < T * k; i += NTHREADS) {
        const int t = i / k;
        const int e = sh.fin_i[i];
        if (write_global) {
            p.topk_idx[i] = e;
            p.topk_w[i] = sh.fin_w[i];
        }
        if (e >= 0 && e < E) atomicOr(&sh.tmask[e], 1ull << t);
    }
    lds_barrier();

    // ---- union (ascending) via a block scan over experts: rank of each
    //      union expert and offset of its CSR row ----
    const int e = tid;
    const unsigned long long msk = e < E ? sh.tmask[e] : 0ull;
    const int cnt = __popcll(msk);
    const int flag = cnt > 0;
    const unsigned long long bal = __ballot(flag);
    const int rank_in_wave = __popcll(bal & ((1ull << lane) - 1ull));
    const int incl = wave_incl_scan(cnt);
    if (lane == 63) {
        sh.wtot[w] = __popcll(bal);
        sh.wtot[NW + w] = incl;
    }
    lds_barrier();
    int base_flag = 0, base_cnt = 0, U = 0;
    for (int q = 0; q < NW; ++q) {
        if (q < w) {
            base_flag += sh.wtot[q];
            base_cnt += sh.wtot[NW + q];
        }
        U += sh.wtot[q];
    }
    // g (scratch) is reused as the per-expert CSR offset, inP as the rank
    int *csr_off = reinterpret_cast<int *>(sh.g);
    if (e < E) {
        const int rank = base_flag + rank_in_wave;
        const int off = base_cnt + incl - cnt;
        csr_off[e] = off;
        sh.inP[e] = rank;
        if (flag) {
            sexp[rank] = e;
            if (write_global) {
                p.union_experts[rank] = e;
                p.csr_ptr[rank] = off;
                p.slot_expert[rank] = e;
            }
            // tokens of this slot that do not route to it get weight 0
            for (int t = 0; t < T; ++t) {
                if (!((msk >> t) & 1ull)) {
                    tw[rank * T + t] = 0.f;
                    if (write_global) {
                        p.tokw[(size_t)rank * T + t] = 0.f;
                        p.tokpos[(size_t)rank * T + t] = -1;
                    }
                }
            }
        }
    }
    lds_barrier();
    // ---- CSR entries: one thread per (token, rank) ----
    for (int i = tid; i < T * k; i += NTHREADS) {
        const int t = i / k;
        const int ex = sh.fin_i[i];
        if (ex < 0 || ex >= E) continue;
        const unsigned long long m = sh.tmask[ex];
        const int pos = csr_off[ex] + __popcll(m & ((1ull << t) - 1ull));
        const int rank = sh.inP[ex];
        const float wt = sh.fin_w[i];
        tw[rank * T + t] = wt;
        if (write_global) {
            p.csr_tok[pos] = t;
            p.csr_w[pos] = wt;
            p.tpos[i] = pos;
            p.tokw[(size_t)rank * T + t] = wt;
            p.tokpos[(size_t)rank * T + t] = pos;
        }
    }
    if (p.has_shared && tid < T) {
        if (tid == 0) sexp[U] = E;
        tw[U * T + tid] = 1.f;
        if (write_global) {
            if (tid == 0) p.slot_expert[U] = E;
            p.tokw[(size_t)U * T + tid] = 1.f;
            p.tokpos[(size_t)U * T + tid] = T * k + tid;
        }
    }
    if (tid == 0) {
        *nslots_lds = U + p.has_shared;
        if (write_global) {
            const int np = bias ? sh.misc[1] : 0;
            p.csr_ptr[U] = T * k;
            p.meta[0] = U;
            p.meta[1] = U + p.has_shared;
            p.meta[2] = np;
            if (p.union_size_out) p.union_size_out[0] = U;
            if (p.pstar_size_out) p.pstar_size_out[0] = np;
        }
    }
    lds_barrier();
}

}  // namespace moe
