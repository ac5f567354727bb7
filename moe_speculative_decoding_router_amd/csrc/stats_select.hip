// Per-layer union statistics and batched cost-aware greedy draft selection.
//
// [S2-MoE] = walkthrough of S^2-MoE: motivation, challenge 2 defines the
// reuse ratio as the number of distinct experts over s * k.
// [EcoSpec] = review of "Less Experts, Faster Decoding": §3.2 (global expert
// buffer B, rebuilt from empty every step) and §3.3 (score = path
// probability / (new (layer, expert) pairs + eps), greedy gamma times).
#include "common.h"
#include "internal.h"

namespace moe {
namespace {

// One workgroup per layer: LDS bitset of E bits, OR of the k experts of every
// token, popcount.  Out-of-range entries are ignored.
__global__ __launch_bounds__(256) void union_stats_kernel(const int32_t *__restrict__ topk, int T, int k,
                                                          int E, int32_t *counts, float *reuse) {
    extern __shared__ unsigned bits[];
    __shared__ int wsum[4];
    const int l = blockIdx.x;
    const int nw = (E + 31) / 32;
    for (int i = threadIdx.x; i < nw; i += 256) bits[i] = 0u;
    __syncthreads();
    const int32_t *a = topk + (size_t)l * T * k;
    for (int i = threadIdx.x; i < T * k; i += 256) {
        const int e = a[i];
        if (e >= 0 && e < E) atomicOr(&bits[e >> 5], 1u << (e & 31));
    }
    __syncthreads();
    int c = 0;
    for (int i = threadIdx.x; i < nw; i += 256) c += __popc(bits[i]);
    c = wave_sum_int(c);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
        counts[l] = total;
        reuse[l] = __fdiv_rn((float)total, (float)(T * k));
    }
}

// One workgroup (256 threads) per tree.  The tree's footprints are staged in
// LDS with 16-byte loads.  Each round, groups of TPN threads (a power of two
// dividing the wave) popcount the words of F & ~B of their nodes and reduce
// the count inside the group, so every node is scored in parallel; wave 0
// then takes the arg-max in (score desc, node asc) order and all threads add
// the chosen footprint to B.
constexpr int kSelThreads = 256;

__global__ __launch_bounds__(kSelThreads) void select_kernel(int N, const float *__restrict__ P,
                                                             const uint32_t *__restrict__ F, int W, int gamma,
                                                             float eps, int nt, int tpn, int32_t *S) {
    extern __shared__ uint32_t lds[];
    uint32_t *Fs = lds;                                   // [N * W]
    uint32_t *Bs = Fs + (size_t)N * W;                    // [W]
    float *sc = reinterpret_cast<float *>(Bs + W);        // [N]
    uint32_t *chosen = reinterpret_cast<uint32_t *>(sc + N);  // [ceil(N / 32)]
    __shared__ int best_sh;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int tree = blockIdx.x;
    if (tree >= nt) return;
    const uint32_t *Ft = F + (size_t)tree * N * W;
    const float *Pt = P + (size_t)tree * N;
    const int nwords = N * W;
    if (((nwords & 3) == 0) && ((reinterpret_cast<uintptr_t>(Ft) & 15) == 0)) {
        // every load of a thread is issued before its LDS stores (one round trip)
        constexpr int kPer = kSelectMaxLdsWords / 4 / kSelThreads;
        const u32x4 *src = reinterpret_cast<const u32x4 *>(Ft);
        u32x4 *dst = reinterpret_cast<u32x4 *>(Fs);
        const int n4 = nwords / 4;
        u32x4 v[kPer];
#pragma unroll
        for (int r = 0; r < kPer; ++r) v[r] = __builtin_nontemporal_load(src + min(tid + r * kSelThreads, n4 - 1));
#pragma unroll
        for (int r = 0; r < kPer; ++r)
            if (tid + r * kSelThreads < n4) dst[tid + r * kSelThreads] = v[r];
    } else {
        for (int i = tid; i < nwords; i += kSelThreads) Fs[i] = Ft[i];
    }
    for (int i = tid; i < W; i += kSelThreads) Bs[i] = 0u;
    for (int i = tid; i < (N + 31) / 32; i += kSelThreads) chosen[i] = 0u;
    __syncthreads();

    const int grp = tid / tpn, sub = tid - grp * tpn, ngrp = kSelThreads / tpn;
    for (int r = 0; r < gamma; ++r) {
        // ---- score every node (groups of tpn threads per node) ----
        for (int n0 = 0; n0 < N; n0 += ngrp) {
            const int n = n0 + grp;
            int c = 0;
            if (n < N)
                for (int i = sub; i < W; i += tpn) c += __popc(Fs[(size_t)n * W + i] & ~Bs[i]);
            for (int off = tpn >> 1; off >= 1; off >>= 1) c += __shfl_xor(c, off);
            if (n < N && sub == 0) sc[n] = __fdiv_rn(Pt[n], __fadd_rn((float)c, eps));
        }
        __syncthreads();
        // ---- arg-max over unchosen nodes: (score desc, node asc) ----
        if (wv == 0) {
            float bv = -INFINITY;
            int bi = INT_MAX;
            for (int n = lane; n < N; n += 64) {
                if ((chosen[n >> 5] >> (n & 31)) & 1u) continue;
                const float v = sc[n] != sc[n] ? -INFINITY : sc[n];
                if (better(v, n, bv, bi)) {
                    bv = v;
                    bi = n;
                }
            }
            wave_argmax(bv, bi);
            if (lane == 0) {
                if (bi < 0 || bi >= N) {  // unreachable for N > r; kept memory-safe
                    bi = 0;
                    while (bi < N - 1 && ((chosen[bi >> 5] >> (bi & 31)) & 1u)) ++bi;
                }
                best_sh = bi;
                S[(size_t)tree * gamma + r] = bi;
                chosen[bi >> 5] |= 1u << (bi & 31);
            }
        }
        __syncthreads();
        const int best = best_sh;
        for (int i = tid; i < W; i += kSelThreads) Bs[i] |= Fs[(size_t)best * W + i];
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_union_stats(const int32_t *topk_idx, int nL, int T, int k, int E, int32_t *counts,
                              float *reuse, hipStream_t s) {
    const size_t lds = (size_t)((E + 31) / 32) * 4;
    hipLaunchKernelGGL(union_stats_kernel, dim3(nL), dim3(256), lds, s, topk_idx, T, k, E, counts, reuse);
    return hipGetLastError();
}

hipError_t launch_select(int N, const float *P, const uint32_t *F, int W, int gamma, float eps, int nt,
                         int32_t *S, hipStream_t s) {
    const size_t lds = ((size_t)N * W + W + N + (N + 31) / 32) * 4;
    // threads per node: the largest power of two <= min(64, 256 / N), at least 1
    int tpn = 1;
    while (tpn * 2 <= 64 && tpn * 2 * N <= kSelThreads) tpn *= 2;
    hipLaunchKernelGGL(select_kernel, dim3(nt), dim3(kSelThreads), lds, s, N, P, F, W, gamma, eps, nt, tpn, S);
    return hipGetLastError();
}

}  // namespace moe
