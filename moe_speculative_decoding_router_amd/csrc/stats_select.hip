// Per-layer union statistics and batched cost-aware greedy draft selection.
//
// [S2-MoE] = walkthrough of S^2-MoE: motivation, challenge 2 defines the
// reuse ratio as the number of distinct experts over s * k.
// [EcoSpec] = review of "Less Experts, Faster Decoding": §3.2 (global expert
// buffer B, rebuilt from empty every step) and §3.3 (score = path
// probability / (new (layer, expert) pairs + eps), greedy gamma times).
// [S2-MoE] component 1 = routing-aware adaptive expansion: a draft token
// joins while p * T_AR >= (new experts) * T_exp + draft cost.
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
// the chosen footprint to B (left empty for the static-cost ablation, where
// every node pays its whole footprint).
constexpr int kSelThreads = 256;

// STAGED: the tree's footprints are copied into LDS once; otherwise (a tree
// larger than the LDS stage) every round reads them from global memory, where
// after the first round they are L2 hits.
template <bool STAGED>
__global__ __launch_bounds__(kSelThreads) void select_kernel(int N, const float *__restrict__ P,
                                                             const uint32_t *__restrict__ F, int W, int gamma,
                                                             float eps, int nt, int tpn, int update_b, int32_t *S) {
    extern __shared__ uint32_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int tree = blockIdx.x;
    if (tree >= nt) return;
    const uint32_t *Ft = F + (size_t)tree * N * W;
    const uint32_t *Fs = STAGED ? lds : Ft;                                   // [N * W]
    uint32_t *Bs = lds + (STAGED ? (size_t)N * W : 0);                        // [W]
    float *sc = reinterpret_cast<float *>(Bs + W);        // [N]
    uint32_t *chosen = reinterpret_cast<uint32_t *>(sc + N);  // [ceil(N / 32)]
    __shared__ int best_sh;
    const float *Pt = P + (size_t)tree * N;
    const int nwords = N * W;
    if (!STAGED) {
    } else if (((nwords & 3) == 0) && ((reinterpret_cast<uintptr_t>(Ft) & 15) == 0)) {
        // every load of a thread is issued before its LDS stores (one round trip)
        constexpr int kPer = kSelectMaxLdsWords / 4 / kSelThreads;
        const u32x4 *src = reinterpret_cast<const u32x4 *>(Ft);
        u32x4 *dst = reinterpret_cast<u32x4 *>(lds);
        const int n4 = nwords / 4;
        u32x4 v[kPer];
#pragma unroll
        for (int r = 0; r < kPer; ++r) v[r] = __builtin_nontemporal_load(src + min(tid + r * kSelThreads, n4 - 1));
#pragma unroll
        for (int r = 0; r < kPer; ++r)
            if (tid + r * kSelThreads < n4) dst[tid + r * kSelThreads] = v[r];
    } else {
        for (int i = tid; i < nwords; i += kSelThreads) lds[i] = Ft[i];
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
        if (update_b)  // the static-cost ablation keeps B empty
            for (int i = tid; i < W; i += kSelThreads) Bs[i] |= Fs[(size_t)best * W + i];
        __syncthreads();
    }
}


// The 16 node counts of a one-wave-per-tree kernel (c[n]: this lane's part
// of node n's count) folded across the wave, halving the counts a lane keeps
// at every step: partners are the mirror lane in the row (lane bit 3), in
// the half row (bit 2), then quad xor 2 (bit 1) and xor 1 (bit 0), so lane
// i ends with its row's sum for node i % 16; the four rows are then added.
// Integer sums, exact in any order.
__device__ __forceinline__ int fold_node_counts(const int (&c)[16]) {
    const int lane = threadIdx.x & 63;
    const bool h3 = (lane >> 3) & 1, h2 = (lane >> 2) & 1, h1 = (lane >> 1) & 1, h0 = lane & 1;
    int c8[8], c4[4], c2[2];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        c8[k] = (h3 ? c[k + 8] : c[k]) + __builtin_amdgcn_update_dpp(0, h3 ? c[k] : c[k + 8], 0x140, 0xF, 0xF, false);
#pragma unroll
    for (int k = 0; k < 4; ++k)
        c4[k] = (h2 ? c8[k + 4] : c8[k]) + __builtin_amdgcn_update_dpp(0, h2 ? c8[k] : c8[k + 4], 0x141, 0xF, 0xF, false);
#pragma unroll
    for (int k = 0; k < 2; ++k)
        c2[k] = (h1 ? c4[k + 2] : c4[k]) + __builtin_amdgcn_update_dpp(0, h1 ? c4[k] : c4[k + 2], 0x4E, 0xF, 0xF, false);
    int cnt = (h0 ? c2[1] : c2[0]) + __builtin_amdgcn_update_dpp(0, h0 ? c2[0] : c2[1], 0xB1, 0xF, 0xF, false);
    cnt += __shfl_xor(cnt, 16);
    cnt += __shfl_xor(cnt, 32);
    return cnt;
}

// Small trees (N <= 16 nodes, W <= 64 MW words) in large batches: one wave
// per tree, four trees per workgroup, the whole tree in registers.  Lane l
// holds word l + 64 m (m < MW) of every node's footprint and of B, so a
// round is 16 MW and-not-popcounts per lane, a fold of the 16 counts across
// the wave that leaves lane i with the count of node i % 16, one score per
// lane and a wave arg-max: no LDS and no barrier.
// The scores, their order and the tie rule are those of select_kernel.
// Against it at 4096 trees of 14 nodes: 54.0 -> 24.4 us (376 words),
// 35.3 -> 18.0 (144), 59.0 -> 29.2 (464); with one wave sum per node instead
// of the fold, 32.9 / 23.5 / 37.9.  A single tree takes longer in one wave
// (11.5 against 8.2 us at 144 words), so small batches keep select_kernel.
constexpr int kSelWaveNodes = 16;
constexpr int kSelWaveMinTrees = 512;  // batches from which one wave per tree pays

template <int MW>
__global__ __launch_bounds__(256) void select_wave_kernel(int N, const float *__restrict__ P,
                                                          const uint32_t *__restrict__ F, int W, int gamma,
                                                          float eps, int nt, int update_b, int32_t *S) {
    constexpr int NM = kSelWaveNodes;
    const int lane = threadIdx.x & 63;
    const int tree = (int)blockIdx.x * 4 + ((int)threadIdx.x >> 6);
    if (tree >= nt) return;  // whole waves only; nothing below synchronises
    const uint32_t *Ft = F + (size_t)tree * N * W;
    uint32_t f[NM][MW], b[MW];
    float pn[NM];
#pragma unroll
    for (int n = 0; n < NM; ++n) {
#pragma unroll
        for (int m = 0; m < MW; ++m) {
            const int i = lane + 64 * m;
            f[n][m] = (n < N && i < W) ? __builtin_nontemporal_load(Ft + (size_t)n * W + i) : 0u;
        }
        pn[n] = n < N ? P[(size_t)tree * N + n] : 0.f;
    }
#pragma unroll
    for (int m = 0; m < MW; ++m) b[m] = 0u;
    uint32_t chosen = 0u;
    for (int r = 0; r < gamma; ++r) {
        // every node's count, with no branch between them so that the 16
        // wave sums interleave
        int c[NM];
#pragma unroll
        for (int n = 0; n < NM; ++n) {
            int x = 0;
#pragma unroll
            for (int m = 0; m < MW; ++m) x += __popc(f[n][m] & ~b[m]);
            c[n] = x;
        }
        // lane i scores node i % 16 (one division per lane), and one wave
        // arg-max picks the best
        const int me = lane & (NM - 1);
        const int cme = fold_node_counts(c);
        float pme = 0.f;
#pragma unroll
        for (int n = 0; n < NM; ++n) pme = me == n ? pn[n] : pme;
        float bv = -INFINITY;
        int bi = INT_MAX;
        if (me < N && !((chosen >> me) & 1u)) {
            const float v = __fdiv_rn(pme, __fadd_rn((float)cme, eps));
            bv = v != v ? -INFINITY : v;
            bi = me;
        }
        wave_argmax(bv, bi);
        bi = __builtin_amdgcn_readfirstlane(bi);
        if (bi < 0 || bi >= N) {  // unreachable for gamma <= N; kept memory-safe
            bi = 0;
            while (bi < N - 1 && ((chosen >> bi) & 1u)) ++bi;
        }
        if (lane == 0) S[(size_t)tree * gamma + r] = bi;
        chosen |= 1u << bi;
        if (update_b) {
#pragma unroll
            for (int n = 0; n < NM; ++n)
                if (n == bi)
#pragma unroll
                    for (int m = 0; m < MW; ++m) b[m] |= f[n][m];
        }
    }
}

// Utility expansion of small trees in large batches, laid out as in
// select_wave_kernel: one wave per tree, the tree in registers, the node
// counts folded so that lane i holds node i % 16's.  Every round each lane
// tests its node (outside S, its parent in S or the root, at or after the
// scan position, utility test passed) and the lowest passing node joins;
// the passes, the float32 test and the order are those of expand_kernel.
template <int MW>
__global__ __launch_bounds__(256) void expand_wave_kernel(ExpandArgs a, const float *__restrict__ P,
                                                          const uint32_t *__restrict__ F,
                                                          const float *__restrict__ Cd, int32_t *S, int32_t *count) {
    constexpr int NM = kSelWaveNodes;
    const int lane = threadIdx.x & 63;
    const int tree = (int)blockIdx.x * 4 + ((int)threadIdx.x >> 6);
    if (tree >= a.nt) return;  // whole waves only; nothing below synchronises
    const int N = a.N, W = a.W;
    const uint32_t *Ft = F + (size_t)tree * N * W;
    uint32_t f[NM][MW], b[MW];
#pragma unroll
    for (int n = 0; n < NM; ++n)
#pragma unroll
        for (int m = 0; m < MW; ++m) {
            const int i = lane + 64 * m;
            f[n][m] = (n < N && i < W) ? __builtin_nontemporal_load(Ft + (size_t)n * W + i) : 0u;
        }
    const int me = lane & (NM - 1);
    const float pme = me < N ? P[(size_t)tree * N + me] : 0.f;
    const float cdme = (me < N && Cd) ? Cd[(size_t)tree * N + me] : 0.f;
    int par = -1;  // parent of node me (static indices into the argument block)
#pragma unroll
    for (int n = 0; n < NM; ++n)
        if (me == n && n < N) par = a.parent[n];
#pragma unroll
    for (int m = 0; m < MW; ++m) b[m] = 0u;
    uint32_t inS = 0u;
    int pos = 0, nsel = 0;
    bool added = false;
    for (int round = 0; round <= 2 * N; ++round) {
        int c[NM];
#pragma unroll
        for (int n = 0; n < NM; ++n) {
            int x = 0;
#pragma unroll
            for (int m = 0; m < MW; ++m) x += __popc(f[n][m] & ~b[m]);
            c[n] = x;
        }
        const int cme = fold_node_counts(c);
        bool ok = false;
        if (me < N && me >= pos && !((inS >> me) & 1u) && (par < 0 || ((inS >> par) & 1u))) {
            const float num = __fmul_rn(pme, a.t_ar);
            const float den = __fadd_rn(__fmul_rn((float)cme, a.t_exp), cdme);
            ok = num >= den;
        }
        const unsigned long long bal = __ballot(ok) & 0xFFFFull;  // lanes 0..15 hold nodes 0..15
        const int pick = bal ? (int)__builtin_ctzll(bal) : -1;
        if (pick >= 0) {
            inS |= 1u << pick;
            if (lane == 0) S[(size_t)tree * N + nsel] = pick;
#pragma unroll
            for (int n = 0; n < NM; ++n)
                if (n == pick)
#pragma unroll
                    for (int m = 0; m < MW; ++m) b[m] |= f[n][m];
            pos = pick + 1;
            added = true;
            ++nsel;
        } else if (added) {  // a new pass from node 0
            pos = 0;
            added = false;
        } else {
            break;
        }
    }
    for (int i = nsel + lane; i < N; i += 64) S[(size_t)tree * N + i] = -1;
    if (lane == 0) count[tree] = nsel;
}

// One workgroup (256 threads) per tree.  Every round, groups of TPN threads
// count the new pairs popcount(F & ~B) of all nodes outside S in parallel;
// wave 0 then takes, in generation order from the scan position, the first
// node whose parent is in S (or is the root) and whose utility test passes:
//     fl(p * T_AR) >= fl(fl(c * T_exp) + C_draft)
// (float32, no fused multiply-add).  The node joins S and its footprint is
// added to B.  When no node from the scan position passes, a new pass starts
// from node 0 if the last pass added a node, else the tree is done: at most
// 2 N + 1 rounds, and every wave sees the same decision.
template <bool STAGED>
__global__ __launch_bounds__(kSelThreads) void expand_kernel(ExpandArgs a, const float *__restrict__ P,
                                                             const uint32_t *__restrict__ F,
                                                             const float *__restrict__ Cd, int32_t *S,
                                                             int32_t *count) {
    extern __shared__ uint32_t lds[];
    const int N = a.N, W = a.W;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int tree = blockIdx.x;
    if (tree >= a.nt) return;
    const uint32_t *Ft = F + (size_t)tree * N * W;
    const uint32_t *Fs = STAGED ? lds : Ft;                      // [N * W]
    uint32_t *Bs = lds + (STAGED ? (size_t)N * W : 0);           // [W]
    float *Ps = reinterpret_cast<float *>(Bs + W);               // [N]
    float *Cs = Ps + N;                                          // [N]
    int *cnt = reinterpret_cast<int *>(Cs + N);                  // [N]
    uint32_t *inS = reinterpret_cast<uint32_t *>(cnt + N);       // [ceil(N / 32)]
    __shared__ int pick_sh;
    if (STAGED)
        for (int i = tid; i < N * W; i += kSelThreads) lds[i] = Ft[i];
    for (int i = tid; i < W; i += kSelThreads) Bs[i] = 0u;
    for (int i = tid; i < N; i += kSelThreads) {
        Ps[i] = P[(size_t)tree * N + i];
        Cs[i] = Cd ? Cd[(size_t)tree * N + i] : 0.f;
    }
    for (int i = tid; i < (N + 31) / 32; i += kSelThreads) inS[i] = 0u;
    __syncthreads();

    const int tpn = a.tpn;
    const int grp = tid / tpn, sub = tid - grp * tpn, ngrp = kSelThreads / tpn;
    int pos = 0, nsel = 0;
    bool added = false;
    for (int round = 0; round <= 2 * N; ++round) {
        // ---- new pairs of every node outside S ----
        for (int n0 = 0; n0 < N; n0 += ngrp) {
            const int n = n0 + grp;
            int c = 0;
            if (n < N && !((inS[n >> 5] >> (n & 31)) & 1u))
                for (int i = sub; i < W; i += tpn) c += __popc(Fs[(size_t)n * W + i] & ~Bs[i]);
            for (int off = tpn >> 1; off >= 1; off >>= 1) c += __shfl_xor(c, off);
            if (n < N && sub == 0) cnt[n] = c;
        }
        __syncthreads();
        // ---- wave 0: first passing node at or after the scan position ----
        if (wv == 0) {
            int pick = -1;
            for (int base = pos; base < N && pick < 0; base += 64) {
                const int n = base + lane;
                bool ok = false;
                if (n < N && !((inS[n >> 5] >> (n & 31)) & 1u)) {
                    const int par = a.parent[n];
                    if (par < 0 || ((inS[par >> 5] >> (par & 31)) & 1u)) {
                        const float num = __fmul_rn(Ps[n], a.t_ar);
                        const float den = __fadd_rn(__fmul_rn((float)cnt[n], a.t_exp), Cs[n]);
                        ok = num >= den;
                    }
                }
                const unsigned long long bal = __ballot(ok);
                if (bal) pick = base + __ffsll((long long)bal) - 1;
            }
            if (lane == 0) {
                if (pick >= 0) {
                    inS[pick >> 5] |= 1u << (pick & 31);
                    S[(size_t)tree * N + nsel] = pick;
                } else if (added) {
                    pick = -2;  // a new pass from node 0
                }
                pick_sh = pick;
            }
        }
        __syncthreads();
        const int pick = pick_sh;
        if (pick == -1) break;
        if (pick == -2) {
            pos = 0;
            added = false;
        } else {
            for (int i = tid; i < W; i += kSelThreads) Bs[i] |= Fs[(size_t)pick * W + i];
            pos = pick + 1;
            added = true;
            ++nsel;
        }
        __syncthreads();
    }
    for (int i = nsel + tid; i < N; i += kSelThreads) S[(size_t)tree * N + i] = -1;
    if (tid == 0) count[tree] = nsel;
}
}  // namespace

hipError_t launch_union_stats(const int32_t *topk_idx, int nL, int T, int k, int E, int32_t *counts,
                              float *reuse, hipStream_t s) {
    const size_t lds = (size_t)((E + 31) / 32) * 4;
    hipLaunchKernelGGL(union_stats_kernel, dim3(nL), dim3(256), lds, s, topk_idx, T, k, E, counts, reuse);
    return hipGetLastError();
}

size_t expand_lds_bytes(int N, int W, bool staged) {
    return ((staged ? (size_t)N * W : 0) + W + 3 * (size_t)N + (N + 31) / 32) * 4;
}

hipError_t launch_expand(ExpandArgs a, const float *P, const uint32_t *F, const float *Cd, int32_t *S,
                         int32_t *count, hipStream_t s) {
    if (a.N <= kSelWaveNodes && a.W <= 8 * 64 && a.nt >= kSelWaveMinTrees) {
        const dim3 g((a.nt + 3) / 4), b(256);
        const int mw = (a.W + 63) / 64;
        if (mw <= 1) hipLaunchKernelGGL(expand_wave_kernel<1>, g, b, 0, s, a, P, F, Cd, S, count);
        else if (mw <= 2) hipLaunchKernelGGL(expand_wave_kernel<2>, g, b, 0, s, a, P, F, Cd, S, count);
        else if (mw <= 3) hipLaunchKernelGGL(expand_wave_kernel<3>, g, b, 0, s, a, P, F, Cd, S, count);
        else if (mw <= 4) hipLaunchKernelGGL(expand_wave_kernel<4>, g, b, 0, s, a, P, F, Cd, S, count);
        else if (mw <= 6) hipLaunchKernelGGL(expand_wave_kernel<6>, g, b, 0, s, a, P, F, Cd, S, count);
        else hipLaunchKernelGGL(expand_wave_kernel<8>, g, b, 0, s, a, P, F, Cd, S, count);
        return hipGetLastError();
    }
    int tpn = 1;
    while (tpn * 2 <= 64 && tpn * 2 * a.N <= kSelThreads) tpn *= 2;
    a.tpn = tpn;
    const bool staged = expand_lds_bytes(a.N, a.W, true) <= (size_t)kSelectMaxLdsWords * 4;
    if (staged)
        hipLaunchKernelGGL(expand_kernel<true>, dim3(a.nt), dim3(kSelThreads), expand_lds_bytes(a.N, a.W, true), s,
                           a, P, F, Cd, S, count);
    else
        hipLaunchKernelGGL(expand_kernel<false>, dim3(a.nt), dim3(kSelThreads), expand_lds_bytes(a.N, a.W, false),
                           s, a, P, F, Cd, S, count);
    return hipGetLastError();
}

size_t select_lds_bytes(int N, int W, bool staged) {
    return ((staged ? (size_t)N * W : 0) + W + N + (N + 31) / 32) * 4;
}

hipError_t launch_select(int N, const float *P, const uint32_t *F, int W, int gamma, float eps, int nt,
                         int32_t *S, bool update_b, hipStream_t s) {
    if (N <= kSelWaveNodes && W <= 8 * 64 && nt >= kSelWaveMinTrees) {
        const dim3 g((nt + 3) / 4), b(256);
        const int ub = update_b ? 1 : 0;
        const int mw = (W + 63) / 64;
        if (mw <= 1) hipLaunchKernelGGL(select_wave_kernel<1>, g, b, 0, s, N, P, F, W, gamma, eps, nt, ub, S);
        else if (mw <= 2) hipLaunchKernelGGL(select_wave_kernel<2>, g, b, 0, s, N, P, F, W, gamma, eps, nt, ub, S);
        else if (mw <= 3) hipLaunchKernelGGL(select_wave_kernel<3>, g, b, 0, s, N, P, F, W, gamma, eps, nt, ub, S);
        else if (mw <= 4) hipLaunchKernelGGL(select_wave_kernel<4>, g, b, 0, s, N, P, F, W, gamma, eps, nt, ub, S);
        else if (mw <= 6) hipLaunchKernelGGL(select_wave_kernel<6>, g, b, 0, s, N, P, F, W, gamma, eps, nt, ub, S);
        else hipLaunchKernelGGL(select_wave_kernel<8>, g, b, 0, s, N, P, F, W, gamma, eps, nt, ub, S);
        return hipGetLastError();
    }
    // threads per node: the largest power of two <= min(64, 256 / N), at least 1
    int tpn = 1;
    while (tpn * 2 <= 64 && tpn * 2 * N <= kSelThreads) tpn *= 2;
    if (select_lds_bytes(N, W, true) <= (size_t)kSelectMaxLdsWords * 4)
        hipLaunchKernelGGL(select_kernel<true>, dim3(nt), dim3(kSelThreads), select_lds_bytes(N, W, true), s, N, P,
                           F, W, gamma, eps, nt, tpn, update_b ? 1 : 0, S);
    else
        hipLaunchKernelGGL(select_kernel<false>, dim3(nt), dim3(kSelThreads), select_lds_bytes(N, W, false), s, N,
                           P, F, W, gamma, eps, nt, tpn, update_b ? 1 : 0, S);
    return hipGetLastError();
}

}  // namespace moe
