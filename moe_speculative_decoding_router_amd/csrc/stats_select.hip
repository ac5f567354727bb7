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

// One wave per tree.  The tree's footprints are staged in LDS with 16-byte
// loads; the buffer B and the chosen set live in LDS too.  For each node the
// 64 lanes popcount consecutive words of F & ~B and the count is reduced
// across the wave, so every score is computed identically in all lanes.
__global__ __launch_bounds__(64) void select_kernel(int N, const float *__restrict__ P,
                                                    const uint32_t *__restrict__ F, int W, int gamma,
                                                    float eps, int nt, int32_t *S) {
    extern __shared__ uint32_t lds[];
    uint32_t *Fs = lds;                    // [N * W]
    uint32_t *Bs = Fs + (size_t)N * W;     // [W]
    uint32_t *chosen = Bs + W;             // [ceil(N / 32)]
    const int lane = threadIdx.x;
    const int tree = blockIdx.x;
    if (tree >= nt) return;
    const uint32_t *Ft = F + (size_t)tree * N * W;
    const float *Pt = P + (size_t)tree * N;
    const int nwords = N * W;
    const bool aligned16 = ((nwords & 3) == 0) && ((reinterpret_cast<uintptr_t>(Ft) & 15) == 0);
    if (aligned16) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(Ft);
        u32x4 *dst = reinterpret_cast<u32x4 *>(Fs);
        for (int i = lane; i < nwords / 4; i += 64) dst[i] = __builtin_nontemporal_load(src + i);
    } else {
        for (int i = lane; i < nwords; i += 64) Fs[i] = Ft[i];
    }
    for (int i = lane; i < W; i += 64) Bs[i] = 0u;
    for (int i = lane; i < (N + 31) / 32; i += 64) chosen[i] = 0u;
    __syncthreads();

    for (int r = 0; r < gamma; ++r) {
        int best = -1;
        float best_s = -INFINITY;
        for (int n = 0; n < N; ++n) {
            if ((chosen[n >> 5] >> (n & 31)) & 1u) continue;
            int c = 0;
            for (int i = lane; i < W; i += 64) c += __popc(Fs[(size_t)n * W + i] & ~Bs[i]);
            c = wave_sum_int(c);
            const float sc = __fdiv_rn(Pt[n], __fadd_rn((float)c, eps));
            if (sc > best_s) {  // strict: equal scores keep the lower node index
                best_s = sc;
                best = n;
            }
        }
        if (best < 0) {  // only reachable with NaN probabilities: lowest unchosen node
            for (int n = 0; n < N; ++n)
                if (!((chosen[n >> 5] >> (n & 31)) & 1u)) {
                    best = n;
                    break;
                }
        }
        __syncthreads();
        if (lane == 0) {
            S[(size_t)tree * gamma + r] = best;
            chosen[best >> 5] |= 1u << (best & 31);
        }
        for (int i = lane; i < W; i += 64) Bs[i] |= Fs[(size_t)best * W + i];
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
    const size_t lds = ((size_t)N * W + W + (N + 31) / 32) * 4;
    hipLaunchKernelGGL(select_kernel, dim3(nt), dim3(64), lds, s, N, P, F, W, gamma, eps, nt, S);
    return hipGetLastError();
}

}  // namespace moe
