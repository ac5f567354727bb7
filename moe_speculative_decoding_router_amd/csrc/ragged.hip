// Ragged, confidence-gated verify: per-sequence unique-expert statistics of
// a call whose tokens are grouped by sequence, and the per-sequence depth
// choice.
//
// [W-vs-D] = summary of the width-vs-depth article, section 2 (where to
// spend depth): sequences get their own speculation depth in one verify
// step; a batch-wide depth is taken from the live sequences' confidences,
// then each sequence is truncated greedily while that raises the expected
// throughput.  Expected tokens of sequence s at depth d: 1 + c[s,1] + ... +
// c[s,d] (cumulative draft confidences); expected step time: t_base + t_exp
// * (distinct (layer, expert) pairs over all verified tokens), the cost
// model of the expansion step ([S2-MoE] component 1).
#include "common.h"
#include "internal.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// Per-(layer, segment) unique experts.  One workgroup per (layer, segment);
// segment S is the whole call.  LDS bitset of E bits, popcount.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void segment_stats_kernel(const int32_t *__restrict__ topk, int T, int k, int E,
                                                            SegmentArgs a, int32_t *per, int32_t *total) {
    extern __shared__ unsigned bits[];
    __shared__ int wsum[4];
    const int l = blockIdx.x, s = blockIdx.y;
    const int nw = (E + 31) / 32;
    for (int i = threadIdx.x; i < nw; i += 256) bits[i] = 0u;
    __syncthreads();
    const int r0 = s < a.S ? a.off[s] : 0, r1 = s < a.S ? a.off[s + 1] : T;
    const int32_t *rows = topk + ((size_t)l * T + r0) * k;
    for (int i = threadIdx.x; i < (r1 - r0) * k; i += 256) {
        const int e = rows[i];
        if (e >= 0 && e < E) atomicOr(&bits[e >> 5], 1u << (e & 31));
    }
    __syncthreads();
    int c = 0;
    for (int i = threadIdx.x; i < nw; i += 256) c += __popc(bits[i]);
    c = wave_sum_int(c);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        const int n = wsum[0] + wsum[1] + wsum[2] + wsum[3];
        if (s < a.S)
            per[(size_t)l * a.S + s] = n;
        else
            total[l] = n;
    }
}

// ---------------------------------------------------------------------------
// Depth gating.  One workgroup of 256 threads.  cnt[pair] counts the
// verified tokens that hold the pair, so the distinct-pair count U follows
// every token added or removed exactly; each thread owns whole words of the
// bitsets (no two threads touch one counter).  Throughput comparisons are
// made by thread 0 in float32 with fixed summation orders and broadcast.
// ---------------------------------------------------------------------------
constexpr int kGateThreads = 256;

__device__ __forceinline__ int block_sum_int(int v, int *red) {
    v = wave_sum_int(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const int r = red[0] + red[1] + red[2] + red[3];
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kGateThreads) void gate_depths_kernel(const float *__restrict__ c,
                                                                   const uint32_t *__restrict__ Ep, int S, int Dmax,
                                                                   int W, float t_base, float t_exp, int32_t *dout) {
    extern __shared__ uint16_t cnt[];                 // [W * 32]
    __shared__ float apre[kGateMaxSeq][kGateMaxDepth + 1];  // expected tokens at each depth
    __shared__ int dS[kGateMaxSeq];
    __shared__ int red[4];
    __shared__ int flag_sh;
    __shared__ float th_sh;
    const int tid = threadIdx.x;
    const int D1 = Dmax + 1;
    for (int i = tid; i < W * 32; i += kGateThreads) cnt[i] = 0;
    if (tid < S) {
        float acc = 1.f;
        apre[tid][0] = acc;
        for (int j = 1; j <= Dmax; ++j) {
            acc = __fadd_rn(acc, c[(size_t)tid * D1 + j]);
            apre[tid][j] = acc;
        }
    }
    __syncthreads();
    auto word = [&](int s, int j, int w) { return Ep[((size_t)s * D1 + j) * W + w]; };
    // add (+1) or remove (-1) token (s, j); returns the change of U
    auto apply = [&](int s, int j, int sign) {
        int du = 0;
        for (int w = tid; w < W; w += kGateThreads) {
            unsigned b = word(s, j, w);
            while (b) {
                const int bit = __ffs(b) - 1;
                b &= b - 1;
                uint16_t &x = cnt[w * 32 + bit];
                if (sign > 0) {
                    du += x == 0;
                    ++x;
                } else {
                    --x;
                    du -= x == 0;
                }
            }
        }
        return block_sum_int(du, red);
    };
    auto throughput = [&](int U) {  // thread 0 only: fl(total / fl(t_base + fl(t_exp * U)))
        float total = 0.f;
        for (int s = 0; s < S; ++s) total = __fadd_rn(total, apre[s][dS[s]]);
        return __fdiv_rn(total, __fadd_rn(t_base, __fmul_rn(t_exp, (float)U)));
    };

    // ---- batch-wide depth: the smallest D with the largest throughput ----
    int U = 0, bestD = 0;
    float best = 0.f;
    for (int D = 0; D <= Dmax; ++D) {
        for (int s = 0; s < S; ++s) U += apply(s, D, +1);
        if (tid == 0) {
            for (int s = 0; s < S; ++s) dS[s] = D;
            const float th = throughput(U);
            if (D == 0 || th > best) {
                best = th;
                bestD = D;
            }
            flag_sh = bestD;
            th_sh = best;
        }
        __syncthreads();
    }
    bestD = flag_sh;
    best = th_sh;
    for (int D = Dmax; D > bestD; --D)
        for (int s = 0; s < S; ++s) U += apply(s, D, -1);
    if (tid < S) dS[tid] = bestD;
    __syncthreads();

    // ---- greedy truncation, sequence by sequence ----
    for (int s = 0; s < S; ++s) {
        while (true) {
            const int d = dS[s];
            if (d == 0) break;
            // pairs that only token (s, d) holds leave the union with it
            int only = 0;
            for (int w = tid; w < W; w += kGateThreads) {
                unsigned b = word(s, d, w);
                while (b) {
                    const int bit = __ffs(b) - 1;
                    b &= b - 1;
                    only += cnt[w * 32 + bit] == 1;
                }
            }
            only = block_sum_int(only, red);
            if (tid == 0) {
                dS[s] = d - 1;
                const float th = throughput(U - only);
                if (th > best) {
                    best = th;
                    flag_sh = 1;
                } else {
                    dS[s] = d;
                    flag_sh = 0;
                }
            }
            __syncthreads();
            if (!flag_sh) break;
            U += apply(s, d, -1);
        }
    }
    if (tid < S) dout[tid] = dS[tid];
}

}  // namespace

hipError_t launch_segment_stats(const int32_t *topk_idx, int nL, int T, int k, int E, const SegmentArgs &a,
                                int32_t *per, int32_t *total, hipStream_t s) {
    const size_t lds = (size_t)((E + 31) / 32) * 4;
    hipLaunchKernelGGL(segment_stats_kernel, dim3(nL, a.S + 1), dim3(256), lds, s, topk_idx, T, k, E, a, per,
                       total);
    return hipGetLastError();
}

size_t gate_lds_bytes(int W) { return (size_t)W * 32 * sizeof(uint16_t); }

hipError_t launch_gate_depths(const float *c, const uint32_t *Ep, int S, int Dmax, int W, float t_base,
                              float t_exp, int32_t *d, hipStream_t s) {
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(gate_depths_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)gate_lds_bytes(W)) != hipSuccess)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(gate_depths_kernel, dim3(1), dim3(kGateThreads), gate_lds_bytes(W), s, c, Ep, S, Dmax, W,
                       t_base, t_exp, d);
    return hipGetLastError();
}

}  // namespace moe
