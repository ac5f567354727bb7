// Internal declarations shared by the HIP translation units of libmoeverify.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_verify.h"

namespace moe {

constexpr int kMaxSegments = 64;  // sequences of one call (ragged verify, per-sequence bias)

// Everything one verify-layer call needs, passed by value to every kernel.
struct VerifyParams {
    int T, H, I, E, k, wdtype;
    int cols;        // B-operand columns in use: 2T (high/low split) or T
    int cstride;     // B-operand column stride (= cols; lanes past the used columns clamp)
    int split;       // 1 if activations enter the products as a bf16 hi/lo pair
    int has_shared;  // always-on shared expert present
    int bias_on, cap;
    int nseg;        // bias per sequence: tokens seg_off[s] .. seg_off[s+1]-1 form sequence s (0: pooled)
    int seg_off[kMaxSegments + 1];
    int max_slots;   // min(E, T k) + has_shared: bound on the device slot count
    int gu_async_x;  // gate-up: operand staging runs alongside the routing (own LDS region)
    float alpha;

    const float *x, *Wr;
    const void *W_gu, *W_d, *Wsh_gu, *Wsh_d;
    const float *s_gu, *s_d, *ssh_gu, *ssh_d;
    const float *w_conf;
    float *y;

    // routing outputs (caller buffers or workspace)
    float *logits;
    int *topk_idx;
    float *topk_w;
    int *union_experts, *csr_ptr, *csr_tok;
    float *csr_w;
    int *pstar;                            // [max(1, nseg), cap]: each sequence's P*, ascending
    int *union_size_out, *pstar_size_out;  // may be null; pstar_size_out [max(1, nseg)]

    // workspace-only tables
    int *meta;         // [0] union size U, [1] slots (U + shared), [2] sum of |P*| over the sequences
    int *slot_expert;  // [slots] expert id per slot (E = shared expert)
    float *tokw;       // [slots * T] gate weight of token t in slot s (0 if not routed)
    int *tokpos;       // [slots * T] row of ydown for (slot, token), -1 if not routed
    int *tpos;         // [T * k] row of ydown for (token, rank)
    uint16_t *xB;      // [H * cols] bf16 activations in the matrix-core operand order
    uint16_t *hB;      // [max_slots * I * cols] bf16 hidden activations, weighted
    float *h32;        // [max_slots * T * I] float32 hidden (float32 weights)
    float *ydown;      // [(T * k + T) * H] per-(token, expert) outputs (float32 weights)
    float *ypart;      // [kDownMaxGrid * 2 * kDownMaxRowTiles * T * 16] down: partial row groups (bf16 / fp8)
    int *tile_cnt;     // [H / 16] down: pieces finished per row group (zeroed by the router kernel)
    int *gu_ticket;    // [1] gate-up: tail items handed out so far (zeroed by the router kernel)
    float *gu_part;    // [ks][max_slots][I][2][T] gate-up: partial gate and up sums of a split contraction
};

constexpr int kWaveSize = 64;

// Launchers (enqueue only; return hipError_t of the launch).
// Optional timing of one launch: with an event set, the kernel is launched
// through hipExtLaunchKernelGGL so that the events mark the start and the
// end of its execution on the stream (either may be null, so a stage can
// span two launches).
struct KernelEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};

hipError_t launch_router(const VerifyParams &p, hipStream_t s, KernelEvents ev = {});
hipError_t launch_route(const VerifyParams &p, hipStream_t s, KernelEvents ev = {});
hipError_t launch_gateup(const VerifyParams &p, int n_cu, hipStream_t s, KernelEvents ev = {});
bool gateup_fuses_routing(const VerifyParams &p);  // routing runs in the gate-up prologue
// Workgroups sharing the contraction of one gate-up item (1: none); with
// more than one, launch_swiglu finishes the hidden activations.
int gateup_ksplit(const VerifyParams &p);
hipError_t launch_swiglu(const VerifyParams &p, int ks, hipStream_t s, KernelEvents ev = {});
hipError_t launch_down(const VerifyParams &p, int n_cu, hipStream_t s, KernelEvents ev = {});
hipError_t launch_combine(const VerifyParams &p, hipStream_t s, KernelEvents ev = {});
hipError_t launch_pack(const void *src, void *dst, int E, int R, int K, int esz, int interleave, int half,
                       hipStream_t s);
hipError_t launch_read_probe(const void *src, size_t bytes, uint32_t *sink, int n_cu, hipStream_t s);
hipError_t launch_union_stats(const int32_t *topk_idx, int nL, int T, int k, int E, int32_t *counts,
                              float *reuse, hipStream_t s);
hipError_t launch_select(int N, const float *P, const uint32_t *F, int W, int gamma, float eps,
                         int nt, int32_t *S, bool update_b, hipStream_t s);

// Arguments of the expansion kernel (parents by value: no device copy).
constexpr int kMaxExpandNodes = 1024;
struct ExpandArgs {
    int N, W, nt, tpn;
    float t_ar, t_exp;
    int16_t parent[kMaxExpandNodes];
};
size_t expand_lds_bytes(int N, int W, bool staged);
hipError_t launch_expand(ExpandArgs a, const float *P, const uint32_t *F, const float *Cd, int32_t *S,
                         int32_t *count, hipStream_t s);

// Ragged verify: segment offsets by value, depth gating limits.
constexpr int kGateMaxSeq = 64;
constexpr int kGateMaxDepth = 64;
constexpr int kGateMaxWords = 1024;  // (layer, expert) pairs <= 32768: 64 KB of uint16 counters
struct SegmentArgs {
    int S;
    int off[kMaxSegments + 1];
};
hipError_t launch_segment_stats(const int32_t *topk_idx, int nL, int T, int k, int E, const SegmentArgs &a,
                                int32_t *per, int32_t *total, hipStream_t s);
size_t gate_lds_bytes(int W);
hipError_t launch_gate_depths(const float *c, const uint32_t *Ep, int S, int Dmax, int W, float t_base,
                              float t_exp, int32_t *d, hipStream_t s);

// Host helpers of the C ABI (moe_verify.cpp): the error message of the
// calling thread, and the validation plus workspace size of a verify call.
int set_error(int code, const char *msg);
int verify_needs(const ::moe_layer *layer, int T, const ::moe_bias *bias, size_t *need);

// Limits used by the kernels.
constexpr int kMaxTokens = 64;
constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 32;
constexpr int kDownMaxGrid = 1024;    // workgroups of the matrix-core down kernel
constexpr int kDownMaxRowTiles = 4;  // row tiles per down work unit
constexpr int kSelectMaxLdsWords = 16384;  // 64 KB of footprint words per tree

}  // namespace moe
