/*
 * moe_verify.h -- C ABI of libmoeverify.so, the union-expert MoE verify layer
 * and cost-aware draft selection for MI355X (gfx950).
 *
 * Pages cited:
 *   [EcoSpec] review of "Less Experts, Faster Decoding: Cost-Aware Speculative
 *             Decoding for Mixture-of-Experts";
 *   [S2-MoE]  walkthrough of S^2-MoE (self-speculative decoding for MoE on
 *             edge devices);
 *   [W-vs-D]  summary of the width-vs-depth article (batch versus
 *             speculation for MoE on one GPU).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns every
 *     buffer; the library allocates nothing, keeps no per-call state and never
 *     synchronises the stream.  Work is enqueued on `stream` (a hipStream_t
 *     passed as void*; NULL = the null stream); outputs are valid once that
 *     work completes.  Calls on different streams may run concurrently if
 *     their output and workspace buffers are disjoint.
 *   - Arrays are dense, row-major, without padding.
 *   - Return codes: 0 = OK, MOE_EINVAL (null pointer, shape or range error),
 *     MOE_ENOTSUP (shape/dtype outside the built kernels), MOE_EWORKSPACE
 *     (workspace too small), MOE_EHIP (a HIP launch failed).  Arguments are
 *     validated on the host before anything is enqueued; on a non-zero return
 *     nothing has been enqueued, except after MOE_EHIP.  moe_last_error()
 *     gives a message for the calling thread's last non-zero return.
 *   - Non-finite inputs give undefined (but memory-safe) results.
 */
#ifndef MOE_VERIFY_H
#define MOE_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_EINVAL (-1)
#define MOE_ENOTSUP (-2)
#define MOE_EWORKSPACE (-3)
#define MOE_EHIP (-4)

#define MOE_MAX_TOKENS 64
#define MOE_MAX_EXPERTS 512
#define MOE_MAX_TOPK 32
#define MOE_NUM_STAGES 5   /* router, route, gate-up, down, combine */
#define MOE_MAX_SEGMENTS 64 /* sequences of one call with a preferred set of their own */

/* Expert weight formats.  MOE_FP8_E4M3 is OCP FP8 E4M3FN with one float32
 * scale per 128 x 128 block (row block, column block), row-major over blocks:
 * W[i][j] = e4m3fn(q[i][j]) * scale[i / 128][j / 128]. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/* One MoE layer.  Routed experts use SwiGLU:
 *   FFN_e(x) = W_d,e (SiLU(W_g,e x) * (W_u,e x)),  SiLU(z) = z / (1 + e^-z).
 * Logical shapes: the gate-up matrix [2I, H] holds the I gate rows followed by
 * the I up rows; the down matrix is [H, I].
 *   Wr    [E, H]      float32 router, row-major
 *   W_gu  [E, 2I, H]  float32: row-major.  bf16 / fp8: PACKED by
 *                     moe_pack_weights(gate_up = 1), same byte size.
 *   W_d   [E, H, I]   float32: row-major.  bf16 / fp8: PACKED by
 *                     moe_pack_weights(gate_up = 0).
 *   s_gu  [E, 2I/128, H/128] float32, s_d [E, H/128, I/128] float32: fp8 block
 *         scales of the LOGICAL matrices, row-major; NULL otherwise.
 *   Wsh_gu, Wsh_d (+ ssh_gu, ssh_d for fp8): optional always-on shared expert
 *         in the same formats with E = 1, weight 1 for every token, outside the
 *         union; NULL if absent. */
typedef struct {
    int32_t H, I, E, k;
    int32_t wdtype; /* moe_dtype */
    const float *Wr;
    const void *W_gu;
    const void *W_d;
    const float *s_gu, *s_d;
    const void *Wsh_gu, *Wsh_d;
    const float *ssh_gu, *ssh_d;
} moe_layer;

/* Optional reuse-aware soft routing bias ([S2-MoE] component 2, steps 1-3,
 * Fig. 5), applied before the union is formed:
 *   g_e    = sum_b w_conf[b] * softmax(l_b)_e * [e in TopK(l_b)]
 *   P*     = the first `cap` experts by (g desc, index asc) with g_e > 0
 *   lambda_b = alpha * (l_b,(1) - l_b,(k+1))        (float32, no FMA; 0 if k == E)
 *   l'_b,e = l_b,e + lambda_b for e in P*           (float32)
 * The selection is the top-k of l'; gate weights are the softmax of the
 * ORIGINAL logits over that selection.  Requires k <= cap <= E,
 * 0 <= alpha < 1, w_conf [T] float32 (device) non-negative.
 * Sequences ([W-vs-D] section 2, ragged speculation: one call verifies the
 * drafts of several sequences): with nseg = 0 the sums run over all T tokens
 * of the call (one P*); with nseg > 0 the tokens are grouped by sequence,
 * rows seg_off[s] .. seg_off[s+1]-1 forming sequence s, and g and P* are
 * computed over each sequence's own tokens, each token biased toward its own
 * sequence's P* (so no token is pushed toward experts that only other
 * sequences chose).  seg_off (host) [nseg + 1], 0 = seg_off[0] <= ... <=
 * seg_off[nseg] = T (empty sequences allowed), read during the call only;
 * nseg <= MOE_MAX_SEGMENTS.  Errors: EINVAL. */
typedef struct {
    int32_t cap;
    float alpha;
    const float *w_conf;
    int32_t nseg;
    const int32_t *seg_off;
} moe_bias;

/* Optional outputs of moe_verify_layer (device pointers); any field may be
 * NULL, in which case the value lives only in the workspace.
 *   logits [T, E] f32          router logits
 *   topk_idx [T, k] i32        selected experts in rank order (logit desc,
 *                              index asc; biased logits when bias is on)
 *   topk_w [T, k] f32          gate weights
 *   union_size [1] i32         number of unique routed experts U
 *   union_experts [E] i32      first U entries: the union, ascending
 *   csr_ptr [E + 1] i32        first U + 1 entries: offsets into csr_tok
 *   csr_tok [T * k] i32        tokens of each union expert, ascending
 *   csr_w [T * k] f32          gate weight of each (expert, token) entry
 *   pstar [S, cap] i32, pstar_size [S] i32   preferred set of each sequence
 *                              (S = max(1, nseg); row s holds sequence s's P*
 *                              ascending in its first pstar_size[s] entries;
 *                              bias only; without the bias pstar_size[0] = 0)
 *   events: NULL or (host) array of 2 * MOE_NUM_STAGES hipEvent_t handles
 *           created by the caller with timing enabled.  Events 2i and 2i + 1
 *           mark the start and the end of the execution of stage i's kernel
 *           on `stream` (the kernel is launched with hipExtLaunchKernelGGL);
 *           a stage that runs no kernel in this call (the route stage when
 *           the gate-up kernel routes, the combine stage for bf16/fp8)
 *           records both at that point of the stream.  When the gate-up
 *           contraction is split over workgroups (the activation operand
 *           too large for one compute unit's LDS), the gate-up stage spans
 *           the gate-up kernel and the SwiGLU combine that follows it. */
typedef struct {
    float *logits;
    int32_t *topk_idx;
    float *topk_w;
    int32_t *union_size;
    int32_t *union_experts;
    int32_t *csr_ptr;
    int32_t *csr_tok;
    float *csr_w;
    int32_t *pstar;
    int32_t *pstar_size;
    void *const *events;
} moe_aux;

/* Packs row-major expert weights into the matrix-core tile layout that
 * moe_verify_layer streams (bf16 or fp8; one-time weight preparation).
 * src [E, rows, K] row-major (device), dst (device, same byte size, must not
 * overlap src).  gate_up = 1: src is the gate-up matrix, rows = 2I, K = H;
 * gate_up = 0: the down matrix, rows = H, K = I.
 * Layout of dst: per expert, 1 KB tiles of 16 rows x 32 k (bf16) or 16 rows x
 * 64 k (fp8); inside a tile, 16-byte slot l = 0..63 holds tile row l % 16 at
 * k offset (l / 16) * 8 (bf16) or (l / 16) * 16 (fp8), the operand order of
 * v_mfma_f32_16x16x32_bf16, so a wave reads 1 KB of contiguous memory per
 * load.  gate_up = 1: tiles ordered row-tile major, then K-tile; row tile rt
 * holds gate rows 8 rt .. 8 rt + 7 as tile rows 0..7 and up rows
 * I + 8 rt .. I + 8 rt + 7 as tile rows 8..15.  gate_up = 0: tiles ordered in
 * groups of 4 row tiles (64 rows): group major, then K-tile, then the row
 * tile inside the group (rows 16 (4 grp + r) .. + 15).
 * Requires K % 32 (bf16) / K % 64 (fp8) == 0, rows % 32 == 0 for gate_up = 1
 * and rows % 64 == 0 for gate_up = 0. */
int moe_pack_weights(const void *src, void *dst, int32_t E, int32_t rows, int32_t K, int32_t wdtype,
                     int32_t gate_up, void *stream);

/* Streaming-read probe (a measurement aid, not part of the verify path):
 * reads `bytes` of device memory at src with the FFN kernels' load pattern
 * (16-byte non-temporal loads, 1 KB contiguous per wave and load, one
 * workgroup of 8 waves per compute unit) and XORs the 32-bit words into
 * *checksum (device; the caller zeroes it first), so the bytes are used.
 * Its rate is the achievable streaming ceiling against which the FFN
 * kernels' HBM rates are read.  bytes: positive multiple of 16; src 16-byte
 * aligned.  Asynchronous on `stream`. */
int moe_stream_read(const void *src, size_t bytes, uint32_t *checksum, void *stream);

/* Workspace bytes that moe_verify_layer needs for this layer, T and bias
 * (host computation only; bias may be NULL).  Returns 0 for invalid input. */
size_t moe_verify_workspace_bytes(const moe_layer *layer, int32_t T, const moe_bias *bias);

/* The MoE-layer verify step ([EcoSpec] §1-§2: the verify cost at a layer is
 * the union of the experts the verified tokens route to; [S2-MoE] motivation,
 * challenge 2).  For T tokens x [T, H] float32 (device):
 *   logits = x Wr^T; per-token top-k (+ optional bias); gate weights;
 *   union U of the selected experts and the token-by-expert grouping;
 *   y[t] = sum_j w_tj FFN_{e_tj}(x_t) (+ shared expert), y [T, H] float32.
 * Each unique expert's weights are read once and applied to all of its tokens.
 * layer (host), bias (host, NULL = off), aux (host, NULL = no extra outputs).
 * ws: device workspace of at least moe_verify_workspace_bytes() bytes,
 * 256-byte aligned; its contents need no initialisation and are clobbered.
 * y may be x itself (x is read before y is first written); it must not
 * overlap the workspace, the aux outputs or the weights.
 * Limits: 1 <= T <= 64, 1 <= k <= min(E, 32), E <= 512; bf16: H a multiple of
 * 64 and I of 32; fp8: H, I multiples of 128.  Numerics: router GEMV and FFN
 * accumulate in float32; activations enter the bf16/fp8 matrix-core
 * products as a bf16 high/low pair when T <= 8 (as one bf16 otherwise). */
int moe_verify_layer(const moe_layer *layer, const float *x, int32_t T, const moe_bias *bias,
                     float *y, moe_aux *aux, void *ws, size_t ws_bytes, void *stream);

/* moe_verify_layer for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, results and errors as moe_verify_layer,
 * without the workspace: the call uses a file-scope device array of
 * MOE_NOALLOC_SCRATCH_BYTES bytes, one per GPU the library runs on, held
 * until the process ends.  It allocates nothing (no hipMalloc, no allocating
 * library routine).  Every call on a GPU shares that GPU's array and leaves
 * it holding that call's workspace; calls that overlap on one GPU (other
 * streams, other threads) race on it and give undefined results, so
 * serialise them.  A call whose workspace (moe_verify_workspace_bytes)
 * exceeds MOE_NOALLOC_SCRATCH_BYTES returns MOE_EWORKSPACE before anything
 * is enqueued.  The first call on each device looks up the array's device
 * address (hipGetSymbolAddress) and keeps it; make that call outside stream
 * capture. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int moe_verify_layer_noalloc(const moe_layer *layer, const float *x, int32_t T, const moe_bias *bias,
                             float *y, moe_aux *aux, void *stream);

/* Per-layer union statistics ([S2-MoE] motivation, challenge 2: reuse ratio
 * = number of distinct experts over s * k).  topk_idx [nL, T, k] int32
 * (device), entries in [0, E) (entries outside are ignored);
 * counts [nL] int32 = |union of layer l|, reuse [nL] float32 =
 * counts / (T * k), correctly rounded.  Limits: 1 <= E <= 65536. */
int union_stats(const int32_t *topk_idx, int32_t nL, int32_t T, int32_t k, int32_t E,
                int32_t *counts, float *reuse, void *stream);

/* EcoSpec cost-aware greedy draft selection ([EcoSpec] §3.2 global expert
 * buffer, §3.3 score equation and greedy selection), for nt trees with the
 * same shape.
 *   parent (host) [N]: BFS order, parent[i] in [-1, i) (-1 = child of the
 *                  root); validated, so ties go to ancestors.
 *   P [nt, N] float32: path probabilities.
 *   Epred [nt, N, W] uint32: path footprints, bit b = layer * E + expert in
 *                  word b / 32, LSB first.
 * For each tree, starting from an empty buffer B, gamma times: score every
 * unchosen node t as P_t / (popcount(F_t & ~B) + eps) in float32 (add, then
 * divide, each correctly rounded), choose the highest score (ties: lowest
 * node index), B |= F_chosen.  S [nt, gamma] int32 receives node ids in
 * choice order.  P, Epred and S may be NULL when gamma == 0 or nt == 0.
 * Limits: 0 <= gamma <= N <= 4096, 1 <= W <= 4096, eps > 0.  Batches of
 * 512 or more trees with N <= 16 and W <= 512 run one wave per tree with the
 * tree in registers; otherwise one workgroup per tree, and a tree whose
 * footprints fit in 64 KB of LDS (N * W + W + N + N / 32 <= 16384 words) is
 * staged there once, a larger one read from global memory every round.
 * Every path gives the same selections. */
int select_drafts(const int32_t *parent, int32_t N, const float *P, const uint32_t *Epred,
                  int32_t W, int32_t gamma, float eps, int32_t nt, int32_t *S, void *stream);

/* Per-sequence unique experts of a ragged verify call ([W-vs-D] section 2,
 * ragged speculation: sequences verify different numbers of tokens in one
 * call).  The T tokens of the call are grouped by sequence: rows
 * offsets[s] .. offsets[s+1]-1 belong to sequence s.
 *   topk_idx [nL, T, k] int32 (device), entries outside [0, E) ignored
 *   offsets  (host) [S + 1] int32, 0 = offsets[0] <= ... <= offsets[S] = T
 *   per      [nL, S] int32 out: distinct experts of each sequence's tokens
 *   total    [nL] int32 out: distinct experts of the whole call
 * Limits: 1 <= S <= 64.  Errors: EINVAL (NULL, shapes, offsets). */
int union_stats_segments(const int32_t *topk_idx, int32_t nL, int32_t T, int32_t k, int32_t E,
                         const int32_t *offsets, int32_t S, int32_t *per, int32_t *total, void *stream);

/* Confidence-gated per-sequence depths ([W-vs-D] section 2): one batch-wide
 * depth, then greedy per-sequence truncation, maximising the expected
 * throughput
 *     sum_s (1 + c[s,1] + ... + c[s,d_s]) / (t_base + t_exp * U(d)),
 * where U(d) is the number of distinct (layer, expert) pairs over every
 * verified token (the root j = 0 and drafts 1..d_s of each sequence).  The
 * batch-wide depth is the smallest D in 0..Dmax with the largest throughput;
 * then, for s = 0..S-1 in order, d_s is lowered one step at a time while that
 * raises the throughput strictly.  Float32 as fl(total / fl(t_base +
 * fl(t_exp * U))) with A_s summed over j ascending and the total over s
 * ascending.
 *   c     [S, Dmax + 1] float32 cumulative draft confidences (column 0 unused)
 *   Epred [S, Dmax + 1, W] uint32 expert bitsets of each token
 *   d     [S] int32 out: the depths
 * Limits: S <= 64, Dmax <= 64, W <= 1024.  Errors: EINVAL. */
int gate_depths(const float *c, const uint32_t *Epred, int32_t S, int32_t Dmax, int32_t W, float t_base,
                float t_exp, int32_t *d, void *stream);

/* Static-cost ablation of the selection ([EcoSpec] section 4.3): the same
 * greedy loop and arguments as select_drafts, but every node pays the size
 * of its whole footprint, popcount(F_t), and B is never updated, so the
 * result is the top-gamma of P_t / (popcount(F_t) + eps) in float32 with
 * ties to the lower node index. */
int select_drafts_static(const int32_t *parent, int32_t N, const float *P, const uint32_t *Epred, int32_t W,
                         int32_t gamma, float eps, int32_t nt, int32_t *S, void *stream);

/* Utility-driven adaptive expansion of draft trees ([S2-MoE] component 1,
 * routing-aware adaptive speculative expansion).  Per tree, a draft token i
 * joins the expansion set S while its utility
 *     U_i = p_i * T_AR / (|E_i \ union_{j in S} E_j| * T_exp + C_i^draft)
 * is at least 1: candidates are examined in generation (BFS) order, a node
 * only once its parent is in S (or it is a child of the root), and passes
 * repeat until one adds no node.  The test is evaluated in float32 as
 * fl(p * t_ar) >= fl(fl(c * t_exp) + c_draft) with the exact count c of new
 * (layer, expert) pairs; the resulting set does not depend on the order.
 *   parent  (host) [N] int32, BFS order, -1 = child of the root, parent < child
 *   P       [nt, N] float32 acceptance probabilities (e.g. path probabilities)
 *   Epred   [nt, N, W] uint32 footprint bitsets, as for select_drafts (own or
 *           whole-path footprints give the same result, since S is
 *           prefix-closed)
 *   t_ar    saving of one accepted token (one autoregressive step), >= 0
 *   t_exp   latency of one new (layer, expert) pair, >= 0
 *   c_draft [nt, N] float32 draft-side cost of each node, or NULL (zero)
 *   S       [nt, N] int32 out: nodes in the order they join, then -1
 *   count   [nt] int32 out: size of each set
 * Limits: N <= 1024, W <= 4096.  Footprints are staged in LDS when
 * N * W + W + 3 N + N / 32 <= 16384 words, else read from global memory.
 * Errors: EINVAL (NULL, shapes, parent order, t_ar / t_exp). */
int expand_drafts(const int32_t *parent, int32_t N, const float *P, const uint32_t *Epred, int32_t W,
                  float t_ar, float t_exp, const float *c_draft, int32_t nt, int32_t *S, int32_t *count,
                  void *stream);

/* Message for the calling thread's last non-zero return ("" if none). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_VERIFY_H */
