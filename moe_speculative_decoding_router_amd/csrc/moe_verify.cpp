// Host side of libmoeverify: argument validation, workspace layout and the
// launch sequence of one verify-layer call.  No allocation, no
// synchronisation, no per-call state.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/moe_verify.h"
#include "internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

// Compute-unit count per device, queried once (HIP attribute query only).
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu[kMaxDevices];

int cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int v = g_cu[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_cu[dev].store(n, std::memory_order_relaxed);
    return n;
}

struct Layout {
    size_t logits, topk_idx, topk_w, meta, union_experts, csr_ptr, csr_tok, csr_w, pstar;
    size_t slot_expert, tokw, tokpos, tpos, xB, hB, h32, ydown, ypart, tile_cnt, gu_part, total;
    int ks;  // workgroups sharing one gate-up item's contraction
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Activations enter the matrix-core products as a bf16 high/low pair (about
// float32 accuracy) while the 2T columns fit in one 16-column tile; beyond
// that they enter as plain bf16, which keeps the operand traffic per weight
// tile at one tile per 16 tokens.
bool split_mode(int T) { return 2 * T <= 16; }

// Sequences with a preferred set of their own (1 when pooled).
int bias_nseq(const moe_bias *bias) { return bias && bias->nseg > 0 ? bias->nseg : 1; }

// The planning fields of the kernel parameters (what the gate-up plan reads).
moe::VerifyParams plan_params(const moe_layer &L, int T, const moe_bias *bias) {
    moe::VerifyParams p{};
    p.bias_on = bias != nullptr;
    p.nseg = bias && bias->nseg > 0 ? bias->nseg : 0;
    p.T = T;
    p.H = L.H;
    p.I = L.I;
    p.E = L.E;
    p.k = L.k;
    p.wdtype = L.wdtype;
    p.split = split_mode(T) ? 1 : 0;
    p.cols = p.split ? 2 * T : T;
    p.cstride = p.cols;
    p.has_shared = L.Wsh_gu != nullptr;
    p.max_slots = std::min(L.E, T * L.k) + p.has_shared;
    return p;
}

Layout make_layout(const moe_layer &L, int T, const moe_bias *bias) {
    Layout o{};
    o.ks = moe::gateup_ksplit(plan_params(L, T, bias));
    const size_t E = L.E, k = L.k, H = L.H, I = L.I;
    const size_t slots = (size_t)std::min<long>(L.E, (long)T * L.k) + 1;
    const size_t cols = split_mode(T) ? 2 * T : T;
    const size_t cstride = cols;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    o.logits = take(T * E * 4);
    o.topk_idx = take(T * k * 4);
    o.topk_w = take(T * k * 4);
    o.meta = take(16 * 4);
    o.union_experts = take(E * 4);
    o.csr_ptr = take((E + 1) * 4);
    o.csr_tok = take(T * k * 4);
    o.csr_w = take(T * k * 4);
    o.pstar = take(std::max(E, (size_t)bias_nseq(bias) * (bias ? bias->cap : 0)) * 4);
    o.slot_expert = take(slots * 4);
    o.tokw = take(slots * T * 4);
    o.tokpos = take(slots * T * 4);
    o.tpos = take(T * k * 4);
    if (L.wdtype == MOE_F32) {
        o.xB = o.hB = o.ypart = o.tile_cnt = o.gu_part = 0;
        o.h32 = take(slots * T * I * 4);
        o.ydown = take(((size_t)T * k + T) * H * 4);
    } else {
        o.xB = take(H * cstride * 2);
        o.hB = take(slots * I * cstride * 2);
        o.h32 = o.ydown = 0;
        o.ypart = take((size_t)moe::kDownMaxGrid * 2 * moe::kDownMaxRowTiles * T * 16 * 4);
        o.tile_cnt = take((H / 16 + 1) * 4);
        o.gu_part = o.ks > 1 ? take((size_t)o.ks * slots * I * 2 * T * 4) : 0;
    }
    o.total = off;
    return o;
}

int validate_layer(const moe_layer *L, int T, const moe_bias *bias) {
    if (!L) return fail(MOE_EINVAL, "layer is NULL");
    if (T < 1 || T > MOE_MAX_TOKENS) return fail(MOE_EINVAL, "T=%d outside [1, %d]", T, MOE_MAX_TOKENS);
    if (L->H < 1 || L->I < 1) return fail(MOE_EINVAL, "H=%d, I=%d must be positive", L->H, L->I);
    if (L->E < 1 || L->E > MOE_MAX_EXPERTS) return fail(MOE_EINVAL, "E=%d outside [1, %d]", L->E, MOE_MAX_EXPERTS);
    if (L->k < 1 || L->k > L->E || L->k > MOE_MAX_TOPK)
        return fail(MOE_EINVAL, "k=%d outside [1, min(E, %d)]", L->k, MOE_MAX_TOPK);
    if (L->wdtype != MOE_F32 && L->wdtype != MOE_BF16 && L->wdtype != MOE_FP8_E4M3)
        return fail(MOE_EINVAL, "unknown wdtype %d", L->wdtype);
    if (L->wdtype == MOE_BF16 && (L->H % 64 != 0 || L->I % 32 != 0))
        return fail(MOE_ENOTSUP, "bf16 weights need H a multiple of 64 and I of 32 (H=%d, I=%d)", L->H, L->I);
    if (L->wdtype == MOE_FP8_E4M3 && (L->H % 128 != 0 || L->I % 128 != 0))
        return fail(MOE_ENOTSUP, "fp8 weights need H and I multiples of 128 (H=%d, I=%d)", L->H, L->I);
    if ((size_t)L->E * 2 * L->I * (size_t)L->H > ((size_t)1 << 40))
        return fail(MOE_ENOTSUP, "layer too large");
    if ((size_t)L->I * L->H * 2 > (size_t)INT32_MAX * 8)
        return fail(MOE_ENOTSUP, "expert too large");
    if (!L->Wr || !L->W_gu || !L->W_d) return fail(MOE_EINVAL, "Wr, W_gu and W_d must be non-NULL");
    if (L->wdtype == MOE_FP8_E4M3 && (!L->s_gu || !L->s_d))
        return fail(MOE_EINVAL, "fp8 weights need s_gu and s_d");
    if ((L->Wsh_gu == nullptr) != (L->Wsh_d == nullptr))
        return fail(MOE_EINVAL, "shared expert needs both Wsh_gu and Wsh_d");
    if (L->Wsh_gu && L->wdtype == MOE_FP8_E4M3 && (!L->ssh_gu || !L->ssh_d))
        return fail(MOE_EINVAL, "fp8 shared expert needs ssh_gu and ssh_d");
    if (bias) {
        if (bias->cap < L->k || bias->cap > L->E)
            return fail(MOE_EINVAL, "bias cap=%d outside [k=%d, E=%d]", bias->cap, L->k, L->E);
        if (!(bias->alpha >= 0.f && bias->alpha < 1.f))
            return fail(MOE_EINVAL, "bias alpha=%g outside [0, 1)", (double)bias->alpha);
        if (!bias->w_conf) return fail(MOE_EINVAL, "bias w_conf is NULL");
        if (bias->nseg < 0 || bias->nseg > moe::kMaxSegments)
            return fail(MOE_EINVAL, "bias nseg=%d outside [0, %d]", bias->nseg, moe::kMaxSegments);
        if (bias->nseg > 0) {
            const int32_t *o = bias->seg_off;
            if (!o) return fail(MOE_EINVAL, "bias seg_off is NULL with nseg=%d", bias->nseg);
            if (o[0] != 0 || o[bias->nseg] != T)
                return fail(MOE_EINVAL, "bias seg_off must run from 0 to T=%d", T);
            for (int s = 1; s <= bias->nseg; ++s)
                if (o[s] < o[s - 1]) return fail(MOE_EINVAL, "bias seg_off must not decrease");
        }
    }
    return MOE_OK;
}

}  // namespace

namespace moe {

int set_error(int code, const char *msg) { return fail(code, "%s", msg); }

int verify_needs(const moe_layer *layer, int T, const moe_bias *bias, size_t *need) {
    const int rc = validate_layer(layer, T, bias);
    if (rc != MOE_OK) return rc;
    *need = make_layout(*layer, T, bias).total;
    return MOE_OK;
}

}  // namespace moe

extern "C" {

const char *moe_last_error(void) { return g_err; }

size_t moe_verify_workspace_bytes(const moe_layer *layer, int32_t T, const moe_bias *bias) {
    if (validate_layer(layer, T, bias) != MOE_OK) return 0;
    return make_layout(*layer, T, bias).total;
}

int moe_verify_layer(const moe_layer *layer, const float *x, int32_t T, const moe_bias *bias, float *y,
                     moe_aux *aux, void *ws, size_t ws_bytes, void *stream) {
    int rc = validate_layer(layer, T, bias);
    if (rc != MOE_OK) return rc;
    if (!x || !y) return fail(MOE_EINVAL, "x and y must be non-NULL");
    if (!ws) return fail(MOE_EINVAL, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(MOE_EINVAL, "workspace must be 256-byte aligned");
    const moe_layer &L = *layer;
    const Layout lay = make_layout(L, T, bias);
    if (ws_bytes < lay.total)
        return fail(MOE_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, lay.total);
    if (reinterpret_cast<uintptr_t>(x) & 15 || reinterpret_cast<uintptr_t>(y) & 15)
        return fail(MOE_EINVAL, "x and y must be 16-byte aligned");

    char *w = static_cast<char *>(ws);
    moe::VerifyParams p = plan_params(L, T, bias);
    p.cap = bias ? bias->cap : 0;
    for (int s = 0; p.nseg > 0 && s <= p.nseg; ++s) p.seg_off[s] = bias->seg_off[s];
    p.alpha = bias ? bias->alpha : 0.f;
    p.x = x;
    p.Wr = L.Wr;
    p.W_gu = L.W_gu;
    p.W_d = L.W_d;
    p.Wsh_gu = L.Wsh_gu;
    p.Wsh_d = L.Wsh_d;
    p.s_gu = L.s_gu;
    p.s_d = L.s_d;
    p.ssh_gu = L.ssh_gu;
    p.ssh_d = L.ssh_d;
    p.w_conf = bias ? bias->w_conf : nullptr;
    p.y = y;
    auto pick = [&](auto *user, size_t off) {
        using Ptr = decltype(user);
        return user ? user : reinterpret_cast<Ptr>(w + off);
    };
    moe_aux none{};
    const moe_aux &a = aux ? *aux : none;
    p.logits = pick(a.logits, lay.logits);
    p.topk_idx = pick(a.topk_idx, lay.topk_idx);
    p.topk_w = pick(a.topk_w, lay.topk_w);
    p.union_experts = pick(a.union_experts, lay.union_experts);
    p.csr_ptr = pick(a.csr_ptr, lay.csr_ptr);
    p.csr_tok = pick(a.csr_tok, lay.csr_tok);
    p.csr_w = pick(a.csr_w, lay.csr_w);
    p.pstar = pick(a.pstar, lay.pstar);
    p.union_size_out = a.union_size;
    p.pstar_size_out = a.pstar_size;
    p.meta = reinterpret_cast<int *>(w + lay.meta);
    p.slot_expert = reinterpret_cast<int *>(w + lay.slot_expert);
    p.tokw = reinterpret_cast<float *>(w + lay.tokw);
    p.tokpos = reinterpret_cast<int *>(w + lay.tokpos);
    p.tpos = reinterpret_cast<int *>(w + lay.tpos);
    p.xB = L.wdtype == MOE_F32 ? nullptr : reinterpret_cast<uint16_t *>(w + lay.xB);
    p.hB = L.wdtype == MOE_F32 ? nullptr : reinterpret_cast<uint16_t *>(w + lay.hB);
    p.h32 = L.wdtype == MOE_F32 ? reinterpret_cast<float *>(w + lay.h32) : nullptr;
    p.ydown = L.wdtype == MOE_F32 ? reinterpret_cast<float *>(w + lay.ydown) : nullptr;
    p.ypart = L.wdtype == MOE_F32 ? nullptr : reinterpret_cast<float *>(w + lay.ypart);
    p.tile_cnt = L.wdtype == MOE_F32 ? nullptr : reinterpret_cast<int *>(w + lay.tile_cnt);
    p.gu_ticket = L.wdtype == MOE_F32 ? nullptr : p.tile_cnt + L.H / 16;
    p.gu_part = lay.ks > 1 ? reinterpret_cast<float *>(w + lay.gu_part) : nullptr;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int ncu = cu_count();
    moe::KernelEvents kev[MOE_NUM_STAGES];
    if (a.events)
        for (int i = 0; i < MOE_NUM_STAGES; ++i)
            kev[i] = {static_cast<hipEvent_t>(a.events[2 * i]), static_cast<hipEvent_t>(a.events[2 * i + 1])};
    // a stage without a kernel in this call records its two events back to back
    auto no_kernel = [&](int i) -> bool {
        return !a.events ||
               (hipEventRecord(kev[i].start, s) == hipSuccess && hipEventRecord(kev[i].stop, s) == hipSuccess);
    };

    hipError_t err = hipSuccess;
    if ((err = moe::launch_router(p, s, kev[0])) != hipSuccess) goto hip_fail;
    if (!moe::gateup_fuses_routing(p)) {
        if ((err = moe::launch_route(p, s, kev[1])) != hipSuccess) goto hip_fail;
    } else if (!no_kernel(1)) {
        return fail(MOE_EHIP, "hipEventRecord failed");
    }
    if (lay.ks == 1) {
        if ((err = moe::launch_gateup(p, ncu, s, kev[2])) != hipSuccess) goto hip_fail;
    } else {
        // a split gate-up contraction is finished by the SwiGLU combine; the
        // gate-up stage's events span both launches
        if ((err = moe::launch_gateup(p, ncu, s, {kev[2].start, nullptr})) != hipSuccess) goto hip_fail;
        if ((err = moe::launch_swiglu(p, lay.ks, s, {nullptr, kev[2].stop})) != hipSuccess) goto hip_fail;
    }
    if ((err = moe::launch_down(p, ncu, s, kev[3])) != hipSuccess) goto hip_fail;
    if (L.wdtype == MOE_F32) {
        if ((err = moe::launch_combine(p, s, kev[4])) != hipSuccess) goto hip_fail;
    } else if (!no_kernel(4)) {
        return fail(MOE_EHIP, "hipEventRecord failed");
    }
    return MOE_OK;
hip_fail:
    return fail(MOE_EHIP, "kernel launch failed: %s", hipGetErrorString(err));
}

int moe_pack_weights(const void *src, void *dst, int32_t E, int32_t rows, int32_t K, int32_t wdtype,
                     int32_t gate_up, void *stream) {
    if (!src || !dst) return fail(MOE_EINVAL, "NULL pointer");
    if (wdtype != MOE_BF16 && wdtype != MOE_FP8_E4M3) return fail(MOE_EINVAL, "packing covers bf16 and fp8 weights");
    if (E < 1 || rows < 16 || K < 1) return fail(MOE_EINVAL, "need E >= 1, rows >= 16, K >= 1");
    const int kt = wdtype == MOE_BF16 ? 32 : 64;
    if (rows % 16 != 0 || K % kt != 0)
        return fail(MOE_EINVAL, "rows must be a multiple of 16 and K of %d", kt);
    if (gate_up && rows % 32 != 0) return fail(MOE_EINVAL, "gate-up rows (2I) must be a multiple of 32");
    if (!gate_up && rows % 64 != 0) return fail(MOE_EINVAL, "down rows (H) must be a multiple of 64");
    const size_t esz = wdtype == MOE_BF16 ? 2 : 1;
    const size_t bytes = (size_t)E * rows * K * esz;
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    if (a < b + bytes && b < a + bytes) return fail(MOE_EINVAL, "src and dst overlap");
    if ((a | b) & 15) return fail(MOE_EINVAL, "src and dst must be 16-byte aligned");
    hipError_t err = moe::launch_pack(src, dst, E, rows, K, (int)esz, gate_up ? 1 : 0, rows / 2,
                                      static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(MOE_EHIP, "kernel launch failed: %s", hipGetErrorString(err));
    return MOE_OK;
}

int moe_stream_read(const void *src, size_t bytes, uint32_t *checksum, void *stream) {
    if (!src || !checksum) return fail(MOE_EINVAL, "NULL pointer");
    if (bytes == 0 || bytes % 16 != 0) return fail(MOE_EINVAL, "bytes must be a positive multiple of 16");
    if (reinterpret_cast<uintptr_t>(src) & 15) return fail(MOE_EINVAL, "src must be 16-byte aligned");
    hipError_t err = moe::launch_read_probe(src, bytes, checksum, cu_count(), static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(MOE_EHIP, "kernel launch failed: %s", hipGetErrorString(err));
    return MOE_OK;
}

int union_stats(const int32_t *topk_idx, int32_t nL, int32_t T, int32_t k, int32_t E, int32_t *counts,
                float *reuse, void *stream) {
    if (!topk_idx || !counts || !reuse) return fail(MOE_EINVAL, "NULL pointer");
    if (nL < 0 || T < 1 || k < 1) return fail(MOE_EINVAL, "need nL >= 0, T >= 1, k >= 1");
    if (E < 1 || E > 65536) return fail(MOE_EINVAL, "E=%d outside [1, 65536]", E);
    if ((long long)T * k >= (1LL << 24)) return fail(MOE_ENOTSUP, "T * k must be below 2^24");
    if (nL == 0) return MOE_OK;
    hipError_t err = moe::launch_union_stats(topk_idx, nL, T, k, E, counts, reuse, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(MOE_EHIP, "kernel launch failed: %s", hipGetErrorString(err));
    return MOE_OK;
}

static int select_common(const int32_t *parent, int32_t N, const float *P, const uint32_t *Epred, int32_t W,
                  int32_t gamma, float eps, int32_t nt, int32_t *S, bool update_b, void *stream) {
    if (!parent) return fail(MOE_EINVAL, "parent is NULL");
    if (N < 1 || N > 4096) return fail(MOE_EINVAL, "N=%d outside [1, 4096]", N);
    if (W < 1 || W > 4096) return fail(MOE_EINVAL, "W=%d outside [1, 4096]", W);
    if (gamma < 0 || gamma > N) return fail(MOE_EINVAL, "gamma=%d outside [0, N=%d]", gamma, N);
    if (!(eps > 0.f) || !std::isfinite(eps)) return fail(MOE_EINVAL, "eps must be positive and finite");
    if (nt < 0) return fail(MOE_EINVAL, "nt=%d is negative", nt);
    for (int i = 0; i < N; ++i)
        if (parent[i] < -1 || parent[i] >= i)
            return fail(MOE_EINVAL, "parent[%d]=%d: nodes must be in BFS order (parent < child)", i, parent[i]);
    if (nt == 0 || gamma == 0) return MOE_OK;  // nothing to write
    if (!P || !Epred || !S) return fail(MOE_EINVAL, "NULL pointer");
    hipError_t err = moe::launch_select(N, P, Epred, W, gamma, eps, nt, S, update_b, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(MOE_EHIP, "kernel launch failed: %s", hipGetErrorString(err));
    return MOE_OK;
}


int select_drafts(const int32_t *parent, int32_t N, const float *P, const uint32_t *Epred, int32_t W,
                  int32_t gamma, float eps, int32_t nt, int32_t *S, void *stream) {
    return select_common(parent, N, P, Epred, W, gamma, eps, nt, S, true, stream);
}

int select_drafts_static(const int32_t *parent, int32_t N, const float *P, const uint32_t *Epred, int32_t W,
                         int32_t gamma, float eps, int32_t nt, int32_t *S, void *stream) {
    return select_common(parent, N, P, Epred, W, gamma, eps, nt, S, false, stream);
}

int expand_drafts(const int32_t *parent, int32_t N, const float *P, const uint32_t *Epred, int32_t W, float t_ar,
                  float t_exp, const float *c_draft, int32_t nt, int32_t *S, int32_t *count, void *stream) {
    if (!parent) return fail(MOE_EINVAL, "parent is NULL");
    if (N < 1 || N > moe::kMaxExpandNodes) return fail(MOE_EINVAL, "N=%d outside [1, %d]", N, moe::kMaxExpandNodes);
    if (W < 1 || W > 4096) return fail(MOE_EINVAL, "W=%d outside [1, 4096]", W);
    if (!std::isfinite(t_ar) || !std::isfinite(t_exp) || t_ar < 0.f || t_exp < 0.f)
        return fail(MOE_EINVAL, "t_ar and t_exp must be finite and non-negative");
    if (nt < 0) return fail(MOE_EINVAL, "nt=%d is negative", nt);
    moe::ExpandArgs a{};
    for (int i = 0; i < N; ++i) {
        if (parent[i] < -1 || parent[i] >= i)
            return fail(MOE_EINVAL, "parent[%d]=%d: nodes must be in BFS order (parent < child)", i, parent[i]);
        a.parent[i] = (int16_t)parent[i];
    }
    if (moe::expand_lds_bytes(N, W, false) > (size_t)moe::kSelectMaxLdsWords * 4)
        return fail(MOE_ENOTSUP, "tree of %d nodes x %d words needs more than %d words of LDS state", N, W,
                    moe::kSelectMaxLdsWords);
    if (nt == 0) return MOE_OK;
    if (!P || !Epred || !S || !count) return fail(MOE_EINVAL, "NULL pointer");
    a.N = N;
    a.W = W;
    a.nt = nt;
    a.t_ar = t_ar;
    a.t_exp = t_exp;
    hipError_t err = moe::launch_expand(a, P, Epred, c_draft, S, count, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(MOE_EHIP, "kernel launch failed: %s", hipGetErrorString(err));
    return MOE_OK;
}


int union_stats_segments(const int32_t *topk_idx, int32_t nL, int32_t T, int32_t k, int32_t E,
                         const int32_t *offsets, int32_t S, int32_t *per, int32_t *total, void *stream) {
    if (!offsets) return fail(MOE_EINVAL, "offsets is NULL");
    if (nL < 0 || T < 1 || k < 1) return fail(MOE_EINVAL, "need nL >= 0, T >= 1, k >= 1");
    if (E < 1 || E > 65536) return fail(MOE_EINVAL, "E=%d outside [1, 65536]", E);
    if (S < 1 || S > moe::kMaxSegments) return fail(MOE_EINVAL, "S=%d outside [1, %d]", S, moe::kMaxSegments);
    moe::SegmentArgs a{};
    a.S = S;
    if (offsets[0] != 0 || offsets[S] != T) return fail(MOE_EINVAL, "offsets must run from 0 to T=%d", T);
    for (int s = 0; s <= S; ++s) {
        if (s > 0 && offsets[s] < offsets[s - 1]) return fail(MOE_EINVAL, "offsets must not decrease");
        a.off[s] = offsets[s];
    }
    if (nL == 0) return MOE_OK;
    if (!topk_idx || !per || !total) return fail(MOE_EINVAL, "NULL pointer");
    hipError_t err = moe::launch_segment_stats(topk_idx, nL, T, k, E, a, per, total, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(MOE_EHIP, "kernel launch failed: %s", hipGetErrorString(err));
    return MOE_OK;
}

int gate_depths(const float *c, const uint32_t *Epred, int32_t S, int32_t Dmax, int32_t W, float t_base,
                float t_exp, int32_t *d, void *stream) {
    if (S < 1 || S > moe::kGateMaxSeq) return fail(MOE_EINVAL, "S=%d outside [1, %d]", S, moe::kGateMaxSeq);
    if (Dmax < 0 || Dmax > moe::kGateMaxDepth)
        return fail(MOE_EINVAL, "Dmax=%d outside [0, %d]", Dmax, moe::kGateMaxDepth);
    if (W < 1 || W > moe::kGateMaxWords) return fail(MOE_EINVAL, "W=%d outside [1, %d]", W, moe::kGateMaxWords);
    if (!std::isfinite(t_base) || !std::isfinite(t_exp) || !(t_base > 0.f) || t_exp < 0.f)
        return fail(MOE_EINVAL, "need t_base > 0 and t_exp >= 0, finite");
    if (!c || !Epred || !d) return fail(MOE_EINVAL, "NULL pointer");
    hipError_t err = moe::launch_gate_depths(c, Epred, S, Dmax, W, t_base, t_exp, d, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(MOE_EHIP, "kernel launch failed: %s", hipGetErrorString(err));
    return MOE_OK;
}

}  // extern "C"
