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

constexpr int kRouteNJ = kMaxExperts / 64;  // row entries per lane
constexpr int kRankSlots = kMaxTopK + 1;    // k, or k + 1 when the bias needs l_(k+1)
constexpr int kTokWords = kMaxExperts / 32;  // words of a token's expert bitset

__device__ __forceinline__ float nan_to_ninf(float v) { return v != v ? -INFINITY : v; }

// Order-preserving unsigned image of a non-NaN float: a < b <=> ord(a) <
// ord(b), and -0 maps like +0 (the two compare equal as floats).
__device__ __forceinline__ unsigned float_ord(float x) {
    unsigned u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of float_ord (-0 comes back as +0).
__device__ __forceinline__ float ord_float(unsigned k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Unsigned maximum over the wave: DPP row rotations, then the four row
// results; uniform.
__device__ __forceinline__ unsigned wave_umax(unsigned v) {
    int x = (int)v;
    x = (int)max((unsigned)x, (unsigned)dpp_ror<8>(x));
    x = (int)max((unsigned)x, (unsigned)dpp_ror<4>(x));
    x = (int)max((unsigned)x, (unsigned)dpp_ror<2>(x));
    x = (int)max((unsigned)x, (unsigned)dpp_ror<1>(x));
    const unsigned r0 = __builtin_amdgcn_readlane(x, 0), r1 = __builtin_amdgcn_readlane(x, 16);
    const unsigned r2 = __builtin_amdgcn_readlane(x, 32), r3 = __builtin_amdgcn_readlane(x, 48);
    return max(max(r0, r1), max(r2, r3));
}

// Rank order by repeated maxima: round r takes the largest key left and, among
// the entries that hold it, the lowest index, and retires that entry.  Keys
// are float_ord images (entry lane + 64 j in key[j]); invalid entries hold 0,
// below the image of every non-NaN float.  Lane r < K receives rank r (index
// returned, key in *rkey); the keys are consumed.  Each round is one short
// chain of row rotations and ballots, so for small K this beats the radix
// search and needs no ranking pass.
constexpr int kRoundsMaxK = 16;

template <int NJ>
__device__ __forceinline__ int wave_topk_rounds(unsigned (&key)[kRouteNJ], int K, unsigned *rkey) {
    const int lane = threadIdx.x & 63;
    int mine = 0;
    unsigned mk = 0u;
    for (int r = 0; r < K; ++r) {
        unsigned lm = key[0];
#pragma unroll
        for (int j = 1; j < NJ; ++j) lm = max(lm, key[j]);
        const unsigned M = wave_umax(lm);
        int idx = 0;
#pragma unroll
        for (int j = NJ - 1; j >= 0; --j) {
            const unsigned long long b = __ballot(key[j] == M);
            if (b) idx = 64 * j + (int)__builtin_ctzll(b);
        }
        idx = __builtin_amdgcn_readfirstlane(idx);
        if (lane == r) {
            mine = idx;
            mk = M;
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            if (lane + 64 * j == idx) key[j] = 0u;
    }
    *rkey = mk;
    return mine;
}

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

// Marks the K best valid entries of a row held by the wave (entry lane + 64 j
// in slot j < NJ; bit j of `valid` flags it) in the order (key desc, index
// asc).  A radix search from the most significant key bit keeps the bucket
// that holds the K-th best entry and counts the entries above it, and stops
// as soon as the bucket holds exactly the number still missing; if all 32 bits
// are spent, the bucket holds equal keys and the lowest indices are taken.
// Every count is a ballot popcount, so the result is the same in all lanes
// that share the row.  Requires K <= number of valid entries.  Returns bit j
// set where slot j of this lane is selected.
template <int NJ>
__device__ __forceinline__ unsigned wave_topk_mask(const unsigned (&key)[kRouteNJ], unsigned valid, int K) {
    const int lane = threadIdx.x & 63;
    int cand = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) cand += __popcll(__ballot((valid >> j) & 1u));
    int need = K;
    unsigned P = 0u, M = 0u;
    for (int b = 31; b >= 0 && cand != need; --b) {
        const unsigned MM = M | (1u << b), PM = P | (1u << b);
        int c1 = 0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) c1 += __popcll(__ballot(((valid >> j) & 1u) && (key[j] & MM) == PM));
        c1 = __builtin_amdgcn_readfirstlane(c1);
        if (c1 >= need) {
            P = PM;
            cand = c1;
        } else {
            need -= c1;
            cand -= c1;
        }
        M = MM;
        P = __builtin_amdgcn_readfirstlane(P);
        M = __builtin_amdgcn_readfirstlane(M);
    }
    const bool ties = cand != need;  // only once every bit is decided
    const unsigned long long below = (1ull << lane) - 1ull;
    unsigned sel = 0u;
    int left = need;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const bool v = (valid >> j) & 1u;
        const unsigned km = key[j] & M;
        const bool eq = v && km == P;
        const unsigned long long bal = __ballot(eq);
        const bool s = (v && km > P) || (eq && (!ties || (int)__popcll(bal & below) < left));
        left -= __popcll(bal);
        if (s) sel |= 1u << j;
    }
    return sel;
}

// One selected entry on its way to rank order.
struct RankEntry {
    unsigned key;
    int idx;
    float v;   // value the weights are computed from
    float v2;  // second carried value (original logit under the bias)
};

// Puts the K (<= kRankSlots) entries flagged by `sel` into rank order:
// lane r < K receives the entry of rank r under (key desc, index asc).  buf is
// this wave's 2 * kRankSlots entries of LDS.
template <int NJ>
__device__ __forceinline__ RankEntry wave_rank(unsigned sel, const unsigned (&key)[kRouteNJ], const float (&v)[kRouteNJ],
                                               const float (&v2)[kRouteNJ], int K, RankEntry *buf) {
    const int lane = threadIdx.x & 63;
    const unsigned long long below = (1ull << lane) - 1ull;
    int base = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const bool s = (sel >> j) & 1u;
        const unsigned long long bal = __ballot(s);
        if (s) buf[base + __popcll(bal & below)] = RankEntry{key[j], lane + 64 * j, v[j], v2[j]};
        base += __popcll(bal);
    }
    if (lane < K) {
        const RankEntry me = buf[lane];
        int rank = 0;
        for (int q = 0; q < K; ++q) {
            const RankEntry o = buf[q];
            rank += (o.key > me.key || (o.key == me.key && o.idx < me.idx)) ? 1 : 0;
        }
        buf[kRankSlots + rank] = me;
    }
    RankEntry out{0u, 0, -INFINITY, -INFINITY};
    if (lane < K) out = buf[kRankSlots + lane];
    return out;
}

// Lane r < K receives the entry of rank r (value desc, index asc) among the
// valid entries of a row (entry lane + 64 j in slot j; bit j of `valid`);
// v is ranked, v2 is carried along when `carry` (else v2 = v).  Repeated
// maxima for K <= kRoundsMaxK, else the radix search and a ranking pass.
template <int NJ>
__device__ __forceinline__ RankEntry wave_select(const float (&v)[kRouteNJ], const float (&v2)[kRouteNJ],
                                                 unsigned valid, int K, RankEntry *rbuf, bool carry) {
    const int lane = threadIdx.x & 63;
    unsigned key[kRouteNJ];
#pragma unroll
    for (int j = 0; j < kRouteNJ; ++j) key[j] = ((valid >> j) & 1u) ? float_ord(v[j]) : 0u;
    if (K <= kRoundsMaxK) {
        unsigned mk;
        const int idx = wave_topk_rounds<NJ>(key, K, &mk);
        const float val = ord_float(mk);
        float c = val;
        if (carry) {
            // the carried value of the selected entry, from the lane holding it
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const float o = __shfl(v2[j], idx & 63);
                if ((idx >> 6) == j) c = o;
            }
        }
        RankEntry out{0u, 0, -INFINITY, -INFINITY};
        if (lane < K) out = RankEntry{mk, idx, val, c};
        return out;
    }
    const unsigned sel = wave_topk_mask<NJ>(key, valid, K);
    return wave_rank<NJ>(sel, key, v, v2, K, rbuf);
}

// Sequences with a preferred set of their own in a routing call (1 when the
// bias is pooled over the call or off).
__host__ __device__ inline int route_nseq(const VerifyParams &p) { return p.bias_on && p.nseg > 0 ? p.nseg : 1; }

// LDS scratch of block_route, carved from a byte buffer for runtime T, k, E.
struct RouteScratch {
    RankEntry *rank;            // [waves * 2 * kRankSlots]
    unsigned long long *tmask;  // [E] tokens routed to each expert (union members)
    unsigned *tbits;            // [T * kTokWords] experts of each token, one bit each
    unsigned *tbits0;           // [T * kTokWords] first-pass experts of each token (bias only)
    int *sel_i;                 // [T * k] first-pass selection (bias only)
    float *cg;                  // [T * k] w_b * softmax(l_b)_e of the selected e
    int *fin_i;                 // [T * k] final selection
    float *fin_w;               // [T * k]
    int *slot_off;              // [E] CSR offset of each union rank
    unsigned *inP;              // [nseq * kTokWords] preferred set of each sequence, one bit per expert
    float *lam;                 // [T]
    int *wtot;                  // [2 * waves]
    int *misc;                  // [4]: U, sum of |P*|

    // ext_fin: the final selection (fin_i, fin_w) lives outside the scratch;
    // nseq: sequences with a preferred set of their own (1 when pooled)
    __host__ __device__ static size_t bytes(int T, int k, int E, int waves, bool ext_fin = false, int nseq = 1) {
        return (size_t)waves * 2 * kRankSlots * sizeof(RankEntry) + (((size_t)E * 8 + 15) & ~(size_t)15) + (size_t)T * kTokWords * 8 +
               (size_t)T * k * (ext_fin ? 8 : 16) + (size_t)E * 4 + (size_t)nseq * kTokWords * 4 + (size_t)T * 4 +
               (size_t)(2 * waves + 4) * 4 + 64;
    }
    // fin: NULL, or [2 T k] words that receive the final selection (expert
    // ids, then gate weights) and outlive the scratch
    __device__ void carve(unsigned char *base, int T, int k, int E, int waves, int *fin, int nseq) {
        unsigned char *q = base;
        rank = reinterpret_cast<RankEntry *>(q);
        q += (size_t)waves * 2 * kRankSlots * sizeof(RankEntry);
        tmask = reinterpret_cast<unsigned long long *>(q);
        q += ((size_t)E * 8 + 15) & ~(size_t)15;  // tbits rows are read 16 bytes at a time
        tbits = reinterpret_cast<unsigned *>(q);
        q += (size_t)T * kTokWords * 4;
        tbits0 = reinterpret_cast<unsigned *>(q);
        q += (size_t)T * kTokWords * 4;
        sel_i = reinterpret_cast<int *>(q);
        q += (size_t)T * k * 4;
        cg = reinterpret_cast<float *>(q);
        q += (size_t)T * k * 4;
        if (fin) {
            fin_i = fin;
            fin_w = reinterpret_cast<float *>(fin + T * k);
        } else {
            fin_i = reinterpret_cast<int *>(q);
            q += (size_t)T * k * 4;
            fin_w = reinterpret_cast<float *>(q);
            q += (size_t)T * k * 4;
        }
        slot_off = reinterpret_cast<int *>(q);
        q += (size_t)E * 4;
        inP = reinterpret_cast<unsigned *>(q);
        q += (size_t)nseq * kTokWords * 4;
        lam = reinterpret_cast<float *>(q);
        q += (size_t)T * 4;
        wtot = reinterpret_cast<int *>(q);
        q += (size_t)2 * waves * 4;
        misc = reinterpret_cast<int *>(q);
    }
};

// Routes the call with NTHREADS threads (NTHREADS >= E).  Results:
//   LDS: sexp[s] expert of slot s (slot 0 = the shared expert E when there
//        is one, then the union in ascending order), *nslots_lds; when fin
//        is not NULL, fin[t * k + j] / fin[T * k + t * k + j] (as float) the
//        expert and gate weight of rank j of token t.
//   tw (when not NULL; LDS or global, written only): tw[s * T + t] gate
//        weight of token t in slot s (0 if not routed).
//   global (when write_global): topk_idx, topk_w, union, CSR row offsets,
//        P* (each sequence's, ascending), meta, slot_expert; the CSR entries
//        and the slot tables (tokw, tokpos, tpos) of the FFN kernels when
//        write_global, or part blockIdx.x of them when tab_parts > 1 (the
//        tab_parts calling workgroups then write the whole tables together).
// The first pass gives token t to wave t % (NTHREADS / 64); waves without a
// token wait at the barrier that ends it (the caller may hand them other work
// before the call).  Barriers: pass 1, [bias: importance and preferred set
// per sequence, re-selection], union scan, tables.
// NJ: row entries per lane the selections scan (>= ceil(E / 64)).
template <int NTHREADS, int NJ, typename Hook>
__device__ __forceinline__ void block_route_nj(const VerifyParams &p, unsigned char *scratch, int *sexp, float *tw,
                                               int *fin, int *nslots_lds, bool write_global, const Hook &after_pass1,
                                               int tab_parts) {
    static_assert(NTHREADS >= kMaxExperts, "the union scan gives every expert one thread");
    constexpr int NW = NTHREADS / 64;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int T = p.T, E = p.E, k = p.k;
    const bool bias = p.bias_on != 0;
    const int nseq = route_nseq(p);
    RouteScratch sh;
    sh.carve(scratch, T, k, E, NW, fin, nseq);
    RankEntry *rbuf = sh.rank + (size_t)w * 2 * kRankSlots;
    unsigned valid = 0u;  // slots of this lane inside the row
#pragma unroll
    for (int j = 0; j < kRouteNJ; ++j)
        if (lane + 64 * j < E) valid |= 1u << j;

    // A token's experts go to its bitset row (lane L writes word L, so every
    // word is written once and nothing needs clearing); the per-expert token
    // masks are assembled from the rows after the selections.
    auto put_bits = [&](unsigned *rows, int t, int idx, int K) {
        unsigned word = 0u;
        for (int r = 0; r < K; ++r) {
            const int e = __builtin_amdgcn_readlane(idx, r);
            if ((e >> 5) == lane) word |= 1u << (e & 31);
        }
        if (lane < kTokWords) rows[t * kTokWords + lane] = word;
    };

    // ---- pass 1: top-k (k + 1 when the bias needs the (k+1)-th logit);
    //      lane r ends with the entry of rank r ----
    const int R = (bias && k < E) ? k + 1 : k;
    if (tid == 0) sh.misc[1] = 0;  // sum of |P*|, counted after the first barrier
    for (int t = w; t < T; t += NW) {
        float v[kRouteNJ];
        load_logits(p.logits + (size_t)t * E, E, v);
        const float wc = bias ? p.w_conf[t] : 0.f;
        const RankEntry me = wave_select<NJ>(v, v, valid, R, rbuf, false);
        const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(me.v), 0));
        const bool mine = lane < k;
        if (!bias) {
            const float ex = mine ? expf(me.v - m) : 0.f;
            const float s = wave_sum(ex);
            if (mine) {
                const float wt = ex / s;
                sh.fin_i[t * k + lane] = me.idx;
                sh.fin_w[t * k + lane] = wt;
                if (write_global) {
                    p.topk_idx[t * k + lane] = me.idx;
                    p.topk_w[t * k + lane] = wt;
                }
            }
            put_bits(sh.tbits, t, me.idx, k);
        } else {
            // softmax over all E for the importance aggregation (R4)
            float z = 0.f;
#pragma unroll
            for (int j = 0; j < kRouteNJ; ++j)
                if (lane + 64 * j < E) z += expf(v[j] - m);
            z = wave_sum(z);
            if (mine) {
                sh.sel_i[t * k + lane] = me.idx;
                sh.cg[t * k + lane] = wc * (expf(me.v - m) / z);
            }
            put_bits(sh.tbits0, t, me.idx, k);
            // lambda_b = alpha * (l_(1) - l_(k+1)), float32, no contraction (R6)
            if (k < E) {
                const float vk1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(me.v), k));
                if (lane == 0) sh.lam[t] = __fmul_rn(p.alpha, __fsub_rn(m, vk1));
            } else if (lane == 0) {
                sh.lam[t] = 0.f;
            }
        }
    }
    lds_barrier();
    after_pass1();

    if (bias) {
        // ---- per sequence (the whole call when pooled, R16): importance
        //      g_e (R4) of the sequence's first-pass selections, summed in
        //      token order, and its preferred set P*, the top-cap by (g desc,
        //      index asc) among g > 0 (R5).  Wave w takes sequences w,
        //      w + NW, ...; lane l holds experts l + 64 j. ----
        for (int sq = w; sq < nseq; sq += NW) {
            const int t0 = p.nseg > 0 ? p.seg_off[sq] : 0;
            const int t1 = p.nseg > 0 ? p.seg_off[sq + 1] : T;
            unsigned key[kRouteNJ];
            unsigned pos = 0u;
#pragma unroll
            for (int j = 0; j < kRouteNJ; ++j) {
                const int e = lane + 64 * j;
                float g = 0.f;
                if (j < NJ && e < E)
                    for (int t = t0; t < t1; ++t)
                        if ((sh.tbits0[t * kTokWords + (e >> 5)] >> (e & 31)) & 1u)
                            for (int r = 0; r < k; ++r)
                                if (sh.sel_i[t * k + r] == e) g += sh.cg[t * k + r];
                key[j] = float_ord(g);
                if (e < E && g > 0.f) pos |= 1u << j;
            }
            int npos = 0;
#pragma unroll
            for (int j = 0; j < kRouteNJ; ++j)
                if (j < NJ) npos += __popcll(__ballot((pos >> j) & 1u));
            const int n = min(p.cap, npos);
            const unsigned sel = wave_topk_mask<NJ>(key, pos, n);
            const unsigned long long below = (1ull << lane) - 1ull;
            unsigned *prow = sh.inP + sq * kTokWords;
            int base = 0;
#pragma unroll
            for (int j = 0; j < kRouteNJ; ++j) {
                if (j < NJ) {
                    const bool s = (sel >> j) & 1u;
                    const unsigned long long bal = __ballot(s);
                    if (s && write_global) p.pstar[sq * p.cap + base + __popcll(bal & below)] = lane + 64 * j;
                    if (lane < 2) prow[2 * j + lane] = (unsigned)(bal >> (32 * lane));
                    base += __popcll(bal);
                }
            }
            if (lane == 0) {
                atomicAdd(&sh.misc[1], n);
                if (write_global && p.pstar_size_out) p.pstar_size_out[sq] = n;
            }
        }
        lds_barrier();
        // ---- re-select on the biased logits, each token with its own
        //      sequence's P*; weights from the original (R6, R7) ----
        for (int t = w; t < T; t += NW) {
            int sq = 0;
            if (p.nseg > 0)
                while (sq + 1 < p.nseg && p.seg_off[sq + 1] <= t) ++sq;
            const unsigned *prow = sh.inP + sq * kTokWords;
            float v[kRouteNJ], vb[kRouteNJ];
            load_logits(p.logits + (size_t)t * E, E, v);
            const float lam = sh.lam[t];
#pragma unroll
            for (int j = 0; j < kRouteNJ; ++j) {
                const int e = lane + 64 * j;
                vb[j] = (e < E && ((prow[e >> 5] >> (e & 31)) & 1u)) ? __fadd_rn(v[j], lam) : v[j];
            }
            const RankEntry me = wave_select<NJ>(vb, v, valid, k, rbuf, true);
            const bool mine = lane < k;
            const float m = wave_max(mine ? me.v2 : -INFINITY);
            const float ex = mine ? expf(me.v2 - m) : 0.f;
            const float s = wave_sum(ex);
            if (mine) {
                const float wt = ex / s;
                sh.fin_i[t * k + lane] = me.idx;
                sh.fin_w[t * k + lane] = wt;
                if (write_global) {
                    p.topk_idx[t * k + lane] = me.idx;
                    p.topk_w[t * k + lane] = wt;
                }
            }
            put_bits(sh.tbits, t, me.idx, k);
        }
        lds_barrier();
    }

    // ---- union (ascending) and CSR row offsets: wave 0 scans the experts,
    //      NJ groups of 64; slot = rank in the union, after the always-on
    //      shared expert (slot 0) when there is one ----
    const int so = p.has_shared ? 1 : 0;
    int *slot_off = sh.slot_off;
    if (w == 0) {
        const unsigned long long below = (1ull << lane) - 1ull;
        // token masks of this lane's experts (lane + 64 j): the words of 8
        // token rows at a time are read with 16-byte broadcast loads that are
        // all in flight together; expert e sits in word e / 32 = 2 j + lane / 32
        constexpr int NQ = (NJ + 1) / 2;  // 16-byte loads per row (words 0 .. 2 NJ - 1)
        const int hi = lane >> 5;
        unsigned long long mskj[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) mskj[j] = 0ull;
        for (int t0 = 0; t0 < T; t0 += 8) {
            u32x4 rw[8][NQ];
#pragma unroll
            for (int tt = 0; tt < 8; ++tt)
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    rw[tt][q] = t0 + tt < T ? reinterpret_cast<const u32x4 *>(sh.tbits + (t0 + tt) * kTokWords)[q]
                                            : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int tt = 0; tt < 8; ++tt)
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const u32x4 v = rw[tt][j >> 1];
                    const unsigned word = (j & 1) ? (hi ? v.w : v.z) : (hi ? v.y : v.x);
                    mskj[j] |= (unsigned long long)((word >> (lane & 31)) & 1u) << (t0 + tt);
                }
        }
        int base_r = 0, base_c = 0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int e = lane + 64 * j;
            const unsigned long long msk = e < E ? mskj[j] : 0ull;
            const int cnt = __popcll(msk);
            const unsigned long long bal = __ballot(cnt > 0);
            const int incl = wave_incl_scan(cnt);
            if (cnt > 0) {
                const int rank = base_r + __popcll(bal & below);
                const int off = base_c + incl - cnt;
                sexp[rank + so] = e;
                slot_off[rank] = off;
                sh.tmask[e] = msk;
                if (write_global) {
                    p.union_experts[rank] = e;
                    p.csr_ptr[rank] = off;
                    p.slot_expert[rank + so] = e;
                }
            }
            base_r += __popcll(bal);
            base_c += __builtin_amdgcn_readlane(incl, 63);
        }
        if (lane == 0) sh.misc[0] = base_r;
    }
    lds_barrier();

    // ---- slot tables and CSR entries: one thread per (slot, token), each
    //      entry written once.  With tab_parts > 1 the calling workgroups
    //      split the entries: workgroup b computes and writes part b only
    //      (the gate-up kernel, whose workgroups read each token's final
    //      selection instead of the tables) ----
    const int U = sh.misc[0];
    const int nent = U * T;
    const bool wtab = write_global || tab_parts > 1;
    int e0 = 0, e1 = (tw != nullptr || write_global) ? nent : 0;
    if (tab_parts > 1) {
        e0 = (int)((long long)nent * blockIdx.x / tab_parts);
        e1 = (int)((long long)nent * (blockIdx.x + 1) / tab_parts);
    }
    for (int i = e0 + tid; i < e1; i += NTHREADS) {
        const int r = i / T, t = i - r * T;  // union rank, token
        const int s = r + so;                // slot
        const int e = sexp[s];
        const unsigned long long msk = sh.tmask[e];
        float wt = 0.f;
        int pos = -1;
        if ((msk >> t) & 1ull) {
            int jj = 0;
            for (int j = 0; j < k; ++j)
                if (sh.fin_i[t * k + j] == e) jj = j;
            wt = sh.fin_w[t * k + jj];
            pos = slot_off[r] + __popcll(msk & ((1ull << t) - 1ull));
            if (wtab) {
                p.csr_tok[pos] = t;
                p.csr_w[pos] = wt;
                p.tpos[t * k + jj] = pos;
            }
        }
        if (tw) tw[s * T + t] = wt;
        if (wtab) {
            p.tokw[(size_t)s * T + t] = wt;
            p.tokpos[(size_t)s * T + t] = pos;
        }
    }
    if (p.has_shared && tid < T) {  // slot 0: the shared expert, weight 1 for every token
        if (tid == 0) sexp[0] = E;
        if (tw) tw[tid] = 1.f;
        if (write_global) {
            if (tid == 0) p.slot_expert[0] = E;
            p.tokw[tid] = 1.f;
            p.tokpos[tid] = T * k + tid;
        }
    }
    if (tid == 0) {
        *nslots_lds = U + p.has_shared;
        if (write_global) {
            p.csr_ptr[U] = T * k;
            p.meta[0] = U;
            p.meta[1] = U + p.has_shared;
            p.meta[2] = bias ? sh.misc[1] : 0;
            if (p.union_size_out) p.union_size_out[0] = U;
            if (!bias && p.pstar_size_out) p.pstar_size_out[0] = 0;
        }
    }
    lds_barrier();
}

struct NoHook {
    __device__ void operator()() const {}
};

// Routing with the selection loops sized for E.  after_pass1() runs in every
// thread once the per-token selections are done (the caller's chance to
// issue memory work that the remaining, LDS-only steps then overlap).
template <int NTHREADS, typename Hook = NoHook>
__device__ __forceinline__ void block_route(const VerifyParams &p, unsigned char *scratch, int *sexp, float *tw,
                                            int *fin, int *nslots_lds, bool write_global,
                                            const Hook &after_pass1 = Hook{}, int tab_parts = 1) {
    if (p.E <= 128)
        block_route_nj<NTHREADS, 2>(p, scratch, sexp, tw, fin, nslots_lds, write_global, after_pass1, tab_parts);
    else if (p.E <= 256)
        block_route_nj<NTHREADS, 4>(p, scratch, sexp, tw, fin, nslots_lds, write_global, after_pass1, tab_parts);
    else
        block_route_nj<NTHREADS, kRouteNJ>(p, scratch, sexp, tw, fin, nslots_lds, write_global, after_pass1,
                                           tab_parts);
}

}  // namespace moe
