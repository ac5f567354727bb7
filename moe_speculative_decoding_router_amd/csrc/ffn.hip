// Grouped skinny SwiGLU FFN over the union experts only, and the combine.
//
// [EcoSpec] = review of "Less Experts, Faster Decoding" (§1-§2: at one MoE
// layer the verified tokens need the weights of the union of their experts;
// each unique expert is loaded once and applied to all of its tokens).
//
// Work decomposition (bf16 / fp8 weights, one workgroup of 8 waves per
// compute unit):
//   gate-up : the routing runs in every workgroup's prologue (route_block.h).
//             Item = (union slot, 16 packed rows: 8 gate + 8 up rows of the
//             same intermediate indices).  Items go round-robin to the
//             workgroups (the tail by tickets when the activation operand is
//             read from L2); the 8 waves take interleaved batches of the
//             item's contraction, streaming packed 1 KB tiles with 16-byte
//             non-temporal loads straight into the A operand of
//             v_mfma_f32_16x16x32_bf16 (fp8 is decoded exactly to bf16 in
//             registers, each 128-wide block scaled after its products).  The
//             activations are the B operand, staged once per workgroup in
//             LDS: the T tokens as columns, as a bf16 high/low pair when
//             2T <= 16.  When the operand does not fit in LDS the contraction
//             of each item is split over 2 or 4 workgroups and a SwiGLU
//             combine kernel finishes it.  Partial sums meet in LDS in a fixed
//             order; SiLU(gate) * up, times the token's gate weight, is
//             written in the B-operand layout of the down projection.
//   down    : units (row group, slot, k-unit) split evenly over the
//             workgroups (stream-K); a workgroup owning a whole row group
//             writes y, shared row groups exchange pieces through the
//             workspace and the last to finish adds them in workgroup order.
//             No atomics on y: the result does not depend on timing.
// Float32 weights use plain VALU dot products (one wave per output row),
// per-(token, expert) rows of ydown and a combine in rank order.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "internal.h"
#include "launch.h"
#include "route_block.h"

namespace moe {
namespace {

constexpr int kFfnThreads = 256;
constexpr int kGateUpWgPerCu = 1;  // persistent workgroups per CU (8 waves each)
constexpr size_t kLdsPerCu = 160 * 1024;      // LDS of one gfx950 compute unit

// Waits for every vector memory access of this wave (vmcnt(0); expcnt and
// lgkmcnt left at their maxima).  Issued through the builtin so that the
// compiler's wait insertion knows the direct-to-LDS copies are complete and
// adds no waits of its own to later LDS reads; the empty asm statements keep
// memory accesses from moving across it.
__device__ __forceinline__ void wait_vm_all() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70);
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ u32x4 ld_nt(const uint8_t *ptr) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ptr));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16 OCP E4M3FN codes -> two bf16x8 operands (codes 0..7 and 8..15).  The
// hardware conversion yields exact float32 values with at most 4 significant
// bits, so taking their upper halves is an exact bf16 conversion.
__device__ __forceinline__ void fp8x16_to_bf16(u32x4 q, bf16x8 &lo, bf16x8 &hi) {
    u32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x2 f01 = __builtin_amdgcn_cvt_pk_f32_fp8(q[i], false);
        const f32x2 f23 = __builtin_amdgcn_cvt_pk_f32_fp8(q[i], true);
        const unsigned p0 = __builtin_amdgcn_perm(__float_as_uint(f01[1]), __float_as_uint(f01[0]), 0x07060302u);
        const unsigned p1 = __builtin_amdgcn_perm(__float_as_uint(f23[1]), __float_as_uint(f23[0]), 0x07060302u);
        if (i < 2) {
            a[2 * i] = p0;
            a[2 * i + 1] = p1;
        } else {
            b[2 * (i - 2)] = p0;
            b[2 * (i - 2) + 1] = p1;
        }
    }
    lo = as_bf16x8(a);
    hi = as_bf16x8(b);
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu(float z) { return z / (1.f + expf(-z)); }

// ---------------------------------------------------------------------------
// Unit streams.  A unit is one packed tile (bf16: 16 rows x 32 k, one k-step)
// or one 128-wide scale block (fp8: two tiles, four k-steps).  A wave streams
// its units in batches of KU with two register buffers: the loads of batch
// f + 1 are in flight while batch f is multiplied.  Every load is issued
// unconditionally (out-of-range units re-read a valid tile and are skipped
// by a wave-uniform test; B columns past the used ones read the padded,
// never-used part of the operand, which only feeds output columns that are
// discarded), so the loads of a batch form one straight-line group and the
// waits before the products count only older loads.
// ---------------------------------------------------------------------------
template <int WT, int NT, int KU>
struct Batch {
    static constexpr int NA = WT == 1 ? 2 : 1;  // tile loads per unit
    static constexpr int NS = WT == 1 ? 4 : 1;  // k-steps per unit
    u32x4 a[KU][NA];
    u32x4 b[KU][NS][NT];
    float sc[KU];
    bool on[KU];
};

template <int WT, int NT, int KU>
__device__ __forceinline__ void load_unit(Batch<WT, NT, KU> &bt, int u, bool on, const uint8_t *tile,
                                          const uint16_t *bq, size_t bstep, float scale, const int (&coff)[NT]) {
    bt.on[u] = on;
#pragma unroll
    for (int h = 0; h < Batch<WT, NT, KU>::NA; ++h) bt.a[u][h] = ld_nt(tile + h * 1024);
#pragma unroll
    for (int q = 0; q < Batch<WT, NT, KU>::NS; ++q)
#pragma unroll
        for (int n = 0; n < NT; ++n) bt.b[u][q][n] = *reinterpret_cast<const u32x4 *>(bq + q * bstep + coff[n]);
    bt.sc[u] = scale;
}

// Element offsets of this lane's B-operand columns (column n * 16 + lr,
// clamped to the last used column: the clamped lanes re-read a column that
// the wave loads anyway and only feed output columns that are discarded).
template <int NT>
__device__ __forceinline__ void col_offsets(int (&coff)[NT], int lr, int cols) {
#pragma unroll
    for (int n = 0; n < NT; ++n) coff[n] = min(n * 16 + lr, cols - 1) * 8;
}

// Products of one batch.  Consecutive units alternate between two
// accumulator sets so that neighbouring matrix-core instructions are
// independent; the sets are added at the end of an item.
template <int WT, int NT, int KU>
__device__ __forceinline__ void compute_batch(const Batch<WT, NT, KU> &bt, f32x4 (&acc)[2][NT], bool valid) {
    const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < KU; ++u) {
        // skipped units multiply zeros (no branch, so the waits before the
        // products only count loads issued before this batch's own)
        const bool on = valid && bt.on[u];
        f32x4 (&ac)[NT] = acc[u & 1];
        if (WT == 0) {
            const bf16x8 a = as_bf16x8(on ? bt.a[u][0] : zero);
#pragma unroll
            for (int n = 0; n < NT; ++n) ac[n] = mfma(a, as_bf16x8(bt.b[u][0][n]), ac[n]);
        } else {
            f32x4 t[2][NT];
#pragma unroll
            for (int n = 0; n < NT; ++n) t[0][n] = t[1][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                bf16x8 lo, hi;
                fp8x16_to_bf16(bt.a[u][h], lo, hi);
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    t[0][n] = mfma(lo, as_bf16x8(bt.b[u][2 * h][n]), t[0][n]);
                    t[1][n] = mfma(hi, as_bf16x8(bt.b[u][2 * h + 1][n]), t[1][n]);
                }
            }
            const float sc = on ? bt.sc[u] : 0.f;
#pragma unroll
            for (int n = 0; n < NT; ++n) ac[n] += sc * (t[0][n] + t[1][n]);
        }
    }
}

template <int NT>
__device__ __forceinline__ void fold_acc(f32x4 (&acc)[2][NT]) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        acc[0][n] += acc[1][n];
        acc[1][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

// Adds the low-part columns to the high-part columns: column c of tile n is
// token n * 16 + lr; in split mode the low part of token t sits in column
// T + t (tile (T + t) / 16, lane (T + t) % 16 of the same lane group).
template <int NT, bool SPLIT>
__device__ __forceinline__ void combine_split(float (&v)[NT][4], const f32x4 (&acc)[NT], int T, int lane) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int j = 0; j < 4; ++j) v[n][j] = acc[n][j];
    if (!SPLIT) return;
    const int lr = lane & 15;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int clo = T + n * 16 + lr;
        const int nlo = clo >> 4;
        const int src = (lane & ~15) | (clo & 15);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float lo = 0.f;
#pragma unroll
            for (int q = 0; q < NT; ++q) {
                const float a = __shfl(acc[q][j], src);
                if (q == nlo) lo = a;
            }
            v[n][j] += lo;
        }
    }
}

template <int NT, int NW>
__device__ __forceinline__ void reduce_waves(f32x4 (&acc)[NT], f32x4 (*red)[NT][64], int w, int lane) {
    if (w != 0) {
#pragma unroll
        for (int n = 0; n < NT; ++n) red[w][n][lane] = acc[n];
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
        for (int q = 1; q < NW; ++q)
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[n] += red[q][n][lane];
    }
}

// Units per batch of the gate-up stream (wdtype 1 = bf16, 2 = fp8; nt column
// tiles): enough loads in flight per wave, and few empty batch slots when the
// item's units do not fill 8 waves evenly (bf16 with one column tile: 4,
// measured against 2, 6 and 8 at H = 2880 and 4096; with two column tiles:
// 8, against 4 at H = 4096 and 20 tokens, 238.5 -> 235.0 us per batched
// Qwen3 gate-up, where the operand of 2 units in 8 then comes from L2).
// fp8 (2 KB units): 2 up to two column tiles (at H = 7168 and 20-32 tokens
// 13-16% faster than 1, which it also lets take the operand partly from
// L2); with three or four column tiles 2 would spill registers.
constexpr int gu_batch_units(int wdtype, int nt) {
    return wdtype == 2 ? (nt <= 2 ? 2 : 1) : (nt == 1 ? 4 : (nt == 2 ? 8 : 2));
}

template <int WT, int NT>
struct UnitCfg {
    static constexpr int KT = WT == 1 ? 64 : 32;                                    // k per tile
    static constexpr int KU = gu_batch_units(WT == 1 ? 2 : 1, NT);                  // units per batch
    static constexpr size_t USTEP = WT == 1 ? 2048 : 1024;                          // bytes per unit
    static constexpr int KSTEPS = WT == 1 ? 4 : 1;                                  // k-steps per unit
};

// ---------------------------------------------------------------------------
// gate-up: items = (slot, row tile of 8 gate + 8 up rows); a workgroup of 8
// waves takes items round-robin, its waves take interleaved batches of the
// H contraction, and the partial sums meet in LDS in a fixed order.  The
// batches of a wave run across item boundaries, so the next item's weights
// are in flight while the current item is reduced.
// BLDS: the activation operand (identical for every item) is copied into
// LDS once per workgroup, so the only vector-memory traffic of the stream is
// the weights.  TWL: token weights staged in LDS.
// ---------------------------------------------------------------------------
constexpr int kGuWaves = 8;
constexpr int kGuDynDepth = 3;  // items per workgroup left to the ticket counter
constexpr int kGuMaxSplit = 4;  // most workgroups sharing one item's contraction

// KS > 1: the contraction of every item is split over KS workgroups;
// workgroup b takes part b % KS of it and holds only that part's slice of
// the operand in LDS, and its partial gate and up sums go to gu_part for the
// SwiGLU combine.
// NGL > 0 (KS = 1; bf16, or fp8 with one column tile): of every KU
// consecutive units, the last NGL take
// their operand from global memory (where it stays L2-resident: every
// workgroup reads the same few hundred KB) and only the others are staged in
// LDS, so a contraction whose whole operand does not fit in LDS still runs in
// one workgroup: no partial sums, no combine launch.  Which units come from
// where is fixed by the unit's position in its batch, so the loads of a batch
// are the same instructions every time.
template <int WT, int NT, bool SPLIT, bool FUSED, bool BLDS, int KS, int NGL>
__global__ __launch_bounds__(kGuWaves * 64) void gateup_kernel(VerifyParams p) {
    using C = UnitCfg<WT, NT>;
    constexpr int KU = C::KU;
    static_assert(NGL == 0 || (KS == 1 && BLDS && NGL < KU), "mixed operand: one part, LDS, a batch of 2+ units");
    constexpr int KL = KU - NGL;  // units of every KU whose operand is staged in LDS
    using B = Batch<WT, NT, KU>;
    extern __shared__ __align__(16) unsigned char dyn_lds[];
    __shared__ f32x4 red[2][kGuWaves][NT][64];
    __shared__ int sexp[kMaxExperts + 1];
    __shared__ int nslots_sh;
    __shared__ int sitem[4];  // items of the tail, ring by item order
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = lane >> 4, lr = lane & 15;
    const int T = p.T, H = p.H, I = p.I, E = p.E, cstride = p.cstride, cols = p.cols;
    const int nkt = H / C::KT;
    const int rtiles = I / 8;
    const int nunits = WT == 1 ? nkt / 2 : nkt;  // contraction units (1 KB per row tile each for bf16)
    const int hk = KS > 1 ? (int)blockIdx.x % KS : 0;
    const int nuh = nunits / KS;                  // units of one part (the host checks that KS divides)
    const int u0 = hk * nuh;                      // first unit of this workgroup's part
    constexpr int kspu = WT == 1 ? 4 : 1;         // k-steps of 32 per unit
    // dynamic LDS, in order: the activation operand (BLDS), the routing
    // scratch and the tokens' final selections (FUSED).  With gu_async_x the
    // operand has a region of its own and its loads fly while the routing
    // runs; otherwise the routing scratch overlays the end of the operand
    // region: the chunks below it are loaded while the routing runs, the
    // rest after.
    const int nl = NGL == 0 ? nuh : (nuh / KU) * KL + min(nuh % KU, KL);  // units staged in LDS
    const int cpu_ = kspu * 4 * cols;             // 16-byte operand chunks per unit
    const int nx = BLDS ? nl * cpu_ : 0;          // 16-byte operand chunks in LDS
    const size_t xb_bytes = (size_t)nx * 16;
    const size_t scr_bytes =
        FUSED ? (RouteScratch::bytes(T, p.k, E, kGuWaves, true, route_nseq(p)) + 15) & ~(size_t)15 : 0;
    const bool async_x = BLDS && p.gu_async_x != 0;
    // operand chunks that can be loaded before the routing is done
    const int early = async_x ? nx : (BLDS && xb_bytes >= scr_bytes ? (int)((xb_bytes - scr_bytes) / 16) : 0);
    u32x4 *xs = reinterpret_cast<u32x4 *>(dyn_lds);
    unsigned char *scr = dyn_lds + (async_x ? xb_bytes : (size_t)early * 16);
    // [2 T k]: expert id, then gate weight (float bits), of rank j of token t
    int *fin = reinterpret_cast<int *>(
        dyn_lds + (async_x ? xb_bytes + scr_bytes : (xb_bytes > scr_bytes ? xb_bytes : scr_bytes)));
    // Direct global -> LDS copy of operand chunks [c0, c1) by waves
    // w0 .. w0 + nws - 1; lane l of a wave fills chunk i0 + l.  LDS chunk i
    // belongs to staged unit i / cpu_; staged unit li is unit
    // (li / KL) KU + li % KL of the part (all of them when NGL = 0, where the
    // copy is one contiguous block, as the column stride equals the column
    // count).
    const uint16_t *xpart = p.xB + (size_t)u0 * cpu_ * 8;  // the part's slice
    auto src_chunk = [&](int i) -> int {
        if (NGL == 0) return i;
        const int li = i / cpu_, wi = i - li * cpu_;
        return ((li / KL) * KU + li % KL) * cpu_ + wi;
    };
    auto stage_x = [&](int w0, int nws, int c0, int c1) {
        if (w < w0) return;
        for (int i0 = c0 + (w - w0) * 64; i0 < c1; i0 += nws * 64)
            if (i0 + lane < c1) load_lds16(xpart + (size_t)src_chunk(i0 + lane) * 8, xs + i0);
    };

    // y starts at zero for the down kernel's two-piece row groups, which it
    // adds into y.  Zeroed here, at the end of each workgroup's stream (the
    // stores then delay nothing that waits for memory), rather than by the
    // router kernel: x, which that kernel reads, may share memory with y.
    auto zero_y = [&]() {
        for (int i = (int)blockIdx.x * (kGuWaves * 64) + (int)threadIdx.x; i < T * H;
             i += (int)gridDim.x * (kGuWaves * 64))
            p.y[i] = 0.f;
    };

    int nslots;
    if (FUSED) {
        // The chunks that do not overlap the routing scratch are issued by
        // the waves without a token in the routing's first pass, before it;
        // when every wave has tokens, by all waves right after the per-token
        // selections (issued earlier, they would queue ahead of the router
        // logits that the selections wait for).
        if (early > 0 && T < kGuWaves) stage_x(T, kGuWaves - T, 0, early);
        auto after_pass1 = [&]() {
            if (early > 0 && T >= kGuWaves) stage_x(0, kGuWaves, 0, early);
        };
        // An always-on shared expert is slot 0, so this workgroup's first
        // item is its row tile b (while b < rtiles) whatever the routing
        // gives: the waves without a token pull the first half of that
        // item's tiles into L2 during the routing (direct loads into a
        // scratch block of the reduction buffer, which the main loop
        // overwrites later), and that half then streams from L2.  (The whole
        // item, about the size of an XCD's L2 over its 32 workgroups, is
        // mostly evicted before use; half of it gained most: 2.6 us per
        // DeepSeek gate-up against 0.6 for the whole and 1.9 for a quarter.)
        if (KS == 1 && p.has_shared && (int)blockIdx.x < rtiles && T < kGuWaves && w >= T) {
            const uint8_t *sht = static_cast<const uint8_t *>(p.Wsh_gu) + (size_t)blockIdx.x * nkt * 1024 + lane * 16;
            for (int c = w - T; c < nkt / 2; c += kGuWaves - T) load_lds16(sht + (size_t)c * 1024, &red[0][w][0][0]);
        }
        // routing, recomputed by every workgroup (bit-identical results)
        block_route<kGuWaves * 64>(p, scr, sexp, nullptr, fin, &nslots_sh, blockIdx.x == 0, after_pass1,
                                   (int)gridDim.x);
        nslots = nslots_sh;
        if (early < nx) stage_x(0, kGuWaves, early, nx);
    } else {
        nslots = min(p.meta[1], p.max_slots);
        for (int i = threadIdx.x; i < nslots; i += kGuWaves * 64)
            sexp[i] = min(max(p.slot_expert[i], 0), p.has_shared ? E : E - 1);
        stage_x(0, kGuWaves, 0, nx);
    }
    wait_vm_all();
    __syncthreads();
    const int items = nslots * rtiles;
    if ((int)blockIdx.x / KS >= min(items, (int)gridDim.x / KS)) {
        zero_y();
        return;
    }

    // Batches of KU consecutive units; batch b of an item belongs to wave
    // b % kGuWaves, so the workgroup reads one contiguous window that moves
    // through the item.  Every wave runs the same number of batches per item
    // (trailing ones empty), so the reduction barriers line up.
    const int nbi = (nuh + KU - 1) / KU;                    // batches per item
    const int nb = (nbi + kGuWaves - 1) / kGuWaves;         // per wave per item
    // Items: workgroup b takes items b, b + G, ... up to its S0-th (G and b
    // counted among the workgroups of its contraction part).  When the
    // operand is read from L2 (wholly, or for NGL units of every batch), the
    // workgroups' streaming rates vary with L2 contention, and the remaining
    // R items are handed out in order by a device-scope ticket counter, so
    // the workgroups that stream faster take more of the tail.  A ticket is claimed three items
    // ahead of its use (right after the barrier of an item) and published to
    // LDS just before the barrier of the next item, which waits for every
    // outstanding load anyway.
    const int G = gridDim.x / KS, bid = blockIdx.x / KS;
    const bool dyn = KS == 1 && (!BLDS || NGL > 0) && p.gu_ticket != nullptr && items >= (kGuDynDepth + 3) * G;
    const int S0 = dyn ? items / G - kGuDynDepth : 0;
    const int R = items - S0 * G;
    auto item_of = [&](int ord) -> int {
        if (!dyn || ord < S0) {
            const int it = bid + ord * G;
            return it < items ? it : -1;
        }
        return sitem[ord & 3];
    };
    int ticket = 0;  // thread 0: the last claim
    const size_t esz = WT == 1 ? 1 : 2;
    const size_t bstep = (size_t)4 * cstride * 8;                       // global: elements per k-step
    const uint16_t *xb = p.xB + (size_t)g * cstride * 8;                // global: lane group, k-step 0
    int coff[NT];
    col_offsets<NT>(coff, lr, cols);

    // Tile and scale pointers of the item being loaded, refreshed once per
    // item (batches are loaded in increasing order).
    int c_ord = -1;
    const uint8_t *c_tiles = nullptr;
    const float *c_srow = nullptr;
    auto load_batch = [&](B &bt, int f) {
        const int ord = f / nb;
        if (ord != c_ord) {
            c_ord = ord;
            const int item = item_of(ord);
            const int s = item / rtiles, rt = item - s * rtiles;
            const int e = sexp[s];
            const bool sh = e == E;
            c_tiles = (sh ? static_cast<const uint8_t *>(p.Wsh_gu)
                          : static_cast<const uint8_t *>(p.W_gu) + (size_t)e * 2 * I * H * esz) +
                      (size_t)rt * nkt * 1024 + lane * 16;
            if (WT == 1) {
                const int sld = H / 128;
                const float *sb = sh ? p.ssh_gu : p.s_gu + (size_t)e * (2 * I / 128) * sld;
                c_srow = sb + (size_t)((g < 2 ? 8 * rt : I + 8 * rt) / 128) * sld;
            }
        }
        const uint8_t *tiles = c_tiles;
        const float *srow = c_srow;
        const int k0 = ((f % nb) * kGuWaves + w) * KU;
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int kk = k0 + u;                 // unit within the part
            const bool on = kk < nuh;
            const int kr = on ? kk : nuh - 1;
            const int kc = u0 + kr;                // unit within the item
            bt.on[u] = on;
#pragma unroll
            for (int h = 0; h < B::NA; ++h) bt.a[u][h] = ld_nt(tiles + (size_t)kc * C::USTEP + h * 1024);
#pragma unroll
            for (int q = 0; q < B::NS; ++q) {
                const int ks = kc * B::NS + q;
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    if (BLDS && u < KL) {
                        // staged unit of kr (units past the end read staged
                        // unit 0: finite values, multiplied by zeros)
                        const int li = NGL == 0 ? kr : (on ? (kr / KU) * KL + u : 0);
                        bt.b[u][q][n] = xs[((li * B::NS + q) * 4 + g) * cols + (coff[n] >> 3)];
                    } else {
                        bt.b[u][q][n] = *reinterpret_cast<const u32x4 *>(xb + (size_t)ks * bstep + coff[n]);
                    }
                }
            }
            bt.sc[u] = WT == 1 ? srow[kc] : 0.f;
        }
    };
    // End of an item: every wave stores its partial sums into one of two
    // LDS buffers (alternating per item) and passes ONE barrier; then 8 x T
    // threads, starting at a wave that rotates with the item, each finish one
    // (intermediate row, token) output from the buffer while the other waves
    // keep streaming.  The
    // buffer of item i is rewritten at item i + 2 only, after every wave has
    // passed the barrier of item i + 1, i.e. after the readers of item i.
    auto finish_item = [&](f32x4 (&acc2)[2][NT], int f) {
        const int ii = f / nb;
        const int item = item_of(ii);
        const int s = item / rtiles, rt = item - s * rtiles;
        const int buf = ii & 1;
        fold_acc<NT>(acc2);
#pragma unroll
        for (int n = 0; n < NT; ++n) red[buf][w][n][lane] = acc2[0][n];
        // the ticket of item ii + 2, claimed one item ago (ticket t is item
        // S0 G + t; t >= R: none left)
        if (dyn && threadIdx.x == 0 && ii + 2 >= S0) sitem[(ii + 2) & 3] = ticket < R ? S0 * G + ticket : -1;
        __syncthreads();
        if (dyn && threadIdx.x == 0 && ii + 3 >= S0)
            ticket = __hip_atomic_fetch_add(p.gu_ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int nthr = kGuWaves * 64;
        const int o = ((int)threadIdx.x - (ii % kGuWaves) * 64 + nthr) % nthr;  // rotating owner wave
        if (o < 8 * T) {
            // output (intermediate row il = 8 rt + r, token t); D row r is gate,
            // D row 8 + r is up; column t (hi) and T + t (lo, split mode)
            const int r = o / T, t = o - r * T;
            float gv = 0.f, uv = 0.f;
#pragma unroll
            for (int part = 0; part < (SPLIT ? 2 : 1); ++part) {
                const int c = part ? T + t : t;
                const int n = c >> 4, col = c & 15;
                const int lg = 16 * (r >> 2) + col, lu = 16 * (2 + (r >> 2)) + col, j = r & 3;
#pragma unroll
                for (int q = 0; q < kGuWaves; ++q) {
                    gv += red[buf][q][n][lg][j];
                    uv += red[buf][q][n][lu][j];
                }
            }
            const int il = 8 * rt + r;
            if (KS > 1) {
                // this part's sums; the SwiGLU combine adds the parts
                float *pp = p.gu_part + (((size_t)hk * p.max_slots + s) * I + il) * 2 * T;
                pp[t] = gv;
                pp[T + t] = uv;
            } else {
                float wt;
                if (FUSED) {
                    // gate weight of token t for the slot's expert (1 for the
                    // always-on shared expert, 0 if the token is not routed
                    // to it), from the token's final selection
                    const int K = p.k, e = sexp[s];
                    wt = e == E ? 1.f : 0.f;
                    for (int j = 0; j < K; ++j)
                        if (fin[t * K + j] == e) wt = __int_as_float(fin[T * K + t * K + j]);
                } else {
                    wt = p.tokw[(size_t)s * T + t];
                }
                const float hv = wt * (silu(gv) * uv);
                const uint16_t hi = f32_to_bf16_rne(hv);
                uint16_t *hb = p.hB + (size_t)s * I * cstride;
                hb[b_index(il, t, cstride, WT == 1)] = hi;
                if (SPLIT) hb[b_index(il, T + t, cstride, WT == 1)] = f32_to_bf16_rne(hv - bf16_to_f32(hi));
            }
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) acc2[0][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    };

    f32x4 acc[2][NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[0][n] = acc[1][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Two register buffers; the prefetch is issued unconditionally (clamped
    // to the last batch) so the number of loads in flight is static.
    // A batch past the last item re-loads the previous batch and is not
    // computed, so every wave issues the same loads per step.
    int vo = 0;  // item order whose validity is cached (order 0 is valid here)
    bool vv = true;
    auto valid_ord = [&](int ord) {
        if (ord != vo) {
            vo = ord;
            vv = item_of(ord) >= 0;
        }
        return vv;
    };
    // The loop leaves only at its end: an exit between the two halves would
    // give the compiler a path to the loop head with the first half's loads
    // still pending, and it would then wait for them at every iteration.
    // After the last batch the second half re-loads that batch (its
    // products are zeroed) and the loop ends.
    B b0, b1;
    load_batch(b0, 0);
    for (int f = 0;; f += 2) {
        const bool v1 = valid_ord((f + 1) / nb);
        load_batch(b1, v1 ? f + 1 : f);
        compute_batch<WT, NT, KU>(b0, acc, true);
        if (f % nb == nb - 1) finish_item(acc, f);
        const bool v2 = v1 && valid_ord((f + 2) / nb);
        load_batch(b0, v2 ? f + 2 : (v1 ? f + 1 : f));
        compute_batch<WT, NT, KU>(b1, acc, v1);
        if (v1 && (f + 1) % nb == nb - 1) finish_item(acc, f + 1);
        if (!v2) break;
    }
    zero_y();
}

// ---------------------------------------------------------------------------
// down: a unit is RG row tiles (16 rows of H each) x one k-unit of one union
// slot.  A wave loads the unit's activation fragment once and multiplies it
// by the RG weight tiles, so the activation loads per weight byte drop by RG.
// The units (row group, slot, k-unit), row-group major, are split evenly
// over the grid (one workgroup of 8 waves per compute unit), so every compute
// unit streams the same bytes whatever the number of row groups.  Inside a
// row-group segment the waves take interleaved batches, accumulate y for all
// tokens in registers (the gate weights are already folded into the hidden
// activations) and meet in LDS in a fixed order.  A workgroup that owns a
// whole row group writes it to y.  A row group shared by exactly two
// workgroups (every group when the grid is twice the group count) is added
// into y, which the gate-up kernel zeroed, by one float atomic add per
// element from each: 0 + a + b rounds the same in either order, so no
// count, no wait and no re-read.  With three or more pieces, the pieces go
// to the workspace with device-scope stores, and the workgroup that
// completes the group's piece count adds them in workgroup order
// (device-scope loads) and writes y; starting from 0 it rounds exactly as
// the two-piece sum.  The result does not depend on timing, and no
// workgroup waits for another.
// ---------------------------------------------------------------------------
constexpr int kDnWaves = 8;

template <int WT, int NT>
struct DnCfg {
    // row tiles per unit: sharing the activation fragment over 2 row tiles
    // halves its L2 reads, which pays where the fragment is large (fp8: 4
    // k-steps per unit; bf16 with more than 16 columns); for bf16 with one
    // column tile the L2 reads are cheap and single row tiles balance better
    // (whole row tiles per workgroup at H = 4096, fewer pieces elsewhere)
    static constexpr int RG = (WT == 0 && NT == 1) ? 1 : (NT <= 2 || (WT == 0 && NT == 3) ? 2 : 1);
    static constexpr int KT = WT == 1 ? 64 : 32;                          // k per packed tile
    static constexpr int NA = WT == 1 ? 2 : 1;                            // tile loads per row tile
    static constexpr int NS = WT == 1 ? 4 : 1;                            // k-steps per unit
    static constexpr int KU = WT == 0 && NT == 1 ? 2 : 1;                 // units per batch
};

template <int WT, int NT>
struct DnBatch {
    using C = DnCfg<WT, NT>;
    u32x4 a[C::KU][C::RG][C::NA];
    u32x4 b[C::KU][C::NS][NT];
    float sc[C::KU];
    bool on[C::KU];
};

// Products of one batch into acc[row tile][token tile]; skipped units
// multiply zeros (no branch, so the waits before the products only count
// loads issued before this batch's own).
template <int WT, int NT>
__device__ __forceinline__ void dn_compute(const DnBatch<WT, NT> &bt, f32x4 (&acc)[DnCfg<WT, NT>::RG][NT], bool valid) {
    using C = DnCfg<WT, NT>;
    const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < C::KU; ++u) {
        const bool on = valid && bt.on[u];
        if (WT == 0) {
#pragma unroll
            for (int r = 0; r < C::RG; ++r) {
                const bf16x8 a = as_bf16x8(on ? bt.a[u][r][0] : zero);
#pragma unroll
                for (int n = 0; n < NT; ++n) acc[r][n] = mfma(a, as_bf16x8(bt.b[u][0][n]), acc[r][n]);
            }
        } else {
            const float sc = on ? bt.sc[u] : 0.f;
#pragma unroll
            for (int r = 0; r < C::RG; ++r) {
                f32x4 t[2][NT];
#pragma unroll
                for (int n = 0; n < NT; ++n) t[0][n] = t[1][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    bf16x8 lo, hi;
                    fp8x16_to_bf16(bt.a[u][r][h], lo, hi);
#pragma unroll
                    for (int n = 0; n < NT; ++n) {
                        t[0][n] = mfma(lo, as_bf16x8(bt.b[u][2 * h][n]), t[0][n]);
                        t[1][n] = mfma(hi, as_bf16x8(bt.b[u][2 * h + 1][n]), t[1][n]);
                    }
                }
#pragma unroll
                for (int n = 0; n < NT; ++n) acc[r][n] += sc * (t[0][n] + t[1][n]);
            }
        }
    }
}

// Workgroup that owns unit u when W units are split over G workgroups as
// [b W / G, (b + 1) W / G).
__device__ __forceinline__ int unit_owner(long long u, long long W, int G) {
    return (int)(((u + 1) * G - 1) / W);
}

template <int WT, int NT, bool SPLIT>
__global__ __launch_bounds__(kDnWaves * 64) void down_kernel(VerifyParams p) {
    using C = DnCfg<WT, NT>;
    using B = DnBatch<WT, NT>;
    constexpr int RG = C::RG, KU = C::KU;
    __shared__ f32x4 red[kDnWaves][RG][NT][64];
    __shared__ int sexp[kMaxExperts + 1];
    __shared__ int last_sh;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = lane >> 4, lr = lane & 15;
    const int T = p.T, H = p.H, I = p.I, E = p.E, cstride = p.cstride;
    const int nkt = I / C::KT;
    const int rtiles = H / 16;
    const int ngroups = (rtiles + RG - 1) / RG;
    const int nslots = min(p.meta[1], p.max_slots);
    const size_t esz = WT == 1 ? 1 : 2;
    const size_t bstep = (size_t)4 * cstride * 8;
    for (int i = threadIdx.x; i < nslots; i += kDnWaves * 64)
        sexp[i] = min(max(p.slot_expert[i], 0), p.has_shared ? E : E - 1);
    __syncthreads();
    // Units of one row group: (slot, k-unit) slot-major; batches of KU
    // consecutive units go to the waves round-robin, so the workgroup reads
    // a window that moves through the slots' row-group segments.
    const int nunits = WT == 1 ? nkt / 2 : nkt;
    const long long per_group = (long long)nslots * nunits;
    const long long W = per_group * ngroups;
    const int G = gridDim.x, bid = blockIdx.x;
    const long long u0 = (long long)bid * W / G, u1 = (long long)(bid + 1) * W / G;
    const int sld = I / 128;
    const uint16_t *hb0 = p.hB + (size_t)g * cstride * 8;
    int coff[NT];
    col_offsets<NT>(coff, lr, p.cols);
    const int pstride = RG * T * 16;  // floats per piece slot
    float *ypart = p.ypart + (size_t)bid * 2 * pstride;

    for (long long a = u0; a < u1;) {
        const int rg = (int)(a / per_group);
        const long long tb = (long long)rg * per_group, te = tb + per_group;
        const long long ae = u1 < te ? u1 : te;
        const int qa = (int)(a - tb), qb = (int)(ae - tb);  // units [qa, qb) of row group rg
        const int nbt = (qb - qa + KU - 1) / KU;
        const int nbw = nbt > w ? (nbt - w + kDnWaves - 1) / kDnWaves : 0;  // this wave's batches
        // row tiles of the group in the packed layout (groups of 4 row tiles,
        // then K-tile, then the tile inside the group; a ragged last group
        // re-reads its last tile for the missing ones and drops their outputs)
        size_t toff[RG];
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            const int rt = min(rg * RG + r, rtiles - 1);
            toff[r] = ((size_t)(rt >> 2) * nkt * 4 + (rt & 3)) * 1024 + lane * 16;
        }
        const int srow = (16 * rg * RG) / 128;  // 128-row scale block of the group (16 RG <= 128)
        // weight and scale bases of the slot being loaded, refreshed when the
        // wave's units move to the next slot (units are slot-major)
        int c_s = -1;
        const uint8_t *c_wb = nullptr;
        const float *c_sb = nullptr;
        auto load_batch = [&](B &bt, int f) {
            const int q0 = qa + (f * kDnWaves + w) * KU;
#pragma unroll
            for (int u = 0; u < KU; ++u) {
                const int q = q0 + u;
                const bool on = q < qb;
                const int qc = on ? q : qb - 1;
                const int s = qc / nunits, kk = qc - s * nunits;
                if (s != c_s) {
                    c_s = s;
                    const int e = sexp[s];
                    const bool sh = e == E;
                    c_wb = sh ? static_cast<const uint8_t *>(p.Wsh_d)
                              : static_cast<const uint8_t *>(p.W_d) + (size_t)e * H * I * esz;
                    if (WT == 1) c_sb = (sh ? p.ssh_d : p.s_d + (size_t)e * (H / 128) * sld) + srow * sld;
                }
                // K-tile kk * NA + h of row tile r sits 4 KB per K-tile apart
                const uint8_t *wb = c_wb + (size_t)kk * C::NA * 4096;
                bt.on[u] = on;
#pragma unroll
                for (int r = 0; r < RG; ++r)
#pragma unroll
                    for (int h = 0; h < C::NA; ++h) bt.a[u][r][h] = ld_nt(wb + toff[r] + h * 4096);
                const uint16_t *bq = hb0 + (size_t)s * I * cstride + (size_t)kk * C::NS * bstep;
#pragma unroll
                for (int q2 = 0; q2 < C::NS; ++q2)
#pragma unroll
                    for (int n = 0; n < NT; ++n)
                        bt.b[u][q2][n] = *reinterpret_cast<const u32x4 *>(bq + q2 * bstep + coff[n]);
                bt.sc[u] = WT == 1 ? c_sb[kk] : 0.f;
            }
        };
        f32x4 acc[RG][NT];
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[r][n] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (nbw > 0) {
            B b0, b1;
            load_batch(b0, 0);
            // the scheduling barriers keep each batch's loads issued before
            // the products of the batch before it, so one batch is always in
            // flight while the other is multiplied
            for (int f = 0; f < nbw; f += 2) {
                load_batch(b1, min(f + 1, nbw - 1));
                __builtin_amdgcn_sched_barrier(0);
                dn_compute<WT, NT>(b0, acc, true);
                load_batch(b0, min(f + 2, nbw - 1));
                __builtin_amdgcn_sched_barrier(0);
                dn_compute<WT, NT>(b1, acc, f + 1 < nbw);
            }
        }
        // partial sums of the waves meet in LDS in wave order
        if (w != 0) {
#pragma unroll
            for (int r = 0; r < RG; ++r)
#pragma unroll
                for (int n = 0; n < NT; ++n) red[w][r][n][lane] = acc[r][n];
        }
        __syncthreads();
        const bool whole = qa == 0 && qb == per_group;
        const int first = whole ? 0 : unit_owner(tb, W, G), last = whole ? 0 : unit_owner(te - 1, W, G);
        // pieces = workgroups in [first, last] with a non-empty range; a row
        // group of exactly two pieces is added into y (zeroed by the router
        // kernel) by two float atomic adds: 0 + a + b rounds the same in
        // either order, and the same as the fix-up's sum
        int np = 0;
        for (int ob = first; !whole && ob <= last; ++ob)
            np += (long long)ob * W / G < (long long)(ob + 1) * W / G ? 1 : 0;
        const bool pair = !whole && np == 2;
        if (w == 0) {
#pragma unroll
            for (int q2 = 1; q2 < kDnWaves; ++q2)
#pragma unroll
                for (int r = 0; r < RG; ++r)
#pragma unroll
                    for (int n = 0; n < NT; ++n) acc[r][n] += red[q2][r][n][lane];
            // a piece goes to this workgroup's slot (0 for its first row
            // group, 1 for its last)
            float *dst = ypart + (a == u0 ? 0 : pstride) + 4 * g;
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                float v[NT][4];
                combine_split<NT, SPLIT>(v, acc[r], T, lane);
                const int rt = rg * RG + r;
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    const int t = n * 16 + lr;
                    if (t >= T) continue;
                    if (whole) {
                        if (rt < rtiles)
                            *reinterpret_cast<float4 *>(p.y + (size_t)t * H + 16 * rt + 4 * g) =
                                make_float4(v[n][0], v[n][1], v[n][2], v[n][3]);
                    } else if (pair) {
                        if (rt < rtiles)
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                __hip_atomic_fetch_add(p.y + (size_t)t * H + 16 * rt + 4 * g + j, v[n][j],
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            __hip_atomic_store(dst + (size_t)(r * T + t) * 16 + j, v[n][j], __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            }
            if (!whole && !pair) {
                // once the piece's stores have completed, the group's piece
                // counter counts it
                wait_vm_all();
                if (lane == 0) {
                    last_sh = __hip_atomic_fetch_add(p.tile_cnt + rg, 1, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT) == np - 1;
                }
            }
        }
        if (!whole && !pair) {
            __syncthreads();
            if (last_sh && w == 0) {
                // every piece is complete: add them in workgroup order; a
                // workgroup's slot is 0 when this row group is its first one
#pragma unroll
                for (int r = 0; r < RG; ++r) {
                    const int rt = rg * RG + r;
                    float v[NT][4] = {};
                    for (int ob = first; ob <= last; ++ob) {
                        const long long os = (long long)ob * W / G;
                        if (os == (long long)(ob + 1) * W / G) continue;  // empty range: no piece
                        const float *src = p.ypart + (size_t)ob * 2 * pstride + (os / per_group == rg ? 0 : pstride) +
                                           (size_t)r * T * 16 + 4 * g;
#pragma unroll
                        for (int n = 0; n < NT; ++n) {
                            const int t = n * 16 + lr;
                            if (t < T)
#pragma unroll
                                for (int j = 0; j < 4; ++j)
                                    v[n][j] += __hip_atomic_load(src + (size_t)t * 16 + j, __ATOMIC_RELAXED,
                                                                 __HIP_MEMORY_SCOPE_AGENT);
                        }
                    }
#pragma unroll
                    for (int n = 0; n < NT; ++n) {
                        const int t = n * 16 + lr;
                        if (t < T && rt < rtiles)
                            *reinterpret_cast<float4 *>(p.y + (size_t)t * H + 16 * rt + 4 * g) =
                                make_float4(v[n][0], v[n][1], v[n][2], v[n][3]);
                    }
                }
            }
        }
        __syncthreads();
        a = ae;
    }
}

// ---------------------------------------------------------------------------
// SwiGLU of a split contraction: h = w_t * SiLU(sum of the gate parts) *
// (sum of the up parts), parts added in part order, written as the bf16
// operand of the down kernel.  One thread per (slot, intermediate row,
// token); consecutive threads read consecutive tokens.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void swiglu_kernel(VerifyParams p, int ks) {
    const int T = p.T, I = p.I, cstride = p.cstride;
    const bool fp8 = p.wdtype == 2;
    const int nslots = min(p.meta[1], p.max_slots);
    const long long total = (long long)nslots * I * T;
    for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (long long)gridDim.x * 256) {
        const int t = (int)(idx % T);
        const long long r = idx / T;
        const int il = (int)(r % I), s = (int)(r / I);
        float gv = 0.f, uv = 0.f;
        for (int h = 0; h < ks; ++h) {
            const float *pp = p.gu_part + (((size_t)h * p.max_slots + s) * I + il) * 2 * T;
            gv += pp[t];
            uv += pp[T + t];
        }
        const float hv = p.tokw[(size_t)s * T + t] * (silu(gv) * uv);
        const uint16_t hi = f32_to_bf16_rne(hv);
        uint16_t *hb = p.hB + (size_t)s * I * cstride;
        hb[b_index(il, t, cstride, fp8)] = hi;
        if (p.split) hb[b_index(il, T + t, cstride, fp8)] = f32_to_bf16_rne(hv - bf16_to_f32(hi));
    }
}

// ---------------------------------------------------------------------------
// Float32 weights: one wave per (slot, row), lanes over the contraction.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kFfnThreads) void gateup_f32_kernel(VerifyParams p) {
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6), nw = gridDim.x * 4;
    const int T = p.T, H = p.H, I = p.I;
    const int items = min(p.meta[1], p.max_slots) * I;
    for (int item = gw; item < items; item += nw) {
        const int s = item / I, i = item - s * I;
        const int e = min(max(p.slot_expert[s], 0), p.has_shared ? p.E : p.E - 1);
        const float *wg = (e == p.E && p.has_shared ? static_cast<const float *>(p.Wsh_gu)
                                    : static_cast<const float *>(p.W_gu) + (size_t)e * 2 * I * H) +
                          (size_t)i * H;
        const float *wu = wg + (size_t)I * H;
        for (int t0 = 0; t0 < T; t0 += 8) {
            float ag[8], au[8];
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) ag[tt] = au[tt] = 0.f;
            for (int h = lane; h < H; h += 64) {
                const float a = wg[h], b = wu[h];
#pragma unroll
                for (int tt = 0; tt < 8; ++tt) {
                    if (t0 + tt < T) {
                        const float xv = p.x[(size_t)(t0 + tt) * H + h];
                        ag[tt] += a * xv;
                        au[tt] += b * xv;
                    }
                }
            }
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                const float gs = wave_sum(ag[tt]), us = wave_sum(au[tt]);
                const int t = t0 + tt;
                if (lane == 0 && t < T)
                    p.h32[((size_t)s * T + t) * I + i] = p.tokw[(size_t)s * T + t] * (silu(gs) * us);
            }
        }
    }
}

__global__ __launch_bounds__(kFfnThreads) void down_f32_kernel(VerifyParams p) {
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6), nw = gridDim.x * 4;
    const int T = p.T, H = p.H, I = p.I;
    const int items = min(p.meta[1], p.max_slots) * H;
    for (int item = gw; item < items; item += nw) {
        const int s = item / H, r = item - s * H;
        const int e = min(max(p.slot_expert[s], 0), p.has_shared ? p.E : p.E - 1);
        const float *wd = (e == p.E && p.has_shared ? static_cast<const float *>(p.Wsh_d)
                                    : static_cast<const float *>(p.W_d) + (size_t)e * H * I) +
                          (size_t)r * I;
        for (int t0 = 0; t0 < T; t0 += 8) {
            float acc[8];
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) acc[tt] = 0.f;
            for (int i = lane; i < I; i += 64) {
                const float a = wd[i];
#pragma unroll
                for (int tt = 0; tt < 8; ++tt)
                    if (t0 + tt < T) acc[tt] += a * p.h32[((size_t)s * T + t0 + tt) * I + i];
            }
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
                const float v = wave_sum(acc[tt]);
                const int t = t0 + tt;
                if (lane == 0 && t < T) {
                    const int pos = p.tokpos[(size_t)s * T + t];
                    if (pos >= 0 && pos < T * p.k + T) p.ydown[(size_t)pos * H + r] = v;
                }
            }
        }
    }
}

__global__ __launch_bounds__(256) void combine_kernel(VerifyParams p) {
    const int T = p.T, H = p.H, k = p.k;
    const int total = T * H;
    for (int idx = blockIdx.x * 256 + threadIdx.x; idx < total; idx += gridDim.x * 256) {
        const int t = idx / H, r = idx - t * H;
        float acc = 0.f;
        for (int j = 0; j < k; ++j) {
            const int pos = p.tpos[t * k + j];
            if (pos >= 0 && pos < T * k) acc += p.ydown[(size_t)pos * H + r];
        }
        if (p.has_shared) acc += p.ydown[(size_t)(T * k + t) * H + r];
        p.y[idx] = acc;
    }
}


// LDS plan of the gate-up kernel: routing fused into its prologue and the
// activation operand held in LDS when they fit in one compute unit.
// ks: workgroups that share the contraction of an item (the operand slice
// of each must fit in LDS); the smallest that fits is taken.
struct GuPlan {
    bool fused, blds, async_x;
    int ks;   // workgroups sharing one item's contraction
    int ngl;  // units of every batch whose operand is read from global memory
    size_t dyn;
};

// Preference: the whole contraction per workgroup with the operand in LDS;
// then (bf16) the whole contraction with the operand of 1 (or 2) of every
// batch's units read from L2; then the contraction split over 2 or 4
// workgroups (partial sums plus a combine launch); then the operand read
// from L2 alone.  For each, the operand in a region of its own (its copy
// overlaps the routing) before an overlay on the routing scratch.
GuPlan plan_gateup(const VerifyParams &p) {
    const int nt = (p.cols + 15) / 16;
    const size_t stat = sizeof(float) * 4 * 2 * kGuWaves * nt * 64 + sizeof(int) * (kMaxExperts + 6);
    auto al = [](size_t v) { return (v + 15) & ~(size_t)15; };
    const size_t scr = al(RouteScratch::bytes(p.T, p.k, p.E, kGuWaves, true, route_nseq(p)));
    const size_t fin = (size_t)p.T * p.k * 8;
    const int nunits = p.wdtype == 2 ? p.H / 128 : p.H / 32;
    const int kspu = p.wdtype == 2 ? 4 : 1;
    const int ku = gu_batch_units(p.wdtype, nt);
    auto try_plan = [&](int ks, int ngl, GuPlan &out) {
        const int nuh = nunits / ks, kl = ku - ngl;
        const int nl = ngl == 0 ? nuh : (nuh / ku) * kl + std::min(nuh % ku, kl);
        const size_t xb = (size_t)nl * kspu * 4 * p.cols * 16;
        const size_t over = xb > scr ? xb : scr;
        if (xb + scr + fin + stat <= kLdsPerCu) {
            out = {true, true, true, ks, ngl, xb + scr + fin};
            return true;
        }
        if (over + fin + stat <= kLdsPerCu) {
            out = {true, true, false, ks, ngl, over + fin};
            return true;
        }
        return false;
    };
    GuPlan pl{};
    if (try_plan(1, 0, pl)) return pl;
    for (int ngl = 1; ngl < ku && ngl <= 2; ++ngl)
        if (try_plan(1, ngl, pl)) return pl;
    for (int ks = 2; ks <= kGuMaxSplit; ks *= 2) {
        if (nunits % ks != 0) break;
        if (try_plan(ks, 0, pl)) return pl;
    }
    if (scr + fin + stat <= kLdsPerCu) return {true, false, false, 1, 0, scr + fin};
    return {false, false, false, 1, 0, 0};
}

template <typename K>
hipError_t launch_gu(K kernel, const VerifyParams &p, size_t dyn, int n_cu, hipStream_t s, KernelEvents ev) {
    if (dyn > 64 * 1024 &&
        hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)dyn) != hipSuccess)
        return hipErrorInvalidValue;
    return launch_k(kernel, dim3(n_cu * kGateUpWgPerCu), dim3(kGuWaves * 64), dyn, s, ev, p);
}

template <int WT, int NT, bool SPLIT, bool GU>
hipError_t launch_one(const VerifyParams &p, int n_cu, hipStream_t s, KernelEvents ev) {
    if (GU) {
        const GuPlan pl = plan_gateup(p);
        VerifyParams q = p;
        q.gu_async_x = pl.async_x ? 1 : 0;
        if (pl.fused && pl.blds) {
            if constexpr (UnitCfg<WT, NT>::KU > 1) {
                if (pl.ks == 1 && pl.ngl == 1)
                    return launch_gu(gateup_kernel<WT, NT, SPLIT, true, true, 1, 1>, q, pl.dyn, n_cu, s, ev);
                if constexpr (UnitCfg<WT, NT>::KU > 2)
                    if (pl.ks == 1 && pl.ngl == 2)
                        return launch_gu(gateup_kernel<WT, NT, SPLIT, true, true, 1, 2>, q, pl.dyn, n_cu, s, ev);
            }
            if (pl.ngl != 0) return hipErrorInvalidValue;
            if (pl.ks == 1) return launch_gu(gateup_kernel<WT, NT, SPLIT, true, true, 1, 0>, q, pl.dyn, n_cu, s, ev);
            if (pl.ks == 2) return launch_gu(gateup_kernel<WT, NT, SPLIT, true, true, 2, 0>, q, pl.dyn, n_cu, s, ev);
            return launch_gu(gateup_kernel<WT, NT, SPLIT, true, true, 4, 0>, q, pl.dyn, n_cu, s, ev);
        }
        if (pl.fused) return launch_gu(gateup_kernel<WT, NT, SPLIT, true, false, 1, 0>, q, pl.dyn, n_cu, s, ev);
        return launch_gu(gateup_kernel<WT, NT, SPLIT, false, false, 1, 0>, q, 0, n_cu, s, ev);
    } else {
        // one workgroup per compute unit; the work splits evenly over them.
        // When the row groups number at least 80% of the compute units, one
        // workgroup per row group instead: no row group is shared, so no
        // pieces are exchanged, for a small rise in each workgroup's rate
        // (fewer groups would ask more of each workgroup than it streams).
        // With fewer row groups, the largest grid of at least 7/8 of the
        // compute units whose ranges give no row group three pieces (two
        // interior range boundaries), so that every shared group is added
        // into y by the two-piece atomics (GPT-OSS, 180 groups: 240
        // workgroups, down 36.2 -> 34.6 us against 256 with three-piece
        // groups).  Positions are compared in row groups: boundary b sits at
        // b * ngroups / G groups, exactly at a group start when that divides.
        int grid = n_cu < kDownMaxGrid ? n_cu : kDownMaxGrid;
        const int ngroups = (p.H / 16 + DnCfg<WT, NT>::RG - 1) / DnCfg<WT, NT>::RG;
        if (ngroups <= grid && ngroups * 10 >= grid * 8) {
            grid = ngroups;
        } else if (ngroups < grid) {
            for (int G = grid; G * 8 >= grid * 7; --G) {
                bool ok = true;
                for (long long b = 1; ok && b + 1 < G; ++b)
                    ok = (b * ngroups) % G == 0 || ((b + 1) * ngroups) % G == 0 ||
                         (b * ngroups) / G != ((b + 1) * ngroups) / G;
                if (ok) {
                    grid = G;
                    break;
                }
            }
        }
        return launch_k(down_kernel<WT, NT, SPLIT>, dim3(grid), dim3(kDnWaves * 64), 0, s, ev, p);
    }
}

template <int WT, bool GU>
hipError_t launch_mfma(const VerifyParams &p, int n_cu, hipStream_t s, KernelEvents ev) {
    const int nt = (p.cols + 15) / 16;
    if (p.split) {
        switch (nt) {
            case 1: return launch_one<WT, 1, true, GU>(p, n_cu, s, ev);
            case 2: return launch_one<WT, 2, true, GU>(p, n_cu, s, ev);
            case 3: return launch_one<WT, 3, true, GU>(p, n_cu, s, ev);
            default: return launch_one<WT, 4, true, GU>(p, n_cu, s, ev);
        }
    }
    switch (nt) {
        case 1: return launch_one<WT, 1, false, GU>(p, n_cu, s, ev);
        case 2: return launch_one<WT, 2, false, GU>(p, n_cu, s, ev);
        case 3: return launch_one<WT, 3, false, GU>(p, n_cu, s, ev);
        default: return launch_one<WT, 4, false, GU>(p, n_cu, s, ev);
    }
}

}  // namespace

bool gateup_fuses_routing(const VerifyParams &p) { return p.wdtype != 0 && plan_gateup(p).fused; }

int gateup_ksplit(const VerifyParams &p) { return p.wdtype != 0 ? plan_gateup(p).ks : 1; }

hipError_t launch_swiglu(const VerifyParams &p, int ks, hipStream_t s, KernelEvents ev) {
    long long blocks = ((long long)p.max_slots * p.I * p.T + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    return launch_k(swiglu_kernel, dim3((unsigned)blocks), dim3(256), 0, s, ev, p, ks);
}

hipError_t launch_gateup(const VerifyParams &p, int n_cu, hipStream_t s, KernelEvents ev) {
    const int grid = n_cu * 4;
    if (p.wdtype == 0) return launch_k(gateup_f32_kernel, dim3(grid), dim3(kFfnThreads), 0, s, ev, p);
    return p.wdtype == 1 ? launch_mfma<0, true>(p, n_cu, s, ev) : launch_mfma<1, true>(p, n_cu, s, ev);
}

hipError_t launch_down(const VerifyParams &p, int n_cu, hipStream_t s, KernelEvents ev) {
    const int grid = n_cu * 4;
    if (p.wdtype == 0) return launch_k(down_f32_kernel, dim3(grid), dim3(kFfnThreads), 0, s, ev, p);
    return p.wdtype == 1 ? launch_mfma<0, false>(p, n_cu, s, ev) : launch_mfma<1, false>(p, n_cu, s, ev);
}

hipError_t launch_combine(const VerifyParams &p, hipStream_t s, KernelEvents ev) {
    if (p.wdtype != 0) return hipSuccess;  // the matrix-core down kernel writes y itself
    int blocks = (p.T * p.H + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    return launch_k(combine_kernel, dim3(blocks), dim3(256), 0, s, ev, p);
}

}  // namespace moe
