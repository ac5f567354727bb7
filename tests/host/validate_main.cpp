// Host-side checks of libmoeverify's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (g++): argument validation, workspace layout
// and the launch sequence of every entry point, with the kernel launchers
// replaced by recorders (stub_launch.cpp).  Buffers are real host
// allocations standing in for device pointers; nothing is dereferenced on
// the host except the arrays the ABI marks (host).  Exit status 0 = pass.
#include <cstdio>
#include <cstring>
#include <vector>

#include "moe_verify.h"
#include "stub_launch.h"

static int failures = 0;
#define CHECK(cond)                                                                      \
    do {                                                                                 \
        if (!(cond)) {                                                                   \
            std::fprintf(stderr, "FAIL %s:%d: %s (%s)\n", __FILE__, __LINE__, #cond,     \
                         moe_last_error());                                              \
            ++failures;                                                                  \
        }                                                                                \
    } while (0)

// 256-byte aligned host block standing in for device memory
struct Block {
    std::vector<unsigned char> raw;
    unsigned char *p;
    explicit Block(size_t n) : raw(n + 256) {
        p = raw.data() + ((256 - (reinterpret_cast<uintptr_t>(raw.data()) & 255)) & 255);
    }
};

static moe_layer bf16_layer(Block &w, int H = 512, int I = 256, int E = 32, int k = 4) {
    moe_layer L{};
    L.H = H;
    L.I = I;
    L.E = E;
    L.k = k;
    L.wdtype = MOE_BF16;
    L.Wr = reinterpret_cast<const float *>(w.p);
    L.W_gu = w.p;
    L.W_d = w.p;
    return L;
}

int main() {
    Block w(1 << 16), x(1 << 16), y(1 << 16);
    // ---- workspace sizes and shape validation ----
    moe_layer L = bf16_layer(w);
    const size_t ws5 = moe_verify_workspace_bytes(&L, 5, nullptr);
    CHECK(ws5 > 0);
    CHECK(moe_verify_workspace_bytes(&L, 64, nullptr) > ws5);
    CHECK(moe_verify_workspace_bytes(&L, 0, nullptr) == 0);
    CHECK(moe_verify_workspace_bytes(&L, 65, nullptr) == 0);
    CHECK(moe_verify_workspace_bytes(nullptr, 5, nullptr) == 0);
    {
        moe_layer b = L;
        b.E = 513;
        CHECK(moe_verify_workspace_bytes(&b, 5, nullptr) == 0);
        b = L;
        b.k = 33;
        b.E = 64;
        CHECK(moe_verify_workspace_bytes(&b, 5, nullptr) == 0);
        b = L;
        b.wdtype = MOE_FP8_E4M3;
        b.H = 192;
        CHECK(moe_verify_workspace_bytes(&b, 5, nullptr) == 0);
        b = L;
        b.Wsh_gu = w.p;  // half a shared expert
        CHECK(moe_verify_workspace_bytes(&b, 5, nullptr) == 0);
    }
    // ---- the bias and its sequence offsets ----
    float wconf[64] = {};
    moe_bias bias{8, 0.5f, wconf, 0, nullptr};
    CHECK(moe_verify_workspace_bytes(&L, 20, &bias) > 0);
    bias.cap = 3;  // cap < k
    CHECK(moe_verify_workspace_bytes(&L, 20, &bias) == 0);
    bias.cap = 8;
    bias.alpha = 1.0f;
    CHECK(moe_verify_workspace_bytes(&L, 20, &bias) == 0);
    bias.alpha = 0.5f;
    int32_t off[65];
    for (int s = 0; s <= 64; ++s) off[s] = s < 64 ? s : 64;  // 64 sequences of one token
    bias.nseg = 64;
    bias.seg_off = off;
    CHECK(moe_verify_workspace_bytes(&L, 64, &bias) >= moe_verify_workspace_bytes(&L, 64, nullptr));
    bias.nseg = 65;
    CHECK(moe_verify_workspace_bytes(&L, 64, &bias) == 0);
    bias.nseg = 4;
    bias.seg_off = nullptr;
    CHECK(moe_verify_workspace_bytes(&L, 20, &bias) == 0);
    int32_t off4[5] = {0, 5, 10, 15, 19};  // does not end at T
    bias.seg_off = off4;
    CHECK(moe_verify_workspace_bytes(&L, 20, &bias) == 0);
    int32_t off4d[5] = {0, 10, 5, 15, 20};  // decreasing
    bias.seg_off = off4d;
    CHECK(moe_verify_workspace_bytes(&L, 20, &bias) == 0);
    int32_t off4ok[5] = {0, 5, 5, 15, 20};  // an empty sequence
    bias.seg_off = off4ok;
    const size_t wsb = moe_verify_workspace_bytes(&L, 20, &bias);
    CHECK(wsb > 0);

    // ---- moe_verify_layer: errors before any launch, then a full launch ----
    Block ws(wsb + 4096);
    stub::rec = stub::Record{};
    CHECK(moe_verify_layer(&L, nullptr, 20, &bias, reinterpret_cast<float *>(y.p), nullptr, ws.p, wsb, nullptr) ==
          MOE_EINVAL);
    CHECK(moe_verify_layer(&L, reinterpret_cast<float *>(x.p), 20, &bias, reinterpret_cast<float *>(y.p), nullptr,
                           ws.p + 16, wsb, nullptr) == MOE_EINVAL);  // misaligned workspace
    CHECK(moe_verify_layer(&L, reinterpret_cast<float *>(x.p), 20, &bias, reinterpret_cast<float *>(y.p), nullptr,
                           ws.p, wsb - 1, nullptr) == MOE_EWORKSPACE);
    CHECK(moe_verify_layer(&L, reinterpret_cast<float *>(x.p + 4), 20, &bias, reinterpret_cast<float *>(y.p),
                           nullptr, ws.p, wsb, nullptr) == MOE_EINVAL);  // misaligned x
    CHECK(stub::rec.router == 0 && stub::rec.gateup == 0);
    moe_aux aux{};
    std::vector<float> logits(20 * 32);
    aux.logits = logits.data();
    int32_t usize = 0;
    aux.union_size = &usize;
    CHECK(moe_verify_layer(&L, reinterpret_cast<float *>(x.p), 20, &bias, reinterpret_cast<float *>(y.p), &aux,
                           ws.p, wsb, nullptr) == MOE_OK);
    CHECK(stub::rec.router == 1 && stub::rec.gateup == 1 && stub::rec.down == 1 && stub::rec.route == 0);
    CHECK(stub::rec.last.nseg == 4 && stub::rec.last.seg_off[0] == 0 && stub::rec.last.seg_off[2] == 5 &&
          stub::rec.last.seg_off[4] == 20);
    CHECK(stub::rec.last.cap == 8 && stub::rec.last.bias_on == 1 && stub::rec.last.T == 20);
    CHECK(stub::rec.last.logits == logits.data() && stub::rec.last.union_size_out == &usize);
    // every workspace section lies inside the workspace
    const unsigned char *lo = ws.p, *hi = ws.p + wsb;
    auto inside = [&](const void *q) {
        const unsigned char *c = static_cast<const unsigned char *>(q);
        return c >= lo && c < hi;
    };
    CHECK(inside(stub::rec.last.topk_idx) && inside(stub::rec.last.hB) && inside(stub::rec.last.xB) &&
          inside(stub::rec.last.ypart) && inside(stub::rec.last.tile_cnt) && inside(stub::rec.last.meta) &&
          inside(stub::rec.last.pstar) && inside(stub::rec.last.tokw));
    // float32 weights: standalone route kernel and the combine
    {
        moe_layer f = L;
        f.wdtype = MOE_F32;
        const size_t wsf = moe_verify_workspace_bytes(&f, 5, nullptr);
        Block wf(wsf);
        stub::rec = stub::Record{};
        CHECK(moe_verify_layer(&f, reinterpret_cast<float *>(x.p), 5, nullptr, reinterpret_cast<float *>(y.p),
                               nullptr, wf.p, wsf, nullptr) == MOE_OK);
        CHECK(stub::rec.route == 1 && stub::rec.combine == 1 && stub::rec.gateup == 1);
    }

    // ---- statistics, selection, expansion, ragged calls ----
    CHECK(union_stats(nullptr, 1, 5, 8, 128, nullptr, nullptr, nullptr) == MOE_EINVAL);
    CHECK(union_stats(reinterpret_cast<int32_t *>(x.p), 0, 5, 8, 128, reinterpret_cast<int32_t *>(y.p),
                      reinterpret_cast<float *>(y.p), nullptr) == MOE_OK);
    CHECK(union_stats(reinterpret_cast<int32_t *>(x.p), 2, 1 << 20, 32, 128, reinterpret_cast<int32_t *>(y.p),
                      reinterpret_cast<float *>(y.p), nullptr) == MOE_ENOTSUP);
    std::vector<int32_t> parent(4096);
    for (int i = 0; i < 4096; ++i) parent[i] = i == 0 ? -1 : (i - 1) / 2;
    stub::rec = stub::Record{};
    CHECK(select_drafts(parent.data(), 4096, reinterpret_cast<float *>(x.p), reinterpret_cast<uint32_t *>(x.p),
                        4096, 4, 1e-6f, 1, reinterpret_cast<int32_t *>(y.p), nullptr) == MOE_OK);
    CHECK(stub::rec.select == 1 && stub::rec.select_n == 4096);
    parent[100] = 100;
    CHECK(select_drafts(parent.data(), 4096, reinterpret_cast<float *>(x.p), reinterpret_cast<uint32_t *>(x.p), 16,
                        4, 1e-6f, 1, reinterpret_cast<int32_t *>(y.p), nullptr) == MOE_EINVAL);
    parent[100] = 49;
    CHECK(select_drafts(parent.data(), 16, reinterpret_cast<float *>(x.p), reinterpret_cast<uint32_t *>(x.p), 4097,
                        4, 1e-6f, 1, reinterpret_cast<int32_t *>(y.p), nullptr) == MOE_EINVAL);
    stub::rec = stub::Record{};
    CHECK(expand_drafts(parent.data(), 1024, reinterpret_cast<float *>(x.p), reinterpret_cast<uint32_t *>(x.p), 4,
                        1.f, 1.f, nullptr, 1, reinterpret_cast<int32_t *>(y.p), reinterpret_cast<int32_t *>(y.p),
                        nullptr) == MOE_OK);
    CHECK(stub::rec.expand == 1 && stub::rec.expand_last_parent == parent[1023]);
    CHECK(expand_drafts(parent.data(), 1025, reinterpret_cast<float *>(x.p), reinterpret_cast<uint32_t *>(x.p), 4,
                        1.f, 1.f, nullptr, 1, reinterpret_cast<int32_t *>(y.p), reinterpret_cast<int32_t *>(y.p),
                        nullptr) == MOE_EINVAL);
    int32_t seg[65];
    for (int s = 0; s <= 64; ++s) seg[s] = s;
    stub::rec = stub::Record{};
    CHECK(union_stats_segments(reinterpret_cast<int32_t *>(x.p), 3, 64, 4, 128, seg, 64,
                               reinterpret_cast<int32_t *>(y.p), reinterpret_cast<int32_t *>(y.p), nullptr) == MOE_OK);
    CHECK(stub::rec.segments == 1 && stub::rec.seg_last_off == 64);
    CHECK(union_stats_segments(reinterpret_cast<int32_t *>(x.p), 3, 64, 4, 128, seg, 65,
                               reinterpret_cast<int32_t *>(y.p), reinterpret_cast<int32_t *>(y.p), nullptr) ==
          MOE_EINVAL);
    seg[10] = 3;
    CHECK(union_stats_segments(reinterpret_cast<int32_t *>(x.p), 3, 64, 4, 128, seg, 64,
                               reinterpret_cast<int32_t *>(y.p), reinterpret_cast<int32_t *>(y.p), nullptr) ==
          MOE_EINVAL);
    CHECK(gate_depths(reinterpret_cast<float *>(x.p), reinterpret_cast<uint32_t *>(x.p), 65, 4, 4, 1.f, 1.f,
                      reinterpret_cast<int32_t *>(y.p), nullptr) == MOE_EINVAL);
    CHECK(gate_depths(reinterpret_cast<float *>(x.p), reinterpret_cast<uint32_t *>(x.p), 64, 64, 1024, 1.f, 1.f,
                      reinterpret_cast<int32_t *>(y.p), nullptr) == MOE_OK);

    // ---- packing and the read probe ----
    CHECK(moe_pack_weights(x.p, x.p + 64, 1, 64, 64, MOE_BF16, 0, nullptr) == MOE_EINVAL);  // overlap
    CHECK(moe_pack_weights(x.p, y.p, 1, 64, 64, MOE_BF16, 0, nullptr) == MOE_OK);
    CHECK(moe_stream_read(x.p, 1000, reinterpret_cast<uint32_t *>(y.p), nullptr) == MOE_EINVAL);
    CHECK(moe_stream_read(x.p, 1024, reinterpret_cast<uint32_t *>(y.p), nullptr) == MOE_OK);

    if (failures) {
        std::fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    std::printf("host validator: all checks passed\n");
    return 0;
}
