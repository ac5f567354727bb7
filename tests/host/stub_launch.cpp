// Launchers of libmoeverify replaced by recorders, so that the host side
// (argument validation, workspace layout, launch sequence of moe_verify.cpp)
// can run under AddressSanitizer and UndefinedBehaviorSanitizer on a machine
// without a GPU.  Every stub records what it was asked to launch and returns
// hipSuccess; nothing is enqueued.
#include "stub_launch.h"

namespace stub {
Record rec;
}

namespace moe {

using stub::rec;

hipError_t launch_router(const VerifyParams &p, hipStream_t, KernelEvents) {
    ++rec.router;
    rec.last = p;
    return hipSuccess;
}
hipError_t launch_route(const VerifyParams &p, hipStream_t, KernelEvents) {
    ++rec.route;
    rec.last = p;
    return hipSuccess;
}
hipError_t launch_gateup(const VerifyParams &p, int, hipStream_t, KernelEvents) {
    ++rec.gateup;
    rec.last = p;
    return hipSuccess;
}
bool gateup_fuses_routing(const VerifyParams &p) { return p.wdtype != 0; }
int gateup_ksplit(const VerifyParams &) { return 1; }
hipError_t launch_swiglu(const VerifyParams &, int, hipStream_t, KernelEvents) {
    ++rec.swiglu;
    return hipSuccess;
}
hipError_t launch_down(const VerifyParams &, int, hipStream_t, KernelEvents) {
    ++rec.down;
    return hipSuccess;
}
hipError_t launch_combine(const VerifyParams &, hipStream_t, KernelEvents) {
    ++rec.combine;
    return hipSuccess;
}
hipError_t launch_pack(const void *, void *, int, int, int, int, int, int, hipStream_t) {
    ++rec.pack;
    return hipSuccess;
}
hipError_t launch_read_probe(const void *, size_t, uint32_t *, int, hipStream_t) {
    ++rec.probe;
    return hipSuccess;
}
hipError_t launch_union_stats(const int32_t *, int, int, int, int, int32_t *, float *, hipStream_t) {
    ++rec.stats;
    return hipSuccess;
}
hipError_t launch_select(int N, const float *, const uint32_t *, int, int, float, int, int32_t *, bool,
                         hipStream_t) {
    ++rec.select;
    rec.select_n = N;
    return hipSuccess;
}
size_t expand_lds_bytes(int N, int W, bool staged) {
    return ((staged ? (size_t)N * W : 0) + W + 3 * (size_t)N + (N + 31) / 32) * 4;
}
hipError_t launch_expand(ExpandArgs a, const float *, const uint32_t *, const float *, int32_t *, int32_t *,
                         hipStream_t) {
    ++rec.expand;
    rec.expand_last_parent = a.N > 0 ? a.parent[a.N - 1] : -9;
    return hipSuccess;
}
hipError_t launch_segment_stats(const int32_t *, int, int, int, int, const SegmentArgs &a, int32_t *, int32_t *,
                                hipStream_t) {
    ++rec.segments;
    rec.seg_last_off = a.off[a.S];
    return hipSuccess;
}
size_t gate_lds_bytes(int) { return 0; }
hipError_t launch_gate_depths(const float *, const uint32_t *, int, int, int, float, float, int32_t *,
                              hipStream_t) {
    ++rec.gate;
    return hipSuccess;
}

}  // namespace moe
