// Recorder of the launches requested by the host side of libmoeverify (see
// stub_launch.cpp).
#pragma once

#include <hip/hip_runtime.h>

#include "internal.h"

namespace stub {
struct Record {
    int router = 0, route = 0, gateup = 0, swiglu = 0, down = 0, combine = 0, pack = 0, probe = 0, stats = 0,
        select = 0, expand = 0, segments = 0, gate = 0;
    int select_n = 0, expand_last_parent = 0, seg_last_off = 0;
    moe::VerifyParams last{};
};
extern Record rec;
}  // namespace stub
