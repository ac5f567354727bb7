// Kernel launch with optional start/end events, for the HIP translation
// units that launch kernels (the host-side validation in moe_verify.cpp does
// not need it).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "internal.h"

namespace moe {

// With an event set, the kernel is launched through hipExtLaunchKernelGGL so
// that the events mark the start and the end of its execution on the stream
// (either may be null, so a stage can span two launches).
template <typename F, typename... Args>
hipError_t launch_k(F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, KernelEvents ev, Args... args) {
    if (ev.start || ev.stop)
        hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, ev.start, ev.stop, 0u, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
    return hipGetLastError();
}

}  // namespace moe
