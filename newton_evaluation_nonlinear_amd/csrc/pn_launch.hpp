// Kernel launch that can carry its own timing events (HIP kernel files only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "pn_internal.hpp"

namespace pn {

// Launches `kernel`; when the host driver has set launch_timing() for this
// launch, the start and stop events are recorded with the kernel's own
// dispatch (hipExtLaunchKernel) instead of as separate stream commands, and
// the request is consumed.
template <typename F, typename... A>
hipError_t launch_maybe_timed(F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t st, A... args) {
    LaunchTiming& t = launch_timing();
    if (t.start) {
        hipExtLaunchKernelGGL(kernel, grid, block, static_cast<uint32_t>(lds), st, t.start, t.stop, 0u, args...);
        t = LaunchTiming{};
    } else {
        kernel<<<grid, block, lds, st>>>(args...);
    }
    return hipGetLastError();
}

}  // namespace pn
