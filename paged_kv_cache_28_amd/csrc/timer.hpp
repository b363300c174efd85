// Kernel timer: HIP events bound to the library's own kernel launches.
//
// When enabled, each launch of a timed entry point is issued through
// hipExtLaunchKernelGGL with a fresh (start, stop) event pair, so the events carry the
// kernel's own begin and end timestamps; no marker packet is added to the stream and
// the work between kernels is not counted. pkv_timer_read() waits for the recorded
// pairs and returns the summed kernel time.
#pragma once

#include <hip/hip_runtime.h>

namespace pkv {

struct LaunchEvents {
    hipEvent_t start;
    hipEvent_t stop;
};

// Event pair for the next launch of `entry` (a PKV_TIMER_* code), or two null events
// when timing is off or the events could not be created.
LaunchEvents timer_events(int entry);

}  // namespace pkv
