// Optional per-kernel timing with HIP events (see kda_profile_enable in kda.h).
#pragma once

#include <hip/hip_runtime.h>

namespace kda {

// Brackets one kernel launch with a pair of events on its stream when timing
// is enabled on the calling thread; does nothing otherwise.
class LaunchTimer {
public:
    LaunchTimer(const char* name, hipStream_t s);
    ~LaunchTimer();
    LaunchTimer(const LaunchTimer&) = delete;
    LaunchTimer& operator=(const LaunchTimer&) = delete;

private:
    int slot_;
    hipStream_t stream_;
};

}  // namespace kda
