// runtime.h -- host-side launch plumbing shared by the library's entry
// points: descriptor-table uploads, launch timing events, the dispatch
// counter and HIP error reporting.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "internal.h"

namespace mimo {

extern std::atomic<int64_t> g_dispatches;     // kernel launches made so far
extern thread_local hipEvent_t g_launch_start;  // caller's events, or null
extern thread_local hipEvent_t g_launch_stop;

// Records the caller's timing events around one kernel launch.
template <typename Launch>
hipError_t timed_launch(hipStream_t s, Launch &&launch) {
    hipError_t e = hipSuccess;
    if (g_launch_start && (e = hipEventRecord(g_launch_start, s)) != hipSuccess) return e;
    launch();
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (g_launch_stop && (e = hipEventRecord(g_launch_stop, s)) != hipSuccess) return e;
    return hipSuccess;
}

// Copies a host table to device memory on `stream` through a pinned
// staging ring (asynchronous; the host buffer may be reused at once).
hipError_t upload_table(const void *table, size_t bytes, void *dst, hipStream_t stream);

// Records a HIP failure as the thread's last error; returns MIMO_E_HIP.
int hip_error(hipError_t e, const char *what);

inline int check_ptr_align(const void *p, uintptr_t align) {
    return (reinterpret_cast<uintptr_t>(p) & (align - 1)) == 0;
}

}  // namespace mimo
