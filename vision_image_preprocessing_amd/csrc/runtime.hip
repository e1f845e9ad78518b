// runtime.hip -- host-side launch plumbing: the pinned staging ring for
// descriptor tables, launch timing events, the dispatch counter.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "runtime.h"

namespace mimo {

std::atomic<int64_t> g_dispatches{0};
thread_local hipEvent_t g_launch_start = nullptr;
thread_local hipEvent_t g_launch_stop = nullptr;

namespace {

// Pinned host staging for the per-call descriptor tables: a small ring per
// device, each slot fenced by an event so a slot is rewritten only after
// its previous copy has executed.
class TableStaging {
  public:
    struct Slot {
        void *host = nullptr;
        size_t cap = 0;
        hipEvent_t done = nullptr;
        bool pending = false;
    };
    static constexpr int kSlots = 8;

    // Copies bytes from `table` to device `dst` on `stream`, asynchronously.
    hipError_t upload(const void *table, size_t bytes, void *dst, hipStream_t stream) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        std::lock_guard<std::mutex> lock(mu_);
        if (int(rings_.size()) <= dev) rings_.resize(dev + 1);
        Ring &ring = rings_[dev];
        Slot &s = ring.slots[ring.next];
        ring.next = (ring.next + 1) % kSlots;
        if (s.pending) {
            e = hipEventSynchronize(s.done);
            if (e != hipSuccess) return e;
            s.pending = false;
        }
        if (!s.done) {
            e = hipEventCreateWithFlags(&s.done, hipEventDisableTiming);
            if (e != hipSuccess) return e;
        }
        if (s.cap < bytes) {
            if (s.host) (void)hipHostFree(s.host);
            s.host = nullptr;
            s.cap = 0;
            e = hipHostMalloc(&s.host, bytes, hipHostMallocDefault);
            if (e != hipSuccess) return e;
            s.cap = bytes;
        }
        std::memcpy(s.host, table, bytes);
        e = hipMemcpyAsync(dst, s.host, bytes, hipMemcpyHostToDevice, stream);
        if (e != hipSuccess) return e;
        e = hipEventRecord(s.done, stream);
        if (e != hipSuccess) return e;
        s.pending = true;
        return hipSuccess;
    }

  private:
    struct Ring {
        Slot slots[kSlots];
        int next = 0;
    };
    std::mutex mu_;
    std::vector<Ring> rings_;
};

TableStaging &staging() {
    static TableStaging *s = new TableStaging();  // lives until process exit
    return *s;
}

}  // namespace

hipError_t upload_table(const void *table, size_t bytes, void *dst, hipStream_t stream) {
    return staging().upload(table, bytes, dst, stream);
}

int hip_error(hipError_t e, const char *what) {
    return set_error(MIMO_E_HIP, std::string(what) + ": " + hipGetErrorName(e) + " (" +
                                     hipGetErrorString(e) + ")");
}

}  // namespace mimo

using namespace mimo;

extern "C" {

int64_t mimo_dispatch_count(void) { return g_dispatches.load(); }

int mimo_set_launch_events(void *start, void *stop) {
    clear_error();
    if ((start == nullptr) != (stop == nullptr))
        return set_error(MIMO_E_INVALID, "set_launch_events: give both events or neither");
    g_launch_start = static_cast<hipEvent_t>(start);
    g_launch_stop = static_cast<hipEvent_t>(stop);
    return MIMO_OK;
}

}  // extern "C"
