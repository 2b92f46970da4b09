// Status strings, per-thread error detail and the optional launch timing hooks.
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "gc_common.h"

namespace gc {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

int fail(int status, const std::string& msg) {
    g_last_error = msg;
    return status;
}

int check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(GC_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
    return GC_OK;
}

// ---------------------------------------------------------------- timing hooks

// The hooks are the library's only process-wide state besides the scratch
// addresses of the allocation-free entry point.  A launch with timing off
// reads one atomic flag and takes no lock.
namespace {
std::atomic<bool> g_timing_on{false};
std::mutex g_tmu;
std::string g_timed_name;
struct EventPair { hipEvent_t a, b; };
std::vector<EventPair> g_events;
}  // namespace

TimedLaunch::TimedLaunch(const char* name, hipStream_t stream) : stream_(stream) {
    if (!g_timing_on.load(std::memory_order_acquire)) return;
    std::lock_guard<std::mutex> lk(g_tmu);
    if (g_timed_name.empty() || g_timed_name != name) return;
    // timing-only events: no system-scope fence (its cache write-back and
    // invalidate would slow the work after each event)
    if (hipEventCreateWithFlags(&start_, hipEventDisableSystemFence) != hipSuccess) { start_ = nullptr; return; }
    if (hipEventRecord(start_, stream_) != hipSuccess) { (void)hipEventDestroy(start_); start_ = nullptr; }
}

TimedLaunch::~TimedLaunch() {
    if (!start_) return;
    hipEvent_t stop = nullptr;
    if (hipEventCreateWithFlags(&stop, hipEventDisableSystemFence) != hipSuccess) {
        (void)hipEventDestroy(start_);
        return;
    }
    if (hipEventRecord(stop, stream_) != hipSuccess) {
        (void)hipEventDestroy(start_);
        (void)hipEventDestroy(stop);
        return;
    }
    std::lock_guard<std::mutex> lk(g_tmu);
    g_events.push_back({start_, stop});
}

static void drop_events_locked() {
    for (auto& e : g_events) {
        (void)hipEventDestroy(e.a);
        (void)hipEventDestroy(e.b);
    }
    g_events.clear();
}

}  // namespace gc

extern "C" {

const char* gc_status_str(int status) {
    switch (status) {
        case GC_OK: return "GC_OK";
        case GC_ERR_ARG: return "GC_ERR_ARG: invalid argument";
        case GC_ERR_DTYPE: return "GC_ERR_DTYPE: unknown gradient dtype";
        case GC_ERR_WORKSPACE: return "GC_ERR_WORKSPACE: workspace too small";
        case GC_ERR_HIP: return "GC_ERR_HIP: HIP runtime error";
        default: return "unknown status";
    }
}

const char* gc_last_error(void) { return gc::g_last_error.c_str(); }

int gc_timing_enable(const char* kernel_name) {
    std::lock_guard<std::mutex> lk(gc::g_tmu);
    gc::drop_events_locked();
    gc::g_timed_name = kernel_name ? kernel_name : "";
    gc::g_timing_on.store(!gc::g_timed_name.empty(), std::memory_order_release);
    return GC_OK;
}

int gc_timing_read(double* total_ms, int64_t* launches) {
    if (!total_ms || !launches) return gc::fail(GC_ERR_ARG, "gc_timing_read: null output pointer");
    std::lock_guard<std::mutex> lk(gc::g_tmu);
    double sum = 0.0;
    for (auto& e : gc::g_events) {
        if (hipEventSynchronize(e.b) != hipSuccess) {
            gc::drop_events_locked();
            return gc::fail(GC_ERR_HIP, "gc_timing_read: hipEventSynchronize failed");
        }
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, e.a, e.b) != hipSuccess) {
            gc::drop_events_locked();
            return gc::fail(GC_ERR_HIP, "gc_timing_read: hipEventElapsedTime failed");
        }
        sum += ms;
    }
    *total_ms = sum;
    *launches = static_cast<int64_t>(gc::g_events.size());
    gc::drop_events_locked();
    return GC_OK;
}

const char* gc_kernel_names(void) {
    return "topk_prep,topk_accum_hist,topk_capture,topk_select2,topk_refine,"
           "topk_count,topk_emit,topk_materialize,topk_decode_set,topk_decode_add,topk_small,randk_encode,"
           "psgd_pq,psgd_p,psgd_q,psgd_qreduce,psgd_out,psgd_decode,psgd_materialize,"
           "norm_partial,norm_final,passthrough";
}

}  // extern "C"
