// gc_grad_norm without a workspace: the tile partials live in a fixed
// per-device scratch array, for callers that cannot allocate device memory.
//
// `scratch` is a file-scope device array; each device holds its own copy
// until the process ends.  In host code its name is a host-side stand-in, not
// a device address, so host code never passes it to a kernel: the first call
// on a device (with that device current) looks up the device's address with
// hipGetSymbolAddress, keeps it, and the norm kernels get that address as
// their partials buffer, as they get the caller's workspace in gc_grad_norm.
#include <atomic>
#include <mutex>

#include "gc_common.h"

namespace gc {
namespace {

static_assert(GC_NORM_SCRATCH_TILES * sizeof(double) == 512 * 1024, "scratch size stated in gc.h");
static __device__ __align__(256) double scratch[GC_NORM_SCRATCH_TILES];

constexpr int SCRATCH_MAX_DEVICES = 64;
std::atomic<double*> g_scratch_ptr[SCRATCH_MAX_DEVICES];
std::mutex g_scratch_mu;

// The current device's scratch address, looked up once per device and kept.
// NULL, with the error detail set, on failure.
double* device_scratch(const char* fn) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        fail(GC_ERR_HIP, std::string(fn) + ": hipGetDevice: " + hipGetErrorString(e));
        return nullptr;
    }
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) {
        fail(GC_ERR_HIP, std::string(fn) + ": device index out of the supported range");
        return nullptr;
    }
    double* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p) return p;
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !addr) {
        fail(GC_ERR_HIP, std::string(fn) + ": hipGetSymbolAddress(scratch): " + hipGetErrorString(e));
        return nullptr;
    }
    p = static_cast<double*>(addr);
    g_scratch_ptr[dev].store(p, std::memory_order_release);
    return p;
}

}  // namespace
}  // namespace gc

using namespace gc;

extern "C" {

int gc_grad_norm_noalloc(const gc_span* layers, int nlayers, int grad_dtype, float* norms, void* stream) {
    const int rc = check_norm_args("gc_grad_norm_noalloc", layers, nlayers, grad_dtype, norms);
    if (rc != GC_OK) return rc;
    if (partial_count(layers, nlayers) > static_cast<size_t>(GC_NORM_SCRATCH_TILES))
        return fail(GC_ERR_ARG, "gc_grad_norm_noalloc: the layers need more than GC_NORM_SCRATCH_TILES "
                                "16384-entry tiles (the fixed scratch); use gc_grad_norm with a workspace");
    double* partial = device_scratch("gc_grad_norm_noalloc");
    if (!partial) return GC_ERR_HIP;
    return launch_norms(layers, nlayers, grad_dtype, norms, partial, static_cast<hipStream_t>(stream));
}

}  // extern "C"
