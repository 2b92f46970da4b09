// Internal helpers shared by the gfx950 kernels and the C-ABI host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "../../include/gc.h"

namespace gc {

// ---------------------------------------------------------------- host side

void set_error(const std::string& msg);
int fail(int status, const std::string& msg);
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes) {
    uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + bbytes && b0 < a0 + abytes;
}
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Records a HIP event pair around one launch when timing is enabled for `name`.
class TimedLaunch {
public:
    TimedLaunch(const char* name, hipStream_t stream);
    ~TimedLaunch();
private:
    hipEvent_t start_ = nullptr;
    hipStream_t stream_;
};

// Checks the launch status right after a kernel launch.
int check_launch(const char* what);

// ---------------------------------------------------------------- device side

constexpr int WAVE = 64;

__device__ __forceinline__ unsigned key_of(float x) {
    // magnitude key: ordering of keys equals ordering of |x| for non-NaN x
    return __float_as_uint(x) & 0x7FFFFFFFu;
}

__device__ __forceinline__ float bf16_to_f32(unsigned short b) {
    return __uint_as_float(static_cast<unsigned>(b) << 16);
}

// 4 consecutive gradient values as float32 (exact widening for bf16)
template <bool BF16>
__device__ __forceinline__ float4 load_grad4(const void* g, long long i4) {
    if constexpr (BF16) {
        uint2 v = reinterpret_cast<const uint2*>(g)[i4];
        return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                           __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
    } else {
        return reinterpret_cast<const float4*>(g)[i4];
    }
}

template <bool BF16>
__device__ __forceinline__ float load_grad1(const void* g, long long i) {
    if constexpr (BF16) {
        return bf16_to_f32(reinterpret_cast<const unsigned short*>(g)[i]);
    } else {
        return reinterpret_cast<const float*>(g)[i];
    }
}

// fl32(m + fl32(eta*g)), two roundings (the library is built with -ffp-contract=off too)
__device__ __forceinline__ float ef_acc(float m, float eta, float g) {
    return __fadd_rn(m, __fmul_rn(eta, g));
}

__device__ __forceinline__ unsigned long long lanemask_lt() {
    const unsigned lane = __lane_id();
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

// Inclusive prefix sum over a 256-thread block in thread order.  `tmp` is a
// __shared__ array of at least 4 entries; contains a barrier.
__device__ __forceinline__ unsigned block_inclusive_scan_256(unsigned v, unsigned* tmp, unsigned* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        unsigned t = __shfl_up(v, o, WAVE);
        if (lane >= o) v += t;
    }
    if (lane == 63) tmp[w] = v;
    __syncthreads();
    unsigned before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        unsigned t = tmp[i];
        before += (i < w) ? t : 0u;
        all += t;
    }
    __syncthreads();
    *total = all;
    return v + before;
}

// Release this thread's prior global writes/atomics at device scope.
__device__ __forceinline__ void fence_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void fence_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

__device__ __forceinline__ unsigned atomic_load_u32(const unsigned* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// True in every thread of the block that finished last among gridDim.x blocks.
// All global writes made by the block before the call are visible to the last
// block after it returns true.  Contains barriers; call from all threads.
__device__ __forceinline__ bool last_block_done(unsigned* ticket) {
    __shared__ unsigned s_last;
    fence_release();
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned t = atomicAdd(ticket, 1u);
        s_last = (t == gridDim.x - 1) ? 1u : 0u;
    }
    __syncthreads();
    const bool last = s_last != 0;
    if (last) fence_acquire();
    return last;
}

}  // namespace gc
