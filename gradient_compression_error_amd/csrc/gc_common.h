// Internal helpers shared by the gfx950 kernels and the C-ABI host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "gc.h"

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

// Per-layer norms (norm.hip): argument checks, the number of float64 tile
// partials, and the two launches with the partials in `partial`.
int check_norm_args(const char* fn, const gc_span* layers, int nlayers, int grad_dtype, const float* norms);
size_t partial_count(const gc_span* layers, int nlayers);
int launch_norms(const gc_span* layers, int nlayers, int grad_dtype, float* norms, double* partial, hipStream_t s);

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

// Streaming accesses: data touched once per kernel and not again before far
// more than the caches hold has gone by (non-temporal hint on the access).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void store_stream(float4* p, float4 v) {
    __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ float4 load_stream(const float4* p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

// load_grad4 with the streaming hint
template <bool BF16>
__device__ __forceinline__ float4 load_grad4_stream(const void* g, long long i4) {
    if constexpr (BF16) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(g) + i4);
        return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                           __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
    } else {
        return load_stream(reinterpret_cast<const float4*>(g) + i4);
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

// Cross-lane moves through DPP (no LDS round trip).  All 64 lanes must be active.
template <int CTRL>
__device__ __forceinline__ unsigned dpp_u32(unsigned v) {
    return static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_MIRROR = 0x140;
constexpr int DPP_ROR4 = 0x124;        // row_ror:4 (rotate within a 16-lane row)
constexpr int DPP_ROR8 = 0x128;        // row_ror:8

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) { return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v))); }

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const unsigned long long b = __double_as_longlong(v);
    const unsigned lo = dpp_u32<CTRL>(static_cast<unsigned>(b));
    const unsigned hi = dpp_u32<CTRL>(static_cast<unsigned>(b >> 32));
    return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}

template <int CTRL>
__device__ __forceinline__ unsigned dpp_any(unsigned v) { return dpp_u32<CTRL>(v); }
template <int CTRL>
__device__ __forceinline__ float dpp_any(float v) { return dpp_f32<CTRL>(v); }
template <int CTRL>
__device__ __forceinline__ double dpp_any(double v) { return dpp_f64<CTRL>(v); }

__device__ __forceinline__ unsigned readlane_any(unsigned v, int l) {
    return static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(v), l));
}
__device__ __forceinline__ float readlane_any(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double readlane_any(double v, int l) {
    const unsigned long long b = __double_as_longlong(v);
    const unsigned lo = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<unsigned>(b)), l));
    const unsigned hi = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<unsigned>(b >> 32)), l));
    return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}

// Sum over the 64 lanes of a wave, returned (bit-identical) in every lane.
// Rows of 16 lanes are reduced with DPP, the four row sums combined in a
// fixed order.  All lanes must be active.
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
    v += dpp_any<DPP_XOR1>(v);
    v += dpp_any<DPP_XOR2>(v);
    v += dpp_any<DPP_HALF_MIRROR>(v);
    v += dpp_any<DPP_MIRROR>(v);
    return (readlane_any(v, 0) + readlane_any(v, 16)) + (readlane_any(v, 32) + readlane_any(v, 48));
}

// Inclusive prefix sum over a block of NW waves in thread order; `tmp` is a
// __shared__ array of at least NW entries.  Contains barriers; call from all
// threads of the block.
template <int NW>
__device__ __forceinline__ unsigned block_inclusive_scan(unsigned v, unsigned* tmp, unsigned* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const unsigned t = __shfl_up(v, o, WAVE);
        if (lane >= o) v += t;
    }
    if (lane == 63) tmp[w] = v;
    __syncthreads();
    unsigned before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const unsigned t = tmp[i];
        before += (i < w) ? t : 0u;
        all += t;
    }
    __syncthreads();
    *total = all;
    return v + before;
}

__device__ __forceinline__ unsigned block_inclusive_scan_256(unsigned v, unsigned* tmp, unsigned* total) {
    return block_inclusive_scan<4>(v, tmp, total);
}

// Index of the segment containing block `blk`: the last i < count with
// begin[i] <= blk (begin ascending, begin[0] = 0).  Binary search on a
// kernel-argument array (uniform scalar loads).
template <int N>
__device__ __forceinline__ int find_segment(const int (&begin)[N], int count, int blk) {
    int lo = 0, hi = count;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (begin[mid] <= blk) lo = mid;
        else hi = mid;
    }
    return lo;
}

}  // namespace gc
