// Per-layer gradient norms and Accordion's level switch.
//
// Accordion (method section) watches how fast the norm of each layer's
// gradient changes and picks the low-compression level l_low inside a
// critical regime, the high-compression level l_high outside it.
//
//   norm_partial  one pass over all layers at once: each workgroup squares and
//                 sums (float64) one 16384-entry tile of one layer
//   norm_final    one workgroup per layer sums its tile partials in a fixed
//                 order and writes sqrt(sum) as float32
// gc_grad_norm takes the tile partials in the caller's workspace.
// gc_accordion_select is plain host code: the decision needs the norms of
// the previous check, which the caller keeps.
#include <cmath>

#include "gc_common.h"

namespace gc {
namespace {

constexpr int NM_THREADS = 256;
constexpr int NM_UNROLL = 16;
constexpr int NM_TILE = NM_THREADS * 4 * NM_UNROLL;   // 16384
constexpr int NM_MAXL = 160;

// Layer table of one launch; begin[l] = first workgroup of layer l.
struct NmBatch {
    int count;
    int pad;
    double* partial;
    float* norms;
    int begin[NM_MAXL];
    int ntiles[NM_MAXL];
    const void* ptr[NM_MAXL];
    long long len[NM_MAXL];
};
static_assert(sizeof(NmBatch) <= 4096, "kernel argument table must fit 4 KB");

__device__ __forceinline__ double sq4(float4 v) {
    return (static_cast<double>(v.x) * v.x + static_cast<double>(v.y) * v.y) +
           (static_cast<double>(v.z) * v.z + static_cast<double>(v.w) * v.w);
}

template <bool BF16>
__global__ __launch_bounds__(NM_THREADS) void norm_partial(const NmBatch B) {
    __shared__ double s_w[4];
    const int blk = blockIdx.x;
    const int l = find_segment(B.begin, B.count, blk);
    const void* ptr = B.ptr[l];
    const long long len = B.len[l];
    const long long base = static_cast<long long>(blk - B.begin[l]) * NM_TILE;
    double acc = 0.0;
    if (base + NM_TILE <= len) {
        float4 v[NM_UNROLL];
#pragma unroll
        for (int u = 0; u < NM_UNROLL; ++u) v[u] = load_grad4<BF16>(ptr, base / 4 + u * NM_THREADS + threadIdx.x);
#pragma unroll
        for (int u = 0; u < NM_UNROLL; ++u) acc += sq4(v[u]);
    } else {
#pragma unroll 4
        for (long long i = base + threadIdx.x; i < len; i += NM_THREADS) {
            const double x = load_grad1<BF16>(ptr, i);
            acc += x * x;
        }
    }
    acc = wave_sum(acc);
    if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) B.partial[blk] = ((s_w[0] + s_w[1]) + s_w[2]) + s_w[3];
}

__global__ __launch_bounds__(NM_THREADS) void norm_final(const NmBatch B) {
    __shared__ double s_w[4];
    const int l = blockIdx.x;
    double acc = 0.0;
    for (int t = threadIdx.x; t < B.ntiles[l]; t += NM_THREADS) acc += B.partial[B.begin[l] + t];
    acc = wave_sum(acc);
    if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) B.norms[blockIdx.x] = static_cast<float>(sqrt(((s_w[0] + s_w[1]) + s_w[2]) + s_w[3]));
}

}  // namespace

// Tile partials (float64) the norm pass writes for these layers.
size_t partial_count(const gc_span* layers, int nlayers) {
    size_t n = 0;
    for (int i = 0; i < nlayers; ++i) n += static_cast<size_t>((layers[i].len + NM_TILE - 1) / NM_TILE);
    return n;
}

// Argument checks of the norm entry points (fn names the caller).
int check_norm_args(const char* fn, const gc_span* layers, int nlayers, int grad_dtype, const float* norms) {
    const std::string f(fn);
    if (!layers || nlayers < 1 || !norms) return fail(GC_ERR_ARG, f + ": null pointer or nlayers < 1");
    if (grad_dtype != GC_F32 && grad_dtype != GC_BF16)
        return fail(GC_ERR_DTYPE, f + ": grad_dtype must be GC_F32 or GC_BF16");
    if (!aligned16(norms)) return fail(GC_ERR_ARG, f + ": device pointers must be 16-byte aligned");
    for (int i = 0; i < nlayers; ++i) {
        if (!layers[i].ptr || layers[i].len < 1)
            return fail(GC_ERR_ARG, f + ": layer " + std::to_string(i) + " has a null pointer or len < 1");
        if (!aligned16(layers[i].ptr))
            return fail(GC_ERR_ARG, f + ": layer " + std::to_string(i) + " is not 16-byte aligned");
    }
    return GC_OK;
}

// The two norm launches over every layer, the tile partials in `partial`
// (partial_count doubles).
int launch_norms(const gc_span* layers, int nlayers, int grad_dtype, float* norms, double* partial, hipStream_t s) {
    for (int l0 = 0; l0 < nlayers; l0 += NM_MAXL) {
        NmBatch B{};
        B.partial = partial;
        B.norms = norms + l0;
        int blocks = 0;
        for (int l = l0; l < nlayers && B.count < NM_MAXL; ++l) {
            const int i = B.count++;
            B.ptr[i] = layers[l].ptr;
            B.len[i] = layers[l].len;
            B.begin[i] = blocks;
            B.ntiles[i] = static_cast<int>((layers[l].len + NM_TILE - 1) / NM_TILE);
            blocks += B.ntiles[i];
        }
        int rc;
        {
            TimedLaunch tl("norm_partial", s);
            if (grad_dtype == GC_BF16) norm_partial<true><<<blocks, NM_THREADS, 0, s>>>(B);
            else norm_partial<false><<<blocks, NM_THREADS, 0, s>>>(B);
            if ((rc = check_launch("norm_partial")) != GC_OK) return rc;
        }
        {
            TimedLaunch tl("norm_final", s);
            norm_final<<<B.count, NM_THREADS, 0, s>>>(B);
            if ((rc = check_launch("norm_final")) != GC_OK) return rc;
        }
        partial += blocks;
    }
    return GC_OK;
}

}  // namespace gc

using namespace gc;

extern "C" {

size_t gc_grad_norm_workspace_bytes(const gc_span* layers, int nlayers) {
    if (!layers || nlayers < 1) return 0;
    for (int i = 0; i < nlayers; ++i)
        if (layers[i].len < 1) return 0;
    return round_up(partial_count(layers, nlayers) * sizeof(double), 256);
}

int gc_grad_norm(const gc_span* layers, int nlayers, int grad_dtype, float* norms,
                 void* ws, size_t ws_bytes, void* stream) {
    int rc = check_norm_args("gc_grad_norm", layers, nlayers, grad_dtype, norms);
    if (rc != GC_OK) return rc;
    if (!ws) return fail(GC_ERR_ARG, "gc_grad_norm: null workspace");
    if (!aligned16(ws)) return fail(GC_ERR_ARG, "gc_grad_norm: device pointers must be 16-byte aligned");
    if (ws_bytes < gc_grad_norm_workspace_bytes(layers, nlayers))
        return fail(GC_ERR_WORKSPACE, "gc_grad_norm: workspace smaller than gc_grad_norm_workspace_bytes");
    return launch_norms(layers, nlayers, grad_dtype, norms, static_cast<double*>(ws), static_cast<hipStream_t>(stream));
}

int gc_accordion_select(const float* norm_now, float* norm_prev, int nlayers, float threshold,
                        int has_prev, int* level) {
    if (!norm_now || !norm_prev || !level || nlayers < 1)
        return fail(GC_ERR_ARG, "gc_accordion_select: null pointer or nlayers < 1");
    if (!(threshold >= 0.0f)) return fail(GC_ERR_ARG, "gc_accordion_select: threshold must be >= 0");
    const double thr = threshold;
    for (int l = 0; l < nlayers; ++l) {
        int lv = GC_LEVEL_LOW;
        if (has_prev) {
            const double prev = norm_prev[l], now = norm_now[l];
            double rho;
            if (prev == 0.0) rho = now > 0.0 ? INFINITY : 0.0;
            else rho = std::fabs(prev - now) / prev;
            lv = rho >= thr ? GC_LEVEL_LOW : GC_LEVEL_HIGH;
        }
        level[l] = lv;
        norm_prev[l] = norm_now[l];
    }
    return GC_OK;
}

}  // extern "C"
