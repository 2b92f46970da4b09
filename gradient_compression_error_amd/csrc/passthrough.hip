// Tensors sent without compression: out = fl32(eta * grad), memory untouched.
//
// A gradient set mixes matrices, which the low-rank compressor takes, with
// small vectors (batch-norm scales and shifts, biases) that are sent as they
// are (the Accordion paper's method section applies the compressor to the
// weight matrices of ResNet-18 and VGG-19; the vectors carry no low-rank
// structure).  The step of such a tensor is the plain scaled gradient, with
// no error-feedback memory since nothing is dropped.
//
//   passthrough   one launch over every vector of the call: workgroup b takes
//                 one 4096-entry tile of one vector (float4 loads and stores,
//                 a scalar tail), out = eta * grad rounded once to float32
#include <algorithm>
#include <vector>

#include "gc_common.h"

namespace gc {
namespace {

constexpr int PT_THREADS = 256;
constexpr int PT_TILE = PT_THREADS * 4 * 4;   // 4096 entries per workgroup
constexpr int PT_MAXV = 120;                  // vectors per launch (kernel-argument table)

struct PtBatch {
    int count;
    int pad;
    int begin[PT_MAXV];             // first workgroup of vector v
    const void* grad[PT_MAXV];
    float* out[PT_MAXV];
    long long len[PT_MAXV];
};
static_assert(sizeof(PtBatch) <= 4096, "kernel argument table must fit 4 KB");

template <bool BF16>
__global__ __launch_bounds__(PT_THREADS) void passthrough(const PtBatch B, float eta) {
    const int blk = blockIdx.x;
    const int v = find_segment(B.begin, B.count, blk);
    const void* g = B.grad[v];
    float* out = B.out[v];
    const long long len = B.len[v];
    const long long base = static_cast<long long>(blk - B.begin[v]) * PT_TILE;
    if (base + PT_TILE <= len) {
        float4 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x[u] = load_grad4<BF16>(g, base / 4 + u * PT_THREADS + threadIdx.x);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            reinterpret_cast<float4*>(out)[base / 4 + u * PT_THREADS + threadIdx.x] =
                make_float4(__fmul_rn(eta, x[u].x), __fmul_rn(eta, x[u].y), __fmul_rn(eta, x[u].z),
                            __fmul_rn(eta, x[u].w));
    } else {
        const long long end = std::min(len, base + PT_TILE);
        for (long long i = base + threadIdx.x; i < end; i += PT_THREADS) out[i] = __fmul_rn(eta, load_grad1<BF16>(g, i));
    }
}

// True when an output range overlaps any other range (inputs may overlap
// each other: they are only read).
bool outputs_overlap(const gc_vec* vecs, int n, size_t gsize) {
    struct Iv {
        uintptr_t a, b;
        bool out;
    };
    std::vector<Iv> iv;
    iv.reserve(2 * static_cast<size_t>(n));
    for (int i = 0; i < n; ++i) {
        const uintptr_t g = reinterpret_cast<uintptr_t>(vecs[i].grad), o = reinterpret_cast<uintptr_t>(vecs[i].out);
        const size_t len = static_cast<size_t>(vecs[i].len);
        iv.push_back({g, g + len * gsize, false});
        iv.push_back({o, o + len * 4, true});
    }
    std::sort(iv.begin(), iv.end(), [](const Iv& x, const Iv& y) { return x.a < y.a; });
    uintptr_t end_all = 0, end_out = 0;
    for (const Iv& x : iv) {
        if (x.out ? x.a < end_all : x.a < end_out) return true;
        end_all = std::max(end_all, x.b);
        if (x.out) end_out = std::max(end_out, x.b);
    }
    return false;
}

}  // namespace
}  // namespace gc

using namespace gc;

extern "C" {

int gc_passthrough(const gc_vec* vecs, int nvecs, int grad_dtype, float eta, void* stream) {
    if (!vecs || nvecs < 1) return fail(GC_ERR_ARG, "gc_passthrough: need vecs and nvecs >= 1");
    if (grad_dtype != GC_F32 && grad_dtype != GC_BF16)
        return fail(GC_ERR_DTYPE, "gc_passthrough: grad_dtype must be GC_F32 or GC_BF16");
    for (int i = 0; i < nvecs; ++i) {
        const gc_vec& v = vecs[i];
        const std::string pre = "gc_passthrough: vecs[" + std::to_string(i) + "]: ";
        if (!v.grad || !v.out) return fail(GC_ERR_ARG, pre + "null grad or out");
        if (v.len < 1 || v.len > INT32_MAX) return fail(GC_ERR_ARG, pre + "len must be in [1, INT32_MAX]");
        if (!aligned16(v.grad) || !aligned16(v.out))
            return fail(GC_ERR_ARG, pre + "device pointers must be 16-byte aligned");
    }
    if (outputs_overlap(vecs, nvecs, grad_dtype == GC_BF16 ? 2 : 4))
        return fail(GC_ERR_ARG, "gc_passthrough: an output overlaps a gradient or another output");
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int v0 = 0; v0 < nvecs; v0 += PT_MAXV) {
        PtBatch B{};
        long long blocks = 0;
        for (int v = v0; v < nvecs && B.count < PT_MAXV; ++v) {
            const int i = B.count++;
            B.grad[i] = vecs[v].grad;
            B.out[i] = vecs[v].out;
            B.len[i] = vecs[v].len;
            B.begin[i] = static_cast<int>(blocks);
            blocks += (vecs[v].len + PT_TILE - 1) / PT_TILE;
        }
        TimedLaunch tl("passthrough", s);
        if (grad_dtype == GC_BF16) passthrough<true><<<static_cast<unsigned>(blocks), PT_THREADS, 0, s>>>(B, eta);
        else passthrough<false><<<static_cast<unsigned>(blocks), PT_THREADS, 0, s>>>(B, eta);
        const int rc = check_launch("passthrough");
        if (rc != GC_OK) return rc;
    }
    return GC_OK;
}

}  // extern "C"
