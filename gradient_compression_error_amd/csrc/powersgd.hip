// PowerSGD rank-r (r <= 4) compression with error-feedback memory on gfx950.
//
// Per matrix (M = mem + eta*grad, n x m row-major; Q m x r, P n x r column-major):
//     P = M Q;  P^ = Gram-Schmidt(P);  Q' = M^T P^;  out = P^ Q'^T;  mem = M - out
// The pages name PowerSGD and its ranks (Accordion paper, method and results
// sections; utility-of-compression paper, results section); the steps are the
// plain power-iteration step with the memory convention of Mem-SGD.
//
// Orthonormalisation is done in coefficient space: with G = P^T P (float64)
// the Gram-Schmidt recurrence gives an upper-triangular T with P^ = P T, and
// Q' = M^T P^ = (M^T P) T.  So the second pass over M does not wait for the
// orthonormalisation and no n x r vector pass is needed:
//
//   psgd_p       P = M Q_in per row (waves own rows, lanes stride columns),
//                plus per-workgroup partial Gram matrices (float64)
//   psgd_q       partial (M^T P) per (column strip, row chunk) workgroup
//   psgd_qreduce sums the partials in a fixed order, builds T from the summed
//                Gram matrix, writes Q' = (M^T P) T into q (warm start)
//   psgd_out     P^ = P T per row, out = P^ Q'^T, mem = M - out, P^ into p
//
// M is never stored: each pass recomputes it from (mem, grad).  Matrices are
// processed in batches whose gradient+memory bytes fit the 256 MB Infinity
// Cache, so the second and third reads of a batch can hit it.  Every reduction
// has a fixed order: the result bits do not depend on scheduling.
#include "gc_common.h"

namespace gc {
namespace {

constexpr int PS_THREADS = 256;
constexpr int PS_MAXB = 32;          // matrices per launch (kernel-argument table)
constexpr int P_ROWS_WAVE = 4;       // rows per wave in psgd_p
constexpr int P_ROWS_WG = 16;        // rows per workgroup in psgd_p
constexpr int Q_ROWS = 32;           // rows per chunk in psgd_q
constexpr int O_ROWS = 32;           // rows per workgroup in psgd_out
constexpr size_t PS_GROUP_BYTES = size_t(128) << 20;

struct PsMat {
    const void* grad;
    float* mem;
    float* q;
    float* p;
    float* out;
    float* praw;     // [n][4]  P = M Q
    double* gpart;   // [ceil(n/16)][16] partial Gram matrices
    float* qpart;    // [ceil(n/32)][m][4] partial M^T P
    double* tmat;    // [16] T, row-major 4x4
    int n, m, rank;
    int wg_p, wg_q, wg_r, wg_o;
};

struct PsBatch {
    int count;
    float eta;
    int pad[2];
    PsMat mat[PS_MAXB];
};
static_assert(sizeof(PsBatch) <= 4096, "kernel argument table must fit 4 KB");

__device__ __forceinline__ int nstrips_of(int m) {
    const int w = (m % 4 == 0) ? PS_THREADS * 4 : PS_THREADS;
    return (m + w - 1) / w;
}

template <int WHICH>
__device__ __forceinline__ int first_block(const PsMat& M) {
    return WHICH == 0 ? M.wg_p : WHICH == 1 ? M.wg_q : WHICH == 2 ? M.wg_r : M.wg_o;
}

template <int WHICH>
__device__ __forceinline__ int find_mat(const PsBatch& B) {
    const int blk = blockIdx.x;
    int i = 0;
    while (i + 1 < B.count && first_block<WHICH>(B.mat[i + 1]) <= blk) ++i;
    return i;
}

// M values of 4 consecutive entries starting at flat element e (16-byte aligned)
template <bool BF16>
__device__ __forceinline__ float4 load_M4(const PsMat& M, float eta, long long e) {
    const float4 g = load_grad4<BF16>(M.grad, e / 4);
    const float4 mm = reinterpret_cast<const float4*>(M.mem)[e / 4];
    return make_float4(ef_acc(mm.x, eta, g.x), ef_acc(mm.y, eta, g.y), ef_acc(mm.z, eta, g.z),
                       ef_acc(mm.w, eta, g.w));
}

template <bool BF16>
__device__ __forceinline__ float load_M1(const PsMat& M, float eta, long long e) {
    return ef_acc(M.mem[e], eta, load_grad1<BF16>(M.grad, e));
}

// ------------------------------------------------------------------ psgd_p

template <bool BF16, int VEC>
__device__ __forceinline__ void p_rows(const PsMat& M, float eta, int row0, float acc[P_ROWS_WAVE][4]) {
    const int lane = threadIdx.x & 63;
    const int n = M.n, m = M.m, r = M.rank;
    const int nch = m / VEC;
    for (int c = lane; c < nch; c += 64) {
        float qv[VEC][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < r) {
                if constexpr (VEC == 4) {
                    const float4 t = reinterpret_cast<const float4*>(M.q + static_cast<long long>(j) * m)[c];
                    qv[0][j] = t.x; qv[1][j] = t.y; qv[2][j] = t.z; qv[3][j] = t.w;
                } else {
                    qv[0][j] = M.q[static_cast<long long>(j) * m + c];
                }
            } else {
#pragma unroll
                for (int v = 0; v < VEC; ++v) qv[v][j] = 0.0f;
            }
        }
#pragma unroll
        for (int rr = 0; rr < P_ROWS_WAVE; ++rr) {
            const int row = row0 + rr;
            if (row < n) {
                const long long e = static_cast<long long>(row) * m + static_cast<long long>(c) * VEC;
                float mv[VEC];
                if constexpr (VEC == 4) {
                    const float4 t = load_M4<BF16>(M, eta, e);
                    mv[0] = t.x; mv[1] = t.y; mv[2] = t.z; mv[3] = t.w;
                } else {
                    mv[0] = load_M1<BF16>(M, eta, e);
                }
#pragma unroll
                for (int v = 0; v < VEC; ++v)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[rr][j] = fmaf(mv[v], qv[v][j], acc[rr][j]);
            }
        }
    }
}

template <bool BF16>
__global__ __launch_bounds__(PS_THREADS) void psgd_p(const PsBatch B) {
    __shared__ double s_g[4][16];
    const PsMat& M = B.mat[find_mat<0>(B)];
    const int lwg = blockIdx.x - M.wg_p;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row0 = lwg * P_ROWS_WG + w * P_ROWS_WAVE;
    float acc[P_ROWS_WAVE][4];
#pragma unroll
    for (int rr = 0; rr < P_ROWS_WAVE; ++rr)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[rr][j] = 0.0f;
    if (M.m % 4 == 0)
        p_rows<BF16, 4>(M, B.eta, row0, acc);
    else
        p_rows<BF16, 1>(M, B.eta, row0, acc);
#pragma unroll
    for (int rr = 0; rr < P_ROWS_WAVE; ++rr)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[rr][j] = wave_sum(acc[rr][j]);
    // every lane now holds the 4 finished rows of this wave
    double g[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) g[i] = 0.0;
#pragma unroll
    for (int rr = 0; rr < P_ROWS_WAVE; ++rr) {
        const int row = row0 + rr;
        if (row < M.n) {
            if (lane == rr)
                reinterpret_cast<float4*>(M.praw)[row] = make_float4(acc[rr][0], acc[rr][1], acc[rr][2], acc[rr][3]);
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    g[a * 4 + b] += static_cast<double>(acc[rr][a]) * static_cast<double>(acc[rr][b]);
        }
    }
    if (lane < 16) {
        double v = 0.0;
#pragma unroll
        for (int i = 0; i < 16; ++i) v = (lane == i) ? g[i] : v;
        s_g[w][lane] = v;
    }
    __syncthreads();
    if (threadIdx.x < 16) {
        const int i = threadIdx.x;
        M.gpart[static_cast<long long>(lwg) * 16 + i] = ((s_g[0][i] + s_g[1][i]) + s_g[2][i]) + s_g[3][i];
    }
}

// ------------------------------------------------------------------ psgd_q

template <bool BF16, int VEC>
__device__ __forceinline__ void q_chunk(const PsMat& M, float eta, int strip, int chunk) {
    const int n = M.n, m = M.m;
    const int col0 = strip * (PS_THREADS * VEC) + threadIdx.x * VEC;
    if (col0 >= m) return;
    const int r0 = chunk * Q_ROWS;
    const int r1 = min(n, r0 + Q_ROWS);
    float acc[VEC][4];
#pragma unroll
    for (int v = 0; v < VEC; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[v][j] = 0.0f;
    const float4* praw4 = reinterpret_cast<const float4*>(M.praw);
    for (int i = r0; i < r1; ++i) {
        const float4 p = praw4[i];
        const long long e = static_cast<long long>(i) * m + col0;
        float mv[VEC];
        if constexpr (VEC == 4) {
            const float4 t = load_M4<BF16>(M, eta, e);
            mv[0] = t.x; mv[1] = t.y; mv[2] = t.z; mv[3] = t.w;
        } else {
            mv[0] = load_M1<BF16>(M, eta, e);
        }
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            acc[v][0] = fmaf(mv[v], p.x, acc[v][0]);
            acc[v][1] = fmaf(mv[v], p.y, acc[v][1]);
            acc[v][2] = fmaf(mv[v], p.z, acc[v][2]);
            acc[v][3] = fmaf(mv[v], p.w, acc[v][3]);
        }
    }
    float4* dst = reinterpret_cast<float4*>(M.qpart) + static_cast<long long>(chunk) * m + col0;
#pragma unroll
    for (int v = 0; v < VEC; ++v) dst[v] = make_float4(acc[v][0], acc[v][1], acc[v][2], acc[v][3]);
}

template <bool BF16>
__global__ __launch_bounds__(PS_THREADS) void psgd_q(const PsBatch B) {
    const PsMat& M = B.mat[find_mat<1>(B)];
    const int lwg = blockIdx.x - M.wg_q;
    const int ns = nstrips_of(M.m);
    const int strip = lwg % ns, chunk = lwg / ns;
    if (M.m % 4 == 0)
        q_chunk<BF16, 4>(M, B.eta, strip, chunk);
    else
        q_chunk<BF16, 1>(M, B.eta, strip, chunk);
}

// ------------------------------------------------------------------ psgd_qreduce

// Gram-Schmidt on the columns of P expressed through G = P^T P:
// column j of T holds the coefficients of P^_j in the basis of P's columns.
__device__ __forceinline__ void gram_schmidt_coeffs(const double G[16], int r, double T[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) T[i] = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (j < r) {
            double w[4] = {0.0, 0.0, 0.0, 0.0};
            w[j] = 1.0;
#pragma unroll
            for (int i = 0; i < j; ++i) {
                // dot = (P t_i) . (P w) = t_i^T G w
                double dot = 0.0;
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int b = 0; b < 4; ++b) dot += T[a * 4 + i] * G[a * 4 + b] * w[b];
#pragma unroll
                for (int a = 0; a < 4; ++a) w[a] -= dot * T[a * 4 + i];
            }
            double nrm2 = 0.0;
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) nrm2 += w[a] * G[a * 4 + b] * w[b];
            if (nrm2 > 0.0) {
                const double inv = 1.0 / sqrt(nrm2);
#pragma unroll
                for (int a = 0; a < 4; ++a) T[a * 4 + j] = w[a] * inv;
            }
        }
    }
}

__global__ __launch_bounds__(PS_THREADS) void psgd_qreduce(const PsBatch B) {
    __shared__ double s_red[PS_THREADS / 64][16];
    __shared__ double s_T[16];
    const PsMat& M = B.mat[find_mat<2>(B)];
    const int lwg = blockIdx.x - M.wg_r;
    const int n = M.n, m = M.m, r = M.rank;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    // Gram matrix: fixed-order sum of the psgd_p partials
    const int ngp = (n + P_ROWS_WG - 1) / P_ROWS_WG;
    double g[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) g[i] = 0.0;
    for (int b = threadIdx.x; b < ngp; b += PS_THREADS) {
        const double* src = M.gpart + static_cast<long long>(b) * 16;
#pragma unroll
        for (int i = 0; i < 16; ++i) g[i] += src[i];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) g[i] = wave_sum(g[i]);
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s_red[w][i] = g[i];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double G[16], T[16];
        for (int i = 0; i < 16; ++i) G[i] = ((s_red[0][i] + s_red[1][i]) + s_red[2][i]) + s_red[3][i];
        gram_schmidt_coeffs(G, r, T);
        for (int i = 0; i < 16; ++i) s_T[i] = T[i];
        if (lwg == 0)
            for (int i = 0; i < 16; ++i) M.tmat[i] = T[i];
    }
    __syncthreads();
    const int col = lwg * PS_THREADS + threadIdx.x;
    if (col >= m) return;
    const int nch = (n + Q_ROWS - 1) / Q_ROWS;
    double s[4] = {0.0, 0.0, 0.0, 0.0};
    const float4* qp = reinterpret_cast<const float4*>(M.qpart) + col;
    for (int c = 0; c < nch; ++c) {
        const float4 t = qp[static_cast<long long>(c) * m];
        s[0] += t.x; s[1] += t.y; s[2] += t.z; s[3] += t.w;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (j < r) {
            double v = 0.0;
#pragma unroll
            for (int a = 0; a <= j; ++a) v += s[a] * s_T[a * 4 + j];
            M.q[static_cast<long long>(j) * m + col] = static_cast<float>(v);
        }
    }
}

// ------------------------------------------------------------------ psgd_out

template <bool BF16, int VEC>
__device__ __forceinline__ void out_rows(const PsMat& M, float eta, int strip, int chunk) {
    const int n = M.n, m = M.m, r = M.rank;
    const int col0 = strip * (PS_THREADS * VEC) + threadIdx.x * VEC;
    const bool active = col0 < m;
    float T[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) T[i] = static_cast<float>(M.tmat[i]);
    float qv[VEC][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) qv[v][j] = 0.0f;
        if (active && j < r) {
            if constexpr (VEC == 4) {
                const float4 t = reinterpret_cast<const float4*>(M.q + static_cast<long long>(j) * m + col0)[0];
                qv[0][j] = t.x; qv[1][j] = t.y; qv[2][j] = t.z; qv[3][j] = t.w;
            } else {
                qv[0][j] = M.q[static_cast<long long>(j) * m + col0];
            }
        }
    }
    const int r0 = chunk * O_ROWS;
    const int r1 = min(n, r0 + O_ROWS);
    const float4* praw4 = reinterpret_cast<const float4*>(M.praw);
    const bool write_p = M.p != nullptr && strip == 0 && threadIdx.x < static_cast<unsigned>(r);
    for (int i = r0; i < r1; ++i) {
        const float4 pr = praw4[i];
        const float prv[4] = {pr.x, pr.y, pr.z, pr.w};
        float ph[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float v = 0.0f;
#pragma unroll
            for (int a = 0; a <= j; ++a) v = fmaf(prv[a], T[a * 4 + j], v);
            ph[j] = v;
        }
        if (write_p) {
            float mine = ph[0];
#pragma unroll
            for (int j = 1; j < 4; ++j) mine = (threadIdx.x == static_cast<unsigned>(j)) ? ph[j] : mine;
            M.p[static_cast<long long>(threadIdx.x) * n + i] = mine;
        }
        if (!active) continue;
        const long long e = static_cast<long long>(i) * m + col0;
        if constexpr (VEC == 4) {
            const float4 mv = load_M4<BF16>(M, eta, e);
            const float mva[4] = {mv.x, mv.y, mv.z, mv.w};
            float o[4], nm[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float s = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) s = fmaf(ph[j], qv[v][j], s);
                o[v] = s;
                nm[v] = mva[v] - s;
            }
            if (M.out) reinterpret_cast<float4*>(M.out)[e / 4] = make_float4(o[0], o[1], o[2], o[3]);
            reinterpret_cast<float4*>(M.mem)[e / 4] = make_float4(nm[0], nm[1], nm[2], nm[3]);
        } else {
            const float mv = load_M1<BF16>(M, eta, e);
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) s = fmaf(ph[j], qv[0][j], s);
            if (M.out) M.out[e] = s;
            M.mem[e] = mv - s;
        }
    }
}

template <bool BF16>
__global__ __launch_bounds__(PS_THREADS) void psgd_out(const PsBatch B) {
    const PsMat& M = B.mat[find_mat<3>(B)];
    const int lwg = blockIdx.x - M.wg_o;
    const int ns = nstrips_of(M.m);
    const int strip = lwg % ns, chunk = lwg / ns;
    if (M.m % 4 == 0)
        out_rows<BF16, 4>(M, B.eta, strip, chunk);
    else
        out_rows<BF16, 1>(M, B.eta, strip, chunk);
}

// ------------------------------------------------------------------ host side

int nstrips_host(int m) {
    const int w = (m % 4 == 0) ? PS_THREADS * 4 : PS_THREADS;
    return (m + w - 1) / w;
}

struct MatWs {
    size_t praw, gpart, qpart, tmat, bytes;
};

MatWs mat_ws(int n, int m) {
    MatWs W{};
    size_t o = 0;
    W.praw = o;  o += round_up(static_cast<size_t>(n) * 16, 256);
    W.gpart = o; o += round_up(static_cast<size_t>((n + P_ROWS_WG - 1) / P_ROWS_WG) * 16 * 8, 256);
    W.qpart = o; o += round_up(static_cast<size_t>((n + Q_ROWS - 1) / Q_ROWS) * m * 16, 256);
    W.tmat = o;  o += 256;
    W.bytes = o;
    return W;
}

int validate_mat(const gc_mat& a, int i, int dtype) {
    const std::string pre = "gc_powersgd_ef_step: mats[" + std::to_string(i) + "]: ";
    if (!a.grad || !a.mem || !a.q) return fail(GC_ERR_ARG, pre + "null grad/mem/q");
    if (a.n < 1 || a.m < 1) return fail(GC_ERR_ARG, pre + "n and m must be >= 1");
    if (static_cast<long long>(a.n) * a.m > INT32_MAX) return fail(GC_ERR_ARG, pre + "n*m exceeds INT32_MAX");
    if (a.rank < 1 || a.rank > 4 || a.rank > a.n || a.rank > a.m)
        return fail(GC_ERR_ARG, pre + "rank must be in [1, min(4, n, m)]");
    if (!aligned16(a.grad) || !aligned16(a.mem) || !aligned16(a.q) || (a.p && !aligned16(a.p)) ||
        (a.out && !aligned16(a.out)))
        return fail(GC_ERR_ARG, pre + "device pointers must be 16-byte aligned");
    const size_t nm = static_cast<size_t>(a.n) * a.m;
    const size_t gb = nm * (dtype == GC_BF16 ? 2 : 4), mb = nm * 4;
    const size_t qb = static_cast<size_t>(a.m) * a.rank * 4, pb = static_cast<size_t>(a.n) * a.rank * 4;
    bool bad = overlaps(a.grad, gb, a.mem, mb) || overlaps(a.q, qb, a.mem, mb) || overlaps(a.q, qb, a.grad, gb);
    if (a.p) bad = bad || overlaps(a.p, pb, a.mem, mb) || overlaps(a.p, pb, a.q, qb) || overlaps(a.p, pb, a.grad, gb);
    if (a.out)
        bad = bad || overlaps(a.out, mb, a.mem, mb) || overlaps(a.out, mb, a.q, qb) || overlaps(a.out, mb, a.grad, gb) ||
              (a.p && overlaps(a.out, mb, a.p, pb));
    if (bad) return fail(GC_ERR_ARG, pre + "buffers overlap");
    return GC_OK;
}

}  // namespace
}  // namespace gc

using namespace gc;

extern "C" {

size_t gc_powersgd_workspace_bytes(const gc_mat* mats, int nmats) {
    if (!mats || nmats < 1) return 0;
    size_t total = 0;
    for (int i = 0; i < nmats; ++i) {
        const gc_mat& a = mats[i];
        if (a.n < 1 || a.m < 1 || static_cast<long long>(a.n) * a.m > INT32_MAX) return 0;
        total += mat_ws(a.n, a.m).bytes;
    }
    return total;
}

int gc_powersgd_ef_step(const gc_mat* mats, int nmats, int grad_dtype, float eta,
                        void* ws, size_t ws_bytes, void* stream) {
    if (!mats || nmats < 1) return fail(GC_ERR_ARG, "gc_powersgd_ef_step: need mats and nmats >= 1");
    if (grad_dtype != GC_F32 && grad_dtype != GC_BF16)
        return fail(GC_ERR_DTYPE, "gc_powersgd_ef_step: grad_dtype must be GC_F32 or GC_BF16");
    if (!ws) return fail(GC_ERR_ARG, "gc_powersgd_ef_step: null workspace");
    if (!aligned16(ws)) return fail(GC_ERR_ARG, "gc_powersgd_ef_step: workspace must be 16-byte aligned");
    for (int i = 0; i < nmats; ++i) {
        const int rc = validate_mat(mats[i], i, grad_dtype);
        if (rc != GC_OK) return rc;
    }
    const size_t need = gc_powersgd_workspace_bytes(mats, nmats);
    if (ws_bytes < need)
        return fail(GC_ERR_WORKSPACE, "gc_powersgd_ef_step: workspace smaller than gc_powersgd_workspace_bytes");

    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf16 = grad_dtype == GC_BF16;
    const size_t elem_bytes = bf16 ? 6 : 8;   // grad + memory per entry
    char* wp = static_cast<char*>(ws);
    int i = 0;
    while (i < nmats) {
        PsBatch B{};
        B.eta = eta;
        int np = 0, nq = 0, nr = 0, no = 0;
        size_t group = 0;
        while (i < nmats && B.count < PS_MAXB) {
            const gc_mat& a = mats[i];
            const size_t bytes = static_cast<size_t>(a.n) * a.m * elem_bytes;
            if (B.count > 0 && group + bytes > PS_GROUP_BYTES) break;
            group += bytes;
            const MatWs W = mat_ws(a.n, a.m);
            PsMat& M = B.mat[B.count++];
            M.grad = a.grad;
            M.mem = a.mem;
            M.q = a.q;
            M.p = a.p;
            M.out = a.out;
            M.praw = reinterpret_cast<float*>(wp + W.praw);
            M.gpart = reinterpret_cast<double*>(wp + W.gpart);
            M.qpart = reinterpret_cast<float*>(wp + W.qpart);
            M.tmat = reinterpret_cast<double*>(wp + W.tmat);
            M.n = a.n;
            M.m = a.m;
            M.rank = a.rank;
            const int ns = nstrips_host(a.m);
            M.wg_p = np; np += (a.n + P_ROWS_WG - 1) / P_ROWS_WG;
            M.wg_q = nq; nq += ns * ((a.n + Q_ROWS - 1) / Q_ROWS);
            M.wg_r = nr; nr += (a.m + PS_THREADS - 1) / PS_THREADS;
            M.wg_o = no; no += ns * ((a.n + O_ROWS - 1) / O_ROWS);
            wp += W.bytes;
            ++i;
        }
        int rc;
        {
            TimedLaunch tl("psgd_p", s);
            if (bf16) psgd_p<true><<<np, PS_THREADS, 0, s>>>(B);
            else psgd_p<false><<<np, PS_THREADS, 0, s>>>(B);
            if ((rc = check_launch("psgd_p")) != GC_OK) return rc;
        }
        {
            TimedLaunch tl("psgd_q", s);
            if (bf16) psgd_q<true><<<nq, PS_THREADS, 0, s>>>(B);
            else psgd_q<false><<<nq, PS_THREADS, 0, s>>>(B);
            if ((rc = check_launch("psgd_q")) != GC_OK) return rc;
        }
        {
            TimedLaunch tl("psgd_qreduce", s);
            psgd_qreduce<<<nr, PS_THREADS, 0, s>>>(B);
            if ((rc = check_launch("psgd_qreduce")) != GC_OK) return rc;
        }
        {
            TimedLaunch tl("psgd_out", s);
            if (bf16) psgd_out<true><<<no, PS_THREADS, 0, s>>>(B);
            else psgd_out<false><<<no, PS_THREADS, 0, s>>>(B);
            if ((rc = check_launch("psgd_out")) != GC_OK) return rc;
        }
    }
    return GC_OK;
}

}  // extern "C"
