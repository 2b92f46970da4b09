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
// Q' = M^T P^ = (M^T P) T.  So the pass that forms M^T P does not wait for
// the orthonormalisation:
//
//   psgd_pq      one pass over M: a workgroup spanning a row (thread t owns
//                columns 4t..4t+3, and with two chunks per thread also
//                4(t+NT)..) takes rows in groups, finishes each row's
//                P = M Q_in with a DPP reduce-scatter plus one LDS exchange,
//                and adds M[i,:]^T P[i,:] into per-thread M^T P accumulators;
//                one M^T P partial (the rank's planes of m floats) and one
//                Gram (float64) partial per workgroup and matrix.  Five
//                classes by row length (<= 1024, 2048, 4096, 6144, 8192, m a
//                multiple of 4)
//   psgd_pq_teams the same pass for classes 0-2 of a small launch group in
//                one launch (teams of a class's row width in 1024-thread
//                workgroups), small matrices included
//   psgd_small   the same pass, one workgroup per matrix, for n, m <= 1024
//                with m not a multiple of 4
//   psgd_p/psgd_q the same two products as separate passes, for the other
//                shapes (m not a multiple of 4 and n or m > 1024, or m > 8192)
//   psgd_qreduce sums the partials in a fixed order, builds T from the summed
//                Gram matrix, writes Q' = (M^T P) T into q (warm start)
//   psgd_out     P^ = P T per row, out = P^ Q'^T, mem = M - out, P^ into p
//   psgd_decode  the deferred form's output pass: out = P^ Q'^T, P^ into p
//
// Two forms of the memory:
//   explicit     (gc_powersgd_ef_step) M is never stored: psgd_pq and psgd_out
//                each recompute it from (mem, grad), so M's inputs are read
//                twice per step.
//   deferred     (gc_powersgd_ef_step_deferred) mem keeps M, p keeps P^ and q
//                keeps Q between steps.  The next step's first pass rebuilds
//                m' = M - P^ Q^T per entry (residual1, the output pass's own
//                float32 operations), forms M = m' + eta*grad, stores it over
//                mem and runs the products on it; psgd_decode then writes out
//                and P^ only.  Every entry is read once and written once.
//                psgd_out's third mode (materialize) writes the memory out.
// Recorded steps (gc_powersgd_plan / gc_powersgd_run) copy the matrix table
// once and then only launch these kernels.
//
// psgd_pq and psgd_out use a balanced persistent partition: the grid is about
// what the GPU holds at once, and workgroup b takes the rows whose first entry
// falls in the b-th equal share of the batch's entries, so no workgroup waits
// on a second round.  psgd_decode is not persistent: short workgroups in
// address order suit a write-only pass.  Every reduction has a fixed order:
// the result bits do not depend on scheduling.
#include <algorithm>
#include <cstring>
#include <vector>

#include "gc_common.h"

namespace gc {
namespace {

constexpr int PS_THREADS = 256;
constexpr int PS_MAXB = 4096;        // matrices per launch group
constexpr int P_ROWS_WAVE = 2;       // rows per wave in psgd_p
constexpr int P_ROWS_WG = 4 * P_ROWS_WAVE;   // rows per workgroup in psgd_p
// The fused pass partitions a class by cost, not by entries: a row of m
// entries costs m + PQ_ROW_COST units, the constant standing for the per-row
// work that does not scale with the row (its share of a row group's load
// latency, the cross-wave reduction and the P and Gram updates).  On classes
// of one row length the shares are those of an even split of the entries; on
// mixed lengths short rows no longer pile up in one workgroup (ResNet-18's
// 128 x 64 layer put about 72 rows into one share, against 8 for its widest).
constexpr int PQ_ROW_COST = 1024;
// A fused-pass workgroup takes at least this many rows of the class's costliest
// row: on small classes one-row shares cost more in per-workgroup set-up and
// M^T P partials than they gain in parallelism.
constexpr int PQ_ROWS_MIN = 8;
constexpr int Q_ROWS = 32;           // rows per chunk in psgd_q
constexpr int ROW_GROUP = 8;         // rows whose loads are issued together in psgd_q / psgd_out
constexpr int QR_QUAD_BATCH = 2;     // partials whose 4-column loads psgd_qreduce issues together
constexpr int QR_PER_THREAD = 16;    // M^T P partials per psgd_qreduce thread before slicing a column
constexpr int CUS = 256;             // MI355X compute units
constexpr double STREAM_MIN_BYTES = 1e9;   // psgd_out traffic above which it streams
// largest share (entries) of one psgd_pq workgroup: (share + a row group of look-ahead) * 4 bytes < 2^31
constexpr long long PQ_SHARE_MAX_ENTRIES = (1LL << 28) - (1LL << 20);
// psgd_out grid: one resident round (about 4 workgroups fit per CU) for large
// launch groups; two rounds for groups of at most OUT_TWO_ROUNDS_MAX entries.
// On small sets of mixed row lengths the shares are even in entries but not in
// time (short rows carry more per-row work), and the second round lets the
// hardware balance them; on large uniform sets one round is slightly faster.
constexpr int OUT_GRID_MAX = CUS * 4;
constexpr long long OUT_TWO_ROUNDS_MAX = 1LL << 26;

struct PsMat {
    const void* grad;
    float* mem;
    float* q;
    float* p;
    float* out;
    float* praw;     // [n][4]  P = M Q
    double* gpart;   // [ng][16] partial Gram matrices
    float* qpart;    // [nq][4][m] partial M^T P, plane j = component j (planes < rank used)
    double* tmat;    // [16] T, row-major 4x4
    long long off;   // first entry of the matrix in the batch (matrices back to back)
    long long poff;  // fused classes: first unit of the matrix in its class's psgd_pq partition
    int n, m, rank;
    int nq, ng;      // number of M^T P / Gram partials
    int begin_p;     // split path: first workgroup of the matrix in psgd_p
    int begin_q;     // split path: first workgroup in psgd_q
    int begin_r;     // first workgroup in psgd_qreduce
    int qs;          // psgd_qreduce threads per column
    int rcost;       // fused classes: partition units per row (m + PQ_ROW_COST)
    int prank;       // deferred memory: rank of the previous step's P^, Q (0: mem holds the memory itself)
    int pad_;
    long long dbeg;  // deferred step: first psgd_decode tile of the matrix
};
static_assert(sizeof(PsMat) % 8 == 0, "table entries are copied as words");
static_assert(sizeof(PsMat) == 144, "table entry size stated in gc.h");

// Fused-pass classes by row length (m % 4 == 0): m <= 1024, 2048, 4096, 6144,
// 8192, each with its own workgroup shape.  Of the other shapes, the small
// ones (n, m <= 1024) are done whole by one workgroup each; the rest take the
// split path.
constexpr int PQ_CLASSES = 5;
constexpr int SMALL_CLASS = PQ_CLASSES;
constexpr int SPLIT_CLASS = PQ_CLASSES + 1;
constexpr int SMALL_MAX_N = 1024, SMALL_MAX_M = 1024;

// Launch parameters of one launch group; the matrices (sorted by class) are
// in a device table (in the workspace) copied there at the start of the step.
// M^T P partial `part`, component j: m floats (plane j of that partial).
// Writers and psgd_qreduce touch only the planes below the rank, so a rank-r
// step moves r/4 of the bytes of a rank-4 one.
__device__ __forceinline__ float* qplane(const PsMat& M, long long part, int j) {
    return M.qpart + (part * 4 + j) * static_cast<long long>(M.m);
}

struct PsBatch {
    const PsMat* tbl;
    const int* rmap;               // psgd_qreduce workgroup -> matrix (after the table)
    const int* dmap;               // psgd_decode: matrix of tile 64 g, for every g (after rmap)
    int count;
    float eta;
    int cbeg[PQ_CLASSES + 3];      // matrices [cbeg[c], cbeg[c+1]) are of class c (small, split last)
    int cgrid[PQ_CLASSES];         // psgd_pq grid of each fused class
    long long cbase[PQ_CLASSES];   // first partition unit of each fused class
    long long cent[PQ_CLASSES];    // partition units of each fused class
    long long eall;                // entries of all matrices
    int gout;                      // psgd_out grid
    int pad;
};
static_assert(sizeof(PsBatch) <= 4096, "kernel argument table must fit 4 KB");

// Balanced partition: workgroup b of g owns the rows whose first entry s
// satisfies floor(s * g / e) == b, i.e. s in [ceil(b e / g), ceil((b+1) e / g)).
__host__ __device__ __forceinline__ long long share_lo(long long e, int g, int b) {
    return (static_cast<long long>(b) * e + g - 1) / g;
}
__host__ __device__ __forceinline__ int owner_of(long long s, long long e, int g) {
    return static_cast<int>((s * g) / e);
}

// The table is read through the constant address space: uniform indices give
// scalar loads, and a matrix's fields are copied into scalar registers.
typedef const __attribute__((address_space(4))) PsMat* MatTable;

__device__ __forceinline__ MatTable mat_table(const PsBatch& B) { return (MatTable)(B.tbl); }

__device__ __forceinline__ PsMat mat_at(const PsBatch& B, int i) {
    typedef const __attribute__((address_space(4))) unsigned long long* WordTable;
    const WordTable w = (WordTable)(B.tbl + i);
    PsMat r;
    unsigned long long* d = reinterpret_cast<unsigned long long*>(&r);
#pragma unroll
    for (int k = 0; k < static_cast<int>(sizeof(PsMat) / 8); ++k) d[k] = w[k];
    return r;
}

// Last i in [i0, i1) whose first entry (PART: first partition unit) is <= s.
template <bool PART = false>
__device__ __forceinline__ int mat_of_entry(const PsBatch& B, int i0, int i1, long long s) {
    const MatTable T = mat_table(B);
    int lo = i0, hi = i1;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((PART ? T[mid].poff : T[mid].off) <= s) lo = mid;
        else hi = mid;
    }
    return lo;
}

enum BlockMap { MAP_P, MAP_Q };

template <BlockMap K>
__device__ __forceinline__ int first_block(MatTable T, int i) {
    if constexpr (K == MAP_P) return T[i].begin_p;
    else return T[i].begin_q;
}

// Matrix of workgroup blk among matrices [i0, i1) (last i with first block <= blk).
template <BlockMap K>
__device__ __forceinline__ int mat_of_block(const PsBatch& B, int i0, int i1, int blk) {
    const MatTable T = mat_table(B);
    int lo = i0, hi = i1;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (first_block<K>(T, mid) <= blk) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Rows [r0, r1) of an n-row matrix that starts at unit off, w units per row,
// whose first unit lies in [s_lo, s_hi).
__device__ __forceinline__ void rows_in_range(long long off, int n, int w, long long s_lo, long long s_hi,
                                              int& r0, int& r1) {
    const long long a = s_lo - off, b = s_hi - off;
    r0 = a <= 0 ? 0 : static_cast<int>(min(static_cast<long long>(n), (a + w - 1) / w));
    r1 = b <= 0 ? 0 : static_cast<int>(min(static_cast<long long>(n), (b + w - 1) / w));
}
// Rows of matrix M whose first entry lies in [s_lo, s_hi).
__device__ __forceinline__ void rows_in_share(const PsMat& M, long long s_lo, long long s_hi, int& r0, int& r1) {
    rows_in_range(M.off, M.n, M.m, s_lo, s_hi, r0, r1);
}
// Rows of matrix M (of a fused class) whose first partition unit lies in [s_lo, s_hi).
__device__ __forceinline__ void rows_in_part(const PsMat& M, long long s_lo, long long s_hi, int& r0, int& r1) {
    rows_in_range(M.poff, M.n, M.rcost, s_lo, s_hi, r0, r1);
}

// One entry of the residual m' = M - P^ Q^T of a row: ph = the row of P^,
// qr = Q of the column (both zero past the rank).  The explicit step's output
// pass and the deferred step's first pass both form it with these float32
// operations in this order, so the deferred memory has the explicit bits.
__device__ __forceinline__ float residual1(float mv, const float (&ph)[4], const float (&qr)[4]) {
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) s = fmaf(ph[j], qr[j], s);
    return mv - s;
}

// Row `row` of P^_prev (zero past the previous rank), through scalar loads:
// p was written by an earlier kernel and is only read in this one.
__device__ __forceinline__ void prev_phat_row(const PsMat& M, int row, float (&ph)[4]) {
    typedef const __attribute__((address_space(4))) float* ConstF;
    const ConstF pc = (ConstF)(M.p);
#pragma unroll
    for (int j = 0; j < 4; ++j) ph[j] = j < M.prank ? pc[static_cast<long long>(j) * M.n + row] : 0.0f;
}

__device__ __forceinline__ int nstrips_of(int m) {
    const int w = (m % 4 == 0) ? PS_THREADS * 4 : PS_THREADS;
    return (m + w - 1) / w;
}

// M values of 4 consecutive entries starting at flat element e (16-byte
// aligned); STREAM: last read of these entries in the step
template <bool BF16, bool STREAM = false>
__device__ __forceinline__ float4 load_M4(const PsMat& M, float eta, long long e) {
    const float4 g = STREAM ? load_grad4_stream<BF16>(M.grad, e / 4) : load_grad4<BF16>(M.grad, e / 4);
    const float4 mm = STREAM ? load_stream(reinterpret_cast<const float4*>(M.mem) + e / 4)
                             : reinterpret_cast<const float4*>(M.mem)[e / 4];
    return make_float4(ef_acc(mm.x, eta, g.x), ef_acc(mm.y, eta, g.y), ef_acc(mm.z, eta, g.z),
                       ef_acc(mm.w, eta, g.w));
}

template <bool BF16>
__device__ __forceinline__ float load_M1(const PsMat& M, float eta, long long e) {
    return ef_acc(M.mem[e], eta, load_grad1<BF16>(M.grad, e));
}

template <bool BF16, int VEC, bool STREAM = false>
__device__ __forceinline__ void load_Mv(const PsMat& M, float eta, long long e, float (&v)[VEC]) {
    if constexpr (VEC == 4) {
        const float4 t = load_M4<BF16, STREAM>(M, eta, e);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else {
        v[0] = load_M1<BF16>(M, eta, e);
    }
}

// ------------------------------------------------------------------ psgd_p / psgd_q (split path)

// Each wave owns P_ROWS_WAVE rows; lanes stride over the row in VEC-wide
// chunks.  The row loads of one chunk are issued before any use.
template <bool BF16, int VEC, bool DEF>
__device__ __forceinline__ void p_rows(const PsMat& M, float eta, int row0, float (&acc)[P_ROWS_WAVE][4]) {
    const int lane = threadIdx.x & 63;
    const int n = M.n, m = M.m, r = M.rank;
    const int nch = m / VEC;
    const int qn = DEF ? max(r, M.prank) : r;
    int rowc[P_ROWS_WAVE];
    float ph[P_ROWS_WAVE][4];
#pragma unroll
    for (int rr = 0; rr < P_ROWS_WAVE; ++rr) {
        rowc[rr] = min(row0 + rr, n - 1);
        if constexpr (DEF) prev_phat_row(M, rowc[rr], ph[rr]);
    }
#pragma unroll 2
    for (int c = lane; c < nch; c += 64) {
        float qa[VEC][4], qv[VEC][4], qp[VEC][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < qn) {
                if constexpr (VEC == 4) {
                    const float4 t = reinterpret_cast<const float4*>(M.q + static_cast<long long>(j) * m)[c];
                    qa[0][j] = t.x; qa[1][j] = t.y; qa[2][j] = t.z; qa[3][j] = t.w;
                } else {
                    qa[0][j] = M.q[static_cast<long long>(j) * m + c];
                }
            } else {
#pragma unroll
                for (int v = 0; v < VEC; ++v) qa[v][j] = 0.0f;
            }
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                qv[v][j] = j < r ? qa[v][j] : 0.0f;
                qp[v][j] = j < M.prank ? qa[v][j] : 0.0f;
            }
        }
        float mv[P_ROWS_WAVE][VEC];
#pragma unroll
        for (int rr = 0; rr < P_ROWS_WAVE; ++rr) {
            const long long e = static_cast<long long>(rowc[rr]) * m + static_cast<long long>(c) * VEC;
            if constexpr (DEF) {
                // rebuild m' from M_prev, form M and store it over M_prev (the
                // clamped copy of the last row stores nothing)
                float mp[VEC], gv[VEC];
                if constexpr (VEC == 4) {
                    const float4 a = reinterpret_cast<const float4*>(M.mem)[e / 4];
                    const float4 b = load_grad4<BF16>(M.grad, e / 4);
                    mp[0] = a.x; mp[1] = a.y; mp[2] = a.z; mp[3] = a.w;
                    gv[0] = b.x; gv[1] = b.y; gv[2] = b.z; gv[3] = b.w;
                } else {
                    mp[0] = M.mem[e];
                    gv[0] = load_grad1<BF16>(M.grad, e);
                }
#pragma unroll
                for (int v = 0; v < VEC; ++v) mv[rr][v] = ef_acc(residual1(mp[v], ph[rr], qp[v]), eta, gv[v]);
                if (row0 + rr < n) {
                    if constexpr (VEC == 4)
                        reinterpret_cast<float4*>(M.mem)[e / 4] = make_float4(mv[rr][0], mv[rr][1], mv[rr][2], mv[rr][3]);
                    else
                        M.mem[e] = mv[rr][0];
                }
            } else {
                load_Mv<BF16, VEC>(M, eta, e, mv[rr]);
            }
        }
#pragma unroll
        for (int rr = 0; rr < P_ROWS_WAVE; ++rr) {
            if (row0 + rr < n) {
#pragma unroll
                for (int v = 0; v < VEC; ++v)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[rr][j] = fmaf(mv[rr][v], qv[v][j], acc[rr][j]);
            }
        }
    }
}

template <bool BF16, bool DEF>
__global__ __launch_bounds__(PS_THREADS) void psgd_p(const PsBatch B, int i0, int i1) {
    __shared__ double s_g[4][16];
    const PsMat M = mat_at(B, mat_of_block<MAP_P>(B, i0, i1, blockIdx.x));
    const int lwg = blockIdx.x - M.begin_p;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row0 = lwg * P_ROWS_WG + w * P_ROWS_WAVE;
    float acc[P_ROWS_WAVE][4];
#pragma unroll
    for (int rr = 0; rr < P_ROWS_WAVE; ++rr)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[rr][j] = 0.0f;
    if (M.m % 4 == 0)
        p_rows<BF16, 4, DEF>(M, B.eta, row0, acc);
    else
        p_rows<BF16, 1, DEF>(M, B.eta, row0, acc);
#pragma unroll
    for (int rr = 0; rr < P_ROWS_WAVE; ++rr)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[rr][j] = wave_sum(acc[rr][j]);
    // every lane now holds the finished rows of this wave; lane i < 16 keeps
    // Gram entry (i / 4, i % 4) summed over them (float64)
    const int ga = (lane >> 2) & 3, gb = lane & 3;
    double g = 0.0;
#pragma unroll
    for (int rr = 0; rr < P_ROWS_WAVE; ++rr) {
        const int row = row0 + rr;
        if (row < M.n) {
            if (lane == rr)
                reinterpret_cast<float4*>(M.praw)[row] = make_float4(acc[rr][0], acc[rr][1], acc[rr][2], acc[rr][3]);
            float pa = acc[rr][0], pb = acc[rr][0];
#pragma unroll
            for (int j = 1; j < 4; ++j) {
                pa = (ga == j) ? acc[rr][j] : pa;
                pb = (gb == j) ? acc[rr][j] : pb;
            }
            g += static_cast<double>(pa) * static_cast<double>(pb);
        }
    }
    if (lane < 16) s_g[w][lane] = g;
    __syncthreads();
    if (threadIdx.x < 16) {
        const int i = threadIdx.x;
        M.gpart[static_cast<long long>(lwg) * 16 + i] = ((s_g[0][i] + s_g[1][i]) + s_g[2][i]) + s_g[3][i];
    }
}

// ------------------------------------------------------------------ psgd_q

template <bool BF16, int VEC, bool DEF>
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
    for (int i0 = r0; i0 < r1; i0 += ROW_GROUP) {
        float mv[ROW_GROUP][VEC];
#pragma unroll
        for (int u = 0; u < ROW_GROUP; ++u) {
            const int row = min(i0 + u, r1 - 1);
            const long long e = static_cast<long long>(row) * m + col0;
            if constexpr (DEF) {
                // psgd_p stored M in mem
                if constexpr (VEC == 4) {
                    const float4 a = reinterpret_cast<const float4*>(M.mem)[e / 4];
                    mv[u][0] = a.x; mv[u][1] = a.y; mv[u][2] = a.z; mv[u][3] = a.w;
                } else {
                    mv[u][0] = M.mem[e];
                }
            } else {
                load_Mv<BF16, VEC>(M, eta, e, mv[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < ROW_GROUP; ++u) {
            if (i0 + u < r1) {
                const float4 p = praw4[i0 + u];
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    acc[v][0] = fmaf(mv[u][v], p.x, acc[v][0]);
                    acc[v][1] = fmaf(mv[u][v], p.y, acc[v][1]);
                    acc[v][2] = fmaf(mv[u][v], p.z, acc[v][2]);
                    acc[v][3] = fmaf(mv[u][v], p.w, acc[v][3]);
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (j < M.rank) {
            float* dst = qplane(M, chunk, j) + col0;
            if constexpr (VEC == 4)
                *reinterpret_cast<float4*>(dst) = make_float4(acc[0][j], acc[1][j], acc[2][j], acc[3][j]);
            else
                dst[0] = acc[0][j];
        }
    }
}

template <bool BF16, bool DEF>
__global__ __launch_bounds__(PS_THREADS) void psgd_q(const PsBatch B, int i0, int i1) {
    const PsMat M = mat_at(B, mat_of_block<MAP_Q>(B, i0, i1, blockIdx.x));
    const int lwg = blockIdx.x - M.begin_q;
    const int ns = nstrips_of(M.m);
    const int strip = lwg % ns, chunk = lwg / ns;
    if (M.m % 4 == 0)
        q_chunk<BF16, 4, DEF>(M, B.eta, strip, chunk);
    else
        q_chunk<BF16, 1, DEF>(M, B.eta, strip, chunk);
}

// ------------------------------------------------------------------ psgd_pq

// Raw (unconverted) data of one float4 chunk of a row; converted to M only
// when the row is used, so that the loads of the next rows can be in flight.
template <bool BF16>
struct RawChunk;
template <>
struct RawChunk<true> {
    float4 m;
    uint2 g;
};
template <>
struct RawChunk<false> {
    float4 m;
    float4 g;
};

template <bool BF16>
__device__ __forceinline__ float4 raw_grad(const RawChunk<BF16>& r) {
    if constexpr (BF16) {
        return make_float4(__uint_as_float(r.g.x << 16), __uint_as_float(r.g.x & 0xFFFF0000u),
                           __uint_as_float(r.g.y << 16), __uint_as_float(r.g.y & 0xFFFF0000u));
    } else {
        return r.g;
    }
}

template <bool BF16>
__device__ __forceinline__ float4 raw_to_M(const RawChunk<BF16>& r, float eta) {
    const float4 g = raw_grad<BF16>(r);
    return make_float4(ef_acc(r.m.x, eta, g.x), ef_acc(r.m.y, eta, g.y), ef_acc(r.m.z, eta, g.z),
                       ef_acc(r.m.w, eta, g.w));
}

// Deferred memory: M = m' + eta*grad with m' = M_prev - P^_prev Q_prev^T
// rebuilt here from the stored M_prev (4 columns of one row), ph = that row
// of P^_prev, qr[c] = Q_prev of column c (both zero past the previous rank).
template <bool BF16>
__device__ __forceinline__ float4 raw_to_M_def(const RawChunk<BF16>& r, float eta, const float (&ph)[4],
                                               const float (&qr)[4][4]) {
    const float4 g = raw_grad<BF16>(r);
    return make_float4(ef_acc(residual1(r.m.x, ph, qr[0]), eta, g.x), ef_acc(residual1(r.m.y, ph, qr[1]), eta, g.y),
                       ef_acc(residual1(r.m.z, ph, qr[2]), eta, g.z), ef_acc(residual1(r.m.w, ph, qr[3]), eta, g.w));
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Buffer resources over rows [r0, r1) of a matrix.  The whole byte offset of
// a load goes into the vector operand, which the hardware checks against the
// record count: rows past r1, and lanes given an offset of 2^31 or more, read
// zeros without touching memory.
constexpr int BUF_WORD3 = 0x00020000;
constexpr unsigned OOB_OFFSET = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, long long e0, int elem_bytes,
                                                            long long nelem) {
    char* p = const_cast<char*>(static_cast<const char*>(base)) + e0 * elem_bytes;
    return __builtin_amdgcn_make_buffer_rsrc(p, 0, static_cast<int>(nelem * elem_bytes), BUF_WORD3);
}

// One reduce-scatter step across lane pairs: each lane reads its partner's
// registers through the DPP control CTRL.  Lanes whose BIT is clear keep the
// first half of x, the others the second half; a kept entry gains the
// partner's copy of it.  Partners must hold the same entries of x.
template <int CTRL, int BIT, int N>
__device__ __forceinline__ void scatter_step(const float (&x)[N], float (&y)[N / 2], int lane) {
    const bool hi = (lane & BIT) != 0;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
        const float send = hi ? x[i] : x[i + N / 2];
        const float keep = hi ? x[i + N / 2] : x[i];
        y[i] = keep + dpp_f32<CTRL>(send);
    }
}

__device__ __forceinline__ int rev4(int x) {
    return ((x & 1) << 3) | ((x & 2) << 1) | ((x & 4) >> 1) | ((x & 8) >> 3);
}

// Rows [r0, r1) of one matrix, RG rows at a time, by a workgroup of NT
// threads that spans a row: thread t owns the VPT float4 chunks t, t + NT, ...
// (columns 4(t + c NT) .. +3), so Q_in and the M^T P accumulators of its
// columns stay in registers.
//   1. the RG rows' raw data (loaded one group ahead) become M;
//   2. each thread forms its share of the RG x 4 dot products M[i,:] Q_in
//      (its chunks in order);
//   3. a DPP reduce-scatter over each 16-lane row leaves the V = 4 RG sums
//      spread over the row's lanes (lane li holds entry rev(li); with V < 16
//      the lanes past V hold copies and the last steps are plain adds); the
//      NT/16 row partials go to LDS (double-buffered, one barrier per group);
//   4. every wave sums the partials of each value in a fixed order (its lanes
//      split the partials, then lane-exchange adds) and reads the V finished
//      P entries into scalars;
//   5. M^T P accumulators += M[i, cols] P[i, :]; wave 0 stores the P rows and
//      accumulates the Gram matrix (float64).
// The accumulators and Gram entries of the workgroup are partial `part`.
template <bool BF16, int NT, int RG, int VPT, bool DEF>
__device__ __forceinline__ void pq_rows(const PsMat& M, float eta, int r0, int r1, int part,
                                        float (*s_part)[NT / 16][4 * RG], int& par) {
    constexpr int V = 4 * RG;          // P entries per row group
    constexpr int NP = NT / 16;        // partials per entry (16-lane rows of the workgroup)
    constexpr int L = 64 / V;          // lanes sharing the sum of one entry
    constexpr int PER = V > 16 ? V / 16 : 1;   // entries per lane after the reduce-scatter
    static_assert(V == 4 || V == 8 || V == 16 || V == 32, "row groups of 1, 2, 4 or 8 rows");
    static_assert(NP % L == 0, "partials split evenly over the lanes of an entry");
    const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int m = M.m, c4 = m / 4, nr = r1 - r0;
    bool act[VPT];
#pragma unroll
    for (int c = 0; c < VPT; ++c) act[c] = t + c * NT < c4;

    // Q of the thread's columns: Q_in for P = M Q_in, and in the deferred form
    // also Q_prev for the residual rebuild.  Columns past max(rank, prev rank)
    // are zero.  On a rank change the two differ only in columns that meet a
    // zero: past the previous rank the stored P^_prev row is zero (the
    // residual sum gains exact +0 terms), and P's columns past the rank never
    // reach T, Q' or P^ (T is zero there) -- so one copy gives the bits of
    // separately masked ones.
    float q[VPT][4][4], qt[VPT][4][4];
    const int qn = DEF ? max(M.rank, M.prank) : M.rank;
#pragma unroll
    for (int c = 0; c < VPT; ++c) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (act[c] && j < qn) v = reinterpret_cast<const float4*>(M.q + static_cast<long long>(j) * m)[t + c * NT];
            q[c][0][j] = v.x; q[c][1][j] = v.y; q[c][2][j] = v.z; q[c][3][j] = v.w;
        }
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int j = 0; j < 4; ++j) qt[c][cc][j] = 0.0f;
    }

    const long long e0 = static_cast<long long>(r0) * m, ne = static_cast<long long>(nr) * m;
    const __amdgpu_buffer_rsrc_t rm = rows_rsrc(M.mem, e0, 4, ne);
    const __amdgpu_buffer_rsrc_t rg = rows_rsrc(M.grad, e0, BF16 ? 2 : 4, ne);
    unsigned colm[VPT], colg[VPT];
#pragma unroll
    for (int c = 0; c < VPT; ++c) {
        colm[c] = act[c] ? static_cast<unsigned>(t + c * NT) * 16u : OOB_OFFSET;
        colg[c] = act[c] ? static_cast<unsigned>(t + c * NT) * (BF16 ? 8u : 16u) : OOB_OFFSET;
    }
    const unsigned rowm = static_cast<unsigned>(m) * 4u, rowg = static_cast<unsigned>(m) * (BF16 ? 2u : 4u);

    RawChunk<BF16> raw[RG][VPT];
    auto load_group = [&](int k) {
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            const unsigned kr = static_cast<unsigned>(k + r);
#pragma unroll
            for (int c = 0; c < VPT; ++c) {
                raw[r][c].m = __builtin_bit_cast(float4,
                                                 __builtin_amdgcn_raw_buffer_load_b128(rm, colm[c] + kr * rowm, 0, 0));
                if constexpr (BF16)
                    raw[r][c].g = __builtin_bit_cast(uint2,
                                                     __builtin_amdgcn_raw_buffer_load_b64(rg, colg[c] + kr * rowg, 0, 0));
                else
                    raw[r][c].g = __builtin_bit_cast(float4,
                                                     __builtin_amdgcn_raw_buffer_load_b128(rg, colg[c] + kr * rowg, 0, 0));
            }
        }
    };

    const int li = lane & 15, lr = lane >> 4;
    const int vi = lane % V, lg = lane / V;
    const int ga = (lane >> 2) & 3, gb = lane & 3;
    double g = 0.0;
    load_group(0);
    for (int k = 0; k < nr; k += RG) {
        float v[RG][VPT][4];
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            // deferred memory: M replaces M_prev in mem; rows past r1 and idle
            // lanes store nothing.  Rows past r1 read as zero and take a zero
            // P^ row, so their M stays zero (no P, Gram or M^T P terms)
            float ph[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (DEF) {
                if (k + r < nr) prev_phat_row(M, r0 + k + r, ph);
            }
#pragma unroll
            for (int c = 0; c < VPT; ++c) {
                float4 x;
                if constexpr (DEF) {
                    x = raw_to_M_def<BF16>(raw[r][c], eta, ph, q[c]);
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rm,
                                                           colm[c] + static_cast<unsigned>(k + r) * rowm, 0, 0);
                } else {
                    x = raw_to_M<BF16>(raw[r][c], eta);
                }
                v[r][c][0] = x.x; v[r][c][1] = x.y; v[r][c][2] = x.z; v[r][c][3] = x.w;
            }
        }
        load_group(k + RG);
        float xs[V];
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float a = v[r][0][0] * q[0][0][j];
                a = fmaf(v[r][0][1], q[0][1][j], a);
                a = fmaf(v[r][0][2], q[0][2][j], a);
                a = fmaf(v[r][0][3], q[0][3][j], a);
#pragma unroll
                for (int c = 1; c < VPT; ++c)
#pragma unroll
                    for (int cc = 0; cc < 4; ++cc) a = fmaf(v[r][c][cc], q[c][cc][j], a);
                xs[4 * r + j] = a;
            }
        float red[PER];
        if constexpr (V == 32) {
            float x16[16], x8[8], x4[4];
            scatter_step<DPP_XOR1, 1>(xs, x16, lane);
            scatter_step<DPP_XOR2, 2>(x16, x8, lane);
            scatter_step<DPP_ROR4, 4>(x8, x4, lane);
            scatter_step<DPP_ROR8, 8>(x4, red, lane);
        } else if constexpr (V == 16) {
            float x8[8], x4[4], x2[2];
            scatter_step<DPP_XOR1, 1>(xs, x8, lane);
            scatter_step<DPP_XOR2, 2>(x8, x4, lane);
            scatter_step<DPP_ROR4, 4>(x4, x2, lane);
            scatter_step<DPP_ROR8, 8>(x2, red, lane);
        } else if constexpr (V == 8) {
            float x4[4], x2[2], x1[1];
            scatter_step<DPP_XOR1, 1>(xs, x4, lane);
            scatter_step<DPP_XOR2, 2>(x4, x2, lane);
            scatter_step<DPP_ROR4, 4>(x2, x1, lane);
            red[0] = x1[0] + dpp_f32<DPP_ROR8>(x1[0]);
        } else {
            float x2[2], x1[1];
            scatter_step<DPP_XOR1, 1>(xs, x2, lane);
            scatter_step<DPP_XOR2, 2>(x2, x1, lane);
            const float y = x1[0] + dpp_f32<DPP_ROR4>(x1[0]);
            red[0] = y + dpp_f32<DPP_ROR8>(y);
        }
        // lane li of a 16-lane row holds entries PER * rev(li) + i (rev over
        // log2(min(V, 16)) bits); with V < 16 lanes li >= V hold copies
        if (V >= 16 || li < V) {
            const int e = V >= 16 ? PER * rev4(li) : V == 8 ? rev4(li) >> 1 : rev4(li) >> 2;
            float* dst = &s_part[par][w * 4 + lr][e];
#pragma unroll
            for (int i = 0; i < PER; ++i) dst[i] = red[i];
        }
        __syncthreads();
        float pv = 0.0f;
#pragma unroll
        for (int u = 0; u < NP / L; ++u) pv += s_part[par][lg * (NP / L) + u][vi];
#pragma unroll
        for (int sh = V; sh < 64; sh <<= 1) pv += __shfl_xor(pv, sh, WAVE);
        par ^= 1;
        float p[RG][4];
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) p[r][j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pv), 4 * r + j));
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
            for (int c = 0; c < VPT; ++c)
#pragma unroll
                for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                    for (int j = 0; j < 4; ++j) qt[c][cc][j] = fmaf(v[r][c][cc], p[r][j], qt[c][cc][j]);
        if (w == 0) {
            // rows past r1 read as zero: their P entries and Gram terms are zero
            if (lane < V && k + vi / 4 < nr) M.praw[static_cast<long long>(r0 + k) * 4 + vi] = pv;
            if (lane < 16) {
#pragma unroll
                for (int r = 0; r < RG; ++r) {
                    float pa = p[r][0], pb = p[r][0];
#pragma unroll
                    for (int j = 1; j < 4; ++j) {
                        pa = (ga == j) ? p[r][j] : pa;
                        pb = (gb == j) ? p[r][j] : pb;
                    }
                    g = fma(static_cast<double>(pa), static_cast<double>(pb), g);
                }
            }
        }
    }
#pragma unroll
    for (int c = 0; c < VPT; ++c) {
        if (act[c]) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (j < M.rank)
                    *reinterpret_cast<float4*>(qplane(M, part, j) + 4 * (t + c * NT)) =
                        make_float4(qt[c][0][j], qt[c][1][j], qt[c][2][j], qt[c][3][j]);
        }
    }
    if (w == 0 && lane < 16) M.gpart[static_cast<long long>(part) * 16 + lane] = g;
}

// Workgroup shape of each fused class: threads, rows per group, float4 chunks
// per thread, waves per SIMD the kernel is compiled for (bounds its registers).
template <int CLS> struct PqShape;
template <> struct PqShape<0> { static constexpr int NT = 256, RG = 8, VPT = 1, WAVES = 3; };
template <> struct PqShape<1> { static constexpr int NT = 512, RG = 4, VPT = 1, WAVES = 4; };
template <> struct PqShape<2> { static constexpr int NT = 1024, RG = 4, VPT = 1, WAVES = 4; };
template <> struct PqShape<3> { static constexpr int NT = 768, RG = 2, VPT = 2, WAVES = 3; };
template <> struct PqShape<4> { static constexpr int NT = 1024, RG = 1, VPT = 2, WAVES = 4; };

// One pass over the matrices of fused class CLS: workgroup b takes its
// balanced share of their rows, matrix by matrix.
template <bool BF16, int CLS, bool DEF>
__global__ __launch_bounds__(PqShape<CLS>::NT, PqShape<CLS>::WAVES) void psgd_pq(const PsBatch B) {
    constexpr int NT = PqShape<CLS>::NT, RG = PqShape<CLS>::RG, VPT = PqShape<CLS>::VPT;
    __shared__ float s_part[2][NT / 16][4 * RG];
    const int b = blockIdx.x, G = B.cgrid[CLS];
    const int i0 = B.cbeg[CLS], i1 = B.cbeg[CLS + 1];
    const long long E = B.cent[CLS], base = B.cbase[CLS];
    const long long s_lo = base + share_lo(E, G, b), s_hi = base + share_lo(E, G, b + 1);
    int par = 0;
    for (int i = mat_of_entry<true>(B, i0, i1, s_lo); i < i1; ++i) {
        const PsMat M = mat_at(B, i);
        if (M.poff >= s_hi) break;
        int r0, r1;
        rows_in_part(M, s_lo, s_hi, r0, r1);
        if (r0 >= r1) continue;
        pq_rows<BF16, NT, RG, VPT, DEF>(M, B.eta, r0, r1, b - owner_of(M.poff - base, E, G), s_part, par);
    }
}

// ------------------------------------------------------------------ small matrices

// A whole small matrix (n, m <= 1024; any m) by one workgroup of NT threads:
//   1. one wave per row at a time forms M (deferred: rebuilds the residual and
//      stores M over mem) and the row's P = M Q_in, lanes striding over the
//      columns, summed with wave_sum; P goes to LDS and praw;
//   2. after a barrier, threads 0..15 sum the Gram matrix over the rows in
//      order (float64) and every thread forms M^T P for its columns from the
//      matrix (now in the cache) and P in LDS.
// One M^T P and one Gram partial.
template <bool BF16, int NT, bool DEF>
__device__ void small_pq(const PsMat& M, float eta, float* s_p) {
    constexpr int NW = NT / 64;
    const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int n = M.n, m = M.m;
    const int qn = DEF ? max(M.rank, M.prank) : M.rank;   // one copy of Q, as in pq_rows
    for (int i = w; i < n; i += NW) {
        float ph[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (DEF) prev_phat_row(M, i, ph);
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int c = lane; c < m; c += 64) {
            float qv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) qv[j] = j < qn ? M.q[static_cast<long long>(j) * m + c] : 0.0f;
            const long long e = static_cast<long long>(i) * m + c;
            float mv;
            if constexpr (DEF) {
                mv = ef_acc(residual1(M.mem[e], ph, qv), eta, load_grad1<BF16>(M.grad, e));
                M.mem[e] = mv;
            } else {
                mv = load_M1<BF16>(M, eta, e);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = fmaf(mv, qv[j], acc[j]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = wave_sum(acc[j]);
        if (lane < 4) {
            const float v = lane == 0 ? acc[0] : lane == 1 ? acc[1] : lane == 2 ? acc[2] : acc[3];
            s_p[i * 4 + lane] = v;
            M.praw[static_cast<long long>(i) * 4 + lane] = v;
        }
    }
    __syncthreads();
    if (t < 16) {
        const int a = t >> 2, b = t & 3;
        double g = 0.0;
        for (int i = 0; i < n; ++i) g = fma(static_cast<double>(s_p[i * 4 + a]), static_cast<double>(s_p[i * 4 + b]), g);
        M.gpart[t] = g;
    }
    for (int c = t; c < m; c += NT) {
        float qt[4] = {0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < n; ++i) {
            const long long e = static_cast<long long>(i) * m + c;
            const float mv = DEF ? M.mem[e] : load_M1<BF16>(M, eta, e);
#pragma unroll
            for (int j = 0; j < 4; ++j) qt[j] = fmaf(mv, s_p[i * 4 + j], qt[j]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (j < M.rank) qplane(M, 0, j)[c] = qt[j];
    }
}

constexpr int SMALL_THREADS = 256;

// The small class alone (when no team launch carries it): one workgroup per matrix.
template <bool BF16, bool DEF>
__global__ __launch_bounds__(SMALL_THREADS) void psgd_small(const PsBatch B) {
    __shared__ float s_p[SMALL_MAX_N * 4];
    small_pq<BF16, SMALL_THREADS, DEF>(mat_at(B, B.cbeg[SMALL_CLASS] + blockIdx.x), B.eta, s_p);
}

// ------------------------------------------------------------------ psgd_pq_teams

// Small launch groups are launch-bound, so their fused classes run in ONE
// launch of 1024-thread workgroups.  The workgroups of class c follow those of
// the classes before it; a class-c workgroup holds 1024 / TW teams of TW
// threads (TW = 256, 512, 1024: the class's row width), and team j of its w-th
// workgroup is virtual block w * (1024 / TW) + j of the class's balanced
// partition (cgrid[c] virtual blocks): the share, the partial index and the
// arithmetic of one workgroup of the separate class launch.  Every team runs
// the same number of iterations -- the workgroup's largest row-group count --
// with exactly one barrier each, outside any team-dependent branch, so the
// barrier is uniform; a team that has run out of rows idles.
constexpr int TEAM_NT = 1024;
constexpr int TEAM_RG = 4;
constexpr int TEAM_CLASSES = 3;   // the classes a team kernel runs (row widths 256, 512, 1024 threads)
static_assert(TEAM_CLASSES <= PQ_CLASSES, "one team width per team class");
constexpr long long TEAM_MAX_ENTRIES = 1LL << 26;   // launch groups up to this size use the team kernel

__host__ __device__ constexpr int team_width(int cls) { return cls == 0 ? 256 : cls == 1 ? 512 : 1024; }
__host__ __device__ inline int team_wgs(int vblocks, int cls) {
    const int per = TEAM_NT / team_width(cls);
    return (vblocks + per - 1) / per;
}

template <bool BF16, int TW, bool DEF>
__device__ __forceinline__ void pq_teams(const PsBatch& B, int cls, int wg_in_class,
                                         float (*s_part)[TEAM_NT / 16][4 * TEAM_RG], int* s_cnt) {
    constexpr int RG = TEAM_RG, V = 4 * RG, NPT = TW / 16, L = 64 / V, TEAMS = TEAM_NT / TW;
    static_assert(V == 16, "row groups of 4");
    // a team spans whole waves: its index (and all its matrix state) is wave-uniform
    const int tid = threadIdx.x, team = __builtin_amdgcn_readfirstlane(tid / TW), tt = tid % TW;
    const int lane = tid & 63, wt = __builtin_amdgcn_readfirstlane(tt >> 6);
    const int G = B.cgrid[cls];
    const int vb = wg_in_class * TEAMS + team;
    const bool valid = vb < G;
    const int i0 = B.cbeg[cls], i1 = B.cbeg[cls + 1];
    const long long E = B.cent[cls], base = B.cbase[cls];
    long long s_lo = 0, s_hi = 0;
    if (valid) {
        s_lo = base + share_lo(E, G, vb);
        s_hi = base + share_lo(E, G, vb + 1);
    }
    const MatTable T = mat_table(B);

    // the team's row groups over all the matrices of its share
    int ngroups = 0, mfirst = i1;
    if (valid) {
        mfirst = mat_of_entry<true>(B, i0, i1, s_lo);
        for (int i = mfirst; i < i1; ++i) {
            const long long off = T[i].poff;
            if (off >= s_hi) break;
            int a, b;
            rows_in_range(off, T[i].n, T[i].rcost, s_lo, s_hi, a, b);
            if (b > a) ngroups += (b - a + RG - 1) / RG;
        }
    }
    if (tt == 0) s_cnt[team] = ngroups;
    __syncthreads();
    int gmax = 0;
#pragma unroll
    for (int j = 0; j < TEAMS; ++j) gmax = max(gmax, s_cnt[j]);

    // state of the team's current matrix (uniform across the team)
    int mi = mfirst, r0 = 0, r1 = 0, nr = 0, k = 0, part = 0, m = 1;
    PsMat M{};
    bool act = false;
    float q[4][4], qt[4][4], qr[4][4];
    double g = 0.0;
    __amdgpu_buffer_rsrc_t rm = rows_rsrc(nullptr, 0, 4, 0), rg = rows_rsrc(nullptr, 0, 4, 0);
    unsigned colm = OOB_OFFSET, colg = OOB_OFFSET, rowm = 0, rowg = 0;
    RawChunk<BF16> raw[RG];
    auto load_group = [&](int kk) {
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            const unsigned kr = static_cast<unsigned>(kk + r);
            raw[r].m = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rm, colm + kr * rowm, 0, 0));
            if constexpr (BF16)
                raw[r].g = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rg, colg + kr * rowg, 0, 0));
            else
                raw[r].g = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rg, colg + kr * rowg, 0, 0));
        }
    };
    // moves to the first matrix at or after mi with rows in the share and
    // loads its Q_in and first row group; false when there is none
    auto open_matrix = [&]() -> bool {
        for (; mi < i1; ++mi) {
            if (T[mi].poff >= s_hi) {
                mi = i1;
                break;
            }
            M = mat_at(B, mi);
            rows_in_part(M, s_lo, s_hi, r0, r1);
            if (r1 > r0) break;
        }
        if (mi >= i1) return false;
        nr = r1 - r0;
        k = 0;
        part = vb - owner_of(M.poff - base, E, G);
        m = M.m;
        act = tt < m / 4;
        const int qn = DEF ? max(M.rank, M.prank) : M.rank;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float4 qv = make_float4(0.f, 0.f, 0.f, 0.f);
            if (act && j < qn) qv = reinterpret_cast<const float4*>(M.q + static_cast<long long>(j) * m)[tt];
            const bool in = j < M.rank, ip = j < M.prank;
            q[0][j] = in ? qv.x : 0.f; q[1][j] = in ? qv.y : 0.f; q[2][j] = in ? qv.z : 0.f; q[3][j] = in ? qv.w : 0.f;
            qr[0][j] = ip ? qv.x : 0.f; qr[1][j] = ip ? qv.y : 0.f; qr[2][j] = ip ? qv.z : 0.f;
            qr[3][j] = ip ? qv.w : 0.f;
        }
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int j = 0; j < 4; ++j) qt[cc][j] = 0.0f;
        g = 0.0;
        const long long e0 = static_cast<long long>(r0) * m, ne = static_cast<long long>(nr) * m;
        rm = rows_rsrc(M.mem, e0, 4, ne);
        rg = rows_rsrc(M.grad, e0, BF16 ? 2 : 4, ne);
        colm = act ? static_cast<unsigned>(tt) * 16u : OOB_OFFSET;
        colg = act ? static_cast<unsigned>(tt) * (BF16 ? 8u : 16u) : OOB_OFFSET;
        rowm = static_cast<unsigned>(m) * 4u;
        rowg = static_cast<unsigned>(m) * (BF16 ? 2u : 4u);
        load_group(0);
        return true;
    };

    const int li = lane & 15, lr = lane >> 4;
    const int vi = lane % V, lg = lane / V;
    const int ga = (lane >> 2) & 3, gb = lane & 3;
    bool live = valid && open_matrix();
    int par = 0;
    for (int it = 0; it < gmax; ++it) {
        float v[RG][4];
        if (live) {
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                float4 x;
                if constexpr (DEF) {
                    // rows past r1: zero data and a zero P^ row give M = 0
                    float ph[4] = {0.f, 0.f, 0.f, 0.f};
                    if (k + r < nr) prev_phat_row(M, r0 + k + r, ph);
                    x = raw_to_M_def<BF16>(raw[r], B.eta, ph, qr);
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rm,
                                                           colm + static_cast<unsigned>(k + r) * rowm, 0, 0);
                } else {
                    x = raw_to_M<BF16>(raw[r], B.eta);
                }
                v[r][0] = x.x; v[r][1] = x.y; v[r][2] = x.z; v[r][3] = x.w;
            }
            load_group(k + RG);
            float xs[V];
#pragma unroll
            for (int r = 0; r < RG; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float a = v[r][0] * q[0][j];
                    a = fmaf(v[r][1], q[1][j], a);
                    a = fmaf(v[r][2], q[2][j], a);
                    xs[4 * r + j] = fmaf(v[r][3], q[3][j], a);
                }
            float x8[V / 2], x4[V / 4], x2[V / 8], x1[V / 16];
            scatter_step<DPP_XOR1, 1>(xs, x8, lane);
            scatter_step<DPP_XOR2, 2>(x8, x4, lane);
            scatter_step<DPP_ROR4, 4>(x4, x2, lane);
            scatter_step<DPP_ROR8, 8>(x2, x1, lane);
            // lane li of a 16-lane row now holds entry rev4(li)
            s_part[par][team * NPT + wt * 4 + lr][rev4(li)] = x1[0];
        }
        __syncthreads();
        if (live) {
            float pv = 0.0f;
#pragma unroll
            for (int u = 0; u < NPT / L; ++u) pv += s_part[par][team * NPT + lg * (NPT / L) + u][vi];
#pragma unroll
            for (int sh = V; sh < 64; sh <<= 1) pv += __shfl_xor(pv, sh, WAVE);
            float p[RG][4];
#pragma unroll
            for (int r = 0; r < RG; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    p[r][j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pv), 4 * r + j));
#pragma unroll
            for (int r = 0; r < RG; ++r)
#pragma unroll
                for (int cc = 0; cc < 4; ++cc)
#pragma unroll
                    for (int j = 0; j < 4; ++j) qt[cc][j] = fmaf(v[r][cc], p[r][j], qt[cc][j]);
            if (wt == 0) {
                if (lane < V && k + vi / 4 < nr) M.praw[static_cast<long long>(r0 + k) * 4 + vi] = pv;
                if (lane < 16) {
#pragma unroll
                    for (int r = 0; r < RG; ++r) {
                        float pa = p[r][0], pb = p[r][0];
#pragma unroll
                        for (int j = 1; j < 4; ++j) {
                            pa = (ga == j) ? p[r][j] : pa;
                            pb = (gb == j) ? p[r][j] : pb;
                        }
                        g = fma(static_cast<double>(pa), static_cast<double>(pb), g);
                    }
                }
            }
            k += RG;
            if (k >= nr) {
                if (act) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (j < M.rank)
                            *reinterpret_cast<float4*>(qplane(M, part, j) + 4 * tt) =
                                make_float4(qt[0][j], qt[1][j], qt[2][j], qt[3][j]);
                }
                if (wt == 0 && lane < 16) M.gpart[static_cast<long long>(part) * 16 + lane] = g;
                ++mi;
                live = open_matrix();
            }
        }
        par ^= 1;
    }
}

// The workgroups after the classes' ones take one small matrix each.
template <bool BF16, bool DEF>
__global__ __launch_bounds__(TEAM_NT) void psgd_pq_teams(const PsBatch B) {
    __shared__ float s_part[2][TEAM_NT / 16][4 * TEAM_RG];
    __shared__ int s_cnt[TEAM_NT / 256];
    __shared__ float s_p[SMALL_MAX_N * 4];
    int w = blockIdx.x, cls = 0;
    for (; cls < TEAM_CLASSES; ++cls) {
        const int n = team_wgs(B.cgrid[cls], cls);
        if (w < n) break;
        w -= n;
    }
    if (cls == 0) pq_teams<BF16, 256, DEF>(B, 0, w, s_part, s_cnt);
    else if (cls == 1) pq_teams<BF16, 512, DEF>(B, 1, w, s_part, s_cnt);
    else if (cls == 2) pq_teams<BF16, 1024, DEF>(B, 2, w, s_part, s_cnt);
    else small_pq<BF16, TEAM_NT, DEF>(mat_at(B, B.cbeg[SMALL_CLASS] + w), B.eta, s_p);
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

// Q reduction.  A matrix with nq M^T P partials uses S = qr_slices(nq, W)
// threads per column group (a power of two), where a thread covers W = 4
// adjacent columns (float4 loads from each partial plane) when m % 4 == 0, else
// W = 1: workgroup lwg takes the column groups [lwg 256/S, (lwg+1) 256/S),
// thread t sums the partials c = t / (256/S) + S i of column group t % (256/S)
// in order, and the S slice sums are added in slice order through LDS.  Only
// the planes below the rank are read.  The Gram partials are summed the same
// way with 16 slices (16 lanes add one entry's slices each).  Thread 0 builds
// T; the column threads write Q' = (M^T P) T.
__global__ __launch_bounds__(PS_THREADS, 4) void psgd_qreduce(const PsBatch B) {
    __shared__ double s_g[16][16];
    __shared__ double s_T[16];
    __shared__ double4 s_q[4][PS_THREADS];
    // the matrix of this workgroup from the plan's map: one scalar load, where
    // a search of the table would chain eight dependent ones
    typedef const __attribute__((address_space(4))) int* ConstI;
    const PsMat M = mat_at(B, ((ConstI)(B.rmap))[blockIdx.x]);
    const int lwg = blockIdx.x - M.begin_r;
    const int m = M.m, r = M.rank, t = threadIdx.x;
    const int S = M.qs, QC = PS_THREADS / S;
    const bool quad = m % 4 == 0;
    // The partials live in the workspace (global memory): loads through global
    // pointers, unconditional (indices clamped, values past the count replaced
    // by zero), so the loads of a round are in flight together instead of
    // each waiting at the join of its own branch.
    typedef const __attribute__((address_space(1))) double* GD;
    typedef const __attribute__((address_space(1))) f32x4* GF4;
    typedef const __attribute__((address_space(1))) float* GF;
    {
        const int e = t & 15, sl = t >> 4;
        double g = 0.0;
        for (int b = sl; b < M.ng; b += 64) {
            // loads issued together, added in partial order
            double x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int bu = b + 16 * u;
                const double v = ((GD)(M.gpart))[static_cast<long long>(bu < M.ng ? bu : M.ng - 1) * 16 + e];
                x[u] = bu < M.ng ? v : 0.0;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) g += x[u];
        }
        s_g[sl][e] = g;
    }
    const int cl = t % QC, sl = t / QC;
    const int col = (lwg * QC + cl) * (quad ? 4 : 1);
    // sv[c]: the rank components of column col + c
    double4 sv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) sv[c] = make_double4(0.0, 0.0, 0.0, 0.0);
    if (col < m) {
        if (quad) {
            for (int c = sl; c < M.nq; c += QR_QUAD_BATCH * S) {
                float4 x[QR_QUAD_BATCH][4];
#pragma unroll
                for (int u = 0; u < QR_QUAD_BATCH; ++u) {
                    const int cu = c + S * u;
                    const bool in = cu < M.nq;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        // every partial has all four planes allocated
                        const f32x4 v = ((GF4)(qplane(M, in ? cu : M.nq - 1, j) + col))[0];
                        const bool use = in && j < r;
                        x[u][j] = make_float4(use ? v.x : 0.f, use ? v.y : 0.f, use ? v.z : 0.f, use ? v.w : 0.f);
                    }
                }
#pragma unroll
                for (int u = 0; u < QR_QUAD_BATCH; ++u) {
                    sv[0].x += x[u][0].x; sv[1].x += x[u][0].y; sv[2].x += x[u][0].z; sv[3].x += x[u][0].w;
                    sv[0].y += x[u][1].x; sv[1].y += x[u][1].y; sv[2].y += x[u][1].z; sv[3].y += x[u][1].w;
                    sv[0].z += x[u][2].x; sv[1].z += x[u][2].y; sv[2].z += x[u][2].z; sv[3].z += x[u][2].w;
                    sv[0].w += x[u][3].x; sv[1].w += x[u][3].y; sv[2].w += x[u][3].z; sv[3].w += x[u][3].w;
                }
            }
        } else {
            for (int c = sl; c < M.nq; c += 4 * S) {
                float x[4][4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int cu = c + S * u;
#pragma unroll
                    for (int j = 0; j < 4; ++j) x[u][j] = ((GF)(qplane(M, cu < M.nq ? cu : M.nq - 1, j) + col))[0];
                }
                // all 16 loads issued before any is used (the compiler would
                // otherwise move each into the branch of its own condition)
                asm volatile("" : "+v"(x[0][0]), "+v"(x[0][1]), "+v"(x[0][2]), "+v"(x[0][3]), "+v"(x[1][0]),
                                  "+v"(x[1][1]), "+v"(x[1][2]), "+v"(x[1][3]), "+v"(x[2][0]), "+v"(x[2][1]),
                                  "+v"(x[2][2]), "+v"(x[2][3]), "+v"(x[3][0]), "+v"(x[3][1]), "+v"(x[3][2]),
                                  "+v"(x[3][3]));
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int j = 0; j < 4; ++j) x[u][j] = (c + S * u < M.nq && j < r) ? x[u][j] : 0.0f;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    sv[0].x += x[u][0]; sv[0].y += x[u][1]; sv[0].z += x[u][2]; sv[0].w += x[u][3];
                }
            }
        }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) s_q[c][t] = sv[c];
    __syncthreads();
    if (t < 64) {
        // lanes 0..15 of wave 0 each add one Gram entry's 16 slices (in slice
        // order, as one thread would), lane 0 builds T from them
        double g = 0.0;
        if (t < 16) {
#pragma unroll
            for (int k = 0; k < 16; ++k) g += s_g[k][t];
        }
        double G[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) G[i] = readlane_any(g, i);
        if (t == 0) {
            double T[16];
            gram_schmidt_coeffs(G, r, T);
#pragma unroll
            for (int i = 0; i < 16; ++i) s_T[i] = T[i];
            if (lwg == 0) {
#pragma unroll
                for (int i = 0; i < 16; ++i) M.tmat[i] = T[i];
            }
        }
    }
    __syncthreads();
    // one thread per column: column c of group g adds its S slices in order
    const int ncol = quad ? 4 : 1;
    for (int idx = t; idx < QC * ncol; idx += PS_THREADS) {
        const int g = idx % QC, c = idx / QC;
        const int cc = (lwg * QC + g) * ncol + c;
        if (cc >= m) continue;
        double4 a = s_q[c][g];
        for (int k = 1; k < S; ++k) {
            const double4 x = s_q[c][k * QC + g];
            a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
        }
        const double sa[4] = {a.x, a.y, a.z, a.w};
#pragma unroll 1
        for (int j = 0; j < r; ++j) {
            double v = 0.0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i <= j) v += sa[i] * s_T[i * 4 + j];
            M.q[static_cast<long long>(j) * m + cc] = static_cast<float>(v);
        }
    }
}

// ------------------------------------------------------------------ psgd_out

// What the output pass does with a row:
//   OUT_EXPLICIT     M from (mem, grad); out = P^ Q'^T, mem = M - out, P^ into p
//   OUT_DEFERRED     out = P^ Q'^T and P^ into p only: mem already holds M (the
//                    first pass stored it) and keeps it as the deferred memory
//   OUT_MATERIALIZE  mem = M_prev - P^_prev Q_prev^T with P^_prev read from p
//                    (rank prank): the deferred memory written out
enum OutMode { OUT_EXPLICIT, OUT_DEFERRED, OUT_MATERIALIZE };

// Rows [r0, r1) of one matrix, one column strip at a time (Q of the strip in
// registers); loads of ROW_GROUP rows are issued together.  STREAM marks the
// last reads of mem/grad and the writes of mem/out non-temporal, for batches
// far larger than the last-level cache.
template <bool BF16, int VEC, bool STREAM, int MODE>
__device__ __forceinline__ void out_rows(const PsMat& M, float eta, int r0, int r1, int s0 = 0, int s1 = 1 << 30) {
    constexpr bool LOAD = MODE != OUT_DEFERRED;   // reads mem
    const int n = M.n, m = M.m, r = MODE == OUT_MATERIALIZE ? M.prank : M.rank;
    // P and T were written by earlier kernels and are only read here: the
    // constant address space gives scalar loads that no store has to wait for
    typedef const __attribute__((address_space(4))) double* ConstD;
    typedef const __attribute__((address_space(4))) float* ConstF;
    const ConstD tm = (ConstD)(M.tmat);
    const ConstF pr = (ConstF)(M.praw);
    // P^ = P T in float64: T's entries scale like 1 / sigma_min(P), so float32
    // T would scale its rounding by the condition number of P
    double T[10];   // upper triangle, column by column: T[a][j] (a <= j) at j (j + 1) / 2 + a
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int a = 0; a <= j; ++a) T[j * (j + 1) / 2 + a] = tm[a * 4 + j];
    const int ns = min(s1, nstrips_of(m));
    for (int strip = s0; strip < ns; ++strip) {
        const int col0 = strip * (PS_THREADS * VEC) + threadIdx.x * VEC;
        const bool active = col0 < m;
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
        const bool write_p = MODE != OUT_MATERIALIZE && M.p != nullptr && strip == 0 &&
                             threadIdx.x < static_cast<unsigned>(r);
        const int colc = active ? col0 : 0;
        for (int i0 = r0; i0 < r1; i0 += ROW_GROUP) {
            float mv[ROW_GROUP][VEC];
            if constexpr (LOAD) {
#pragma unroll
                for (int u = 0; u < ROW_GROUP; ++u) {
                    const int row = min(i0 + u, r1 - 1);
                    const long long e = static_cast<long long>(row) * m + colc;
                    if constexpr (MODE == OUT_MATERIALIZE) {
                        if constexpr (VEC == 4) {
                            const float4 a = reinterpret_cast<const float4*>(M.mem)[e / 4];
                            mv[u][0] = a.x; mv[u][1] = a.y; mv[u][2] = a.z; mv[u][3] = a.w;
                        } else {
                            mv[u][0] = M.mem[e];
                        }
                    } else {
                        load_Mv<BF16, VEC, STREAM>(M, eta, e, mv[u]);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < ROW_GROUP; ++u) {
                const int i = i0 + u;
                if (i >= r1) break;
                float ph[4];
                if constexpr (MODE == OUT_MATERIALIZE) {
                    prev_phat_row(M, i, ph);
                } else {
                    const float prv[4] = {pr[4 * i], pr[4 * i + 1], pr[4 * i + 2], pr[4 * i + 3]};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        double v = 0.0;
#pragma unroll
                        for (int a = 0; a <= j; ++a) v = fma(static_cast<double>(prv[a]), T[j * (j + 1) / 2 + a], v);
                        ph[j] = static_cast<float>(v);
                    }
                }
                if (write_p) {
                    float mine = ph[0];
#pragma unroll
                    for (int j = 1; j < 4; ++j) mine = (threadIdx.x == static_cast<unsigned>(j)) ? ph[j] : mine;
                    M.p[static_cast<long long>(threadIdx.x) * n + i] = mine;
                }
                if (!active) continue;
                const long long e = static_cast<long long>(i) * m + col0;
                float o[VEC], nm[VEC];
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    // the sum that residual1 forms, kept for the decoded output
                    float sacc = 0.0f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) sacc = fmaf(ph[j], qv[v][j], sacc);
                    o[v] = sacc;
                    nm[v] = LOAD ? mv[u][v] - sacc : 0.0f;
                }
                constexpr bool WRITE_OUT = MODE != OUT_MATERIALIZE, WRITE_MEM = MODE != OUT_DEFERRED;
                if constexpr (VEC == 4) {
                    const float4 ov = make_float4(o[0], o[1], o[2], o[3]), mv4 = make_float4(nm[0], nm[1], nm[2], nm[3]);
                    float4* const op = reinterpret_cast<float4*>(M.out) + e / 4;
                    float4* const mp = reinterpret_cast<float4*>(M.mem) + e / 4;
                    if constexpr (STREAM) {
                        if (WRITE_OUT && M.out) store_stream(op, ov);
                        if (WRITE_MEM) store_stream(mp, mv4);
                    } else {
                        if (WRITE_OUT && M.out) *op = ov;
                        if (WRITE_MEM) *mp = mv4;
                    }
                } else {
                    if (WRITE_OUT && M.out) M.out[e] = o[0];
                    if (WRITE_MEM) M.mem[e] = nm[0];
                }
            }
        }
    }
}

// Decode + residual for every matrix of the table (MODE: OutMode): workgroup
// b takes its balanced share of rows.
template <bool BF16, bool STREAM, int MODE>
__global__ __launch_bounds__(PS_THREADS) void psgd_out(const PsBatch B) {
    const int b = blockIdx.x, G = B.gout;
    const long long E = B.eall;
    const long long s_lo = share_lo(E, G, b), s_hi = share_lo(E, G, b + 1);
    for (int i = mat_of_entry(B, 0, B.count, s_lo); i < B.count; ++i) {
        const PsMat M = mat_at(B, i);
        if (M.off >= s_hi) break;
        if (MODE == OUT_MATERIALIZE && M.prank == 0) continue;   // mem holds the memory already
        int r0, r1;
        rows_in_share(M, s_lo, s_hi, r0, r1);
        if (r0 >= r1) continue;
        if (M.m % 4 == 0)
            out_rows<BF16, 4, STREAM, MODE>(M, B.eta, r0, r1);
        else
            out_rows<BF16, 1, STREAM, MODE>(M, B.eta, r0, r1);
    }
}

// Output pass of the deferred step: out = P^ Q'^T and P^ into p, nothing
// read but P, T and Q'.  A write-only pass runs fastest as many short
// workgroups dispatched in address order (the writes sweep memory front to
// back) rather than as a persistent grid of long contiguous shares.  Tile t
// is DEC_ROWS rows x one column strip of one matrix; the tiles of a matrix
// start at its dbeg, in row-major order of (row block, strip).  Workgroup b
// takes tiles b, b + grid, ... (one each unless the batch has more than
// DEC_GRID_MAX tiles).
constexpr int DEC_ROWS = ROW_GROUP;
constexpr long long DEC_GRID_MAX = 1LL << 30;

template <bool STREAM>
__global__ __launch_bounds__(PS_THREADS) void psgd_decode(const PsBatch B, long long ntiles) {
    const MatTable T = mat_table(B);
    typedef const __attribute__((address_space(4))) int* ConstI;
    for (long long t = blockIdx.x; t < ntiles; t += gridDim.x) {
        // last matrix whose first tile is <= t: the map gives the matrix of
        // tile 64 (t / 64), and at most 63 tiles lie between
        int lo = ((ConstI)(B.dmap))[t >> 6];
        while (lo + 1 < B.count && T[lo + 1].dbeg <= t) ++lo;
        const PsMat M = mat_at(B, lo);
        const long long lt = t - M.dbeg;
        const int ns = nstrips_of(M.m);
        const int strip = static_cast<int>(lt % ns);
        const int r0 = static_cast<int>((lt / ns) * DEC_ROWS);
        const int r1 = min(M.n, r0 + DEC_ROWS);
        if (M.m % 4 == 0)
            out_rows<false, 4, STREAM, OUT_DEFERRED>(M, B.eta, r0, r1, strip, strip + 1);
        else
            out_rows<false, 1, STREAM, OUT_DEFERRED>(M, B.eta, r0, r1, strip, strip + 1);
    }
}

// ------------------------------------------------------------------ host side

int nstrips_host(int m) {
    const int w = (m % 4 == 0) ? PS_THREADS * 4 : PS_THREADS;
    return (m + w - 1) / w;
}

// Class of an n x m matrix: a fused class by row length, the small class,
// or the split path.
struct PqClass { int max_m, threads, blocks_per_cu; };
constexpr PqClass PQ_CLASS[PQ_CLASSES] = {{1024, 256, 3}, {2048, 512, 2}, {4096, 1024, 1}, {6144, 768, 1},
                                          {8192, 1024, 1}};

int shape_class(int n, int m) {
    if (m % 4 == 0)
        for (int c = 0; c < PQ_CLASSES; ++c)
            if (m <= PQ_CLASS[c].max_m) return c;
    if (n <= SMALL_MAX_N && m <= SMALL_MAX_M) return SMALL_CLASS;
    return SPLIT_CLASS;
}

// How the matrices are grouped and partitioned.  Shapes only (not ranks, not
// the gradient dtype): the workspace query and the step make the same plan.
struct PlanMat {
    int idx;            // index in the caller's array
    long long off;      // first entry within the batch
    long long poff;     // fused classes: first partition unit within the batch
    int nq, ng;         // partial counts
    int begin_p, begin_q, begin_r;
    long long dbeg;     // first psgd_decode tile
    int qs;             // psgd_qreduce threads per column
    size_t ws_off;      // workspace offset of this matrix's scratch
};
struct PlanBatch {
    int first, count;                  // into Plan::mats
    size_t tbl_off;                    // workspace offset of the device table
    int cbeg[PQ_CLASSES + 3];
    int cgrid[PQ_CLASSES];
    long long cbase[PQ_CLASSES], cent[PQ_CLASSES];
    long long eall;
    int gout;
    int np, nq, nr;                    // psgd_p / psgd_q / psgd_qreduce grids
    long long nd;                      // psgd_decode grid
};
struct Plan {
    std::vector<PlanMat> mats;
    std::vector<PlanBatch> batches;
    size_t ws_bytes = 0;
};

size_t ws_round(size_t x) { return round_up(x, 256); }

// Entries of the decode's tile map: one per 64 tiles.
size_t dmap_len(long long nd) { return static_cast<size_t>((nd + 63) / 64); }

// Threads per column group in psgd_qreduce: the smallest power of two that
// leaves each thread at most QR_PER_THREAD partial loads (a thread covering
// 4 columns loads 4 values per partial: QR_PER_THREAD / 4 partials), at most 64.
int qr_slices(int nq, int cols_per_thread) {
    const int per = cols_per_thread == 4 ? QR_PER_THREAD / 4 : QR_PER_THREAD;
    int sl = 1;
    while (sl < 64 && sl * per < nq) sl *= 2;
    return sl;
}

// Grid of a balanced pass over e entries whose widest row has mmax entries:
// every share is at least one such row, so a workgroup owns a row of every
// matrix its share overlaps.
int balanced_grid(long long e, long long mmax, int gmax) {
    return e > 0 ? static_cast<int>(std::min<long long>(gmax, std::max<long long>(1, e / mmax))) : 0;
}

Plan make_plan(const gc_mat* mats, int nmats) {
    Plan P;
    size_t o = 0;
    for (int i = 0; i < nmats;) {
        const int j = std::min(nmats, i + PS_MAXB);
        std::vector<int> idx;
        for (int k = i; k < j; ++k) idx.push_back(k);
        std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) {
            return shape_class(mats[a].n, mats[a].m) < shape_class(mats[b].n, mats[b].m);
        });
        PlanBatch pb{};
        pb.first = static_cast<int>(P.mats.size());
        pb.count = j - i;
        int ccount[PQ_CLASSES + 2] = {};
        int cmax[PQ_CLASSES];
        for (int c = 0; c < PQ_CLASSES; ++c) cmax[c] = 1;
        for (int a : idx) {
            const int c = shape_class(mats[a].n, mats[a].m);
            ++ccount[c];
            if (c < PQ_CLASSES) {
                pb.cent[c] += static_cast<long long>(mats[a].n) * (mats[a].m + PQ_ROW_COST);
                cmax[c] = std::max(cmax[c], mats[a].m + PQ_ROW_COST);
            }
        }
        pb.cbeg[0] = 0;
        for (int c = 0; c <= SPLIT_CLASS; ++c) pb.cbeg[c + 1] = pb.cbeg[c] + ccount[c];
        long long base = 0;
        for (int c = 0; c < PQ_CLASSES; ++c) {
            pb.cbase[c] = base;
            base += pb.cent[c];
            pb.cgrid[c] = balanced_grid(pb.cent[c], static_cast<long long>(cmax[c]) * PQ_ROWS_MIN,
                                        CUS * PQ_CLASS[c].blocks_per_cu);
            // psgd_pq addresses a workgroup's share with 32-bit buffer offsets
            // (plus the row group it loads ahead, past the share's last row,
            // and the 2^31 idle-lane offset): keep every share below
            // PQ_SHARE_MAX_ENTRIES units (a share holds fewer entries than
            // units), running extra workgroups in further rounds if a class
            // is that large
            if (pb.cent[c] > 0) {
                const long long need = (pb.cent[c] + PQ_SHARE_MAX_ENTRIES - 1) / PQ_SHARE_MAX_ENTRIES;
                pb.cgrid[c] = static_cast<int>(std::max<long long>(pb.cgrid[c], need));
            }
        }
        long long eall = 0, pall = 0;
        for (int a : idx) {
            PlanMat pm{};
            pm.idx = a;
            pm.off = eall;
            const int n = mats[a].n, m = mats[a].m;
            const int c = shape_class(n, m);
            if (c == SMALL_CLASS) {
                pm.nq = pm.ng = 1;     // one workgroup: one partial of each
            } else if (c < PQ_CLASSES) {
                pm.poff = pall;
                pall += static_cast<long long>(n) * (m + PQ_ROW_COST);
                const long long E = pb.cent[c], rel = pm.poff - pb.cbase[c];
                const int G = pb.cgrid[c];
                pm.nq = pm.ng = owner_of(rel + static_cast<long long>(n - 1) * (m + PQ_ROW_COST), E, G) -
                                owner_of(rel, E, G) + 1;
            } else {
                pm.nq = (n + Q_ROWS - 1) / Q_ROWS;
                pm.ng = (n + P_ROWS_WG - 1) / P_ROWS_WG;
                pm.begin_p = pb.np;
                pb.np += pm.ng;
                pm.begin_q = pb.nq;
                pb.nq += nstrips_host(m) * pm.nq;
            }
            const int cpt = m % 4 == 0 ? 4 : 1;     // psgd_qreduce columns per thread
            pm.qs = qr_slices(pm.nq, cpt);
            pm.begin_r = pb.nr;
            const int qc = PS_THREADS / pm.qs * cpt;
            pb.nr += (m + qc - 1) / qc;
            pm.dbeg = pb.nd;
            pb.nd += static_cast<long long>((n + DEC_ROWS - 1) / DEC_ROWS) * nstrips_host(m);
            pm.ws_off = o;
            o += ws_round(static_cast<size_t>(n) * 16);                       // praw
            o += ws_round(static_cast<size_t>(pm.ng) * 16 * 8);               // gpart
            o += ws_round(static_cast<size_t>(pm.nq) * m * 16);               // qpart
            o += 256;                                                          // tmat
            eall += static_cast<long long>(n) * m;
            P.mats.push_back(pm);
        }
        pb.eall = eall;
        // the device table, then the psgd_qreduce workgroup -> matrix map and
        // the psgd_decode tile -> matrix map (one entry per 64 tiles)
        pb.tbl_off = o;
        o += ws_round(static_cast<size_t>(pb.count) * sizeof(PsMat) +
                      static_cast<size_t>(pb.nr + dmap_len(pb.nd)) * sizeof(int));
        const long long gmax = eall <= OUT_TWO_ROUNDS_MAX ? 2LL * OUT_GRID_MAX : OUT_GRID_MAX;
        pb.gout = static_cast<int>(std::min<long long>(gmax, std::max<long long>(1, eall / 1024)));
        P.batches.push_back(pb);
        i = j;
    }
    P.ws_bytes = o;
    return P;
}

// no_grad: the materialize call, which reads neither grad nor rank.
int validate_mat(const gc_mat& a, int i, int dtype, const std::string& fn, bool no_grad) {
    const std::string pre = fn + ": mats[" + std::to_string(i) + "]: ";
    if ((!no_grad && !a.grad) || !a.mem || !a.q) return fail(GC_ERR_ARG, pre + "null grad/mem/q");
    if (a.n < 1 || a.m < 1) return fail(GC_ERR_ARG, pre + "n and m must be >= 1");
    if (static_cast<long long>(a.n) * a.m > INT32_MAX) return fail(GC_ERR_ARG, pre + "n*m exceeds INT32_MAX");
    if (!no_grad && (a.rank < 1 || a.rank > 4 || a.rank > a.n || a.rank > a.m))
        return fail(GC_ERR_ARG, pre + "rank must be in [1, min(4, n, m)]");
    if (no_grad) {
        // only mem, q and p are touched (q and p read, first prev_rank columns)
        if (!aligned16(a.mem) || !aligned16(a.q) || (a.p && !aligned16(a.p)))
            return fail(GC_ERR_ARG, pre + "device pointers must be 16-byte aligned");
        const size_t mb = static_cast<size_t>(a.n) * a.m * 4;
        const size_t qb = static_cast<size_t>(a.m) * 16, pb = static_cast<size_t>(a.n) * 16;
        if (overlaps(a.q, qb, a.mem, mb) || (a.p && overlaps(a.p, pb, a.mem, mb)))
            return fail(GC_ERR_ARG, pre + "buffers overlap");
        return GC_OK;
    }
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

// Host image of a batch's device table: the matrix entries, then the
// psgd_qreduce map (workgroup b -> the matrix whose Q columns it reduces).
struct TableImage {
    std::vector<PsMat> mats;
    std::vector<int> rmap;
    std::vector<int> dmap;
};

// The table and map go to the device in stream order, as one copy.  From
// pageable memory the runtime stages the bytes before returning, so the
// image may go out of scope.
int copy_table(const PsBatch& B, const TableImage& img, hipStream_t s) {
    const size_t tb = img.mats.size() * sizeof(PsMat), mb = img.rmap.size() * sizeof(int);
    const size_t db = img.dmap.size() * sizeof(int);
    std::vector<char> buf(tb + mb + db);
    std::memcpy(buf.data(), img.mats.data(), tb);
    if (mb) std::memcpy(buf.data() + tb, img.rmap.data(), mb);
    if (db) std::memcpy(buf.data() + tb + mb, img.dmap.data(), db);
    const hipError_t e = hipMemcpyAsync(const_cast<PsMat*>(B.tbl), buf.data(), buf.size(), hipMemcpyHostToDevice, s);
    if (e != hipSuccess)
        return fail(GC_ERR_HIP, std::string("PowerSGD matrix table copy: ") + hipGetErrorString(e));
    return GC_OK;
}

// First passes and Q reduction of one batch.
template <bool BF16, bool DEF>
int launch_encode(const PsBatch& B, const PlanBatch& pb, hipStream_t s) {
    int rc;
    int fused = 0, team_grid = 0;
    for (int c = 0; c < TEAM_CLASSES; ++c) {
        fused += B.cbeg[c + 1] > B.cbeg[c] ? 1 : 0;
        team_grid += team_wgs(B.cgrid[c], c);
    }
    const int nsmall = B.cbeg[SPLIT_CLASS] - B.cbeg[SMALL_CLASS];
    fused += nsmall > 0 ? 1 : 0;
    const bool teams = fused >= 2 && B.eall <= TEAM_MAX_ENTRIES;
    if (teams) {
        // small group, several classes: one launch (the classes' passes side by
        // side, the small matrices after them)
        TimedLaunch tl("psgd_pq", s);
        psgd_pq_teams<BF16, DEF><<<team_grid + nsmall, TEAM_NT, 0, s>>>(B);
        if ((rc = check_launch("psgd_pq")) != GC_OK) return rc;
    } else if (nsmall > 0) {
        TimedLaunch tl("psgd_pq", s);
        psgd_small<BF16, DEF><<<nsmall, SMALL_THREADS, 0, s>>>(B);
        if ((rc = check_launch("psgd_pq")) != GC_OK) return rc;
    }
    for (int c = teams ? TEAM_CLASSES : 0; c < PQ_CLASSES; ++c) {
        if (B.cbeg[c + 1] == B.cbeg[c]) continue;
        TimedLaunch tl("psgd_pq", s);
        const unsigned g = static_cast<unsigned>(B.cgrid[c]);
        switch (c) {
            case 0: psgd_pq<BF16, 0, DEF><<<g, PqShape<0>::NT, 0, s>>>(B); break;
            case 1: psgd_pq<BF16, 1, DEF><<<g, PqShape<1>::NT, 0, s>>>(B); break;
            case 2: psgd_pq<BF16, 2, DEF><<<g, PqShape<2>::NT, 0, s>>>(B); break;
            case 3: psgd_pq<BF16, 3, DEF><<<g, PqShape<3>::NT, 0, s>>>(B); break;
            default: psgd_pq<BF16, 4, DEF><<<g, PqShape<4>::NT, 0, s>>>(B); break;
        }
        if ((rc = check_launch("psgd_pq")) != GC_OK) return rc;
    }
    const int s0 = B.cbeg[SPLIT_CLASS];
    if (s0 < B.count) {
        {
            TimedLaunch tl("psgd_p", s);
            psgd_p<BF16, DEF><<<pb.np, PS_THREADS, 0, s>>>(B, s0, B.count);
            if ((rc = check_launch("psgd_p")) != GC_OK) return rc;
        }
        {
            TimedLaunch tl("psgd_q", s);
            psgd_q<BF16, DEF><<<pb.nq, PS_THREADS, 0, s>>>(B, s0, B.count);
            if ((rc = check_launch("psgd_q")) != GC_OK) return rc;
        }
    }
    {
        TimedLaunch tl("psgd_qreduce", s);
        psgd_qreduce<<<pb.nr, PS_THREADS, 0, s>>>(B);
        if ((rc = check_launch("psgd_qreduce")) != GC_OK) return rc;
    }
    return GC_OK;
}

// Output pass of one batch.
template <bool BF16, bool DEF>
int launch_decode(const PsBatch& B, const PlanBatch& pb, hipStream_t s) {
    int rc;
    {
        const char* name = DEF ? "psgd_decode" : "psgd_out";
        TimedLaunch tl(name, s);
        // streaming accesses only pay when the pass moves far more than the
        // 256 MB last-level cache holds
        const double bytes_per_entry = DEF ? 4.0 : (BF16 ? 14.0 : 16.0);
        const bool stream = static_cast<double>(B.eall) * bytes_per_entry > STREAM_MIN_BYTES;
        if constexpr (DEF) {
            const unsigned grid = static_cast<unsigned>(std::min<long long>(pb.nd, DEC_GRID_MAX));
            if (stream) psgd_decode<true><<<grid, PS_THREADS, 0, s>>>(B, pb.nd);
            else psgd_decode<false><<<grid, PS_THREADS, 0, s>>>(B, pb.nd);
        } else if (stream) {
            psgd_out<BF16, true, OUT_EXPLICIT><<<B.gout, PS_THREADS, 0, s>>>(B);
        } else {
            psgd_out<BF16, false, OUT_EXPLICIT><<<B.gout, PS_THREADS, 0, s>>>(B);
        }
        if ((rc = check_launch(name)) != GC_OK) return rc;
    }
    return GC_OK;
}

// Launches the kernels of one batch: with PH_ENCODE the fused classes, the
// split path and the Q reduction (P^ and Q' complete); with PH_DECODE the
// output pass.  DEF: the deferred step (the first passes rebuild the
// previous residual and store M in mem; the output pass writes out and P^
// only).
enum Phase { PH_ENCODE = 1, PH_DECODE = 2, PH_ALL = 3 };

template <bool BF16, bool DEF>
int launch_batch(const PsBatch& B, const PlanBatch& pb, hipStream_t s, int phases = PH_ALL) {
    int rc;
    if (phases & PH_ENCODE) {
        if ((rc = launch_encode<BF16, DEF>(B, pb, s)) != GC_OK) return rc;
    }
    if (phases & PH_DECODE) {
        if ((rc = launch_decode<BF16, DEF>(B, pb, s)) != GC_OK) return rc;
    }
    return GC_OK;
}

template <bool BF16, bool DEF>
int run_batch(const PsBatch& B, const PlanBatch& pb, const TableImage& tbl, hipStream_t s) {
    const int rc = copy_table(B, tbl, s);
    return rc != GC_OK ? rc : launch_batch<BF16, DEF>(B, pb, s);
}

int launch_any(bool bf16, bool def, const PsBatch& B, const PlanBatch& pb, hipStream_t s, int phases) {
    if (def) return bf16 ? launch_batch<true, true>(B, pb, s, phases) : launch_batch<false, true>(B, pb, s, phases);
    return bf16 ? launch_batch<true, false>(B, pb, s, phases) : launch_batch<false, false>(B, pb, s, phases);
}

// mem = M_prev - P^_prev Q_prev^T for the matrices with prank > 0.
int run_materialize(const PsBatch& B, const TableImage& tbl, hipStream_t s) {
    int rc;
    if ((rc = copy_table(B, tbl, s)) != GC_OK) return rc;
    TimedLaunch tl("psgd_materialize", s);
    psgd_out<false, false, OUT_MATERIALIZE><<<B.gout, PS_THREADS, 0, s>>>(B);
    return check_launch("psgd_materialize");
}

enum StepKind { STEP_EXPLICIT, STEP_DEFERRED, STEP_MATERIALIZE };

// Validation, plan, table and launches shared by the three PowerSGD calls.
// prank: [host] previous ranks (deferred and materialize calls), else NULL.
// One batch of a recorded step: its launch parameters (the table is in ws).
struct PlanEntry {
    PsBatch B;
    PlanBatch pb;
};

// rec != NULL: record the step instead of running it (tables copied, no launch).
int powersgd_call(const char* fn, StepKind kind, const gc_mat* mats, const int32_t* prank, int nmats,
                  int grad_dtype, float eta, void* ws, size_t ws_bytes, hipStream_t s,
                  std::vector<PlanEntry>* rec = nullptr) {
    const std::string f(fn);
    if (!mats || nmats < 1) return fail(GC_ERR_ARG, f + ": need mats and nmats >= 1");
    if (kind != STEP_EXPLICIT && !prank) return fail(GC_ERR_ARG, f + ": null prev_rank");
    if (grad_dtype != GC_F32 && grad_dtype != GC_BF16)
        return fail(GC_ERR_DTYPE, f + ": grad_dtype must be GC_F32 or GC_BF16");
    if (!ws) return fail(GC_ERR_ARG, f + ": null workspace");
    if (!aligned16(ws)) return fail(GC_ERR_ARG, f + ": workspace must be 16-byte aligned");
    for (int i = 0; i < nmats; ++i) {
        const int rc = validate_mat(mats[i], i, grad_dtype, f, kind == STEP_MATERIALIZE);
        if (rc != GC_OK) return rc;
        if (kind != STEP_EXPLICIT) {
            const gc_mat& a = mats[i];
            const std::string pre = f + ": mats[" + std::to_string(i) + "]: ";
            if (!a.p) return fail(GC_ERR_ARG, pre + "p is required (it keeps P^ for the deferred memory)");
            if (prank[i] < 0 || prank[i] > 4 || prank[i] > a.n || prank[i] > a.m)
                return fail(GC_ERR_ARG, pre + "prev_rank must be in [0, min(4, n, m)]");
        }
    }
    const Plan P = make_plan(mats, nmats);
    if (ws_bytes < P.ws_bytes)
        return fail(GC_ERR_WORKSPACE, f + ": workspace smaller than gc_powersgd_workspace_bytes");

    char* wp = static_cast<char*>(ws);
    for (const PlanBatch& pb : P.batches) {
        PsBatch B{};
        B.tbl = reinterpret_cast<const PsMat*>(wp + pb.tbl_off);
        B.rmap = reinterpret_cast<const int*>(wp + pb.tbl_off + static_cast<size_t>(pb.count) * sizeof(PsMat));
        B.dmap = B.rmap + pb.nr;
        B.count = pb.count;
        B.eta = eta;
        for (int c = 0; c < PQ_CLASSES + 3; ++c) B.cbeg[c] = pb.cbeg[c];
        for (int c = 0; c < PQ_CLASSES; ++c) {
            B.cgrid[c] = pb.cgrid[c];
            B.cbase[c] = pb.cbase[c];
            B.cent[c] = pb.cent[c];
        }
        B.eall = pb.eall;
        B.gout = pb.gout;
        TableImage tbl;
        tbl.mats.resize(pb.count);
        tbl.rmap.resize(pb.nr);
        tbl.dmap.resize(dmap_len(pb.nd));
        for (size_t g = 0, k = 0; g < tbl.dmap.size(); ++g) {
            const long long t0 = static_cast<long long>(g) * 64;
            while (k + 1 < static_cast<size_t>(pb.count) && P.mats[pb.first + k + 1].dbeg <= t0) ++k;
            tbl.dmap[g] = static_cast<int>(k);
        }
        for (int k = 0; k < pb.count; ++k) {
            const PlanMat& pm = P.mats[pb.first + k];
            const gc_mat& a = mats[pm.idx];
            const int rend = k + 1 < pb.count ? P.mats[pb.first + k + 1].begin_r : pb.nr;
            for (int b = pm.begin_r; b < rend; ++b) tbl.rmap[b] = k;
            char* base = wp + pm.ws_off;
            PsMat& M = tbl.mats[k];
            M.grad = a.grad;
            M.mem = a.mem;
            M.q = a.q;
            M.p = a.p;
            M.out = a.out;
            M.praw = reinterpret_cast<float*>(base);
            base += ws_round(static_cast<size_t>(a.n) * 16);
            M.gpart = reinterpret_cast<double*>(base);
            base += ws_round(static_cast<size_t>(pm.ng) * 16 * 8);
            M.qpart = reinterpret_cast<float*>(base);
            base += ws_round(static_cast<size_t>(pm.nq) * a.m * 16);
            M.tmat = reinterpret_cast<double*>(base);
            M.off = pm.off;
            M.poff = pm.poff;
            M.rcost = a.m + PQ_ROW_COST;
            M.n = a.n;
            M.m = a.m;
            M.rank = kind == STEP_MATERIALIZE ? 1 : a.rank;
            M.nq = pm.nq;
            M.ng = pm.ng;
            M.begin_p = pm.begin_p;
            M.begin_q = pm.begin_q;
            M.begin_r = pm.begin_r;
            M.dbeg = pm.dbeg;
            M.qs = pm.qs;
            M.prank = kind == STEP_EXPLICIT ? 0 : prank[pm.idx];
        }
        int rc;
        if (rec) {
            if ((rc = copy_table(B, tbl, s)) != GC_OK) return rc;
            rec->push_back(PlanEntry{B, pb});
            continue;
        }
        if (kind == STEP_MATERIALIZE) rc = run_materialize(B, tbl, s);
        else if (kind == STEP_DEFERRED)
            rc = grad_dtype == GC_BF16 ? run_batch<true, true>(B, pb, tbl, s) : run_batch<false, true>(B, pb, tbl, s);
        else
            rc = grad_dtype == GC_BF16 ? run_batch<true, false>(B, pb, tbl, s) : run_batch<false, false>(B, pb, tbl, s);
        if (rc != GC_OK) return rc;
    }
    return GC_OK;
}

// Host plan buffer: a header, then one PlanEntry per batch (copied with
// memcpy: the caller's buffer needs no alignment).
constexpr unsigned long long PLAN_MAGIC = 0x31504e414c504347ULL;   // "GCPLANP1"
struct PlanHeader {
    unsigned long long magic;
    int nbatches;
    int grad_dtype;
    int deferred;
    int pad;
    const void* ws;
    size_t ws_bytes;
};

size_t plan_bytes_for(int nmats) {
    const int nb = (nmats + PS_MAXB - 1) / PS_MAXB;
    return sizeof(PlanHeader) + static_cast<size_t>(nb) * sizeof(PlanEntry);
}

// Launches the given phases of every batch of a plan.  Every matrix has its
// own workspace region (P, partials, T), so all encode launches may run
// before all decode launches.
int run_plan(const char* fn, const void* plan, size_t plan_bytes, float eta, void* ws, int phases, hipStream_t s) {
    if (!plan || plan_bytes < sizeof(PlanHeader)) return fail(GC_ERR_ARG, std::string(fn) + ": null or short plan");
    PlanHeader h;
    std::memcpy(&h, plan, sizeof(h));
    if (h.magic != PLAN_MAGIC || h.nbatches < 1 || h.nbatches > (INT32_MAX / PS_MAXB) + 1)
        return fail(GC_ERR_ARG, std::string(fn) + ": not a plan written by gc_powersgd_plan");
    if (plan_bytes < sizeof(PlanHeader) + static_cast<size_t>(h.nbatches) * sizeof(PlanEntry))
        return fail(GC_ERR_ARG, std::string(fn) + ": plan buffer shorter than the plan");
    if (ws != h.ws) return fail(GC_ERR_ARG, std::string(fn) + ": ws is not the workspace the plan was made with");
    const char* in = static_cast<const char*>(plan) + sizeof(PlanHeader);
    for (int b = 0; b < h.nbatches; ++b) {
        PlanEntry e;
        std::memcpy(&e, in + static_cast<size_t>(b) * sizeof(PlanEntry), sizeof(e));
        e.B.eta = eta;
        const int rc = launch_any(h.grad_dtype == GC_BF16, h.deferred != 0, e.B, e.pb, s, phases);
        if (rc != GC_OK) return rc;
    }
    return GC_OK;
}

}  // namespace
}  // namespace gc

using namespace gc;

extern "C" {

size_t gc_powersgd_workspace_bytes(const gc_mat* mats, int nmats) {
    if (!mats || nmats < 1) return 0;
    for (int i = 0; i < nmats; ++i) {
        const gc_mat& a = mats[i];
        if (a.n < 1 || a.m < 1 || static_cast<long long>(a.n) * a.m > INT32_MAX) return 0;
    }
    return make_plan(mats, nmats).ws_bytes;
}

int gc_powersgd_ef_step(const gc_mat* mats, int nmats, int grad_dtype, float eta,
                        void* ws, size_t ws_bytes, void* stream) {
    return powersgd_call("gc_powersgd_ef_step", STEP_EXPLICIT, mats, nullptr, nmats, grad_dtype, eta, ws, ws_bytes,
                         static_cast<hipStream_t>(stream));
}

int gc_powersgd_ef_step_deferred(const gc_mat* mats, const int32_t* prev_rank, int nmats, int grad_dtype,
                                 float eta, void* ws, size_t ws_bytes, void* stream) {
    return powersgd_call("gc_powersgd_ef_step_deferred", STEP_DEFERRED, mats, prev_rank, nmats, grad_dtype, eta, ws,
                         ws_bytes, static_cast<hipStream_t>(stream));
}

size_t gc_powersgd_plan_bytes(const gc_mat* mats, int nmats) {
    if (!mats || nmats < 1) return 0;
    return plan_bytes_for(nmats);
}

int gc_powersgd_plan(const gc_mat* mats, const int32_t* prev_rank, int nmats, int grad_dtype, void* plan,
                     size_t plan_bytes, void* ws, size_t ws_bytes, void* stream) {
    if (!plan) return fail(GC_ERR_ARG, "gc_powersgd_plan: null plan buffer");
    if (!mats || nmats < 1) return fail(GC_ERR_ARG, "gc_powersgd_plan: need mats and nmats >= 1");
    if (plan_bytes < plan_bytes_for(nmats))
        return fail(GC_ERR_ARG, "gc_powersgd_plan: plan buffer smaller than gc_powersgd_plan_bytes");
    const bool def = prev_rank != nullptr;
    std::vector<PlanEntry> rec;
    const int rc = powersgd_call("gc_powersgd_plan", def ? STEP_DEFERRED : STEP_EXPLICIT, mats, prev_rank, nmats,
                                 grad_dtype, 1.0f, ws, ws_bytes, static_cast<hipStream_t>(stream), &rec);
    if (rc != GC_OK) return rc;
    PlanHeader h{};
    h.magic = PLAN_MAGIC;
    h.nbatches = static_cast<int>(rec.size());
    h.grad_dtype = grad_dtype;
    h.deferred = def ? 1 : 0;
    h.ws = ws;
    h.ws_bytes = ws_bytes;
    char* out = static_cast<char*>(plan);
    std::memcpy(out, &h, sizeof(h));
    std::memcpy(out + sizeof(h), rec.data(), rec.size() * sizeof(PlanEntry));
    return GC_OK;
}

int gc_powersgd_run_phases(const void* plan, size_t plan_bytes, float eta, void* ws, int phases, void* stream) {
    if (phases < 1 || phases > PH_ALL) return fail(GC_ERR_ARG, "gc_powersgd_run_phases: phases must be 1, 2 or 3");
    return run_plan("gc_powersgd_run_phases", plan, plan_bytes, eta, ws, phases, static_cast<hipStream_t>(stream));
}

int gc_powersgd_run(const void* plan, size_t plan_bytes, float eta, void* ws, void* stream) {
    return run_plan("gc_powersgd_run", plan, plan_bytes, eta, ws, PH_ALL, static_cast<hipStream_t>(stream));
}

int gc_powersgd_materialize(const gc_mat* mats, const int32_t* prev_rank, int nmats, void* ws, size_t ws_bytes,
                            void* stream) {
    return powersgd_call("gc_powersgd_materialize", STEP_MATERIALIZE, mats, prev_rank, nmats, GC_F32, 1.0f, ws,
                         ws_bytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"
