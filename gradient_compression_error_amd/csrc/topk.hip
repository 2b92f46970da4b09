// Mem-SGD top-k sparsification with error-feedback memory on gfx950.
//
// Method ("Sparsified SGD with Memory", method section):
//     acc = m_t + eta * grad;  g_t = comp_k(acc);  m_{t+1} = acc - g_t
// with comp_k = top-k by magnitude (abstract: the most significant entries).
//
// The selection is exact.  The magnitude key of a float is its bit pattern
// without the sign (31 bits; key order == |x| order for non-NaN x).  The
// threshold key T is found by a three-level radix select (12 + 12 + 7 bits):
//
//   topk_prep        zeroes the histograms; one workgroup samples 16384 entries
//                    of acc and sets a guess G below the expected threshold
//   topk_accum_hist  acc = fl32(m + fl32(eta*g)) written over m; 4096-bin LDS
//                    histogram of key>>19 per workgroup, merged with device
//                    atomics into one of 8 copies; every entry with key >= G
//                    is appended, in index order, to its tile's slot region
//                    (wave ballots + a cross-wave prefix); the captured
//                    entries are counted.
//   topk_capture     every workgroup finds bin b1 of the k-th largest key
//                    with one wave, scanning the level-1 bins from G's bin
//                    with the captured count as the count above it.  When
//                    at least k entries were captured (G <= b1's lower edge)
//                    every candidate is already in the slots: only the
//                    level-2 histogram of bin b1 is built from them.
//                    Otherwise re-reads acc and appends every entry with
//                    key>>19 >= b1 instead.  topk_select2 -> bin b2
//   topk_refine      level-3 histogram over the captured entries only (8
//                    copies, like levels 1 and 2).
//   topk_count       threshold T and ties to take from the level-3 histogram
//                    (every workgroup), then #(key > T) and #(key == T) over
//                    the workgroup's contiguous range of tiles.
//   topk_emit        same ranges: output offset from the earlier ranges'
//                    counts, then the k (index, value) pairs in ascending
//                    index order; zeroes the selected memory entries.
//
// Vectors of at most 16384 entries skip that chain: topk_small does the
// accumulate, the three levels, the compaction and the memory in one
// workgroup, with the same arithmetic and the same bits.
//
// Deferred memory (gc_topk_ef_encode_deferred): topk_emit leaves the selected
// entries as they are (no scattered writes) and topk_count / topk_emit write
// a selection record {T, index of the last tie taken}; the next call's
// topk_prep and topk_accum_hist read those entries as +0.0 (mem_of), and
// topk_materialize writes the zeros when the explicit memory is wanted.
//
// Only topk_accum_hist touches all d entries when the guess holds (12 B/entry
// for fp32 gradients); the rest work on the captured entries, which are a
// superset of the candidates at or above the threshold in index order, so
// the later kernels filter by key.  The guess only decides how much work is
// done, never the result.  The level-1 bin is found at the start of the
// kernel that needs it, by every workgroup; the level-2 bin by a
// single-workgroup kernel (a 4096-bin search that every workgroup repeating
// would cost more than the launch).  The kernel boundary is the only
// cross-workgroup synchronisation (a per-workgroup device-scope release fence
// would write back the L2 once per workgroup).
#include <cmath>

#include "gc_common.h"

namespace gc {
namespace {

constexpr int TK_THREADS = 256;
constexpr int TK_SUB = TK_THREADS * 4 * 4;   // 4096 entries: 4 float4 per thread
constexpr int TK_SUBS = 4;
constexpr int TK_TILE = TK_SUB * TK_SUBS;    // 16384 entries per workgroup / slot tile
constexpr int H1_BINS = 4096;
constexpr int H1_SHIFT = 19;   // key bits 30..19
constexpr int H2_BINS = 4096;
constexpr int H2_SHIFT = 7;    // key bits 18..7
constexpr int H3_BINS = 128;   // key bits 6..0
constexpr int NCOPY = 8;       // copies of the level-1/2 histograms (spreads the device atomics)
// The counters zeroed by topk_prep, one block: word offsets from its start.
constexpr int HIST1_W = 0;                                // NCOPY x 4096 level-1 bins
constexpr int HIST2_W = HIST1_W + NCOPY * H1_BINS;        // NCOPY x 4096 level-2 bins
constexpr int HIST3_W = HIST2_W + NCOPY * H2_BINS;        // NCOPY x 128 level-3 bins
constexpr int CAP_W = HIST3_W + NCOPY * H3_BINS;          // NCOPY counts of captured entries,
constexpr int CAP_STRIDE = 32;                            // one 128-byte line each
constexpr int COUNTERS_W = CAP_W + NCOPY * CAP_STRIDE;
static_assert(COUNTERS_W % 64 == 0, "256-byte multiple");
constexpr int TK_SMALL_GRID = 2048;      // workgroups of the candidate passes: one per tile, at most this many
constexpr int DEC_TILE = 4096;
constexpr int PREP_ZERO_BLOCKS = 32;     // topk_prep blocks that zero the histograms
constexpr int FAST_GRID = 256;           // workgroups of topk_capture's slot pass
constexpr int CAP_GROUP = 4;             // tiles per round trip in topk_capture's slot pass
constexpr int CAP_SPEC = 2;              // slots per thread and tile read before the tile's count

struct TopkState {
    unsigned b1, above1;       // level-1 bin, #keys in higher level-1 bins
    unsigned prefix2, above2;  // (b1 << 12) | b2, #keys with (key >> 7) > prefix2
    unsigned thr, above3;      // threshold key T, #keys > T
    unsigned need;             // #keys == T taken (lowest indices first)
    unsigned guess;            // keys >= guess are captured by topk_accum_hist
    unsigned fast;             // 1: the captured slots hold every key >= b1 << 19
    unsigned pad[7];
};
static_assert(sizeof(TopkState) == 64, "TopkState layout");

struct TopkLayout {
    size_t state, counters, tile_cnt, wg_gt, wg_eq;
    size_t slot_idx, slot_val, total, zero_from, zero_end;
    long long ntiles;
};

TopkLayout topk_layout(long long d) {
    TopkLayout L{};
    L.ntiles = (d + TK_TILE - 1) / TK_TILE;
    const size_t nt = static_cast<size_t>(L.ntiles);
    size_t o = 0;
    L.state = o;     o += round_up(sizeof(TopkState), 256);
    L.zero_from = o;
    L.counters = o;  o += COUNTERS_W * 4;
    L.zero_end = o;
    L.tile_cnt = o;  o += round_up(nt * 4, 256);
    L.wg_gt = o;     o += TK_SMALL_GRID * 4;
    L.wg_eq = o;     o += TK_SMALL_GRID * 4;
    L.slot_idx = o;  o += round_up(nt * TK_TILE * 4, 256);
    L.slot_val = o;  o += round_up(nt * TK_TILE * 4, 256);
    L.total = o;
    return L;
}

// ---------------------------------------------------------------- device helpers

// Deferred memory: mem holds acc of the previous step, and the selection
// record {thr, cut} says which entries that step selected -- key > thr, or
// key == thr and index <= cut (the ties it took, lowest indices first).  Those
// entries are +0.0 in the memory the method carries.
struct PrevSel {
    unsigned thr;
    long long cut;
};

__device__ __forceinline__ PrevSel read_sel(const unsigned* sel) {
    PrevSel ps;
    ps.thr = sel[0];
    ps.cut = static_cast<int>(sel[1]);
    return ps;
}

__device__ __forceinline__ bool was_selected(float a, long long i, const PrevSel& ps) {
    const unsigned key = key_of(a);
    return key > ps.thr || (key == ps.thr && i <= ps.cut);
}

__device__ __forceinline__ float mem_of(float a, long long i, const PrevSel& ps) {
    return was_selected(a, i, ps) ? 0.0f : a;
}

// Bin b of the histogram (sum of NC copies spaced `stride` words apart,
// scanned from the top) with
//   sum(hist[b+1 ..]) < need <= sum(hist[b ..]);
// *bin = b and *above = sum(hist[b+1 ..]).  Needs 1 <= need <= sum(hist).
// The histogram was completed by the previous kernel; its copies are summed
// into LDS first (all loads independent).  Whole block; results in shared
// memory after the final barrier.
template <int NBINS, int NC, int NT = TK_THREADS>
__device__ void select_bin(const unsigned* hist, int stride, unsigned need, unsigned* s_h,
                           unsigned* s_tmp, unsigned* s_bin, unsigned* s_above) {
    constexpr int PER = (NBINS + NT - 1) / NT;
    const int t = threadIdx.x;
    if (t == 0) {
        *s_bin = 0u;
        *s_above = 0u;
    }
    unsigned v[PER][NC];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int b = t + i * NT;
#pragma unroll
        for (int k = 0; k < NC; ++k) v[i][k] = (b < NBINS) ? hist[k * stride + b] : 0u;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int b = t + i * NT;
        unsigned c = 0;
#pragma unroll
        for (int k = 0; k < NC; ++k) c += v[i][k];
        if (b < NBINS) s_h[b] = c;
    }
    __syncthreads();
    // thread t scans bins [hi - PER, hi) from the top
    const int hi = NBINS - t * PER;
    unsigned cnt[PER];
    unsigned s = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int b = hi - PER + i;
        cnt[i] = (b >= 0 && b < NBINS) ? s_h[b] : 0u;
        s += cnt[i];
    }
    unsigned total;
    const unsigned incl = block_inclusive_scan<NT / 64>(s, s_tmp, &total);
    const unsigned excl = incl - s;
    if (s > 0 && excl < need && need <= incl) {
        unsigned run = excl;
        bool found = false;
#pragma unroll
        for (int i = PER - 1; i >= 0; --i) {
            const int b = hi - PER + i;
            if (!found && b >= 0) {
                if (run + cnt[i] >= need) {
                    *s_bin = static_cast<unsigned>(b);
                    *s_above = run;
                    found = true;
                }
                run += cnt[i];
            }
        }
    }
    __syncthreads();
}

// Inclusive prefix sum over the 64 lanes of one wave (all lanes active).
__device__ __forceinline__ unsigned wave_inclusive_scan(unsigned v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const unsigned t = __shfl_up(v, o, WAVE);
        if (lane >= o) v += t;
    }
    return v;
}

// Level-1 bin b1 of the k-th largest key, found by one wave from the
// captured count instead of the whole histogram.  With S(b) = #keys whose
// level-1 bin is >= b, b1 is the highest bin with S(b1) >= k and
// S(g0) = ncap is known for the guess bin g0 (every key with bin >= g0 was
// captured).  ncap >= k: b1 >= g0; windows of 64 bins are scanned upwards
// from g0, S falling by each window's count.  ncap < k: b1 < g0; windows are
// scanned downwards from g0 - 1, S rising by each window's count.  S(4096) = 0
// < k and S(0) = d >= k, so at most 64 windows.  Lane j holds one bin of the
// window (NCOPY copies summed).  Every lane gets b1 and S(b1 + 1).
struct BinPick {
    unsigned bin, above;
};

__device__ __forceinline__ BinPick find_b1_wave(const unsigned* __restrict__ hist1, unsigned ncap, int g0,
                                                unsigned k) {
    const int lane = threadIdx.x & 63;
    if (ncap >= k) {
        unsigned s_lo = ncap;   // S(lo)
        for (int lo = g0; lo < H1_BINS; lo += 64) {
            const int b = lo + lane;
            unsigned c = 0;
            if (b < H1_BINS) {
#pragma unroll
                for (int cp = 0; cp < NCOPY; ++cp) c += hist1[cp * H1_BINS + b];
            }
            const unsigned incl = wave_inclusive_scan(c);
            const unsigned excl = incl - c;
            // S(lo + j) = s_lo - excl(j) >= k  <=>  excl(j) <= s_lo - k  (s_lo >= k here)
            const unsigned long long keep = __ballot(excl <= s_lo - k);
            const int j = 63 - __builtin_clzll(keep);   // highest such lane (lane 0 always qualifies)
            const unsigned total = readlane_any(incl, 63);
            if (j < 63 || s_lo - total < k)
                return BinPick{static_cast<unsigned>(lo + j), s_lo - readlane_any(incl, j)};
            s_lo -= total;
        }
        return BinPick{H1_BINS - 1, 0u};   // not reached for a consistent histogram
    }
    unsigned s_hi = ncap;   // S(hi)
    for (int hi = g0; hi > 0; hi -= 64) {
        const int b = hi - 1 - lane;
        unsigned c = 0;
        if (b >= 0) {
#pragma unroll
            for (int cp = 0; cp < NCOPY; ++cp) c += hist1[cp * H1_BINS + b];
        }
        const unsigned incl = wave_inclusive_scan(c);
        // S(hi - 1 - j) = s_hi + incl(j): the first lane where it reaches k
        const unsigned long long hit = __ballot(s_hi + incl >= k);
        if (hit) {
            const int j = __builtin_ctzll(hit);
            return BinPick{static_cast<unsigned>(hi - 1 - j), s_hi + readlane_any(incl - c, j)};
        }
        s_hi += readlane_any(incl, 63);
    }
    return BinPick{0u, 0u};   // not reached for a consistent histogram
}

// Adds a workgroup's 4096-bin LDS histogram into one device copy: the 16 LDS
// reads of a thread are issued together, then the nonzero bins are added.
__device__ __forceinline__ void merge_hist4096(const unsigned* h, unsigned* __restrict__ dst) {
    static_assert(H1_BINS == 4096 && H2_BINS == 4096, "level-1 and level-2 histograms of 4096 bins");
    constexpr int PER = 4096 / TK_THREADS;
    unsigned c[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) c[j] = h[threadIdx.x + j * TK_THREADS];
#pragma unroll
    for (int j = 0; j < PER; ++j)
        if (c[j]) atomicAdd(dst + threadIdx.x + j * TK_THREADS, c[j]);
}

// ---------------------------------------------------------------- kernels

constexpr int PREP_THREADS = 1024;
constexpr int SAMPLE_RUN = 64;                       // consecutive entries per sampled run
constexpr int SAMPLE_RUNS = 256;
constexpr int SAMPLES = SAMPLE_RUN * SAMPLE_RUNS;    // entries sampled for the guess
constexpr int SAMPLES_PER_THREAD = SAMPLES / PREP_THREADS;

// Block 0: writes the state record (zeros and the guess).  It samples
// S = min(d, 16384) entries of acc -- all of them when d <= 16384, else 256
// runs of 64 consecutive entries starting at floor(r d / 256) (a wave reads
// one run: few cache lines and pages) -- histograms their level-1 bins and
// sets guess = lower edge of the bin holding the sample of rank `rank_g` from
// the top (rank_g >= S: guess = 0, capture all).  Blocks 1..: zero the
// histograms.
template <bool BF16, bool DEFR>
__global__ __launch_bounds__(PREP_THREADS) void topk_prep(
        const void* __restrict__ grad, const float* __restrict__ mem, long long d, float eta,
        unsigned rank_g, TopkState* __restrict__ st, uint4* __restrict__ zero, int n16,
        const unsigned* __restrict__ sel) {
    if (blockIdx.x > 0) {
        const int stride = (gridDim.x - 1) * PREP_THREADS;
        for (int i = (blockIdx.x - 1) * PREP_THREADS + threadIdx.x; i < n16; i += stride)
            zero[i] = make_uint4(0u, 0u, 0u, 0u);
        return;
    }
    __shared__ unsigned h[H1_BINS];
    __shared__ unsigned s_tmp[PREP_THREADS / 64];
    __shared__ unsigned s_bin, s_above;
    for (int i = threadIdx.x; i < H1_BINS; i += PREP_THREADS) h[i] = 0u;
    __syncthreads();
    const long long S = d < SAMPLES ? d : SAMPLES;
    float mv[SAMPLES_PER_THREAD], gv[SAMPLES_PER_THREAD];
#pragma unroll
    for (int u = 0; u < SAMPLES_PER_THREAD; ++u) {
        const long long smp = threadIdx.x + static_cast<long long>(u) * PREP_THREADS;
        long long pos = 0;
        if (smp < S) {
            const long long run = smp / SAMPLE_RUN;
            pos = S == d ? smp : run * d / SAMPLE_RUNS + smp % SAMPLE_RUN;
        }
        mv[u] = mem[pos];
        gv[u] = load_grad1<BF16>(grad, pos);
        if constexpr (DEFR) mv[u] = mem_of(mv[u], pos, read_sel(sel));
    }
#pragma unroll
    for (int u = 0; u < SAMPLES_PER_THREAD; ++u) {
        const long long smp = threadIdx.x + static_cast<long long>(u) * PREP_THREADS;
        if (smp < S) atomicAdd(&h[key_of(ef_acc(mv[u], eta, gv[u])) >> H1_SHIFT], 1u);
    }
    __syncthreads();
    unsigned guess = 0u;
    if (rank_g < static_cast<unsigned>(S)) {
        select_bin<H1_BINS, 1, PREP_THREADS>(h, H1_BINS, rank_g, h, s_tmp, &s_bin, &s_above);
        guess = s_bin << H1_SHIFT;
    }
    if (threadIdx.x == 0) {
        TopkState z{};
        z.guess = guess;
        *st = z;
    }
}

template <bool BF16>
__device__ __forceinline__ void load_sub(const void* __restrict__ grad, const float* __restrict__ mem, long long b4,
                                         float4 (&gv)[4], float4 (&mv)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const long long i4 = b4 + u * TK_THREADS + threadIdx.x;
        gv[u] = load_grad4<BF16>(grad, i4);
        mv[u] = reinterpret_cast<const float4*>(mem)[i4];
    }
}

// In-order append of the flagged entries of U chunks of the tile.  In chunk u
// entry j of thread t comes after every flagged entry of lower threads (all
// waves) and of lower j, and chunks follow each other.  `cnt` holds the
// per-(chunk, wave) counts, double-buffered by parity: one barrier.  Returns
// the number appended by the whole workgroup.
template <int U, int J>
__device__ __forceinline__ unsigned append_chunks(const bool (&flag)[U][J], const float (&val)[U][J],
                                                  const long long (&idx0)[U], unsigned running,
                                                  int* __restrict__ sidx, float* __restrict__ sval,
                                                  unsigned (*cnt)[TK_SUBS][4], int& parity) {
    static_assert(U <= TK_SUBS, "chunks per append");
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const unsigned long long lt = lanemask_lt();
    unsigned before[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        unsigned b = 0, wtot = 0;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const unsigned long long bal = __ballot(flag[u][j]);
            b += __popcll(bal & lt);
            wtot += __popcll(bal);
        }
        before[u] = b;
        if (lane == 0) cnt[parity][u][w] = wtot;
    }
    __syncthreads();
    unsigned run = running;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        unsigned wbefore = 0, ctot = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const unsigned c = cnt[parity][u][i];
            wbefore += (i < w) ? c : 0u;
            ctot += c;
        }
        unsigned pos = run + wbefore + before[u];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            if (flag[u][j]) {
                sidx[pos] = static_cast<int>(idx0[u] + j);
                sval[pos] = val[u][j];
                ++pos;
            }
        }
        run += ctot;
    }
    parity ^= 1;
    return run - running;
}

// acc = fl32(m + fl32(eta*g)) over TK_TILE entries per workgroup (sub-tile s+1
// is loaded before sub-tile s is stored), with a level-1 histogram in LDS;
// entries with key >= guess go to the tile's slots in index order.
template <bool BF16, bool DEFR>
__global__ __launch_bounds__(TK_THREADS) void topk_accum_hist(
        const void* __restrict__ grad, float* __restrict__ mem, long long d, float eta,
        const TopkState* __restrict__ st, unsigned* __restrict__ ctr, int* __restrict__ slot_idx,
        float* __restrict__ slot_val, unsigned* __restrict__ tile_cnt, const unsigned* __restrict__ sel) {
    __shared__ unsigned h[H1_BINS];
    __shared__ unsigned s_cnt[2][TK_SUBS][4];
    for (int i = threadIdx.x; i < H1_BINS; i += TK_THREADS) h[i] = 0u;
    __syncthreads();

    const unsigned guess = st->guess;
    PrevSel ps{};
    if constexpr (DEFR) ps = read_sel(sel);
    const long long base = static_cast<long long>(blockIdx.x) * TK_TILE;
    int* const sidx = slot_idx + base;
    float* const sval = slot_val + base;
    unsigned running = 0;
    int parity = 0;
    long long nfull = (d - base) / TK_SUB;
    if (nfull > TK_SUBS) nfull = TK_SUBS;
    float4 gv[4], mv[4];
    if (nfull > 0) load_sub<BF16>(grad, mem, base / 4, gv, mv);
    for (int sb = 0; sb < nfull; ++sb) {
        const long long b4 = (base + static_cast<long long>(sb) * TK_SUB) / 4;
        float4 gn[4], mn[4];
        if (sb + 1 < nfull) load_sub<BF16>(grad, mem, b4 + TK_SUB / 4, gn, mn);
        float a[4][4];
        bool cap[4][4];
        long long e0[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const long long i4 = b4 + u * TK_THREADS + threadIdx.x;
            if constexpr (DEFR) {
                mv[u].x = mem_of(mv[u].x, i4 * 4, ps);
                mv[u].y = mem_of(mv[u].y, i4 * 4 + 1, ps);
                mv[u].z = mem_of(mv[u].z, i4 * 4 + 2, ps);
                mv[u].w = mem_of(mv[u].w, i4 * 4 + 3, ps);
            }
            a[u][0] = ef_acc(mv[u].x, eta, gv[u].x);
            a[u][1] = ef_acc(mv[u].y, eta, gv[u].y);
            a[u][2] = ef_acc(mv[u].z, eta, gv[u].z);
            a[u][3] = ef_acc(mv[u].w, eta, gv[u].w);
            e0[u] = i4 * 4;
            reinterpret_cast<float4*>(mem)[i4] = make_float4(a[u][0], a[u][1], a[u][2], a[u][3]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const unsigned key = key_of(a[u][j]);
                atomicAdd(&h[key >> H1_SHIFT], 1u);
                cap[u][j] = key >= guess;
            }
        }
        running += append_chunks<4, 4>(cap, a, e0, running, sidx, sval, s_cnt, parity);
        if (sb + 1 < nfull) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                gv[u] = gn[u];
                mv[u] = mn[u];
            }
        }
    }
    const long long t0 = base + nfull * TK_SUB;
    const long long t1 = min(d, base + static_cast<long long>(TK_TILE));
    for (long long i0 = t0; i0 < t1; i0 += TK_THREADS) {
        const long long i = i0 + threadIdx.x;
        bool cap[1][1] = {{false}};
        float a[1][1] = {{0.0f}};
        const long long e0[1] = {i};
        if (i < t1) {
            float mi = mem[i];
            if constexpr (DEFR) mi = mem_of(mi, i, ps);
            a[0][0] = ef_acc(mi, eta, load_grad1<BF16>(grad, i));
            mem[i] = a[0][0];
            const unsigned key = key_of(a[0][0]);
            atomicAdd(&h[key >> H1_SHIFT], 1u);
            cap[0][0] = key >= guess;
        }
        running += append_chunks<1, 1>(cap, a, e0, running, sidx, sval, s_cnt, parity);
    }
    if (threadIdx.x == 0) {
        tile_cnt[blockIdx.x] = running;
        if (running) atomicAdd(ctr + CAP_W + (blockIdx.x % NCOPY) * CAP_STRIDE, running);
    }
    __syncthreads();
    merge_hist4096(h, ctr + HIST1_W + (blockIdx.x % NCOPY) * H1_BINS);
}

// Level-1 bin b1 (the bin of the k-th largest key; every workgroup finds it
// with find_b1_wave, workgroup 0 records it), then the level-2 histogram of
// bin b1.  Fast case (every key >= b1 << 19 is already
// in the slots): from the tile's slots.  Otherwise re-reads acc and replaces
// the tile's slots with the entries of key>>19 >= b1, in index order.
// The fast case holds exactly when at least k entries were captured: the
// slots hold the keys of level-1 bin >= bin(guess), and b1 is the highest
// bin whose count from the top reaches k.
__global__ __launch_bounds__(TK_THREADS) void topk_capture(
        const float* __restrict__ acc, long long d, unsigned k, TopkState* __restrict__ st,
        unsigned* __restrict__ ctr, int* __restrict__ slot_idx, float* __restrict__ slot_val,
        unsigned* __restrict__ tile_cnt) {
    __shared__ unsigned h[H2_BINS];
    __shared__ unsigned s_cnt[2][TK_SUBS][4];
    __shared__ unsigned s_b1;
    // both loads in flight together: the guess bin addresses the first window
    const int g0 = static_cast<int>(st->guess >> H1_SHIFT);
    unsigned ncap = 0;
#pragma unroll
    for (int c = 0; c < NCOPY; ++c) ncap += ctr[CAP_W + c * CAP_STRIDE];
    asm volatile("" ::"s"(g0));   // keeps the guess load here instead of after the exit test
    const bool fast = ncap >= k;
    // fast case: the first FAST_GRID workgroups stride over the tiles' slots; the rest exit
    if (fast && static_cast<int>(blockIdx.x) >= FAST_GRID) return;
    if (threadIdx.x < 64) {
        const BinPick p1 = find_b1_wave(ctr + HIST1_W, ncap, g0, k);
        if (threadIdx.x == 0) {
            s_b1 = p1.bin;
            if (blockIdx.x == 0) {
                st->b1 = p1.bin;
                st->above1 = p1.above;
                st->fast = fast ? 1u : 0u;
            }
        }
    }
    for (int i = threadIdx.x; i < H2_BINS; i += TK_THREADS) h[i] = 0u;
    __syncthreads();

    const unsigned b1 = s_b1;
    const long long base = static_cast<long long>(blockIdx.x) * TK_TILE;
    int* const sidx = slot_idx + base;
    float* const sval = slot_val + base;
    if (fast) {
        // Tiles b, b + FAST_GRID, ... of this workgroup, CAP_GROUP at a time: their
        // counts and the first CAP_SPEC slots per thread of each are loaded
        // together, before the counts are known (the slot region of every tile
        // is allocated; what lies past a count is read and ignored), so a group
        // costs one memory round trip instead of one per tile and slot row.
        const int ntiles = static_cast<int>(gridDim.x);
        auto count_l2 = [&](float v) {
            const unsigned key = key_of(v);
            if ((key >> H1_SHIFT) == b1) atomicAdd(&h[(key >> H2_SHIFT) & (H2_BINS - 1)], 1u);
        };
        for (int t0 = blockIdx.x; t0 < ntiles; t0 += CAP_GROUP * FAST_GRID) {
            unsigned cnt[CAP_GROUP];
            float v[CAP_GROUP][CAP_SPEC];
#pragma unroll
            for (int g = 0; g < CAP_GROUP; ++g) {
                const int t = t0 + g * FAST_GRID;
                const bool real = t < ntiles;
                const float* tv = slot_val + static_cast<long long>(real ? t : t0) * TK_TILE;
                cnt[g] = real ? tile_cnt[t] : 0u;
#pragma unroll
                for (int sp = 0; sp < CAP_SPEC; ++sp) v[g][sp] = tv[threadIdx.x + sp * TK_THREADS];
            }
#pragma unroll
            for (int g = 0; g < CAP_GROUP; ++g) {
#pragma unroll
                for (int sp = 0; sp < CAP_SPEC; ++sp)
                    if (threadIdx.x + sp * TK_THREADS < cnt[g]) count_l2(v[g][sp]);
                // the rest of a longer tile, 4 slot rows per round trip (indices
                // clamped into the tile, the values past the count ignored)
                const float* tv = slot_val + static_cast<long long>(t0 + g * FAST_GRID) * TK_TILE;
                for (unsigned e = threadIdx.x + CAP_SPEC * TK_THREADS; e < cnt[g]; e += 4 * TK_THREADS) {
                    float w[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) w[q] = tv[min(e + q * TK_THREADS, static_cast<unsigned>(TK_TILE - 1))];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (e + q * TK_THREADS < cnt[g]) count_l2(w[q]);
                }
            }
        }
    } else {
        unsigned running = 0;
        int parity = 0;
        for (int sb = 0; sb < TK_SUBS; ++sb) {
            const long long sbase = base + static_cast<long long>(sb) * TK_SUB;
            if (sbase >= d) break;
            float v[4][4];
            bool ok[4][4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const long long e0 = sbase + u * (TK_THREADS * 4) + threadIdx.x * 4;
                if (e0 + 3 < d) {
                    const float4 x = reinterpret_cast<const float4*>(acc)[e0 / 4];
                    v[u][0] = x.x; v[u][1] = x.y; v[u][2] = x.z; v[u][3] = x.w;
                    ok[u][0] = ok[u][1] = ok[u][2] = ok[u][3] = true;
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        ok[u][j] = (e0 + j) < d;
                        v[u][j] = ok[u][j] ? acc[e0 + j] : 0.0f;
                    }
                }
            }
            bool cap[4][4];
            long long e0[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                e0[u] = sbase + u * (TK_THREADS * 4) + threadIdx.x * 4;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const unsigned key = key_of(v[u][j]);
                    const unsigned bin = key >> H1_SHIFT;
                    cap[u][j] = ok[u][j] && bin >= b1;
                    if (ok[u][j] && bin == b1) atomicAdd(&h[(key >> H2_SHIFT) & (H2_BINS - 1)], 1u);
                }
            }
            running += append_chunks<4, 4>(cap, v, e0, running, sidx, sval, s_cnt, parity);
        }
        if (threadIdx.x == 0) tile_cnt[blockIdx.x] = running;
    }
    __syncthreads();
    merge_hist4096(h, ctr + HIST2_W + (blockIdx.x % NCOPY) * H2_BINS);
}

constexpr int SEL_THREADS = 1024;   // single-workgroup selection kernel

__global__ __launch_bounds__(SEL_THREADS) void topk_select2(const unsigned* __restrict__ hist2, unsigned k,
                                                            TopkState* __restrict__ st) {
    __shared__ unsigned s_h[H2_BINS];
    __shared__ unsigned s_tmp[SEL_THREADS / 64];
    __shared__ unsigned s_bin, s_above;
    const unsigned above1 = st->above1;
    select_bin<H2_BINS, NCOPY, SEL_THREADS>(hist2, H2_BINS, k - above1, s_h, s_tmp, &s_bin, &s_above);
    if (threadIdx.x == 0) {
        st->prefix2 = (st->b1 << 12) | s_bin;
        st->above2 = above1 + s_above;
    }
}

__global__ __launch_bounds__(TK_THREADS) void topk_refine(
        const TopkState* __restrict__ st, unsigned* __restrict__ hist3,
        const float* __restrict__ slot_val, const unsigned* __restrict__ tile_cnt, int ntiles) {
    __shared__ unsigned h[H3_BINS];
    const unsigned prefix2 = st->prefix2;
    auto count_l3 = [&](float v) {
        const unsigned key = key_of(v);
        if ((key >> H2_SHIFT) == prefix2) atomicAdd(&h[key & (H3_BINS - 1)], 1u);
    };
    // the tile's count and its first two slot rows are read together with
    // prefix2 (grid <= ntiles, so every workgroup has a tile)
    int t = blockIdx.x;
    unsigned cnt = tile_cnt[t];
    const float* sv = slot_val + static_cast<long long>(t) * TK_TILE;
    float v0 = sv[threadIdx.x], v1 = sv[threadIdx.x + TK_THREADS];
    for (int i = threadIdx.x; i < H3_BINS; i += TK_THREADS) h[i] = 0u;
    __syncthreads();
    while (true) {
        if (threadIdx.x < cnt) count_l3(v0);
        if (threadIdx.x + TK_THREADS < cnt) count_l3(v1);
        for (unsigned e = threadIdx.x + 2 * TK_THREADS; e < cnt; e += 4 * TK_THREADS) {
            float w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) w[q] = sv[min(e + q * TK_THREADS, static_cast<unsigned>(TK_TILE - 1))];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (e + q * TK_THREADS < cnt) count_l3(w[q]);
        }
        t += gridDim.x;
        if (t >= ntiles) break;
        cnt = tile_cnt[t];
        sv = slot_val + static_cast<long long>(t) * TK_TILE;
        v0 = sv[threadIdx.x];
        v1 = sv[threadIdx.x + TK_THREADS];
    }
    __syncthreads();
    // merged into one of NCOPY copies: every workgroup adds to the same 128
    // bins, so one copy would serialise the atomics
    unsigned* dst = hist3 + (blockIdx.x % NCOPY) * H3_BINS;
    for (int i = threadIdx.x; i < H3_BINS; i += TK_THREADS) {
        const unsigned c = h[i];
        if (c) atomicAdd(dst + i, c);
    }
}

// Tiles [b n / G, (b+1) n / G) of workgroup b of G (the same partition in
// topk_count and topk_emit).
__device__ __forceinline__ int tile_lo(int b, int g, int ntiles) {
    return static_cast<int>(static_cast<long long>(b) * ntiles / g);
}

// Every workgroup finds the threshold key T from the level-3 histogram (128
// bins); workgroup 0 records it.  Then per tile of the workgroup's range:
// #(key > T), #(key == T), and the range totals.
__global__ __launch_bounds__(TK_THREADS) void topk_count(
        TopkState* __restrict__ st, const unsigned* __restrict__ hist3, unsigned k,
        const float* __restrict__ slot_val, const unsigned* __restrict__ tile_cnt, int ntiles,
        unsigned* __restrict__ wg_gt, unsigned* __restrict__ wg_eq, unsigned* __restrict__ sel_out) {
    __shared__ unsigned s_red[8];
    __shared__ unsigned s_h[H3_BINS];
    __shared__ unsigned s_tmp[4];
    __shared__ unsigned s_bin, s_above;
    const unsigned above2 = st->above2, prefix2 = st->prefix2;
    // the first tile's count and two slot rows are read with the level-3
    // histogram (grid <= ntiles: every workgroup has a tile)
    const int t0 = tile_lo(blockIdx.x, gridDim.x, ntiles), t1 = tile_lo(blockIdx.x + 1, gridDim.x, ntiles);
    unsigned cnt = tile_cnt[t0];
    const float* sv = slot_val + static_cast<long long>(t0) * TK_TILE;
    float v0 = sv[threadIdx.x], v1 = sv[threadIdx.x + TK_THREADS];
    select_bin<H3_BINS, NCOPY>(hist3, H3_BINS, k - above2, s_h, s_tmp, &s_bin, &s_above);
    const unsigned thr = (prefix2 << H2_SHIFT) | s_bin;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        const unsigned above3 = above2 + s_above;
        st->thr = thr;
        st->above3 = above3;
        st->need = k - above3;
        if (sel_out) {
            // the selection record of a deferred call; topk_emit sets the cut
            // when ties are taken
            sel_out[0] = thr;
            sel_out[1] = 0xFFFFFFFFu;   // -1: no tie taken
        }
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    unsigned rgt = 0, req = 0;
    for (int t = t0; t < t1; ++t) {
        if (t > t0) {
            cnt = tile_cnt[t];
            sv = slot_val + static_cast<long long>(t) * TK_TILE;
            v0 = sv[threadIdx.x];
            v1 = sv[threadIdx.x + TK_THREADS];
        }
        unsigned gt = 0, eq = 0;
        auto tally = [&](float v) {
            const unsigned key = key_of(v);
            gt += key > thr;
            eq += key == thr;
        };
        if (threadIdx.x < cnt) tally(v0);
        if (threadIdx.x + TK_THREADS < cnt) tally(v1);
        for (unsigned e = threadIdx.x + 2 * TK_THREADS; e < cnt; e += 4 * TK_THREADS) {
            float w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) w[q] = sv[min(e + q * TK_THREADS, static_cast<unsigned>(TK_TILE - 1))];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (e + q * TK_THREADS < cnt) tally(w[q]);
        }
        gt = wave_sum(gt);
        eq = wave_sum(eq);
        if (lane == 0) {
            s_red[w] = gt;
            s_red[4 + w] = eq;
        }
        __syncthreads();
        rgt += s_red[0] + s_red[1] + s_red[2] + s_red[3];
        req += s_red[4] + s_red[5] + s_red[6] + s_red[7];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        wg_gt[blockIdx.x] = rgt;
        wg_eq[blockIdx.x] = req;
    }
}

__global__ __launch_bounds__(TK_THREADS) void topk_emit(
        const TopkState* __restrict__ st, const int* __restrict__ slot_idx,
        const float* __restrict__ slot_val, const unsigned* __restrict__ tile_cnt,
        const unsigned* __restrict__ wg_gt, const unsigned* __restrict__ wg_eq, int ntiles,
        unsigned k, int* __restrict__ out_idx, float* __restrict__ out_val, float* __restrict__ mem,
        unsigned* __restrict__ sel_out) {
    __shared__ unsigned s_eq[4], s_sel[4];
    const unsigned thr = st->thr;
    const unsigned need = st->need;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const unsigned long long lt = lanemask_lt();
    // the first slot row of the first tile is read with the counts below
    // (grid <= ntiles: every workgroup has a tile)
    const int t0 = tile_lo(blockIdx.x, gridDim.x, ntiles), t1 = tile_lo(blockIdx.x + 1, gridDim.x, ntiles);
    unsigned cnt = tile_cnt[t0];
    long long sbase = static_cast<long long>(t0) * TK_TILE;
    float v = slot_val[sbase + threadIdx.x];
    int ix = slot_idx[sbase + threadIdx.x];
    // ties and selected entries before this workgroup's tile range: the ties
    // are taken in index order, so min(need, ties before) of them precede it.
    // Eight loads per thread and round trip (indices clamped, extra values
    // ignored).
    unsigned pgt = 0, peq = 0;
    const int nb = static_cast<int>(blockIdx.x);
    for (int b0 = threadIdx.x; b0 < nb; b0 += 8 * TK_THREADS) {
        unsigned a[8], c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int b = min(b0 + j * TK_THREADS, nb - 1);
            a[j] = wg_gt[b];
            c[j] = wg_eq[b];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (b0 + j * TK_THREADS < nb) {
                pgt += a[j];
                peq += c[j];
            }
        }
    }
    pgt = wave_sum(pgt);
    peq = wave_sum(peq);
    if (lane == 0) {
        s_eq[w] = pgt;
        s_sel[w] = peq;
    }
    __syncthreads();
    unsigned eqr = ((s_sel[0] + s_sel[1]) + s_sel[2]) + s_sel[3];
    unsigned off = (((s_eq[0] + s_eq[1]) + s_eq[2]) + s_eq[3]) + min(need, eqr);
    __syncthreads();
    for (int t = t0; t < t1; ++t) {
        if (t > t0) {
            cnt = tile_cnt[t];
            sbase = static_cast<long long>(t) * TK_TILE;
            v = slot_val[sbase + threadIdx.x];
            ix = slot_idx[sbase + threadIdx.x];
        }
        for (unsigned c0 = 0; c0 < cnt; c0 += TK_THREADS) {
            const unsigned e = c0 + threadIdx.x;
            const bool valid = e < cnt;   // v and ix past the count are read but not used
            // the next slot row of the tile, read while this one is placed
            float vn = 0.0f;
            int ixn = 0;
            if (c0 + TK_THREADS < cnt) {
                const unsigned en = min(e + TK_THREADS, static_cast<unsigned>(TK_TILE - 1));
                vn = slot_val[sbase + en];
                ixn = slot_idx[sbase + en];
            }
            const unsigned key = key_of(v);
            const bool is_eq = valid && key == thr;
            const bool is_gt = valid && key > thr;
            const unsigned long long beq = __ballot(is_eq);
            if (lane == 0) s_eq[w] = __popcll(beq);
            __syncthreads();
            unsigned weq = 0, teq = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                weq += (i < w) ? s_eq[i] : 0u;
                teq += s_eq[i];
            }
            const unsigned rank = eqr + weq + __popcll(beq & lt);
            const bool sel = is_gt || (is_eq && rank < need);
            const unsigned long long bsel = __ballot(sel);
            if (lane == 0) s_sel[w] = __popcll(bsel);
            __syncthreads();
            unsigned wsel = 0, tsel = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                wsel += (i < w) ? s_sel[i] : 0u;
                tsel += s_sel[i];
            }
            const unsigned pos = off + wsel + __popcll(bsel & lt);
            if (sel && pos < k) {
                out_idx[pos] = ix;
                out_val[pos] = v;
                // deferred memory: the selection record stands in for the zeros
                if (!sel_out) mem[ix] = 0.0f;
                else if (is_eq && rank + 1 == need) sel_out[1] = static_cast<unsigned>(ix);
            }
            eqr += teq;
            off += tsel;
            v = vn;
            ix = ixn;
            __syncthreads();
        }
    }
}

// Writes the deferred memory out: the entries the selection record marks
// become +0.0 (all d entries read, the selected ones written).
__global__ __launch_bounds__(256) void topk_materialize(float* __restrict__ mem, long long d,
                                                        const unsigned* __restrict__ sel) {
    const PrevSel ps = read_sel(sel);
    const long long stride = static_cast<long long>(gridDim.x) * 256;
    for (long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x; i < d; i += stride) {
        if (was_selected(mem[i], i, ps)) mem[i] = 0.0f;
    }
}

// First position p in idx[0..k) with idx[p] >= target (idx ascending), found
// by one wave with 64-way probes.  All lanes of the wave get the result.
__device__ long long wave_lower_bound(const int* __restrict__ idx, long long k, long long target) {
    const int lane = threadIdx.x & 63;
    long long lo = 0, hi = k;
    while (hi - lo > 64) {
        const long long step = (hi - lo + 63) / 64;
        const long long pos = lo + lane * step;
        const bool less = pos < hi && static_cast<long long>(idx[pos]) < target;
        const int c = __popcll(__ballot(less));
        const long long nlo = c > 0 ? lo + static_cast<long long>(c - 1) * step + 1 : lo;
        const long long nhi = c < 64 ? min(hi, lo + static_cast<long long>(c) * step) : hi;
        lo = nlo;
        hi = nhi;
    }
    const long long pos = lo + lane;
    const bool less = pos < hi && static_cast<long long>(idx[pos]) < target;
    return lo + __popcll(__ballot(less));
}

__global__ __launch_bounds__(256) void topk_decode_set(
        const int* __restrict__ idx, const float* __restrict__ val, long long k,
        float* __restrict__ out, long long d) {
    __shared__ float4 buf4[DEC_TILE / 4];
    __shared__ long long s_lo, s_hi;
    float* buf = reinterpret_cast<float*>(buf4);
    const long long t0 = static_cast<long long>(blockIdx.x) * DEC_TILE;
    const long long t1 = min(d, t0 + DEC_TILE);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (w == 0) {
        const long long r = wave_lower_bound(idx, k, t0);
        if (lane == 0) s_lo = r;
    } else if (w == 1) {
        const long long r = wave_lower_bound(idx, k, t1);
        if (lane == 0) s_hi = r;
    }
    for (int i = threadIdx.x; i < DEC_TILE / 4; i += 256) buf4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();
    for (long long p = s_lo + threadIdx.x; p < s_hi; p += 256) {
        const long long i = idx[p];
        if (i >= t0 && i < t1) buf[i - t0] = val[p];
    }
    __syncthreads();
    if (t1 - t0 == DEC_TILE) {
        float4* o4 = reinterpret_cast<float4*>(out + t0);
        for (int i = threadIdx.x; i < DEC_TILE / 4; i += 256) o4[i] = buf4[i];
    } else {
        for (long long i = t0 + threadIdx.x; i < t1; i += 256) out[i] = buf[i - t0];
    }
}

__global__ __launch_bounds__(256) void topk_decode_add(
        const int* __restrict__ idx, const float* __restrict__ val, long long k,
        float* __restrict__ out, long long d) {
    const long long p = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
    if (p < k) {
        const long long i = idx[p];
        if (i >= 0 && i < d) out[i] = __fadd_rn(out[i], val[p]);
    }
}

// ---------------------------------------------------------------- small vectors

// The whole encode of a vector of d <= SMALL_D entries in one workgroup, where
// the multi-kernel path would be seven dependent launches of almost no work.
// Thread t holds the SMALL_PER consecutive entries [t SMALL_PER, (t+1)
// SMALL_PER), so index order is thread order and then register order, and
// one block scan places every selected entry.  Same arithmetic and selection
// as the general path: acc = fl32(m + fl32(eta * g)); the 12 + 12 + 7-bit
// radix select on the magnitude key, in LDS; the entries above the threshold
// key T, then ties in index order.  Memory, pairs and the selection record get
// the same bits.
constexpr int SMALL_THREADS = 1024;
constexpr int SMALL_PER = 16;
constexpr long long SMALL_D = static_cast<long long>(SMALL_THREADS) * SMALL_PER;   // 16384

template <bool BF16, bool DEFR>
__global__ __launch_bounds__(SMALL_THREADS) void topk_small(
        const void* __restrict__ grad, float* __restrict__ mem, long long d, float eta, unsigned k,
        int* __restrict__ out_idx, float* __restrict__ out_val, unsigned* __restrict__ sel) {
    __shared__ unsigned h[H1_BINS];
    __shared__ unsigned s_tmp[SMALL_THREADS / 64];
    __shared__ unsigned s_bin, s_above;
    const int t = threadIdx.x;
    const long long i0 = static_cast<long long>(t) * SMALL_PER;
    const int n = static_cast<int>(i0 < d ? (d - i0 < SMALL_PER ? d - i0 : SMALL_PER) : 0);   // entries held
    PrevSel ps{};
    if constexpr (DEFR) ps = read_sel(sel);
    float a[SMALL_PER];
    unsigned key[SMALL_PER];
    if (n == SMALL_PER) {
#pragma unroll
        for (int u = 0; u < SMALL_PER / 4; ++u) {
            const float4 m4 = reinterpret_cast<const float4*>(mem)[i0 / 4 + u];
            const float4 g4 = load_grad4<BF16>(grad, i0 / 4 + u);
            const float mv[4] = {m4.x, m4.y, m4.z, m4.w}, gv[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float m = mv[j];
                if constexpr (DEFR) m = mem_of(m, i0 + 4 * u + j, ps);
                a[4 * u + j] = ef_acc(m, eta, gv[j]);
            }
        }
    } else {
#pragma unroll
        for (int c = 0; c < SMALL_PER; ++c) {
            a[c] = 0.0f;
            if (c < n) {
                float m = mem[i0 + c];
                if constexpr (DEFR) m = mem_of(m, i0 + c, ps);
                a[c] = ef_acc(m, eta, load_grad1<BF16>(grad, i0 + c));
            }
        }
    }
#pragma unroll
    for (int c = 0; c < SMALL_PER; ++c) key[c] = key_of(a[c]);
    // level 1: key >> 19
    for (int b = t; b < H1_BINS; b += SMALL_THREADS) h[b] = 0u;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < SMALL_PER; ++c)
        if (c < n) atomicAdd(&h[key[c] >> H1_SHIFT], 1u);
    __syncthreads();
    select_bin<H1_BINS, 1, SMALL_THREADS>(h, H1_BINS, k, h, s_tmp, &s_bin, &s_above);
    const unsigned b1 = s_bin, above1 = s_above;
    // level 2: (key >> 7) & 4095 within b1
    for (int b = t; b < H2_BINS; b += SMALL_THREADS) h[b] = 0u;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < SMALL_PER; ++c)
        if (c < n && (key[c] >> H1_SHIFT) == b1) atomicAdd(&h[(key[c] >> H2_SHIFT) & (H2_BINS - 1)], 1u);
    __syncthreads();
    select_bin<H2_BINS, 1, SMALL_THREADS>(h, H2_BINS, k - above1, h, s_tmp, &s_bin, &s_above);
    const unsigned prefix2 = (b1 << 12) | s_bin, above2 = above1 + s_above;
    // level 3: key & 127 within prefix2
    for (int b = t; b < H3_BINS; b += SMALL_THREADS) h[b] = 0u;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < SMALL_PER; ++c)
        if (c < n && (key[c] >> H2_SHIFT) == prefix2) atomicAdd(&h[key[c] & (H3_BINS - 1)], 1u);
    __syncthreads();
    select_bin<H3_BINS, 1, SMALL_THREADS>(h, H3_BINS, k - above2, h, s_tmp, &s_bin, &s_above);
    const unsigned thr = (prefix2 << H2_SHIFT) | s_bin;
    const unsigned need = k - (above2 + s_above);   // ties of key thr taken, lowest indices first
    // one block scan of the packed per-thread counts (above thr in the low 16
    // bits, equal to thr in the high 16) places every entry
    unsigned cgt = 0, ceq = 0;
#pragma unroll
    for (int c = 0; c < SMALL_PER; ++c) {
        cgt += (c < n && key[c] > thr) ? 1u : 0u;
        ceq += (c < n && key[c] == thr) ? 1u : 0u;
    }
    const unsigned v = cgt | (ceq << 16);
    unsigned total;
    const unsigned excl = block_inclusive_scan<SMALL_THREADS / 64>(v, s_tmp, &total) - v;
    unsigned gt_before = excl & 0xFFFFu, eq_before = excl >> 16;
    int cut = -1;
    unsigned taken = 0;          // bit c: entry c selected
#pragma unroll
    for (int c = 0; c < SMALL_PER; ++c) {
        if (c < n) {
            const bool gt = key[c] > thr, eq = key[c] == thr;
            const bool take = gt || (eq && eq_before < need);
            if (take) {
                const unsigned pos = gt_before + (eq_before < need ? eq_before : need);
                out_idx[pos] = static_cast<int>(i0 + c);
                out_val[pos] = a[c];
                if (eq && eq_before + 1 == need) cut = static_cast<int>(i0 + c);
                taken |= 1u << c;
            }
            gt_before += gt ? 1u : 0u;
            eq_before += eq ? 1u : 0u;
        }
    }
    // explicit memory: the selected entries become +0.0; deferred: acc stays
    // and the record marks them
    const unsigned zero = sel ? 0u : taken;
    float* const mrow = mem + i0;
    if (n == SMALL_PER) {
#pragma unroll
        for (int u = 0; u < SMALL_PER / 4; ++u) {
            float4 x;
            x.x = (zero >> (4 * u)) & 1u ? 0.0f : a[4 * u];
            x.y = (zero >> (4 * u + 1)) & 1u ? 0.0f : a[4 * u + 1];
            x.z = (zero >> (4 * u + 2)) & 1u ? 0.0f : a[4 * u + 2];
            x.w = (zero >> (4 * u + 3)) & 1u ? 0.0f : a[4 * u + 3];
            reinterpret_cast<float4*>(mrow)[u] = x;
        }
    } else {
#pragma unroll
        for (int c = 0; c < SMALL_PER; ++c)
            if (c < n) mrow[c] = (zero >> c) & 1u ? 0.0f : a[c];
    }
    if (sel) {
        // the selection record of a deferred call: at most one thread holds
        // the cut (none when no tie is taken); thread 0 writes the record
        if (t == 0) s_bin = 0xFFFFFFFFu;
        __syncthreads();
        if (cut >= 0) s_bin = static_cast<unsigned>(cut);
        __syncthreads();
        if (t == 0) {
            sel[0] = thr;
            sel[1] = s_bin;
        }
    }
}

// ---------------------------------------------------------------- rand-k

// Rand-k with memory ("Sparsified SGD with Memory", method section): comp_k
// keeps k given coordinates.  One workgroup per RK_TILE entries: acc of the
// tile into LDS, the tile's slice of the (ascending) index list found by two
// wave searches, the selected values read out and zeroed in LDS, then the
// memory written once.  Indices outside [0, d) fall in no tile's slice.
constexpr int RK_TILE = 4096;

template <bool BF16>
__global__ __launch_bounds__(256) void randk_encode(const void* __restrict__ grad, float* __restrict__ mem, long long d,
                                                    float eta, const int* __restrict__ idx, long long k,
                                                    float* __restrict__ out_val) {
    __shared__ float4 s_acc4[RK_TILE / 4];
    __shared__ long long s_range[2];
    float* const s_acc = reinterpret_cast<float*>(s_acc4);
    const int t = threadIdx.x;
    const long long lo = static_cast<long long>(blockIdx.x) * RK_TILE;
    const long long hi = min(d, lo + RK_TILE);
    const int n = static_cast<int>(hi - lo);
    if (t < 64) {
        const long long a = wave_lower_bound(idx, k, lo);
        const long long b = wave_lower_bound(idx, k, hi);
        if (t == 0) {
            s_range[0] = a;
            s_range[1] = b;
        }
    }
    if (n == RK_TILE) {
        float4 g[4], m[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const long long i4 = lo / 4 + u * 256 + t;
            g[u] = load_grad4<BF16>(grad, i4);
            m[u] = reinterpret_cast<const float4*>(mem)[i4];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            s_acc4[u * 256 + t] = make_float4(ef_acc(m[u].x, eta, g[u].x), ef_acc(m[u].y, eta, g[u].y),
                                              ef_acc(m[u].z, eta, g[u].z), ef_acc(m[u].w, eta, g[u].w));
    } else {
        for (int e = t; e < n; e += 256) s_acc[e] = ef_acc(mem[lo + e], eta, load_grad1<BF16>(grad, lo + e));
    }
    __syncthreads();
    const long long a = s_range[0], b = s_range[1];
    for (long long j = a + t; j < b; j += 256) {
        const int e = static_cast<int>(idx[j] - lo);
        out_val[j] = s_acc[e];
        s_acc[e] = 0.0f;
    }
    __syncthreads();
    if (n == RK_TILE) {
#pragma unroll
        for (int u = 0; u < 4; ++u) reinterpret_cast<float4*>(mem)[lo / 4 + u * 256 + t] = s_acc4[u * 256 + t];
    } else {
        for (int e = t; e < n; e += 256) mem[lo + e] = s_acc[e];
    }
}

// Rank (from the top, among the sampled entries) whose level-1 bin edge is
// taken as the capture guess: the expected sample count above the threshold
// plus 25%, four standard deviations and 16, so that a sampled guess above
// the true threshold is practically impossible (it would only cost the
// re-reading capture pass).  >= the sample count: capture everything.
unsigned guess_rank(long long d, long long k) {
    const double S = static_cast<double>(d < SAMPLES ? d : SAMPLES);
    const double mean = S * static_cast<double>(k) / static_cast<double>(d);
    const double r = std::ceil(1.25 * mean + 4.0 * std::sqrt(mean) + 16.0);
    return r >= S ? static_cast<unsigned>(S) : static_cast<unsigned>(r);
}

int topk_encode(const char* fname, const void* grad, int grad_dtype, float* mem, int64_t d, float eta, int64_t k,
                int32_t* out_idx, float* out_val, unsigned* sel, bool deferred, bool has_prev, void* ws,
                size_t ws_bytes, void* stream) {
    const std::string fn(fname);
    if (!grad || !mem || !out_idx || !out_val || !ws)
        return fail(GC_ERR_ARG, fn + ": null pointer argument");
    if (grad_dtype != GC_F32 && grad_dtype != GC_BF16)
        return fail(GC_ERR_DTYPE, fn + ": grad_dtype must be GC_F32 or GC_BF16");
    if (d < 1 || d > INT32_MAX)
        return fail(GC_ERR_ARG, fn + ": d must be in [1, INT32_MAX]");
    if (k < 1 || k > d) return fail(GC_ERR_ARG, fn + ": k must be in [1, d]");
    if (!aligned16(grad) || !aligned16(mem) || !aligned16(out_idx) || !aligned16(out_val) || !aligned16(ws))
        return fail(GC_ERR_ARG, fn + ": device pointers must be 16-byte aligned");
    const size_t gbytes = static_cast<size_t>(d) * (grad_dtype == GC_BF16 ? 2 : 4);
    const size_t mbytes = static_cast<size_t>(d) * 4, kbytes = static_cast<size_t>(k) * 4;
    if (overlaps(out_idx, kbytes, mem, mbytes) || overlaps(out_val, kbytes, mem, mbytes) ||
        overlaps(out_idx, kbytes, out_val, kbytes) || overlaps(grad, gbytes, mem, mbytes) ||
        overlaps(out_idx, kbytes, grad, gbytes) || overlaps(out_val, kbytes, grad, gbytes))
        return fail(GC_ERR_ARG, fn + ": output buffers overlap an input or each other");
    if (deferred) {
        if (!sel) return fail(GC_ERR_ARG, fn + ": null selection record");
        if (!aligned16(sel)) return fail(GC_ERR_ARG, fn + ": the selection record must be 16-byte aligned");
        if (overlaps(sel, 16, mem, mbytes) || overlaps(sel, 16, grad, gbytes) || overlaps(sel, 16, out_idx, kbytes) ||
            overlaps(sel, 16, out_val, kbytes))
            return fail(GC_ERR_ARG, fn + ": the selection record overlaps another buffer");
    }
    unsigned* sel_out = deferred ? sel : nullptr;
    const bool defr = deferred && has_prev;
    const TopkLayout L = topk_layout(d);
    if (ws_bytes < L.total)
        return fail(GC_ERR_WORKSPACE, fn + ": workspace smaller than gc_topk_workspace_bytes");

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (d <= SMALL_D) {
        // one workgroup does the whole encode (the workspace is not touched)
        TimedLaunch tl("topk_small", s);
        const unsigned ku = static_cast<unsigned>(k);
        if (grad_dtype == GC_BF16 && defr)
            topk_small<true, true><<<1, SMALL_THREADS, 0, s>>>(grad, mem, d, eta, ku, out_idx, out_val, sel_out);
        else if (grad_dtype == GC_BF16)
            topk_small<true, false><<<1, SMALL_THREADS, 0, s>>>(grad, mem, d, eta, ku, out_idx, out_val, sel_out);
        else if (defr)
            topk_small<false, true><<<1, SMALL_THREADS, 0, s>>>(grad, mem, d, eta, ku, out_idx, out_val, sel_out);
        else
            topk_small<false, false><<<1, SMALL_THREADS, 0, s>>>(grad, mem, d, eta, ku, out_idx, out_val, sel_out);
        return check_launch("topk_small");
    }
    char* w = static_cast<char*>(ws);
    auto* st = reinterpret_cast<TopkState*>(w + L.state);
    auto* ctr = reinterpret_cast<unsigned*>(w + L.counters);
    auto* hist3 = ctr + HIST3_W;
    auto* tile_cnt = reinterpret_cast<unsigned*>(w + L.tile_cnt);
    auto* wg_gt = reinterpret_cast<unsigned*>(w + L.wg_gt);
    auto* wg_eq = reinterpret_cast<unsigned*>(w + L.wg_eq);
    auto* slot_idx = reinterpret_cast<int*>(w + L.slot_idx);
    auto* slot_val = reinterpret_cast<float*>(w + L.slot_val);
    const int ntiles = static_cast<int>(L.ntiles);
    const int small_grid = ntiles < TK_SMALL_GRID ? ntiles : TK_SMALL_GRID;
    const unsigned ku = static_cast<unsigned>(k);
    int rc;

    {
        TimedLaunch tl("topk_prep", s);
        const unsigned rank_g = guess_rank(d, k);
        uint4* zero = reinterpret_cast<uint4*>(w + L.zero_from);
        const int n16 = static_cast<int>((L.zero_end - L.zero_from) / 16);
        const dim3 g(1 + PREP_ZERO_BLOCKS);
        if (grad_dtype == GC_BF16 && defr)
            topk_prep<true, true><<<g, PREP_THREADS, 0, s>>>(grad, mem, d, eta, rank_g, st, zero, n16, sel);
        else if (grad_dtype == GC_BF16)
            topk_prep<true, false><<<g, PREP_THREADS, 0, s>>>(grad, mem, d, eta, rank_g, st, zero, n16, sel);
        else if (defr)
            topk_prep<false, true><<<g, PREP_THREADS, 0, s>>>(grad, mem, d, eta, rank_g, st, zero, n16, sel);
        else
            topk_prep<false, false><<<g, PREP_THREADS, 0, s>>>(grad, mem, d, eta, rank_g, st, zero, n16, sel);
        if ((rc = check_launch("topk_prep")) != GC_OK) return rc;
    }
    {
        TimedLaunch tl("topk_accum_hist", s);
        if (grad_dtype == GC_BF16 && defr)
            topk_accum_hist<true, true><<<ntiles, TK_THREADS, 0, s>>>(
                grad, mem, d, eta, st, ctr, slot_idx, slot_val, tile_cnt, sel);
        else if (grad_dtype == GC_BF16)
            topk_accum_hist<true, false><<<ntiles, TK_THREADS, 0, s>>>(
                grad, mem, d, eta, st, ctr, slot_idx, slot_val, tile_cnt, sel);
        else if (defr)
            topk_accum_hist<false, true><<<ntiles, TK_THREADS, 0, s>>>(
                grad, mem, d, eta, st, ctr, slot_idx, slot_val, tile_cnt, sel);
        else
            topk_accum_hist<false, false><<<ntiles, TK_THREADS, 0, s>>>(
                grad, mem, d, eta, st, ctr, slot_idx, slot_val, tile_cnt, sel);
        if ((rc = check_launch("topk_accum_hist")) != GC_OK) return rc;
    }
    {
        TimedLaunch tl("topk_capture", s);
        topk_capture<<<ntiles, TK_THREADS, 0, s>>>(mem, d, ku, st, ctr, slot_idx, slot_val, tile_cnt);
        if ((rc = check_launch("topk_capture")) != GC_OK) return rc;
    }
    {
        TimedLaunch tl("topk_select2", s);
        topk_select2<<<1, SEL_THREADS, 0, s>>>(ctr + HIST2_W, ku, st);
        if ((rc = check_launch("topk_select2")) != GC_OK) return rc;
    }
    {
        TimedLaunch tl("topk_refine", s);
        topk_refine<<<small_grid, TK_THREADS, 0, s>>>(st, hist3, slot_val, tile_cnt, ntiles);
        if ((rc = check_launch("topk_refine")) != GC_OK) return rc;
    }
    {
        TimedLaunch tl("topk_count", s);
        topk_count<<<small_grid, TK_THREADS, 0, s>>>(st, hist3, ku, slot_val, tile_cnt, ntiles, wg_gt, wg_eq,
                                                     sel_out);
        if ((rc = check_launch("topk_count")) != GC_OK) return rc;
    }
    {
        TimedLaunch tl("topk_emit", s);
        topk_emit<<<small_grid, TK_THREADS, 0, s>>>(st, slot_idx, slot_val, tile_cnt, wg_gt, wg_eq,
                                                    ntiles, ku, out_idx, out_val, mem, sel_out);
        if ((rc = check_launch("topk_emit")) != GC_OK) return rc;
    }
    return GC_OK;
}

}  // namespace
}  // namespace gc

using namespace gc;

extern "C" {

size_t gc_topk_workspace_bytes(int64_t d, int64_t k) {
    if (d < 1 || d > INT32_MAX || k < 1 || k > d) return 0;
    return topk_layout(d).total;
}

int gc_topk_ef_encode(const void* grad, int grad_dtype, float* mem, int64_t d, float eta,
                      int64_t k, int32_t* out_idx, float* out_val,
                      void* ws, size_t ws_bytes, void* stream) {
    return topk_encode("gc_topk_ef_encode", grad, grad_dtype, mem, d, eta, k, out_idx, out_val, nullptr, false, false,
                       ws, ws_bytes, stream);
}

int gc_topk_ef_encode_deferred(const void* grad, int grad_dtype, float* mem, int64_t d, float eta, int64_t k,
                               int32_t* out_idx, float* out_val, uint32_t* sel, int has_prev, void* ws,
                               size_t ws_bytes, void* stream) {
    return topk_encode("gc_topk_ef_encode_deferred", grad, grad_dtype, mem, d, eta, k, out_idx, out_val, sel, true,
                       has_prev != 0, ws, ws_bytes, stream);
}

int gc_topk_materialize(float* mem, int64_t d, const uint32_t* sel, void* stream) {
    if (!mem || !sel) return fail(GC_ERR_ARG, "gc_topk_materialize: null pointer argument");
    if (d < 1 || d > INT32_MAX) return fail(GC_ERR_ARG, "gc_topk_materialize: d must be in [1, INT32_MAX]");
    if (!aligned16(mem) || !aligned16(sel))
        return fail(GC_ERR_ARG, "gc_topk_materialize: device pointers must be 16-byte aligned");
    if (overlaps(sel, 16, mem, static_cast<size_t>(d) * 4))
        return fail(GC_ERR_ARG, "gc_topk_materialize: the selection record overlaps mem");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const long long blocks = std::min<long long>((d + 255) / 256, 4096);
    TimedLaunch tl("topk_materialize", s);
    topk_materialize<<<static_cast<unsigned>(blocks), 256, 0, s>>>(mem, d, sel);
    return check_launch("topk_materialize");
}

int gc_topk_decode(const int32_t* idx, const float* val, int64_t k, float* out, int64_t d,
                   int accumulate, void* stream) {
    if (!out) return fail(GC_ERR_ARG, "gc_topk_decode: null out");
    if (d < 1 || d > INT32_MAX) return fail(GC_ERR_ARG, "gc_topk_decode: d must be in [1, INT32_MAX]");
    if (k < 0 || k > d) return fail(GC_ERR_ARG, "gc_topk_decode: k must be in [0, d]");
    if (k > 0 && (!idx || !val)) return fail(GC_ERR_ARG, "gc_topk_decode: null idx/val");
    if (!aligned16(out) || (k > 0 && (!aligned16(idx) || !aligned16(val))))
        return fail(GC_ERR_ARG, "gc_topk_decode: device pointers must be 16-byte aligned");
    const size_t kb = static_cast<size_t>(k) * 4, db = static_cast<size_t>(d) * 4;
    if (k > 0 && (overlaps(out, db, idx, kb) || overlaps(out, db, val, kb)))
        return fail(GC_ERR_ARG, "gc_topk_decode: out overlaps idx/val");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (accumulate) {
        if (k == 0) return GC_OK;
        TimedLaunch tl("topk_decode_add", s);
        const long long blocks = (k + 255) / 256;
        topk_decode_add<<<static_cast<unsigned>(blocks), 256, 0, s>>>(idx, val, k, out, d);
        return check_launch("topk_decode_add");
    }
    TimedLaunch tl("topk_decode_set", s);
    const long long blocks = (d + DEC_TILE - 1) / DEC_TILE;
    topk_decode_set<<<static_cast<unsigned>(blocks), 256, 0, s>>>(idx, val, k, out, d);
    return check_launch("topk_decode_set");
}

int gc_randk_ef_encode(const void* grad, int grad_dtype, float* mem, int64_t d, float eta,
                       const int32_t* idx, int64_t k, float* out_val, void* stream) {
    if (!grad || !mem || !idx || !out_val) return fail(GC_ERR_ARG, "gc_randk_ef_encode: null pointer argument");
    if (grad_dtype != GC_F32 && grad_dtype != GC_BF16)
        return fail(GC_ERR_DTYPE, "gc_randk_ef_encode: grad_dtype must be GC_F32 or GC_BF16");
    if (d < 1 || d > INT32_MAX) return fail(GC_ERR_ARG, "gc_randk_ef_encode: d must be in [1, INT32_MAX]");
    if (k < 1 || k > d) return fail(GC_ERR_ARG, "gc_randk_ef_encode: k must be in [1, d]");
    if (!aligned16(grad) || !aligned16(mem) || !aligned16(idx) || !aligned16(out_val))
        return fail(GC_ERR_ARG, "gc_randk_ef_encode: device pointers must be 16-byte aligned");
    const size_t gbytes = static_cast<size_t>(d) * (grad_dtype == GC_BF16 ? 2 : 4);
    const size_t mbytes = static_cast<size_t>(d) * 4, kbytes = static_cast<size_t>(k) * 4;
    if (overlaps(out_val, kbytes, mem, mbytes) || overlaps(out_val, kbytes, grad, gbytes) ||
        overlaps(out_val, kbytes, idx, kbytes) || overlaps(idx, kbytes, mem, mbytes) || overlaps(grad, gbytes, mem, mbytes))
        return fail(GC_ERR_ARG, "gc_randk_ef_encode: buffers overlap");
    hipStream_t s = static_cast<hipStream_t>(stream);
    TimedLaunch tl("randk_encode", s);
    const long long blocks = (d + RK_TILE - 1) / RK_TILE;
    if (grad_dtype == GC_BF16)
        randk_encode<true><<<static_cast<unsigned>(blocks), 256, 0, s>>>(grad, mem, d, eta, idx, k, out_val);
    else
        randk_encode<false><<<static_cast<unsigned>(blocks), 256, 0, s>>>(grad, mem, d, eta, idx, k, out_val);
    return check_launch("randk_encode");
}

}  // extern "C"
