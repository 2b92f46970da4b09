/*
 * gc.h -- C ABI of the MI355X (gfx950) gradient-compressor library libgc.so.
 *
 * The library implements the per-step hot path of error-feedback gradient
 * compression for data-parallel training on one GPU:
 *   - Mem-SGD top-k sparsification with memory ("Sparsified SGD with Memory",
 *     method section: g_t = comp_k(m_t + eta*grad), m_{t+1} = m_t + eta*grad - g_t),
 *   - PowerSGD rank-r compression with the residual kept in memory (named as the
 *     low-rank compressor in the Accordion paper's method section and in the
 *     utility-of-compression paper's method/results sections),
 *   - the per-layer gradient norms and the two-level switch of Accordion
 *     (Accordion paper, method section: l_low / l_high chosen from the rate of
 *     change of the gradient norm).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller unless marked
 *     [host].  The library never allocates device memory and never frees
 *     anything the caller passed.
 *   - Scratch memory is passed as (ws, ws_bytes); query the size with the
 *     matching *_workspace_bytes function.  Contents of ws on entry are
 *     ignored; on return they are unspecified.
 *   - Calls only enqueue work on `stream` (a hipStream_t; NULL = the default
 *     stream) and return; nothing is synchronised.  gc_accordion_select is a
 *     pure host function.
 *   - Every device pointer must be 16-byte aligned.
 *   - Return value: GC_OK or an error code.  Arguments are validated before any
 *     work is enqueued, so a call that fails validation changes no buffer.
 *     gc_last_error() gives a message for the last failure on this thread.
 *   - Gradients may be float32 (GC_F32) or bfloat16 (GC_BF16); memory, factors
 *     and decoded outputs are always float32.
 *   - Results are deterministic: the same inputs give the same bits on every
 *     call (all reductions have a fixed order; no floating-point atomics).
 *   - Calls that share a workspace must not overlap in time (use one stream).
 *   - Process-wide state: the library keeps none in its compute calls, so
 *     calls on different streams with their own buffers are independent.  Two
 *     exceptions, both documented where declared: the measurement hooks
 *     (gc_timing_enable / gc_timing_read) and the per-device scratch array of
 *     the allocation-free entry point gc_grad_norm_noalloc.
 */
#ifndef GC_H
#define GC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define GC_OK            0
#define GC_ERR_ARG       1   /* a null/misaligned pointer, a size or rank out of range, aliasing */
#define GC_ERR_DTYPE     2   /* unknown gradient dtype */
#define GC_ERR_WORKSPACE 3   /* ws_bytes smaller than the query result */
#define GC_ERR_HIP       4   /* a HIP runtime call (kernel launch, event) failed */

/* gradient dtypes */
#define GC_F32  0
#define GC_BF16 1

/* Accordion levels */
#define GC_LEVEL_LOW  0   /* l_low: low compression, used in critical regimes */
#define GC_LEVEL_HIGH 1   /* l_high: high compression */

/* Static description of a status code; never NULL. */
const char* gc_status_str(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* gc_last_error(void);

/* ------------------------------------------------------------------------ */
/* Top-k sparsification with error-feedback memory                          */
/* ------------------------------------------------------------------------ */

/* Workspace bytes needed by gc_topk_ef_encode for a vector of d entries.
 * Returns 0 when (d, k) is out of range. */
size_t gc_topk_workspace_bytes(int64_t d, int64_t k);

/* One Mem-SGD encode step ("Sparsified SGD with Memory", method section):
 *     acc_i   = fl32(mem_i + fl32(eta * grad_i))   (two float32 roundings, no FMA)
 *     g_t     = top_k(acc)                         (k largest |acc_i|)
 *     mem_i  <- acc_i - g_t,i                      (+0.0 where selected)
 * The message is written as k (index, value) pairs in ascending index order:
 * out_idx[j] = i, out_val[j] = acc_i.  Among equal |acc| (including +x / -x)
 * the lower index is taken first; the selection is exact (no sampling).
 *
 *   grad      [d] float32 or bf16 (grad_dtype), read only
 *   mem       [d] float32, in/out: m_t on entry, m_{t+1} on return
 *   d         1 <= d <= INT32_MAX
 *   eta       step size, used as a float32 value
 *   k         1 <= k <= d
 *   out_idx   [k] int32, out
 *   out_val   [k] float32, out
 *   ws        >= gc_topk_workspace_bytes(d, k) bytes
 * Errors: GC_ERR_ARG (null pointer, d or k out of range, misalignment,
 * out_idx/out_val overlapping mem or each other), GC_ERR_DTYPE,
 * GC_ERR_WORKSPACE, GC_ERR_HIP.  NaN inputs are outside the contract. */
int gc_topk_ef_encode(const void* grad, int grad_dtype, float* mem, int64_t d, float eta,
                      int64_t k, int32_t* out_idx, float* out_val,
                      void* ws, size_t ws_bytes, void* stream);

/* The same top-k step with the memory in deferred form.  The selected
 * entries are not set to +0.0 in mem (a scattered write of k entries).
 * Instead mem keeps acc, and a 16-byte selection record `sel` (device,
 * caller-owned, 16-byte aligned) describes the selection:
 *   sel[0] = T     the threshold key (|x| bits without the sign)
 *   sel[1] = cut   the index of the last tie taken, as int32 (-1: none)
 * An entry i is selected, and +0.0 in the memory the method carries
 * (Sparsified SGD with Memory, method section), iff key(acc_i) > T, or
 * key(acc_i) == T and i <= cut.  The next deferred call reads the record in
 * its accumulate pass and takes those entries as +0.0.
 *   has_prev == 0: mem holds the memory itself (the first call, or after
 *                  gc_topk_materialize); sel is only written.
 *   has_prev != 0: mem and sel are as the previous deferred call left them.
 * out_idx and out_val get the bits of gc_topk_ef_encode.  mem becomes that
 * call's memory after gc_topk_materialize.
 * Errors: those of gc_topk_ef_encode, and GC_ERR_ARG for a NULL, misaligned
 * or overlapping sel. */
int gc_topk_ef_encode_deferred(const void* grad, int grad_dtype, float* mem, int64_t d, float eta, int64_t k,
                               int32_t* out_idx, float* out_val, uint32_t* sel, int has_prev, void* ws,
                               size_t ws_bytes, void* stream);

/* Writes a deferred top-k memory out: the entries sel marks become +0.0
 * (every entry is read; the selected ones are written).  Afterwards mem holds
 * the memory itself, and the next deferred call takes has_prev = 0.
 * Errors: GC_ERR_ARG (NULL, misaligned or overlapping pointers, d out of
 * [1, INT32_MAX]), GC_ERR_HIP. */
int gc_topk_materialize(float* mem, int64_t d, const uint32_t* sel, void* stream);

/* Dense decode of a top-k message (the scatter side of the same method):
 *   accumulate == 0:  out = 0 everywhere, then out[idx[j]] = val[j]
 *                     (idx must be strictly ascending, as gc_topk_ef_encode writes it)
 *   accumulate != 0:  out[idx[j]] += val[j] in float32 (idx must be unique)
 *   idx [k] int32, val [k] float32, out [d] float32; 0 <= k <= d; 1 <= d <= INT32_MAX.
 * Entries of idx outside [0, d) are ignored (never written).
 * Errors: GC_ERR_ARG, GC_ERR_HIP. */
int gc_topk_decode(const int32_t* idx, const float* val, int64_t k, float* out, int64_t d,
                   int accumulate, void* stream);

/* Rand-k sparsification with error-feedback memory ("Sparsified SGD with
 * Memory", method section: rand-k is the second k-contraction operator beside
 * top-k).  The caller draws the random subset and passes it in:
 *     acc = fl32(mem + fl32(eta*grad))          (as in gc_topk_ef_encode)
 *     out_val[j] = acc[idx[j]];  mem = acc, with mem[idx[j]] = +0.0
 * The message (idx, out_val) decodes with gc_topk_decode.
 *   grad      [d] float32 or bf16 (grad_dtype), read only
 *   mem       [d] float32, in/out
 *   idx       [k] int32, strictly ascending, within [0, d), read only
 *   out_val   [k] float32 out
 * No workspace.  Indices outside [0, d) are never dereferenced (their out_val
 * entries are not written); an index list that is not strictly ascending gives
 * unspecified values but no access outside the buffers.
 * Errors: GC_ERR_ARG (null pointer, d or k out of range, misalignment,
 * overlapping buffers), GC_ERR_DTYPE, GC_ERR_HIP. */
int gc_randk_ef_encode(const void* grad, int grad_dtype, float* mem, int64_t d, float eta,
                       const int32_t* idx, int64_t k, float* out_val, void* stream);

/* ------------------------------------------------------------------------ */
/* PowerSGD rank-r with error feedback                                      */
/* ------------------------------------------------------------------------ */

/* One matrix of a PowerSGD step.  M = mem + eta*grad is n x m, row-major
 * (a conv weight reshaped to out x (in*kh*kw)).  Q is m x rank and P is
 * n x rank, both column-major with leading dimensions m and n, so the first
 * columns stay in place when the rank changes. */
typedef struct gc_mat {
    const void* grad;  /* [n*m] float32 or bf16, read only                      */
    float* mem;        /* [n*m] in/out: memory before / residual after          */
    float* q;          /* [m*rank] in/out: warm-start Q in, new Q out           */
    float* p;          /* [n*rank] out: orthonormal P^ (may be NULL)            */
    float* out;        /* [n*m] out: decoded rank-r gradient P^ Q^T (may be NULL) */
    int32_t n, m;      /* 1 <= n, m; n*m <= INT32_MAX                            */
    int32_t rank;      /* 1 <= rank <= min(4, n, m)                             */
} gc_mat;

/* Workspace bytes for gc_powersgd_ef_step on these matrices ([host] array).
 * The workspace layout is planned from the shapes and their order (not the
 * ranks, dtype or pointers): query with the same array, in the same order,
 * that the step will receive.  Returns 0 when an entry is out of range. */
size_t gc_powersgd_workspace_bytes(const gc_mat* mats, int nmats);

/* One PowerSGD step with error feedback on every matrix of mats ([host], nmats >= 1):
 *     M   = mem + eta*grad
 *     P   = M Q;  P^ = Gram-Schmidt(P)  (a zero column stays zero)
 *     Q   = M^T P^                      (written back to q: warm start)
 *     out = P^ Q^T;  mem = M - out
 * float32 storage; the Gram matrix and the orthonormalisation are in float64.
 * Buffers of different matrices must not overlap.
 * The call copies a small matrix table (144 bytes per matrix) from host memory
 * into ws with one hipMemcpyAsync on `stream`, then enqueues the kernels; the
 * host array may be reused as soon as the call returns.  Because of that copy
 * the call is not for graph capture (a replay would read freed host memory).
 * Errors: GC_ERR_ARG, GC_ERR_DTYPE, GC_ERR_WORKSPACE, GC_ERR_HIP. */
int gc_powersgd_ef_step(const gc_mat* mats, int nmats, int grad_dtype, float eta,
                        void* ws, size_t ws_bytes, void* stream);

/* The same PowerSGD step with the error-feedback memory kept in deferred form.
 * The memory the method carries to the next step, m' = M - P^ Q^T, is not
 * written out.  It is held as three parts instead: mem keeps M, p keeps P^
 * (the first `rank` columns) and q keeps Q.  The next deferred call rebuilds
 * m' from them in its first pass over mem, then forms M = m' + eta*grad and
 * stores M over mem.  The output pass writes only out and p.
 *
 * This is the memory convention of Mem-SGD (Sparsified SGD with Memory,
 * method section: the memory keeps what the compressed update left out),
 * held as the factors that define it.
 * Each entry moves (grad bytes + 12) bytes per step instead of
 * (grad bytes + 12) + (grad bytes + 4): M is read once, not twice.
 * out, q and p get the bits of gc_powersgd_ef_step.  After
 * gc_powersgd_materialize, mem holds that call's bits too (the residual is
 * formed with the same float32 operations in the same order).
 *
 * prev_rank ([host], nmats entries) says what mem holds on entry:
 *   0      mem holds the memory itself (the first call, or after
 *          gc_powersgd_materialize);
 *   r' > 0 mem holds M of the previous deferred call, and its P^ and Q are
 *          still in the first r' columns of p and q.  r' is that call's rank.
 * On return mem holds M of this call: pass prev_rank[i] = mats[i].rank next
 * time.
 * On a rank change, columns past r' of q may be refilled (a warm start for a
 * higher rank) before the call.  The first min(r', rank) columns must be
 * left as the previous call wrote them.
 * p is required (non-NULL), since it carries P^ to the next call.
 * Workspace: gc_powersgd_workspace_bytes on the same array.
 * Errors: those of gc_powersgd_ef_step, and GC_ERR_ARG for a NULL prev_rank,
 * a NULL p, or prev_rank[i] outside [0, min(4, n, m)]. */
int gc_powersgd_ef_step_deferred(const gc_mat* mats, const int32_t* prev_rank, int nmats, int grad_dtype,
                                 float eta, void* ws, size_t ws_bytes, void* stream);

/* ---- Recorded PowerSGD steps: upload once, then launch kernels only ---- */

/* Host bytes of a plan for nmats matrices (0 for NULL mats or nmats < 1). */
size_t gc_powersgd_plan_bytes(const gc_mat* mats, int nmats);

/* Records one PowerSGD step of these matrices for gc_powersgd_run.  It checks
 * every argument exactly as the step would.  It copies the matrix table into
 * ws with one hipMemcpyAsync on `stream`, and it writes the launch parameters
 * into `plan` (caller-owned host memory of gc_powersgd_plan_bytes bytes, any
 * alignment).  Nothing is launched.
 *   prev_rank == NULL: the step of gc_powersgd_ef_step (explicit memory);
 *   prev_rank != NULL: the step of gc_powersgd_ef_step_deferred with these
 *                      previous ranks ([host], nmats entries).
 * The plan fixes pointers, shapes, ranks and previous ranks; eta is given
 * per run.  A deferred plan made with prev_rank = rank describes every step
 * after the first one at unchanged ranks.
 * Errors: those of the recorded step, and GC_ERR_ARG for a NULL plan or
 * plan_bytes below gc_powersgd_plan_bytes. */
int gc_powersgd_plan(const gc_mat* mats, const int32_t* prev_rank, int nmats, int grad_dtype, void* plan,
                     size_t plan_bytes, void* ws, size_t ws_bytes, void* stream);

/* Runs a recorded step on `stream`: kernel launches only.  There is no copy,
 * no allocation and no host synchronisation, so the call may be captured in a
 * HIP graph.  It computes what the recorded call would compute on the
 * buffers' contents at run time.
 * The buffers named in the plan must still be valid.  ws must be the
 * workspace given to gc_powersgd_plan, with no other PowerSGD call on it
 * since.  The run must be ordered after the plan call's table copy: use the
 * same stream, or synchronise.
 * Errors: GC_ERR_ARG for a NULL, short or foreign plan, or another ws;
 * GC_ERR_HIP. */
int gc_powersgd_run(const void* plan, size_t plan_bytes, float eta, void* ws, void* stream);

/* One or both phases of a recorded step.  The utility-of-compression paper's
 * method section splits a compressed step into encode, exchange and decode;
 * for the low-rank compressor the P and Q products are the encode and
 * out = P^ Q'^T is the decode.
 *   phases = 1 (encode): the first passes and the Q reduction.  On return
 *            (in stream order) q holds Q' = M^T P^, and the workspace holds
 *            P and the triangular factor T with P^ = P T.  For explicit
 *            memory, mem is not yet updated.
 *   phases = 2 (decode): the output pass.  It writes out, and P^ into p.
 *            For explicit memory it also writes mem = M - out.  It must run
 *            after the encode of the same plan, with no other run of the
 *            plan in between.
 *   phases = 3: both, the same as gc_powersgd_run.
 * Between the two phases the stream may carry unrelated work, or other
 * streams may run beside the decode.  The split point is where a
 * data-parallel step would exchange Q'.  That alone would not make a correct
 * multi-worker step: the fused encode forms M^T P from this worker's own P
 * before orthonormalising, whereas a multi-worker step has to reduce P over
 * the workers first, which needs the encode split again (P pass, exchange of
 * P, then the Q pass).  These phases are the single-worker step.
 * Errors: those of gc_powersgd_run, and GC_ERR_ARG for phases outside 1..3. */
int gc_powersgd_run_phases(const void* plan, size_t plan_bytes, float eta, void* ws, int phases, void* stream);

/* Writes the deferred memory out: for every matrix with prev_rank[i] > 0,
 * mem = mem - P^ Q^T over the first prev_rank[i] columns of p and q.
 * Afterwards mem holds m', bit for bit what gc_powersgd_ef_step would have
 * left there, and the next step takes prev_rank 0.
 * Reads mem, p and q; grad, rank and out are not used (grad may be NULL).
 * Matrices with prev_rank[i] == 0 are left alone.
 * Workspace: gc_powersgd_workspace_bytes on the same array.
 * Errors: GC_ERR_ARG (NULL mats, prev_rank, mem, q or p -- p is checked
 * for every matrix; prev_rank out of range; misaligned or overlapping
 * buffers), GC_ERR_WORKSPACE, GC_ERR_HIP. */
int gc_powersgd_materialize(const gc_mat* mats, const int32_t* prev_rank, int nmats, void* ws, size_t ws_bytes,
                            void* stream);

/* ------------------------------------------------------------------------ */
/* Tensors sent uncompressed                                                 */
/* ------------------------------------------------------------------------ */

/* One vector sent without compression (a batch-norm scale or shift, a bias). */
typedef struct gc_vec {
    const void* grad;  /* [len] float32 or bf16, read only   */
    float* out;        /* [len] float32 out                  */
    int64_t len;       /* 1 <= len <= INT32_MAX              */
} gc_vec;

/* The step of the tensors a gradient set sends as they are: the compressors
 * of the Accordion paper's method section work on the weight matrices, and
 * the vectors of the set (batch-norm parameters, biases) go out uncompressed:
 *     out = fl32(eta * grad)            (one float32 rounding)
 * They keep no error-feedback memory: nothing is left out.  One launch per
 * 120 vectors ([host] array vecs, nvecs >= 1).
 * Errors: GC_ERR_ARG (null pointer, len out of range, misalignment, an out
 * overlapping any gradient or another out), GC_ERR_DTYPE, GC_ERR_HIP. */
int gc_passthrough(const gc_vec* vecs, int nvecs, int grad_dtype, float eta, void* stream);

/* ------------------------------------------------------------------------ */
/* Accordion: per-layer norms and the l_low / l_high switch                 */
/* ------------------------------------------------------------------------ */

typedef struct gc_span {
    const void* ptr;   /* device pointer to one layer's gradient */
    int64_t len;       /* elements, >= 1 */
} gc_span;

/* Workspace bytes for gc_grad_norm on these layers ([host] array). */
size_t gc_grad_norm_workspace_bytes(const gc_span* layers, int nlayers);

/* norms[l] = ||layer l||_2 for every layer in one pass (the quantity whose
 * rate of change Accordion's method section monitors).  Squares are summed in
 * float64; norms [nlayers] float32 device output.
 * Errors: GC_ERR_ARG, GC_ERR_DTYPE, GC_ERR_WORKSPACE, GC_ERR_HIP. */
int gc_grad_norm(const gc_span* layers, int nlayers, int grad_dtype, float* norms,
                 void* ws, size_t ws_bytes, void* stream);

/* Tiles (16384 entries each) of the per-device scratch of gc_grad_norm_noalloc. */
#define GC_NORM_SCRATCH_TILES 65536

/* gc_grad_norm without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops, harnesses that forbid
 * allocation).  The float64 tile partials go to a fixed scratch array that
 * the library holds on each device (512 KiB, GC_NORM_SCRATCH_TILES tiles)
 * until the process ends.  The call allocates nothing.
 *   - The calling thread's current device must be the device of `stream`
 *     and of the buffers; the first call on a device looks up that device's
 *     scratch address once.
 *   - Limit: the sum over layers of ceil(len / 16384) must be at most
 *     GC_NORM_SCRATCH_TILES (2^30 entries in all when every len is a
 *     multiple of 16384); larger calls fail with GC_ERR_ARG.
 *   - Every call on a device shares that device's scratch: calls that overlap
 *     in time on one device (different streams, other threads) race and give
 *     wrong norms.  Calls on one stream are ordered and safe.  Nothing in the
 *     scratch needs clearing: every partial a call reads it writes first.
 * Results are bit for bit those of gc_grad_norm (same kernels, same order).
 * Errors: those of gc_grad_norm (without GC_ERR_WORKSPACE), GC_ERR_ARG above
 * the limit, GC_ERR_HIP when the scratch address cannot be looked up. */
int gc_grad_norm_noalloc(const gc_span* layers, int nlayers, int grad_dtype, float* norms, void* stream);

/* Host-only level choice for one check (Accordion, method section), per layer l:
 *   has_prev == 0            -> GC_LEVEL_LOW
 *   rho = |prev - now| / prev (prev == 0: rho = +inf if now > 0, else 0)
 *   rho >= threshold         -> GC_LEVEL_LOW (critical regime), else GC_LEVEL_HIGH
 * then norm_prev[l] = norm_now[l].  rho is computed in double.
 *   norm_now [host, nlayers], norm_prev [host, nlayers] in/out, level [host, nlayers] out.
 * Errors: GC_ERR_ARG (null pointer, nlayers < 1, negative or NaN threshold). */
int gc_accordion_select(const float* norm_now, float* norm_prev, int nlayers, float threshold,
                        int has_prev, int* level);

/* ------------------------------------------------------------------------ */
/* Measurement hooks                                                         */
/* ------------------------------------------------------------------------ */

/* Bracket every launch of the kernel named `kernel_name` (as listed by
 * gc_kernel_names) with a pair of HIP events recorded on the launch stream;
 * NULL or "" switches timing off and drops recorded events.
 * These hooks are process-wide state (one timed kernel name and its recorded
 * events, behind a mutex).  With timing off a launch only reads one atomic
 * flag and takes no lock. */
int gc_timing_enable(const char* kernel_name);

/* Synchronise on the recorded events and return the summed duration (ms) and
 * the number of launches timed since gc_timing_enable; clears the record. */
int gc_timing_read(double* total_ms, int64_t* launches);

/* Comma-separated names of the library's kernels (static string). */
const char* gc_kernel_names(void);

#ifdef __cplusplus
}
#endif

#endif /* GC_H */
