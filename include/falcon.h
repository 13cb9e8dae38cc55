/*
 * falcon.h -- C ABI of the Falcon fast-weight recurrence on AMD Instinct
 * MI355X (gfx950).
 *
 * The method ("Fast Weight Attention for Continual Learning", authors'
 * abstract): a fixed-size state S (d_v x d_k per batch and head) is updated
 * once per token as one step of an online learner on the prefix-aligned
 * example (x_t, y_t) = (k_{t-1}, v_t), and read after the write,
 * o_t = S_t q_t.  Each step first decays S by the positive gate alpha_t and
 * then applies a normalized first-order write (the KLA abstract on the same
 * listing gives the key-norm step eta_t / (||x_t||^2 + eps) and the
 * decay-then-delta order):
 *
 *   FALCON_F1   scalar NLMS:        S = S' + (y - S'x) u^T, u = eta x / (||x||^2 + eps)
 *   FALCON_F2   per-column NLMS:    same with u_j = eta x_j / (|x_j| ||x||_1 + eps)
 *   FALCON_F3   window mini-batch:  S = S' + b sum_{w<W} (y_{t-w} - S'x_{t-w}) x_{t-w}^T,
 *                                   b = eta / (sum_{w<W} ||x_{t-w}||^2 + eps)
 *   FALCON_F1A / F2A / F3A          inner-product counterparts: the target y is
 *                                   written instead of the residual.
 *   (S' = alpha_t S_{t-1}; the Falcon-2 and Falcon-3 formulas are this
 *   library's reading of "per-column extension" and "sliding-window
 *   mini-batch update"; the authors' text gives them in words only.)
 *
 * Alignment.  By default step t learns the prefix-aligned pair
 * (k_{t-1}, v_t).  OR-ing FALCON_SAME_STEP into the variant selects the
 * same-step pair (k_t, v_t), the alignment of the KLA / gated-delta-rule
 * recurrences the pages contrast the method with (with it, FALCON_F1 is KLA
 * with beta_t = eta_t / (||k_t||^2 + eps)).  Every entry point accepts the
 * flag; halos and caches keep their meaning (the last W keys, the last W-1
 * values), a same-step pair w simply takes k_{t-w} instead of k_{t-1-w}.
 *
 * Feature map.  The pages leave phi open and the default is the identity.
 * OR-ing FALCON_PHI_L2 (x / ||x||, 0 for a zero vector) or FALCON_PHI_SILU
 * (x / (1 + e^-x), elementwise) into the variant applies that map to every key
 * (halo and cache keys included) and every query before the step: x = phi(k),
 * o = S phi(q).  Halos and caches keep the raw keys.  For falcon_chunk_fwd the
 * mapped keys and queries go through the workspace (the size queries include
 * them when the flag is set).
 *
 * The abstract states that each rule has a chunk-parallel form with
 * positive-decay renormalization; falcon_chunk_fwd computes that form
 * (cumulative decays kept as chunk-local log sums, every factor a ratio
 * later/earlier <= 1).  falcon_decode_step (and falcon_decode_step_window for
 * the window rules) advances the recurrence by one token for many
 * independent heads.
 *
 * Conventions for every entry point
 *   - Pointers are device memory owned by the caller, except where noted.
 *     The library never allocates, frees or synchronizes, and keeps no
 *     global mutable state besides the per-device address of the scratch
 *     buffer built into it for falcon_chunk_fwd_noalloc (re-entrant;
 *     concurrent calls on different streams are safe when their buffers do
 *     not overlap, which for falcon_chunk_fwd_noalloc means: not on one GPU).
 *   - Work is enqueued on `stream` (NULL = the default stream); the call
 *     returns without waiting for it.
 *   - Arguments are validated on the host before anything is launched; an
 *     invalid argument returns its negative status and launches nothing.
 *     A launch failure reported by HIP returns FALCON_ERR_HIP.  Faults that
 *     happen later on the device surface at the caller's next
 *     synchronization, as HIP errors.
 *   - Layouts are contiguous and head-major: [B, H, T, d] for sequences,
 *     S row-major as [.., d_v, d_k] so that o = S q.
 *   - alpha must lie in (0, 1] and eta should be >= 0; values outside are
 *     not checked on the device and give undefined results.
 */
#ifndef FALCON_H
#define FALCON_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FALCON_OK = 0,
    FALCON_ERR_NULL = -1,        /* a required pointer is NULL */
    FALCON_ERR_SHAPE = -2,       /* a size is out of range or inconsistent */
    FALCON_ERR_UNSUPPORTED = -3, /* valid, but not in the support matrix below */
    FALCON_ERR_WORKSPACE = -4,   /* workspace missing or too small */
    FALCON_ERR_HIP = -5,         /* HIP reported an error at launch */
    FALCON_ERR_SCRATCH = -6      /* falcon_chunk_fwd_noalloc: the call needs more scratch
                                    than FALCON_NOALLOC_SCRATCH_BYTES */
} falcon_status;

/* Size of the built-in device scratch buffer of falcon_chunk_fwd_noalloc. */
#define FALCON_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

typedef enum {
    FALCON_F1 = 1,
    FALCON_F2 = 2,
    FALCON_F3 = 3,
    FALCON_F1A = 11,
    FALCON_F2A = 12,
    FALCON_F3A = 13,
    FALCON_SAME_STEP = 0x100, /* flag OR-ed into a variant: same-step pairs (k_t, v_t) */
    FALCON_PHI_L2 = 0x200,    /* flag: feature map x / ||x|| (0 for x = 0) on keys and queries */
    FALCON_PHI_SILU = 0x400   /* flag: feature map x / (1 + exp(-x)) on keys and queries */
} falcon_variant;

typedef enum { FALCON_FP32 = 0, FALCON_BF16 = 1 } falcon_dtype;

/*
 * Workspace bytes falcon_chunk_fwd needs for these arguments (0 when none).
 * Returns 0 as well for arguments falcon_chunk_fwd would reject.  The size
 * follows the kernels the forward runs (for the window rules at bf16 without
 * a feature map, the collapsed form's records); the backward and the saving
 * forward have their own queries.
 */
size_t falcon_chunk_fwd_workspace(int B, int H, int T, int dk, int dv, falcon_dtype dt,
                                  falcon_variant var, int window, int chunk);

/*
 * Chunk-parallel forward pass over whole sequences.
 *
 *   q, k      [B,H,T,dk]  dtype dt
 *   v         [B,H,T,dv]  dtype dt
 *   alpha     [B,H,T]     fp32, decay gate in (0,1]
 *   eta       [B,H,T]     fp32, step size (eta >= 0)
 *   S0        [B,H,dv,dk] fp32 initial state, or NULL for S0 = 0
 *   k_prev    [B,H,W,dk]  dtype dt: the W keys before the sequence,
 *                         k_{-W} .. k_{-1} (oldest first), or NULL for zeros
 *                         (then x_0 = 0 and step 0 writes nothing)
 *   v_prev    [B,H,W-1,dv] dtype dt: v_{-(W-1)} .. v_{-1}, or NULL for zeros
 *                         (ignored when W = 1)
 *   o         [B,H,T,dv]  dtype dt output, o_t = S_t q_t (rounded to nearest even
 *                         for bf16).  Must not alias any input.
 *   S_final   [B,H,dv,dk] fp32 output state S_T, or NULL to skip it.  May
 *                         alias S0 (read before written, per workgroup).
 *   W = window: 1 for F1/F2/F1A/F2A, 1..8 for F3/F3A.
 *   chunk: rows per tile of the chunk form, one of 16, 32, 64.  A tile holds
 *          floor(chunk / W) time steps, each contributing W window examples.
 *   eps > 0 is recommended (eps = 0 with a zero key divides 0 by 0).
 *   workspace / workspace_bytes: at least falcon_chunk_fwd_workspace(...)
 *          bytes of device memory (may be NULL when that is 0).
 *
 * Support matrix: dk = dv in {64, 128}; T >= 0 (T = 0 only copies S0 to
 * S_final); B*H >= 1; dt fp32 or bf16.  Continuing a sequence: pass the
 * previous call's S_final as S0 and its last W keys / W-1 values as
 * k_prev / v_prev; the result equals one call over the concatenation.
 */
int falcon_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                     const float* eta, const float* S0, const void* k_prev, const void* v_prev,
                     void* o, float* S_final, int B, int H, int T, int dk, int dv,
                     falcon_dtype dt, falcon_variant var, int window, int chunk, float eps,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * falcon_chunk_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the workspace is a scratch buffer built
 * into the library, FALCON_NOALLOC_SCRATCH_BYTES (128 MiB) of device memory
 * per GPU, which each GPU the library runs on holds until the process ends.
 * The call allocates nothing (no hipMalloc, no allocating library routine).
 *
 * Arguments, results and errors are those of falcon_chunk_fwd, plus
 * FALCON_ERR_SCRATCH when falcon_chunk_fwd_workspace(...) for these
 * arguments exceeds FALCON_NOALLOC_SCRATCH_BYTES (nothing is launched then).
 * The result equals falcon_chunk_fwd's bit for bit.
 *
 * Every call on one GPU shares that GPU's scratch buffer: calls that overlap
 * in time on one GPU (on different streams, or from different threads
 * without ordering between their streams) race and give undefined results.
 * Calls ordered on one stream are safe; the buffer keeps the last call's
 * contents and no call depends on what it held before.  The first call on a
 * device looks up that device's copy of the buffer (hipGetSymbolAddress)
 * with the device current; later calls reuse the address.
 */
int falcon_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* alpha,
                             const float* eta, const float* S0, const void* k_prev,
                             const void* v_prev, void* o, float* S_final, int B, int H, int T,
                             int dk, int dv, falcon_dtype dt, falcon_variant var, int window,
                             int chunk, float eps, hipStream_t stream);

/*
 * Chunk-parallel forward over N packed sequences of different lengths.  Each
 * head's plane holds the sequences back to back; the recurrence restarts at
 * every boundary, so the result equals one falcon_chunk_fwd call per
 * sequence.
 *
 *   q, k        [H,total_T,dk]  dtype dt
 *   v           [H,total_T,dv]  dtype dt
 *   alpha, eta  [H,total_T]     fp32
 *   cu_seqlens  [N+1] int32, device memory: sequence n covers rows
 *               cu_seqlens[n] .. cu_seqlens[n+1]-1 of every head's plane
 *               (non-decreasing, cu_seqlens[N] <= total_T, every length
 *               <= max_seqlen).  The device clamps offsets outside this
 *               contract so that no access leaves the buffers; the results
 *               for such offsets are unspecified.
 *   S0, S_final [N,H,dv,dk]  fp32 or NULL, per sequence (as in falcon_chunk_fwd)
 *   k_prev      [N,H,W,dk], v_prev [N,H,W-1,dv], or NULL: per-sequence halos
 *   o           [H,total_T,dv] dtype dt; rows outside every sequence are not
 *               written
 *   workspace   falcon_chunk_fwd_varlen_workspace(...) bytes (it grows with
 *               N * H * max_seqlen)
 *
 * Everything else (variants, FALCON_SAME_STEP, window, chunk, eps, support
 * matrix, errors) is as for falcon_chunk_fwd.
 */
size_t falcon_chunk_fwd_varlen_workspace(int N, int H, int max_seqlen, int dk, int dv,
                                         falcon_dtype dt, falcon_variant var, int window,
                                         int chunk);
int falcon_chunk_fwd_varlen(const void* q, const void* k, const void* v, const float* alpha,
                            const float* eta, const float* S0, const void* k_prev,
                            const void* v_prev, void* o, float* S_final, const int* cu_seqlens,
                            int N, int H, int total_T, int max_seqlen, int dk, int dv,
                            falcon_dtype dt, falcon_variant var, int window, int chunk, float eps,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Backward pass of falcon_chunk_fwd (the gradients of a loss through o and
 * S_T; "Fast Weight Attention for Continual Learning", authors' abstract: the
 * rules have a chunk-parallel form, whose derivative this computes).  Given
 * the forward's inputs and the cotangents d_o = dL/do and dS_final =
 * dL/dS_T, writes dL/d(q, k, v, alpha, eta, S0, k_prev).  The forward is
 * recomputed inside the call (its checkpoints live in the workspace).
 *
 *   q, k, v, alpha, eta, S0, k_prev, v_prev
 *               as for falcon_chunk_fwd (inputs of the forward)
 *   d_o         [B,H,T,dv]  dtype dt
 *   dS_final    [B,H,dv,dk] fp32, or NULL for zero
 *   dq, dk, dv  [B,H,T,d]   dtype dt outputs (rounded to nearest even)
 *   dalpha, deta [B,H,T]    fp32 outputs
 *   dS0         [B,H,dv,dk] fp32 output, or NULL (not wanted)
 *   dk_prev     [B,H,W,dk]  dtype dt output, or NULL (not wanted); zero where
 *               no pair reads the halo key (or k_prev is NULL)
 *   dv_prev     [B,H,W-1,dv] dtype dt output, or NULL (not wanted); zero
 *               where v_prev is NULL; unused for a window of one
 *   workspace   falcon_chunk_bwd_workspace(...) bytes: the forward's
 *               records, then the bf16 state at every tile start, the state
 *               gradient at every tile end and Delta of every tile (about
 *               B*H*ntiles*dk*(4 dk + 2 chunk) bytes, ntiles =
 *               ceil(T / (chunk / W))); with a window above one also the
 *               per-row gradients of the targets and keys (2 B*H*ntiles*
 *               chunk*dk*2 bytes), summed into dv / dk at the end
 * Outputs must not alias inputs or each other.
 *
 * Support matrix: dt bf16, dk = dv in {64, 128}, chunk 64, every variant
 * (window 1..8 for F3 / F3A), with FALCON_SAME_STEP and the feature-map
 * flags.  Other arguments that falcon_chunk_fwd accepts return
 * FALCON_ERR_UNSUPPORTED; errors otherwise as for falcon_chunk_fwd.
 * falcon_chunk_bwd_workspace returns 0 for unsupported arguments and T = 0.
 */
size_t falcon_chunk_bwd_workspace(int B, int H, int T, int dk, int dv, falcon_dtype dt,
                                  falcon_variant var, int window, int chunk);
int falcon_chunk_bwd(const void* q, const void* k, const void* v, const float* alpha,
                     const float* eta, const float* S0, const void* k_prev, const void* v_prev,
                     const void* d_o, const float* dS_final, void* dq, void* dk, void* dv,
                     float* dalpha, float* deta, float* dS0, void* dk_prev, void* dv_prev,
                     int B, int H, int T, int dk_dim, int dv_dim, falcon_dtype dt,
                     falcon_variant var, int window, int chunk, float eps, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * Backward pass of falcon_chunk_fwd_varlen: the gradients for N packed
 * sequences, in the layouts of that call (q, k, v, d_o and dq, dk, dv
 * [H,total_T,d]; gates and their gradients [H,total_T]; S0, dS_final, dS0,
 * the halos and their gradients per sequence).  Rows outside every sequence
 * are not written.  The result equals one falcon_chunk_bwd call per
 * sequence.  Support matrix and errors as for falcon_chunk_bwd; the
 * workspace is falcon_chunk_bwd_varlen_workspace(...) bytes (0 for
 * unsupported arguments).
 */
size_t falcon_chunk_bwd_varlen_workspace(int N, int H, int max_seqlen, int dk, int dv,
                                         falcon_dtype dt, falcon_variant var, int window,
                                         int chunk);
int falcon_chunk_bwd_varlen(const void* q, const void* k, const void* v, const float* alpha,
                            const float* eta, const float* S0, const void* k_prev,
                            const void* v_prev, const void* d_o, const float* dS_final, void* dq,
                            void* dk, void* dv, float* dalpha, float* deta, float* dS0,
                            void* dk_prev, void* dv_prev, const int* cu_seqlens, int N, int H,
                            int total_T, int max_seqlen, int dk_dim, int dv_dim, falcon_dtype dt,
                            falcon_variant var, int window, int chunk, float eps, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * Training form of the pair above (the chunk form and its derivative; "Fast
 * Weight Attention for Continual Learning", authors' abstract): the forward
 * and the backward of one step without recomputing the forward.  Callers that can hold the checkpoints
 * between the two calls (a training step) save the backward's forward
 * re-run this way; the results are those of falcon_chunk_fwd and
 * falcon_chunk_bwd (same kernels, same arithmetic).
 *
 * falcon_chunk_fwd_save: as falcon_chunk_fwd (same arguments and outputs),
 *   and it also leaves in `saved` the records and checkpoints the backward
 *   reads.  saved: falcon_chunk_bwd_workspace(...) bytes of device memory
 *   owned by the caller.  Support matrix as for falcon_chunk_bwd.  When
 *   S_final aliases S0 and falcon_chunk_fwd would run other kernels than the
 *   checkpoint run (window rules with W >= 2, Falcon-1A), S_final comes from
 *   the checkpoint run's kernels: the same recurrence, equal up to rounding
 *   (o is still falcon_chunk_fwd's, bit for bit).
 * falcon_chunk_bwd_saved: as falcon_chunk_bwd (same arguments and outputs),
 *   reading `saved` as a falcon_chunk_fwd_save call on the same inputs and
 *   sizes left it instead of re-running the forward (it also writes its own
 *   scratch regions there; the saved part stays intact, so it may be called
 *   again with other cotangents).  A `saved` buffer from other inputs, or
 *   not filled, gives meaningless results, not an error.
 * The _varlen forms pair falcon_chunk_fwd_varlen and falcon_chunk_bwd_varlen
 * in the same way, with falcon_chunk_bwd_varlen_workspace(...) bytes.
 */
int falcon_chunk_fwd_save(const void* q, const void* k, const void* v, const float* alpha,
                          const float* eta, const float* S0, const void* k_prev, const void* v_prev,
                          void* o, float* S_final, int B, int H, int T, int dk, int dv,
                          falcon_dtype dt, falcon_variant var, int window, int chunk, float eps,
                          void* saved, size_t saved_bytes, hipStream_t stream);
int falcon_chunk_bwd_saved(const void* q, const void* k, const void* v, const float* alpha,
                           const float* eta, const float* S0, const void* k_prev,
                           const void* v_prev, const void* d_o, const float* dS_final, void* dq,
                           void* dk, void* dv, float* dalpha, float* deta, float* dS0,
                           void* dk_prev, void* dv_prev, int B, int H, int T, int dk_dim,
                           int dv_dim, falcon_dtype dt, falcon_variant var, int window, int chunk,
                           float eps, void* saved, size_t saved_bytes, hipStream_t stream);
int falcon_chunk_fwd_varlen_save(const void* q, const void* k, const void* v, const float* alpha,
                                 const float* eta, const float* S0, const void* k_prev,
                                 const void* v_prev, void* o, float* S_final,
                                 const int* cu_seqlens, int N, int H, int total_T, int max_seqlen,
                                 int dk, int dv, falcon_dtype dt, falcon_variant var, int window,
                                 int chunk, float eps, void* saved, size_t saved_bytes,
                                 hipStream_t stream);
int falcon_chunk_bwd_varlen_saved(const void* q, const void* k, const void* v, const float* alpha,
                                  const float* eta, const float* S0, const void* k_prev,
                                  const void* v_prev, const void* d_o, const float* dS_final,
                                  void* dq, void* dk, void* dv, float* dalpha, float* deta,
                                  float* dS0, void* dk_prev, void* dv_prev, const int* cu_seqlens,
                                  int N, int H, int total_T, int max_seqlen, int dk_dim, int dv_dim,
                                  falcon_dtype dt, falcon_variant var, int window, int chunk,
                                  float eps, void* saved, size_t saved_bytes, hipStream_t stream);

/*
 * One decode step for N independent sequences x H heads (one token each):
 * x = k_cache (the previous key; with FALCON_SAME_STEP the new key k),
 * S' = alpha S, write as above, o = S q, then k_cache <- k.
 *
 *   S         [N,H,dv,dk] fp32, read and overwritten in place
 *   k_cache   [N,H,W,dk]  dtype dt, holds k_{t-1}; overwritten with k_t
 *   q, k      [N,H,dk]    dtype dt
 *   v         [N,H,dv]    dtype dt
 *   alpha,eta [N,H]       fp32
 *   o         [N,H,dv]    dtype dt output (must not alias inputs)
 *
 * Support matrix: var in {F1, F2, F1A, F2A} with window = 1; dk = dv in
 * {64, 128}; dt fp32 or bf16.
 */
int falcon_decode_step(float* S, void* k_cache, const void* q, const void* k, const void* v,
                       const float* alpha, const float* eta, void* o, int N, int H, int dk,
                       int dv, falcon_dtype dt, falcon_variant var, int window, float eps,
                       hipStream_t stream);

/*
 * One decode step of Falcon-3 / Falcon-3A (the sliding-window mini-batch
 * rule, "Fast Weight Attention for Continual Learning", authors' abstract)
 * for N sequences x H heads.  The window of the W most recent prefix-aligned
 * pairs is carried in two caches, newest first:
 *
 *   S         [N,H,dv,dk]  fp32, read and overwritten in place
 *   k_cache   [N,H,W,dk]   dtype dt, slot w holds k_{t-1-w} (x_{t-w});
 *                          on return slot 0 holds k_t and the rest moved one slot
 *   v_cache   [N,H,W-1,dv] dtype dt, slot w-1 holds v_{t-w} (y_{t-w}, w >= 1);
 *                          on return slot 0 holds v_t; may be NULL when W = 1
 *   q, k      [N,H,dk]     dtype dt
 *   v         [N,H,dv]     dtype dt (y_t)
 *   alpha,eta [N,H]        fp32
 *   o         [N,H,dv]     dtype dt output, o = S q after the write (must not
 *                          alias inputs)
 *
 * The step: S' = alpha S, b = eta / (sum_w ||x_{t-w}||^2 + eps), then
 * S = S' + b sum_w (y_{t-w} - S' x_{t-w}) x_{t-w}^T (Falcon-3A writes
 * y_{t-w} instead of the residual), o = S q: the step falcon_chunk_fwd takes
 * at time t.  With FALCON_SAME_STEP pair w's key is k_{t-w}: the new key k
 * for w = 0 and k_cache slot w-1 after (the last slot is then only carried).  Caches filled from a chunk call's halo: k_cache[w] = k_prev[W-1-w],
 * v_cache[w-1] = v_prev[W-1-w].
 *
 * Support matrix: var in {F3, F3A}; window W in 1..8; dk = dv in {64, 128};
 * dt fp32 or bf16.
 */
int falcon_decode_step_window(float* S, void* k_cache, void* v_cache, const void* q,
                              const void* k, const void* v, const float* alpha,
                              const float* eta, void* o, int N, int H, int dk, int dv,
                              falcon_dtype dt, falcon_variant var, int window, float eps,
                              hipStream_t stream);

/* Static, human-readable text for a status code (never NULL). */
const char* falcon_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FALCON_H */
