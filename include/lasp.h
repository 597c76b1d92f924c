/*
 * lasp.h - C ABI of the MI355X (gfx950) chunked causal linear attention library.
 *
 * What it computes (one head of one sequence, tokens p = 0..L-1, row vectors
 * q_p, k_p, v_p of length d, decay lambda; lambda = 1 means no decay):
 *
 *   kv_p  = lambda * kv_{p-1} + k_p^T v_p,   kv_{-1} = M_in,   o_p = q_p kv_p
 *   M_out = kv_{L-1}
 *
 * i.e. o_p = sum_{i<=p} lambda^(p-i) (q_p . k_i) v_i + lambda^(p+1) q_p M_in.
 * Sources: "Linear Attention Sequence Parallelism" (arXiv 2404.02882), Sec. 3.2,
 * Eqs. 4-6 (token form and recurrence), Eqs. 7-11 (chunked intra/inter form,
 * Algorithm 2) and Eqs. 12-23 (backward, Algorithm 3); "LASP-2: Rethinking
 * Sequence Parallelism for Linear Attention and Its Hybrid" (arXiv 2502.07563),
 * review page: the chunk memory state M_t = K_t^T V_t and its prefix sums.
 * The Norm(.) of LASP Eq. 2 is not applied (the derivations omit it); Q, K, V
 * are used as given (no feature map, no scaling).
 *
 * M_in stands for the state handed over by the previous device in the pages'
 * sequence-parallel scheme (LASP Alg. 2, the received KV_{t-1}); M_out is the
 * state that device would send on.  The backward takes dM_out (the gradient of
 * the following device) and returns dM_in (LASP Alg. 3, dKV sent back).
 *
 * Data layout (all device memory, row-major, contiguous):
 *   Q, K, V, O, dO, dQ, dK, dV : [B, H, N, d], element type = dtype
 *   M_in, M_out, dM_out, dM_in : [S, H, d, d] float32, row = key feature,
 *                                column = value feature; S = B, or nseq for a
 *                                packed batch
 *   decay                      : float32 [H] (lambda per head, in [0, 1]: the
 *                                decay of LASP Sec. 3.2), or NULL (= 1)
 *   cu_seqlens                 : int32 [nseq + 1] for a packed batch (B = 1,
 *                                N = total tokens, sequence i = tokens
 *                                [cu[i], cu[i+1]) of every head), else NULL
 * The state is reset at every sequence start of a packed batch.  Sequences may
 * be empty; N need not be a multiple of the chunk.
 *
 * Ownership and threading: the caller owns every buffer; the library never
 * allocates or frees memory.  Between calls it keeps only a per-thread copy of
 * the text of the last HIP error it saw (for lasp_status_string) and, once
 * lasp_fwd_noalloc has run on a GPU, that GPU's address of the static scratch
 * array (see there); calls of every other entry point on different threads and
 * streams are independent.  Calls are asynchronous on the
 * given HIP stream (hipStream_t passed as void*, NULL = the default stream):
 * buffers must stay alive until the stream reaches them.  Outputs are fully
 * overwritten; outputs must not overlap inputs.
 *
 * Errors: every argument is checked before anything is enqueued; on error
 * nothing runs and a lasp_status code is returned.  A launch that fails returns
 * LASP_EHIP with that launch's own error (an error left pending by the caller's
 * earlier HIP calls is neither reported nor cleared).  The contents of
 * cu_seqlens (monotone, cu[0] = 0, cu[nseq] = N) and of decay (every lambda in
 * [0, 1]) are trusted unless the environment has LASP_DEBUG=1: then each call
 * copies them to the host (synchronizing the stream) and returns LASP_EINVAL
 * if they are malformed.  Even unchecked, a malformed cu_seqlens cannot make
 * the kernels access memory outside the [B, H, N, d] tensors (sequence bounds
 * are clamped to [0, N]); the results are then meaningless, as they are for a
 * lambda outside [0, 1].  NaN/Inf inputs propagate.
 * Numbers: bf16 inputs are multiplied on bf16 MFMA with float32 accumulation;
 * states are float32 in HBM between kernels and rounded to bf16 where they are
 * MFMA operands.  float32 inputs use float32 MFMA throughout.
 */
#ifndef LASP_H
#define LASP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LASP_FP32 = 0, LASP_BF16 = 1 } lasp_dtype;

typedef enum {
    LASP_OK = 0,
    LASP_EINVAL = 1,        /* bad argument: dims, NULL, alignment, overlap, nseq/B */
    LASP_EUNSUPPORTED = 2,  /* d not in {32,64,128}, chunk not in {64,128,256}, dtype;
                               the gated and unmasked forms' own limits */
    LASP_EWORKSPACE = 3,    /* workspace_bytes smaller than the size query returns */
    LASP_EHIP = 4,          /* a HIP call or kernel launch failed */
    LASP_ESCRATCH = 5       /* lasp_fwd_noalloc: the call needs more scratch than its
                               static array holds */
} lasp_status;

/* B: batch; H: heads; N: tokens per sequence (packed batch: total tokens);
 * d: head dimension; chunk: chunk length C; nseq: 0, or the number of packed
 * sequences (then B must be 1 and cu_seqlens is required). */
typedef struct {
    int32_t B, H, N, d, chunk, nseq;
} lasp_shape;

/* Size in bytes of the state cache written by lasp_fwd and read by lasp_bwd:
 * the states the backward pass reuses (LASP Sec. 3.2, the cached KV_{t-1}):
 * per-chunk states (fp32) or the states entering each segment of chunks, and
 * each sequence's final state.  Depends only on the shape and dtype. */
size_t lasp_state_cache_bytes(const lasp_shape *shape, lasp_dtype dtype);

/* Workspace needed by lasp_fwd / lasp_bwd.  with_state_cache != 0 means the
 * call is given a state cache buffer; without one the workspace also holds the
 * states (and lasp_bwd recomputes them). */
size_t lasp_fwd_workspace_bytes(const lasp_shape *shape, lasp_dtype dtype,
                                int with_state_cache);
size_t lasp_bwd_workspace_bytes(const lasp_shape *shape, lasp_dtype dtype,
                                int with_state_cache);

/* All sizes at once, for an explicit segment length.  Work is split into
 * segments of G consecutive chunks (one workgroup sweeps a segment; states are
 * scanned across segments: the one-device form of LASP-2's prefix sum over the
 * gathered chunk states).  segment_chunks = 0 gives the library's choice of G,
 * a pure function of the shape and dtype, which the plain entry points and the
 * queries above use; segment_chunks > 0 forces G (a tuning and testing knob of
 * the _ex entry points).  form: 0 = causal and unmasked entry points, 1 = gated,
 * 2 = normalised (lasp_fwd_norm / lasp_bwd_norm: segment_chunks must be 0).
 * Returns LASP_OK and fills *out, or the status lasp_fwd would return for the
 * shape (LASP_EINVAL also for a negative segment_chunks or a NULL out). */
typedef struct {
    size_t state_cache;        /* bytes of the state cache */
    size_t fwd_workspace[2];   /* forward workspace: [0] without, [1] with a state cache */
    size_t bwd_workspace[2];   /* backward workspace: [0] without, [1] with a state cache */
    int segment_chunks;        /* G: chunks per segment used (the chunks of the gated
                                  form count 64 tokens) */
} lasp_sizes;
int lasp_query_sizes(const lasp_shape *shape, lasp_dtype dtype, int form, int segment_chunks,
                     lasp_sizes *out);

/* Forward pass (LASP Alg. 2 on one device; LASP-2 prefix sums of M_t).
 *   Q, K, V     inputs (required)
 *   decay       device float32 [H] or NULL
 *   cu_seqlens  device int32 [nseq+1] or NULL (nseq == 0)
 *   M_in        device float32 [S,H,d,d] or NULL (= zero state)
 *   O           output (required)
 *   M_out       output float32 [S,H,d,d] or NULL (not written)
 *   state_cache lasp_state_cache_bytes() bytes, or NULL; pass the same buffer to
 *               lasp_bwd to skip recomputing the states there
 *   workspace   lasp_fwd_workspace_bytes(shape, dtype, state_cache != NULL)
 *               bytes of device scratch (may be NULL if that size is 0)
 * All device pointers must be 16-byte aligned. */
int lasp_fwd(const lasp_shape *shape, lasp_dtype dtype,
             const void *Q, const void *K, const void *V,
             const float *decay, const int32_t *cu_seqlens, const float *M_in,
             void *O, float *M_out, void *state_cache,
             void *workspace, size_t workspace_bytes, void *stream);

/* Allocation-free forward, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Arguments and results as lasp_fwd, without the workspace: the
 * scratch lasp_fwd would take from its workspace (segment totals, packed-batch
 * tables, and the states when state_cache is NULL) lives in a static device
 * array of lasp_noalloc_scratch_bytes() bytes (64 MiB), one copy per GPU,
 * which each GPU the library runs on holds until the process ends.  The call
 * makes no hipMalloc / hipFree or other allocating call; its first call on a
 * GPU looks up that GPU's copy (hipGetSymbolAddress).  Every call on one GPU
 * shares that GPU's array and leaves its contents behind (nothing in it needs
 * to start at zero): calls that overlap in time on one GPU (other streams,
 * other threads) race and must not be issued.  Returns LASP_ESCRATCH, before
 * touching the device, when lasp_fwd_workspace_bytes(shape, dtype,
 * state_cache != NULL) exceeds the array (at d = 128, chunk 256: B1 H32 with
 * N up to 2^20 needs 16 to 32 MiB with a state cache, 34 to 66 MiB without).
 * A state cache written here is read by lasp_bwd as usual. */
size_t lasp_noalloc_scratch_bytes(void);
int lasp_fwd_noalloc(const lasp_shape *shape, lasp_dtype dtype,
                     const void *Q, const void *K, const void *V,
                     const float *decay, const int32_t *cu_seqlens, const float *M_in,
                     void *O, float *M_out, void *state_cache, void *stream);

/* Backward pass (LASP Alg. 3 on one device; LASP-2 suffix sums of dM_t) for the
 * loss l = <dO, O> + <dM_out, M_out>.
 *   Q, K, V, dO, decay, cu_seqlens, M_in : as given to lasp_fwd
 *   dM_out      device float32 [S,H,d,d] or NULL (= zero)
 *   state_cache the buffer lasp_fwd filled for the same inputs, or NULL
 *               (then the states are recomputed from K, V, M_in)
 *   dQ, dK, dV  outputs (required); dM_in output or NULL (not written)
 *   workspace   lasp_bwd_workspace_bytes(shape, dtype, state_cache != NULL) */
int lasp_bwd(const lasp_shape *shape, lasp_dtype dtype,
             const void *Q, const void *K, const void *V, const void *dO,
             const float *decay, const int32_t *cu_seqlens, const float *M_in,
             const float *dM_out, const void *state_cache,
             void *dQ, void *dK, void *dV, float *dM_in,
             void *workspace, size_t workspace_bytes, void *stream);

/* As lasp_fwd / lasp_bwd, plus two knobs:
 *   events          NULL, or an array of 4 hipEvent_t (created by the caller)
 *                   recorded on the stream before the segment-total kernel,
 *                   before the cross-segment scan, before the last kernel
 *                   (output, resp. gradients) and after it (per-kernel timing);
 *   segment_chunks  0 (the library's segment length, as lasp_fwd / lasp_bwd),
 *                   or G > 0 chunks per segment.  The state cache and the
 *                   workspace must then be sized by lasp_query_sizes with the
 *                   same G, and a lasp_bwd_ex that reads a state cache must get
 *                   the G of the lasp_fwd_ex that wrote it.
 * Nothing else changes. */
int lasp_fwd_ex(const lasp_shape *shape, lasp_dtype dtype,
                const void *Q, const void *K, const void *V,
                const float *decay, const int32_t *cu_seqlens, const float *M_in,
                void *O, float *M_out, void *state_cache,
                void *workspace, size_t workspace_bytes, void *stream, void **events,
                int segment_chunks);
int lasp_bwd_ex(const lasp_shape *shape, lasp_dtype dtype,
                const void *Q, const void *K, const void *V, const void *dO,
                const float *decay, const int32_t *cu_seqlens, const float *M_in,
                const float *dM_out, const void *state_cache,
                void *dQ, void *dK, void *dV, float *dM_in,
                void *workspace, size_t workspace_bytes, void *stream, void **events,
                int segment_chunks);

/* Normalised output: LASP Sec. 3.1, Eq. 2, O = Norm((Q K^T . M) V), which the
 * pages define only as "a normalization operation" and leave out of every
 * derivation.  Reading implemented: a root-mean-square normalisation of each
 * output row (one token of one head) over its d features, without a gain,
 *
 *   Y_p = o_p * rstd_p,   rstd_p = 1 / sqrt(mean_j o_pj^2 + LASP_NORM_EPS),
 *
 * o_p the causal output of lasp_fwd (decay, M_in, packed batches as there).
 * M_out is the carried state, not normalised.
 *   lasp_fwd_norm: as lasp_fwd, writing Y (the layout and dtype of O) and rstd
 *     (device float32 [B, H, N], one value per row, 4-byte aligned) instead of O.
 *   lasp_bwd_norm: as lasp_bwd for l = <dY, Y> + <dM_out, M_out>, given the
 *     forward's Y and rstd and the gradient dY (the layout of Y); it first
 *     forms dO = rstd (dY - Y mean_j(dY_j Y_j)) per row in the workspace, then
 *     runs lasp_bwd's kernels on it.  Its workspace is lasp_query_sizes(form
 *     2).bwd_workspace: lasp_bwd's plus one [B, H, N, d] array.
 * Errors as lasp_fwd / lasp_bwd (Y, rstd required). */
#define LASP_NORM_EPS 1e-6f
int lasp_fwd_norm(const lasp_shape *shape, lasp_dtype dtype,
                  const void *Q, const void *K, const void *V,
                  const float *decay, const int32_t *cu_seqlens, const float *M_in,
                  void *Y, float *rstd, float *M_out, void *state_cache,
                  void *workspace, size_t workspace_bytes, void *stream);
int lasp_bwd_norm(const lasp_shape *shape, lasp_dtype dtype,
                  const void *Q, const void *K, const void *V,
                  const void *Y, const float *rstd, const void *dY,
                  const float *decay, const int32_t *cu_seqlens, const float *M_in,
                  const float *dM_out, const void *state_cache,
                  void *dQ, void *dK, void *dV, float *dM_in,
                  void *workspace, size_t workspace_bytes, void *stream);

/* Unmasked (bidirectional) form: LASP Eq. 3 without Norm, every token attends
 * to every token of its sequence, no decay; with sequence parallelism each
 * device sums all chunk states (LASP-2 review page: one AllGather of the M_t,
 * then their sum M_(1:T)):
 *
 *   M = M_in + sum_i k_i^T v_i,   o_p = q_p M   (= sum_i (q_p . k_i) v_i + q_p M_in)
 *   M_out = M
 *
 * M_in stands for the summed states of the other devices' chunks.  The
 * backward, for l = <dO, O> + <dM_out, M_out>, returns
 *   dM = sum_p q_p^T do_p + dM_out,  dq_p = do_p M^T,  dk_j = v_j dM^T,
 *   dv_j = k_j dM,  dM_in = dM.
 * Arguments, layouts, size queries (the same shape gives the same workspace
 * and state-cache sizes as lasp_fwd / lasp_bwd; shape->chunk only sets the
 * work split) and errors as for lasp_fwd / lasp_bwd; there is no decay
 * argument.  Both dtypes (float32 computes the products in float32 MFMAs).
 * The state cache carries M from lasp_fwd_bidir to lasp_bwd_bidir. */
int lasp_fwd_bidir(const lasp_shape *shape, lasp_dtype dtype,
                   const void *Q, const void *K, const void *V,
                   const int32_t *cu_seqlens, const float *M_in,
                   void *O, float *M_out, void *state_cache,
                   void *workspace, size_t workspace_bytes, void *stream);
int lasp_bwd_bidir(const lasp_shape *shape, lasp_dtype dtype,
                   const void *Q, const void *K, const void *V, const void *dO,
                   const int32_t *cu_seqlens, const float *M_in,
                   const float *dM_out, const void *state_cache,
                   void *dQ, void *dK, void *dV, float *dM_in,
                   void *workspace, size_t workspace_bytes, void *stream);
/* The unmasked form with the knobs of lasp_fwd_ex / lasp_bwd_ex (the events
 * bracket the same three kernels: totals, scan, row-block products). */
int lasp_fwd_bidir_ex(const lasp_shape *shape, lasp_dtype dtype,
                      const void *Q, const void *K, const void *V,
                      const int32_t *cu_seqlens, const float *M_in,
                      void *O, float *M_out, void *state_cache,
                      void *workspace, size_t workspace_bytes, void *stream, void **events,
                      int segment_chunks);
int lasp_bwd_bidir_ex(const lasp_shape *shape, lasp_dtype dtype,
                      const void *Q, const void *K, const void *V, const void *dO,
                      const int32_t *cu_seqlens, const float *M_in,
                      const float *dM_out, const void *state_cache,
                      void *dQ, void *dK, void *dV, float *dM_in,
                      void *workspace, size_t workspace_bytes, void *stream, void **events,
                      int segment_chunks);

/* Gated form: a per-token, per-key-channel gate g_p in (0, 1]^d (LASP
 * Appendix A.4: the general recurrence of Eq. 24 with the GLA / GateLoop row
 * of Table 5):
 *
 *   kv_p = Diag(g_p) kv_{p-1} + k_p^T v_p,   kv_{-1} = M_in,   o_p = q_p kv_p
 *   M_out = kv_{L-1}
 *
 * i.e. o_p = sum_{i<=p} (q_p . (k_i * G_(i,p))) v_i + (q_p * G_(-1,p)) M_in with
 * G_(i,p) = g_(i+1) * ... * g_p per channel.  The gate scales the key rows of
 * the d x d state.  With every g_p = lambda this is lasp_fwd with decay lambda.
 *   log_g   device float32 [B, H, N, d] (the layout of Q): log g_p, finite and
 *           <= 0.  Larger values are accepted but products of gates above 1 may
 *           overflow.
 * The backward, for l = <dO, O> + <dM_out, M_out>, also returns
 *   dlog_g  device float32 [B, H, N, d]: dl/d(log g_p).
 * Chunking: the gated kernels work on chunks of 64 tokens whatever supported
 * length shape->chunk names (64, 128 or 256: the result does not depend on
 * it); sizes and segment_chunks count 64-token chunks.  Numbers: inside a chunk
 * the gates enter the bf16 MFMA operands as factors 2^(b_s - b_m) and
 * 2^(b_m - b_i) (b: running log2 of the gates; m: the first row of a 32-row
 * query tile), each at most 1 off the diagonal tiles; a diagonal tile whose
 * gates fall by more than 2^80 is summed pair by pair in float32 instead.
 * The log-gate gradient of a token is a suffix sum over the sequence; inside
 * a chunk it is summed token by token, across chunks it is carried from the
 * chunks' totals formed from the inter-chunk terms alone, and reset to its
 * exact value rowsum(R . P) of the states at every 8th chunk boundary and at
 * each segment's end.
 * Sizes come from the lasp_gated_* queries or lasp_query_sizes with form 1 (the
 * gated state cache holds the segment states, each sequence's final state and
 * the segments' gate products: no per-chunk data); buffers, pointers,
 * alignment, errors and the knobs of the _ex variants are as for lasp_fwd /
 * lasp_bwd (no decay argument). */
size_t lasp_gated_state_cache_bytes(const lasp_shape *shape, lasp_dtype dtype);
size_t lasp_gated_fwd_workspace_bytes(const lasp_shape *shape, lasp_dtype dtype,
                                      int with_state_cache);
size_t lasp_gated_bwd_workspace_bytes(const lasp_shape *shape, lasp_dtype dtype,
                                      int with_state_cache);
int lasp_fwd_gated(const lasp_shape *shape, lasp_dtype dtype,
                   const void *Q, const void *K, const void *V, const float *log_g,
                   const int32_t *cu_seqlens, const float *M_in,
                   void *O, float *M_out, void *state_cache,
                   void *workspace, size_t workspace_bytes, void *stream);
int lasp_bwd_gated(const lasp_shape *shape, lasp_dtype dtype,
                   const void *Q, const void *K, const void *V, const float *log_g,
                   const void *dO, const int32_t *cu_seqlens, const float *M_in,
                   const float *dM_out, const void *state_cache,
                   void *dQ, void *dK, void *dV, float *dlog_g, float *dM_in,
                   void *workspace, size_t workspace_bytes, void *stream);
int lasp_fwd_gated_ex(const lasp_shape *shape, lasp_dtype dtype,
                      const void *Q, const void *K, const void *V, const float *log_g,
                      const int32_t *cu_seqlens, const float *M_in,
                      void *O, float *M_out, void *state_cache,
                      void *workspace, size_t workspace_bytes, void *stream, void **events,
                      int segment_chunks);
int lasp_bwd_gated_ex(const lasp_shape *shape, lasp_dtype dtype,
                      const void *Q, const void *K, const void *V, const float *log_g,
                      const void *dO, const int32_t *cu_seqlens, const float *M_in,
                      const float *dM_out, const void *state_cache,
                      void *dQ, void *dK, void *dV, float *dlog_g, float *dM_in,
                      void *workspace, size_t workspace_bytes, void *stream, void **events,
                      int segment_chunks);

/* Human-readable text for a status code (for LASP_EHIP: the HIP error text of
 * the last call on the calling thread that returned LASP_EHIP). */
const char *lasp_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int lasp_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LASP_H */
