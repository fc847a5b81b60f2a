/*
 * kdn.h -- C ABI of libkdn, a gfx950 (MI355X) implementation of the forward
 * pass and the one-token decode step of the Kalman Delta Network (KDN) layer.
 *
 * Model (sources: "Kalman Delta Networks: Uncertainty-aware Associative
 * Memory", English abstract; ai-feeds.com summary of the same paper, section
 * "方法 / 关键模块", steps 1-3):
 *   Each head keeps a memory S (d_v x d_k) read as the latent state of a
 *   linear-Gaussian state-space model; token t is the noisy observation
 *   v_t = S k_t + N(0, r_t).  The transition scales the memory by a_t and adds
 *   process noise of variance qnoise_t.  The rows of S share one covariance,
 *   approximated as diagonal (one precision per key dimension, "Diagonal
 *   KDN") or isotropic (one precision per head, "Isotropic KDN").  Per token:
 *     lambda^- = lambda / (a^2 + qnoise * lambda)                (predict)
 *     w        = P^- k / (k^T P^- k + r),   P^- = 1 / lambda^-   (Kalman gain)
 *     lambda   = lambda^- + k.k / r     (diagonal: keep the posterior diagonal)
 *              = lambda^- + |k|^2 / (d_k r)   (isotropic: mean over key dims)
 *     S_t      = a S_{t-1} + (v - a S_{t-1} k) w^T,   o_t = S_t q_t
 *   The precision recurrence is the Moebius map of the 2x2 matrix
 *   [[1 + b qnoise, b a^2], [qnoise, a^2]] (b = k_i^2 / r, or |k|^2/(d_k r)),
 *   so it is computed with an associative scan (same pages: the uncertainty
 *   recurrences are Moebius maps admitting log-depth associative scans).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers, contiguous, head-major:
 *       q, k [B,H,T,d_k]   v, o [B,H,T,d_v]   a, qnoise, r [B,H,T]
 *       lambda [B,H,d_k] (diagonal) or [B,H] (isotropic), float32
 *       S [B,H,d_v,d_k] row-major, float32
 *   - Element types come from the descriptor (KDN_F32 = float,
 *     KDN_BF16 = bfloat16 stored as uint16).  State (S, lambda) is float32.
 *   - The caller owns every buffer, including the workspace; the library
 *     never allocates device memory, never synchronises the stream and keeps
 *     no state between calls.  Work is enqueued on `stream` (a hipStream_t;
 *     NULL = the default stream) and is asynchronous.
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued and reported as a kdn_status; KDN_ERR_HIP means a launch was
 *     rejected by the HIP runtime.  Faults inside a kernel surface at the
 *     caller's next synchronisation.  No C++ exception crosses this ABI.
 *   - Preconditions that are not checked on the device: r > 0, 0 < a <= 1,
 *     qnoise >= 0, lambda0 > 0, all inputs finite.
 */
#ifndef KDN_H
#define KDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KDN_DIAGONAL = 0, KDN_ISOTROPIC = 1 } kdn_variant;
typedef enum { KDN_F32 = 0, KDN_BF16 = 1 } kdn_dtype;
typedef enum {
    KDN_OK = 0,
    KDN_ERR_NULL = 1,        /* a required pointer is NULL */
    KDN_ERR_SHAPE = 2,       /* negative or inconsistent sizes */
    KDN_ERR_UNSUPPORTED = 3, /* size / dtype / chunk combination not built */
    KDN_ERR_WORKSPACE = 4,   /* workspace smaller than the *_workspace_bytes answer */
    KDN_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned */
    KDN_ERR_HIP = 6          /* the HIP runtime rejected a launch */
} kdn_status;

/* Problem description.  Supported: d_k, d_v in {32, 64, 128}; chunk in
 * {16, 32, 64} (float32 inputs with d_k = 128 need chunk <= 32: the
 * chunk kernel's LDS budget); any T >= 0 (a last partial chunk is masked);
 * B, H >= 0 with B*H <= 65535 for the chunked entry points.
 * qkv_dtype is the type of q, k, v and o; gate_dtype the type of a, qnoise
 * and r; gain_dtype the type of the gain keys w that kdn_gain writes and
 * kdn_chunk_delta reads (must equal qkv_dtype for kdn_chunk_delta). */
typedef struct {
    int32_t B, H, T, d_k, d_v, chunk;
    int32_t variant;    /* kdn_variant */
    int32_t qkv_dtype;  /* kdn_dtype */
    int32_t gate_dtype; /* kdn_dtype */
    int32_t gain_dtype; /* kdn_dtype */
} kdn_desc;

/* Human-readable text of a status; never NULL. */
const char *kdn_status_string(kdn_status s);

/* Host-only check of a descriptor (no GPU call).  KDN_OK if every entry point
 * that takes it supports it. */
kdn_status kdn_validate(const kdn_desc *d);

/* Bytes of device workspace kdn_forward needs for this descriptor (0 if the
 * descriptor is invalid).  Host-only. */
size_t kdn_forward_workspace_bytes(const kdn_desc *d);

/* Number of sequence segments the chunk state pass of kdn_forward runs over
 * for this descriptor (host-only; 0 if the descriptor is invalid).  1: one
 * sequential pass per (head, d_v tile).  With few heads and many chunks
 * (fewer than 128 such workgroups and at least 16 chunks) each head's chunks
 * may be cut into segments of consecutive chunks, their count chosen by an
 * estimate of each split's run time: every segment's memory update is an
 * affine map S -> S A + B of its start state (the rows of S evolve
 * independently, each by the same matrix A), so the maps of segments 1 ..
 * n - 2 are formed in parallel beside segment 0's own read-out, composed in
 * order, and segments 1 .. n - 1 then run their read-out from their own start
 * states.  The result is the same recurrence re-associated (up to rounding);
 * the workspace holds the maps. */
int32_t kdn_forward_segments(const kdn_desc *d);

/* Full layer forward (predict, gain, projection, chunkwise memory write and
 * read-out for all T tokens of all B*H heads).
 *   lambda0: NULL -> all ones; S0: NULL -> zeros (the posterior at t = 0).
 *   o: output [B,H,T,d_v] in qkv_dtype.
 *   S_T, lambda_T: NULL or outputs; S_T may alias S0 and lambda_T may alias
 *   lambda0 (read before written); o must not alias an input.
 *   ws: device workspace of at least kdn_forward_workspace_bytes(d) bytes,
 *   16-byte aligned; its contents on entry are ignored. */
kdn_status kdn_forward(const kdn_desc *d, const void *q, const void *k, const void *v,
                       const void *a, const void *qnoise, const void *r,
                       const float *lambda0, const float *S0, void *o, float *S_T,
                       float *lambda_T, void *ws, size_t ws_bytes, void *stream);

/* kdn_forward with timing: events is NULL or an array of 8 hipEvent_t
 * (entries may be NULL) created by the caller; events 2i and 2i + 1 are the
 * start and stop of kernel i (0 scan reduce, 1 scan carry, 2 chunk prep,
 * 3 chunk state), handed to the kernel dispatches (hipExtLaunchKernel) on
 * `stream`.  The HIP runtime records them with packets of its own around each
 * dispatch, which put a few microseconds between the kernels and can slow the
 * kernel that follows; kdn_forward_repeat times the kernels without them.
 * Otherwise identical to kdn_forward. */
kdn_status kdn_forward_events(const kdn_desc *d, const void *q, const void *k, const void *v,
                              const void *a, const void *qnoise, const void *r,
                              const float *lambda0, const float *S0, void *o, float *S_T,
                              float *lambda_T, void *ws, size_t ws_bytes, void *stream,
                              void *const *events);

/* Timing aid: kernels first..last of kdn_forward (0 scan reduce, 1 scan
 * carry, 2 chunk prep, 3 chunk state -- for few heads over long sequences the
 * three launches of the segmented state pass), in order, `reps` times over,
 * back to back on `stream`, with the arguments kdn_forward takes.  The time
 * between two events around a call, divided by reps, is the time of those
 * kernels as they run in the forward; differences between calls that stop one
 * kernel apart give each kernel's own duration without events between the
 * kernels (the HIP runtime records such events with packets of its own, which
 * put microseconds between the kernels and slow the one that follows).  A
 * range not starting at 0 reads what the kernels before it left in ws: ws must
 * hold what a kdn_forward call with the same arguments left there.  Every pass
 * rewrites the same values into ws and the outputs.  S_T must not alias S0 nor
 * lambda_T alias lambda0 here (KDN_ERR_SHAPE, as for a range outside 0-3 or
 * reps < 0); otherwise the argument checks and errors are kdn_forward's. */
kdn_status kdn_forward_repeat(const kdn_desc *d, const void *q, const void *k, const void *v,
                              const void *a, const void *qnoise, const void *r,
                              const float *lambda0, const float *S0, void *o, float *S_T,
                              float *lambda_T, void *ws, size_t ws_bytes, void *stream,
                              int32_t first, int32_t last, int32_t reps);

/* ------------------------------------------------------------------------
 * Allocation-free forward, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  kdn_forward_noalloc is kdn_forward (same arguments, same
 * kernels, same results bit for bit) with its workspace in a static device
 * array of KDN_NOALLOC_SCRATCH_BYTES instead of a caller buffer; it calls no
 * allocating routine.  Each GPU it runs on holds its own copy of the array
 * until the process ends; the array's device address is looked up once per
 * device (hipGetSymbolAddress) on the first call on it, with the device
 * current.  Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (other streams, other threads) race on it and must be ordered by
 * the caller.  Returns KDN_ERR_WORKSPACE when kdn_forward_workspace_bytes(d)
 * exceeds the array (B8 H16 T4096 d128 chunk 64 fits; B1 H16 T65536 does
 * not), KDN_ERR_HIP if the array's address cannot be obtained. */
#define KDN_NOALLOC_SCRATCH_BYTES ((size_t)320 << 20)
size_t kdn_noalloc_scratch_bytes(void);
kdn_status kdn_forward_noalloc(const kdn_desc *d, const void *q, const void *k, const void *v,
                               const void *a, const void *qnoise, const void *r,
                               const float *lambda0, const float *S0, void *o, float *S_T,
                               float *lambda_T, void *stream);

/* Bytes of workspace kdn_mobius_scan needs (0 if invalid). */
size_t kdn_mobius_scan_workspace_bytes(const kdn_desc *d);

/* Precision recurrence alone: the associative scan of the per-token Moebius
 * matrices (same pages: uncertainty recurrence as a Moebius map, associative
 * scan of logarithmic depth).  Reads k, a, qnoise, r and lambda0 (NULL ->
 * ones).  Writes, each optional (NULL skips it):
 *   lambda_minus [B,H,T,d_k] (diagonal) or [B,H,T] (isotropic), float32:
 *       the predictive precision of every token;
 *   lambda_chunk [B,H,ceil(T/chunk)+1,d_k] (or [...,1]): the posterior
 *       precision at every chunk boundary (index 0 = lambda0, last = lambda_T);
 *   lambda_T [B,H,d_k] or [B,H]. */
kdn_status kdn_mobius_scan(const kdn_desc *d, const void *k, const void *a,
                           const void *qnoise, const void *r, const float *lambda0,
                           float *lambda_minus, float *lambda_chunk, float *lambda_T,
                           void *ws, size_t ws_bytes, void *stream);

/* Kalman gain of every token from given predictive precisions (same pages:
 * how strongly a token's residual is written depends on how much evidence the
 * memory already holds and on how noisy the token's observation is):  w = P^- k / (k^T P^- k + r),  P^- = 1/lambda^-.
 *   lambda_minus: float32 [B,H,T,d_k] (diagonal) or [B,H,T] (isotropic).
 *   w: output [B,H,T,d_k] in gain_dtype. */
kdn_status kdn_gain(const kdn_desc *d, const void *k, const void *r,
                    const float *lambda_minus, void *w, void *stream);

/* Bytes of workspace kdn_chunk_delta needs (0 if invalid). */
size_t kdn_chunk_delta_workspace_bytes(const kdn_desc *d);

/* Memory write and read-out given the gain keys w (chunkwise form of
 * S_t = a S_{t-1} + (v - a S_{t-1} k) w^T, o_t = S_t q_t; ai-feeds.com
 * summary, section 方法 step 3: the write is computed chunk by chunk).
 * w [B,H,T,d_k] has qkv_dtype (gain_dtype must equal qkv_dtype); qnoise and r
 * are not needed because w already carries them.
 *   S0: NULL -> zeros.  o: [B,H,T,d_v] qkv_dtype.  S_T: NULL or output,
 *   may alias S0.  ws: at least kdn_chunk_delta_workspace_bytes(d) bytes. */
kdn_status kdn_chunk_delta(const kdn_desc *d, const void *q, const void *k, const void *v,
                           const void *a, const void *w, const float *S0, void *o,
                           float *S_T, void *ws, size_t ws_bytes, void *stream);

/* One-token recurrent decode step, in place (same pages: constant-memory
 * decoding).  d->B is the number of sequences N, d->T and d->chunk are
 * ignored.  q, k [N,H,d_k]; v, o [N,H,d_v] (qkv_dtype); a, qnoise, r [N,H]
 * (gate_dtype); S [N,H,d_v,d_k] and lambda [N,H,d_k] / [N,H] float32 are read
 * and overwritten with the state after the token.  o must not alias S.
 * q, k, S and lambda must be 16-byte aligned (KDN_ERR_ALIGN otherwise). */
kdn_status kdn_decode_step(const kdn_desc *d, const void *q, const void *k, const void *v,
                           const void *a, const void *qnoise, const void *r, float *S,
                           float *lambda, void *o, void *stream);

/* Exact KDN gain ("Kalman Delta Networks", English abstract: tracking the
 * key-space posterior exactly needs a full covariance with a state-dependent
 * Riccati update, which the two variants approximate):
 * per head one d_k x d_k covariance P, per token P^- = a^2 P + qnoise I,
 * w = P^- k / (k^T P^- k + r), P = P^- - (P^- k)(P^- k)^T / (k^T P^- k + r).
 * k [B,H,T,d_k] (qkv_dtype); a, qnoise, r [B,H,T]; P0 [B,H,d_k,d_k] float32
 * (NULL: identity), the covariance at t = 0; w: output [B,H,T,d_k] (gain_dtype,
 * which must equal qkv_dtype); P_T: NULL or output [B,H,d_k,d_k].  d_k is 32,
 * 64 or 128 (KDN_ERR_UNSUPPORTED otherwise); d_v and chunk are not read; the
 * variant field must hold either value and does not change the result.  k and
 * w must be 16-byte aligned (KDN_ERR_ALIGN otherwise).  The memory write and
 * read-out with these gains is
 * kdn_chunk_delta.  One workgroup per head, sequential over T: meant for the
 * small d_k and head counts where the exact filter is affordable. */
kdn_status kdn_dense_gain(const kdn_desc *d, const void *k, const void *a, const void *qnoise,
                          const void *r, const float *P0, void *w, float *P_T, void *stream);

/* ------------------------------------------------------------------ layer
 * The KDN layer around the recurrence, on caller-given weights ("Kalman Delta
 * Networks", English abstract: a drop-in replacement for linear attention;
 * KDN summary, 关键模块: queries, keys, values and the gates a, nu, r):
 *   Z = x W_in^T, with W_in [H(2 d_k + d_v) + 3H, d_model] stored out-features
 *       major (row i of W_in gives column i of Z), the rows in the order q
 *       (head-major), k, v, then the logits of a, nu and r (H each);
 *   q_h, k_h divided by max(|q_h|, 1e-6) and max(|k_h|, 1e-6);
 *   a = sigmoid(z_a + b_a), nu = softplus(z_nu + b_nu), r = softplus(z_r + b_r),
 *       b_gate [3H] float32 in the same order;
 *   o = kdn_forward(q, k, v, a, nu, r, lambda0, S0) over B*H heads;
 *   y = [o_1 .. o_H] W_out^T, W_out [d_model, H d_v] (out-features major).
 * x [B, T, d_model] and y [B, T, d_model] are token rows.  Every tensor but
 * b_gate, lambda0, S0, S_T and lambda_T is in `dtype`; the GEMMs accumulate in
 * float32 and round their outputs to dtype.  The two GEMMs run in hipBLASLt on
 * a handle from kdn_blas_create; the rest in this library's kernels. */
typedef struct {
    int32_t B, T, H, d_model, d_k, d_v, chunk;
    int32_t variant; /* kdn_variant of the recurrence */
    int32_t dtype;   /* kdn_dtype of x, the weights, y and every activation */
} kdn_layer_desc;

/* A hipBLASLt context for kdn_layer_forward: the library handle and the GEMM
 * algorithm chosen per shape (hipBLASLt's first heuristic choice within a
 * 32 MiB workspace, which is part of the layer workspace; chosen on the first
 * call with a shape and kept).  Creating it allocates (inside hipBLASLt); the
 * caller owns it, creates it once and frees it with kdn_blas_destroy.  A
 * context serves one call at a time; each call runs on its own stream. */
kdn_status kdn_blas_create(void **handle);
kdn_status kdn_blas_destroy(void *handle);

/* Bytes of workspace kdn_layer_forward needs (0 if the descriptor is invalid:
 * the recurrence's limits of kdn_validate, d_model a positive multiple of 8,
 * 3H <= 256, B*T <= 2^31 - 1).  Host-only. */
size_t kdn_layer_workspace_bytes(const kdn_layer_desc *d);

/* The layer forward.  lambda0, S0 (NULL: ones, zeros), S_T, lambda_T (NULL:
 * not written) as in kdn_forward; x, W_in, W_out, y and ws 16-byte aligned;
 * ws of at least kdn_layer_workspace_bytes(d) bytes; y must not alias x. */
kdn_status kdn_layer_forward(const kdn_layer_desc *d, void *blas, const void *x, const void *W_in,
                             const float *b_gate, const void *W_out, const float *lambda0,
                             const float *S0, void *y, float *S_T, float *lambda_T, void *ws,
                             size_t ws_bytes, void *stream);

/* kdn_layer_forward with timing: events is NULL or 10 hipEvent_t (entries may
 * be NULL) recorded on `stream` around the five stages (0-1 input GEMM, 2-3
 * normalisation and gates, 4-5 recurrence, 6-7 read-out to token rows, 8-9
 * output GEMM). */
kdn_status kdn_layer_forward_events(const kdn_layer_desc *d, void *blas, const void *x,
                                    const void *W_in, const float *b_gate, const void *W_out,
                                    const float *lambda0, const float *S0, void *y, float *S_T,
                                    float *lambda_T, void *ws, size_t ws_bytes, void *stream,
                                    void *const *events);

/* Bytes of workspace kdn_forward_varlen needs (0 if invalid); sized from d
 * alone (d->B sequences, d->T tokens per head in all). */
size_t kdn_forward_varlen_workspace_bytes(const kdn_desc *d);

/* Forward of a packed batch of d->B variable-length sequences (serving: the
 * prefill of many prompts in one call; "Kalman Delta Networks", English
 * abstract: the layer is meant for fast inference over long contexts).  Every head's rows hold
 * the sequences one after another: q, k [H, T, d_k]; v, o [H, T, d_v]; a,
 * qnoise, r [H, T], with T = d->T the total token count; sequence s has rows
 * cu_seqlens[s] .. cu_seqlens[s+1] (device int32 [B+1], non-decreasing, from 0
 * to T).  Each sequence starts from its own lambda0 / S0 ([B,H,d_k] or [B,H];
 * [B,H,d_v,d_k]; NULL: ones / zeros) and ends in its own lambda_T / S_T (same
 * shapes, required).  max_seqlen (host) must be at least the longest
 * sequence: it sizes the grids.  Offsets outside [0, T] or decreasing are
 * clamped (no memory outside the buffers is touched), but then the results
 * are not those of the sequences meant; the same holds for a max_seqlen that
 * is too small.  The result for each sequence is kdn_forward's for that
 * sequence alone. */
kdn_status kdn_forward_varlen(const kdn_desc *d, const int32_t *cu_seqlens, int32_t max_seqlen,
                              const void *q, const void *k, const void *v, const void *a,
                              const void *qnoise, const void *r, const float *lambda0,
                              const float *S0, void *o, float *S_T, float *lambda_T, void *ws,
                              size_t ws_bytes, void *stream);

/* Continuous-batching decode step (serving; "Kalman Delta Networks", English
 * abstract: decoding whose memory does not grow with the context):
 * kdn_decode_step for d->B active sequences whose states live in a cache of
 * n_slots entries.  S_cache [n_slots,H,d_v,d_k] and
 * lambda_cache [n_slots,H,d_k] (or [n_slots,H]) float32 are read and updated in
 * place at the slots slot[0..B-1] (device int32); q, k, v, a, qnoise, r and o
 * are indexed by the active sequence as in kdn_decode_step.  A slot outside
 * [0, n_slots) marks an idle sequence: its state and its o row are not
 * touched.  Slots of active sequences must be distinct (two sequences on one
 * slot race); the call does not check this.  q, k, S_cache and lambda_cache
 * must be 16-byte aligned. */
kdn_status kdn_decode_step_indexed(const kdn_desc *d, const void *q, const void *k,
                                   const void *v, const void *a, const void *qnoise,
                                   const void *r, float *S_cache, float *lambda_cache,
                                   const int32_t *slot, int32_t n_slots, void *o, void *stream);

/* Bytes of workspace kdn_backward needs (0 if the descriptor is invalid or
 * the backward does not support it).  Host-only. */
size_t kdn_backward_workspace_bytes(const kdn_desc *d);

/* Backward pass of kdn_forward (both variants): the gradient of
 *     L = <dO, o> + <dS_T, S_T> + <dlambda_T, lambda_T>
 * with respect to every input, as training the layer needs ("Kalman Delta
 * Networks", English abstract: the variants are pretrained inside language
 * models of 750M and 1.3B parameters).  The forward's intermediates are
 * recomputed from the inputs (nothing is kept between the two calls).
 *   Inputs as kdn_forward (same descriptor, same q, k, v, a, qnoise, r,
 *   lambda0, S0); dO [B,H,T,d_v] in qkv_dtype; dS_T [B,H,d_v,d_k] and
 *   dlambda_T (shaped like lambda0) float32 or NULL (zero).
 *   Outputs, float32 whatever the input dtypes: dq, dk [B,H,T,d_k];
 *   dv [B,H,T,d_v]; da, dqnoise, dr [B,H,T]; dlambda0 (like lambda0) and
 *   dS0 [B,H,d_v,d_k] (either may be NULL to skip it; they are the gradient
 *   at the given lambda0 / S0, or at ones / zeros when those are NULL).
 *   No output may alias an input.  ws: at least
 *   kdn_backward_workspace_bytes(d) bytes, 16-byte aligned, contents ignored.
 * Returns KDN_ERR_UNSUPPORTED for shapes the chunk kernels do not take
 * (kdn_backward_workspace_bytes returns 0 for them). */
kdn_status kdn_backward(const kdn_desc *d, const void *q, const void *k, const void *v,
                        const void *a, const void *qnoise, const void *r,
                        const float *lambda0, const float *S0, const void *dO,
                        const float *dS_T, const float *dlambda_T, float *dq, float *dk,
                        float *dv, float *da, float *dqnoise, float *dr, float *dlambda0,
                        float *dS0, void *ws, size_t ws_bytes, void *stream);

/* kdn_backward with timing: events is NULL or an array of 14 hipEvent_t
 * (entries may be NULL); events 2i and 2i + 1 are recorded by the dispatches
 * that start and end stage i: 0 scan reduce, 1 scan carry, 2 chunk prep,
 * 3 chunk state (the forward recompute), 4 reverse state pass, 5 per-chunk
 * gradients, 6 gain and precision recursion (three kernels).  Otherwise
 * identical to kdn_backward. */
kdn_status kdn_backward_events(const kdn_desc *d, const void *q, const void *k, const void *v,
                               const void *a, const void *qnoise, const void *r,
                               const float *lambda0, const float *S0, const void *dO,
                               const float *dS_T, const float *dlambda_T, float *dq,
                               float *dk, float *dv, float *da, float *dqnoise, float *dr,
                               float *dlambda0, float *dS0, void *ws, size_t ws_bytes,
                               void *stream, void *const *events);

/* A training step without the backward's recompute: kdn_forward_keep runs the
 * forward (same arguments and outputs as kdn_forward) into a workspace of
 * kdn_backward_workspace_bytes(d) bytes and leaves in it everything the
 * backward needs (the gain keys, T matrices, decays, boundary precisions,
 * 1/D of every token and the state at every chunk start).  kdn_backward_kept
 * then takes the arguments of kdn_backward and skips the recompute; it must
 * get the same descriptor, inputs and workspace, unchanged since the
 * kdn_forward_keep call (nothing checks this).  The gradients are the ones
 * kdn_backward returns.  kdn_backward_kept_events: events as for
 * kdn_backward_events; stages 0-3 are not run and their events not recorded. */
kdn_status kdn_forward_keep(const kdn_desc *d, const void *q, const void *k, const void *v,
                            const void *a, const void *qnoise, const void *r,
                            const float *lambda0, const float *S0, void *o, float *S_T,
                            float *lambda_T, void *ws, size_t ws_bytes, void *stream);
kdn_status kdn_backward_kept(const kdn_desc *d, const void *q, const void *k, const void *v,
                             const void *a, const void *qnoise, const void *r,
                             const float *lambda0, const float *S0, const void *dO,
                             const float *dS_T, const float *dlambda_T, float *dq, float *dk,
                             float *dv, float *da, float *dqnoise, float *dr, float *dlambda0,
                             float *dS0, void *ws, size_t ws_bytes, void *stream);
kdn_status kdn_backward_kept_events(const kdn_desc *d, const void *q, const void *k,
                                    const void *v, const void *a, const void *qnoise,
                                    const void *r, const float *lambda0, const float *S0,
                                    const void *dO, const float *dS_T, const float *dlambda_T,
                                    float *dq, float *dk, float *dv, float *da, float *dqnoise,
                                    float *dr, float *dlambda0, float *dS0, void *ws,
                                    size_t ws_bytes, void *stream, void *const *events);

#ifdef __cplusplus
}
#endif

#endif /* KDN_H */
