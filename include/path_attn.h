/*
 * path_attn.h -- C ABI of the PaTH attention library (libpathattn.so, gfx950).
 *
 * PaTH attention (PaTH summary, gist.science/ko/paper/2505.16381, section 2
 * "core mechanism") is causal softmax attention whose logit for query i and
 * key j <= i is
 *
 *     z_ij = scale * k_j^T (H_{j+1} H_{j+2} ... H_i) q_i + bias_ij,
 *     H_s  = I - beta_s w_s w_s^T,
 *
 * with bias_ij = sum_{s=j+1..i} f_s for PaTH-FoX (same page, section 2
 * "PaTH-FoX") and 0 otherwise.  out_i = sum_j softmax_j(z_ij) v_j and
 * lse_i = ln sum_j exp(z_ij).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or synchronises, and keeps no global mutable
 *     state (except path_decode_step_noalloc's fixed per-device scratch
 *     array, described there).  All work is enqueued asynchronously on
 *     `stream` (a hipStream_t; NULL is the null stream).
 *   - Layouts are dense row-major: q, k, v, w, out are [B, H, L, d] with d
 *     fastest; beta, log_forget, lse are [B, H, L].  Element type of q, k, v,
 *     w and out is `dtype`; beta, log_forget and lse are always fp32.
 *   - Every pointer must be 16-byte aligned.
 *   - All validation happens on the host before any launch; a failed check
 *     returns an error and enqueues nothing.  Launch failures return
 *     PATH_ERR_HIP.  Device data is never inspected: NaN in gives NaN out,
 *     and beta outside [0, 2] is accepted but its numerics are the caller's
 *     concern.  w is used as given (no renormalisation).
 *   - No call aborts or throws across the ABI.
 */
#ifndef PATH_ATTN_H
#define PATH_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PATH_ABI_VERSION 9

typedef enum {
  PATH_OK = 0,
  PATH_ERR_INVALID_ARG = 1, /* null pointer, negative size, t >= capacity, workspace too small, ... */
  PATH_ERR_UNSUPPORTED = 2, /* head dim / chunk / dtype combination not built, misaligned pointer */
  PATH_ERR_HIP = 3,         /* a HIP launch or runtime call failed */
  PATH_ERR_SCRATCH = 4      /* the problem exceeds the fixed scratch buffer of a no-allocation entry point */
} path_status;

typedef enum { PATH_DTYPE_F32 = 0, PATH_DTYPE_BF16 = 1 } path_dtype;

/*
 * Precision of the running-query transport between chunks (bf16 path only):
 * PATH_TRANSPORT_BF16 rounds the running query and the chunk product to bf16
 * for each matrix-core product; PATH_TRANSPORT_BF16X3 splits both into
 * hi + lo bf16 parts and sums hi*hi + hi*lo + lo*hi, and also scores keys
 * against the hi + lo query, which keeps long scans (tens of thousands of
 * tokens with beta near 2) and large logits within bf16-input tolerance.
 * The fp32 path always transports in fp32.
 */
typedef enum { PATH_TRANSPORT_BF16 = 0, PATH_TRANSPORT_BF16X3 = 1 } path_transport;

/* Library ABI version (PATH_ABI_VERSION of the build). */
int path_abi_version(void);

/* Static description of a status code; never NULL. */
const char* path_status_string(int status);

/*
 * Bytes of device workspace path_attn_fwd needs for this problem (written to
 * *bytes).  Pure host function.  Returns PATH_ERR_UNSUPPORTED for
 * combinations the library does not build, PATH_ERR_INVALID_ARG for bad sizes.
 */
path_status path_attn_fwd_workspace_bytes(int64_t B, int64_t H, int64_t L, int d, int chunk, int dtype,
                                          int transport, size_t* bytes);

/*
 * PaTH / PaTH-FoX prefill forward (summary, section 3 "efficient training and
 * inference": compact UT form of each chunk's transitions, boundary-adjusted
 * query/key rows per chunk, right-to-left scan over key chunks that carries the
 * transition product, FlashAttention-style online softmax).
 *
 *   q, k, v, w   [B,H,L,d] dtype        queries, keys, values, transition directions
 *   beta         [B,H,L]   fp32         transition strengths (expected in [0, 2])
 *   log_forget   [B,H,L]   fp32 or NULL PaTH-FoX per-token log forget gates f_s
 *   out          [B,H,L,d] dtype        attention output (written)
 *   lse          [B,H,L]   fp32 or NULL natural-log log-sum-exp of each row (written)
 *   scale        multiplies k^T(...)q; the FoX bias is added after scaling
 *   chunk        block length C of the scan; results do not depend on it beyond rounding;
 *                0 selects the fastest measured chunk for the path and length: on the
 *                matrix-core path 64 for L <= 4096 and 256 for longer sequences, on the
 *                vector path 64; the same choice in every call with the same L
 *   workspace    device buffer of at least path_attn_fwd_workspace_bytes bytes,
 *                caller-owned; its contents on return hold the per-chunk terms
 *                described by path_attn_workspace_layout
 *
 * Supported: dtype F32 with d in {16,32,64} and chunk in {16,32,64};
 * dtype BF16 with the same set, plus d = 64 with chunk 64, 128 or 256 on the
 * matrix-core path (128 and 256 are built from 64-token sub-chunks; the scan
 * then moves its queries once per chunk).  Any L >= 0 (a ragged last chunk is padded internally with
 * identity transitions); B, H, L may be 0 (nothing is enqueued).
 */
path_status path_attn_fwd(const void* q, const void* k, const void* v, const void* w, const float* beta,
                          const float* log_forget, void* out, float* lse, int64_t B, int64_t H, int64_t L,
                          int d, int chunk, float scale, int dtype, int transport, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * The two phases of path_attn_fwd, for callers that time or reuse them
 * separately.  path_attn_prep computes every chunk's compact-form terms into
 * the workspace (reads q, k, v, w, beta, log_forget; writes only the
 * workspace); the logit scale is applied here (the boundary-adjusted queries
 * and in-chunk logits are stored multiplied by scale * log2(e)), so the scan
 * takes no scale.  path_attn_scan runs the right-to-left attention scan from a
 * workspace that path_attn_prep filled with the SAME B, H, L, d, chunk, dtype,
 * transport and the same log_forget presence (non-NULL vs NULL); it reads v
 * and writes out and lse.  log_forget is only tested for NULL by
 * path_attn_scan, which reads v in both paths.  path_attn_fwd == prep followed
 * by scan on the same stream.
 */
path_status path_attn_prep(const void* q, const void* k, const void* v, const void* w, const float* beta,
                           const float* log_forget, int64_t B, int64_t H, int64_t L, int d, int chunk, float scale,
                           int dtype, int transport, void* workspace, size_t workspace_bytes, void* stream);

path_status path_attn_scan(const void* v, const float* log_forget, void* out, float* lse, int64_t B, int64_t H,
                           int64_t L, int d, int chunk, int dtype, int transport, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Where path_attn_fwd leaves its per-chunk terms inside the workspace (byte
 * offsets, -1 when a term is not materialised by the selected kernels).  Used
 * to inspect intermediate results; the layout of each term is stated in
 * `layout_id`:
 *   layout_id 0 (vector path): qtilde, ktilde [B*H, M*C, d] fp32; P [B*H, M, d, d] fp32
 *     (row-major, P = H_first ... H_last of the chunk); S [B*H, M, C, C] fp32 ([query][key],
 *     lower triangle incl. diagonal).  qtilde and S are stored multiplied by scale * log2(e).
 *   layout_id 1 (matrix-core path): qtilde, ktilde [B*H, M*C, d] bf16 with columns permuted
 *     within each 32-wide block (stored slot 8g+j holds column 16(j/4)+4g+(j%4));
 *     qtilde_lo (bf16x3 transport only): the bf16 residual qtilde - qtilde_hi, same layout;
 *     P (hi) and P_lo [B*H, M, d, d] bf16 (rows natural, columns permuted); S fp32 as in layout 0
 *     but packed per chunk as the lower triangle in groups of 4 columns: row a holds columns
 *     0 .. 4 floor(a/4) + 3 (those past the diagonal unspecified) and starts at float
 *     4 (a + 2u(u-1) + uv), u = floor(a/4), v = a mod 4; a chunk takes 2176 floats;
 *     qtilde (hi + lo) and S carry the factor scale * log2(e) as in layout 0.
 *   layout_id 2 (matrix-core path, chunk 128 or 256 = G sub-chunks of 64): every term of layout 1
 *     for the 64-token sub-chunks (C = 64, M = num_sub_chunks), plus ktilde_c2 [B*H, M*64, d] bf16:
 *     each sub-chunk's keys carried to the top of its chunk (ktilde_s P_{s+1} ... P_{top} in row
 *     form, columns permuted as ktilde; rows of a chunk's top sub-chunk are not written), and
 *     P_c2 (hi) / P_c2_lo [B*H, floor(M / G), d, d] = the product of each whole chunk's G sub-chunk
 *     matrices (layout of P).
 * M = num_chunks = ceil(L / chunk); num_sub_chunks = ceil(L / 64) on the matrix-core path (else M);
 * fields of terms a layout does not have are -1.
 */
typedef struct {
  int layout_id;
  int64_t num_chunks;
  int64_t off_qtilde, off_qtilde_lo, off_ktilde, off_p, off_p_lo, off_s, off_fox_local, off_fox_total;
  int64_t total_bytes;
  int64_t num_sub_chunks;
  int64_t off_ktilde_c2, off_p_c2, off_p_c2_lo;
} path_ws_layout;

path_status path_attn_workspace_layout(int64_t B, int64_t H, int64_t L, int d, int chunk, int dtype,
                                       int transport, path_ws_layout* layout);

/*
 * Bytes of device workspace path_decode_step needs (written to *bytes) for
 * `splits` key ranges per (batch, head); splits = 0 selects the automatic
 * count for a cache of `capacity` slots.
 */
path_status path_decode_workspace_bytes(int64_t B, int64_t H, int d, int64_t capacity, int splits,
                                        size_t* bytes);

/*
 * One PaTH / PaTH-FoX decode step (summary, section 3 "inference": the cached
 * keys are updated in place with the current transition, so no transition
 * vectors are cached, and the attention itself is a FlashDecoding-style
 * split-key pass).
 *
 *   kcache, vcache [B,H,capacity,d] dtype  slots 0..t_b-1 hold the current cache
 *   fcache         [B,H,capacity] fp32 or NULL  PaTH-FoX slot biases (see below)
 *   t              tokens already cached, the same for the whole batch, 0 <= t < capacity;
 *                  with t_batch, an upper bound on every entry of t_batch
 *   t_batch        [B] int32 or NULL       per-sequence token counts t_b (ragged batch);
 *                  NULL means t_b = t for every sequence
 *   q_t,k_t,v_t,w_t [B,H,d] dtype          the new token's query, key, value, direction
 *   beta_t         [B,H] fp32              the new token's transition strength
 *   log_forget_t   [B,H] fp32 or NULL      PaTH-FoX: the new token's log forget gate f_t
 *   out            [B,H,d] dtype           attention output of the new token (written)
 *   lse            [B,H] fp32 or NULL      natural-log log-sum-exp (written)
 *
 * Effect, for every (b, h) with t_b = t_batch[b] (or t): k_j <- (I - beta_t w_t w_t^T) k_j for
 * j < t_b, rounded to dtype and written back in place; slot t_b <- (k_t, v_t) untransformed;
 * then out = softmax_j(scale * q_t . k_j + bias_j) v_j over j = 0..t_b.  Slots beyond t_b are
 * untouched.  PaTH-FoX (summary, section 2 "PaTH-FoX": bias_j = sum_{s=j+1..t_b} f_s): fcache
 * holds each slot's bias as of the previous step; the step adds f_t to slots j < t_b in place
 * and sets slot t_b to 0, the same in-place rule the keys follow.  Plain PaTH: both fcache and
 * log_forget_t NULL (bias 0); passing exactly one of them is PATH_ERR_INVALID_ARG.  An entry of
 * t_batch outside [0, t] is not an error the host can see: that sequence's out and lse are NaN
 * and none of its slots are touched.  Supported: d in {16,32,64,128}, dtype F32 or BF16.
 */
path_status path_decode_step(void* kcache, void* vcache, float* fcache, int64_t capacity, int64_t t,
                             const int* t_batch, const void* q_t, const void* k_t, const void* v_t, const void* w_t,
                             const float* beta_t, const float* log_forget_t, void* out, float* lse, int64_t B,
                             int64_t H, int d, float scale, int dtype, int splits, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * path_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, kernels and results as
 * path_decode_step (bit for bit); the split partials go to a fixed scratch
 * array inside the library instead of a caller workspace.  Nothing is
 * allocated or freed and nothing synchronises.
 *
 * Limit: B * H * S * (d + 2) * 4 bytes must fit the scratch array
 * (path_decode_noalloc_scratch_bytes(), 32 MiB), where S is `splits` or, for
 * splits = 0, the automatic count (about one split per 1024 keys).  Larger
 * problems return PATH_ERR_SCRATCH and enqueue nothing.  The batch-32,
 * 24-head, d = 64 decode with a 64K-token cache uses 13.2 MiB.
 *
 * Each GPU holds its own copy of the array for the life of the process, and
 * every call on that GPU shares it (its contents are left over from the last
 * call; the kernels overwrite every partial they read, so nothing needs
 * clearing).  Calls that overlap on one GPU -- concurrent streams, or threads
 * sharing a device -- race on the array: serialise them.  The first call on a
 * device resolves the array's device address (a host-side lookup, not an
 * allocation).
 */
path_status path_decode_step_noalloc(void* kcache, void* vcache, float* fcache, int64_t capacity, int64_t t,
                                     const int* t_batch, const void* q_t, const void* k_t, const void* v_t,
                                     const void* w_t, const float* beta_t, const float* log_forget_t, void* out,
                                     float* lse, int64_t B, int64_t H, int d, float scale, int dtype, int splits,
                                     void* stream);

/* Size in bytes of path_decode_step_noalloc's fixed scratch array. */
size_t path_decode_noalloc_scratch_bytes(void);

/*
 * Decode with deferred key updates.  The step is path_decode_step's (same
 * attention output for the same inputs, up to rounding), but the cached keys
 * are brought up to date only every `period` steps; in between, a step moves
 * its query back through the transitions not yet applied to the keys
 * (k_j^T (H_{j+1} ... H_t q_t) is the in-place rule's logit read from the other
 * side), so the keys are only read, not read and written.  The transitions
 * waiting to be applied (and their PaTH-FoX gates) live in `state`.
 *
 *   t_cur     slots 0..t_cur-1 are current (they have absorbed every transition
 *             of steps < t_cur); slots t_cur..t-1 hold their keys as appended;
 *             t_cur <= t and t - t_cur < period
 *   period    1..16: the step with t - t_cur + 1 == period applies every waiting
 *             transition to the keys (and FoX gates to fcache), writes them back,
 *             and leaves all slots 0..t current: the next step passes t_cur = t + 1.
 *             Any other step leaves t_cur unchanged and records its own transition
 *             in `state`.  Passing period = t - t_cur + 1 forces the update now.
 *   state     device buffer of path_decode_deferred_state_bytes bytes per batch,
 *             owned by the caller, carried from step to step; no initialisation
 *             needed when starting from a current cache (t_cur = t)
 * Other arguments as path_decode_step (uniform t; no ragged batches here).
 * The cache after an updating step equals path_decode_step's up to rounding
 * (fewer roundings: each slot is rounded once per update).
 */
path_status path_decode_deferred_state_bytes(int64_t B, int64_t H, int d, size_t* bytes);

path_status path_decode_step_deferred(void* kcache, void* vcache, float* fcache, int64_t capacity, int64_t t,
                                      int64_t t_cur, int period, float* state, size_t state_bytes,
                                      const void* q_t, const void* k_t, const void* v_t, const void* w_t,
                                      const float* beta_t, const float* log_forget_t, void* out, float* lse,
                                      int64_t B, int64_t H, int d, float scale, int dtype, int splits,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Prefill -> decode hand-off: fills a decode cache from a prefill workspace
 * (summary, section 3, inference: decoding keeps the keys updated in place by
 * every later transition, so after a prompt of L tokens cache slot j must hold
 * H_{L-1} ... H_{j+2} H_{j+1} k_j).  The slots are built from the per-chunk
 * terms path_attn_prep (or path_attn_fwd) left in `workspace` for the SAME
 * B, H, L, d, chunk, dtype and transport: slot j of chunk n is the row
 * ktilde_j (P_{n+1} ... P_{M-1}) (row form; the chunk products are chained right
 * to left), so the prompt's transitions are not read again.  path_decode_step
 * can then continue at t = L.
 *
 *   v               [B,H,L,d] dtype         the prompt's values (copied)
 *   log_forget      [B,H,L] fp32 or NULL    PaTH-FoX: the prompt's gates
 *   workspace       prefill workspace: its per-chunk terms are read; on the
 *                   matrix-core path its hand-off scratch (sized into
 *                   path_attn_fwd_workspace_bytes, after every per-chunk term)
 *                   is written
 *   kcache, vcache  [B,H,capacity,d] dtype  slots 0..L-1 written; slots >= L untouched
 *   fcache          [B,H,capacity] fp32 or NULL  PaTH-FoX: slot j <- sum_{s=j+1..L-1} f_s
 *                   (the slot bias path_decode_step expects); given iff log_forget is
 *   capacity        >= L (PATH_ERR_INVALID_ARG otherwise)
 *
 * The bf16 path chains the chunk products with fp32 accumulation (the running
 * product enters the matrix cores as hi + lo bf16) and rounds each slot to bf16
 * once; with fewer than 128 (b, h) pairs it cuts each pair's chain into
 * segments run in parallel (products of whole segments kept as hi + lo bf16,
 * their suffix products in fp32).  The fp32 path works in fp32.  Slot biases are
 * fp32 sums.
 */
path_status path_attn_cache_from_prefill(const void* v, const float* log_forget, void* workspace,
                                         size_t workspace_bytes, void* kcache, void* vcache, float* fcache,
                                         int64_t capacity, int64_t B, int64_t H, int64_t L, int d, int chunk,
                                         int dtype, int transport, void* stream);

/*
 * Backward pass: gradients of the prefill (PaTH or PaTH-FoX) for an upstream
 * gradient dout of its output, i.e. of the loss sum(dout * out).  The pages give
 * the forward only (summary, sections 2 and 3; the lecture notes' "limitations"
 * say the backward is the costlier part); this differentiates the blockwise
 * forward with the chain rule: logits of each pair of chunks are recomputed from
 * lse, the running queries and their gradients of each (query chunk, key chunk)
 * pair are kept in the workspace (a transition with beta = 1 is singular, so
 * they cannot be recovered backwards) for one band of about 4 sqrt(L / chunk)
 * query chunks at a time, the key-side sums carrying over from band to band,
 * and each chunk's UT-transform terms are differentiated back to q, k, w and
 * beta.
 *
 *   q, k, v, w     [B,H,L,d] dtype          the forward's inputs
 *   beta           [B,H,L] fp32
 *   log_forget     [B,H,L] fp32 or NULL     PaTH-FoX gates f (as in the forward)
 *   out            [B,H,L,d] dtype          the forward's output
 *   lse            [B,H,L] fp32             the forward's log-sum-exp (required)
 *   dout           [B,H,L,d] dtype          upstream gradient of out
 *   dq, dk, dv, dw [B,H,L,d] dtype          written
 *   dbeta          [B,H,L] fp32             written
 *   dlog_forget    [B,H,L] fp32 or NULL     written; given iff log_forget is
 *   chunk          16, 32 or 64 (0 = 64); d 16, 32 or 64
 *
 * Accumulation is fp32 and gradients are rounded to the input dtype once.  With
 * bf16 inputs at d = chunk = 64 the matrix products run on the bf16 matrix
 * cores from the prefill's own per-chunk terms (bf16 transport form): the
 * running queries are rounded to bf16 after every chunk transition as in the
 * forward; the probabilities p and logit gradients dz enter their products
 * (dv, dktilde and the incoming state gradient) rounded to bf16 once, as
 * flash-attention backward kernels round P and dS; other fp32 operands are
 * split into hi + lo bf16 (about 2^-16 relative); fp32 inputs keep fp32
 * products throughout.
 * Workspace: path_attn_bwd_workspace_bytes; it grows as B*H*L*d*sqrt(L/chunk)
 * (two vectors per key of every chunk pair of one band, bf16 for bf16 inputs:
 * about 6.4 GB at B=8, H=24, L=4096, d=64, chunk 64 and 16.6 GB at B=1, H=24,
 * L=32768; 11.4 and 31.8 GB for fp32 inputs).  The kernels are deterministic:
 * the same inputs give the same bits.  Errors as for path_attn_fwd; nothing is
 * enqueued on an error.
 */
path_status path_attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t L, int d, int chunk, int dtype,
                                          size_t* bytes);

path_status path_attn_bwd(const void* q, const void* k, const void* v, const void* w, const float* beta,
                          const float* log_forget, const void* out, const float* lse, const void* dout, void* dq,
                          void* dk, void* dv, void* dw, float* dbeta, float* dlog_forget, int64_t B, int64_t H,
                          int64_t L, int d, int chunk, float scale, int dtype, void* workspace,
                          size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PATH_ATTN_H */
