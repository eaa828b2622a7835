/*
 * sa.h — C ABI of the Sketch Attention (SA) compression library (libsa.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * What the library computes.  SequenceO1's Sketch Attention compresses one
 * user's behaviour history H_u (n_u tokens of width d) into a fixed k x d
 * sketch using k learnable prototypes P and prototype-wise normalisation:
 *   - arXiv abstract (mlsanity paper page, "Abstract"): learnable prototypes
 *     and prototype-wise normalisation compress the raw history into a
 *     fixed-size, target-agnostic user representation; a fused FlashSA kernel
 *     keeps the computation practical;
 *   - blog "100,000 videos in your pocket", "How it works" item 1: every
 *     history item is softly assigned across the k prototypes and distributes
 *     its mass over them; the output is a k x d sketch; item 3: the fused
 *     kernel runs under ragged batches without materialising the huge
 *     intermediates;
 *   - review page (evolve.pub), FAQ on how SA differs from standard
 *     attention: normalisation runs across prototypes, not the sequence.
 * With K = H_u Wk, V = H_u Wv (row vectors), for every token t and prototype j
 *     L[j,t] = p_j . k_t / sqrt(d)
 *     A[j,t] = exp(L[j,t]) / sum_j' exp(L[j',t])          (softmax over j)
 *     m_j    = sum_t A[j,t]                                (prototype mass)
 *     S_u[j] = (sum_t A[j,t] v_t) / m_j                    (0 where m_j = 0)
 * An empty user (n_u = 0, or every token masked) gives S_u = 0 and m = 0.
 *
 * Ownership and threading.  The caller owns every buffer.  All pointers
 * except `problem` and `bytes` are DEVICE pointers on the current HIP device.
 * The library allocates nothing and keeps no mutable global state; calls on
 * different streams with different workspaces may run concurrently.
 * sa_compress is asynchronous and stream-ordered: on SA_OK the work is queued
 * on `stream` (a hipStream_t; NULL = the default stream) and S / mass are
 * valid once the stream reaches that point.  No C++ exception crosses this
 * ABI.
 */
#ifndef SA_H_
#define SA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Argument errors are detected on the host before any launch. */
typedef enum {
  SA_OK = 0,
  SA_E_INVALID = 1,      /* NULL pointer, negative size, inconsistent sizes   */
  SA_E_UNSUPPORTED = 2,  /* valid problem outside the built kernels' shapes   */
  SA_E_WORKSPACE = 3,    /* workspace NULL or smaller than sa_workspace_size   */
  SA_E_HIP = 4           /* a HIP runtime call or kernel launch failed         */
} sa_status;

/* Element type of H, Wk, Wv and P.  Outputs are always float32. */
typedef enum {
  SA_BF16 = 0,           /* bfloat16 inputs; MFMA on fp16 operands, fp32 sums */
  SA_F32 = 1             /* float32 inputs; fp32 arithmetic throughout         */
} sa_dtype;

/*
 * One batch of users.
 *   num_users    R >= 0.
 *   total_tokens N >= 0, equal to offsets[R] (a host copy, so that no
 *                device-to-host read is needed).
 *   d            history / key / value width.  Built: 64 or 128.
 *   k            number of prototypes.  Built: a multiple of 64, 64..4096.
 *   dtype        an sa_dtype value.
 */
typedef struct {
  int64_t num_users;
  int64_t total_tokens;
  int32_t d;
  int32_t k;
  int32_t dtype;
  int32_t flags;         /* 0, or one of the SA_FLAG_* path requests */
} sa_problem;

/*
 * Path requests (sa_problem.flags; results agree within rounding either way).
 * For bf16 inputs with k = 256 * 2^i (i = 0..4) the library can run the
 * one-pass kernel: groups of k / 256 co-resident workgroups exchange
 * per-token partial softmax denominators, so every logit is computed once.
 * Otherwise it runs two passes (per-token logsumexp, then allocations and
 * sums), computing every logit twice.  0 lets the library choose (currently
 * two passes, the faster on MI355X).  Setting both flags is SA_E_INVALID.
 *   SA_FLAG_TWO_PASS  always run the two-pass kernels.
 *   SA_FLAG_ONE_PASS  run the one-pass kernel whenever the shape and device
 *                     allow it.
 */
#define SA_FLAG_TWO_PASS 1
#define SA_FLAG_ONE_PASS 2

/*
 * Workspace size for `problem`.  Writes the byte count to *bytes.  Returns
 * SA_E_INVALID / SA_E_UNSUPPORTED for a problem sa_compress would reject.
 * Pure host code; needs no GPU.  The size grows linearly in N, R and k; for
 * bf16 the fp16 copy of the (tile-padded) token rows, 2d bytes per token,
 * dominates for long histories.
 */
sa_status sa_workspace_size(const sa_problem* problem, size_t* bytes);

/*
 * The same workspace size as a return value: sa_workspace_size's byte count
 * for a problem sa_compress accepts, and 0 for one it rejects (including
 * problem = NULL).  Pure host code.
 */
size_t sa_workspace_bytes(const sa_problem* problem);

/*
 * Compress a ragged batch of R user histories into R sketches.
 *
 *   H           [N, d] row-major, dtype `problem->dtype`, 16-byte aligned.
 *               User u owns rows offsets[u] .. offsets[u+1]-1.  For SA_BF16,
 *               magnitudes of unmasked entries must not exceed 65504: they are
 *               widened exactly to fp16 MFMA operands; a larger, infinite or
 *               NaN kept value raises SA_DEVICE_ERR_RANGE (that call's
 *               outputs are invalid).
 *   offsets     [R+1] int64, 0 = offsets[0] <= offsets[1] <= ... <= offsets[R]
 *               = N.  Device memory, 8-byte aligned.  If the sequence breaks this contract
 *               the kernels treat every user as empty (S = 0, mass = 0) and
 *               raise the device error flag read by sa_read_device_error.
 *   token_mask  [N] uint8, 1 = keep the token, 0 = drop it entirely (it takes
 *               no part in allocation, mass or sums; NaN in a dropped row
 *               does not propagate).  NULL keeps every token.
 *   Wk, Wv      [d, d] row-major, K = H Wk and V = H Wv, 16-byte aligned.
 *   P           [k, d] row-major prototypes, 16-byte aligned.
 *               (A misaligned H, Wk, Wv, P or offsets is SA_E_INVALID.)
 *   S           [R, k, d] float32 output, fully overwritten.
 *   mass        [R, k] float32 output m_j (fully overwritten), or NULL.
 *   workspace   device scratch of at least sa_workspace_size bytes, 256-byte
 *               aligned.  Its contents on entry are ignored.  One workspace
 *               must not be shared by calls that may run concurrently.
 *   stream      hipStream_t to queue the kernels on (NULL = default stream).
 *
 * R = 0 is a no-op.  N = 0 writes zero sketches.
 */
sa_status sa_compress(const sa_problem* problem,
                      const void* H,
                      const int64_t* offsets,
                      const uint8_t* token_mask,
                      const void* Wk,
                      const void* Wv,
                      const void* P,
                      float* S,
                      float* mass,
                      void* workspace,
                      size_t workspace_bytes,
                      void* stream);

/* Number of phase-boundary events sa_compress_with_events records. */
#define SA_NUM_PHASE_EVENTS 5

/*
 * sa_compress, recording caller-created HIP events (hipEvent_t handles) on
 * `stream` at the phase boundaries, for timing with hipEventElapsedTime:
 *   events[0] before the query/schedule preparation,
 *   events[1] after it (start of the token pass: the per-token logsumexp of
 *             the two-pass path, or the fp16 packing of the one-pass path),
 *   events[2] after the token pass (start of the accumulation: allocations
 *             and sums),
 *   events[3] after the accumulation (start of the normalise /
 *             value-projection step),
 *   events[4] after the last kernel.
 * `events` may be NULL (then this is sa_compress).  A phase with no work
 * (e.g. N = 0) records its two events back to back.  Same arguments, errors
 * and semantics as sa_compress otherwise.
 */
sa_status sa_compress_with_events(const sa_problem* problem,
                                  const void* H,
                                  const int64_t* offsets,
                                  const uint8_t* token_mask,
                                  const void* Wk,
                                  const void* Wv,
                                  const void* P,
                                  float* S,
                                  float* mass,
                                  void* workspace,
                                  size_t workspace_bytes,
                                  void* stream,
                                  void* const* events);

/*
 * For callers that cannot allocate device memory at call time (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * sa_compress without a workspace argument.  Its workspace is a static
 * device array of SA_STATIC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends; the call itself allocates nothing
 * (no hipMalloc, hipFree or allocating library routine).
 *   - Problems whose sa_workspace_size exceeds SA_STATIC_SCRATCH_BYTES are
 *     SA_E_WORKSPACE (64 MiB: e.g. one 100,000-token user at k = 1024,
 *     d = 128, or any batch of up to about 30,000 tokens at k <= 1024).
 *   - Every call on one GPU shares that GPU's array: calls that may overlap
 *     on one GPU (different streams, other threads) race and give undefined
 *     results.  Serialise them, e.g. on one stream.
 *   - device_error: optional [1] int32 device pointer; when non-NULL it
 *     receives the call's device error flags (the SA_DEVICE_ERR_* bits that
 *     sa_read_device_error reports for a workspace), stream-ordered.
 * Arguments, results and errors otherwise as sa_compress.
 */
#define SA_STATIC_SCRATCH_BYTES (64u << 20)

sa_status sa_compress_static(const sa_problem* problem,
                             const void* H,
                             const int64_t* offsets,
                             const uint8_t* token_mask,
                             const void* Wk,
                             const void* Wv,
                             const void* P,
                             float* S,
                             float* mass,
                             int32_t* device_error,
                             void* stream);

/*
 * sa_compress_with_events that also writes the mass-normalised rows
 *     Sbar [R, k, d] float32,  Sbar_u[j] = (sum_t A[j,t] h_t) / m_j
 * (0 where m_j = 0), i.e. S_u = Sbar_u Wv before the value projection.  A
 * training step keeps Sbar and mass and hands both to
 * sa_compress_backward_with_sbar, which then skips recomputing the per-user
 * sums.  mass and Sbar must be non-NULL when R > 0 (SA_E_INVALID otherwise);
 * S, events and everything else as sa_compress_with_events.
 */
sa_status sa_compress_with_sbar(const sa_problem* problem,
                                const void* H,
                                const int64_t* offsets,
                                const uint8_t* token_mask,
                                const void* Wk,
                                const void* Wv,
                                const void* P,
                                float* S,
                                float* mass,
                                float* Sbar,
                                void* workspace,
                                size_t workspace_bytes,
                                void* stream,
                                void* const* events);

/*
 * The backward pass (gradients of a loss through the sketches).
 *
 * SequenceO1 trains the compressor end to end: the blog "100,000 videos in
 * your pocket" ("How it works", item 1) notes that the compression is
 * differentiable, so the ranking loss's gradients flow back through it, and
 * its "Takeaways" list training the compressor on the real loss.  The pages
 * give no backward formulas; the library computes the chain rule of the
 * forward definition above.  Given dS = dLoss/dS_u for every user:
 *   dH    [N, d] float32   dLoss/dh_t for every token (zero rows for tokens
 *                          that token_mask drops), fully overwritten;
 *   dP    [k, d] float32   dLoss/dP,  summed over the users, overwritten;
 *   dWk   [d, d] float32   dLoss/dWk, summed over the users, overwritten;
 *   dWv   [d, d] float32   dLoss/dWv, summed over the users, overwritten.
 * A sketch row with zero mass is the constant 0 and passes no gradient;
 * empty users contribute nothing.
 *
 * Built for bf16 inputs (problem->dtype = SA_BF16) with the same d and k as
 * sa_compress; SA_F32 or SA_FLAG_ONE_PASS give SA_E_UNSUPPORTED (the
 * backward recomputes the two-pass forward's per-token state).  Internally
 * the products use fp16 MFMA operands (the token rows widened exactly, the
 * allocations, their gradients and dS / m scaled by powers of two into fp16
 * range) with fp32 sums.  dS must be finite.
 *
 * Workspace: sa_backward_workspace_size bytes (more than sa_compress needs).
 * Same ownership, stream and threading rules as sa_compress; the offsets
 * contract is the same, and on a violation every user counts as empty (all
 * four gradients zero) and the device error flag is raised.  R = 0 writes
 * zero dP, dWk and dWv and needs no workspace or offsets.
 */
sa_status sa_backward_workspace_size(const sa_problem* problem, size_t* bytes);

sa_status sa_compress_backward(const sa_problem* problem,
                               const void* H,
                               const int64_t* offsets,
                               const uint8_t* token_mask,
                               const void* Wk,
                               const void* Wv,
                               const void* P,
                               const float* dS,      /* [R, k, d] float32 */
                               float* dH,
                               float* dP,
                               float* dWk,
                               float* dWv,
                               void* workspace,
                               size_t workspace_bytes,
                               void* stream);

/* Number of phase-boundary events sa_compress_backward_with_events records. */
#define SA_NUM_BWD_PHASE_EVENTS 6

/*
 * sa_compress_backward, recording caller-created HIP events on `stream`:
 *   events[0] before the first kernel,
 *   events[1] after the forward recomputation (queries, per-token
 *             logsumexps and fp16 rows, per-user sums),
 *   events[2] after the per-user step (Z = (dS / m) Wv^T and its scale),
 *   events[3] after the token-major kernel (dH),
 *   events[4] after the prototype-major kernel (E = sum_t dL h_t),
 *   events[5] after the last kernel (dP, dWk, dWv).
 * `events` may be NULL.  Same arguments, errors and semantics otherwise.
 */
sa_status sa_compress_backward_with_events(const sa_problem* problem,
                                           const void* H,
                                           const int64_t* offsets,
                                           const uint8_t* token_mask,
                                           const void* Wk,
                                           const void* Wv,
                                           const void* P,
                                           const float* dS,
                                           float* dH,
                                           float* dP,
                                           float* dWk,
                                           float* dWv,
                                           void* workspace,
                                           size_t workspace_bytes,
                                           void* stream,
                                           void* const* events);

/*
 * sa_compress_backward_with_events given the forward's Sbar [R, k, d] and
 * mass [R, k] (both float32, device, from sa_compress_with_sbar on the same
 * problem and inputs): the per-user sums are taken from them instead of
 * being recomputed, which removes the forward's accumulation pass from the
 * backward (events[1] then marks the end of the per-token logsumexp pass).
 * The chain rule needs Sbar and m; the per-token allocations are still
 * recomputed.  Sbar and mass must be non-NULL when R > 0 (SA_E_INVALID).  If they do not come
 * from the same inputs the gradients are those of a different forward; no
 * memory outside the stated shapes is read either way.  Same workspace
 * (sa_backward_workspace_size), outputs, errors and semantics otherwise.
 */
sa_status sa_compress_backward_with_sbar(const sa_problem* problem,
                                         const void* H,
                                         const int64_t* offsets,
                                         const uint8_t* token_mask,
                                         const void* Wk,
                                         const void* Wv,
                                         const void* P,
                                         const float* Sbar,
                                         const float* mass,
                                         const float* dS,
                                         float* dH,
                                         float* dP,
                                         float* dWk,
                                         float* dWv,
                                         void* workspace,
                                         size_t workspace_bytes,
                                         void* stream,
                                         void* const* events);

/*
 * Sketch-branch target attention with user-level batching.
 *
 * After compression each candidate item attends over its user's cached
 * sketch (blog "100,000 videos in your pocket", "How it works" item 2: the
 * sketch branch of STCA), and a user's many candidates share one read of the
 * sketch (same page, item 3: multi-request user-level batching).  The pages
 * define STCA's stacking only by reference to an earlier paper; this is the
 * single-layer reading, single-head scaled dot-product attention whose keys
 * and values are the k sketch rows s_j of the candidate's user:
 *     out_c = sum_j softmax_j(q_c . s_j / sqrt(d)) s_j
 * Projections of the candidate or the sketch, further layers and the fusion
 * with the recent-history branch are the caller's.
 *
 *   problem       num_users R, total_tokens = C (the total candidate count),
 *                 d and k as for sa_compress; dtype SA_BF16 (the candidate
 *                 queries); flags 0.
 *   Q             [C, d] bf16 candidate queries, user by user, 16-byte aligned.
 *   cand_offsets  [R+1] int64 device: user u owns candidates
 *                 cand_offsets[u] .. cand_offsets[u+1]-1 (same contract and
 *                 device error flag as sa_compress's offsets; on a violation
 *                 out and lse are zero).
 *   S             [R, k, d] float32 sketches (sa_compress's output layout),
 *                 16-byte aligned; entries must not exceed 65504 in magnitude
 *                 (fp16 MFMA operands; a larger or non-finite entry, or such
 *                 a query value, raises SA_DEVICE_ERR_RANGE).
 *   out           [C, d] float32, fully overwritten.
 *   lse           [C] float32 natural-log normaliser log sum_j exp(q . s_j /
 *                 sqrt(d)), or NULL.
 *   workspace     sa_target_attention_workspace_size bytes, 256-byte aligned.
 * Candidate queries are widened exactly to fp16, sketch rows rounded to fp16,
 * sums in fp32.  Asynchronous on `stream`; R = 0 is a no-op.
 */
sa_status sa_target_attention_workspace_size(const sa_problem* problem, size_t* bytes);

sa_status sa_target_attention(const sa_problem* problem,
                              const void* Q,
                              const int64_t* cand_offsets,
                              const float* S,
                              float* out,
                              float* lse,
                              void* workspace,
                              size_t workspace_bytes,
                              void* stream);

/*
 * sa_target_attention with the sketches read through a row index: user u's
 * sketch is S[sketch_rows[u]], where S holds sketch_count sketches
 * [sketch_count, k, d] and sketch_rows is [R] int32 device memory, e.g. the
 * slots of a sketch cache's slab (sa_cache_*), so cached sketches are
 * attended in place without a gather.  An index outside [0, sketch_count)
 * reads nothing: that user's candidates get zero out and lse rows and the
 * device error flag SA_DEVICE_ERR_SKETCH_ROW is raised.  sketch_rows = NULL
 * with sketch_count = R is sa_target_attention.  sketch_count < 0 is
 * SA_E_INVALID.
 */
sa_status sa_target_attention_rows(const sa_problem* problem,
                                   const void* Q,
                                   const int64_t* cand_offsets,
                                   const float* S,
                                   const int32_t* sketch_rows,
                                   int64_t sketch_count,
                                   float* out,
                                   float* lse,
                                   void* workspace,
                                   size_t workspace_bytes,
                                   void* stream);

/*
 * User-keyed sketch cache and its cache-miss driver.
 *
 * The sketch is user-only and target-agnostic, so it is cached: a local
 * cache in training reuses a user's sketch across repeated instances (3 h
 * lifetime, hit rate about 0.5) and a serving cache across consecutive
 * requests (1 h, about 0.6); a hit skips storing, moving and processing the
 * raw history, and computing the misses overlaps other work (blog "100,000
 * videos in your pocket", "How it works" item 3 and "The numbers"; review
 * page, "Summary").
 *
 * sa_cache_create: a host object over a caller-owned device slab
 *   slab [capacity, k, d] float32 (16-byte aligned) and optionally
 *   mass_slab [capacity, k] float32; slot i holds one user's sketch.  An
 *   entry is fresh while now - t_computed < ttl_seconds.  The object is not
 *   thread-safe; sa_cache_destroy frees it (not the slab).
 * sa_cache_lookup (pure host): for requests users[0..n-1] at time `now`,
 *   in order, writes slots[i] (where request i's sketch is, once the misses
 *   are filled) and the miss list (miss_users, miss_slots, *n_miss; arrays
 *   of n entries).  A fresh entry is a hit; the first request of any other
 *   user is a miss and takes a slot: a free one, else an expired entry, else
 *   the least recently used entry that no request of this batch uses; later
 *   requests of the same user in the batch share that slot and count as
 *   hits.  A stale entry is recomputed in place (counted as a miss and as
 *   expired).  More distinct users in one batch than slots is SA_E_INVALID,
 *   checked before anything changes: the cache is left as it was.
 * sa_cache_fill: gathers the miss users' history rows from the caller's
 *   packed store (H_store [N_store, d] with host store_offsets [R_store+1],
 *   optional mask_store [N_store]; `store` describes it: num_users =
 *   R_store, total_tokens = N_store, d, k, dtype) into one ragged batch,
 *   runs one sa_compress on it and scatters the sketches (and masses) into
 *   the miss slots.  Stream-ordered on `stream` (typically a side stream:
 *   the caller makes the consumers wait on an event after it).  At most
 *   65535 misses per call.  Workspace: sa_cache_fill_workspace_size for the
 *   largest (miss users, miss tokens) a call will see, 256-byte aligned.
 */
typedef struct sa_cache sa_cache;

typedef struct {
  int64_t hits;
  int64_t misses;
  int64_t evictions;   /* entries of other users removed to make room */
  int64_t expired;     /* misses that recomputed a stale entry in place */
} sa_cache_stats;

sa_status sa_cache_create(int32_t capacity, int32_t k, int32_t d, double ttl_seconds, float* slab,
                          float* mass_slab, sa_cache** cache);

sa_status sa_cache_destroy(sa_cache* cache);

sa_status sa_cache_lookup(sa_cache* cache, const int64_t* users, int64_t n, double now, int32_t* slots,
                          int64_t* miss_users, int32_t* miss_slots, int64_t* n_miss, sa_cache_stats* stats);

sa_status sa_cache_fill_workspace_size(const sa_problem* store, int64_t max_miss_users, int64_t max_miss_tokens,
                                       size_t* bytes);

sa_status sa_cache_fill(sa_cache* cache, const sa_problem* store, const void* H_store, const int64_t* store_offsets,
                        const uint8_t* mask_store, const void* Wk, const void* Wv, const void* P,
                        const int64_t* miss_users, const int32_t* miss_slots, int64_t n_miss, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Device error flag bits. */
#define SA_DEVICE_ERR_OFFSETS 1   /* offsets broke their contract: all users empty */
#define SA_DEVICE_ERR_EXCHANGE 2  /* one-pass: a bounded wait between workgroups
                                     expired; the sketches of that call are invalid */
#define SA_DEVICE_ERR_RANGE 4     /* a kept bf16 history value (or, in target
                                     attention, a candidate query or sketch value)
                                     lies outside fp16's finite range: |x| > 65504,
                                     an infinity or a NaN.  Such values become fp16
                                     MFMA operands, so the outputs of that call are
                                     invalid; masked tokens are not checked. */
#define SA_DEVICE_ERR_SKETCH_ROW 8 /* sa_target_attention_rows: a sketch_rows index
                                     outside [0, sketch_count); that user's outputs
                                     are zero */

/*
 * Synchronously read the device error flags that the last call on
 * `workspace` set (sa_compress and its variants, the backward, target
 * attention; 0 = none, else a combination of SA_DEVICE_ERR_*).  Waits for
 * `stream`.  Returns SA_E_HIP if the copy fails.
 */
sa_status sa_read_device_error(const void* workspace, void* stream, int32_t* flag);

/*
 * Measurement helper, not part of the compression path: how fast the matrix
 * cores run on a given kind of operand data.  Queues one launch of a loop of
 * fp16 32x32x16 MFMAs with no memory traffic: 512 workgroups of 4 waves (two
 * waves per SIMD on 256 CUs), each wave `iters` x 8 MFMAs over four
 * accumulator chains with its operands in registers.  `operands`: 0 all
 * zeros, 1 one constant value, 2 uniform values in [-1, 1) that differ per
 * lane and per instruction.  The launch does 2048 x iters x 8 x 32768 FLOP;
 * timed with events on `stream`, it gives the MFMA rate on that data (the
 * clock of a power-limited part depends on how many operand bits toggle).
 * `sink` (device, SA_PROBE_SINK_FLOATS floats, caller-owned) receives one sum
 * per thread so that the work is not optimised away.  SA_E_INVALID for a NULL
 * sink, `operands` outside 0..2 or `iters` outside 1..1,000,000; SA_E_HIP if
 * the launch fails.
 */
#define SA_PROBE_SINK_FLOATS 131072
sa_status sa_probe_mfma(int32_t operands, int32_t iters, float* sink, void* stream);

/* Static text for a status code.  Never NULL. */
const char* sa_status_string(sa_status status);

/* Library version as "major.minor.patch". */
const char* sa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SA_H_ */
