/*
 * bsattn.h -- C ABI of libbsattn.so: block-sparse (BigBird-ITC) and banded
 * (Longformer) self-attention on AMD Instinct MI355X (gfx950).
 *
 * The library takes per-head, post-projection Q, K, V and computes the attention
 * of each head over a sparse pattern.  Projections, the sum over heads and the
 * residual connection stay with the caller.
 *
 * Sources for what is computed:
 *   [BB]  "Big Bird: Transformers for Longer Sequences": §2 eq. (AT) (attention of
 *         query i over a key set N(i)); §2 "global tokens" (global tokens attend to
 *         all tokens and all tokens attend to them); App. D "Implementation details"
 *         with eq. (13), Fig. 4 and Fig. 6 (sparsity on b x b blocks; each query
 *         block sees the global blocks, w window blocks and r random blocks; the
 *         global row-block is a full row); hyper-parameter table of App. E
 *         (b = 64, g = 2b, w = 3b, r = 3b).
 *   [BW]  Chinese walkthrough of Big Bird (gitcode.csdn.net), §2.1-2.3 (r random
 *         keys per query, w/2 neighbours per side, g global tokens) and §4.2.
 *   [LF]  "Longformer: The Long-Document Transformer": §3.1 "Sliding Window" (w/2
 *         tokens per side), "Global Attention" (symmetric attention on preselected
 *         positions), eq. (1) (softmax(Q K^T / sqrt(d_k)) V); §3.2 and App. A
 *         (banded matrix product).
 *
 * Conventions for every call
 *   - Tensors are dense row-major [batch, heads, n, d] with d fastest; element
 *     type given by bsattn_dtype (bf16 = raw 16-bit bfloat16 bits).
 *   - lse is float32 [batch, heads, n], natural-log log-sum-exp of the scaled
 *     scores of each query row over its allowed keys.
 *   - Products of the bf16 operands are taken exactly and accumulated in fp32; the
 *     score scale is applied in fp32; the softmax runs in fp32 and the
 *     probabilities are rounded to bf16 as MFMA operands.  Outputs are rounded
 *     (nearest-even) to the input type.
 *   - o_lo (optional, bf16 only): the forward can also write the rounding residual
 *     of O, o_lo = bf16(O - bf16(O)) from the fp32 O, in the layout of O.  Passed
 *     to the backward it makes D = rowsum(dout * O), which enters every gradient
 *     through dS = P * (dP - D), exact to about 2^-17 instead of 2^-9 relative:
 *     with a peaked softmax (scores of 20 and more) the backward's D from the
 *     rounded O alone costs dQ and dK more than 2e-2 beyond their own bf16
 *     rounding.  NULL skips it (forward: not written; backward: D from O).
 *   - Device pointers must be 16-byte aligned.  All device work is enqueued on
 *     `stream` and is asynchronous unless a function says otherwise.
 *   - The caller owns every tensor and every workspace.  Compute calls never
 *     allocate.  Handles (bsattn_layout, lfattn_plan) own their own small device
 *     arrays, allocated at build time and freed by the matching destroy call; a
 *     built handle is read-only for compute calls and may be shared by streams.
 *   - Errors are returned as negative bsattn_status codes; nothing is thrown
 *     across the ABI.  Arguments are checked on the host before any launch;
 *     bsattn_last_error() returns a message for the calling thread's last error.
 *   - The environment variable BSATTN_DEBUG, read once per process: 1 logs every
 *     compute call, kernel launch and error to stderr; 2 also synchronises the
 *     stream after each compute call (not while the stream is being captured into
 *     a graph) and returns BSATTN_EHIP from the call whose kernels failed, or whose
 *     kernels wrote into the 64 bytes after the workspace bytes the call needs
 *     (checked when the workspace passed has that much spare).  Unset or 0: no
 *     logging and no extra synchronisation.
 */
#ifndef BSATTN_H
#define BSATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSATTN_OK = 0,
  BSATTN_EINVAL = -1,       /* bad argument: shape, pattern, pointer, workspace size */
  BSATTN_EUNSUPPORTED = -2, /* valid but not built: block size, head dim, dtype     */
  BSATTN_EHIP = -3,         /* a HIP runtime call or kernel launch failed           */
  BSATTN_ENOMEM = -4        /* device allocation failed while building a handle     */
} bsattn_status;

typedef enum { BSATTN_F32 = 0, BSATTN_BF16 = 1 } bsattn_dtype;

/* ------------------------------------------------------------------------- */
/* BigBird-ITC block layout                                                   */
/* ------------------------------------------------------------------------- */

typedef struct bsattn_layout bsattn_layout;

/*
 * Build the block layout of [BB] App. D on the device: for every head h and query
 * block i (nb = ceil(n / b) blocks, [BB] App. D eq. (13)), the ascending key-block list
 *     N(i) = G  U  W_i  U  R_i      for i not in G,      N(i) = {0..nb-1} for i in G,
 * where G = global_blocks, W_i = { j : |i - j| <= (w-1)/2, 0 <= j < nb } and R_i
 * holds min(r, m) blocks drawn uniformly without replacement from the m blocks not
 * in G U W_i.  The draw is a partial Fisher-Yates over the ascending candidate
 * list, step t (t = 0..) swapping entries t and t + (u mod (m - t)), where u is
 * SplitMix64 output number (h*nb + i)*r + t + 1 of the stream seeded with `seed`.
 * The transpose (for each key block, the ascending list of query blocks that see
 * it) is built too.  One layout serves every batch element.
 *
 *   n, b            sequence length and block size; b must be 64 (else
 *                   EUNSUPPORTED), n >= 1 with ceil(n/b) <= 4096.  When b does not
 *                   divide n the last block holds n - b*(nb - 1) tokens: the layout
 *                   is that of nb full blocks and the missing positions are simply
 *                   not tokens (no query, no key; nothing is padded or written).
 *   heads           number of heads, >= 1; each head draws its own random blocks.
 *   global_blocks   HOST array of g block ids, sorted, unique, in [0, nb);
 *                   may be NULL when g == 0.
 *   w               window width in blocks, odd, >= 1.
 *   r               random blocks per query block, 0 <= r <= 64.
 *   seed            64-bit generator seed.
 *   stream          stream for the build kernels.
 *   out             receives the handle.  The build is asynchronous; the handle
 *                   may be used by later work on `stream` at once.
 * Returns OK, EINVAL, EUNSUPPORTED, ENOMEM or EHIP.
 */
int bsattn_layout_build(int n, int b, int heads, const int32_t* global_blocks, int g,
                        int w, int r, uint64_t seed, hipStream_t stream,
                        bsattn_layout** out);

/* Redraw the random blocks of an existing layout with a new seed, in place, on
 * `stream`.  No allocation.  Work already enqueued with the old layout on other
 * streams must have finished.  Returns OK, EINVAL or EHIP. */
int bsattn_layout_rebuild(bsattn_layout* layout, uint64_t seed, hipStream_t stream);

/* Sizes of a layout: blocks per head, heads, and total stored block pairs over all
 * heads (the length of col_idx and of csc_idx).  Any output pointer may be NULL.
 * Every head stores the same number of pairs, nnzb_total / heads: a row's length
 * depends on its block index, the global set, w and r, never on the random draws
 * ("Big Bird", App. D: r random blocks per row beside the window and the globals). */
int bsattn_layout_info(const bsattn_layout* layout, int* nb, int* heads,
                       int64_t* nnzb_total);

/*
 * Copy a layout to host memory (synchronous; waits for the layout's last build or
 * redraw, not for other work on the device).
 *   row_ptr [heads*nb + 1]  head h, query block i: keys at col_idx[row_ptr[h*nb+i] ..
 *                           row_ptr[h*nb+i+1]), ascending.
 *   col_idx [nnzb_total]
 *   csc_ptr [heads*nb + 1]  head h, key block j: queries at csc_idx[csc_ptr[h*nb+j] ..
 *                           csc_ptr[h*nb+j+1]), ascending.
 *   csc_idx [nnzb_total]
 * Any pointer may be NULL to skip that array.  Returns OK, EINVAL or EHIP.
 */
int bsattn_layout_to_host(const bsattn_layout* layout, int32_t* row_ptr, int32_t* col_idx,
                          int32_t* csc_ptr, int32_t* csc_idx);

/* Free a layout.  Waits for its last build or redraw; work enqueued with it must be
 * ordered before this call by the caller (the device arrays are released with
 * hipFree).  NULL is accepted. */
int bsattn_layout_destroy(bsattn_layout* layout);

/* ------------------------------------------------------------------------- */
/* BigBird-ITC forward and backward                                           */
/* ------------------------------------------------------------------------- */

/* Workspace bytes bsattn_fwd / bsattn_bwd need for this layout, batch and head
 * dimension d (64 or 128; may be 0).  Returns 0 for invalid arguments as well.
 * For d = 64 the forward's size serves both dtypes: bf16 uses it for the segments
 * of split global rows, fp32 for the segments of rows split when the problem has
 * fewer query blocks than half the device's work-group slots (small,
 * latency-bound problems); for d = 128 (bf16 only) it is the bf16 size.  Past 16
 * segments per global row (long sequences) both sizes include an area for the
 * first level of a two-level merge of the segments' fp32 partials. */
size_t bsattn_fwd_workspace(const bsattn_layout* layout, int batch, int d);
size_t bsattn_bwd_workspace(const bsattn_layout* layout, int batch, int d);

/*
 * Forward ([BB] eq. (AT) inner part, per head; scores scaled as in [LF] eq. (1)):
 *   O[p] = sum_{q : block(q) in N(block(p))} softmax_q(scale * Q[p].K[q]) V[q]
 *   lse[p] = log sum_q exp(scale * Q[p].K[q]) over the same keys.
 * Rows of global query blocks are full rows ([BB] Fig. 6 "direct multiplication").
 *
 *   layout      built layout (heads and n taken from it).
 *   batch       >= 1.
 *   d           head dimension: 64, or 128 with BSATTN_BF16 (EUNSUPPORTED
 *               otherwise).  Every configuration of [BB] and [LF] has d = 64.
 *   dt          BSATTN_BF16 (bf16 MFMA products, fp32 softmax) or BSATTN_F32.
 *   scale       score scale, e.g. 1/sqrt(d).
 *   q, k, v     DEVICE [batch, heads, n, d] of type dt.
 *   o           DEVICE [batch, heads, n, d] of type dt, written.
 *   lse         DEVICE float32 [batch, heads, n], written; may be NULL.
 *   o_lo        DEVICE bf16 [batch, heads, n, d], the rounding residual of O
 *               (see the conventions above), written; may be NULL; must be NULL
 *               for BSATTN_F32 (EINVAL otherwise).
 *   workspace   DEVICE scratch of at least bsattn_fwd_workspace() bytes (NULL if 0).
 * Returns OK, EINVAL, EUNSUPPORTED or EHIP.
 */
int bsattn_fwd(const bsattn_layout* layout, int batch, int d, bsattn_dtype dt, float scale,
               const void* q, const void* k, const void* v, void* o, float* lse, void* o_lo,
               void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Backward: the exact gradient of bsattn_fwd for the loss <dout, O>.
 *   d           head dimension, 64 or 128 (EUNSUPPORTED otherwise).
 *   q, k, v, o  DEVICE [batch, heads, n, d] (o from bsattn_fwd).
 *   o_lo        DEVICE bf16 [batch, heads, n, d] from bsattn_fwd, or NULL.
 *   lse         DEVICE float32 [batch, heads, n] from bsattn_fwd (required).
 *   dout        DEVICE [batch, heads, n, d].
 *   dq, dk, dv  DEVICE [batch, heads, n, d], written.
 *   workspace   DEVICE scratch of at least bsattn_bwd_workspace() bytes.
 * dK and dV of each key block are accumulated by the one work-group that owns it,
 * walking the transposed layout; dQ by the owner of the query block.  No atomics,
 * so results are bitwise reproducible.  dt must be BSATTN_BF16 (else
 * EUNSUPPORTED).  Returns OK, EINVAL, EUNSUPPORTED or EHIP.
 */
int bsattn_bwd(const bsattn_layout* layout, int batch, int d, bsattn_dtype dt, float scale,
               const void* q, const void* k, const void* v, const void* o,
               const void* o_lo, const float* lse, const void* dout, void* dq, void* dk,
               void* dv, void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * bsattn_bwd without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving or training loops, harnesses
 * that forbid hipMalloc).  Same arguments, kernels, results and return codes as
 * bsattn_bwd, minus workspace and ws_bytes: its scratch (D and the partials of
 * split global rows and columns, bsattn_bwd_workspace() bytes) lives in a static
 * device array of BSATTN_BWD_NOALLOC_SCRATCH_BYTES (64 MiB), one per device, held
 * until the process ends.  Nothing in it needs to start at zero: every byte
 * a call reads was written earlier in the same call.  The call allocates nothing
 * (its first call on a device looks up the array's address once).
 *   - EINVAL when this layout and batch need more scratch than the array holds
 *     (e.g. B = 4, 12 heads, n = 4096 needs about 20 MB; the limit leaves room
 *     for about three times that); use bsattn_bwd then.
 *   - All calls on one device share the array: calls that may overlap in time on
 *     one device (other streams, other threads) race; order them on one stream.
 */
#define BSATTN_BWD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int bsattn_bwd_noalloc(const bsattn_layout* layout, int batch, int d, bsattn_dtype dt,
                       float scale, const void* q, const void* k, const void* v,
                       const void* o, const void* o_lo, const float* lse, const void* dout,
                       void* dq, void* dk, void* dv, hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Longformer sliding window + symmetric global attention                     */
/* ------------------------------------------------------------------------- */

typedef struct lfattn_plan lfattn_plan;

/*
 * Plan for [LF] §3.1: token p attends to token q iff |p - q| <= window_one_side,
 * or p is global, or q is global (window clipped at the sequence ends).
 *   n                sequence length, 1 .. 262144 (any length: a last partial
 *                    64-token tile is masked inside the kernels).
 *   window_one_side  keys per side, >= 0 (the token itself is always included).
 *   global_tokens    HOST array of n_global positions, sorted, unique, in [0, n);
 *                    may be NULL when n_global == 0.
 * The plan copies the global set to the device on `stream`.  Returns OK, EINVAL,
 * ENOMEM or EHIP.  Such a plan serves any head count.
 */
int lfattn_plan_build(int n, int window_one_side, const int32_t* global_tokens,
                      int n_global, hipStream_t stream, lfattn_plan** out);

/*
 * Plan for the BigBird-ETC construction ([BB] §2 "global tokens", App. E: the
 * BigBird-etc configurations, block length 84 or 169, g = 230 ... 430 added
 * global tokens, a window of 3 blocks, no random blocks): a sequence of g + n
 * tokens whose first g are added global tokens (they attend to every token and
 * every token attends to them), followed by n ordinary tokens in ceil(n / b)
 * blocks of b tokens (the last block shorter when b does not divide n; nothing is
 * padded).  An ordinary token of block k attends to the ordinary tokens of blocks
 * k - (w-1)/2 ... k + (w-1)/2, clipped at the ends, and to the global tokens.
 *   g   >= 0;  n >= 1;  g + n <= 262144.
 *   b   block length, >= 1.
 *   w   window in blocks, odd, >= 1.
 * Tensors for lfattn_fwd / lfattn_bwd are then [batch, heads, g + n, d]; the plan
 * serves any head count.  Returns OK, EINVAL (bad argument), EUNSUPPORTED
 * (too long), ENOMEM or EHIP.
 */
int lfattn_plan_build_etc(int g, int n, int b, int w, hipStream_t stream, lfattn_plan** out);

/*
 * Plan with a dilation per head and an optional autoregressive mode: [LF] §3.1
 * "Dilated Sliding Window" (Fig. 2(c): gaps of d tokens between the attended
 * tokens; a different dilation per head) and §4.1 with App. B (a window of
 * earlier tokens only).  Head h's window of token p holds the tokens
 * p + k*(dilation[h] + 1) inside [0, n), for k in [-window_one_side,
 * window_one_side], or k in [-window_one_side, 0] when causal = 1; global tokens
 * act as in lfattn_plan_build.
 *   heads      >= 1 and <= 4096; calls with this plan must pass this head count
 *              (EINVAL otherwise; the workspace queries then return 0).
 *   dilation   HOST int32[heads], each in [0, 1023]; NULL means 0 for every head.
 *   causal     0 or 1.  With 1, n_global must be 0 (EINVAL otherwise): a global
 *              token would attend to later tokens.
 * Other arguments, limits and return codes as lfattn_plan_build; EUNSUPPORTED
 * also when window_one_side * (dilation + 1) exceeds 2^30.
 */
int lfattn_plan_build_dilated(int n, int window_one_side, const int32_t* global_tokens,
                              int n_global, int heads, const int32_t* dilation, int causal,
                              hipStream_t stream, lfattn_plan** out);

/* Free a plan.  Waits for its build-time uploads; work enqueued with it must be
 * ordered before this call by the caller (the device arrays are released with
 * hipFree).  NULL is accepted. */
int lfattn_plan_destroy(lfattn_plan* plan);

/* Workspace bytes lfattn_fwd needs (d = 64 or 128).  0 for invalid arguments.  The
 * size depends on batch and heads (the global rows are cut into segments sized from
 * the whole call's work), so query it with the values the call will use. */
size_t lfattn_fwd_workspace(const lfattn_plan* plan, int batch, int heads, int d);

/*
 * Longformer forward: O, lse and o_lo as in bsattn_fwd, with the plan's token
 * pattern.  Query rows of global tokens are full rows.  q, k, v, o are DEVICE
 * [batch, heads, n, d]; lse DEVICE float32 [batch, heads, n] or NULL; o_lo DEVICE
 * bf16 [batch, heads, n, d] or NULL.  dt must be BSATTN_BF16.  d = 64 (every
 * configuration of [LF] and of the BigBird-ETC tables in [BB] App. E) or 128.
 * Returns OK, EINVAL, EUNSUPPORTED or EHIP.
 */
int lfattn_fwd(const lfattn_plan* plan, int batch, int heads, int d, bsattn_dtype dt,
               float scale, const void* q, const void* k, const void* v, void* o,
               float* lse, void* o_lo, void* workspace, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes lfattn_bwd needs (d = 64 or 128).  0 for invalid arguments.  Like
 * lfattn_fwd_workspace, it depends on batch and heads.  Past 16 segments per global
 * row or column (long sequences) both sizes include an area for the first level of a
 * two-level merge of the segments' fp32 partials. */
size_t lfattn_bwd_workspace(const lfattn_plan* plan, int batch, int heads, int d);

/*
 * Longformer backward: the exact gradient of lfattn_fwd for the loss <dout, O>
 * (the page describes the forward only; the gradient is the plain one of
 * softmax attention restricted to the plan's token pattern).
 *   q, k, v, o  DEVICE [batch, heads, n, d] (o from lfattn_fwd).
 *   o_lo        DEVICE bf16 [batch, heads, n, d] from lfattn_fwd, or NULL.
 *   lse         DEVICE float32 [batch, heads, n] from lfattn_fwd (required).
 *   dout        DEVICE [batch, heads, n, d].
 *   dq, dk, dv  DEVICE [batch, heads, n, d], written.
 *   workspace   DEVICE scratch of at least lfattn_bwd_workspace() bytes.
 * Every output tile has a single owning work-group; the full rows of global
 * queries and the full columns of key tiles holding global keys are split into
 * segments whose fp32 partials are summed in a fixed order.  A column holding a
 * global key sums over every row, and with a short window each row may put a
 * large share of its mass there, so those columns also feed the bf16 rounding
 * residues of P and dS through their products (about 2^-17 instead of 2^-9
 * relative per term).  No atomics, so results are bitwise reproducible.  dt must
 * be BSATTN_BF16 and d 64 or 128 (else EUNSUPPORTED).  Returns OK, EINVAL,
 * EUNSUPPORTED or EHIP.
 */
int lfattn_bwd(const lfattn_plan* plan, int batch, int heads, int d, bsattn_dtype dt,
               float scale, const void* q, const void* k, const void* v, const void* o,
               const void* o_lo, const float* lse, const void* dout, void* dq, void* dk,
               void* dv, void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Separate projections for the global attention ([LF] §3.1 "Linear Projections for
 * Global Attention": one set Q_s, K_s, V_s for the sliding-window attention and
 * another Q_g, K_g, V_g for the global attention, the second starting equal to
 * the first).  Reading: the row of a global token (which covers every token) is
 * computed from Qg at that token and Kg, Vg at every token; every other row (its
 * window and the global keys) from Q, K, V.  So O and lse are those of lfattn_fwd
 * with the global rows recomputed on the second set; passing qg = q, kg = k,
 * vg = v gives lfattn_fwd's result.
 *   qg, kg, vg   DEVICE [batch, heads, n, d], the second projection set.
 * Other arguments, workspace size (lfattn_fwd_workspace) and return codes as
 * lfattn_fwd; EINVAL when qg, kg or vg is NULL.
 */
int lfattn_fwd_gproj(const lfattn_plan* plan, int batch, int heads, int d, bsattn_dtype dt,
                     float scale, const void* q, const void* k, const void* v, const void* qg,
                     const void* kg, const void* vg, void* o, float* lse, void* o_lo,
                     void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Gradient of lfattn_fwd_gproj for the loss <dout, O>: dq, dk, dv for the first
 * set (dq is 0 on the rows of global tokens) and dqg, dkg, dvg for the second
 * (dqg is 0 on the other rows; dkg, dvg collect the global rows' attention over
 * every token).  The six outputs must be distinct buffers (EINVAL otherwise).
 * Workspace size lfattn_bwd_workspace; other arguments and codes as lfattn_bwd.
 */
int lfattn_bwd_gproj(const lfattn_plan* plan, int batch, int heads, int d, bsattn_dtype dt,
                     float scale, const void* q, const void* k, const void* v, const void* qg,
                     const void* kg, const void* vg, const void* o, const void* o_lo,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                     void* dqg, void* dkg, void* dvg, void* workspace, size_t ws_bytes,
                     hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* Diagnostics                                                                */
/* ------------------------------------------------------------------------- */

/* Static name of a status code. */
const char* bsattn_status_str(int status);

/* Message for the calling thread's most recent error ("" if none). */
const char* bsattn_last_error(void);

/* Library version string. */
const char* bsattn_version(void);

/*
 * Per-kernel timing for measurement tools.  While enabled (on != 0), every kernel
 * the library launches is bracketed by two hipEvents recorded on the stream it is
 * launched on.  bsattn_profile_read waits for those events and reports, for up to
 * max_kernels distinct kernel names, the name (NUL-terminated, at most 47 chars,
 * stored at names + 48*i), the number of launches and their summed elapsed time
 * in milliseconds; it then forgets the recorded launches.  *n_kernels receives
 * the number of names written.  Timing adds event records between launches, so
 * measure end-to-end throughput with profiling off.  Returns OK, EINVAL or EHIP.
 */
int bsattn_profile_enable(int on);
int bsattn_profile_read(int max_kernels, char* names, int64_t* counts, double* total_ms,
                        int* n_kernels);

#ifdef __cplusplus
}
#endif

#endif /* BSATTN_H */
