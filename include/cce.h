/*
 * cce.h -- C ABI of libcce.so: fused classifier-head matmul + cross-entropy
 * ("Cut Cross-Entropy", CCE) forward and backward on one AMD MI355X (gfx950).
 *
 * What is computed (per non-ignored row i, classifier row e_v, label y_i):
 *   z_iv   = <h_i, e_v>                       (never stored in device memory)
 *   lse_i  = log sum_v exp(z_iv)
 *   loss_i = lse_i - z_{i,y_i}
 *   dH_i   = sum_v g_iv e_v,   dE_v = sum_i g_iv h_i,
 *   g_iv   = dloss_i * (p_iv * [block(i,v) survives or v == y_i] - [v == y_i]),
 *   p_iv   = exp(z_iv - lse_i).
 * Cross-entropy needs only the correct-token logit (an indexed matmul) and the
 * log-sum-exp over the vocabulary, computed blockwise on chip without writing
 * the [rows x vocabulary] product to memory (lit note "The loss and the mask:
 * Cut Cross-Entropy + FlexAttention", section "Contribution").  The backward
 * recomputes logits blockwise and skips blocks whose softmax entries all fall
 * below a threshold (gradient filtering; a vocabulary sort clusters the
 * surviving blocks) -- CCE paper summary "Cut Your Losses in Large-Vocabulary
 * Language Models", section "Approach".  The classifier gradient is
 * accumulated across blocks with Kahan compensation (same summary, section
 * "Limitations").
 *
 * Conventions shared by every entry point:
 *  - Every pointer is a DEVICE pointer owned by the caller, except where a
 *    comment says otherwise.  The library allocates and frees nothing and keeps
 *    no mutable global state; calls are reentrant.  Calls that run at the same
 *    time must not share a workspace.
 *  - H is [N, D] and E is [V, D], row-major with D innermost, both of one dtype
 *    (cce_dtype).  D % 8 == 0; H, E, dH, dE and the workspace are 16-byte
 *    aligned.  1 <= N <= 2^31 - 2^16, 1 <= V <= 2^31 - 2^16, 8 <= D <= 65536.
 *  - labels are int64 [N]; a row whose label equals ignore_index is ignored.
 *    Any other label outside [0, V) is undefined behaviour (cce_check_labels
 *    detects it).
 *  - loss, lse and dloss are fp32 [N].  dH and dE take the input dtype and are
 *    overwritten (not accumulated into).
 *  - stream is a hipStream_t passed as void* (NULL = the default stream).  All
 *    work is enqueued on it; no entry point synchronises the host.
 *  - Errors in the arguments are reported before any work is enqueued, and the
 *    outputs are then left untouched.  CCE_ERR_HIP reports a failed launch.
 *    Faults inside a kernel surface at the caller's next synchronisation, as
 *    for any asynchronous HIP work.
 *  - Results are deterministic: the same inputs give bit-identical outputs.
 */
#ifndef CCE_H_
#define CCE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CCE_OK = 0,
    CCE_ERR_NULL = 1,       /* a required pointer is NULL */
    CCE_ERR_SHAPE = 2,      /* N, D or V out of the supported range */
    CCE_ERR_DTYPE = 3,      /* unknown cce_dtype */
    CCE_ERR_ALIGN = 4,      /* a pointer is not 16-byte aligned */
    CCE_ERR_WORKSPACE = 5,  /* workspace smaller than the *_workspace_bytes query */
    CCE_ERR_HIP = 6,        /* a HIP launch failed */
    CCE_ERR_ARG = 7         /* another argument is invalid (e.g. NaN or negative filter_eps) */
} cce_status;

typedef enum { CCE_F32 = 0, CCE_BF16 = 1 } cce_dtype;

/* cce_backward flags. */
#define CCE_BWD_NO_KAHAN 1u /* plain fp32 accumulation of dE across blocks (numerics studies) */
#define CCE_BWD_FULL_DE 2u  /* dE from every block (unfiltered, Kahan-compensated), dH filtered:
                               the "full classifier gradient" variant; every tile is recomputed */
#define CCE_BWD_FINE_FILTER 8u /* the filter decides per 32 x 32 sub-tile (32 valid tokens x 32 vocabulary
                                  entries in processing order, a quarter of a filter block's side) instead
                                  of per 128 x 128 block: a sub-tile keeps the softmax part of its entries
                                  iff one of them other than a label entry has p >= filter_eps, and the
                                  dH / dE products skip the sub-tiles left all zero.  Not combined with
                                  CCE_BWD_FULL_DE (CCE_ERR_ARG). */
#define CCE_BWD_DEBUG_STORE_LIMIT 4u /* debug: kept blocks take store slots only below half of the store's
                                        capacity, as if the pass plan had overfilled it; the blocks left
                                        without a slot are dropped and counted in stats[5] (the gradients
                                        are then incomplete).  Exercises the overflow report. */

/* Human-readable name of a status code (static string, never NULL). */
const char *cce_status_string(cce_status s);

/* Library version as major*10000 + minor*100 + patch. */
int cce_version(void);

/*
 * Block geometry of the gradient filter, written to host ints (either may be
 * NULL): rows (valid tokens, in order) x vocabulary entries (in processing
 * order: sorted order when a permutation is given) per filter block.
 */
void cce_filter_block(int *block_rows, int *block_vocab);

/* Workspace bytes for cce_forward with these sizes (0 on invalid sizes). */
size_t cce_forward_workspace_bytes(int64_t N, int64_t D, int64_t V, cce_dtype dtype);

/* Workspace bytes for cce_backward with these sizes (0 on invalid sizes).
 * It grows linearly in N and in V: a fixed-width slice of the logit gradient
 * (rows x a bounded number of vocabulary columns) and fp32 dH accumulators;
 * never rows x vocabulary. */
size_t cce_backward_workspace_bytes(int64_t N, int64_t D, int64_t V, cce_dtype dtype);

/* Workspace bytes for cce_vocab_order (0 on invalid sizes). */
size_t cce_vocab_order_workspace_bytes(int64_t N, int64_t D, int64_t V, cce_dtype dtype);

/* Elements (fp32) of the optional block-max table of cce_forward /
 * cce_backward: 4 * ceil(N / 256) * ceil(V / 256) (one per 128 x 128 block of
 * the logit matrix) + N (one label logit per row); 0 on invalid sizes. */
size_t cce_block_max_elems(int64_t N, int64_t V);

/*
 * Forward: loss[i] and lse[i] for every row (fp32, device, [N]).
 * Ignored rows get loss = lse = 0.  The log-sum-exp is accumulated per
 * vocabulary split on chip (online max / sum-exp) and the splits are merged in
 * a fixed order, so the result does not depend on scheduling.
 * perm: NULL, or a permutation of 0..V-1 (int32, device, [V], e.g. from
 *   cce_vocab_order): vocabulary entries are visited in the order perm[0],
 *   perm[1], ...  The loss only changes by rounding order; entries of perm
 *   outside [0, V) read entry 0 instead (the caller guarantees a permutation).
 * block_max: NULL, or device fp32 [cce_block_max_elems(N, V)] that receives
 *   (1) the largest logit other than a label entry (i, y_i) of every
 *   128 x 128 block of the logit matrix of the non-ignored rows (in order) and
 *   the vocabulary in processing order, row-major over [2 ceil(N / 256) row
 *   blocks, 2 ceil(V / 256) vocabulary blocks] (-inf for blocks with no valid
 *   row), then (2) the label logit z_{i, y_i} of every non-ignored row i with
 *   a valid label, at index i of an [N] array (other entries untouched), as
 *   the logit tiles computed it.
 * ws: device scratch of at least cce_forward_workspace_bytes bytes.
 */
cce_status cce_forward(const void *H, const void *E, const int64_t *labels,
                       int64_t N, int64_t D, int64_t V, cce_dtype dtype,
                       int64_t ignore_index, const int32_t *perm, float *loss, float *lse,
                       float *block_max, void *ws, size_t ws_bytes, void *stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory or
 * pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Computes exactly what cce_forward
 * computes (bit-identical outputs) with the workspace in a file-scope device
 * array of CCE_NOALLOC_SCRATCH_BYTES bytes that the library holds on every
 * GPU it runs on until the process ends; it calls no allocation routine.
 * The stream must belong to the current device.  Returns CCE_ERR_WORKSPACE
 * (before any work is enqueued) when cce_forward_workspace_bytes(N, D, V,
 * dtype) exceeds CCE_NOALLOC_SCRATCH_BYTES (e.g. N = 2^20 tokens, or
 * V = 2^22 entries).  All calls on one GPU share that array: calls that
 * overlap in time on one GPU (other streams, other host threads) race and
 * must be serialised by the caller.  The first call on a device looks the
 * array's address up (HIP loads the code object if it is not yet loaded).
 */
#define CCE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
cce_status cce_forward_noalloc(const void *H, const void *E, const int64_t *labels,
                               int64_t N, int64_t D, int64_t V, cce_dtype dtype,
                               int64_t ignore_index, const int32_t *perm, float *loss, float *lse,
                               float *block_max, void *stream);

/*
 * Vocabulary order for the backward (optional): key_v = mean over
 * non-ignored rows of z_iv = <mean_i h_i, e_v>, sorted descending, ties by
 * ascending id (stable).  perm[k] (int32, device, [V]) receives the original
 * id at sorted position k.  keys (fp32, device, [V]) may be NULL; if given it
 * receives key_v indexed by original id.  With no valid row all keys are 0 and
 * perm is the identity.
 * The lit note's "Contribution": a vocabulary sort groups the surviving
 * blocks so that skipping at block granularity pays.
 */
cce_status cce_vocab_order(const void *H, const void *E, const int64_t *labels,
                           int64_t N, int64_t D, int64_t V, cce_dtype dtype,
                           int64_t ignore_index, int32_t *perm, float *keys,
                           void *ws, size_t ws_bytes, void *stream);

/*
 * Backward: dH [N, D] and dE [V, D] (input dtype, device) of
 * L = sum_i dloss[i] * loss_i, given lse from cce_forward.
 *  - dloss: fp32 [N]; it carries the caller's reduction (1/N_valid for a mean).
 *  - block_max: NULL, or the table cce_forward wrote for these same H, E,
 *    labels and perm.  With it (and filter_eps > 0), a 128 x 128 block
 *    whose largest non-label logit is so far below the smallest lse of its
 *    rows that every such p_iv is < filter_eps / 2 cannot keep its softmax
 *    part, and a 256 x 256 logit tile made only of such blocks is not
 *    recomputed (its label entries take the table's label logits); the
 *    outputs are bit-identical to the run without the table.
 *  - filter_eps >= 0: a filter block (see cce_filter_block) drops the
 *    softmax part of its entries when every p_iv in it other than a label
 *    entry is < filter_eps; 0 disables filtering.  A label entry (i, y_i)
 *    always keeps its whole gradient dloss_i (p_{i,y_i} - 1).
 *  - perm: NULL, or the permutation from cce_vocab_order (int32 [V]); it only
 *    changes which vocabulary entries share a filter block.
 *  - flags: 0 or any of CCE_BWD_NO_KAHAN, CCE_BWD_FULL_DE, CCE_BWD_FINE_FILTER,
 *    CCE_BWD_DEBUG_STORE_LIMIT.
 *  - stats: NULL, or device int64 [7] that receives (softmax-surviving blocks,
 *    label-only blocks, total blocks, valid rows, recomputed blocks, kept
 *    blocks dropped because a pass's block store was full, 32 x 32 sub-tiles
 *    whose softmax part is kept).  Entry 5 is 0 unless
 *    CCE_BWD_DEBUG_STORE_LIMIT is set: the pass plan sizes every pass to fit
 *    the store, and a nonzero count means the gradients are incomplete.
 *    Entry 6 counts all 16 sub-tiles of a surviving block unless
 *    CCE_BWD_FINE_FILTER is set.
 * Ignored rows get dH = 0 and add nothing to dE.
 * ws: device scratch of at least cce_backward_workspace_bytes bytes.
 */
cce_status cce_backward(const void *H, const void *E, const int64_t *labels,
                        const float *lse, const float *dloss, const float *block_max,
                        int64_t N, int64_t D, int64_t V, cce_dtype dtype,
                        int64_t ignore_index, float filter_eps,
                        const int32_t *perm, unsigned flags,
                        void *dH, void *dE, int64_t *stats,
                        void *ws, size_t ws_bytes, void *stream);

/*
 * Composite head (the lit note's "What transfers to us": a base classifier
 * plus a second block of rows placed at an id offset, with a dead gap
 * between them; the log-sum-exp is composed over the two blocks and the gap
 * contributes nothing).  Ids [0, V0) are rows of E0 [V0, D]; ids
 * [off1, off1 + V1) are rows of E1 [V1, D]; ids in [V0, off1) have no row
 * (logit -inf) and are never a valid label.  Requires V0, V1 >= 1 and
 * off1 >= V0.  The kernels see one vocabulary of V = V0 + V1 entries (E0's
 * rows, then E1's): workspace queries, cce_block_max_elems and perm
 * (int32 [V0 + V1]) take that V, and perm / keys index that space (entry
 * V0 + j is row j of E1).  Labels keep the caller's ids.  Everything else is
 * as for cce_forward / cce_vocab_order / cce_backward; dE0 [V0, D] and
 * dE1 [V1, D] receive the gradients of the two blocks.  A label in the gap
 * or past the second block gets loss = lse = NaN (undefined, as any label
 * out of range).
 */
cce_status cce_forward_composite(const void *H, const void *E0, int64_t V0, const void *E1, int64_t V1,
                                 int64_t off1, const int64_t *labels, int64_t N, int64_t D, cce_dtype dtype,
                                 int64_t ignore_index, const int32_t *perm, float *loss, float *lse,
                                 float *block_max, void *ws, size_t ws_bytes, void *stream);
cce_status cce_vocab_order_composite(const void *H, const void *E0, int64_t V0, const void *E1, int64_t V1,
                                     const int64_t *labels, int64_t N, int64_t D, cce_dtype dtype,
                                     int64_t ignore_index, int32_t *perm, float *keys, void *ws, size_t ws_bytes,
                                     void *stream);
cce_status cce_backward_composite(const void *H, const void *E0, int64_t V0, const void *E1, int64_t V1,
                                  int64_t off1, const int64_t *labels, const float *lse, const float *dloss,
                                  const float *block_max, int64_t N, int64_t D, cce_dtype dtype,
                                  int64_t ignore_index, float filter_eps, const int32_t *perm, unsigned flags,
                                  void *dH, void *dE0, void *dE1, int64_t *stats, void *ws, size_t ws_bytes,
                                  void *stream);

/*
 * Debug check of the labels: *n_bad (device int64) receives the number of rows
 * whose label is neither ignore_index nor in [0, V).
 */
cce_status cce_check_labels(const int64_t *labels, int64_t N, int64_t V,
                            int64_t ignore_index, int64_t *n_bad, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CCE_H_ */
