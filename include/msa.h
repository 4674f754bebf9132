/*
 * msa.h -- C ABI of libmsa.so, the MI355X (gfx950) MiniMax Sparse Attention hot path.
 *
 * The operations are those of the page "MiniMax-M3: MSA 技术报告速读"
 * (mloasisblog.com/blog/ML/minimax-m3-msa-tech-report), section 核心机制:
 *   index branch (索引分支): token scores S^idx = Q_idx K_idx^T / sqrt(d_idx) for
 *     visible keys, causal max-pool into fixed-size key blocks (M^idx), and a
 *     per-GQA-group TopK over blocks with the query's own block always kept;
 *   main branch (主分支): softmax(Q K[I]^T / sqrt(d_h)) V[I] over the visible
 *     tokens of the selected blocks I, all query heads of a group sharing the
 *     group's selection.
 *
 * Conventions shared by every entry point
 *   - All pointers are DEVICE pointers to dense, contiguous, row-major buffers
 *     owned by the caller. The library keeps no pointer after a call returns,
 *     never allocates, frees or synchronises, and enqueues its kernels on
 *     `stream` (a hipStream_t; NULL is the default stream).
 *   - A query row t (0 <= t < n_q) sits at absolute position p = q_start + t and
 *     sees keys j <= p. Head h belongs to group r = h / (h_q / h_kv).
 *     Block c covers keys [c*block_size, (c+1)*block_size); n_blocks =
 *     ceil(n_k / block_size); the local block of row t is floor(p / block_size).
 *   - Layouts (K, V and K_idx have a token stride of kv_capacity, n_k of which
 *     are valid):
 *       q      [batch, h_q,  n_q, d_h]          k, v   [batch, h_kv, kv_capacity, d_h]
 *       q_idx  [batch, h_kv, n_q, d_idx]        k_idx  [batch, kv_capacity, d_idx]
 *       sel    [batch, h_kv, n_q, top_k] int32  o      [batch, h_q, n_q, d_h]
 *       lse    [batch, h_q, n_q] float32        block_scores [batch, h_kv, n_q, n_blocks] float32
 *     q, k, v, q_idx, k_idx and o share the element type `dtype`.
 *   - Errors: a call validates everything it can on the host first; on any
 *     error it returns a negative code, enqueues nothing and sets the text
 *     returned by msa_last_error(). Launch failures return MSA_ERR_HIP.
 *   - Empty calls: with batch == 0 or n_q == 0 there is nothing to compute. Such a
 *     call still checks the shape and the supported set, then returns MSA_OK
 *     without touching any pointer or enqueueing anything; workspace sizes are 0.
 *
 * Supported set: dtype F32 or BF16; d_h in {64, 128}; d_idx in {32, 64};
 * block_size in {32, 64}; 1 <= top_k <= 64; h_kv and h_q / h_kv in
 * {1, 2, 4, 8, 16}; at most 2048 * 2048 / (top_k - 1) candidate blocks before the
 * last row's own block.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MSA_F32 = 0, MSA_BF16 = 1 } msa_dtype;

enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = -1, /* null pointer, bad size, range or divisibility */
  MSA_ERR_UNSUPPORTED = -2, /* a dtype / d_h / d_idx / block_size / top_k combination with no kernel */
  MSA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than *_workspace_size reports */
  MSA_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
};

typedef struct {
  int32_t batch;       /* sequences, >= 0 (0: empty call) */
  int32_t n_q;         /* query rows per sequence, >= 0 (0: empty call) */
  int32_t n_k;         /* valid keys per sequence, >= 0; q_start + n_q <= n_k */
  int32_t q_start;     /* absolute position of row 0, >= 0 */
  int32_t h_q;         /* query heads */
  int32_t h_kv;        /* KV heads = GQA groups = index heads */
  int32_t d_h;         /* head dim of q, k, v, o */
  int32_t d_idx;       /* head dim of q_idx, k_idx */
  int32_t block_size;  /* tokens per key block */
  int32_t top_k;       /* blocks selected per (row, group), counting the local block */
  int32_t dtype;       /* msa_dtype */
  int32_t kv_capacity; /* token stride of k, v, k_idx; 0 means n_k; else >= n_k */
} msa_shape;

/*
 * Workspace bytes msa_index_topk needs for `shape` (block maxima and top-k
 * candidates). Returns MSA_OK and writes *bytes, or an error code.
 */
int msa_index_topk_workspace_size(const msa_shape *shape, size_t *bytes);

/*
 * Index branch: block selection (S^idx, causal block max-pool M^idx and TopK of
 * the index-branch equations, with the local block forced).
 *   q_idx, k_idx  inputs (layouts above)
 *   sel           out: for each (b, group, row) the selected blocks in ascending
 *                 order, -1 padded. Selection: the local block, plus the top_k-1
 *                 earlier blocks with the highest block score, equal scores going
 *                 to the lower block index; a row that sees top_k blocks or fewer
 *                 selects all of them. The positive 1/sqrt(d_idx) factor does not
 *                 change the order and is not applied.
 *   block_scores  optional out (NULL to skip): raw block maxima of q_idx . k_idx
 *                 over visible keys, -inf for blocks after the local block.
 *   workspace     device scratch of at least msa_index_topk_workspace_size bytes.
 * Scores accumulate in fp32 from exact products of the inputs.
 */
int msa_index_topk(const msa_shape *shape, const void *q_idx, const void *k_idx, int32_t *sel,
                   float *block_scores, void *workspace, size_t workspace_bytes, void *stream);

/*
 * msa_index_topk as two stages on one workspace (for timing or overlapping them
 * separately): running msa_index_topk_scores then msa_index_topk_select on the same
 * stream, with the same shape, block_scores (both NULL, or both the same buffer) and
 * workspace, does exactly what msa_index_topk does with those arguments.
 *   msa_index_topk_scores  S^idx and the causal block max-pool M^idx: the block
 *                          maxima (into block_scores if given, else the workspace)
 *                          and, for rows with more than 2048 candidate blocks, the
 *                          largest score of every aligned run of 32 blocks, which
 *                          lets the select stage read only the runs that can hold a
 *                          winner. Decode shapes: the first selection stage as well.
 *   msa_index_topk_select  the TopK with the local block forced, from the workspace
 *                          (and block_scores) the scores stage filled; writes sel.
 * Arguments, layouts and errors as for msa_index_topk; the workspace holds the
 * stage-1 results until the select stage has run.
 */
int msa_index_topk_scores(const msa_shape *shape, const void *q_idx, const void *k_idx,
                          float *block_scores, void *workspace, size_t workspace_bytes,
                          void *stream);
int msa_index_topk_select(const msa_shape *shape, const float *block_scores, int32_t *sel,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * The index branch in two calls with the block scores in a caller-owned buffer
 * and no shared workspace: the same index kernel as msa_index_topk, then a TopK
 * that ranks every candidate of the scores (rows with more than 2048 candidates in
 * chunks of 2048 plus a merge):
 *
 * msa_index_block_scores: token scores and causal block max-pool only. Writes,
 *   for every (b, group, row), the raw block maxima of q_idx . k_idx over the
 *   visible keys of every block up to the row's local block; entries after the
 *   local block are -inf or left unwritten (pre-fill the buffer if they matter).
 *   block_scores [batch, h_kv, n_q, n_blocks] float32, caller-owned.
 */
int msa_index_block_scores(const msa_shape *shape, const void *q_idx, const void *k_idx,
                           float *block_scores, void *stream);

/* Workspace bytes msa_topk_from_block_scores needs (top-k chunk candidates). */
int msa_topk_workspace_size(const msa_shape *shape, size_t *bytes);

/*
 * msa_topk_from_block_scores: the TopK step with the local block forced, from
 *   block scores as written by msa_index_block_scores (only entries before each
 *   row's local block are read). Output `sel` as for msa_index_topk. d_idx is
 *   not used.
 */
int msa_topk_from_block_scores(const msa_shape *shape, const float *block_scores, int32_t *sel,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * Workspace bytes the attention entry points need for `shape`: the prefill lists
 * and partials, or for a decode shape (n_q == 1, q_start == n_k - 1) the larger of
 * that and the decode split partials, so either entry point can use it.
 * Returns MSA_OK and writes *bytes.
 */
int msa_sparse_attn_workspace_size(const msa_shape *shape, size_t *bytes);

/*
 * Main branch, prefill or chunked prefill (any n_q, q_start): for every head h of
 * group r and row t, o = softmax(q k_T^T / sqrt(d_h)) v_T over T = the visible
 * tokens (j <= p) of the blocks listed in sel[b, r, t, :] (entries < 0 ignored).
 *   q, k, v  inputs; sel as produced by msa_index_topk (ascending, -1 padded; each
 *            valid entry must be a block whose first key is <= p)
 *   o        out, dtype of q; rounded to nearest even for bf16
 *   lse      optional out (NULL to skip): natural-log sum of exp of the scaled scores
 *   workspace at least msa_sparse_attn_workspace_size bytes: the per-block query lists
 *            and one unnormalised partial output per (row, group, selected block), i.e.
 *            about batch * h_kv * n_q * top_k * (h_q / h_kv) * d_h * sizeof(dtype) bytes.
 * Computed KV-block-outer: each selected block is staged once per chunk of the rows that
 * chose it, and the partials are merged with log-sum-exp weights (no float atomics).
 * Per call: fewer than 2^31 selection entries (batch * h_kv * n_q * top_k), n_q < 2^25
 * and batch * h_q * n_q * d_h < 2^35 output elements; larger calls return UNSUPPORTED.
 */
int msa_sparse_attn_prefill(const msa_shape *shape, const void *q, const void *k, const void *v,
                            const int32_t *sel, void *o, float *lse, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * The three stages of msa_sparse_attn_prefill as separate calls, for callers that
 * schedule or time them apart. Called in this order with the same shape and the same
 * workspace (whose contents carry over from one stage to the next) on one stream, they
 * give the same bits as the single call; the workspace size is the same too.
 *   _plan      reads sel and builds the per-block query lists in the workspace.
 *   _partials  reads q, k, v and the lists; writes one partial output per selection.
 *   _merge     reads sel and the partials; writes o and (optional) lse.
 * Arguments mean what they mean for msa_sparse_attn_prefill; the same errors apply.
 */
int msa_sparse_attn_prefill_plan(const msa_shape *shape, const int32_t *sel, void *workspace,
                                 size_t workspace_bytes, void *stream);
int msa_sparse_attn_prefill_partials(const msa_shape *shape, const void *q, const void *k,
                                     const void *v, void *workspace, size_t workspace_bytes,
                                     void *stream);
int msa_sparse_attn_prefill_merge(const msa_shape *shape, const int32_t *sel, void *o, float *lse,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Main branch, single-token decode: n_q == 1 and q_start == n_k - 1 (the new
 * token's k, v and k_idx are already in the caches at position n_k - 1). Same
 * result as msa_sparse_attn_prefill for that row, computed by a split over the
 * selected blocks and a log-sum-exp merge (pre-scheduled, no atomics). Any n_k.
 *   workspace  at least msa_sparse_attn_workspace_size bytes.
 */
int msa_sparse_attn_decode(const msa_shape *shape, const void *q, const void *k_cache,
                           const void *v_cache, const int32_t *sel, void *o, float *lse,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * One whole decode step ("MiniMax-M3: MSA 技术报告速读", section 核心机制: the index-branch
 * score, max-pool and TopK equations with the forced local block, then the main-branch
 * equation): the same sel as msa_index_topk and the same o and lse, within rounding, as
 * msa_sparse_attn_decode on that sel, in two launches instead of four. The index kernel
 * streams k_idx and ranks each key range; one kernel then merges the ranges' winners,
 * attends the selected blocks and merges the log-sum-exp partials, the last of a (sequence,
 * group)'s workgroups to finish combining them (the pages' split with a second merge stage,
 * with a device-scope arrival counter per (sequence, group) that the index kernel of the
 * same call clears).
 *   shape   n_q == 1 and q_start == n_k - 1; d_idx, d_h, block_size and top_k as for the
 *           two calls it replaces (top_k == 1, or more candidate blocks than one merge
 *           takes, runs those two calls on this workspace instead).
 *   q, k_cache, v_cache, q_idx, k_idx   as for msa_sparse_attn_decode and msa_index_topk.
 *   sel     out [batch, h_kv, 1, top_k] int32, as msa_index_topk writes it.
 *   o, lse  out, as msa_sparse_attn_decode writes them (lse may be NULL).
 *   workspace  at least msa_decode_step_workspace_size bytes, caller-owned; its first
 *           bytes hold the counters, which the call clears itself (no zero fill needed).
 *           Calls that share one workspace must not overlap in time.
 * Errors: those of msa_index_topk and msa_sparse_attn_decode.
 */
int msa_decode_step_workspace_size(const msa_shape *shape, size_t *bytes);
int msa_decode_step(const msa_shape *shape, const void *q, const void *k_cache, const void *v_cache,
                    const void *q_idx, const void *k_idx, int32_t *sel, void *o, float *lse,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * msa_decode_step for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels, the
 * same results bit for bit, with the workspace taken from a scratch array of
 * MSA_DECODE_STEP_SCRATCH_BYTES that the library holds in device memory, one per GPU, for
 * the life of the process. The call allocates and frees nothing.
 *   Arguments as for msa_decode_step, without the workspace.
 *   Shapes whose msa_decode_step_workspace_size exceeds MSA_DECODE_STEP_SCRATCH_BYTES are
 *   rejected with MSA_ERR_WORKSPACE before anything is enqueued (32 MiB covers, e.g.,
 *   32 sequences of 262144 tokens or 4 of 1048576 at 32 heads, 4 groups, d_h 128, top_k 32).
 *   Every call on one GPU uses that GPU's one array: calls that overlap in time on the same
 *   GPU (two streams, two threads) race and give wrong results; the caller serialises
 *   them. The array keeps the last call's contents; what must start at zero (the arrival
 *   counters) is cleared by each call's own first kernel.
 * Errors: those of msa_decode_step; MSA_ERR_HIP when the array's address cannot be taken.
 */
#define MSA_DECODE_STEP_SCRATCH_BYTES ((size_t)32 << 20)
int msa_decode_step_noalloc(const msa_shape *shape, const void *q, const void *k_cache,
                            const void *v_cache, const void *q_idx, const void *k_idx, int32_t *sel,
                            void *o, float *lse, void *stream);

/*
 * Index-branch alignment loss ("MiniMax-M3: MSA 技术报告速读", section 训练: the equations
 * for P^idx, P^(r) and L_KL), for every (b, group r, row t) over T = the visible tokens of
 * the blocks in sel[b, r, t, :]:
 *   student  P^idx = softmax over T of S^idx_j = q_idx . k_idx_j / sqrt(d_idx)
 *   teacher  P^(r) = mean over the group's G heads h of softmax over T of q_h . k_j / sqrt(d_h)
 *   kl[b, r, t] = KL(P^(r) || P^idx) = sum_j P^(r)_j (ln P^(r)_j - ln P^idx_j)
 *   q, k, q_idx, k_idx, sel  as for msa_sparse_attn_prefill and msa_index_topk (any n_q and
 *            q_start, decode rows included)
 *   lse      [batch, h_q, n_q] float32: the natural-log LSE the attention entry points
 *            write for the same q, k and sel; the teacher's probabilities are
 *            exp(q_h . k_j / sqrt(d_h) - lse)
 *   kl       out [batch, h_kv, n_q] float32
 *   lse_idx  optional out (NULL to skip) [batch, h_kv, n_q] float32: ln sum_T exp(S^idx_j),
 *            the student's normaliser
 *   workspace at least msa_sparse_attn_workspace_size bytes (its lists and partials).
 * Computed KV-block-outer over the same per-block row lists as the prefill attention:
 * per selection, the block's sums of t ln t, t S^idx and t (t the teacher's weight) and
 * the index scores' max and sum of exponentials, then a per-row merge. Supported set and
 * size limits as for msa_sparse_attn_prefill plus d_idx in {32, 64}.
 */
int msa_index_kl(const msa_shape *shape, const void *q, const void *k, const void *q_idx,
                 const void *k_idx, const int32_t *sel, const float *lse, float *kl,
                 float *lse_idx, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The index branch's two projections ("MiniMax-M3: MSA 技术报告速读", section 核心机制,
 * 索引分支: standard GQA plus an index query with one head per group and an index key
 * shared by the groups), from the hidden states of the call's rows:
 *   q_idx[b, r, t, d]          = sum_i x[b, t, i] * w_qidx[r * d_idx + d, i]
 *   k_idx[b, q_start + t, d]   = sum_i x[b, t, i] * w_kidx[d, i]
 *   x        [batch, n_q, d_model], dtype; row t is the token at position q_start + t
 *   w_qidx   [h_kv * d_idx, d_model], dtype, one row per output (a linear layer's weight)
 *   w_kidx   [d_idx, d_model], dtype
 *   q_idx    out [batch, h_kv, n_q, d_idx] (the layout msa_index_topk reads)
 *   k_idx    the index-key cache [batch, kv_capacity, d_idx]: rows q_start .. q_start +
 *            n_q - 1 are written (the append of the call's tokens; for a decode shape the
 *            new token's row n_k - 1), every other row is left as it is
 * fp32 accumulation, results rounded to nearest even for bf16. No workspace. Uses batch,
 * n_q, q_start, h_kv, d_idx, dtype and kv_capacity of the shape (the rest must still be a
 * valid shape). Supported: d_idx in {32, 64}, d_model a positive multiple of 64, fewer than
 * 2^36 rows per call.
 */
int msa_index_project(const msa_shape *shape, int32_t d_model, const void *x, const void *w_qidx,
                      const void *w_kidx, void *q_idx, void *k_idx, void *stream);
/*
 * Workspace bytes msa_sparse_attn_backward needs for `shape`: the per-block query lists,
 * one partial dq per (row, group, selected block, head) (about batch * h_kv * n_q *
 * top_k * (h_q / h_kv) * d_h * sizeof(dtype) bytes, as for the prefill), D per (b, h, t)
 * and the fp32 dk/dv partials of the per-block pass. Returns MSA_OK and writes *bytes.
 */
int msa_sparse_attn_backward_workspace_size(const msa_shape *shape, size_t *bytes);
/*
 * Gradients of the main branch ("MiniMax-M3: MSA 技术报告速读", section 核心机制 for the
 * forward; section 训练 detaches the index branch, so sel is a constant here) with respect
 * to q, k and v, for the forward msa_sparse_attn_prefill computes on the same shape. For
 * each head h of group r and row t, over T = the visible tokens of the blocks in
 * sel[b, r, t, :], with P_j = exp(q . k_j / sqrt(d_h) - lse), dP_j = dout . v_j and
 * D = dout . o:
 *   dq      = sum_j P_j (dP_j - D) k_j / sqrt(d_h)
 *   dk_j   += P_j (dP_j - D) q / sqrt(d_h)     summed over every (row, head) whose T holds j
 *   dv_j   += P_j dout                         likewise
 *   q, k, v, sel  the forward's inputs (layouts above)
 *   o, lse   the forward's outputs for them (lse: natural log, as msa_sparse_attn_prefill
 *            writes it)
 *   dout     [batch, h_q, n_q, d_h], dtype of q: the gradient of the loss with respect to o
 *   dq       out [batch, h_q, n_q, d_h], dtype of q
 *   dk, dv   out [batch, h_kv, kv_capacity, d_h], dtype of q: rows 0..n_k-1 are written
 *            (zero for keys no row of the call sees); rows from n_k on are not touched
 *   workspace at least msa_sparse_attn_backward_workspace_size bytes.
 * Computed KV-block-outer over the same per-block row lists as the prefill: each staged
 * block yields its dk, dv rows and one partial dq per selection, then the dq partials are
 * summed per row and the block partials per block, in fixed orders (no float atomics).
 * dk and dv sum each chunk of a block's rows in list order, which the list build sets
 * with integer atomics, so they can differ in the last bits between calls; dq does not.
 * Supported set and size limits as for msa_sparse_attn_prefill.
 */
int msa_sparse_attn_backward(const msa_shape *shape, const void *q, const void *k, const void *v,
                             const int32_t *sel, const void *o, const float *lse, const void *dout,
                             void *dq, void *dk, void *dv, void *workspace, size_t workspace_bytes,
                             void *stream);
/*
 * The backward in three calls, for callers that schedule or time the stages apart. Called
 * in this order with the same shape and workspace (whose contents carry over) on one
 * stream, they compute what msa_sparse_attn_backward computes (dq bit for bit; dk and dv
 * up to the last-bit effect of the list order described above).
 *   _plan      reads sel, o and dout: builds the per-block query lists and D = dout . o.
 *   _partials  reads q, k, v, lse, dout and the lists: writes the dq partials and the
 *              dk/dv block partials.
 *   _merge     reads sel and the partials: writes dq, dk and dv.
 * Arguments mean what they mean for msa_sparse_attn_backward; the same errors apply.
 */
int msa_sparse_attn_backward_plan(const msa_shape *shape, const int32_t *sel, const void *o,
                                  const void *dout, void *workspace, size_t workspace_bytes,
                                  void *stream);
int msa_sparse_attn_backward_partials(const msa_shape *shape, const void *q, const void *k,
                                      const void *v, const float *lse, const void *dout,
                                      void *workspace, size_t workspace_bytes, void *stream);
int msa_sparse_attn_backward_merge(const msa_shape *shape, const int32_t *sel, void *dq, void *dk,
                                   void *dv, void *workspace, size_t workspace_bytes, void *stream);
/* Text of the last error on the calling thread (empty after a successful call). */
const char *msa_last_error(void);

/* ABI version of this header: 1. */
int msa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
