/*
 * dsai.h - C ABI of the MI355X (gfx950) DSA lightning-indexer selection library.
 *
 * The library computes the DeepSeek-Sparse-Attention indexer's token
 * selection with hand-written HIP kernels:
 *
 *   - dsai_score_topk: per-head index scores of bf16 index_q against bf16
 *     index_k, ReLU per head, fp32 per-head weights reducing over heads,
 *     the causal mask under compress_ratio, and a per-query top-k, fused in
 *     one kernel so the [S, Skv] score matrix never reaches device memory.
 *     Contract from the NeMo AutoModel page
 *     "nemo_automodel.components.models.deepseek_v4.kernels.tilelang_indexer"
 *     (V4IndexerFunction / v4_lighting_indexer: SBHD layout, index_q
 *     [seqlen, batch, heads, dim] bf16, index_k [seqlen_kv, batch, dim] bf16,
 *     weights [seqlen, batch, heads] fp32, compress_ratio, topk, result
 *     [batch, seqlen, topk]).
 *   - the pooled decode pipeline of the page "Module glm5next_dsa"
 *     ("Shape of the pipeline"): dsai_kpool_compress -> dsai_index_scores ->
 *     dsai_topk_pools -> dsai_expand (dsai_select runs the middle two).
 *
 * Conventions for every call:
 *   - Pointers to tensors are DEVICE pointers, owned by the caller; the
 *     library never keeps them past the call and never allocates device
 *     memory inside a compute call.  bf16 tensors are passed as `const void*`
 *     to 2-byte bfloat16 elements.  All tensors are dense, row-major
 *     (last index fastest), with the shapes given per call.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Compute calls
 *     only enqueue work on it and return; results are ready when the stream
 *     reaches that point.
 *   - Calls return a dsai status (DSAI_OK = 0, negative on error).  When a
 *     call returns an error before any launch, nothing was enqueued; on
 *     DSAI_ERR_HIP a launch failed and the HIP error code is kept in the
 *     handle (dsai_last_hip_error).  No C++ exception crosses the ABI.
 *   - A handle is used by one host thread at a time.  Calls that share
 *     output buffers on one stream are ordered by that stream.
 *   - Argument validation runs on the host before any HIP call, so every
 *     error code below can be raised without a GPU.
 */
#ifndef DSAI_H_
#define DSAI_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define DSAI_OK 0
#define DSAI_ERR_INVALID_ARG (-1) /* a size, ratio, topk or config value out of range */
#define DSAI_ERR_UNSUPPORTED (-2) /* a legal request this build does not implement   */
#define DSAI_ERR_WORKSPACE (-3)   /* workspace pointer NULL or smaller than required   */
#define DSAI_ERR_NULLPTR (-4)     /* a required pointer is NULL                        */
#define DSAI_ERR_HIP (-5)         /* a HIP call or kernel launch failed                */

/* Most pool slots kpool_compress holds (the "Module glm5next_dsa" page,
 * constant KERNEL_MAX_KPOOL: larger index_kpool values are refused at
 * configuration time instead of silently dropping slots). */
#define DSAI_MAX_KPOOL 8
/* Largest topk / select_k the fused selection supports (LDS capacity). */
#define DSAI_MAX_TOPK 8192
/* Heads and head dims the kernels are compiled for: heads 1..64
 * (zero-padded to 32 or 64 on the matrix cores), dim 32, 64 or 128. */
#define DSAI_MAX_HEADS 64

/* Rank the filter store's cuts keep (dsai_config.cuts); rows longer than
 * the dense store only.  Either way the rows are the exact top k:
 *   DSAI_CUTS_ESTIMATED  a cut after n of a row's N keys keeps k n / N plus
 *                        six standard deviations of that count and 32
 *                        (the share of the top k the first n keys hold when
 *                        key order says nothing about the scores); a row
 *                        that ends with fewer than k entries although it
 *                        has k keys makes its block of rows run its keys
 *                        again with cuts to k (about twice that block's
 *                        time);
 *   DSAI_CUTS_TOPK       every cut keeps k: for callers whose key order
 *                        predicts the scores (e.g. scores that fall along
 *                        the sequence), where estimated cuts would rerun. */
#define DSAI_CUTS_ESTIMATED 0
#define DSAI_CUTS_TOPK 1

/* Order of the entries of a top-k row (dsai_config.order). */
#define DSAI_ORDER_SCORE 0 /* score descending, lower index first among equal scores */
#define DSAI_ORDER_INDEX 1 /* ascending index (the same set, no sorting pass)          */

/* ---- configuration / handle -------------------------------------------- */
typedef struct dsai_config {
  int heads;      /* H, index heads per query, 1..64                          */
  int dim;        /* D, index head dim: 32, 64 or 128                          */
  int kpool;      /* index_kpool: token slots per pool, 1..DSAI_MAX_KPOOL      */
  int index_topk; /* tokens selected per pooled row: a nonzero multiple of
                     kpool (config invariant on the "Module glm5next_dsa"
                     page); select_k = index_topk / kpool pools per row       */
  int first_key;  /* first cached token that pools (>= 0)                      */
  int chunk_rows; /* query rows per launch of the scores at supplied
                     indices (0: all rows in one launch)                     */
  int order;      /* DSAI_ORDER_SCORE (default 0) or DSAI_ORDER_INDEX: order of
                     the entries of each dsai_score_topk / dsai_topk_pools /
                     dsai_select row (padding is always at the tail)         */
  int cuts;       /* DSAI_CUTS_ESTIMATED (default 0) or DSAI_CUTS_TOPK: rank
                     the filter store's cuts keep (same results)             */
} dsai_config;

typedef struct dsai_context* dsai_handle;

/* Validate `cfg` and create a handle in *out.  Refuses (DSAI_ERR_INVALID_ARG)
 * kpool outside 1..8, index_topk not a positive multiple of kpool,
 * index_topk / kpool > DSAI_MAX_TOPK, heads < 1, first_key < 0,
 * chunk_rows < 0, order not DSAI_ORDER_SCORE / DSAI_ORDER_INDEX, cuts not
 * DSAI_CUTS_ESTIMATED / DSAI_CUTS_TOPK;
 * DSAI_ERR_UNSUPPORTED for heads > 64 or dim not 32/64/128;
 * DSAI_ERR_NULLPTR for a NULL cfg or out.  Makes no HIP call. */
int dsai_create(const dsai_config* cfg, dsai_handle* out);

/* Release a handle (NULL is accepted).  Waits for nothing. */
int dsai_destroy(dsai_handle h);

/* Static text for a status code (never NULL). */
const char* dsai_status_string(int status);

/* HIP error code (hipError_t value) of the last failed launch on `h`, 0 if none. */
int dsai_last_hip_error(dsai_handle h);

/* ---- unpooled lightning indexer ---------------------------------------- */
/* Fused score + causal/compressed mask + top-k (v4_lighting_indexer forward).
 *
 *   index_q  [S, B, H, D]  bf16   (SBHD: query position, batch, head, dim)
 *   index_k  [Skv, B, D]   bf16
 *   weights  [S, B, H]     fp32
 *   out_idx  [B, S, topk]  int32  written
 *   out_score[B, S, topk]  fp32   written
 *
 * Score of key s for query position t in batch b:
 *   I = sum_h weights[t,b,h] * max(0, sum_d index_q[t,b,h,d] * index_k[s,b,d])
 * (products accumulated in fp32 on the matrix cores).  Key s is visible iff
 * s < min(Skv, floor((t+1) / compress_ratio)).  Each output row lists the
 * visible keys with the `topk` largest scores (ties at the boundary go to
 * the lower key index; +0 and -0 are equal), ordered by score descending and
 * the lower index first among equal scores (cfg.order DSAI_ORDER_SCORE) or
 * by ascending index (DSAI_ORDER_INDEX); rows with fewer visible keys are
 * padded with index -1 and score -inf.  Every output element is written.
 *
 * S, Skv, B >= 0 (S == 0 or B == 0: nothing is written or launched);
 * Skv < 2^31; compress_ratio >= 1; 1 <= topk <= DSAI_MAX_TOPK
 * (DSAI_ERR_INVALID_ARG otherwise); index_k must span < 4 GiB
 * (Skv * B * D * 2 bytes; DSAI_ERR_UNSUPPORTED otherwise).  The selection
 * runs as one launch on `stream` (plus the row-sort launch in score order);
 * no scratch memory is used and no score matrix is formed, at any size.
 * cfg.chunk_rows does not apply to the selection: the one launch covers
 * every row, its workgroups numbered from the last (longest) rows to the
 * first, so no chunk boundary leaves the GPU idle while a chunk's longest
 * rows finish.  Rows longer than the kernel's dense store (about 4600 keys
 * at dim 128) keep a filter store whose cuts follow cfg.cuts; the results
 * are the same with either setting, only the time differs (see
 * DSAI_CUTS_ESTIMATED).
 *
 * Scores at supplied indices (the page's optional topk_indices
 * [batch, seqlen, topk] int32, and pytorch_extract_topk_scores): when
 * topk_indices is not NULL no key is selected.  For each entry s of row
 * (b, t), in the supplied order, out_idx/out_score receive (s, I) if
 * 0 <= s < min(Skv, floor((t+1) / compress_ratio)), else (-1, -inf); I is
 * bit-identical to the score the selection reports for that key.
 * topk_indices is device memory, 16-byte aligned (DSAI_ERR_INVALID_ARG
 * otherwise), and may be out_idx itself (in place); cfg.order does not
 * apply; index_k has no 4 GiB limit on this form.  Its rows are scored in
 * launches of cfg.chunk_rows rows (all rows if 0); with more than one
 * chunk, consecutive chunks run on two streams the handle owns, forked from
 * `stream` (after the work already on it) and joined back to it (work
 * enqueued on `stream` later waits for every chunk); the streams and their
 * events are created at the first such call on a device and released by
 * dsai_destroy. */
int dsai_score_topk(dsai_handle h, const void* index_q, const void* index_k,
                    const float* weights, int64_t S, int64_t Skv, int64_t B,
                    int compress_ratio, int topk, const int32_t* topk_indices,
                    int32_t* out_idx, float* out_score, void* stream);

/* Packed sequences ("packed-sequence dispatch" among the local modifications
 * listed on the NeMo AutoModel page
 * "nemo_automodel.components.models.deepseek_v4.kernels"; the
 * tilelang_indexer page offers a per-sample interface).  The page gives no layout
 * for it; this call takes the plain reading that a packed batch is a set of
 * independent samples laid end to end, each the B = 1 problem of
 * dsai_score_topk:
 *
 *   index_q  [Tq, H, D]   bf16   rows of all sequences, concatenated
 *   index_k  [Tk, D]      bf16
 *   weights  [Tq, H]      fp32
 *   cu_seqlens_q, cu_seqlens_k: HOST arrays of nseq + 1 int64 offsets,
 *            0 = cu[0] <= cu[1] <= ... <= cu[nseq] = Tq (resp. Tk)
 *   topk_indices NULL, or [Tq, topk] int32 (scores at supplied indices)
 *   out_idx  [Tq, topk]   int32  written
 *   out_score[Tq, topk]   fp32   written
 *
 * Sequence i owns query rows cu_seqlens_q[i] .. cu_seqlens_q[i+1] - 1 and
 * keys cu_seqlens_k[i] .. cu_seqlens_k[i+1] - 1.  Its row at local position t
 * (0 at the sequence's first row) sees its local keys s < min(len_k,
 * floor((t+1) / compress_ratio)); indices, in and out, are local to the
 * sequence (what dsai_score_topk returns for that sequence alone), with the
 * same scores, ordering (cfg.order), ties and padding.  A sequence with no
 * keys gets padding rows.
 *
 * topk % 4 == 0 (every sequence's output then starts 16-byte aligned), nseq
 * >= 0, offsets as above, Tq and Tk < 2^31, compress_ratio >= 1
 * (DSAI_ERR_INVALID_ARG otherwise); a sequence whose keys span 4 GiB or
 * more, or a topk the selection cannot hold, gives DSAI_ERR_UNSUPPORTED;
 * every refusal comes before the first launch.  The selection runs as one
 * launch per 64 non-empty sequences, on `stream`, sequences taken from the
 * longest row down (a table in the launch arguments maps each workgroup to
 * its sequence); then, in score order, one row sort over all Tq rows on
 * `stream`.  With supplied indices: one launch per non-empty sequence (one
 * per cfg.chunk_rows rows of it, in order, if chunked), consecutive
 * sequences alternating between the handle's two streams, forked from
 * `stream` and joined back to it. */
int dsai_score_topk_packed(dsai_handle h, const void* index_q, const void* index_k,
                           const float* weights, int64_t nseq, const int64_t* cu_seqlens_q,
                           const int64_t* cu_seqlens_k, int compress_ratio, int topk,
                           const int32_t* topk_indices, int32_t* out_idx, float* out_score,
                           void* stream);

/* ---- backward: gradients of the selected scores ------------------------- */
/* Workspace bytes of dsai_indexer_backward for these sizes (the same
 * arguments as the call): an fp32 [Skv, B, cfg.dim] accumulator of grad_k
 * plus, when the entries are grouped by key block (Skv <= 262144 and
 * B <= 65535), (B * S) * (ceil(Skv / 256) + 1) int32 bucket bounds and
 * B * S * topk 8-byte bucketed entries.  Host-only; DSAI_ERR_INVALID_ARG for
 * the sizes dsai_indexer_backward refuses. */
int dsai_backward_workspace_size(dsai_handle h, int64_t S, int64_t Skv, int64_t B, int topk,
                                 int compress_ratio, size_t* bytes);

/* The backward of the indexer's autograd function (NeMo AutoModel page
 * "...deepseek_v4.kernels.tilelang_indexer", V4IndexerFunction.backward with
 * grad_scores and grad_indices): the gradient of the returned scores with
 * respect to index_q, index_k and weights.  The indices are integers and
 * take no gradient.  Entry j of row (b, t), key s = topk_indices[b,t,j], is
 * usable iff 0 <= s < min(Skv, floor((t+1) / compress_ratio)) (the forward
 * gives any other entry the constant score -inf); with g =
 * grad_scores[b,t,j] and d_h = sum_d index_q[t,b,h,d] * index_k[s,b,d], each
 * usable entry adds
 *   grad_weights[t,b,h] += g * max(0, d_h)
 *   grad_q[t,b,h,:]     += g * weights[t,b,h] * (d_h > 0) * index_k[s,b,:]
 *   grad_k[s,b,:]       += g * sum_h weights[t,b,h] * (d_h > 0) * index_q[t,b,h,:]
 * (ReLU's derivative is 0 at 0; repeated entries add once each).
 *
 *   index_q [S,B,H,D] bf16, index_k [Skv,B,D] bf16, weights [S,B,H] fp32,
 *   topk_indices [B,S,topk] int32 (e.g. dsai_score_topk's out_idx),
 *   grad_scores [B,S,topk] fp32;
 *   grad_q [S,B,H,D] bf16, grad_k [Skv,B,D] bf16, grad_weights [S,B,H] fp32
 *   written, every element (zero where nothing contributes).
 *
 * Arithmetic: d_h in fp32 on the matrix cores (the forward's products); the
 * gated weight g * weights * (d_h > 0) is rounded to bf16 as the operand of
 * the two gradient products, which accumulate in fp32 (for grad_k, the g of
 * a key listed more than once in a row are summed first); grad_k's sum over
 * query rows is accumulated in fp32 in the workspace (per key block and row
 * chunk, then added with fp32 atomics: the order of those additions is
 * unspecified); grad_q and grad_k are rounded to bf16 (nearest even) once
 * at the end.
 * With S and Skv both positive, the key gradients and the per-row
 * gradients run concurrently on the two streams the handle owns (see
 * dsai_score_topk), forked from `stream` and joined back to it.
 *
 * S, Skv, B >= 0 (< 2^31, also S*B and Skv*B); compress_ratio >= 1;
 * 1 <= topk <= DSAI_MAX_TOPK (DSAI_ERR_INVALID_ARG otherwise).  B == 0 or
 * S == Skv == 0: nothing is written or launched; S == 0 writes grad_k = 0.
 * workspace: device memory of dsai_backward_workspace_size bytes (same
 * sizes), 256-byte aligned (DSAI_ERR_WORKSPACE otherwise), overwritten.  index_q, index_k,
 * grad_q, grad_k 16-byte aligned; the other arrays 4-byte aligned
 * (DSAI_ERR_INVALID_ARG otherwise).  All arrays are device memory. */
int dsai_indexer_backward(dsai_handle h, const void* index_q, const void* index_k,
                          const float* weights, const int32_t* topk_indices,
                          const float* grad_scores, int64_t S, int64_t Skv, int64_t B,
                          int compress_ratio, int topk, void* grad_q, void* grad_k,
                          float* grad_weights, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Packed sequences for the backward (the reading of dsai_score_topk_packed:
 * samples laid end to end, each the B = 1 problem on its own rows and keys,
 * key indices local to the sequence):
 *   index_q, grad_q [Tq, H, D] bf16; weights, grad_weights [Tq, H] fp32;
 *   topk_indices [Tq, topk] int32, grad_scores [Tq, topk] fp32;
 *   index_k, grad_k [Tk, D] bf16; cu_seqlens_q / cu_seqlens_k: HOST arrays
 *   of nseq + 1 int64 offsets as for dsai_score_topk_packed.
 * Sequence i's rows and keys get exactly what dsai_indexer_backward gives
 * the sequence alone (a sequence with no rows gets zero grad_k on its keys,
 * one with no keys zero grad_q / grad_weights).  One dsai_indexer_backward
 * per sequence, in order on `stream`, all sharing `workspace`, which must
 * hold dsai_backward_packed_workspace_size bytes (the largest sequence's
 * need; 256-byte aligned).  Offsets as for dsai_score_topk_packed, topk and
 * compress_ratio as for dsai_indexer_backward (DSAI_ERR_INVALID_ARG or
 * DSAI_ERR_NULLPTR otherwise); every refusal comes before the first
 * launch. */
int dsai_backward_packed_workspace_size(dsai_handle h, int64_t nseq, const int64_t* cu_seqlens_q,
                                        const int64_t* cu_seqlens_k, int topk,
                                        int compress_ratio, size_t* bytes);
int dsai_indexer_backward_packed(dsai_handle h, const void* index_q, const void* index_k,
                                 const float* weights, const int32_t* topk_indices,
                                 const float* grad_scores, int64_t nseq,
                                 const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_k,
                                 int compress_ratio, int topk, void* grad_q, void* grad_k,
                                 float* grad_weights, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* ---- pooled decode pipeline ("Module glm5next_dsa") -------------------- */
/* P = floor(max(0, N - first_key) / kpool): the number of pools of a cache
 * of N tokens (pooling starts at first_key; a trailing partial pool is not a
 * pool).  Host-only. */
int dsai_pool_count(dsai_handle h, int64_t N, int64_t* P);

/* kpool_compress: pool p covers tokens first_key + p*KP + j, j < KP.
 *   k_normed  [N, D] bf16, gate [N, D] fp32, valid [N] uint8 (0 = invalid),
 *   ape       [KP, D] fp32
 *   pool_k    [P, D] bf16 written: per channel c, softmax over the slots j
 *             of (gate[tok_j,c] + ape[j,c]) weighting k_normed[tok_j,c],
 *             computed in fp32 and rounded to bf16 (nearest even)
 *   pool_tok  [P] int32 written: first token of the pool
 *   pool_valid[P] uint8 written: 1 iff every slot's token is valid
 * N >= 0; nothing is launched when P == 0. */
int dsai_kpool_compress(dsai_handle h, const void* k_normed, const float* gate,
                        const uint8_t* valid, const float* ape, int64_t N,
                        void* pool_k, int32_t* pool_tok, uint8_t* pool_valid,
                        void* stream);

/* index_scores: [Q, P] fp32 scores of decode queries against pool keys.
 *   q [Q, H, D] bf16, w [Q, H] fp32, pool_k [P, D] bf16, pool_valid [P] uint8
 *   scores[q, p] = sum_h w[q,h] * max(0, q[q,h,:] . pool_k[p,:]) if
 *   pool_valid[p], else -inf (an invalid candidate).  No causal mask.
 *   pool_limit: NULL (every row sees every pool) or [Q] int32 device array,
 *   4-byte aligned: row q's pools p >= pool_limit[q] are invalid candidates
 *   for that row (-inf), e.g. the pools not wholly before a query of a
 *   multi-token decode step; a bound below 0 acts as 0, above P as P.
 *   (The page "Module glm5next_dsa" has index_scores return [Q, P] scores
 *   plus candidate validity; the per-row bound is this library's reading of
 *   validity for rows at different positions.)
 * Q, P >= 0; P < 2^31. */
int dsai_index_scores(dsai_handle h, const void* q, const float* w, const void* pool_k,
                      const uint8_t* pool_valid, const int32_t* pool_limit, int64_t Q, int64_t P,
                      float* scores, void* stream);

/* topk_pools: per row of scores [Q, P] (from dsai_index_scores), the
 * select_k = index_topk / kpool pools with the largest finite scores, by
 * score descending and the lower pool id first among equal scores; -inf
 * marks an invalid pool, which is never selected.  Rows with fewer valid
 * pools are padded with id -1 / score -inf.
 *   pool_ids [Q, select_k] int32 written, pool_scores [Q, select_k] fp32 written. */
int dsai_topk_pools(dsai_handle h, const float* scores, int64_t Q, int64_t P,
                    int32_t* pool_ids, float* pool_scores, void* stream);

/* Bytes of workspace dsai_select needs for Q rows and P pools (the [Q, P]
 * fp32 score matrix).  Host-only. */
int dsai_select_workspace_size(dsai_handle h, int64_t Q, int64_t P, size_t* bytes);

/* dsai_index_scores (with its optional per-row pool_limit) followed by
 * dsai_topk_pools on one stream, with the [Q, P] scores held in the caller's
 * `workspace` (at least
 * dsai_select_workspace_size bytes, 256-byte aligned; DSAI_ERR_WORKSPACE
 * otherwise).  The workspace is free again once the stream passes the call. */
int dsai_select(dsai_handle h, const void* q, const float* w, const void* pool_k,
                const uint8_t* pool_valid, const int32_t* pool_limit, int64_t Q, int64_t P,
                int32_t* pool_ids, float* pool_scores, void* workspace, size_t workspace_bytes,
                void* stream);

/* expand_selection: pool ids [Q, select_k] int32 (each -1 or a pool id in
 * [0, P)) -> token ids [Q, index_topk] int32 (index_topk = select_k *
 * kpool).  Slot i*kpool + j receives first_key + pool_ids[q,i]*kpool + j,
 * or -1 when pool_ids[q,i] is negative; every slot is written exactly once.
 * Token ids are int32: an id above (2^31 - 1 - first_key + 1) / kpool - 1,
 * whose token ids would not fit, is written as missing (-1) like a negative
 * one (ids of a cache of N <= 2^31 - 1 tokens never are).  Q >= 0. */
int dsai_expand(dsai_handle h, const int32_t* pool_ids, int64_t Q, int32_t* tokens,
                void* stream);

/* dsai_select followed by dsai_expand of its pool ids, in one call: the same
 * pool_ids, pool_scores and tokens [Q, index_topk] int32 (16-byte aligned,
 * DSAI_ERR_INVALID_ARG otherwise), with the same workspace.  The pools' token
 * ids must fit int32: first_key + P * kpool - 1 <= 2^31 - 1
 * (DSAI_ERR_INVALID_ARG otherwise).  Where the
 * selection's rows are final when its kernel ends (P <= 32768, and in score
 * order select_k <= 512), that kernel writes the token ids too, with no
 * separate expand launch (the "Shape of the pipeline" of "Module glm5next_dsa"
 * runs topk_pools then expand_selection; their outputs are unchanged).
 * Every refusal (including DSAI_ERR_UNSUPPORTED for a select_k the
 * selection cannot hold) comes before the first launch. */
int dsai_select_expand(dsai_handle h, const void* q, const float* w, const void* pool_k,
                       const uint8_t* pool_valid, const int32_t* pool_limit, int64_t Q,
                       int64_t P, int32_t* pool_ids, float* pool_scores, int32_t* tokens,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the static device array dsai_select_expand_static keeps its
 * [Q, P] scores in (one array per device). */
#define DSAI_STATIC_SCRATCH_BYTES (16u << 20)

/* For callers that cannot allocate device memory (work recorded under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * dsai_select_expand with no workspace argument.  The [Q, P] fp32 scores
 * live in a static device array of DSAI_STATIC_SCRATCH_BYTES that the
 * library holds on each device it runs on until the process ends; its
 * address is looked up at the first call on a device (with that device
 * current).  The call allocates nothing (no hipMalloc / hipFree) and clears
 * nothing: index_scores writes every score before topk_pools reads it.
 * Outputs, argument rules and errors as dsai_select_expand, plus
 * DSAI_ERR_WORKSPACE when Q * P * 4 > DSAI_STATIC_SCRATCH_BYTES (before any
 * HIP call).  Every call on a device shares that device's array: calls that
 * overlap on one device (other streams, other handles, other host threads)
 * race on it and must be ordered by the caller. */
int dsai_select_expand_static(dsai_handle h, const void* q, const float* w, const void* pool_k,
                              const uint8_t* pool_valid, const int32_t* pool_limit, int64_t Q,
                              int64_t P, int32_t* pool_ids, float* pool_scores, int32_t* tokens,
                              void* stream);

/* ---- cache write: the indexer's k_norm ------------------------------------ */
/* k_norm ("Module glm5next_dsa", "Checkpoint and kernel facts": indexer.k_norm
 * is a LayerNorm with a bias; Constants: the BF16 LayerNorm module): the
 * producer of the k_normed rows kpool_compress reads.  Per row n of N:
 *   mean = sum_c x[n,c] / D,  var = sum_c (x[n,c] - mean)^2 / D   (biased)
 *   k_normed[n,c] = bf16( (x[n,c] - mean) / sqrt(var + eps) * gamma[c] + beta[c] )
 * computed in fp32, rounded to nearest even.
 *   k_raw [N, D] bf16, gamma [D] bf16, beta [D] bf16, k_normed [N, D] bf16
 *   written (e.g. the cache rows the new tokens occupy; it may be k_raw
 *   itself).  D = cfg.dim.  All device memory, 16-byte aligned
 *   (DSAI_ERR_INVALID_ARG otherwise).  N >= 0 (0: nothing launched);
 *   eps > 0 and finite (DSAI_ERR_INVALID_ARG otherwise). */
int dsai_k_norm(dsai_handle h, const void* k_raw, const void* gamma, const void* beta, float eps,
                int64_t N, void* k_normed, void* stream);

/* ---- row order ----------------------------------------------------------- */
/* Reorder `rows` top-k rows of k (index, score) entries in place, row r at
 * idx[r * k .. r * k + k) / score[r * k .. r * k + k): by score descending,
 * the lower index first among equal scores, entries with a negative index
 * last as (-1, -inf).  This is the step that turns a DSAI_ORDER_INDEX result
 * of dsai_score_topk or dsai_topk_pools into the DSAI_ORDER_SCORE result
 * (those calls run it themselves under DSAI_ORDER_SCORE); the real entries of
 * each row must be listed in ascending index order, as DSAI_ORDER_INDEX
 * writes them (rows in another order get the same entries in score order,
 * equal scores in an unspecified order).  Scores are finite.
 * rows >= 0 (< 2^31), 1 <= k <= DSAI_MAX_TOPK (DSAI_ERR_INVALID_ARG
 * otherwise); nothing is launched when rows == 0 or k == 1. */
int dsai_sort_rows(dsai_handle h, int32_t* idx, float* score, int64_t rows, int k,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSAI_H_ */
