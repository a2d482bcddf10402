/*
 * msa.h — C ABI of libmsa.so, the MI355X (gfx950) implementation of the
 * MiniMax Sparse Attention (MSA) hot path over grouped-query attention.
 *
 * Sources (web pages; cited by title and section):
 *   [M3-evo]  "MiniMax 模型迭代与竞品分析：从 Text-01、M1、M2 到 M3", §2
 *             "从 Lightning Attention 到 MSA": the softmax-attention equation,
 *             GQA head sharing, and the four inference steps of MSA
 *             (global index scoring, 128-token block max-pooling, 16 blocks
 *             per query and GQA group with the local block counted among the
 *             16, exact softmax over at most 16x128 = 2048 tokens).
 *   [M-line]  "MiniMax：Text-01 / M1 → M2.7 → M3，注意力选择如何与 Agent RL、
 *             KV 和内核一起演进", §5: the Index Branch scores KV blocks per GQA
 *             group and picks Top-k; the Main Branch attends over the picked
 *             blocks only.
 *   [FA3-M3]  "前沿架构解码手记（三）：MiniMax M2.7 → M3——稀疏注意力的跨越",
 *             §2.1 "KV-Block-Major Prefill": the KV cache is nested
 *             block -> token -> head -> dim so that the tokens of one block
 *             are contiguous and a selected block is read as one large piece.
 *   [M2-rep]  "深度解读：The MiniMax-M2 Series", §2: 48 query heads and 8 KV
 *             heads (GQA 6:1).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every array argument is a DEVICE pointer unless its name ends in _host.
 *   Device pointers must be 16-byte aligned.
 * - bf16 means IEEE-754 binary32 truncated to its upper 16 bits (bfloat16),
 *   stored as 2-byte little-endian words.
 * - Every call only validates its arguments on the host and enqueues kernels
 *   on `stream` (a hipStream_t; NULL = the default stream).  It never
 *   synchronises, never allocates device or pinned memory, and keeps no
 *   state between calls; scratch memory is a caller-owned workspace.  The
 *   caller owns every buffer and keeps it alive until the stream has drained.
 * - Errors are return codes; the library never aborts and never prints.
 *   Every check listed under "Errors" runs on the host before the first HIP
 *   call, so a rejected call has enqueued nothing.  msa_last_error() returns
 *   a thread-local human-readable detail of the last failure.
 * - Per-token device metadata (block_table entries, the device copies of
 *   seq_lens and cu_q) cannot be read by the host without a synchronisation;
 *   it is a precondition that seq_lens and cu_q equal their host mirrors.
 *   A block_table entry outside [0, num_blocks) is never dereferenced: the
 *   logical block it names holds no keys.  msa_index_score gives such a
 *   block the pooled score -inf (the max over no keys), so msa_block_topk
 *   picks it only as the forced local block or when fewer than top_k - 1
 *   earlier blocks hold keys; every attention call skips it; and a row whose
 *   selected blocks all hold no keys gets output 0.
 *
 * Positions, blocks and groups
 * ----------------------------
 * - Sequence s holds seq_lens[s] tokens (after this step's append).  Its
 *   queries are its LAST nq_s = cu_q[s+1] - cu_q[s] positions, so query row
 *   r = cu_q[s] + i sits at absolute position t = seq_lens[s] - nq_s + i.
 *   Prefill of a fresh sequence has nq_s = seq_lens[s]; decode has nq_s = 1;
 *   a prefill chunk onto an existing cache has 1 <= nq_s < seq_lens[s].
 *   The new token attends to itself (it is appended before attention).
 * - Logical block b of a sequence holds absolute positions [128b, 128b+127];
 *   block_table[s][b] names its physical block in the cache.
 * - The current ("local") block of a query at position t is c = t / 128.
 * - Query head h belongs to GQA group g = h / (num_q_heads / num_kv_heads),
 *   and group g reads KV head g.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_ABI_VERSION 3

typedef enum msa_status {
  MSA_OK = 0,
  MSA_ERR_NULL_POINTER = 1, /* a required pointer (struct, array, host mirror) is NULL */
  MSA_ERR_BAD_SHAPE = 2,    /* inconsistent sizes: Hq % Hkv != 0, cu_q not monotone,
                               nq_s > seq_lens[s], ld too small, negative counts */
  MSA_ERR_UNSUPPORTED = 3,  /* a size outside the compiled specialisations: head_dim
                               not in {64,128}, index_dim not in {32,64}, block_size
                               != 128, top_k != 16, num_kv_heads not a power of two
                               in [1,32], group size Hq/Hkv > 16 */
  MSA_ERR_MISALIGNED = 4,   /* a device pointer is not 16-byte aligned */
  MSA_ERR_CAPACITY = 5,     /* seq_lens[s] > max_blocks_per_seq * 128, or a size that
                               overflows the 32-bit indexing the kernels use */
  MSA_ERR_WORKSPACE = 6,    /* workspace NULL or ws_bytes < msa_workspace_size(...) */
  MSA_ERR_HIP = 7           /* a HIP launch failed; detail in msa_last_error() */
} msa_status;

/* Head and block geometry.  softmax_scale <= 0 selects 1/sqrt(head_dim), the
 * scale of the softmax-attention equation in [M3-evo] §2. */
typedef struct msa_dims {
  int32_t num_q_heads;   /* Hq */
  int32_t num_kv_heads;  /* Hkv = number of GQA groups */
  int32_t head_dim;      /* D: 64 or 128 */
  int32_t index_dim;     /* d_idx: width of Q_idx / K_idx, 32 or 64 */
  int32_t block_size;    /* tokens per KV block: must be 128 ([M3-evo] §2) */
  int32_t top_k;         /* blocks kept per query and group: must be 16 ([M3-evo] §2) */
  float softmax_scale;
} msa_dims;

/* Block-major paged KV cache ([FA3-M3] §2.1).  One physical block holds 128
 * consecutive tokens; inside it the tokens are contiguous, each token holding
 * all KV heads, each head holding head_dim values.  K and V are separate
 * arrays with the same nesting.  The index keys K_idx (one per token, shared
 * by every group: [M3-evo] §2) live in a third array with the same block
 * paging. */
typedef struct msa_cache {
  void* k;                    /* bf16 [num_blocks][128][Hkv][D] */
  void* v;                    /* bf16 [num_blocks][128][Hkv][D] */
  void* k_idx;                /* bf16 [num_blocks][128][d_idx]  */
  const int32_t* block_table; /* int32 [num_seqs][max_blocks_per_seq], logical -> physical */
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
} msa_cache;

/* A batch of sequences and the query rows this step computes. */
typedef struct msa_batch {
  int32_t num_seqs;
  int32_t total_q;               /* = cu_q[num_seqs] */
  const int32_t* seq_lens;       /* device int32 [num_seqs]: length after the append */
  const int32_t* cu_q;           /* device int32 [num_seqs+1]: row offsets, cu_q[0] = 0 */
  const int32_t* seq_lens_host;  /* host mirror of seq_lens (validation, grid sizing) */
  const int32_t* cu_q_host;      /* host mirror of cu_q */
} msa_batch;

/* Which call msa_workspace_size() sizes. */
typedef enum msa_call {
  MSA_CALL_SPARSE_ATTN_PREFILL = 1,
  MSA_CALL_SPARSE_ATTN_DECODE = 2,
  MSA_CALL_DENSE_ATTN_DECODE = 3,
  MSA_CALL_INDEX_SELECT = 4,
  MSA_CALL_SPARSE_ATTN_PREFILL_PLAN = 5,  /* the plan buffer of msa_sparse_attn_prefill_plan */
  MSA_CALL_SPARSE_ATTN_PREFILL_RUN = 6,   /* the workspace of msa_sparse_attn_prefill_run */
  MSA_CALL_DECODE_STEP = 7                /* the workspace of msa_decode_step */
} msa_call;

/* ------------------------------------------------------------------------- *
 * msa_kv_append — store the keys and values of this step's new tokens.
 * Past K/V are cached for later queries and past queries are not ([M3-evo]
 * §2, Q/K/V paragraph); the cache is block-major ([FA3-M3] §2.1).
 *   k_new, v_new : bf16 [total_q][Hkv][D], row r = token at the position of
 *                  query row r (see "Positions" above).
 *   k_idx_new    : bf16 [total_q][d_idx], the index key of the same token.
 * Writes cache.k/v/k_idx at (block_table[s][t/128], t%128) for every new row.
 * Reads nothing else; other cache slots are left untouched.
 * Errors: NULL_POINTER, BAD_SHAPE, UNSUPPORTED, MISALIGNED, CAPACITY, HIP.
 * ------------------------------------------------------------------------- */
msa_status msa_kv_append(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch,
                         const void* k_new, const void* v_new, const void* k_idx_new,
                         void* stream);

/* ------------------------------------------------------------------------- *
 * msa_index_score — Index Branch scoring plus block max-pooling
 * ([M3-evo] §2 steps 1–2; [M-line] §5).  For query row r at position t, group
 * g and every causal block b <= c = t/128:
 *     s_i          = sum_d q_idx[r][g][d] * k_idx[i][d]      (0 <= i <= t)
 *     scores[r][g][b] = max { s_i : 128b <= i <= min(128b+127, t) }
 * computed as bf16 x bf16 products accumulated in fp32; -0.0 is written as
 * +0.0.  The score is a plain dot product (no scale, no activation): a
 * positive scale would not change any selection, and the pages name none.
 *   q_idx        : bf16 [total_q][Hkv][d_idx]
 *   block_scores : fp32 [total_q][Hkv][ld], ld >= max_s ceil(seq_lens[s]/128).
 *                  Entries b > c of a row are NOT written.
 * Errors: NULL_POINTER, BAD_SHAPE (ld too small), UNSUPPORTED, MISALIGNED,
 *         CAPACITY, HIP.
 * ------------------------------------------------------------------------- */
msa_status msa_index_score(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch,
                           const void* q_idx, float* block_scores, int64_t ld, void* stream);

/* ------------------------------------------------------------------------- *
 * msa_block_topk — block selection ([M3-evo] §2 step 3).  For row r, group g
 * with local block c = t/128:
 *   - if c + 1 <= top_k: sel = {0, 1, ..., c};
 *   - else sel = {c} plus the top_k - 1 best of blocks 0..c-1, ordered by
 *     (score descending, block index ascending), so equal scores go to the
 *     lower block index and the local block takes one of the top_k slots.
 * No exponential is evaluated: selection only compares scores.
 *   block_scores : fp32 [total_q][Hkv][ld] as written by msa_index_score
 *                  (only entries b < c are read).
 *   sel          : int32 [total_q][Hkv][top_k], logical block ids in
 *                  ascending order, padded with -1 after the last one.
 * Errors: NULL_POINTER, BAD_SHAPE, UNSUPPORTED, MISALIGNED, HIP.
 * ------------------------------------------------------------------------- */
msa_status msa_block_topk(const msa_dims* dims, const msa_batch* batch, const float* block_scores,
                          int64_t ld, int32_t* sel, void* stream);

/* ------------------------------------------------------------------------- *
 * msa_index_select — msa_index_score followed by msa_block_topk ([M3-evo] §2
 * steps 1–3) without handing the pooled scores to the caller: the batch is
 * cut into chunks of query rows (whole sequences, or row ranges of one long
 * sequence), and each chunk's pooled scores live in the workspace only
 * until its selection is made.  sel is identical to the two calls'.
 *   q_idx     : bf16 [total_q][Hkv][d_idx]
 *   sel       : int32 [total_q][Hkv][top_k], as msa_block_topk
 *   workspace : device scratch; it must hold 256 bytes plus the pooled
 *               scores of one query row (Hkv x the blocks of the longest
 *               sequence, fp32), and the rows per chunk are as many as it
 *               holds.  msa_workspace_size(..., MSA_CALL_INDEX_SELECT) gives
 *               a size that keeps a chunk's scores within about 192 MB (so
 *               they stay in the 256 MB Infinity Cache) or the whole batch if
 *               smaller.  Contents on entry are ignored.
 * Errors: NULL_POINTER, BAD_SHAPE, UNSUPPORTED, MISALIGNED, CAPACITY,
 *         WORKSPACE, HIP.
 * ------------------------------------------------------------------------- */
msa_status msa_index_select(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch,
                            const void* q_idx, int32_t* sel, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * msa_sparse_attn_prefill — Main Branch ([M3-evo] §2 step 4 and the
 * softmax-attention equation): for query row r at position t and head h of
 * group g,
 *     I  = union over b in sel[r][g] of [128b, min(128b+127, t)]
 *     z_i = softmax_scale * (q[r][h] . k[i][g]),  p = softmax(z over I)
 *     out[r][h] = sum_{i in I} p_i v[i][g]
 * in bf16 x bf16 -> fp32 arithmetic, output rounded to bf16.  Designed for
 * many query rows per sequence (blocks outer, queries inner).
 *   q    : bf16 [total_q][Hq][D]
 *   sel  : int32 [total_q][Hkv][top_k] as produced by msa_block_topk
 *   out  : bf16 [total_q][Hq][D]
 *   workspace : device scratch of at least
 *               msa_workspace_size(dims, cache, batch, MSA_CALL_SPARSE_ATTN_PREFILL)
 *               bytes; its contents on entry are ignored.
 * Errors: NULL_POINTER, BAD_SHAPE, UNSUPPORTED, MISALIGNED, CAPACITY,
 *         WORKSPACE, HIP.
 * ------------------------------------------------------------------------- */
msa_status msa_sparse_attn_prefill(const msa_dims* dims, const msa_cache* cache,
                                   const msa_batch* batch, const void* q, const int32_t* sel,
                                   void* out, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * msa_sparse_attn_prefill_plan / msa_sparse_attn_prefill_run — the same
 * Main Branch ([M3-evo] §2 step 4) in two calls, so that a caller can
 * prepare the next batch's plan on another stream while this batch attends.
 * Together they compute exactly what msa_sparse_attn_prefill computes (it is
 * plan followed by run).
 *   plan: inverts the selections into one list of (row, slot) entries per
 *         (sequence, group, block) in `plan`, a device buffer of at least
 *         msa_workspace_size(dims, cache, batch, MSA_CALL_SPARSE_ATTN_PREFILL_PLAN)
 *         bytes owned by the caller; its contents on entry are ignored.
 *   run:  attends every listed row to its block and merges the slots.  `plan`
 *         must hold the result of msa_sparse_attn_prefill_plan for the same
 *         dims, cache, batch and sel, unmodified since (run only reads it, so
 *         one plan serves any number of runs); with anything else the result
 *         is undefined.  `workspace` holds the partial outputs: at least
 *         msa_workspace_size(dims, cache, batch, MSA_CALL_SPARSE_ATTN_PREFILL_RUN)
 *         bytes, contents on entry ignored.  q, sel and out as in
 *         msa_sparse_attn_prefill.
 * Errors: NULL_POINTER, BAD_SHAPE, UNSUPPORTED, MISALIGNED, CAPACITY,
 *         WORKSPACE, HIP.
 * ------------------------------------------------------------------------- */
msa_status msa_sparse_attn_prefill_plan(const msa_dims* dims, const msa_cache* cache,
                                        const msa_batch* batch, const int32_t* sel,
                                        void* plan, size_t plan_bytes, void* stream);
msa_status msa_sparse_attn_prefill_run(const msa_dims* dims, const msa_cache* cache,
                                       const msa_batch* batch, const void* q, const int32_t* sel,
                                       const void* plan, void* out, void* workspace, size_t ws_bytes,
                                       void* stream);

/* ------------------------------------------------------------------------- *
 * msa_sparse_attn_decode — the same Main Branch computation for one query
 * row per sequence (cu_q[s+1] - cu_q[s] == 1 for every s; BAD_SHAPE
 * otherwise), split across the selected blocks and merged by log-sum-exp.
 * Arguments and errors as msa_sparse_attn_prefill, workspace sized with
 * MSA_CALL_SPARSE_ATTN_DECODE.
 * ------------------------------------------------------------------------- */
msa_status msa_sparse_attn_decode(const msa_dims* dims, const msa_cache* cache,
                                  const msa_batch* batch, const void* q, const int32_t* sel,
                                  void* out, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * msa_decode_step — one whole decode step of MSA ([M3-evo] §2, the four
 * inference steps, for one new token per sequence): the calls msa_kv_append,
 * msa_index_score, msa_block_topk and msa_sparse_attn_decode in sequence,
 * with the same arguments and the same results bit for bit (block_scores,
 * sel, out and the cache), in fewer kernels: the append of each sequence's
 * new token is fused into the K_idx scan, and for batches of fewer than 128
 * (sequence, group) pairs the block selection, the attention and the merge
 * of the 16 slots run as one kernel (the workgroup that finishes a row last
 * merges it; two kernels instead of five).  Larger batches run the top-k
 * and the attention after the fused scan (three kernels instead of four:
 * from 128 to 255 pairs two workgroups per pair, the second to finish
 * merging the two halves; from 256 on one workgroup per pair).  The
 * attention kernels and their arithmetic are those of
 * msa_sparse_attn_decode.  Fewer launches shorten a step whose work is one
 * HBM-bound scan followed by latency-bound tails.
 *   Requires cu_q[s+1] - cu_q[s] == 1 for every s (BAD_SHAPE otherwise).
 *   k_new, v_new, k_idx_new : as msa_kv_append
 *   q_idx                   : as msa_index_score
 *   q, sel, out             : as msa_sparse_attn_decode (sel is written)
 *   block_scores, ld        : as msa_index_score (written)
 *   workspace : device scratch of at least
 *               msa_workspace_size(dims, cache, batch, MSA_CALL_DECODE_STEP)
 *               bytes; contents on entry are ignored.
 * Errors: NULL_POINTER, BAD_SHAPE, UNSUPPORTED, MISALIGNED, CAPACITY,
 *         WORKSPACE, HIP.
 * ------------------------------------------------------------------------- */
msa_status msa_decode_step(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch,
                           const void* k_new, const void* v_new, const void* k_idx_new,
                           const void* q_idx, const void* q, float* block_scores, int64_t ld,
                           int32_t* sel, void* out, void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * msa_sparse_attn_decode_noalloc — msa_sparse_attn_decode without a caller
 * workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).  It
 * computes exactly what msa_sparse_attn_decode computes (same kernels, same
 * results bit for bit).  Its scratch memory is a static array inside the
 * library: about 8.2 MB per GPU, held from the first call on that GPU until
 * the process ends, enough for every decode batch (batches of 256 or more
 * (sequence, group) pairs need none, batches of 128 to 255 at most 4.3 MB;
 * smaller ones need msa_workspace_size(..., MSA_CALL_SPARSE_ATTN_DECODE)
 * bytes of it, at most the array's size).  The call allocates nothing and calls no allocating
 * routine.  Every call on one GPU shares that GPU's array: calls that overlap
 * in time on one GPU (on different streams, or from different threads without
 * ordering) race and may return wrong results; calls ordered on one stream are
 * safe.  The array keeps the last call's contents; no call relies on them.
 *   q, sel, out : as msa_sparse_attn_decode.
 * Errors: NULL_POINTER, BAD_SHAPE, UNSUPPORTED, MISALIGNED, CAPACITY,
 *         WORKSPACE (a batch that would need more scratch than the array
 *         holds), HIP.
 * ------------------------------------------------------------------------- */
msa_status msa_sparse_attn_decode_noalloc(const msa_dims* dims, const msa_cache* cache,
                                          const msa_batch* batch, const void* q, const int32_t* sel,
                                          void* out, void* stream);

/* ------------------------------------------------------------------------- *
 * msa_block_attn_mass — attention mass per block for a sample of query rows
 * ([M3-evo] §2: MSA is judged by how much of the attention its chosen blocks
 * cover, and in training the Main Branch forms a group-averaged importance
 * distribution P over the candidate blocks).  For sampled row k (query row
 * r = rows[k] at position t, local block c = t/128) and group g, with I the
 * token set:
 *     mass[k][g][b] = (1/G) * sum over the group's heads h of
 *                     sum over tokens i of block b in I of softmax_i(z_h),
 *     z_h,i = softmax_scale * (q[r][h] . k[i][g]), softmax over i in I,
 * for b = 0..c (entries b > c are not written).  fp32 arithmetic.
 *   sel == NULL : I = every causal token i <= t (the dense mass);
 *   sel != NULL : I = the tokens i <= t of the blocks in sel[r][g] (the Main
 *                 Branch's own softmax of msa_sparse_attn_prefill), so the
 *                 mass is P over the candidate blocks: it sums to 1 over the
 *                 selected blocks and is 0 on every other block b <= c.
 *   q    : bf16 [total_q][Hq][D] (the Main Branch queries)
 *   sel  : NULL, or int32 [total_q][Hkv][top_k] as from msa_block_topk
 *   rows : int32 [n_rows], query-row indices into the batch; a row outside
 *          [0, total_q) is skipped (its outputs are not written).
 *   mass : fp32 [n_rows][Hkv][ld], ld >= the blocks of the longest sequence.
 * Reads K of every block of I through the block table (twice: once for the
 * softmax statistics, once for the masses).  Meant for sampled rows: with
 * sel == NULL the work is that of dense attention without the values.
 * Errors: NULL_POINTER, BAD_SHAPE, UNSUPPORTED, MISALIGNED, CAPACITY, HIP.
 * ------------------------------------------------------------------------- */
msa_status msa_block_attn_mass(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch,
                               const void* q, const int32_t* sel, const int32_t* rows, int32_t n_rows,
                               float* mass, int64_t ld, void* stream);

/* ------------------------------------------------------------------------- *
 * msa_selection_quality — how well the selections of the sampled rows match
 * the attention, and the indexer's training target ([M3-evo] §2: MSA is
 * judged by selection recall and by the share of attention score the chosen
 * blocks cover; the indexer is trained by D_KL(P || Q), P the Main Branch's
 * group-averaged importance over the candidate blocks, Q the indexer's
 * distribution).  For sampled row k and group g, with c = t/128, S the
 * selected blocks (ids in 0..c), M the dense mass and P the candidate mass
 * (msa_block_attn_mass without and with sel):
 *   coverage = sum of M[b] over b in S;
 *   recall   = |S AND top| / |top|, top = the min(top_k, c+1) blocks of
 *              largest M (equal masses go to the lower block index);
 *   kl       = sum over b in S with P[b] > 0 of P[b] (ln P[b] - ln Q[b]),
 *              Q[b] = exp(score[b]) / sum over b' in S of exp(score[b']),
 *              the softmax of the pooled index scores over the same blocks.
 *   rows         : int32 [n_rows] as for msa_block_attn_mass
 *   mass         : fp32 [n_rows][Hkv][ld], the dense mass M
 *   sel_mass     : fp32 [n_rows][Hkv][ld], the candidate mass P
 *   block_scores : fp32 [total_q][Hkv][ld] from msa_index_score
 *   sel          : int32 [total_q][Hkv][top_k] from msa_block_topk
 *   quality      : fp32 [n_rows][Hkv][3] = (coverage, recall, kl)
 * Errors: NULL_POINTER, BAD_SHAPE, UNSUPPORTED, MISALIGNED, HIP.
 * ------------------------------------------------------------------------- */
msa_status msa_selection_quality(const msa_dims* dims, const msa_batch* batch, const int32_t* rows,
                                 int32_t n_rows, const float* mass, const float* sel_mass,
                                 const float* block_scores, const int32_t* sel, int64_t ld, float* quality,
                                 void* stream);

/* ------------------------------------------------------------------------- *
 * msa_dense_attn_prefill — dense causal attention over the same cache
 * ([M3-evo] §2, the softmax-attention equation; §2–§3: the layers and the
 * training warmup that keep full attention).  For query row r at position t
 * and head h of group g = h / (Hq/Hkv):
 *     z_i = softmax_scale * (q[r][h] . k[i][g])  for every i <= t,
 *     out[r][h] = sum_{i <= t} softmax(z)_i v[i][g]
 * i.e. msa_sparse_attn_prefill with every causal block selected.  bf16 x bf16
 * -> fp32 arithmetic, output rounded to bf16.  Blocks whose block-table
 * entry lies outside [0, num_blocks) hold no keys (skipped, as in the sparse
 * calls).  Designed for many query rows per sequence (query tiles of 128
 * rows); correct for any batch.
 *   q    : bf16 [total_q][Hq][D]
 *   out  : bf16 [total_q][Hq][D]
 * No workspace.
 * Errors: NULL_POINTER, BAD_SHAPE, UNSUPPORTED, MISALIGNED, CAPACITY, HIP.
 * ------------------------------------------------------------------------- */
msa_status msa_dense_attn_prefill(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch,
                                  const void* q, void* out, void* stream);

/* ------------------------------------------------------------------------- *
 * msa_dense_attn_decode — msa_dense_attn_prefill for one query row per
 * sequence (cu_q[s+1] - cu_q[s] == 1 for every s; BAD_SHAPE otherwise):
 * the context is split over workgroups of 64 blocks and the splits merged
 * by log-sum-exp.
 *   q, out    : as msa_dense_attn_prefill
 *   workspace : device scratch of at least
 *               msa_workspace_size(dims, cache, batch, MSA_CALL_DENSE_ATTN_DECODE)
 *               bytes; its contents on entry are ignored.
 * Errors: NULL_POINTER, BAD_SHAPE, UNSUPPORTED, MISALIGNED, CAPACITY,
 *         WORKSPACE, HIP.
 * ------------------------------------------------------------------------- */
msa_status msa_dense_attn_decode(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch,
                                 const void* q, void* out, void* workspace, size_t ws_bytes, void* stream);

/* Bytes of workspace `call` needs for this problem; 0 if the arguments are
 * invalid (the failing check is reported by msa_last_error()). */
size_t msa_workspace_size(const msa_dims* dims, const msa_cache* cache, const msa_batch* batch,
                          int32_t call);

/* Static text for a status code; never NULL. */
const char* msa_status_string(msa_status status);

/* Thread-local detail of the last failing call on this thread; "" if none. */
const char* msa_last_error(void);

/* MSA_ABI_VERSION of the library that is loaded. */
int32_t msa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
