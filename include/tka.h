/*
 * tka.h - C ABI of the MI355X (gfx950) top-k sparse decode-attention library
 * (libtka.so).
 *
 * One decode step of top-k sparse attention, as the pages state it: for the
 * current query, score every cached position (or block of positions), keep
 * the k highest scores, then run exact softmax attention over the kept keys
 * and values only ("Sparse Attention in LLM Inference: Practical
 * Trade-Offs", "The Role of the Indexer" workflow; "Evolution of Sparse
 * Attention in Long-Context LLMs", section 2; the scoring variants are those
 * of "Sparse Attention Landscape", "Block Sparse Attention" and "Token Sparse
 * Attention").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every data pointer is caller-owned DEVICE memory. The library allocates
 *   and frees nothing; scratch comes from a caller workspace whose size the
 *   *_workspace_size calls report. Inputs are never written; outputs are
 *   overwritten in full. Outputs must not overlap inputs.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls
 *   only enqueue work; the library never synchronises. A device fault shows
 *   up at the caller's next synchronisation.
 * - All argument checks run on the host before any launch and need no GPU.
 *   A failed check returns its status and launches nothing;
 *   tka_last_error() then names the argument (per calling thread).
 * - Base pointers and row strides must be 16-byte aligned (128-bit loads);
 *   otherwise TKA_ERR_ALIGNMENT.
 * - Same inputs, shapes and device give bitwise-identical outputs; the fused
 *   topk_decode equals the three-call composition bitwise.
 * - Calls are stateless and reentrant; concurrent calls on different streams
 *   need distinct workspaces.
 *
 * Shapes (all contiguous unless a stride is given; element counts):
 *   q          [B, Hq, d]       in qkv_dtype
 *   K, V cache [B, Hkv, L, d]   in qkv_dtype, element strides kv_stride_b/h/l,
 *                               the d elements of a row contiguous
 *   out        [B, Hq, d]       fp32
 *   Query head h reads KV head h / (Hq / Hkv) (contiguous groups).
 */
#ifndef TKA_H
#define TKA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TKA_ABI_VERSION 3

typedef enum {
  TKA_OK = 0,
  TKA_ERR_INVALID_ARG = 1, /* bad shape, count, null pointer or overlap */
  TKA_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim, dtype, head grouping */
  TKA_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than required */
  TKA_ERR_ALIGNMENT = 4,   /* pointer or stride not 16-byte aligned */
  TKA_ERR_HIP = 5          /* a HIP launch reported an error */
} tka_status;

typedef enum { TKA_F32 = 0, TKA_BF16 = 1, TKA_FP8_E4M3 = 2 /* OCP E4M3FN */ } tka_dtype;

typedef enum {
  /* s[b,h,i] = scale * <q[b,h], K[b,g(h),i]>, i < L; one kept set per (b, h).
     ("Sparse Attention Landscape", "Token Sparse Attention", s_i = f(q_t, k_i).) */
  TKA_SCORE_EXACT = 0,
  /* r[b,h,j] = <q[b,h], mean of K[b,g(h)] over block j>, j < m-1, m = ceil(L/b),
     no scale; keep the top-k blocks, then also attend the current block m-1.
     ("Sparse Attention Landscape", "Block Sparse Attention", MoBA mean-pooling.) */
  TKA_SCORE_BLOCK_MEAN = 1,
  /* I[b,i] = sum_j w[b,j] * max(0, <qI[b,j], kI[b,i]>), no scale; one kept set per
     sequence, shared by every head. ("Sparse Attention Landscape", "Token Sparse
     Attention", lightning indexer with query-dependent head weights.) */
  TKA_SCORE_INDEXER = 2,
  /* Two levels ("Sparse Attention Landscape", "Hierarchical Sparse Attention"):
     r[b,h,j] = <q[b,h], mean of K[b,g(h)] over block j> for every block j < m
     (no scale; the partial last block competes too), the top_blocks blocks
     kept; then the exact scores scale * <q, K_i> of their tokens only, the
     top_k tokens kept (topk_hisa_decode). */
  TKA_SCORE_HISA = 3
} tka_score_mode;

typedef struct {
  int32_t batch;      /* B >= 1 */
  int32_t n_q_heads;  /* Hq >= 1, a multiple of n_kv_heads */
  int32_t n_kv_heads; /* Hkv >= 1 */
  int32_t head_dim;   /* d: 64, 128 or 256 */
  int32_t seq_len;    /* L >= 1 cached keys; the query sits at position L-1 (no causal mask) */
  int32_t top_k;      /* k >= 1 tokens (EXACT, INDEXER) or blocks (BLOCK_MEAN); k' = min(k, candidates) */
  int64_t kv_stride_b, kv_stride_h, kv_stride_l; /* element strides of the K and V caches */
  tka_dtype qkv_dtype; /* TKA_F32 or TKA_BF16 (q, K, V) */
  float scale;         /* softmax logit scale; <= 0 selects 1/sqrt(d) */
  tka_score_mode mode;
  int32_t block_size;  /* BLOCK_MEAN: b >= 1 */
  int32_t n_idx_heads; /* INDEXER: H_I in [1, 128] */
  int32_t idx_dim;     /* INDEXER: d_I, a multiple of 64 up to 256 */
  tka_dtype idx_dtype; /* INDEXER: TKA_FP8_E4M3 */
  int32_t block_capacity; /* BLOCK_MEAN: block slots per (b, KV head) of the block-mean buffer, >= ceil(L/b),
                             so a buffer sized for the longest sequence serves every length; 0 = ceil(L/b) */
  int32_t idx_capacity;   /* INDEXER: positions per sequence of the indexer-key buffer, >= L (the same for the
                             indexer keys of every length); 0 = L */
  int32_t top_blocks;     /* HISA: K_B >= 1, the blocks kept by the coarse level (block_size, block_capacity
                             as for BLOCK_MEAN) */
  int32_t n_queries;      /* EXACT: M query tokens per sequence (0 or 1: one). With M > 1 the queries sit at
                             positions L-M .. L-1 of the cache and attend causally: query t sees keys
                             0 .. L-M+t and keeps min(k, L-M+t+1) of them ("Evolution of Sparse Attention in
                             Long-Context LLMs", section 6: current length x K). Then q and out are
                             [B,M,Hq,d], scores [B,M,Hq,L] (a position a query cannot see is NaN), index
                             lists [B,M,Hq,n]; built for bf16 with M * Hq/Hkv <= 64 (topk_attn_score,
                             sparse_attn_gather, topk_decode, and topk_attn_score_threshold for M <= 4;
                             TKA_ERR_UNSUPPORTED elsewhere). */
  int32_t decode_path;    /* topk_decode in EXACT mode: TKA_PATH_AUTO (0), TKA_PATH_PREFILTER or
                             TKA_PATH_DENSE; see topk_decode. The results are the same bits on every path. */
} tka_problem;

/* tka_problem.decode_path */
enum { TKA_PATH_AUTO = 0, TKA_PATH_PREFILTER = 1, TKA_PATH_DENSE = 2 };

/*
 * Scoring pass (one of the three variants above), writes fp32 scores.
 *   EXACT:      q [B,Hq,d]; keys = K cache; scores [B,Hq,L].
 *   BLOCK_MEAN: q [B,Hq,d]; keys = block means [B,Hkv,mc,d] fp32 contiguous (from
 *               topk_block_mean_build; mc = block_capacity, or m if 0); scores
 *               [B,Hq,m-1] (the current block does not compete). Nothing is
 *               written when m == 1.
 *   HISA:       q [B,Hq,d]; keys = block means as for BLOCK_MEAN; scores
 *               [B,Hq,m]: the coarse score of every block.
 *   INDEXER:    q = qI [B,H_I,d_I] E4M3FN; keys = kI [B,Lc,d_I] E4M3FN (Lc =
 *               idx_capacity, or L if 0; positions >= L unread);
 *               idx_w [B,H_I] fp32; scores [B,L].
 * idx_w must be NULL unless mode is INDEXER.
 */
tka_status topk_attn_score(const tka_problem* p, const void* q, const void* keys, const float* idx_w,
                           float* scores, void* stream);

/*
 * Thresholded scoring pass: scores every cached key as topk_attn_score does
 * (EXACT, bytewise the same fp32 values) and keeps, per row r = b*Hq + h, the
 * (score, position) pairs that rank at or above thresholds[r] in the
 * topk_select order (so a score equal to the threshold is kept). Any
 * threshold not above the row's k-th largest score keeps all of the row's k
 * largest ("Sparse Attention in LLM Inference", "The Role of the Indexer":
 * only a small candidate set goes on to the exact computation).
 * Append semantics: pairs found for row r are written to
 * cand_scores/cand_pos [r*capacity + counts[r] ...] in no particular order
 * and counts[r] is increased by their number; pairs that would land at or
 * beyond capacity are counted but not stored. Needs bf16 caches and
 * 2 <= Hq/Hkv <= 16 (TKA_ERR_UNSUPPORTED otherwise).
 * Several queries (n_queries = M, 2 <= M <= 4): q is [B,M,Hq,d] and rows are
 * r = (b*M + t)*Hq + h (thresholds, counts and lists [B*M*Hq, capacity]);
 * query t keeps only positions 0 .. L-M+t it can see.
 * A NaN threshold keeps every position the row can see.
 */
tka_status topk_attn_score_threshold(const tka_problem* p, const void* q, const void* k_cache,
                                     const float* thresholds, uint32_t* counts, float* cand_scores, int32_t* cand_pos,
                                     int32_t capacity, void* stream);

/*
 * Exact top-k of each score row ("Sparse Attention Landscape", "Block Sparse
 * Attention", the TopK_j s_j operator). Order: i before j when s_i > s_j, or
 * s_i == s_j and i < j; -0 equals +0; NaN ranks below every number. Row r
 * holds row_len fp32 values at scores + r*row_stride.
 *   idx_out       [n_rows, k] int32: the k' = min(k, row_len) kept positions in
 *                 ascending order, then -1 up to k.
 *   sel_scores_out [n_rows, k] fp32 or NULL: the kept scores aligned with idx_out
 *                 (bit patterns copied), -inf in padded slots.
 * ws/ws_bytes: scratch of at least topk_select_workspace_size bytes.
 * Fewer than 128 rows longer than 16384 are split over workgroups; such rows
 * may hold at most about 12 million values (TKA_ERR_UNSUPPORTED beyond; the
 * same bound applies to the rows that topk_decode and topk_hisa_decode select).
 */
tka_status topk_select(const float* scores, int64_t n_rows, int32_t row_len, int64_t row_stride, int32_t k,
                       int32_t* idx_out, float* sel_scores_out, void* ws, size_t ws_bytes, void* stream);

tka_status topk_select_workspace_size(int64_t n_rows, int32_t row_len, int32_t k, size_t* bytes);

/*
 * Certified adaptive top-k ("A Mathematical Theory of Top-k Sparse Attention
 * via Total Variation Distance", abstract: the total-variation distance
 * between a softmax P and its top-k truncation equals the softmax mass the
 * truncation discards). Each row of n = row_len fp32 logits s (P_i ~ exp s_i)
 * keeps the smallest k whose top-k, in the topk_select order, holds at least
 * 1 - eps of the mass, clamped to [max(k_min, 1), min(k_max, n)] (a row with
 * no mass keeps max(k_min, 1)).
 *   idx_out        [n_rows, k_max] int32: the kept positions ascending, then -1.
 *   k_out          [n_rows] int32: the kept count k.
 *   tau_out        [n_rows] fp32: the discarded mass of the kept set over the
 *                  row total (the certified TV distance; <= eps unless k_max
 *                  or k_min bound k); NaN for a row with no mass.
 *   sel_scores_out [n_rows, k_max] fp32 or NULL, as topk_select.
 * Masses are exp(s_i - max s) in fp32 (an element equal to the maximum has
 * mass 1, NaN has none) summed in 2^-40 fixed point, so k and tau do not
 * depend on the order of the parallel sums. eps must be finite and >= 0.
 * ws/ws_bytes: scratch of at least topk_select_adaptive_workspace_size bytes.
 */
tka_status topk_select_adaptive(const float* scores, int64_t n_rows, int32_t row_len, int64_t row_stride, float eps,
                                int32_t k_min, int32_t k_max, int32_t* idx_out, int32_t* k_out, float* tau_out,
                                float* sel_scores_out, void* ws, size_t ws_bytes, void* stream);

tka_status topk_select_adaptive_workspace_size(int64_t n_rows, int32_t row_len, int32_t k_max, size_t* bytes);

/*
 * Exact softmax attention over kept positions only ("Sparse Attention in LLM
 * Inference", "Changes in Caching Strategy": batch reads of the KV cache
 * through a position index built from the Top-K result; "Computational and
 * Memory Access Benefits": O(K d) work per query).
 *   idx: [B,Hq,n_idx] lists (one per query head) or, with
 *        shared_across_heads != 0, [B,n_idx] lists used by every head of b.
 *   idx_unit: 0 -> entries are token positions; b >= 1 -> entries are block ids
 *        covering [j b, min((j+1) b, L)) and the current block ceil(L/b)-1 is
 *        attended as well (ids outside [0, ceil(L/b)-1) are skipped).
 *        Entries < 0 or >= L (tokens) are skipped.
 *   sel_scores: NULL, or (idx_unit 0, per-head lists only) the logits of the
 *        listed tokens aligned with idx, i.e. scale*<q,K_i> as written by
 *        topk_attn_score (EXACT) and topk_select; K rows are then not re-read.
 *   out: [B,Hq,d] fp32, o = sum_i e^(z_i - M) V_i / sum_i e^(z_i - M) with
 *        z_i = scale*<q, K_i>; a row with no valid entry is written as zeros.
 */
tka_status sparse_attn_gather(const tka_problem* p, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* idx, int32_t n_idx, int32_t idx_unit, int32_t shared_across_heads,
                              const float* sel_scores, float* out, void* ws, size_t ws_bytes, void* stream);

tka_status sparse_attn_gather_workspace_size(const tka_problem* p, int32_t n_idx, int32_t idx_unit,
                                             int32_t shared_across_heads, size_t* bytes);

/*
 * The whole step in one call, on one stream: score -> select -> gather, with
 * results bitwise equal to the three calls above.
 *   EXACT bf16 with 2 <= Hq/Hkv <= 16, 8192 <= L <= 262144, k' <= L/8 and
 *   n_queries <= 4 can run the candidate prefilter instead of writing the score
 *   array: sampled thresholds, one thresholded scan, an exact select over the
 *   candidates, a full rescore of any row whose candidates cannot hold the answer
 *   ("Sparse Attention in LLM Inference", "The Overhead of the Indexer": filter
 *   coarsely, then sort finely among the survivors). decode_path TKA_PATH_AUTO
 *   takes it when B * n_queries * Hq * L >= 2^22 scores (below that its six
 *   launches cost more than the score array saves), TKA_PATH_PREFILTER whenever
 *   it applies, TKA_PATH_DENSE never; any other value is TKA_ERR_INVALID_ARG.
 *   EXACT:      proxy_keys, q_idx, idx_w NULL; the gather uses the selected scores.
 *   BLOCK_MEAN: proxy_keys = block means [B,Hkv,mc,d] fp32; idx_out (if given)
 *               [B,Hq,k] block ids without the current block.
 *   INDEXER:    proxy_keys = kI [B,Lc,d_I], q_idx = qI [B,H_I,d_I], idx_w [B,H_I];
 *               idx_out (if given) [B,k].
 * idx_out may be NULL (the indices then live in the workspace).
 */
tka_status topk_decode(const tka_problem* p, const void* q, const void* k_cache, const void* v_cache,
                       const void* proxy_keys, const void* q_idx, const float* idx_w, float* out,
                       int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

tka_status topk_decode_workspace_size(const tka_problem* p, size_t* bytes);

/*
 * topk_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. The
 * same checks, kernels and results (bitwise) as topk_decode, without the
 * workspace argument: the scratch is a device array inside the library,
 * TKA_NOALLOC_SCRATCH_BYTES per GPU, set up on the first call on each device
 * (with that device current) and held until the process ends. Nothing is
 * allocated or freed by the call itself. A problem whose topk_decode workspace
 * (topk_decode_workspace_size) exceeds that size returns TKA_ERR_UNSUPPORTED
 * and launches nothing. Every call on a GPU uses that GPU's one array (its
 * contents are whatever the last call left; the step needs nothing zeroed in
 * advance): calls that may overlap in time on one GPU (different streams or
 * host threads without ordering between them) race and must not be made.
 */
#define TKA_NOALLOC_SCRATCH_BYTES (256u << 20)
tka_status topk_decode_noalloc(const tka_problem* p, const void* q, const void* k_cache, const void* v_cache,
                               const void* proxy_keys, const void* q_idx, const float* idx_w, float* out,
                               int32_t* idx_out, void* stream);

/*
 * The certified step (TKA_SCORE_EXACT only): full exact scores, the adaptive
 * k of topk_select_adaptive with k_max = p->top_k, then the gather over the
 * kept positions with their scores as logits. Same kernels as
 * topk_attn_score -> topk_select_adaptive -> sparse_attn_gather (bitwise
 * equal results).
 *   out [B,Hq,d] fp32; idx_out [B,Hq,top_k] (or NULL), k_out [B,Hq] (or NULL),
 *   tau_out [B,Hq] (or NULL): as topk_select_adaptive.
 */
tka_status topk_decode_adaptive(const tka_problem* p, const void* q, const void* k_cache, const void* v_cache,
                                float eps, int32_t k_min, float* out, int32_t* idx_out, int32_t* k_out,
                                float* tau_out, void* ws, size_t ws_bytes, void* stream);

tka_status topk_decode_adaptive_workspace_size(const tka_problem* p, size_t* bytes);

/*
 * The two-level step (mode TKA_SCORE_HISA; "Sparse Attention Landscape",
 * "Hierarchical Sparse Attention": the fine scores run only over the tokens
 * of the top_blocks blocks with the best coarse scores, about K_B b of them
 * instead of L). Coarse scores of every block from the block means, the top
 * K_B blocks (select order), the exact scores of their tokens, the top
 * k' = min(top_k, their token count) tokens (select order, ties to the lower
 * position), attention over those with their exact scores as logits.
 *   means [B,Hkv,mc,d] fp32 from topk_block_mean_build (mode HISA or
 *     BLOCK_MEAN layout).
 *   out [B,Hq,d] fp32; idx_out [B,Hq,top_k] token positions ascending, -1
 *     after k' (or NULL).
 *   Optional (NULL: kept in the workspace): blk_out [B,Hq,K_B] the kept
 *     blocks ascending, -1 padded; block_scores_out [B,Hq,m] the coarse
 *     scores; cand_scores_out [B,Hq,K_B*b]: entry j*b+i is the exact score of
 *     token blk[j]*b+i, NaN where that is no token (blk[j] = -1 or past L).
 */
tka_status topk_hisa_decode(const tka_problem* p, const void* q, const void* k_cache, const void* v_cache,
                            const float* means, float* out, int32_t* idx_out, int32_t* blk_out,
                            float* block_scores_out, float* cand_scores_out, void* ws, size_t ws_bytes,
                            void* stream);

tka_status topk_hisa_decode_workspace_size(const tka_problem* p, size_t* bytes);

/*
 * Block-mean key cache for BLOCK_MEAN ("Sparse Attention Landscape", "Block
 * Sparse Attention": MoBA mean-pools the keys of each block): means[b,g,j,:] =
 * (1/n_j) sum over the n_j keys of block j of K[b,g,i,:], fp32, [B,Hkv,mc,d]
 * contiguous (mc = block_capacity, or m = ceil(L/b) if 0), blocks j < m
 * written (the last block may be partial; slots j >= m are left as they are).
 * Built once, off the decode step; topk_cache_append keeps it current.
 */
tka_status topk_block_mean_build(const tka_problem* p, const void* k_cache, float* means, void* stream);

/*
 * Append one decode step to the caches ("Sparse Attention in LLM Inference",
 * "Changes in Caching Strategy": the sparse layer reads its cache through a
 * position index, so the caches hold one row per position). p->seq_len = L is
 * the length after the append; the new token goes to position L-1. Any group
 * below may be skipped by passing NULL for all of its pointers.
 *   k_new, v_new [B,Hkv,d] in qkv_dtype, contiguous: to row L-1 of every
 *     (b, KV head) of k_cache / v_cache (strides from p).
 *   means (BLOCK_MEAN only) [B,Hkv,mc,d] fp32 (as topk_block_mean_build): the mean of block
 *     (L-1)/b is recomputed from k_cache after the append, bitwise what
 *     topk_block_mean_build writes for length L ("Sparse Attention Landscape",
 *     "Block Sparse Attention": MoBA mean-pools each block's keys).
 *   kI_new (INDEXER only) [B,d_I] fp32 -> kI_cache [B,Lc,d_I] row L-1 as OCP
 *     E4M3FN: nearest code, ties to even, |x| >= 448 saturates to 448, NaN ->
 *     0x7f (the low-dimensional indexer keys of "Sparse Attention Landscape",
 *     "Token Sparse Attention").
 */
tka_status topk_cache_append(const tka_problem* p, const void* k_new, const void* v_new, void* k_cache,
                             void* v_cache, const float* kI_new, void* kI_cache, float* means, void* stream);

/*
 * One workspace query for the steps of a problem (the per-call queries above
 * give the same numbers):
 *   which = TKA_WS_SELECT:  topk_select over the problem's score rows (B*Hq rows
 *                           of L, or of m-1 blocks; B rows of L for INDEXER), k = top_k;
 *   which = TKA_WS_GATHER:  sparse_attn_gather with top_k entries per list, in the
 *                           problem's unit (tokens, or blocks for BLOCK_MEAN) and
 *                           sharing (one list per sequence for INDEXER);
 *   which = TKA_WS_DECODE:  topk_decode (topk_hisa_decode for mode HISA);
 *   which = TKA_WS_DECODE_ADAPTIVE: topk_decode_adaptive.
 * Any other value of which: TKA_ERR_INVALID_ARG.
 */
enum { TKA_WS_SELECT = 0, TKA_WS_GATHER = 1, TKA_WS_DECODE = 2, TKA_WS_DECODE_ADAPTIVE = 3 };
tka_status topk_workspace_size(const tka_problem* p, int32_t which, size_t* bytes);

const char* tka_status_str(tka_status s);
/* detail of the last failed argument check in the calling thread ("" if none) */
const char* tka_last_error(void);
int32_t tka_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TKA_H */
