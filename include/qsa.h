/*
 * qsa.h - C ABI of libqsa, the QSA (Qwen Sparse Attention) decode path on AMD gfx950.
 *
 * The method, as the article "Qwen 4 QSA gets decode context parallelism: inside vLLM's
 * draft PR for Qwen3.8-Flash-Next" (orcarouter.ai blog) describes it:
 *   - section "What the pull request actually changes", second paragraph: a light
 *     indexer pools the keys of every 4 consecutive tokens (a micro-block) and scores each pool; the 512
 *     best blocks (about 2,048 positions) are kept; the final softmax and the value
 *     aggregation use the full K and V rows of the kept tokens, not pooled ones.
 *   - same section, first paragraph and bullets, and section "Questions worth answering
 *     directly" (DCP versus TP): under DCP every rank scans one contiguous piece of a
 *     request's context, and the per-piece attention partials are joined in a second
 *     step. Here the P pieces (slices) of one request are read on one GPU and joined by
 *     log-sum-exp.
 *
 * One decode step of one QSA layer is the chain
 *     qsa_index_score -> qsa_topk_select -> qsa_sparse_attn_decode -> qsa_lse_merge
 * (or qsa_decode, which runs the four on one stream). The indexer's side cache of pooled keys
 * (qsa_pool_build, qsa_cache_append, qsa_index_score_pooled, qsa_decode_pooled,
 * qsa_decode_multi_pooled) gives the same chain with a scan that reads half the bytes.
 * Several new tokens per request (draft tokens of speculative decoding, prefill chunks) run
 * through qsa_decode_multi and qsa_index_score_multi, each token decoded at its own length.
 *
 * Conventions for every entry point
 *   Memory     every pointer is device memory of the current HIP device, unless noted.
 *              The caller owns every buffer. No call allocates device memory or keeps a
 *              pointer, view or handle of the caller's after it returns; the one memory of
 *              the library's own is the static scratch array of qsa_decode_noalloc (a
 *              device symbol of the code object, per device, from load to process end).
 *   Streams    `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue
 *              work and return; they never synchronize. Buffers must stay alive until the
 *              stream has passed the work. Inputs are read-only; outputs must not alias
 *              inputs.
 *   Layouts    row-major, densely packed, base pointers 16-byte aligned.
 *              indexer keys  idx_cache  [num_pages, page_size, n_idx_heads, idx_dim] int8
 *              keys, values  k_cache, v_cache [num_pages, page_size, Hkv, head_dim] bf16
 *              page table    page_table [B, max_pages_per_seq] int32 (physical page ids)
 *              lengths       context_lens [B] int32, 0 <= L_b <= max_pages_per_seq*page_size
 *              Token t of request b lives in page page_table[b][t / page_size], row
 *              t % page_size, in all three caches (one page table for the indexer keys
 *              and K/V, as the article's bullet on the single cache group has it).
 *   Compiled   page_size 64, n_idx_heads 4, idx_dim 64, head_dim 128, Hq/Hkv <= 16,
 *              k <= 512. Other values return QSA_ERR_UNSUPPORTED.
 *   Errors     arguments visible on the host are checked before anything is enqueued;
 *              a failing check returns its code and launches nothing. Launch failures
 *              return QSA_ERR_HIP (see qsa_last_hip_error). Device-side preconditions
 *              (page ids in range, lengths within the page table) are the caller's and
 *              are not checked by the compute calls; qsa_check_pages checks them on
 *              request. No C++ exception crosses this interface.
 *   Workspace  entry points that take a workspace need qsa_*_workspace_size() bytes,
 *              16-byte aligned; when that size is 0 the pointer may be NULL. A workspace
 *              carries intermediates from one kernel of a call to the next; every byte a
 *              kernel reads was written earlier in the same call, so a workspace needs no
 *              initialisation and keeps nothing between calls. Calls that share a
 *              workspace must not overlap in time.
 *   Threads    stateless and re-entrant apart from the thread-local qsa_last_hip_error and
 *              the thread-local request of qsa_time_next_scan.
 */
#ifndef QSA_H_
#define QSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QSA_OK = 0,
  QSA_ERR_NULL = 1,         /* a required pointer is NULL                          */
  QSA_ERR_SHAPE = 2,        /* sizes are negative or inconsistent                  */
  QSA_ERR_UNSUPPORTED = 3,  /* a size outside what the kernels are compiled for    */
  QSA_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required          */
  QSA_ERR_HIP = 5,          /* the HIP runtime reported an error                   */
  QSA_ERR_SCRATCH = 6       /* qsa_decode_noalloc: the call needs more than the
                               library's static scratch (QSA_NOALLOC_SCRATCH_BYTES)  */
} qsa_status_t;

/* Static description of a status code; never NULL. */
const char* qsa_status_string(int status);

/* hipError_t of the last HIP failure seen by this thread (0 if none). */
int qsa_last_hip_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int qsa_version(void);

/*
 * qsa_index_score - indexer scan, micro-block pooling and block scoring.
 *
 * Article, section "What the pull request actually changes", second paragraph: the
 * indexer pools the keys of every 4 consecutive tokens and scores each pool. With the
 * compiled shapes, for request b of length L_b and block j < ceil(L_b/4):
 *     pooled[j][h][d] = sum of idx key[t][h][d] over tokens t = 4j .. min(4j+3, L_b-1)
 *     block_scores[b][j] = sum_h sum_d q_idx[b][h][d] * pooled[j][h][d]      (exact)
 * The score always fits int32 (|S| <= 4*256*128*128 = 2^24).
 *
 *   q_idx        [B, n_idx_heads, idx_dim] int8   indexer query of the decode token
 *   idx_cache    paged indexer keys (see Layouts)
 *   page_table   [B, max_pages_per_seq] int32
 *   context_lens [B] int32
 *   max_blocks   row stride of block_scores; must be >= max_pages_per_seq*page_size/4
 *   block_scores out [B, max_blocks] int32; entries j >= ceil(L_b/4) are not written
 *   page_max     out [B, max_pages_per_seq] int32, or NULL: the largest block score of
 *                each page p < ceil(L_b/64) (a by-product for qsa_topk_select)
 * B == 0 is a no-op.
 */
qsa_status_t qsa_index_score(const int8_t* q_idx, const int8_t* idx_cache,
                             const int32_t* page_table, const int32_t* context_lens,
                             int B, int n_idx_heads, int idx_dim, int page_size,
                             int max_pages_per_seq, int max_blocks,
                             int32_t* block_scores, int32_t* page_max, void* stream);

/*
 * qsa_topk_select - keep the best k micro-blocks of each request.
 *
 * Article, same paragraph: the best 512 blocks are kept. For request b with
 * n_b = ceil(L_b/4) blocks, K_b = min(k, n_b) blocks are kept: the first K_b under the
 * strict order (higher score first, then lower block index). Exactly one set satisfies
 * this, so the result is deterministic.
 *
 *   block_scores [B, max_blocks] int32 (as written by qsa_index_score); max_blocks must
 *                be a multiple of 4 and at most 262144 (contexts up to 1,048,576 tokens)
 *   context_lens [B] int32, with ceil(L_b/4) <= max_blocks
 *   page_max     [B, max_pages_per_seq] int32 as written by qsa_index_score, or NULL. When
 *                given (then 16*max_pages_per_seq must be >= max_blocks - 15), requests with
 *                at least k pages read only the scores of the pages whose maximum reaches
 *                the k-th largest page maximum. The result is the same either way.
 *   k            blocks to keep, 1 <= k <= 512
 *   sel_blocks   out [B, k] int32: the kept block ids in ascending order, then -1
 *   sel_count    out [B] int32: K_b
 *   workspace    qsa_topk_workspace_size(B, max_blocks, k) bytes (see Workspace)
 */
size_t qsa_topk_workspace_size(int B, int max_blocks, int k);
qsa_status_t qsa_topk_select(const int32_t* block_scores, const int32_t* context_lens,
                             const int32_t* page_max, int B, int max_blocks,
                             int max_pages_per_seq, int k,
                             int32_t* sel_blocks, int32_t* sel_count,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * qsa_sparse_attn_decode - attention of the decode query over the kept tokens, per slice.
 *
 * Article, same paragraph: the final softmax and the value aggregation use the
 * full (not pooled) K and V rows of the kept positions; section "What the pull request actually
 * changes", first paragraph and bullets: under DCP a rank attends over its own contiguous
 * piece of the context. Request b's pages are cut into P contiguous runs of S_b = ceil(ceil(L_b/64)/P)
 * pages; slice p covers tokens [64*p*S_b, min(64*(p+1)*S_b, L_b)). For each slice p and
 * query head h (KV head g = h / (Hq/Hkv)), over the kept tokens t of slice p:
 *     s_t = softmax_scale * dot(q[b][h], K[t][g])
 *     partial_out[b][p][h] = sum_t exp(s_t - m) V[t][g] / sum_t exp(s_t - m),  m = max s_t
 *     partial_lse[b][p][h] = m + ln(sum_t exp(s_t - m))
 * A slice without kept tokens gives partial_out = 0 and partial_lse = -inf.
 *
 *   q            [B, Hq, head_dim] bf16
 *   k_cache, v_cache, page_table, context_lens: see Layouts
 *   sel_blocks   [B, k] int32 and sel_count [B] int32, as written by qsa_topk_select
 *   P            slices per request, 1 <= P <= 64
 *   partial_out  out [B, P, Hq, head_dim] float32 (each slice normalised on its own)
 *   partial_lse  out [B, P, Hq] float32, natural log
 *   workspace    qsa_attn_workspace_size(B, Hq, Hkv, k, P) bytes (see Workspace). Each
 *                slice's kept tokens are split into C shares attended in parallel, C the
 *                largest power of two <= min(32, ceil(512 / (B*Hkv*P))) (at least 1); the
 *                workspace holds the share partials, B*P*C*Hq*head_dim + B*P*C*Hq floats
 *                (each part rounded up to 256 bytes), which are merged into the slice
 *                partials by log-sum-exp. With C = 1 the size is 0 (the slice partials
 *                are written directly).
 */
size_t qsa_attn_workspace_size(int B, int Hq, int Hkv, int k, int P);
qsa_status_t qsa_sparse_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* page_table, const int32_t* context_lens,
                                    const int32_t* sel_blocks, const int32_t* sel_count,
                                    int B, int Hq, int Hkv, int head_dim, int page_size,
                                    int max_pages_per_seq, int k, int P, float softmax_scale,
                                    float* partial_out, float* partial_lse,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * qsa_lse_merge - combine the P slice partials of every (request, head).
 *
 * Article, section "What the pull request actually changes", bullets, and section
 * "Questions worth answering directly" (DCP versus TP): the per-slice partials are joined
 * once every slice has been read. With M = max over p of the finite
 * partial_lse, w_p = exp(partial_lse - M):
 *     out = sum_p w_p partial_out[p] / sum_p w_p,   out_lse = M + ln(sum_p w_p)
 * Slices with lse = -inf carry no weight; if every slice is -inf, out = 0, out_lse = -inf.
 *
 *   partial_out  [B, P, Hq, head_dim] float32,  partial_lse [B, P, Hq] float32
 *   out          out [B, Hq, head_dim] float32
 *   out_lse      out [B, Hq] float32, or NULL
 */
qsa_status_t qsa_lse_merge(const float* partial_out, const float* partial_lse,
                           int B, int P, int Hq, int head_dim,
                           float* out, float* out_lse, void* stream);

/*
 * qsa_decode - the whole chain on one stream, one workspace for everything.
 * Arguments as in the four calls above. block_scores, sel_blocks, sel_count,
 * partial_out and partial_lse are still caller buffers, so the intermediates stay
 * inspectable; out_lse may be NULL. The workspace (qsa_decode_workspace_size bytes, no
 * initialisation needed) holds the per-page maxima passed from the scan to the selection
 * (B * ceil(max_blocks/16) int32, rounded up to 256 bytes), then the attention workspace.
 * The slice partials and the merged output are formed by one kernel, with the same
 * operations as qsa_lse_merge, so the results equal those of the four separate calls bit
 * for bit.
 */
size_t qsa_decode_workspace_size(int B, int Hq, int Hkv, int max_blocks, int k, int P);
qsa_status_t qsa_decode(const void* q, const int8_t* q_idx, const int8_t* idx_cache,
                        const void* k_cache, const void* v_cache,
                        const int32_t* page_table, const int32_t* context_lens,
                        int B, int Hq, int Hkv, int head_dim, int n_idx_heads, int idx_dim,
                        int page_size, int max_pages_per_seq, int max_blocks, int k, int P,
                        float softmax_scale,
                        int32_t* block_scores, int32_t* sel_blocks, int32_t* sel_count,
                        float* partial_out, float* partial_lse, float* out, float* out_lse,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * qsa_time_next_scan - measurement hook. The next launch of an indexer scan kernel made by
 * this thread (through qsa_index_score, qsa_decode, qsa_decode_noalloc, qsa_decode_multi,
 * qsa_index_score_multi, or the side-cache scan of qsa_index_score_pooled, qsa_decode_pooled,
 * qsa_decode_multi_pooled and qsa_decode_step_pooled) records start_event when the kernel begins executing and stop_event when it
 * ends (both hipEvent_t created with timing enabled, either may be NULL), so the kernel's own
 * duration can be read with hipEventElapsedTime, inside a chain, without marker packets
 * around it. Used once, then cleared; NULL, NULL clears it. Always returns QSA_OK.
 */
qsa_status_t qsa_time_next_scan(void* start_event, void* stop_event);

/*
 * qsa_decode_noalloc - qsa_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same chain
 * and the same results, bit for bit, with the workspace taken from a static device array of
 * the library instead of a caller buffer. The caller still passes every input and output.
 *
 * The array holds QSA_NOALLOC_SCRATCH_BYTES bytes on each device the library runs on, from
 * the library's load until the process ends. Its device address is looked up once per device
 * (hipGetSymbolAddress, on the call's current device) at the first call there. A call whose
 * qsa_decode_workspace_size(B, Hq, Hkv, max_blocks, k, P) exceeds the array returns
 * QSA_ERR_SCRATCH and launches nothing. The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine). Nothing in the array needs to start at zero: every word the
 * chain reads there is written earlier in the same call.
 *
 * Every call on one device shares that device's array: calls that may overlap on one device
 * (different streams, or one stream and another thread) race on it and must be serialised by
 * the caller. Arguments and errors otherwise as qsa_decode.
 */
#define QSA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
qsa_status_t qsa_decode_noalloc(const void* q, const int8_t* q_idx, const int8_t* idx_cache,
                                const void* k_cache, const void* v_cache,
                                const int32_t* page_table, const int32_t* context_lens,
                                int B, int Hq, int Hkv, int head_dim, int n_idx_heads, int idx_dim,
                                int page_size, int max_pages_per_seq, int max_blocks, int k, int P,
                                float softmax_scale,
                                int32_t* block_scores, int32_t* sel_blocks, int32_t* sel_count,
                                float* partial_out, float* partial_lse, float* out, float* out_lse,
                                void* stream);

/*
 * qsa_decode_multi - multi-token decode: T new tokens per request, 1 <= T <= 4096, B*T <= 65535
 * (draft tokens of speculative decoding with a multi-token-prediction head, T <= 4, or a
 * prefill chunk). The scan runs as an int8 matrix product of the T queries with every page's
 * keys on the matrix cores, except for T = 1 and, on batches of fewer than 4,096 pages, for
 * T <= 4, where it uses int8 dot products per query; the scores are the same integers. From
 * T = 16 on, at Hq = 8*Hkv, neighbouring new tokens share attention workgroups that read the
 * union of their kept blocks once; the results are defined exactly as below either way.
 *
 * The T new tokens are the last T positions of each request's cache (context_lens counts them
 * all). Draft token t, at position L_b - T + t, is decoded exactly as qsa_decode decodes a
 * single token at length L_b - T + 1 + t (its own indexer query and top-k selection, attention
 * over its own kept tokens, slices of that length), so it sees itself and the tokens before
 * it; a length that would be below 0 is 0. The indexer keys are read once for all T queries.
 *   q        [B, T, Hq, head_dim] bf16;  q_idx [B, T, n_idx_heads, idx_dim] int8
 *   results  for virtual request r = b*T + t: block_scores [B*T, max_blocks],
 *            sel_blocks [B*T, k], sel_count [B*T], partial_out [B*T, P, Hq, head_dim],
 *            partial_lse [B*T, P, Hq], out [B*T, Hq, head_dim], out_lse [B*T, Hq]
 *   workspace qsa_decode_multi_workspace_size(B, T, ...) bytes (= qsa_decode's for B*T).
 * Everything else as qsa_decode; T = 1 gives qsa_decode's results.
 */
size_t qsa_decode_multi_workspace_size(int B, int T, int Hq, int Hkv, int max_blocks, int k, int P);

/* The multi-token decode's indexer scan on its own: scores (and, if page_max is not NULL,
 * per-page maxima [B*T, max_pages_per_seq]) of all T draft tokens of every request, from one
 * read of the indexer keys. q_idx [B, T, n_idx_heads, idx_dim]; block_scores [B*T, max_blocks];
 * row b*T + t holds draft token t's scores for blocks < ceil((L_b - T + 1 + t) / 4). Page
 * maxima row b*T + t is written for the pages p < ceil(L_b/64) only: the largest of the
 * token's scores there, INT32_MIN on a page where it has none. Checks as
 * qsa_index_score, plus 1 <= T <= 4096, B*T <= 65535, max_blocks % 4 == 0 and block_scores
 * 16-byte aligned. */
qsa_status_t qsa_index_score_multi(const int8_t* q_idx, const int8_t* idx_cache,
                                   const int32_t* page_table, const int32_t* context_lens, int B,
                                   int T, int n_idx_heads, int idx_dim, int page_size,
                                   int max_pages_per_seq, int max_blocks, int32_t* block_scores,
                                   int32_t* page_max, void* stream);
qsa_status_t qsa_decode_multi(const void* q, const int8_t* q_idx, const int8_t* idx_cache,
                              const void* k_cache, const void* v_cache,
                              const int32_t* page_table, const int32_t* context_lens,
                              int B, int T, int Hq, int Hkv, int head_dim, int n_idx_heads,
                              int idx_dim, int page_size, int max_pages_per_seq, int max_blocks,
                              int k, int P, float softmax_scale,
                              int32_t* block_scores, int32_t* sel_blocks, int32_t* sel_count,
                              float* partial_out, float* partial_lse, float* out, float* out_lse,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * The indexer's side cache of pooled keys.
 *
 * Article, section "What the pull request actually changes": besides the main cache the
 * indexer keeps caches of its own, a selector cache and side caches (second paragraph), grouped with the
 * main cache, and synthetic batches must not write the side caches (bullets). The side cache
 * here holds the pooled key of every micro-block - the int sum of the int8 indexer keys of
 * its up to 4 tokens (|sum| <= 512), as int16 - so the scan reads 512 bytes per block instead
 * of 1024:
 *   pooled_cache [num_pages, page_size/4, n_idx_heads, idx_dim] int16, page-aligned with the
 *   main caches: block j of request b lives in page page_table[b][j / 16], slot j % 16.
 * Entries of blocks past ceil(L_b/4) are never read.
 */

/* Build the side-cache entries of every block of every request (the prefill-time path):
 * entry of block j = sum of the indexer rows of tokens 4j .. min(4j+3, L_b-1). Other entries
 * are left as they are. Checks as qsa_index_score; pooled_cache 16-byte aligned. */
qsa_status_t qsa_pool_build(const int8_t* idx_cache, const int32_t* page_table,
                            const int32_t* context_lens, int B, int n_idx_heads, int idx_dim,
                            int page_size, int max_pages_per_seq, int16_t* pooled_cache,
                            void* stream);

/* The decode step's cache writes. context_lens counts the new token, which sits at
 * t = L_b - 1: its rows k_new[b] ([Hkv, head_dim] bf16), v_new[b] and idx_new[b]
 * ([n_idx_heads, idx_dim] int8) are written to row t % page_size of page
 * page_table[b][t / page_size] of k_cache, v_cache and idx_cache, and, when pooled_cache is
 * not NULL, the side-cache entry of block t / 4 becomes the sum of that block's indexer rows
 * at positions <= t. write ([B] int32, NULL = every request writes): a request with
 * write[b] == 0 (a padding or synthetic entry of the batch) writes nothing, main or side;
 * neither does a request with L_b == 0. Requests of one call must not share a page row. */
qsa_status_t qsa_cache_append(const void* k_new, const void* v_new, const int8_t* idx_new,
                              const int32_t* write, void* k_cache, void* v_cache, int8_t* idx_cache,
                              int16_t* pooled_cache, const int32_t* page_table,
                              const int32_t* context_lens, int B, int Hkv, int head_dim,
                              int n_idx_heads, int idx_dim, int page_size, int max_pages_per_seq,
                              void* stream);

/* qsa_index_score reading the side cache: the same block scores (bit for bit) and optional
 * per-page maxima, from half the bytes. Arguments as qsa_index_score, with pooled_cache in
 * place of idx_cache. */
qsa_status_t qsa_index_score_pooled(const int8_t* q_idx, const int16_t* pooled_cache,
                                    const int32_t* page_table, const int32_t* context_lens, int B,
                                    int n_idx_heads, int idx_dim, int page_size,
                                    int max_pages_per_seq, int max_blocks, int32_t* block_scores,
                                    int32_t* page_max, void* stream);

/* qsa_decode with the scan reading the side cache instead of the int8 keys; every other
 * argument, the workspace and every result are as qsa_decode's (the results are the same
 * bits). */
qsa_status_t qsa_decode_pooled(const void* q, const int8_t* q_idx, const int16_t* pooled_cache,
                               const void* k_cache, const void* v_cache,
                               const int32_t* page_table, const int32_t* context_lens,
                               int B, int Hq, int Hkv, int head_dim, int n_idx_heads, int idx_dim,
                               int page_size, int max_pages_per_seq, int max_blocks, int k, int P,
                               float softmax_scale,
                               int32_t* block_scores, int32_t* sel_blocks, int32_t* sel_count,
                               float* partial_out, float* partial_lse, float* out, float* out_lse,
                               void* workspace, size_t workspace_bytes, void* stream);

/* qsa_decode_multi with the scan reading the side cache: 2 <= T <= 4 draft tokens per request
 * (T = 1 is qsa_decode_pooled), the same results bit for bit as qsa_decode_multi. The T draft
 * tokens' rows are already in all caches, pooled_cache included (its entry for a block holds
 * the sum of every indexer row of the block below context_lens), so the side-cache entries of
 * the blocks holding draft positions pool keys that earlier draft tokens must not see: the
 * scan reads those pages (the pages within T-1 tokens of L_b, at most two per request) from
 * idx_cache instead, token by token, and every other page from pooled_cache. Arguments,
 * workspace (qsa_decode_multi_workspace_size) and results as qsa_decode_multi, plus
 * pooled_cache; T > 4 returns QSA_ERR_UNSUPPORTED. */
qsa_status_t qsa_decode_multi_pooled(const void* q, const int8_t* q_idx, const int8_t* idx_cache,
                                     const int16_t* pooled_cache, const void* k_cache,
                                     const void* v_cache, const int32_t* page_table,
                                     const int32_t* context_lens, int B, int T, int Hq, int Hkv,
                                     int head_dim, int n_idx_heads, int idx_dim, int page_size,
                                     int max_pages_per_seq, int max_blocks, int k, int P,
                                     float softmax_scale, int32_t* block_scores, int32_t* sel_blocks,
                                     int32_t* sel_count, float* partial_out, float* partial_lse,
                                     float* out, float* out_lse, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* One decode step on the side cache: qsa_cache_append (with pooled_cache) followed by
 * qsa_decode_pooled, in one call and with the same results. The cache writes are made by the
 * scan (the wave that reads the page holding the new token), which saves a launch. Arguments
 * as in those two calls; k_cache, v_cache, idx_cache and pooled_cache are written. */
qsa_status_t qsa_decode_step_pooled(const void* k_new, const void* v_new, const int8_t* idx_new,
                                    const int32_t* write, void* k_cache, void* v_cache,
                                    int8_t* idx_cache, int16_t* pooled_cache,
                                    const void* q, const int8_t* q_idx,
                                    const int32_t* page_table, const int32_t* context_lens,
                                    int B, int Hq, int Hkv, int head_dim, int n_idx_heads,
                                    int idx_dim, int page_size, int max_pages_per_seq,
                                    int max_blocks, int k, int P, float softmax_scale,
                                    int32_t* block_scores, int32_t* sel_blocks, int32_t* sel_count,
                                    float* partial_out, float* partial_lse, float* out,
                                    float* out_lse, void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * qsa_check_pages - check, on the device, the preconditions the compute calls do not check.
 *
 * The page table is the article's one cache group (section "What the pull request actually
 * changes", bullets): token t of request b lives in page page_table[b][t / page_size] of all
 * three caches, which hold num_pages pages. The compute calls trust the table; a page id out
 * of range there is an out-of-bounds read. This call reads only page_table and context_lens
 * (never a cache row, so a bad table cannot make it fault) and writes one verdict per request:
 *   verdict[b] = -1   valid: 0 <= L_b <= max_pages_per_seq*page_size and every id
 *                     page_table[b][p], p < ceil(L_b/page_size), lies in [0, num_pages)
 *   verdict[b] = -2   L_b < 0 or L_b > max_pages_per_seq*page_size
 *   verdict[b] = p    the first page slot p whose id lies outside [0, num_pages)
 *
 *   page_table   [B, max_pages_per_seq] int32;  context_lens [B] int32
 *   verdict      out [B] int32 (device)
 * Host checks: B >= 0 (B <= 65535), max_pages_per_seq >= 1, page_size >= 1, num_pages >= 0.
 */
qsa_status_t qsa_check_pages(const int32_t* page_table, const int32_t* context_lens, int B,
                             int max_pages_per_seq, int page_size, int num_pages, int32_t* verdict,
                             void* stream);

/* Fill a workspace with zero bytes on `stream`. No entry point needs it (a workspace needs no
 * initialisation); it is there for callers that want known memory contents. */
qsa_status_t qsa_workspace_clear(void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* QSA_H_ */
