/*
 * isb.h - C ABI of libisb: one layer of indexed block-sparse paged-attention
 * decode on an AMD Instinct MI355X (gfx950).
 *
 * The layer's steps are separate calls on one HIP stream, each taking plain
 * device pointers and sizes (a whole layer step can run as two launches:
 * isb_index_score, then isb_select_attend):
 *
 *   isb_index_score              score every 128-token block of each request's
 *                                paged index-key cache with the index query;
 *   isb_topk_select              keep the top-k blocks of each (token, KV head);
 *   isb_emit_sparse_block_table  turn the selection into a sparse page table;
 *   isb_topk_select_emit         both of the above in one launch;
 *   isb_sparse_pa_decode         paged attention over the selected pages only
 *                                (split-K flash decode; the last split of a
 *                                row merges it, in the same launch);
 *   isb_select_attend            top-k, emit and attention in one launch;
 *   isb_topk_merge               a row's selection from the (score, block id)
 *                                picks of shards of its blocks (the merge
 *                                step of context parallelism).
 *
 * In front of them, the cache writer of the same decode step:
 *
 *   isb_write_cache              quantise the step's new keys, values and
 *                                index keys into the pools;
 *   isb_quantize_e4m3            the unit-scale e4m3 cast of a query;
 *   isb_prepare_query            a query's QK-norm and rope, then its bf16 or
 *                                e4m3 form.
 *
 * The calls follow the decode call of the vLLM API page for
 * vllm.models.minimax_m3.amd.sparse_attention_msa (MiniMaxM3SparseAiterPAImpl
 * .forward: query, K/V caches, top-k indices, block_table, seq_lens,
 * num_kv_heads, scale, output, k_scale / v_scale, decode_query_len,
 * sparse_block_table, sparse_context_lens), and the index caches and MXFP4
 * pages of ROCm/ATOM PR 2962 ("[MiniMax-M3.1] MXFP4 index cache and MXFP4 KV
 * cache", Summary).
 *
 * Common conventions
 * ------------------
 *  - Every pointer is device memory owned by the caller.  The library never
 *    allocates, frees or synchronises; it only enqueues kernels on `stream`
 *    (NULL = the default stream).  Calls may therefore be captured into a HIP
 *    graph.  Inputs are read-only; outputs are fully written by every call, so
 *    their prior contents never matter.  (The attention workspace is the one
 *    buffer with a contract on its contents: see isb_sparse_pa_decode.)
 *  - R requests, q = decode_query_len, T = R q query tokens.  Token t = r q + i
 *    of request r has causal length L_t = max(0, seq_lens[r] - (q - 1 - i)) and
 *    n_t = ceil(L_t / 128) valid blocks.  Rows with n_t = 0 (pad requests of
 *    length 0) select nothing and produce zeros.
 *  - head_dim is 128.  H_kv KV heads; H_q query heads (G = H_q / H_kv <= 16);
 *    H_idx index heads (a multiple of H_kv).
 *  - Return value: ISB_OK (0) or a negative isb_status.  Nothing is enqueued
 *    when an argument check fails.  ISB_E_LAUNCH reports hipGetLastError after
 *    the launches.  Device-side data (page ids in range, seq_lens <= the table
 *    width times 128) is the caller's contract; kernels treat an out-of-range
 *    page id as poison (the affected scores / outputs become NaN) and never
 *    dereference it.
 *
 * Pool layout (one page id addresses the K page and the V page alike)
 * -------------------------------------------------------------------
 *  index cache, one page per 128-token block (page id = block id):
 *    ISB_BF16      eight 16-token tiles, each laid out as a bf16 K page
 *                  below (token 16 i + c of the block is key c of tile i,
 *                  tile i at byte 4096 i)                        32768 B
 *    ISB_FP8_E4M3  the same with e4m3 tiles of 2048 B, x idx_scale 16384 B
 *    ISB_MXFP4     128 x 64 B e2m1 (token j at 64 j, dim 2c in the low
 *                  nibble of byte c, 2c+1 in the high nibble) then
 *                  128 x 4 B e8m0 (token j at 8192 + 4 j, scale s for
 *                  dims 32 s .. 32 s + 31)                       8704 B
 *  K/V caches, bf16 / fp8: 16-token pages, 8 per block; block b of a request
 *    is pages 8 block_table[r][b] + 0..7.  With e bytes per element (1 or 2),
 *    a page is 2048 e bytes in the order the kernel's lanes read it:
 *      K: key c, dim d at 1024 ((d mod 32) div (16/e)) + 256 (d div 32)
 *         + 16 c + e (d mod (16/e));
 *      V: key t, dim d = 16 dt + c at 1024 (dt div (4/e)) + 256 (t div 4)
 *         + 16 c + 4 e (dt mod (4/e)) + e (t mod 4).
 *    fp8 values times k_scale / v_scale.
 *  K/V caches, MXFP4: one 8704 B page per block for K and one for V.
 *  A K/V page id holds one page per KV head, [num_pages][H_kv][page bytes];
 *  row (t, g) reads head g's page.  The index cache has one key per token,
 *  shared by all index heads.
 */
#ifndef ISB_H
#define ISB_H

#include <stddef.h>
#include <stdint.h>

/* Exported entry points; everything else in the library is hidden. */
#define ISB_API __attribute__((visibility("default")))

#ifdef __cplusplus
extern "C" {
#endif

/* Layout-compatible with hipStream_t; NULL selects the default stream. */
typedef struct ihipStream_t* isb_stream_t;

typedef enum isb_dtype {
  ISB_BF16 = 0,      /* bfloat16 */
  ISB_FP8_E4M3 = 1,  /* OCP float8 e4m3fn (no infinities, 0x7F / 0xFF are NaN) */
  ISB_MXFP4 = 2      /* OCP MX: e2m1 elements + one e8m0 scale per 32 */
} isb_dtype;

typedef enum isb_status {
  ISB_OK = 0,
  ISB_E_INVALID_ARG = -1,       /* null pointer or negative / zero size */
  ISB_E_UNSUPPORTED_DTYPE = -2, /* dtype not valid for this argument */
  ISB_E_SHAPE = -3,             /* shape relation violated (see each call) */
  ISB_E_WORKSPACE = -4,         /* workspace smaller than required */
  ISB_E_LAUNCH = -5             /* a kernel launch failed */
} isb_status;

/* Library version, major * 10000 + minor * 100 + patch. */
ISB_API int isb_version(void);

/* Static, human-readable text for an isb_status value. */
ISB_API const char* isb_strerror(int status);

/*
 * isb_index_score - block scores of every (KV head, token, block).
 *
 * Defines (ROCm/ATOM PR 2962, Known limits: one fp32 score per index head,
 * row and 128-token block; Summary: e4m3 index query for the MXFP4 index):
 *   scores[g][t][b] = sum over index heads h of group g of
 *                     max over tokens j of block b with position < L_t of
 *                     dot(q_idx[t][h][:], k_idx[j][:])          (fp32)
 * for b < n_t, and -inf for n_t <= b < max_blocks.  The fp8 index cache
 * multiplies by idx_scale (ignored otherwise).  A NaN among a block's causally
 * valid keys makes that score NaN.
 *
 *   q_idx        [T][num_idx_heads][128], q_idx_dtype ISB_BF16 or ISB_FP8_E4M3
 *   idx_pool     [idx_pool_blocks] pages of idx_dtype (layout above)
 *   block_table  [num_reqs][block_table_stride] int32 block ids; entries past a
 *                request's ceil(seq_len/128) blocks are never read
 *   seq_lens     [num_reqs] int32, each <= 128 * min(max_blocks, stride)
 *   scores       out, [num_kv_heads][T][max_blocks] fp32
 * decode_query_len may be a prefill chunk: up to 16 tokens and 64 query rows
 * (decode_query_len * num_idx_heads) a request take the decode kernels; more
 * take a kernel that holds a block's keys in registers and runs them against
 * up to 128 query rows a wave, which needs num_idx_heads to divide 16.
 * Shape errors: num_idx_heads % num_kv_heads != 0, max_blocks > stride,
 * more than 16 tokens or 64 rows with 16 % num_idx_heads != 0,
 * decode_query_len * num_idx_heads > 2^20, num_reqs * decode_query_len
 * > 2^31 - 1, num_reqs > 65535.
 */
ISB_API int isb_index_score(isb_stream_t stream,
                    const void* q_idx, int q_idx_dtype, int num_idx_heads,
                    const void* idx_pool, int idx_dtype, float idx_scale,
                    int64_t idx_pool_blocks,
                    const int32_t* block_table, int block_table_stride,
                    const int32_t* seq_lens, int num_reqs, int decode_query_len,
                    int num_kv_heads, int max_blocks, float* scores);

/*
 * isb_topk_select - the blocks each (KV head, token) row attends to.
 *
 * Per row (PR 2962: the tail block is part of every selection; pad rows compute
 * nothing): the tail block n_t - 1, plus the top_k - 1 best of blocks
 * [0, n_t - 1) by score, ties to the lower block index, NaN below every number
 * and -0.0 equal to +0.0.  Written ascending, padded with -1; a row with
 * n_t = 0 is all -1.  Bit-exact for given fp32 scores.
 *
 *   scores    [num_kv_heads][T][max_blocks] fp32 (as isb_index_score writes)
 *   topk_idx  out, [num_kv_heads][T][top_k] int32
 * Shape errors: top_k < 1, top_k > max_blocks, max_blocks > 1048576.
 */
ISB_API int isb_topk_select(isb_stream_t stream, const float* scores,
                    const int32_t* seq_lens, int num_reqs, int decode_query_len,
                    int num_kv_heads, int max_blocks, int top_k, int32_t* topk_idx);

/*
 * isb_emit_sparse_block_table - selection -> sparse page table.
 *
 * Row (t, g) = t * num_kv_heads + g (token-major, as the vLLM page slices
 * sparse_bt_buffer[: nd * kvh]).  The k-th selected block b of the row
 * (entries >= 0 in order) becomes pages
 *   sparse_bt[row][k * ppb + p] = block_table[r][b] * ppb + p,  p < ppb,
 * unused slots are -1, and
 *   sparse_ctx[row] = (m - 1) * 128 + (L_t - 128 (n_t - 1))
 * for m >= 1 selected blocks (the tail block last), else 0.
 * pages_per_block (ppb) is 8 for bf16 / fp8 K/V and 1 for MXFP4 K/V
 * (PR 2962: pages_per_block is an emit parameter, 8 or 1).  Entries >= the
 * table stride are treated as -1.
 *
 *   topk_idx    [num_kv_heads][T][top_k] int32
 *   sparse_bt   out, [T * num_kv_heads][top_k * ppb] int32
 *   sparse_ctx  out, [T * num_kv_heads] int32
 * Shape errors: ppb not 1 or 8.
 */
ISB_API int isb_emit_sparse_block_table(isb_stream_t stream, const int32_t* topk_idx,
                                const int32_t* block_table, int block_table_stride,
                                const int32_t* seq_lens, int num_reqs,
                                int decode_query_len, int num_kv_heads, int top_k,
                                int pages_per_block, int32_t* sparse_bt,
                                int32_t* sparse_ctx);

/*
 * isb_topk_select_emit - isb_topk_select followed by
 * isb_emit_sparse_block_table, in one launch: each row's workgroup selects its
 * blocks and writes their pages, so the selection never leaves the chip
 * between the two steps.  Writes exactly what the two calls write (topk_idx,
 * sparse_bt, sparse_ctx; same layouts, bit-identical).  Rows too wide for one
 * workgroup's LDS run as the two separate launches.
 *
 * Arguments as in the two calls; max_blocks must not exceed
 * block_table_stride.  Shape errors: those of both calls.
 */
ISB_API int isb_topk_select_emit(isb_stream_t stream, const float* scores,
                                 const int32_t* seq_lens, int num_reqs,
                                 int decode_query_len, int num_kv_heads, int max_blocks,
                                 int top_k, const int32_t* block_table,
                                 int block_table_stride, int pages_per_block,
                                 int32_t* topk_idx, int32_t* sparse_bt,
                                 int32_t* sparse_ctx);

/*
 * isb_topk_merge - the selection of each (KV head, token) row from candidates.
 *
 * The merge step of context parallelism (ROCm/ATOM PR 2962 lists a candidate
 * exchange among the users of the emit helper).  When each shard of a row's
 * blocks (a contiguous range) is selected by isb_topk_select as if it were the
 * whole row, the shards' picks, gathered with their scores, hold the row's
 * true winners, and this call returns exactly what isb_topk_select returns on
 * the whole row: the tail n_t - 1 plus the best top_k - 1 candidates with ids
 * in [0, n_t - 1) (score descending, NaN below every number, -0.0 == +0.0,
 * ties to the lower block index), ascending, -1 padded; a row with
 * n_t - 1 <= top_k - 1 takes all its blocks.  n_t as in isb_topk_select,
 * clamped to max_blocks.
 *
 *   cand_scores  [num_kv_heads][T][num_cands] fp32
 *   cand_ids     [num_kv_heads][T][num_cands] int32 block ids, distinct within
 *                a row; -1 (or any id outside [0, n_t - 1)) = no candidate
 *   seq_lens     [num_reqs] int32
 *   topk_idx     out, [num_kv_heads][T][top_k] int32
 * Shape errors: num_cands > 1024, top_k < 1 or > max_blocks,
 * num_reqs * decode_query_len * num_kv_heads > 2^31 - 1.
 */
ISB_API int isb_topk_merge(isb_stream_t stream, const float* cand_scores,
                           const int32_t* cand_ids, int num_cands, const int32_t* seq_lens,
                           int num_reqs, int decode_query_len, int num_kv_heads,
                           int max_blocks, int top_k, int32_t* topk_idx);

/*
 * Bytes of workspace isb_sparse_pa_decode needs for these arguments: the
 * split-K partial results of every (row, split), 16 heads x (128 + 2) fp32
 * each.  0 when every row takes one split (nothing is published), or for
 * invalid arguments.
 */
ISB_API size_t isb_sparse_pa_workspace_bytes(int num_tokens, int num_q_heads, int num_kv_heads,
                                     int sparse_bt_stride, int kv_dtype);

/*
 * isb_sparse_pa_decode - attention over the selected pages.
 *
 * For row (t, g) and query head h of KV group g (vLLM API page, the decode
 * call): z_u = sm_scale * dot(q[t][h], K_u) over sparse positions
 * u < sparse_ctx[row]; out[t][h] = sum_u softmax(z)_u V_u, in fp32, written as
 * bf16.  A row's pages are split across workgroups; each publishes its
 * partial result, and a workgroup that finds every other split of its row
 * published merges the row (log-sum-exp weights, in split order, so results
 * do not depend on timing).  One launch.  Position u is slot u mod P of page
 * sparse_bt[row][u div P], with
 * P = 16 tokens per page (bf16 / fp8 K/V) or 128 (MXFP4 K/V).  fp8 K/V are
 * multiplied by k_scale / v_scale.  Rows with sparse_ctx = 0 output zeros.
 *
 *   q           [num_tokens][num_q_heads][128], q_dtype ISB_BF16 or ISB_FP8_E4M3
 *   decode_query_len  query tokens per request (the decode call's own
 *               argument): num_tokens is a multiple of it, and the rows of
 *               one request's tokens may select the same pages.  It changes
 *               only how pages are read (with 1, no page is read twice in a
 *               call and pages are streamed past the caches), never a result.
 *   k_pool, v_pool  [num_pages][num_kv_heads] pages of kv_dtype (layout above)
 *   sparse_bt   [num_tokens * num_kv_heads][sparse_bt_stride] int32 page ids
 *   sparse_ctx  [num_tokens * num_kv_heads] int32, <= sparse_bt_stride * P
 *   workspace   >= isb_sparse_pa_workspace_bytes(...) bytes, 16-byte aligned,
 *               zero-filled before its first use (one fill of the buffer): a
 *               slot of split partials is free when all its words are zero,
 *               and a published word never is.  Every completed call leaves
 *               the workspace zero; calls that share a workspace must not
 *               overlap in time.  May be NULL when the size query gives 0.
 *   out         out, [num_tokens][num_q_heads][128] bf16
 * Shape errors: head_dim != 128, num_q_heads % num_kv_heads, G > 16,
 * num_tokens % decode_query_len.
 */
ISB_API int isb_sparse_pa_decode(isb_stream_t stream,
                         const void* q, int q_dtype,
                         const void* k_pool, const void* v_pool, int kv_dtype,
                         int64_t num_pages, float k_scale, float v_scale,
                         const int32_t* sparse_bt, int sparse_bt_stride,
                         const int32_t* sparse_ctx, int num_tokens,
                         int decode_query_len, int num_q_heads, int num_kv_heads,
                         int head_dim, float sm_scale, void* workspace,
                         size_t workspace_bytes, void* out);

/*
 * isb_sparse_pa_decode_noalloc - isb_sparse_pa_decode without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, hosts that forbid allocation).  The
 * split partials go to the library's own zero-initialised device array
 * (8 MiB, one per device, held until the process ends; every completed call
 * leaves it zero).  Arguments, results and errors as isb_sparse_pa_decode;
 * ISB_E_WORKSPACE when the partials these arguments need
 * (isb_sparse_pa_workspace_bytes) exceed 8 MiB.  The stream must belong to
 * the current device.  Calls that overlap in time on one device share the
 * array and race.
 */
ISB_API int isb_sparse_pa_decode_noalloc(isb_stream_t stream,
                         const void* q, int q_dtype,
                         const void* k_pool, const void* v_pool, int kv_dtype,
                         int64_t num_pages, float k_scale, float v_scale,
                         const int32_t* sparse_bt, int sparse_bt_stride,
                         const int32_t* sparse_ctx, int num_tokens,
                         int decode_query_len, int num_q_heads, int num_kv_heads,
                         int head_dim, float sm_scale, void* out);

/*
 * isb_select_attend - isb_topk_select_emit followed by isb_sparse_pa_decode,
 * in one launch where it can: each attention workgroup selects its row's
 * blocks itself (from the row's scores and block-table row) and takes its
 * page ids from there; the first split of each row also writes topk_idx,
 * sparse_bt and sparse_ctx.  Writes exactly what the two calls write (the
 * selection, table and lengths bit-identical; the output as
 * isb_sparse_pa_decode computes it).  One launch (any K/V dtype) with
 * max_blocks <= 2048, max_blocks and block_table_stride multiples of 4 and
 * 16-byte aligned scores and block table; otherwise the two calls in turn.
 *
 * Arguments as in isb_topk_select_emit and isb_sparse_pa_decode (the sparse
 * table stride is top_k * pages_per_block, 8 or 1 by kv_dtype; head_dim 128).
 * The workspace is the one isb_sparse_pa_workspace_bytes gives for
 * sparse_bt_stride = top_k * pages_per_block, with the same contract.
 */
ISB_API int isb_select_attend(isb_stream_t stream, const float* scores,
                              const int32_t* seq_lens, int num_reqs,
                              int decode_query_len, int num_kv_heads, int max_blocks,
                              int top_k, const int32_t* block_table,
                              int block_table_stride, const void* q, int q_dtype,
                              const void* k_pool, const void* v_pool, int kv_dtype,
                              int64_t num_pages, float k_scale, float v_scale,
                              int num_q_heads, float sm_scale, void* workspace,
                              size_t workspace_bytes, int32_t* topk_idx,
                              int32_t* sparse_bt, int32_t* sparse_ctx, void* out);

/*
 * Prefill batches
 * ---------------
 * The prefill call of the vLLM API page for sparse_attention_msa
 * (MiniMaxM3SparseAiterPAImpl.forward, prefill branch) gives every query
 * token its own request and position instead of a uniform chunk:
 *   query_req_id   [num_tokens] int32: the token's row of block_table;
 *   query_abs_pos  [num_tokens] int32: its 0-based position in the request.
 * Token t attends to positions 0 .. query_abs_pos[t] of its request: causal
 * length L_t = query_abs_pos[t] + 1 (the token's own key is already in the
 * cache) and n_t = ceil(L_t / 128) blocks.  Tokens may come in any order, of
 * any requests; a scheduler's order (each request's tokens together,
 * positions ascending) lets the scorer read a block once for many tokens.
 * Every other rule, layout and output is the decode call's with T =
 * num_tokens: scores [num_kv_heads][T][max_blocks], topk_idx
 * [num_kv_heads][T][top_k], sparse_bt / sparse_ctx rows t * num_kv_heads + g,
 * out [T][num_q_heads][128].  A token whose request id is outside
 * [0, num_reqs) or whose position is outside [0, 128 * max_blocks) (the
 * block-table width for the emit call) is an empty row: -inf scores, no
 * selection, sparse length 0, zero output; nothing is read through it.
 */

/*
 * isb_index_score_prefill - isb_index_score for a prefill batch.  Takes the
 * wide variant whatever the batch (query tiles of 128 rows of consecutive
 * tokens; each run of one request's tokens in a tile reads its blocks once).
 * Shape errors: those of isb_index_score, 16 % num_idx_heads != 0,
 * num_tokens * num_idx_heads > 2^31 - 1 or more than 65535 tiles of 128 rows.
 */
ISB_API int isb_index_score_prefill(isb_stream_t stream, const void* q_idx, int q_idx_dtype,
                                    int num_idx_heads, const void* idx_pool, int idx_dtype,
                                    float idx_scale, int64_t idx_pool_blocks,
                                    const int32_t* block_table, int block_table_stride, int num_reqs,
                                    const int32_t* query_req_id, const int32_t* query_abs_pos,
                                    int num_tokens, int num_kv_heads, int max_blocks, float* scores);

/* isb_topk_select_prefill - isb_topk_select for a prefill batch. */
ISB_API int isb_topk_select_prefill(isb_stream_t stream, const float* scores, int num_reqs,
                                    const int32_t* query_req_id, const int32_t* query_abs_pos,
                                    int num_tokens, int num_kv_heads, int max_blocks, int top_k,
                                    int32_t* topk_idx);

/*
 * isb_emit_sparse_block_table_prefill - isb_emit_sparse_block_table for a
 * prefill batch; positions are valid below 128 * block_table_stride.
 */
ISB_API int isb_emit_sparse_block_table_prefill(isb_stream_t stream, const int32_t* topk_idx,
                                                const int32_t* block_table, int block_table_stride,
                                                int num_reqs, const int32_t* query_req_id,
                                                const int32_t* query_abs_pos, int num_tokens,
                                                int num_kv_heads, int top_k, int pages_per_block,
                                                int32_t* sparse_bt, int32_t* sparse_ctx);

/* isb_topk_select_emit_prefill - isb_topk_select_emit for a prefill batch. */
ISB_API int isb_topk_select_emit_prefill(isb_stream_t stream, const float* scores, int num_reqs,
                                         const int32_t* query_req_id, const int32_t* query_abs_pos,
                                         int num_tokens, int num_kv_heads, int max_blocks, int top_k,
                                         const int32_t* block_table, int block_table_stride,
                                         int pages_per_block, int32_t* topk_idx, int32_t* sparse_bt,
                                         int32_t* sparse_ctx);

/*
 * isb_sparse_pa_prefill - isb_sparse_pa_decode for the rows of a prefill
 * batch (the prefill call's sparse_bt / sparse_ctx): the same results; the
 * rows of one request share many pages, which are read through the caches.
 * Workspace as isb_sparse_pa_workspace_bytes(num_tokens, ...) gives, with the
 * same contract.
 */
ISB_API int isb_sparse_pa_prefill(isb_stream_t stream, const void* q, int q_dtype,
                                  const void* k_pool, const void* v_pool, int kv_dtype,
                                  int64_t num_pages, float k_scale, float v_scale,
                                  const int32_t* sparse_bt, int sparse_bt_stride,
                                  const int32_t* sparse_ctx, int num_tokens, int num_q_heads,
                                  int num_kv_heads, int head_dim, float sm_scale, void* workspace,
                                  size_t workspace_bytes, void* out);

/* isb_select_attend_prefill - isb_select_attend for a prefill batch. */
ISB_API int isb_select_attend_prefill(isb_stream_t stream, const float* scores, int num_reqs,
                                      const int32_t* query_req_id, const int32_t* query_abs_pos,
                                      int num_tokens, int num_kv_heads, int max_blocks, int top_k,
                                      const int32_t* block_table, int block_table_stride,
                                      const void* q, int q_dtype, const void* k_pool,
                                      const void* v_pool, int kv_dtype, int64_t num_pages,
                                      float k_scale, float v_scale, int num_q_heads, float sm_scale,
                                      void* workspace, size_t workspace_bytes, int32_t* topk_idx,
                                      int32_t* sparse_bt, int32_t* sparse_ctx, void* out);

/*
 * The optional QK-norm and rope of the fused cache writer (ROCm/ATOM PR 2962,
 * Follow-ups: the fused QK-norm / rope / cache writer; the pages give none of
 * the step's parameters, so the caller does).  For one 128-dim head vector x
 * at position p, in fp32:
 *   norm  (norm_weight != NULL)  y_d = norm_weight[d] x_d / sqrt(mean(x^2) + eps)
 *   rope  (rope_cos != NULL)     dim pairs (a, b) -> (a c - b s, b c + a s) with
 *         c = rope_cos[p][i], s = rope_sin[p][i] for pair i < rot_dim / 2:
 *         pairs (i, i + rot_dim / 2) when neox, else (2i, 2i + 1); dims past
 *         rot_dim unchanged.
 * norm_weight [128], rope_cos and rope_sin [rope_positions][rot_dim / 2]: fp32
 * device arrays owned by the caller; eps >= 0; rot_dim a multiple of 4 in
 * 4..128 (ISB_E_SHAPE otherwise).  A NULL isb_norm_rope, or one with both
 * norm_weight and rope_cos NULL, applies nothing.
 */
typedef struct isb_norm_rope {
  const float* norm_weight;
  float eps;
  const float* rope_cos;
  const float* rope_sin;
  int64_t rope_positions;
  int rot_dim;
  int neox;
} isb_norm_rope;

/*
 * isb_write_cache - store the new tokens of a step into the paged caches.
 *
 * The cache write in front of the decode (ROCm/ATOM PR 2962, the commit
 * messages under Follow-ups: one fused kernel encodes K, V and the index key
 * directly in the MXFP4 / fp8 page format; a layer whose selection comes from
 * an earlier layer keeps no index keys of its own).  Token t = r q + i is stored at position
 * p = seq_lens[r] - q + i of request r (seq_lens count the new tokens), in
 * block block_table[r][p div 128], slot p mod 128; tokens with p < 0 (pad
 * requests) are skipped.  Encodings:
 *   ISB_FP8_E4M3  the e4m3fn code of x / scale (the quotient formed in fp32),
 *                 rounded to nearest with ties to the even code, magnitudes
 *                 above 448 saturated, NaN stored as 0x7F, the sign kept;
 *   ISB_MXFP4     per 32 dims an e8m0 exponent floor(log2 amax) - 2, clamped to
 *                 [-127, 127] (-127 for an all-zero group), and each element's
 *                 e2m1 code of x / 2^exponent, rounded to nearest with ties to
 *                 the even code, saturated at 6 (OCP MX v1.0);
 *   ISB_BF16      the value as given.
 * Only the bytes of the written tokens change.  K (every KV head) and the
 * index key first take the QK-norm and rope of k_norm_rope / idx_norm_rope at
 * the token's position (see isb_norm_rope; NULL = stored as given); V is
 * stored as given.  With a transform, a bf16 pool takes the fp32 result
 * rounded to nearest even.
 *
 *   k_new, v_new  [T][num_kv_heads][128] bf16, 4-byte aligned
 *   idx_new       [T][128] bf16, or NULL (then idx_pool must be NULL too and
 *                 the index arguments are ignored)
 *   block_table   [num_reqs][block_table_stride] int32 block ids
 *   seq_lens      [num_reqs] int32
 *   k_pool, v_pool  in/out, [num_pages][num_kv_heads] pages of kv_dtype
 *                 (layout above: a bf16 / fp8 block is pages 8 b .. 8 b + 7);
 *                 k_scale / v_scale > 0 for fp8
 *   idx_pool      in/out, [idx_pool_blocks] index pages of idx_dtype;
 *                 idx_scale > 0 for fp8
 * Positions past the table (p div 128 >= block_table_stride), positions at
 * or past a given rope table's rope_positions, and block ids whose pages fall
 * outside the pools are skipped, never written.  Calls that
 * write the same slot must not overlap in time.  Shape errors: num_kv_heads >
 * 65535, num_reqs * decode_query_len > 2^31 - 1.
 */
ISB_API int isb_write_cache(isb_stream_t stream, const void* k_new, const void* v_new,
                            const void* idx_new, const int32_t* block_table,
                            int block_table_stride, const int32_t* seq_lens, int num_reqs,
                            int decode_query_len, int num_kv_heads, void* k_pool, void* v_pool,
                            int kv_dtype, float k_scale, float v_scale, int64_t num_pages,
                            void* idx_pool, int idx_dtype, float idx_scale,
                            int64_t idx_pool_blocks, const isb_norm_rope* k_norm_rope,
                            const isb_norm_rope* idx_norm_rope);

/*
 * isb_quantize_e4m3 - out[i] = the e4m3fn code of x[i] with a unit scale
 * (rounding and saturation as ISB_FP8_E4M3 of isb_write_cache), for n bf16
 * elements.  The query cast of the same fused writer (ROCm/ATOM PR 2962,
 * Follow-ups: it emits the attention query, and on request the index query,
 * in float8_e4m3fn, scale 1, clamped at the format's maximum); its output is a valid
 * ISB_FP8_E4M3 query for isb_index_score and isb_sparse_pa_decode.
 */
ISB_API int isb_quantize_e4m3(isb_stream_t stream, const void* x, int64_t n, void* out);

/*
 * isb_prepare_query - the query side of the fused writer: each head vector of
 * q [T][num_heads][128] bf16 (T = num_reqs * decode_query_len, token t = r q + i
 * at position seq_lens[r] - q + i) takes the QK-norm and rope of norm_rope
 * (NULL: none) and is written to out [T][num_heads][128] as bf16 (rounded to
 * nearest even) or, with out_dtype ISB_FP8_E4M3, as the unit-scale e4m3 cast
 * of isb_quantize_e4m3 (ROCm/ATOM PR 2962, Follow-ups: the fused writer emits
 * the attention query in e4m3, and the index query on request).  Rows of pad tokens
 * (position < 0) are written as zeros, rows at or past rope_positions as NaN.
 * q and out 4-byte aligned.  Shape errors: num_heads > 65535,
 * num_reqs * decode_query_len > 2^31 - 1.
 */
ISB_API int isb_prepare_query(isb_stream_t stream, const void* q, int num_heads,
                              const int32_t* seq_lens, int num_reqs, int decode_query_len,
                              const isb_norm_rope* norm_rope, int out_dtype, void* out);

#ifdef __cplusplus
}
#endif

#endif /* ISB_H */
