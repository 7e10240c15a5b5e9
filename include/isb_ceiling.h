/*
 * isb_ceiling.h - measurement kernels of libisb_ceiling: the page reads of
 * the layer's two large launches with no arithmetic.
 *
 * They are the ceilings the benchmark reports beside the layer's own
 * durations: how fast the memory system delivers exactly the bytes a launch
 * reads, in the launch's own grid and load pattern.  Each kernel issues the
 * same loads, to the same pages, with the same cache policy, in the same
 * order a wave of the real kernel does, keeps every load of a wave in flight
 * before using any, and folds what it read into one word so that no load is
 * dropped.  They compute nothing of the layer.
 *
 * Arguments are those of the calls they mirror (include/isb.h); the pools,
 * tables and lengths are read-only, and `out` receives the folded words.
 * Return 0 or a negative isb_status; nothing is enqueued when a check fails.
 */
#ifndef ISB_CEILING_H
#define ISB_CEILING_H

#include <stddef.h>
#include <stdint.h>

#include "isb.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The index pages isb_index_score reads for these arguments: every block of
 * every request (blocks past a request's length read nothing), in the grid of
 * the scorer variant that the call takes for decode_query_len and
 * num_idx_heads up to 16 tokens / 64 rows (two fp8 blocks a wave for one query
 * row, one block a wave otherwise), nontemporal loads.
 *   out  [num_reqs][max_blocks] fp32: one folded word per block, as bits.
 * Shape errors: those of isb_index_score, and prefill chunks (more than 16
 * tokens or 64 rows a request).
 */
ISB_API int isb_ceiling_index_gather(isb_stream_t stream, const void* idx_pool, int idx_dtype,
                                     int64_t idx_pool_blocks, const int32_t* block_table,
                                     int block_table_stride, const int32_t* seq_lens, int num_reqs,
                                     int decode_query_len, int num_idx_heads, int max_blocks,
                                     float* out);

/*
 * The K and V pages isb_sparse_pa_decode reads for these arguments, in its
 * grid and plan (rows x splits workgroups, or one wave a row for batches of
 * many rows of 16-token pages), each wave's pages of a round issued at once,
 * with the cache policy the call takes for decode_query_len.
 *   out  >= isb_ceiling_attention_words(...) uint32 words, one per wave.
 */
ISB_API int isb_ceiling_attention_gather(isb_stream_t stream, const void* k_pool, const void* v_pool,
                                         int kv_dtype, int64_t num_pages, const int32_t* sparse_bt,
                                         int sparse_bt_stride, const int32_t* sparse_ctx,
                                         int num_tokens, int decode_query_len, int num_kv_heads,
                                         uint32_t* out, size_t out_words);

/* Words isb_ceiling_attention_gather writes for these arguments (0 if invalid). */
ISB_API size_t isb_ceiling_attention_words(int num_tokens, int num_kv_heads, int sparse_bt_stride,
                                           int kv_dtype);

#ifdef __cplusplus
}
#endif

#endif /* ISB_CEILING_H */
