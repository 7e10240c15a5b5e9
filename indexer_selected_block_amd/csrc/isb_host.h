// Host-side helpers shared by the C-ABI entry points: status codes, argument
// checks and launch-error mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "isb.h"

namespace isb {

inline hipStream_t as_hip(isb_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

inline bool is_pool_dtype(int d) { return d == ISB_BF16 || d == ISB_FP8_E4M3 || d == ISB_MXFP4; }
inline bool is_query_dtype(int d) { return d == ISB_BF16 || d == ISB_FP8_E4M3; }

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? ISB_OK : ISB_E_LAUNCH;
}

inline int64_t idx_page_bytes(int dt) {
  return dt == ISB_BF16 ? 32768 : dt == ISB_FP8_E4M3 ? 16384 : 8704;
}

// Split-K plan of isb_sparse_pa_decode; shared by the workspace query so the
// two always agree.  A split is one workgroup of four waves; a wave attends a
// run of `pages_per_wave` consecutive pages whose loads it issues at once:
// 8 fp8 / 4 bf16 16-token pages (32 KiB of K and V), or one 128-token MXFP4
// page.  Decode launches are latency-bound, so a wave takes the largest run
// its registers hold: fewer, fuller waves and fewer partials to merge.
struct PaPlan {
  int rows;             // num_tokens * num_kv_heads
  int max_pages;        // sparse_bt_stride
  int pages_per_wave;   // run of one wave
  int pages_per_split;  // pages one workgroup attends
  int splits;           // workgroups per row
};

inline PaPlan pa_plan(int num_tokens, int num_kv_heads, int sparse_bt_stride, int kv_dtype) {
  PaPlan p;
  p.rows = num_tokens * num_kv_heads;
  p.max_pages = sparse_bt_stride;
  p.pages_per_wave = kv_dtype == ISB_MXFP4 ? 1 : kv_dtype == ISB_BF16 ? 4 : 8;
  p.pages_per_split = 4 * p.pages_per_wave;
  p.splits = (p.max_pages + p.pages_per_split - 1) / p.pages_per_split;
  if (p.splits < 1) p.splits = 1;
  return p;
}

// Workspace: one arrival counter per row (padded to 256 B), then the partial
// results per (row, split): 16 heads x 128 dims fp32, then 16 x (m, l).
constexpr size_t kPartialO = 16 * 128;
constexpr size_t kPartialML = 16 * 2;

inline size_t pa_arrival_bytes(const PaPlan& p) { return ((size_t)p.rows * 4 + 255) / 256 * 256; }

inline size_t pa_workspace_bytes(const PaPlan& p) {
  return pa_arrival_bytes(p) + (size_t)p.rows * p.splits * (kPartialO + kPartialML) * sizeof(float);
}

// The standalone emit launch (emit.hip); the fused top-k entry point falls
// back to it for rows too wide for LDS.
int emit_launch(hipStream_t st, const int32_t* topk_idx, const int32_t* block_table,
                int block_table_stride, const int32_t* seq_lens, int num_reqs, int decode_query_len,
                int num_kv_heads, int top_k, int pages_per_block, int32_t* sparse_bt,
                int32_t* sparse_ctx);

}  // namespace isb
