// isb_emit_sparse_block_table: selected blocks -> sparse page table + lengths.
//
// The emit step of ROCm/ATOM PR 2962 (Pad-row fix: the causal length is
// clamped where it enters, so a pad row emits nothing; pages_per_block 8 for
// the page-16 cache, 1 for page-128 caches), with the row order of the vLLM API
// page's sparse_bt_buffer (one row per token and KV head, token-major).
//
// One thread per output slot; each thread finds its slot's selected block by
// a scan of the (short) top-k row, so rows with -1 holes still compact.
#include "isb_device.h"
#include "isb_host.h"

namespace isb {

__global__ __launch_bounds__(256) void emit_kernel(const int32_t* __restrict__ topk,
                                                   const int32_t* __restrict__ bt, int bt_stride,
                                                   TokenMap tm, int H_kv, int T, int K, int ppb,
                                                   int32_t* __restrict__ sbt,
                                                   int32_t* __restrict__ sctx) {
  const long long slots = (long long)K * ppb;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)T * H_kv * slots) return;
  const int row = (int)(idx / slots);
  const int slot = (int)(idx % slots);
  const int kk = slot / ppb, p = slot % ppb;
  const int t = row / H_kv, g = row % H_kv;
  const TokenPos tp = token_pos(tm, t);
  const int Lt = tp.L;
  const int nt = (Lt + kBlockTokens - 1) / kBlockTokens;
  const int32_t* sel = topk + ((size_t)g * T + t) * K;
  int m = 0, b = -1;
  for (int j = 0; j < K; ++j) {
    const int v = sel[j];
    if (v >= 0 && v < bt_stride) {
      if (m == kk) b = v;
      ++m;
    }
  }
  int32_t page = -1;
  if (nt > 0 && b >= 0) page = bt[(size_t)tp.r * bt_stride + b] * ppb + p;
  sbt[(size_t)row * slots + slot] = page;
  if (slot == 0)
    sctx[row] = (nt > 0 && m > 0) ? (m - 1) * kBlockTokens + (Lt - kBlockTokens * (nt - 1)) : 0;
}

}  // namespace isb

int isb::emit_launch(hipStream_t st, const int32_t* topk_idx, const int32_t* block_table,
                     int block_table_stride, const TokenMap& tm, int num_tokens, int num_kv_heads,
                     int top_k, int pages_per_block, int32_t* sparse_bt, int32_t* sparse_ctx) {
  using namespace isb;
  const long long total = (long long)num_tokens * num_kv_heads * top_k * pages_per_block;
  const long long blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFFLL) return ISB_E_SHAPE;
  hipLaunchKernelGGL(emit_kernel, dim3((unsigned)blocks), dim3(256), 0, st, topk_idx, block_table,
                     block_table_stride, tm, num_kv_heads, num_tokens, top_k, pages_per_block, sparse_bt,
                     sparse_ctx);
  return launch_status();
}

extern "C" int isb_emit_sparse_block_table(isb_stream_t stream, const int32_t* topk_idx,
                                           const int32_t* block_table, int block_table_stride,
                                           const int32_t* seq_lens, int num_reqs,
                                           int decode_query_len, int num_kv_heads, int top_k,
                                           int pages_per_block, int32_t* sparse_bt,
                                           int32_t* sparse_ctx) {
  using namespace isb;
  if (!topk_idx || !block_table || !seq_lens || !sparse_bt || !sparse_ctx) return ISB_E_INVALID_ARG;
  if (num_reqs <= 0 || decode_query_len <= 0 || num_kv_heads <= 0 || top_k <= 0 ||
      block_table_stride <= 0)
    return ISB_E_INVALID_ARG;
  if (pages_per_block != 1 && pages_per_block != 8) return ISB_E_SHAPE;
  if ((long long)num_reqs * decode_query_len > 0x7FFFFFFFLL) return ISB_E_SHAPE;
  return emit_launch(as_hip(stream), topk_idx, block_table, block_table_stride,
                     decode_map(seq_lens, decode_query_len), num_reqs * decode_query_len, num_kv_heads,
                     top_k, pages_per_block, sparse_bt, sparse_ctx);
}

extern "C" int isb_emit_sparse_block_table_prefill(isb_stream_t stream, const int32_t* topk_idx,
                                                   const int32_t* block_table, int block_table_stride,
                                                   int num_reqs, const int32_t* query_req_id,
                                                   const int32_t* query_abs_pos, int num_tokens,
                                                   int num_kv_heads, int top_k, int pages_per_block,
                                                   int32_t* sparse_bt, int32_t* sparse_ctx) {
  using namespace isb;
  if (!topk_idx || !block_table || !query_req_id || !query_abs_pos || !sparse_bt || !sparse_ctx)
    return ISB_E_INVALID_ARG;
  if (num_reqs <= 0 || num_tokens <= 0 || num_kv_heads <= 0 || top_k <= 0 || block_table_stride <= 0)
    return ISB_E_INVALID_ARG;
  if (pages_per_block != 1 && pages_per_block != 8) return ISB_E_SHAPE;
  return emit_launch(as_hip(stream), topk_idx, block_table, block_table_stride,
                     prefill_map(query_req_id, query_abs_pos, num_reqs, block_table_stride), num_tokens,
                     num_kv_heads, top_k, pages_per_block, sparse_bt, sparse_ctx);
}
