// isb_topk_select: per (KV head, token) row, the tail block plus the top_k - 1
// best earlier blocks, written ascending.  isb_topk_select_emit does the same
// and also writes the sparse page table of the selection (the work of
// isb_emit_sparse_block_table) from the same workgroup.
//
// ROCm/ATOM PR 2962 fixes the tail rule (the decode commit keeps the tail page
// in every selection) and the clamp (the pad-row fix: a row of causal length 0
// computes nothing); ties go to the lower block index.
//
// One workgroup selects one row by radix select on order-preserving 32-bit
// keys: four 8-bit passes build a 256-bin histogram of the keys that match
// the prefix found so far, and one scan over the bins finds the digit where
// the count of larger keys reaches top_k - 1.  The threshold key is then
// exact; keys above it are taken, and keys equal to it are taken in
// block-index order until the count is met (a block-wide prefix count).  The
// selected indices are compacted in index order, which gives the ascending
// output without a sort.
//
// Rows of up to 8192 blocks are read from HBM once, into registers, together
// with the row's length (and, for the fused emit on rows of up to 2048
// blocks, its block-table row, into LDS; wider rows read only the selected
// entries of it, after the selection).  Wider rows use the same algorithm
// over global memory.
#include "isb_device.h"
#include "isb_host.h"
#include "select_device.h"

namespace isb {

struct TopkArgs {
  const float* scores;
  TokenMap tm;
  const int32_t* bt;  // fused emit only
  int32_t* topk;
  int32_t* sbt;       // fused emit only
  int32_t* sctx;      // fused emit only
  int T, MB, K, H_kv, bt_stride, ppb;
};

// Causal geometry of topk row `row` (= g * T + t).
struct RowGeom {
  int g, t, r, Lt, nt;
};
__device__ __forceinline__ RowGeom row_geom(const TopkArgs& a, int row) {
  RowGeom q;
  q.g = row / a.T;
  q.t = row % a.T;
  const TokenPos tp = token_pos(a.tm, q.t);
  q.r = tp.r;
  q.Lt = tp.L;
  // n_t never exceeds the score row (decode callers keep seq_lens <= 128
  // max_blocks; prefill positions past it are empty rows)
  q.nt = min((q.Lt + kBlockTokens - 1) / kBlockTokens, a.MB);
  return q;
}

// Selects the row whose keys KEY(j), j < W, are given; writes the K - 1
// chosen candidates ascending through put(pos, j).  need = K - 1 < W.
template <int NT, typename KeyFn, typename PutFn>
__device__ __forceinline__ void radix_select(int W, int need, KeyFn key, PutFn put, int* s_hist,
                                             int* s_wave, int* s_pick) {
  const int tid = threadIdx.x;
  const int keep = need;
  uint32_t prefix = 0u, pmask = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int x = tid; x < 256; x += NT) s_hist[x] = 0;
    __syncthreads();
    for (int j = tid; j < W; j += NT) {
      const uint32_t k = key(j);
      if ((k & pmask) == prefix) atomicAdd(&s_hist[(k >> shift) & 0xFF], 1);
    }
    __syncthreads();
    // thread x < 256 holds bin 255 - x, so the inclusive scan counts keys >= that bin.
    const int c = tid < 256 ? s_hist[255 - tid] : 0;
    const int incl = block_incl_scan<NT>(c, s_wave);
    if (tid < 256 && incl - c < need && need <= incl) {
      s_pick[0] = 255 - tid;
      s_pick[1] = incl - c;
    }
    __syncthreads();
    prefix |= (uint32_t)s_pick[0] << shift;
    pmask |= 0xFFu << shift;
    need -= s_pick[1];
    __syncthreads();
  }
  // prefix is the exact threshold key; `need` keys equal to it are taken, the
  // lowest block indices first.
  const int chunk = (W + NT - 1) / NT;
  const int j0 = tid * chunk;
  const int j1 = min(W, j0 + chunk);
  int eq = 0;
  for (int j = j0; j < j1; ++j) eq += key(j) == prefix;
  const int eq_before = block_incl_scan<NT>(eq, s_wave) - eq;
  int take = 0, seen = eq_before;
  for (int j = j0; j < j1; ++j) {
    const uint32_t k = key(j);
    if (k > prefix) ++take;
    else if (k == prefix) take += (seen++ < need);
  }
  int pos = block_incl_scan<NT>(take, s_wave) - take;
  seen = eq_before;
  for (int j = j0; j < j1; ++j) {
    const uint32_t k = key(j);
    bool sel = k > prefix;
    if (k == prefix) sel = seen++ < need;
    if (sel && pos < keep) put(pos++, j);
  }
}

// Rows of up to 8192 blocks: NT threads, E keys each in registers (thread t
// owns blocks E t .. E t + E - 1, so the compaction is in block order).  Each
// radix pass: every wave builds its own 256-bin histogram (no contention
// between waves), wave 0 sums the waves' bins and finds the digit, two
// barriers a pass.  Dynamic LDS: (BT_LDS) the block-table row [MB], then
// (EMIT) the selection [K].
template <int NT, int E, bool EMIT, bool BT_LDS, bool VEC>
__global__ __launch_bounds__(NT) void topk_reg_kernel(TopkArgs a) {
  extern __shared__ int32_t s_dyn[];
  __shared__ SelectLds<NT> sl;
  int32_t* s_bt = s_dyn;
  int32_t* s_sel = s_dyn + (BT_LDS ? a.MB : 0);
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  // Every global load first: length, scores and (fused, narrow rows) the
  // block-table row, so the workgroup waits for one round trip.
  const RowGeom q = row_geom(a, row);
  const float* s = a.scores + (size_t)row * a.MB;
  float sc[E];
  int32_t btv[E];
  load_run<E, VEC>(s, E * tid, a.MB, sc);
  if constexpr (BT_LDS) load_run<E, VEC>(a.bt + (size_t)q.r * a.bt_stride, E * tid, a.MB, btv);
  if constexpr (BT_LDS) {
#pragma unroll
    for (int i = 0; i < E; ++i)
      if (E * tid + i < a.MB) s_bt[E * tid + i] = btv[i];
  }
  int32_t* o = a.topk + (size_t)row * a.K;
  const int m = select_row<NT, E>(sc, q.nt, a.K, sl, [&](int k, int b) {
    o[k] = b;
    if constexpr (EMIT) s_sel[k] = b;
  });
  if constexpr (EMIT) {
    __syncthreads();
    const int slots = a.K * a.ppb;
    const int erow = q.t * a.H_kv + q.g;
    int32_t* so = a.sbt + (size_t)erow * slots;
    for (int x = tid; x < slots; x += NT) {
      const int kk = x / a.ppb, p = x % a.ppb;
      int32_t page = -1;
      if (kk < m) {
        const int b = s_sel[kk];
        const int32_t blk = BT_LDS ? s_bt[b] : a.bt[(size_t)q.r * a.bt_stride + b];
        page = blk * a.ppb + p;
      }
      so[x] = page;
    }
    if (tid == 0) a.sctx[erow] = m > 0 ? (m - 1) * kBlockTokens + (q.Lt - kBlockTokens * (q.nt - 1)) : 0;
  }
}

// Rows wider than LDS holds: the same selection over global memory.
__global__ __launch_bounds__(256) void topk_global_kernel(TopkArgs a) {
  __shared__ int s_hist[256];
  __shared__ int s_wave[4];
  __shared__ int s_pick[2];
  const int row = blockIdx.x;
  const RowGeom q = row_geom(a, row);
  int32_t* o = a.topk + (size_t)row * a.K;
  const float* s = a.scores + (size_t)row * a.MB;
  const int W = q.nt - 1;
  if (q.nt == 0 || W <= a.K - 1) {
    for (int j = threadIdx.x; j < a.K; j += 256) o[j] = j < q.nt ? j : -1;
    return;
  }
  radix_select<256>(
      W, a.K - 1, [&](int j) { return order_key(s[j]); }, [&](int pos, int j) { o[pos] = j; }, s_hist,
      s_wave, s_pick);
  if (threadIdx.x == 0) o[a.K - 1] = W;
}

// Widest rows whose block-table row the fused top-k + emit reads up front.
constexpr int kBtLdsMaxBlocks = 2048;

// Dynamic LDS of topk_reg_kernel, or 0 when the row does not fit.
inline size_t topk_lds_bytes(int MB, int K, bool emit, bool bt_lds) {
  if (MB > 8192) return 0;
  const size_t b = 4 * ((bt_lds ? (size_t)MB : 0) + (emit ? (size_t)K : 0));
  return b <= 40 * 1024 ? (b ? b : 4) : 0;
}

template <bool EMIT, bool BT_LDS, bool VEC>
static void launch_reg_v(const TopkArgs& a, unsigned rows, size_t lds, hipStream_t st) {
  const dim3 g(rows);
  if (a.MB <= 256)
    hipLaunchKernelGGL((topk_reg_kernel<256, 1, EMIT, BT_LDS, VEC>), g, dim3(256), lds, st, a);
  else if (a.MB <= 512)
    hipLaunchKernelGGL((topk_reg_kernel<256, 2, EMIT, BT_LDS, VEC>), g, dim3(256), lds, st, a);
  else if (a.MB <= 1024)
    hipLaunchKernelGGL((topk_reg_kernel<256, 4, EMIT, BT_LDS, VEC>), g, dim3(256), lds, st, a);
  else if (a.MB <= 2048)
    hipLaunchKernelGGL((topk_reg_kernel<256, 8, EMIT, BT_LDS, VEC>), g, dim3(256), lds, st, a);
  else if (a.MB <= 4096)
    hipLaunchKernelGGL((topk_reg_kernel<1024, 4, EMIT, BT_LDS, VEC>), g, dim3(1024), lds, st, a);
  else
    hipLaunchKernelGGL((topk_reg_kernel<1024, 8, EMIT, BT_LDS, VEC>), g, dim3(1024), lds, st, a);
}

template <bool EMIT, bool BT_LDS>
static void launch_reg(const TopkArgs& a, unsigned rows, size_t lds, hipStream_t st) {
  const bool vec = a.MB % 4 == 0 && reinterpret_cast<uintptr_t>(a.scores) % 16 == 0 &&
                   (!BT_LDS || (a.bt_stride % 4 == 0 && reinterpret_cast<uintptr_t>(a.bt) % 16 == 0));
  if (vec)
    launch_reg_v<EMIT, BT_LDS, true>(a, rows, lds, st);
  else
    launch_reg_v<EMIT, BT_LDS, false>(a, rows, lds, st);
}

// Shared argument checks of the entry points; 0 or an ISB_E_* code.
static int check_topk(const float* scores, int32_t* topk_idx, long long num_tokens, int num_kv_heads,
                      int max_blocks, int top_k) {
  if (!scores || !topk_idx) return ISB_E_INVALID_ARG;
  if (num_tokens <= 0 || num_kv_heads <= 0 || max_blocks <= 0) return ISB_E_INVALID_ARG;
  if (top_k < 1 || top_k > max_blocks || max_blocks > (1 << 20)) return ISB_E_SHAPE;
  if (num_tokens * num_kv_heads > 0x7FFFFFFFLL) return ISB_E_SHAPE;
  return ISB_OK;
}

static int topk_select_run(hipStream_t st, const float* scores, const TokenMap& tm, int T, int num_kv_heads,
                           int max_blocks, int top_k, int32_t* topk_idx) {
  TopkArgs a{scores, tm, nullptr, topk_idx, nullptr, nullptr, T, max_blocks, top_k, num_kv_heads, 0, 0};
  const unsigned rows = (unsigned)((long long)T * num_kv_heads);
  const size_t lds = topk_lds_bytes(max_blocks, top_k, false, false);
  if (lds)
    launch_reg<false, false>(a, rows, lds, st);
  else
    hipLaunchKernelGGL(topk_global_kernel, dim3(rows), dim3(256), 0, st, a);
  return launch_status();
}

int topk_select_emit_run(hipStream_t st, const float* scores, const TokenMap& tm, int T,
                                int num_kv_heads, int max_blocks, int top_k, const int32_t* block_table,
                                int block_table_stride, int pages_per_block, int32_t* topk_idx,
                                int32_t* sparse_bt, int32_t* sparse_ctx) {
  if (!block_table || !sparse_bt || !sparse_ctx) return ISB_E_INVALID_ARG;
  if (block_table_stride <= 0) return ISB_E_INVALID_ARG;
  if (pages_per_block != 1 && pages_per_block != 8) return ISB_E_SHAPE;
  if (max_blocks > block_table_stride) return ISB_E_SHAPE;
  const long long slots = (long long)T * num_kv_heads * top_k * pages_per_block;
  if (slots > 0x7FFFFFFFLL) return ISB_E_SHAPE;
  TopkArgs a{scores, tm, block_table, topk_idx, sparse_bt, sparse_ctx, T, max_blocks, top_k, num_kv_heads,
             block_table_stride, pages_per_block};
  const unsigned rows = (unsigned)((long long)T * num_kv_heads);
  // The block-table row rides along with the scores when it is small; a wide
  // row's table would double what each workgroup reads before it can select,
  // so there only the selected blocks' entries are read, after the selection.
  size_t lds = max_blocks <= kBtLdsMaxBlocks ? topk_lds_bytes(max_blocks, top_k, true, true) : 0;
  if (lds) {
    launch_reg<true, true>(a, rows, lds, st);
  } else if ((lds = topk_lds_bytes(max_blocks, top_k, true, false)) != 0) {
    launch_reg<true, false>(a, rows, lds, st);
  } else {
    hipLaunchKernelGGL(topk_global_kernel, dim3(rows), dim3(256), 0, st, a);
    const int e = launch_status();
    if (e) return e;
    return emit_launch(st, topk_idx, block_table, block_table_stride, tm, T, num_kv_heads, top_k,
                       pages_per_block, sparse_bt, sparse_ctx);
  }
  return launch_status();
}

}  // namespace isb

extern "C" int isb_topk_select(isb_stream_t stream, const float* scores, const int32_t* seq_lens,
                               int num_reqs, int decode_query_len, int num_kv_heads,
                               int max_blocks, int top_k, int32_t* topk_idx) {
  using namespace isb;
  if (!seq_lens || num_reqs <= 0 || decode_query_len <= 0) return ISB_E_INVALID_ARG;
  const long long T = (long long)num_reqs * decode_query_len;
  const int err = check_topk(scores, topk_idx, T, num_kv_heads, max_blocks, top_k);
  if (err) return err;
  return topk_select_run(as_hip(stream), scores, decode_map(seq_lens, decode_query_len), (int)T, num_kv_heads,
                         max_blocks, top_k, topk_idx);
}

extern "C" int isb_topk_select_prefill(isb_stream_t stream, const float* scores, int num_reqs,
                                       const int32_t* query_req_id, const int32_t* query_abs_pos,
                                       int num_tokens, int num_kv_heads, int max_blocks, int top_k,
                                       int32_t* topk_idx) {
  using namespace isb;
  if (!query_req_id || !query_abs_pos || num_reqs <= 0) return ISB_E_INVALID_ARG;
  const int err = check_topk(scores, topk_idx, num_tokens, num_kv_heads, max_blocks, top_k);
  if (err) return err;
  return topk_select_run(as_hip(stream), scores, prefill_map(query_req_id, query_abs_pos, num_reqs, max_blocks),
                         num_tokens, num_kv_heads, max_blocks, top_k, topk_idx);
}

extern "C" int isb_topk_select_emit(isb_stream_t stream, const float* scores,
                                    const int32_t* seq_lens, int num_reqs, int decode_query_len,
                                    int num_kv_heads, int max_blocks, int top_k,
                                    const int32_t* block_table, int block_table_stride,
                                    int pages_per_block, int32_t* topk_idx, int32_t* sparse_bt,
                                    int32_t* sparse_ctx) {
  using namespace isb;
  if (!seq_lens || num_reqs <= 0 || decode_query_len <= 0) return ISB_E_INVALID_ARG;
  const long long T = (long long)num_reqs * decode_query_len;
  const int err = check_topk(scores, topk_idx, T, num_kv_heads, max_blocks, top_k);
  if (err) return err;
  return topk_select_emit_run(as_hip(stream), scores, decode_map(seq_lens, decode_query_len), (int)T,
                              num_kv_heads, max_blocks, top_k, block_table, block_table_stride, pages_per_block,
                              topk_idx, sparse_bt, sparse_ctx);
}

extern "C" int isb_topk_select_emit_prefill(isb_stream_t stream, const float* scores, int num_reqs,
                                            const int32_t* query_req_id, const int32_t* query_abs_pos,
                                            int num_tokens, int num_kv_heads, int max_blocks, int top_k,
                                            const int32_t* block_table, int block_table_stride,
                                            int pages_per_block, int32_t* topk_idx, int32_t* sparse_bt,
                                            int32_t* sparse_ctx) {
  using namespace isb;
  if (!query_req_id || !query_abs_pos || num_reqs <= 0) return ISB_E_INVALID_ARG;
  const int err = check_topk(scores, topk_idx, num_tokens, num_kv_heads, max_blocks, top_k);
  if (err) return err;
  return topk_select_emit_run(as_hip(stream), scores,
                              prefill_map(query_req_id, query_abs_pos, num_reqs, max_blocks), num_tokens,
                              num_kv_heads, max_blocks, top_k, block_table, block_table_stride, pages_per_block,
                              topk_idx, sparse_bt, sparse_ctx);
}
