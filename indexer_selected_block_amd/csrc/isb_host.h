// Host-side helpers shared by the C-ABI entry points: status codes, argument
// checks and launch-error mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "isb.h"
#include "isb_device.h"

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
// two always agree.  A wave attends a run of `pages_per_wave` consecutive
// pages whose loads it issues at once: 8 fp8 / 4 bf16 16-token pages (32 KiB
// of K and V), or one 128-token MXFP4 page; a workgroup of `waves` waves
// covers one run a wave a round.  The chip holds kPaResidentWaves such waves
// at once (two a SIMD).  When every run of the batch fits in that at once and
// eight-wave workgroups still reach a quarter of the CUs, a workgroup of fp8
// pages has eight waves (a row needs half as many splits, so half as many
// partials are merged, and the rows of a small batch, which are latency-bound,
// wait on fewer hand-offs); otherwise four.  Rows are cut into just enough
// splits to fill the chip; a split longer than one round is walked round by
// round.  Batches that fill the chip by themselves thus take one split a row,
// with nothing to merge between workgroups, and small batches spread a row
// over several workgroups that each read everything they attend in one round.
constexpr int kPaResidentWaves = 2048;  // 256 CUs x 4 SIMDs x 2 waves
constexpr int kPaCUs = 256;
// 16-token-page batches whose rows fill every round of resident waves (at
// least kPaRowWaveRows of each kPaResidentWaves) give each row one wave of its
// own (row_wave): the rows of a round are resident together, one wave walks a
// row's runs in order, and rows of one request, dealt to one die, read the
// blocks they share through its L2 while they are there.  A last round that
// is only partly full would leave most of the chip idle for a whole row's
// runs: such batches keep four waves a row.
constexpr int kPaRowWaveRows = 2048 - 64;

struct PaPlan {
  int rows;             // num_tokens * num_kv_heads
  int max_pages;        // sparse_bt_stride
  int pages_per_wave;   // run of one wave
  int waves;            // waves a workgroup: 4 or 8
  int pages_per_round;  // one run a wave: what a workgroup reads at once
  int pages_per_split;  // a whole number of rounds
  int splits;           // workgroups per row
  bool row_wave;        // one wave a row, four rows a workgroup, runs in turn
};

inline PaPlan pa_plan(int num_tokens, int num_kv_heads, int sparse_bt_stride, int kv_dtype) {
  PaPlan p;
  p.rows = num_tokens * num_kv_heads;
  p.max_pages = sparse_bt_stride;
  p.pages_per_wave = kv_dtype == ISB_MXFP4 ? 1 : kv_dtype == ISB_BF16 ? 4 : 8;
  p.waves = 4;
  const int last = p.rows % kPaResidentWaves;  // rows of the last round
  p.row_wave = kv_dtype != ISB_MXFP4 && p.rows >= kPaRowWaveRows && (last == 0 || last >= kPaRowWaveRows);
  if (p.row_wave) {
    p.pages_per_round = p.pages_per_wave;
    p.pages_per_split = p.max_pages;
    p.splits = 1;
    return p;
  }
  const long long runs = (p.max_pages + p.pages_per_wave - 1) / p.pages_per_wave;  // of a whole row
  if (kv_dtype == ISB_FP8_E4M3 && (long long)p.rows * runs <= kPaResidentWaves &&
      (long long)p.rows * ((runs + 7) / 8) >= kPaCUs / 4)
    p.waves = 8;
  p.pages_per_round = p.waves * p.pages_per_wave;
  const int rounds = (p.max_pages + p.pages_per_round - 1) / p.pages_per_round;  // of a whole row
  const int resident = kPaResidentWaves / p.waves;  // workgroups the chip holds at once
  int want = (resident + p.rows - 1) / (p.rows > 0 ? p.rows : 1);
  if (want > rounds) want = rounds;
  if (want < 1) want = 1;
  const int rounds_per_split = (rounds + want - 1) / want;
  p.pages_per_split = rounds_per_split * p.pages_per_round;
  p.splits = (p.max_pages + p.pages_per_split - 1) / p.pages_per_split;
  if (p.splits < 1) p.splits = 1;
  return p;
}

// Workspace: the partial results per (row, split): 16 heads x 128 dims fp32,
// then 16 x (m, l).  A slot is free when every word of it is zero; the
// workspace starts that way (zero-filled), and every completed call leaves it
// that way.  Rows of one split publish nothing, so a plan of one split a row
// needs none.
constexpr size_t kPartialO = 16 * 128;
constexpr size_t kPartialML = 16 * 2;

inline size_t pa_workspace_bytes(const PaPlan& p) {
  return p.splits > 1 ? (size_t)p.rows * p.splits * (kPartialO + kPartialML) * sizeof(float) : 0;
}

// Token maps (isb_device.h) of the two batch forms.  A prefill position is
// valid below 128 max_blocks (the table width the call reads), and at most
// 2^31 - 2 so that its causal length fits an int.
inline TokenMap decode_map(const int32_t* seq_lens, int q_len) {
  return TokenMap{seq_lens, nullptr, nullptr, q_len, 0, 0};
}
inline TokenMap prefill_map(const int32_t* req_id, const int32_t* abs_pos, int num_reqs, int max_blocks) {
  const long long len = 128LL * max_blocks;
  return TokenMap{nullptr, req_id, abs_pos, 1, num_reqs, len < 0x7FFFFFFFLL ? (int)len : 0x7FFFFFFF};
}

// The standalone emit launch (emit.hip); the fused top-k entry points fall
// back to it for rows too wide for LDS.
int emit_launch(hipStream_t st, const int32_t* topk_idx, const int32_t* block_table,
                int block_table_stride, const TokenMap& tm, int num_tokens, int num_kv_heads,
                int top_k, int pages_per_block, int32_t* sparse_bt, int32_t* sparse_ctx);

// Top-k and emit in one launch for either batch form (topk_select.hip);
// the select + attend entry points fall back to it for rows they cannot
// take in one launch.  Checks the emit arguments; the top-k ones are the
// caller's.
int topk_select_emit_run(hipStream_t st, const float* scores, const TokenMap& tm, int T, int num_kv_heads,
                         int max_blocks, int top_k, const int32_t* block_table, int block_table_stride,
                         int pages_per_block, int32_t* topk_idx, int32_t* sparse_bt, int32_t* sparse_ctx);

}  // namespace isb
