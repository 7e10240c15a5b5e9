// isb_topk_merge: a row's selection from candidate (score, block id) pairs,
// the merge step of context parallelism.
//
// ROCm/ATOM PR 2962 lists a candidate exchange among the users of the emit
// helper, for context parallelism of the indexer.  When each shard of a
// row's blocks selects as if it were the whole row (its last block kept, plus
// its top_k - 1 best), every block of the row's true top_k - 1 is among the
// shards' picks: at most top_k - 2 blocks beat it in the whole row, so at most
// that many in its shard.  Taking the top_k - 1 of the gathered picks under
// the selection's own order (score descending, NaN last, -0.0 == +0.0, then
// the lower block index), excluding the row's tail, and adding the tail
// gives exactly the one-GPU selection.
//
// One workgroup a row: the row's candidates are staged in LDS; four lanes
// share a candidate, each ranking it against a quarter of the list (16-byte
// LDS reads; the quarters start 16 bytes apart modulo the bank width, so the
// four addresses a wave reads hit different banks) and two lane exchanges add
// the counts.  A chosen candidate's output slot is the number of chosen
// candidates with a lower block index, so the output is ascending without a
// sort.  Candidate counts are a few hundred (shards x top_k).
#include "isb_device.h"
#include "isb_host.h"
#include "select_device.h"

namespace isb {

constexpr int kMergeThreads = 1024;  // four lanes a candidate
constexpr int kMergeMaxCands = 1024;

struct MergeArgs {
  const float* sc;      // [rows][C]
  const int32_t* ids;   // [rows][C], -1 = empty
  const int32_t* seq_lens;
  int32_t* topk;        // [rows][K]
  int C, q_len, T, K, MB;
};

__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(MergeArgs a) {
  __shared__ alignas(16) uint32_t s_key[kMergeMaxCands];
  __shared__ alignas(16) int32_t s_id[kMergeMaxCands];
  __shared__ alignas(16) int32_t s_sel[kMergeMaxCands];
  __shared__ int s_cnt;
  const int tid = threadIdx.x;
  const int row = blockIdx.x;  // g * T + t
  const int t = row % a.T;
  const int r = t / a.q_len, i = t % a.q_len;
  int Lt = a.seq_lens[r] - (a.q_len - 1 - i);
  Lt = Lt > 0 ? Lt : 0;
  const int nt = min((Lt + kBlockTokens - 1) / kBlockTokens, a.MB);
  int32_t* o = a.topk + (size_t)row * a.K;
  const int tail = nt - 1;
  if (nt == 0 || tail <= a.K - 1) {  // every block of the row is selected
    for (int j = tid; j < a.K; j += kMergeThreads) o[j] = j < nt ? j : -1;
    return;
  }
  const float* sc = a.sc + (size_t)row * a.C;
  const int32_t* id = a.ids + (size_t)row * a.C;
  // staged up to a multiple of 4 (the padding is no candidate), so the
  // ranking loops read four entries a 16-byte LDS load
  const int C4 = (a.C + 3) & ~3;
  for (int c = tid; c < C4; c += kMergeThreads) {
    const int32_t b = c < a.C ? id[c] : -1;
    const float v = c < a.C ? sc[c] : 0.f;
    const bool ok = b >= 0 && b < tail;  // the tail is added below
    s_id[c] = ok ? b : -1;
    s_key[c] = ok ? order_key(v) : 0u;
  }
  if (tid == 0) s_cnt = 0;
  __syncthreads();
  const int need = a.K - 1;
  // quarter q of the list: entries [q Q, min(C4, (q + 1) Q)), Q a multiple of
  // 4 but not of 32, so the quarters start in four different banks
  const int q = tid & 3;
  const int Q0 = ((C4 >> 2) + 3) & ~3;
  const int Q = Q0 + ((Q0 & 31) == 0 ? 4 : 0);
  const int x0 = q * Q, x1 = min(C4, x0 + Q);
  for (int c = tid >> 2; c < C4; c += kMergeThreads >> 2) {  // the four lanes move together
    const int32_t b = s_id[c];
    const uint32_t k = s_key[c];
    int ahead = 0;  // valid candidates before this one in the selection order
#pragma unroll 4
    for (int x = x0; x < x1; x += 4) {
      const int4 bx = *reinterpret_cast<const int4*>(&s_id[x]);
      const uint4 kx = *reinterpret_cast<const uint4*>(&s_key[x]);
      ahead += (bx.x >= 0) & ((kx.x > k) | ((kx.x == k) & (bx.x < b)));
      ahead += (bx.y >= 0) & ((kx.y > k) | ((kx.y == k) & (bx.y < b)));
      ahead += (bx.z >= 0) & ((kx.z > k) | ((kx.z == k) & (bx.z < b)));
      ahead += (bx.w >= 0) & ((kx.w > k) | ((kx.w == k) & (bx.w < b)));
    }
    ahead += __shfl_xor(ahead, 1, kWave);
    ahead += __shfl_xor(ahead, 2, kWave);
    const int sel = b >= 0 && ahead < need;
    if (q == 0) {
      s_sel[c] = sel;
      if (sel) atomicAdd(&s_cnt, 1);
    }
  }
  __syncthreads();
  for (int c = tid >> 2; c < C4; c += kMergeThreads >> 2) {
    const int32_t b = s_id[c];
    int pos = 0;
#pragma unroll 4
    for (int x = x0; x < x1; x += 4) {
      const int4 sx = *reinterpret_cast<const int4*>(&s_sel[x]);
      const int4 bx = *reinterpret_cast<const int4*>(&s_id[x]);
      pos += (sx.x & (bx.x < b)) + (sx.y & (bx.y < b)) + (sx.z & (bx.z < b)) + (sx.w & (bx.w < b));
    }
    pos += __shfl_xor(pos, 1, kWave);
    pos += __shfl_xor(pos, 2, kWave);
    if (q == 0 && s_sel[c] && pos < need) o[pos] = b;
  }
  const int m = min(s_cnt, need) + 1;  // chosen candidates and the tail
  if (tid == 0) o[m - 1] = tail;
  for (int j = m + tid; j < a.K; j += kMergeThreads) o[j] = -1;
}

}  // namespace isb

extern "C" int isb_topk_merge(isb_stream_t stream, const float* cand_scores, const int32_t* cand_ids,
                              int num_cands, const int32_t* seq_lens, int num_reqs, int decode_query_len,
                              int num_kv_heads, int max_blocks, int top_k, int32_t* topk_idx) {
  using namespace isb;
  if (!cand_scores || !cand_ids || !seq_lens || !topk_idx) return ISB_E_INVALID_ARG;
  if (num_cands <= 0 || num_reqs <= 0 || decode_query_len <= 0 || num_kv_heads <= 0 || max_blocks <= 0)
    return ISB_E_INVALID_ARG;
  if (num_cands > kMergeMaxCands || top_k < 1 || top_k > max_blocks) return ISB_E_SHAPE;
  const long long rows = (long long)num_reqs * decode_query_len * num_kv_heads;
  if (rows > 0x7FFFFFFFLL) return ISB_E_SHAPE;
  MergeArgs a{cand_scores, cand_ids, seq_lens, topk_idx, num_cands, decode_query_len,
              num_reqs * decode_query_len, top_k, max_blocks};
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)rows), dim3(kMergeThreads), 0, as_hip(stream), a);
  return launch_status();
}
