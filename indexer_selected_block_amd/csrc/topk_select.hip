// isb_topk_select: per (KV head, token) row, the tail block plus the top_k - 1
// best earlier blocks, written ascending.
//
// ROCm/ATOM PR 2962 (decode commit: the tail page is always selected; Pad-row
// fix: a row of causal length 0 computes nothing) fixes the tail rule and the
// clamp; ties go to the lower block index.
//
// One workgroup selects one row by radix select on order-preserving 32-bit
// keys: four 8-bit passes build a 256-bin LDS histogram of the keys that match
// the prefix found so far, and one wave-scanned pass over the bins finds the
// digit where the count of larger keys reaches top_k - 1.  The threshold key
// is then exact; keys above it are taken, and keys equal to it are taken in
// block-index order until the count is met (a block-wide prefix count).  The
// selected indices are compacted in index order, which gives the ascending
// output without a sort.
#include "isb_device.h"
#include "isb_host.h"

namespace isb {

constexpr int kTopkThreads = 256;

// Order-preserving key: larger score -> larger key; -0.0 == +0.0; every NaN
// maps to 0, below -inf (0x007FFFFF).
__device__ __forceinline__ uint32_t order_key(float s) {
  if (s != s) return 0u;
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 256 threads of the workgroup.
__device__ __forceinline__ int block_incl_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w) {
    const int c = s_wave[w];
    before += w < wave ? c : 0;
    all += c;
  }
  __syncthreads();
  if (total) *total = all;
  return x + before;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores,
                                                            const int32_t* __restrict__ seq_lens,
                                                            int q_len, int T, int MB, int K,
                                                            int32_t* __restrict__ out) {
  __shared__ int s_hist[256];
  __shared__ int s_wave[kTopkThreads / 64];
  __shared__ int s_pick[2];
  const int tid = threadIdx.x;
  const int row = blockIdx.x;          // g * T + t
  const int t = row % T;
  const int r = t / q_len, i = t % q_len;
  int Lt = seq_lens[r] - (q_len - 1 - i);
  Lt = Lt > 0 ? Lt : 0;
  // n_t never exceeds the score row (callers keep seq_lens <= 128 max_blocks)
  const int nt = min((Lt + kBlockTokens - 1) / kBlockTokens, MB);
  int32_t* o = out + (size_t)row * K;
  const float* s = scores + (size_t)row * MB;
  const int W = nt - 1;                 // candidates [0, W); block W is the tail
  if (nt == 0 || W <= K - 1) {
    for (int j = tid; j < K; j += kTopkThreads) o[j] = j < nt ? j : -1;
    return;
  }
  int need = K - 1;
  uint32_t prefix = 0u, pmask = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    s_hist[tid] = 0;
    __syncthreads();
    for (int j = tid; j < W; j += kTopkThreads) {
      const uint32_t k = order_key(s[j]);
      if ((k & pmask) == prefix) atomicAdd(&s_hist[(k >> shift) & 0xFF], 1);
    }
    __syncthreads();
    // thread x holds bin 255 - x, so the inclusive scan counts keys >= that bin.
    const int c = s_hist[255 - tid];
    const int incl = block_incl_scan(c, s_wave, nullptr);
    if (incl - c < need && need <= incl) {
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
  const int chunk = (W + kTopkThreads - 1) / kTopkThreads;
  const int j0 = tid * chunk;
  const int j1 = min(W, j0 + chunk);
  int eq = 0;
  for (int j = j0; j < j1; ++j) eq += order_key(s[j]) == prefix;
  const int eq_before = block_incl_scan(eq, s_wave, nullptr) - eq;
  int take = 0, seen = eq_before;
  for (int j = j0; j < j1; ++j) {
    const uint32_t k = order_key(s[j]);
    if (k > prefix) ++take;
    else if (k == prefix) take += (seen++ < need);
  }
  int pos = block_incl_scan(take, s_wave, nullptr) - take;
  seen = eq_before;
  for (int j = j0; j < j1; ++j) {
    const uint32_t k = order_key(s[j]);
    bool sel = k > prefix;
    if (k == prefix) sel = seen++ < need;
    if (sel && pos < K - 1) o[pos++] = j;
  }
  if (tid == 0) o[K - 1] = W;           // the tail block, larger than every candidate
}

}  // namespace isb

extern "C" int isb_topk_select(isb_stream_t stream, const float* scores, const int32_t* seq_lens,
                               int num_reqs, int decode_query_len, int num_kv_heads,
                               int max_blocks, int top_k, int32_t* topk_idx) {
  using namespace isb;
  if (!scores || !seq_lens || !topk_idx) return ISB_E_INVALID_ARG;
  if (num_reqs <= 0 || decode_query_len <= 0 || num_kv_heads <= 0 || max_blocks <= 0)
    return ISB_E_INVALID_ARG;
  if (top_k < 1 || top_k > max_blocks || max_blocks > (1 << 20)) return ISB_E_SHAPE;
  const int T = num_reqs * decode_query_len;
  const long long rows = (long long)T * num_kv_heads;
  if (rows > 0x7FFFFFFFLL) return ISB_E_SHAPE;
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)rows), dim3(kTopkThreads), 0, as_hip(stream),
                     scores, seq_lens, decode_query_len, T, max_blocks, top_k, topk_idx);
  return launch_status();
}
