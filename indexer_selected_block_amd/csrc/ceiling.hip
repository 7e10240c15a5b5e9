// Measurement kernels (libisb_ceiling): the page reads of the index scan and
// of the attention launch, with no arithmetic, in the same grids, split plan,
// load pattern and cache policy as the kernels they mirror (index_score.hip,
// sparse_pa.hip).  Every load a wave issues for a block or a round is in
// flight before any is used; what was read is folded into one word per block
// or per wave so that no load can be dropped.
#include "grid_maps.h"
#include "isb_ceiling.h"
#include "isb_device.h"
#include "isb_host.h"

namespace isb {
namespace {

__device__ __forceinline__ u32x2 bl8_nt(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 2));
}
__device__ __forceinline__ u32x2 bl8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

// One whole page of PB bytes (a multiple of 512): full KiB loads of 16 bytes
// a lane, then the last 512 bytes (MXFP4 scales) as 8 bytes a lane.
template <int PB>
struct PageData {
  static constexpr int NL = PB / 1024;
  static constexpr bool TAIL = PB % 1024 != 0;
  u32x4 d[NL];
  u32x2 t;
};

template <int PB, bool NT>
__device__ __forceinline__ void load_page(PageData<PB>& p, __amdgpu_buffer_rsrc_t r, int lane) {
#pragma unroll
  for (int i = 0; i < PageData<PB>::NL; ++i) p.d[i] = NT ? bl16_nt(r, 16 * lane, 1024 * i) : bl16(r, 16 * lane, 1024 * i);
  if constexpr (PageData<PB>::TAIL)
    p.t = NT ? bl8_nt(r, 8 * lane, 1024 * PageData<PB>::NL) : bl8(r, 8 * lane, 1024 * PageData<PB>::NL);
}

template <int PB>
__device__ __forceinline__ uint32_t fold_page(const PageData<PB>& p) {
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < PageData<PB>::NL; ++i) x ^= fold(p.d[i]);
  if constexpr (PageData<PB>::TAIL) x ^= p.t[0] ^ p.t[1];
  return x;
}

// ----------------------------------------------------------------- index scan
struct IdxArgs {
  const uint8_t* pool;
  const int32_t* bt;
  const int32_t* seq_lens;
  float* out;
  int64_t pool_blocks;
  int bt_stride, MB;
};

// grid (ceil(MB / (4 NB)), R): wave w of workgroup column x takes blocks
// NB (4 x' + w) .. + NB - 1 of request y, x' = the scorer's column map.
template <int PB, int NB>
__global__ __launch_bounds__(256) void index_gather_kernel(IdxArgs a) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int r = blockIdx.y;
  const int b0 = (score_column<kScoreWaves * NB>(blockIdx.x, gridDim.x, r) * kScoreWaves + wave) * NB;
  if (b0 >= a.MB) return;
  const int L = a.seq_lens[r];
  const int nr = (L + kBlockTokens - 1) / kBlockTokens;
  float* orow = a.out + (size_t)r * a.MB;
  if (b0 >= nr) {
    if (lane < NB && b0 + lane < a.MB) orow[b0 + lane] = 0.f;
    return;
  }
  int64_t blk[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const int b = b0 + n < nr ? b0 + n : b0;
    blk[n] = __builtin_amdgcn_readfirstlane(a.bt[(size_t)r * a.bt_stride + b]);
    if (blk[n] < 0 || blk[n] >= a.pool_blocks) blk[n] = 0;
  }
  PageData<PB> pg[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) load_page<PB, true>(pg[n], page_rsrc(a.pool + blk[n] * PB, PB), lane);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    uint32_t x = fold_page<PB>(pg[n]);
    x ^= __shfl_xor(x, 1);
    if (lane == 0 && b0 + n < nr && b0 + n < a.MB) orow[b0 + n] = __uint_as_float(x);
  }
}

template <int PB, int NB>
void launch_index(const IdxArgs& a, int R, hipStream_t st) {
  const int per = kScoreWaves * NB;
  hipLaunchKernelGGL((index_gather_kernel<PB, NB>), dim3((a.MB + per - 1) / per, R), dim3(256), 0, st, a);
}

// ----------------------------------------------------------------- attention
struct AttArgs {
  const uint8_t* kp;
  const uint8_t* vp;
  const int32_t* sbt;
  const int32_t* sctx;
  uint32_t* out;
  int64_t num_pages;
  int sbt_stride, H_kv, pps;
};

// 16-token pages: grid (rows, splits), NW waves; a round is NW runs of RUN
// pages, one a wave, every K page of the run then every V page issued at once
// (the attention kernel's order); page ids fetched for 64 / RUN rounds at a
// time as the attention kernel does.
template <int PB, int RUN, bool NT, int NW>
__global__ __launch_bounds__(64 * NW) void attention_gather16_kernel(AttArgs a) {
  constexpr int ROUND = NW * RUN, IDS = 64 / RUN;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int row = grid_row(blockIdx.x, gridDim.x), split = blockIdx.y;
  const int kvh = row % a.H_kv;
  const int p0 = split * a.pps;
  const int pend = min(a.sbt_stride, p0 + a.pps);
  const int32_t* pages = a.sbt + (size_t)row * a.sbt_stride;
  auto ids = [&](int r0) {
    const int pidx = p0 + (r0 + lane / RUN) * ROUND + wave * RUN + lane % RUN;
    return pidx < pend ? pages[pidx] : -1;
  };
  int my_ids = ids(0);
  const int n_tok = a.sctx[row];
  uint32_t acc = 0;
  const int npages = min((n_tok + 15) / 16, a.sbt_stride);
  const int p1 = min(npages, p0 + a.pps);
  const int nrounds = p1 > p0 ? (p1 - p0 + ROUND - 1) / ROUND : 0;
  const int64_t hstride = (int64_t)a.H_kv * PB, hoff = (int64_t)kvh * PB;
  for (int r = 0; r < nrounds; ++r) {
    if (r > 0 && r % IDS == 0) my_ids = ids(r);
    const int wb = p0 + r * ROUND + wave * RUN;
    const int cnt = max(0, min(RUN, p1 - wb));
    if (cnt == 0) continue;
    const int ibase = (r % IDS) * RUN;
    PageData<PB> k[RUN], v[RUN];
    int64_t use[RUN];
#pragma unroll
    for (int j = 0; j < RUN; ++j) {
      const int64_t id = __builtin_amdgcn_readlane(my_ids, ibase + (j < cnt ? j : 0));
      use[j] = (id >= 0 && id < a.num_pages ? id : 0) * hstride + hoff;
      load_page<PB, NT>(k[j], page_rsrc(a.kp + use[j], PB), lane);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < RUN; ++j) {
      load_page<PB, NT>(v[j], page_rsrc(a.vp + use[j], PB), lane);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < RUN; ++j)
      if (j < cnt) acc ^= fold_page<PB>(k[j]) ^ fold_page<PB>(v[j]);
  }
  acc ^= __shfl_xor(acc, 1);
  if (lane == 0) a.out[((size_t)blockIdx.y * gridDim.x + blockIdx.x) * NW + wave] = acc;
}

template <int PB, int RUN, bool NT>
void launch_gather16(const AttArgs& a, dim3 grid, int nw, hipStream_t st) {
  if (nw == 8) hipLaunchKernelGGL((attention_gather16_kernel<PB, RUN, NT, 8>), grid, dim3(512), 0, st, a);
  else hipLaunchKernelGGL((attention_gather16_kernel<PB, RUN, NT, 4>), grid, dim3(256), 0, st, a);
}

// The row_wave plan: grid (ceil(rows / 4)), wave w of workgroup x takes row
// 4 grid_row(x) + w alone and walks its runs in order, each run's loads
// issued at once as in the attention kernel.
template <int PB, int RUN, bool NT>
__global__ __launch_bounds__(256) void attention_gather16_row_kernel(AttArgs a, int rows) {
  constexpr int IDS = 64 / RUN;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int row = 4 * grid_row(blockIdx.x, gridDim.x) + wave;
  if (row >= rows) return;
  const int kvh = row % a.H_kv;
  const int32_t* pages = a.sbt + (size_t)row * a.sbt_stride;
  auto ids = [&](int r0) {
    const int pidx = r0 * RUN + lane;
    return pidx < a.sbt_stride ? pages[pidx] : -1;
  };
  int my_ids = ids(0);
  const int n_tok = a.sctx[row];
  uint32_t acc = 0;
  const int npages = min((n_tok + 15) / 16, a.sbt_stride);
  const int nruns = (npages + RUN - 1) / RUN;
  const int64_t hstride = (int64_t)a.H_kv * PB, hoff = (int64_t)kvh * PB;
  for (int r = 0; r < nruns; ++r) {
    if (r > 0 && r % IDS == 0) my_ids = ids(r);
    const int cnt = min(RUN, npages - r * RUN);
    const int ibase = (r % IDS) * RUN;
    PageData<PB> k[RUN], v[RUN];
    int64_t use[RUN];
#pragma unroll
    for (int j = 0; j < RUN; ++j) {
      const int64_t id = __builtin_amdgcn_readlane(my_ids, ibase + (j < cnt ? j : 0));
      use[j] = (id >= 0 && id < a.num_pages ? id : 0) * hstride + hoff;
      load_page<PB, NT>(k[j], page_rsrc(a.kp + use[j], PB), lane);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < RUN; ++j) {
      load_page<PB, NT>(v[j], page_rsrc(a.vp + use[j], PB), lane);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < RUN; ++j)
      if (j < cnt) acc ^= fold_page<PB>(k[j]) ^ fold_page<PB>(v[j]);
  }
  acc ^= __shfl_xor(acc, 1);
  if (lane == 0) a.out[row] = acc;
}

template <int PB, int RUN, bool NT>
void launch_gather16_rows(const AttArgs& a, int rows, hipStream_t st) {
  hipLaunchKernelGGL((attention_gather16_row_kernel<PB, RUN, NT>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                     st, a, rows);
}

// MXFP4 pages: one 8704 B page of K and one of V a wave, page p0 + wave of
// the split.
__global__ __launch_bounds__(256) void attention_gather_mx_kernel(AttArgs a) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int row = grid_row(blockIdx.x, gridDim.x), split = blockIdx.y;
  const int kvh = row % a.H_kv;
  const int p = split * a.pps + wave;
  const int n_tok = a.sctx[row];
  const int32_t id_raw = p < a.sbt_stride ? a.sbt[(size_t)row * a.sbt_stride + p] : -1;
  const int npages = min((n_tok + kBlockTokens - 1) / kBlockTokens, a.sbt_stride);
  uint32_t acc = 0;
  if (p < npages) {
    const int64_t id = __builtin_amdgcn_readfirstlane(id_raw);
    const int64_t pg = ((id >= 0 && id < a.num_pages ? id : 0) * a.H_kv + kvh) * kMxPageBytes;
    PageData<kMxPageBytes> k, v;
    load_page<kMxPageBytes, false>(k, page_rsrc(a.kp + pg, kMxPageBytes), lane);
    load_page<kMxPageBytes, false>(v, page_rsrc(a.vp + pg, kMxPageBytes), lane);
    __builtin_amdgcn_sched_barrier(0);
    acc = fold_page<kMxPageBytes>(k) ^ fold_page<kMxPageBytes>(v);
  }
  acc ^= __shfl_xor(acc, 1);
  if (lane == 0) a.out[((size_t)blockIdx.y * gridDim.x + blockIdx.x) * 4 + wave] = acc;
}

}  // namespace
}  // namespace isb

extern "C" int isb_ceiling_index_gather(isb_stream_t stream, const void* idx_pool, int idx_dtype,
                                        int64_t idx_pool_blocks, const int32_t* block_table,
                                        int block_table_stride, const int32_t* seq_lens, int num_reqs,
                                        int decode_query_len, int num_idx_heads, int max_blocks, float* out) {
  using namespace isb;
  if (!idx_pool || !block_table || !seq_lens || !out) return ISB_E_INVALID_ARG;
  if (idx_pool_blocks <= 0 || block_table_stride <= 0 || num_reqs <= 0 || decode_query_len <= 0 ||
      num_idx_heads <= 0 || max_blocks <= 0)
    return ISB_E_INVALID_ARG;
  if (!is_pool_dtype(idx_dtype)) return ISB_E_UNSUPPORTED_DTYPE;
  if (max_blocks > block_table_stride || num_reqs > 65535) return ISB_E_SHAPE;
  if (decode_query_len > 16 || (long long)decode_query_len * num_idx_heads > 64) return ISB_E_SHAPE;
  IdxArgs a{(const uint8_t*)idx_pool, block_table, seq_lens, out, idx_pool_blocks, block_table_stride, max_blocks};
  hipStream_t st = as_hip(stream);
  const bool one_row = decode_query_len * num_idx_heads == 1;
  if (idx_dtype == ISB_FP8_E4M3) {
    if (one_row) launch_index<16384, 2>(a, num_reqs, st);
    else launch_index<16384, 1>(a, num_reqs, st);
  } else if (idx_dtype == ISB_BF16) {
    launch_index<32768, 1>(a, num_reqs, st);
  } else {
    launch_index<kMxPageBytes, 1>(a, num_reqs, st);
  }
  return launch_status();
}

extern "C" size_t isb_ceiling_attention_words(int num_tokens, int num_kv_heads, int sparse_bt_stride,
                                              int kv_dtype) {
  using namespace isb;
  if (num_tokens <= 0 || num_kv_heads <= 0 || sparse_bt_stride <= 0 || !is_pool_dtype(kv_dtype)) return 0;
  const PaPlan p = pa_plan(num_tokens, num_kv_heads, sparse_bt_stride, kv_dtype);
  return p.row_wave ? (size_t)p.rows : (size_t)p.rows * p.splits * p.waves;
}

extern "C" int isb_ceiling_attention_gather(isb_stream_t stream, const void* k_pool, const void* v_pool,
                                            int kv_dtype, int64_t num_pages, const int32_t* sparse_bt,
                                            int sparse_bt_stride, const int32_t* sparse_ctx, int num_tokens,
                                            int decode_query_len, int num_kv_heads, uint32_t* out,
                                            size_t out_words) {
  using namespace isb;
  if (!k_pool || !v_pool || !sparse_bt || !sparse_ctx || !out) return ISB_E_INVALID_ARG;
  if (num_pages <= 0 || sparse_bt_stride <= 0 || num_tokens <= 0 || decode_query_len <= 0 || num_kv_heads <= 0)
    return ISB_E_INVALID_ARG;
  if (!is_pool_dtype(kv_dtype)) return ISB_E_UNSUPPORTED_DTYPE;
  if (num_tokens % decode_query_len != 0 || (long long)num_tokens * num_kv_heads > 0x7FFFFFFFLL) return ISB_E_SHAPE;
  const PaPlan p = pa_plan(num_tokens, num_kv_heads, sparse_bt_stride, kv_dtype);
  if (p.splits > 65535) return ISB_E_SHAPE;
  if (out_words < (p.row_wave ? (size_t)p.rows : (size_t)p.rows * p.splits * p.waves)) return ISB_E_WORKSPACE;
  AttArgs a{(const uint8_t*)k_pool, (const uint8_t*)v_pool, sparse_bt, sparse_ctx, out, num_pages, sparse_bt_stride,
            num_kv_heads, p.pages_per_split};
  hipStream_t st = as_hip(stream);
  const dim3 grid((unsigned)p.rows, p.splits);
  const bool nt = decode_query_len == 1;
  if (p.row_wave) {  // 16-token pages only
    if (kv_dtype == ISB_FP8_E4M3) {
      if (nt) launch_gather16_rows<2048, 8, true>(a, p.rows, st);
      else launch_gather16_rows<2048, 8, false>(a, p.rows, st);
    } else {
      if (nt) launch_gather16_rows<4096, 4, true>(a, p.rows, st);
      else launch_gather16_rows<4096, 4, false>(a, p.rows, st);
    }
    return launch_status();
  }
  if (kv_dtype == ISB_MXFP4) {
    hipLaunchKernelGGL(attention_gather_mx_kernel, grid, dim3(256), 0, st, a);
  } else if (kv_dtype == ISB_FP8_E4M3) {
    if (nt) launch_gather16<2048, 8, true>(a, grid, p.waves, st);
    else launch_gather16<2048, 8, false>(a, grid, p.waves, st);
  } else {
    if (nt) launch_gather16<4096, 4, true>(a, grid, p.waves, st);
    else launch_gather16<4096, 4, false>(a, grid, p.waves, st);
  }
  return launch_status();
}
