// isb_index_score: one score per (KV head, query token, 128-token block).
//
// The indexer of ROCm/ATOM PR 2962 ("[MiniMax-M3.1] MXFP4 index cache and
// MXFP4 KV cache", Summary and Known limits) scores every 128-token block of a
// request's paged index-key cache with the index query into an fp32
// (head, row, block) workspace.  Here a block's score for one index head is the
// largest dot product over the block's causally valid keys, and the index
// heads of a KV group are summed.
//
// One wavefront scores one block of one request against every query row of
// that request (q tokens x H_idx heads), so the block's keys cross HBM once
// however many tokens the request decodes.  Three variants:
//   * stream  - one query row (q = 1, H_idx = 1), bf16 / fp8 keys: a
//               coalesced HBM stream with packed bf16 dot products on the VALU
//               (2 flop per key byte leaves the VALU far from busy);
//   * tile    - several query rows: keys converted to bf16 in registers and
//               multiplied on v_mfma_f32_16x16x32_bf16, 16 keys x 16 rows a tile;
//   * fp4     - MXFP4 keys with an e4m3 query: v_mfma_scale_f32_16x16x128_f8f6f4
//               consumes the e2m1 data and its e8m0 scales directly, one
//               instruction per 16 keys x 16 rows x 128 dims.
#include "isb_device.h"
#include "isb_host.h"

namespace isb {

struct ScoreArgs {
  const uint8_t* q_idx;
  const uint8_t* pool;
  const int32_t* bt;
  const int32_t* seq_lens;
  float* scores;
  int64_t pool_blocks;
  float idx_scale;
  int q_dt, idx_dt, H_idx, bt_stride, R, q_len, H_kv, MB;
};

constexpr int kScoreWaves = 4;        // waves (blocks) per workgroup
constexpr int kMaxQueryRows = 64;     // q_len * H_idx

// Loads 8 consecutive dims of one query row as bf16 (exact for e4m3).
__device__ __forceinline__ bf16x8 load_q8(const uint8_t* row, int q_dt, int dim0) {
  if (q_dt == ISB_BF16) return u32x4_as_bf16x8(ld16(row + 2 * dim0));
  u32x2 w = ld8(row + dim0);
  bf16x4 a = e4m3x4_to_bf16x4(w[0]);
  bf16x4 b = e4m3x4_to_bf16x4(w[1]);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ int causal_len(int L, int q_len, int i) {
  int v = L - (q_len - 1 - i);
  return v > 0 ? v : 0;
}

// Writes -inf (or `v`) for every (token, group) of request r at block b.
__device__ __forceinline__ void write_scores(const ScoreArgs& a, int r, int b, int lane,
                                             const float* vals /* per (i,g) or null */) {
  const int T = a.R * a.q_len;
  for (int x = lane; x < a.q_len * a.H_kv; x += kWave) {
    const int i = x / a.H_kv, g = x % a.H_kv;
    const float v = vals ? vals[x] : neg_inf();
    a.scores[((size_t)g * T + (size_t)r * a.q_len + i) * a.MB + b] = v;
  }
}

// Group sums of per-row block maxima held in `rowmax[QR]` (wave-private LDS).
__device__ __forceinline__ void finish(const ScoreArgs& a, int r, int b, int lane,
                                       const float* rowmax, float* outv) {
  const int per = a.H_idx / a.H_kv;
  for (int x = lane; x < a.q_len * a.H_kv; x += kWave) {
    const int i = x / a.H_kv, g = x % a.H_kv;
    float s = 0.f;
    for (int h = 0; h < per; ++h) s += rowmax[i * a.H_idx + g * per + h];
    outv[x] = s * (a.idx_dt == ISB_FP8_E4M3 ? a.idx_scale : 1.0f);
  }
}

// ----------------------------------------------------------------- stream
// One query row.  fp8: lane l reads 16 B of key (8 i + l/8) for i < 16 (one
// coalesced KiB per instruction); bf16: 16 B of key (4 i + l/16) for i < 32.
template <int KEY_DT>
__device__ __forceinline__ float stream_block(const ScoreArgs& a, const uint8_t* page,
                                              const uint8_t* qrow, int lane, int nvalid) {
  float best = neg_inf();
  bool nan = false;
  if constexpr (KEY_DT == ISB_FP8_E4M3) {
    const int sub = lane & 7, tok0 = lane >> 3;
    bf16x8 q0 = load_q8(qrow, a.q_dt, 16 * sub);
    bf16x8 q1 = load_q8(qrow, a.q_dt, 16 * sub + 8);
    bf16x2 qv[8] = {{q0[0], q0[1]}, {q0[2], q0[3]}, {q0[4], q0[5]}, {q0[6], q0[7]},
                    {q1[0], q1[1]}, {q1[2], q1[3]}, {q1[4], q1[5]}, {q1[6], q1[7]}};
    u32x4 raw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) raw[i] = ld16(page + (8 * i + tok0) * 128 + 16 * sub);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc = __builtin_amdgcn_fdot2_f32_bf16(e4m3x2_to_bf16x2(raw[i][w], false), qv[2 * w], acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(e4m3x2_to_bf16x2(raw[i][w], true), qv[2 * w + 1], acc, false);
      }
      acc += dpp_f32<kDppXor1>(acc);
      acc += dpp_f32<kDppXor2>(acc);
      acc += dpp_f32<kDppHalfMirror>(acc);
      if (8 * i + tok0 < nvalid) {
        nan |= acc != acc;
        best = fmaxf(best, acc);
      }
    }
    best = fmaxf(best, shfl_xor_f32(best, 8));
  } else {  // bf16 keys
    const int sub = lane & 15, tok0 = lane >> 4;
    bf16x8 q0 = load_q8(qrow, a.q_dt, 8 * sub);
    bf16x2 qv[4] = {{q0[0], q0[1]}, {q0[2], q0[3]}, {q0[4], q0[5]}, {q0[6], q0[7]}};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4 raw[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) raw[i] = ld16(page + (4 * (16 * half + i) + tok0) * 256 + 16 * sub);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) acc = __builtin_amdgcn_fdot2_f32_bf16(u32_as_bf16x2(raw[i][w]), qv[w], acc, false);
        acc += dpp_f32<kDppXor1>(acc);
        acc += dpp_f32<kDppXor2>(acc);
        acc += dpp_f32<kDppHalfMirror>(acc);
        acc += dpp_f32<kDppMirror>(acc);
        if (4 * (16 * half + i) + tok0 < nvalid) {
          nan |= acc != acc;
          best = fmaxf(best, acc);
        }
      }
    }
  }
  best = max_over_groups(best);
  if (__ballot(nan)) best = qnan();
  return best;
}

// ----------------------------------------------------------------- tiles
// Block maxima for query rows [qt*16, qt*16+16) of request r, bf16 MFMA.
// Lane (m = lane & 15, g = lane >> 4) supplies key m of a 16-key tile, dims
// 32 g .. 32 g + 31, and query row m of the tile, the same dims; MFMA j
// contracts dims 32 g + 8 j .. 32 g + 8 j + 7 of every lane group.
template <int KEY_DT>
__device__ __forceinline__ float tile_block_bf16(const ScoreArgs& a, const uint8_t* page, int r,
                                                 int qt, int QR, int lane, const int* nvalid_row) {
  const int m = lane & 15, g = lane >> 4;
  const int qbytes = a.q_dt == ISB_BF16 ? 2 : 1;
  const int n = qt * 16 + m;
  bf16x8 qb[4];
  if (n < QR) {
    const int i = n / a.H_idx, h = n % a.H_idx;
    const uint8_t* qrow = a.q_idx + ((size_t)(r * a.q_len + i) * a.H_idx + h) * kHeadDim * qbytes;
#pragma unroll
    for (int j = 0; j < 4; ++j) qb[j] = load_q8(qrow, a.q_dt, 32 * g + 8 * j);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) qb[j] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
  const int nv = n < QR ? nvalid_row[n / a.H_idx] : 0;
  float best = neg_inf();
  bool nan = false;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    bf16x8 kb[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int tok = 16 * (4 * half + tt) + m;
      if constexpr (KEY_DT == ISB_BF16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) kb[tt][j] = u32x4_as_bf16x8(ld16(page + tok * 256 + 64 * g + 16 * j));
      } else if constexpr (KEY_DT == ISB_FP8_E4M3) {
        u32x4 w0 = ld16(page + tok * 128 + 32 * g);
        u32x4 w1 = ld16(page + tok * 128 + 32 * g + 16);
        uint32_t w[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x4 lo = e4m3x4_to_bf16x4(w[2 * j]);
          bf16x4 hi = e4m3x4_to_bf16x4(w[2 * j + 1]);
          kb[tt][j] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      } else {  // MXFP4 keys, bf16 query
        u32x4 w = ld16(page + tok * 64 + 16 * g);
        const float sc = e8m0_to_f32(ld4(page + kMxDataBytes + 4 * tok) >> (8 * g));
#pragma unroll
        for (int j = 0; j < 4; ++j) kb[tt][j] = e2m1x8_to_bf16x8(w[j], sc);
      }
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = mfma_16x16x32_bf16(kb[tt][j], qb[j], acc);
      // acc[e] = dot(key 16 tile + 4 g + e, query row n)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (16 * (4 * half + tt) + 4 * g + e < nv) {
          nan |= acc[e] != acc[e];
          best = fmaxf(best, acc[e]);
        }
      }
    }
  }
  best = max_over_groups(best);
  nan = (__ballot(nan) >> m & 0x0001000100010001ull) != 0;
  return nan ? qnan() : best;
}

// MXFP4 keys and an e4m3 query on the scaled MFMA: one instruction a tile.
__device__ __forceinline__ float tile_block_fp4(const ScoreArgs& a, const uint8_t* page, int r,
                                                int qt, int QR, int lane, const int* nvalid_row) {
  const int m = lane & 15, g = lane >> 4;
  const int n = qt * 16 + m;
  i32x8 qb = {0, 0, 0, 0, 0, 0, 0, 0};
  if (n < QR) {
    const int i = n / a.H_idx, h = n % a.H_idx;
    const uint8_t* qrow = a.q_idx + ((size_t)(r * a.q_len + i) * a.H_idx + h) * kHeadDim;
    u32x4 lo = ld16(qrow + 16 * g);
    u32x4 hi = ld16(qrow + 64 + 16 * g);
    qb = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  const int nv = n < QR ? nvalid_row[n / a.H_idx] : 0;
  u32x4 data[8];
  uint32_t scl[8];
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
    const int tok = 16 * tt + m;
    data[tt] = ld16(page + tok * 64 + 16 * g);
    scl[tt] = ld4(page + kMxDataBytes + 4 * tok);
  }
  float best = neg_inf();
  bool nan = false;
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
    i32x8 ka = {(int)data[tt][0], (int)data[tt][1], (int)data[tt][2], (int)data[tt][3], 0, 0, 0, 0};
    const int sa = (int)((scl[tt] >> (8 * g)) & 0xFFu);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = mfma_scale_fp4_e4m3(ka, qb, acc, sa);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (16 * tt + 4 * g + e < nv) {
        nan |= acc[e] != acc[e];
        best = fmaxf(best, acc[e]);
      }
    }
  }
  best = max_over_groups(best);
  nan = (__ballot(nan) >> m & 0x0001000100010001ull) != 0;
  return nan ? qnan() : best;
}

// ----------------------------------------------------------------- kernel
// grid (ceil(MB / 4), R), 4 waves a workgroup, wave w scores block 4 x + w.
template <int VARIANT, int KEY_DT>
__global__ __launch_bounds__(256) void index_score_kernel(ScoreArgs a) {
  __shared__ float s_rowmax[kScoreWaves][kMaxQueryRows];
  __shared__ float s_out[kScoreWaves][kMaxQueryRows];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.y;
  const int b = blockIdx.x * kScoreWaves + wave;
  if (b >= a.MB) return;
  const int L = a.seq_lens[r];
  const int nr = (L + kBlockTokens - 1) / kBlockTokens;
  if (b >= nr) {
    write_scores(a, r, b, lane, nullptr);
    return;
  }
  const int QR = a.q_len * a.H_idx;
  // valid keys of this block for each query token (wave-private LDS)
  __shared__ int s_nvalid[kScoreWaves][16];
  for (int i = lane; i < a.q_len; i += kWave) {
    int v = causal_len(L, a.q_len, i) - b * kBlockTokens;
    s_nvalid[wave][i] = v < 0 ? 0 : (v > kBlockTokens ? kBlockTokens : v);
  }
  const int* nvalid_row = s_nvalid[wave];
  const int64_t blk = a.bt[(size_t)r * a.bt_stride + b];
  if (blk < 0 || blk >= a.pool_blocks) {
    // An out-of-range block id is poison: NaN where the block is causally
    // visible, -inf elsewhere.  Nothing is read through it.
    for (int x = lane; x < a.q_len * a.H_kv; x += kWave)
      s_out[wave][x] = s_nvalid[wave][x / a.H_kv] > 0 ? qnan() : neg_inf();
    write_scores(a, r, b, lane, s_out[wave]);
    return;
  }
  const uint8_t* page = a.pool + blk * (KEY_DT == ISB_BF16 ? 32768 : KEY_DT == ISB_FP8_E4M3 ? 16384 : kMxPageBytes);
  if constexpr (VARIANT == 0) {
    const int qbytes = a.q_dt == ISB_BF16 ? 2 : 1;
    const uint8_t* qrow = a.q_idx + (size_t)r * kHeadDim * qbytes;  // q_len = H_idx = 1
    float best = stream_block<KEY_DT>(a, page, qrow, lane, s_nvalid[wave][0]);
    if (lane == 0) s_rowmax[wave][0] = best;
  } else {
    for (int qt = 0; qt * 16 < QR; ++qt) {
      float best;
      if constexpr (VARIANT == 1) best = tile_block_bf16<KEY_DT>(a, page, r, qt, QR, lane, nvalid_row);
      else best = tile_block_fp4(a, page, r, qt, QR, lane, nvalid_row);
      if (lane < 16 && qt * 16 + lane < QR) s_rowmax[wave][qt * 16 + lane] = best;
    }
  }
  finish(a, r, b, lane, s_rowmax[wave], s_out[wave]);
  write_scores(a, r, b, lane, s_out[wave]);
}

template <int VARIANT, int KEY_DT>
static void launch(const ScoreArgs& a, hipStream_t st) {
  dim3 grid((a.MB + kScoreWaves - 1) / kScoreWaves, a.R);
  hipLaunchKernelGGL((index_score_kernel<VARIANT, KEY_DT>), grid, dim3(256), 0, st, a);
}

}  // namespace isb

extern "C" int isb_index_score(isb_stream_t stream, const void* q_idx, int q_idx_dtype,
                               int num_idx_heads, const void* idx_pool, int idx_dtype,
                               float idx_scale, int64_t idx_pool_blocks,
                               const int32_t* block_table, int block_table_stride,
                               const int32_t* seq_lens, int num_reqs, int decode_query_len,
                               int num_kv_heads, int max_blocks, float* scores) {
  using namespace isb;
  if (!q_idx || !idx_pool || !block_table || !seq_lens || !scores) return ISB_E_INVALID_ARG;
  if (num_idx_heads <= 0 || num_reqs <= 0 || decode_query_len <= 0 || num_kv_heads <= 0 ||
      max_blocks <= 0 || block_table_stride <= 0 || idx_pool_blocks <= 0)
    return ISB_E_INVALID_ARG;
  if (!is_query_dtype(q_idx_dtype) || !is_pool_dtype(idx_dtype)) return ISB_E_UNSUPPORTED_DTYPE;
  if (num_idx_heads % num_kv_heads != 0 || max_blocks > block_table_stride) return ISB_E_SHAPE;
  if (decode_query_len > 16 || decode_query_len * num_idx_heads > kMaxQueryRows) return ISB_E_SHAPE;
  if (!(idx_scale > 0.f) && idx_dtype == ISB_FP8_E4M3) return ISB_E_INVALID_ARG;
  ScoreArgs a{(const uint8_t*)q_idx, (const uint8_t*)idx_pool, block_table, seq_lens, scores,
              idx_pool_blocks, idx_scale, q_idx_dtype, idx_dtype, num_idx_heads,
              block_table_stride, num_reqs, decode_query_len, num_kv_heads, max_blocks};
  hipStream_t st = as_hip(stream);
  const bool one_row = decode_query_len * num_idx_heads == 1;
  if (idx_dtype == ISB_MXFP4) {
    if (q_idx_dtype == ISB_FP8_E4M3) launch<2, ISB_MXFP4>(a, st);
    else launch<1, ISB_MXFP4>(a, st);
  } else if (idx_dtype == ISB_FP8_E4M3) {
    if (one_row) launch<0, ISB_FP8_E4M3>(a, st);
    else launch<1, ISB_FP8_E4M3>(a, st);
  } else {
    if (one_row) launch<0, ISB_BF16>(a, st);
    else launch<1, ISB_BF16>(a, st);
  }
  return launch_status();
}
