// isb_index_score: one score per (KV head, query token, 128-token block).
//
// The indexer of ROCm/ATOM PR 2962 ("[MiniMax-M3.1] MXFP4 index cache and
// MXFP4 KV cache", Summary and Known limits) scores every 128-token block of a
// request's paged index-key cache with the index query into an fp32
// (head, row, block) workspace.  Here a block's score for one index head is the
// largest dot product over the block's causally valid keys, and the index
// heads of a KV group are summed.
//
// One wavefront scores a block of one request against every query row of
// that request (q tokens x H_idx heads), so the block's keys cross HBM once
// however many tokens the request decodes.  Every load of a wave is issued
// before any math, and pages are read with nontemporal loads (they are read
// once per launch).  Three variants:
//   * stream - one query row (q = 1, H_idx = 1), bf16 / fp8 keys, two blocks
//              a wave: packed bf16 dot products on the VALU (2 flop per key
//              byte leaves it far from busy), partial sums combined across the
//              four lane groups;
//   * tile   - several query rows: keys converted to bf16 in registers and
//              multiplied on v_mfma_f32_16x16x32_bf16, 16 keys x 16 rows a tile;
//   * fp4    - MXFP4 keys with an e4m3 query: v_mfma_scale_f32_16x16x128_f8f6f4
//              consumes the e2m1 data and its e8m0 scales directly, one
//              instruction per 16 keys x 16 rows x 128 dims;
//   * wide   - many query rows (a chunk of prefill tokens, more than 16 tokens
//              or 64 rows): a wave loads its block's keys once, keeps them in
//              registers and runs them against up to kWideTiles 16-row query
//              tiles (the grid's third dimension takes the rest), with the
//              MFMA of the key type above; each row's causal length is
//              computed in the loop, and the index heads of a KV group are
//              summed across the lanes that hold them.
// bf16 / fp8 index pages are eight 16-key tiles in the lane order of the K
// pages (chunk h of lane l = 16 g + m at byte 1024 h + 16 l of the tile holds
// key m's dims 32 g + (16 / esize) h ...), so each load instruction reads one
// contiguous KiB; MXFP4 pages keep their token-major format (64 B a key: one
// 16-key tile is also one contiguous KiB a load).
#include "grid_maps.h"
#include "isb_device.h"
#include "isb_host.h"

namespace isb {

struct ScoreArgs {
  const uint8_t* q_idx;
  const uint8_t* pool;
  const int32_t* bt;
  const int32_t* seq_lens;  // decode batches
  float* scores;
  int64_t pool_blocks;
  float idx_scale;
  int H_idx, bt_stride, R, q_len, H_kv, MB;
  TokenMap tm;  // wide variant: each token's request and causal length (both batch forms)
  int T;        // query tokens
};

constexpr int kMaxQueryRows = 64;     // q_len * H_idx of the tile / stream variants
constexpr long long kMaxWideRows = 1 << 20;  // q_len * H_idx of the wide variant

template <int Q_DT>
__device__ __forceinline__ bf16x8 load_q8(const uint8_t* row, int dim0) {
  if constexpr (Q_DT == ISB_BF16) {
    return u32x4_as_bf16x8(ld16(row + 2 * dim0));
  } else {
    const u32x2 w = ld8(row + dim0);
    return e4m3x8_to_bf16x8(w[0], w[1]);
  }
}

__device__ __forceinline__ int causal_len(int L, int q_len, int i) {
  const int v = L - (q_len - 1 - i);
  return v > 0 ? v : 0;
}

// Writes vals[x] (or -inf) for every (token, group) x of request r at block b.
__device__ __forceinline__ void write_scores(const ScoreArgs& a, int r, int b, int lane,
                                             const float* vals) {
  const int T = a.R * a.q_len;
  for (int x = lane; x < a.q_len * a.H_kv; x += kWave) {
    const int i = x / a.H_kv, g = x % a.H_kv;
    const float v = vals ? vals[x] : neg_inf();
    a.scores[((size_t)g * T + (size_t)r * a.q_len + i) * a.MB + b] = v;
  }
}

// Group sums of per-row block maxima held in `rowmax[QR]` (wave-private LDS).
template <int KEY_DT>
__device__ __forceinline__ void finish(const ScoreArgs& a, int lane, const float* rowmax, float* outv) {
  const int per = a.H_idx / a.H_kv;
  for (int x = lane; x < a.q_len * a.H_kv; x += kWave) {
    const int i = x / a.H_kv, g = x % a.H_kv;
    float s = 0.f;
    for (int h = 0; h < per; ++h) s += rowmax[i * a.H_idx + g * per + h];
    outv[x] = KEY_DT == ISB_FP8_E4M3 ? s * a.idx_scale : s;
  }
}

// Raw chunks of one 16-key tile for this lane (bf16 / fp8 index pages).
template <int KEY_DT>
struct TileRegs {
  static constexpr int NC = KEY_DT == ISB_BF16 ? 4 : 2;
  u32x4 c[NC];
};

template <int KEY_DT>
__device__ __forceinline__ void load_tile(TileRegs<KEY_DT>& t, __amdgpu_buffer_rsrc_t page, int tile_off,
                                          int lane) {
#pragma unroll
  for (int h = 0; h < TileRegs<KEY_DT>::NC; ++h) t.c[h] = bl16_nt(page, 1024 * h + 16 * lane, tile_off);
}

// MFMA A operand of a tile: dims 32 g + 8 j .. + 7 of key m in kb[j].
template <int KEY_DT>
__device__ __forceinline__ void tile_operand(const TileRegs<KEY_DT>& t, bf16x8 (&kb)[4]) {
  if constexpr (KEY_DT == ISB_BF16) {
#pragma unroll
    for (int h = 0; h < 4; ++h) kb[h] = u32x4_as_bf16x8(t.c[h]);
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int q = 0; q < 2; ++q) kb[2 * h + q] = e4m3x8_to_bf16x8(t.c[h][2 * q], t.c[h][2 * q + 1]);
  }
}

// ----------------------------------------------------------------- stream
// One query row (q = 1, H_idx = H_kv = 1): scores[r][b].  grid
// (ceil(MB / (4 NB)), R); wave w of workgroup x scores blocks NB (4 x + w) + n,
// NB = 2 for fp8 keys, 1 for bf16 keys.  Lane (g, m) takes key m of every tile, dims
// 32 g .. 32 g + 31; its partial dot products are summed over the four lane
// groups, the keys' maximum over the sixteen lanes of a group.  Both blocks'
// loads are issued before any math; a block past the request's end re-reads
// the wave's first page (a cache hit) so that no load sits behind a branch.
template <int KEY_DT>
constexpr int stream_blocks() { return KEY_DT == ISB_BF16 ? 1 : 2; }  // 32 KiB of keys a wave

template <int KEY_DT, int Q_DT>
__global__ __launch_bounds__(256) void index_stream_kernel(ScoreArgs a) {
  constexpr int TB = KEY_DT == ISB_BF16 ? 4096 : 2048;  // bytes of a 16-key tile
  constexpr int64_t PB = 8 * TB;
  constexpr int NB = stream_blocks<KEY_DT>();
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;
  const int r = blockIdx.y;
  const int b0 = (score_column<kScoreWaves * NB>(blockIdx.x, gridDim.x, blockIdx.y) * kScoreWaves + wave) * NB;
  if (b0 >= a.MB) return;
  const int L = a.seq_lens[r];
  const int nr = (L + kBlockTokens - 1) / kBlockTokens;
  float* srow = a.scores + (size_t)r * a.MB;
  if (b0 >= nr) {
    if (lane < NB && b0 + lane < a.MB) srow[b0 + lane] = neg_inf();
    return;
  }
  int64_t blk[NB];
  bool bad[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const int b = b0 + n < nr ? b0 + n : b0;
    blk[n] = __builtin_amdgcn_readfirstlane(a.bt[(size_t)r * a.bt_stride + b]);
    // an out-of-range block id is poison: its score is NaN, nothing is read through it
    bad[n] = blk[n] < 0 || blk[n] >= a.pool_blocks;
    if (bad[n]) blk[n] = 0;
  }
  // the query first: the load counter is in order, so what is used first is
  // loaded first
  bf16x2 qv[16];
  {
    const uint8_t* qrow = a.q_idx + (size_t)r * kHeadDim * (Q_DT == ISB_BF16 ? 2 : 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 q8 = load_q8<Q_DT>(qrow, 32 * g + 8 * j);
#pragma unroll
      for (int x = 0; x < 4; ++x) qv[4 * j + x] = bf16x2{q8[2 * x], q8[2 * x + 1]};
    }
  }
  TileRegs<KEY_DT> t[NB][8];
#pragma unroll
  for (int n = 0; n < NB; ++n)
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) load_tile<KEY_DT>(t[n][tt], page_rsrc(a.pool + blk[n] * PB, PB), tt * TB, lane);
  // every page load of the wave is in flight before the first use
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const int b = b0 + n;
    const int nvalid = min(L - b * kBlockTokens, kBlockTokens);  // <= 0 past the end
    float best = neg_inf();
    bool nan = false;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      float acc = 0.f;
      if constexpr (KEY_DT == ISB_BF16) {
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
          for (int w = 0; w < 4; ++w)
            acc = __builtin_amdgcn_fdot2_f32_bf16(u32_as_bf16x2(t[n][tt].c[h][w]), qv[4 * h + w], acc, false);
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            acc = __builtin_amdgcn_fdot2_f32_bf16(e4m3x2_to_bf16x2(t[n][tt].c[h][w], false), qv[8 * h + 2 * w],
                                                  acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(e4m3x2_to_bf16x2(t[n][tt].c[h][w], true),
                                                  qv[8 * h + 2 * w + 1], acc, false);
          }
      }
      acc += shfl_xor_f32(acc, 16);
      acc += shfl_xor_f32(acc, 32);
      if (16 * tt + m < nvalid) {
        nan |= acc != acc;
        best = fmaxf(best, acc);
      }
    }
    // maximum over the sixteen keys of a tile column (lanes of one row of 16)
    best = fmaxf(best, dpp_f32<kDppXor1>(best));
    best = fmaxf(best, dpp_f32<kDppXor2>(best));
    best = fmaxf(best, dpp_f32<kDppHalfMirror>(best));
    best = fmaxf(best, dpp_f32<kDppMirror>(best));
    if (__ballot(nan) || bad[n]) best = qnan();
    if (KEY_DT == ISB_FP8_E4M3) best *= a.idx_scale;
    if (lane == 0 && b < a.MB) srow[b] = nvalid > 0 ? best : neg_inf();
  }
}

// ----------------------------------------------------------------- tiles
// Block maxima for query rows [qt*16, qt*16+16) of request r, bf16 MFMA.
// Lane (g, m) supplies key m of a tile and query row m, both at dims
// 32 g .. 32 g + 31; the result lane holds keys 4 g + e of query row m.
template <int KEY_DT, int Q_DT>
__device__ __forceinline__ float tile_block_bf16(const ScoreArgs& a, __amdgpu_buffer_rsrc_t page, int r,
                                                 int qt, int QR, int lane, const int* nvalid_row) {
  constexpr int QB = Q_DT == ISB_BF16 ? 2 : 1;
  const int m = lane & 15, g = lane >> 4;
  const int n = qt * 16 + m;
  const int nq = n < QR ? n : 0;
  bf16x8 qb[4];
  {
    const int i = nq / a.H_idx, h = nq % a.H_idx;
    const uint8_t* qrow = a.q_idx + ((size_t)(r * a.q_len + i) * a.H_idx + h) * kHeadDim * QB;
#pragma unroll
    for (int j = 0; j < 4; ++j) qb[j] = load_q8<Q_DT>(qrow, 32 * g + 8 * j);
  }
  float best = neg_inf();
  bool nan = false;
  if constexpr (KEY_DT == ISB_MXFP4) {
    u32x4 data[8];
    uint32_t scl[8];
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      data[tt] = bl16_nt(page, 64 * m + 16 * g, 1024 * tt);
      scl[tt] = bl4_nt(page, 4 * m, kMxDataBytes + 64 * tt);
    }
    const int nv = n < QR ? nvalid_row[n / a.H_idx] : 0;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const float sc = e8m0_to_f32(scl[tt] >> (8 * g));
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = mfma_16x16x32_bf16(e2m1x8_to_bf16x8(data[tt][j], sc), qb[j], acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (16 * tt + 4 * g + e < nv) {
          nan |= acc[e] != acc[e];
          best = fmaxf(best, acc[e]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    constexpr int TB = KEY_DT == ISB_BF16 ? 4096 : 2048;
    constexpr int HALF = KEY_DT == ISB_BF16 ? 4 : 8;
    const int nv = n < QR ? nvalid_row[n / a.H_idx] : 0;
#pragma unroll
    for (int part = 0; part < 8 / HALF; ++part) {
      TileRegs<KEY_DT> t[HALF];
#pragma unroll
      for (int tt = 0; tt < HALF; ++tt) load_tile<KEY_DT>(t[tt], page, (part * HALF + tt) * TB, lane);
#pragma unroll
      for (int tt = 0; tt < HALF; ++tt) {
        bf16x8 kb[4];
        tile_operand<KEY_DT>(t[tt], kb);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = mfma_16x16x32_bf16(kb[j], qb[j], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (16 * (part * HALF + tt) + 4 * g + e < nv) {
            nan |= acc[e] != acc[e];
            best = fmaxf(best, acc[e]);
          }
        }
        // one tile's operands at a time: converting every tile up front would
        // hold 128 more registers and halve the waves in flight
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  best = max_over_groups(best);
  nan = (__ballot(nan) >> m & 0x0001000100010001ull) != 0;
  return nan ? qnan() : best;
}

// MXFP4 keys and an e4m3 query on the scaled MFMA: one instruction a tile.
__device__ __forceinline__ float tile_block_fp4(const ScoreArgs& a, __amdgpu_buffer_rsrc_t page, int r,
                                                int qt, int QR, int lane, const int* nvalid_row) {
  const int m = lane & 15, g = lane >> 4;
  const int n = qt * 16 + m;
  const int nq = n < QR ? n : 0;
  u32x4 data[8];
  uint32_t scl[8];
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
    data[tt] = bl16_nt(page, 64 * m + 16 * g, 1024 * tt);
    scl[tt] = bl4_nt(page, 4 * m, kMxDataBytes + 64 * tt);
  }
  i32x8 qb;
  {
    const int i = nq / a.H_idx, h = nq % a.H_idx;
    const uint8_t* qrow = a.q_idx + ((size_t)(r * a.q_len + i) * a.H_idx + h) * kHeadDim;
    const u32x4 lo = ld16(qrow + 16 * g);
    const u32x4 hi = ld16(qrow + 64 + 16 * g);
    qb = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
  const int nv = n < QR ? nvalid_row[n / a.H_idx] : 0;
  float best = neg_inf();
  bool nan = false;
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
    const i32x8 ka = {(int)data[tt][0], (int)data[tt][1], (int)data[tt][2], (int)data[tt][3], 0, 0, 0, 0};
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

// ----------------------------------------------------------------- wide
// Query tiles (16 rows each) a wave of the wide variant runs its block against.
constexpr int kWideTiles = 8;

// Key tiles of a block the wide variant converts to MFMA operands at once
// (a part): two for bf16 and fp8 keys (32 registers of bf16 operands, which
// keeps four waves a SIMD), four for MXFP4 keys; the raw bytes of the next
// part are loaded while this part's tiles run against the query tiles.
template <int KEY_DT>
constexpr int wide_part_tiles() { return KEY_DT == ISB_MXFP4 ? 4 : 2; }

// Raw bytes of one part of a block, as loaded.
template <int KEY_DT>
struct PartRaw {
  TileRegs<KEY_DT> t[wide_part_tiles<KEY_DT>()];
};
template <>
struct PartRaw<ISB_MXFP4> {
  u32x4 data[4];    // key m of tile tt, dims 32 g .. 32 g + 31 (e2m1)
  uint32_t scl[4];  // key m's four e8m0 scales
};

template <int KEY_DT>
__device__ __forceinline__ void load_part_raw(PartRaw<KEY_DT>& k, __amdgpu_buffer_rsrc_t page, int part, int lane) {
  constexpr int NT = wide_part_tiles<KEY_DT>();
  if constexpr (KEY_DT == ISB_MXFP4) {
    const int m = lane & 15, g = lane >> 4;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      k.data[tt] = bl16_nt(page, 64 * m + 16 * g, 1024 * (part * NT + tt));
      k.scl[tt] = bl4_nt(page, 4 * m, kMxDataBytes + 64 * (part * NT + tt));
    }
  } else {
    constexpr int TB = KEY_DT == ISB_BF16 ? 4096 : 2048;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) load_tile<KEY_DT>(k.t[tt], page, (part * NT + tt) * TB, lane);
  }
}

// MFMA operands of one part: bf16 for the bf16 MFMA (keys converted once,
// whatever the number of query tiles), or the raw e2m1 data and scales for
// the scaled fp4 x e4m3 MFMA.
template <int KEY_DT, int Q_DT>
struct PartOps {
  bf16x8 kb[wide_part_tiles<KEY_DT>()][4];  // tile tt: dims 32 g + 8 j .. of key m in kb[tt][j]
};
template <>
struct PartOps<ISB_MXFP4, ISB_FP8_E4M3> {
  u32x4 data[4];  // e2m1, as loaded
  int sa[4];      // this lane's e8m0 scale byte of each tile
};
// e4m3 keys against an e4m3 query: the keys as loaded (lane (g, m) of a tile
// holds key m's dims 32 g .. 32 g + 31), multiplied on the fp8 MFMA
template <>
struct PartOps<ISB_FP8_E4M3, ISB_FP8_E4M3> {
  i32x8 k8[2];
};

template <int KEY_DT, int Q_DT>
__device__ __forceinline__ void part_operands(const PartRaw<KEY_DT>& k, int lane, PartOps<KEY_DT, Q_DT>& o) {
  constexpr int NT = wide_part_tiles<KEY_DT>();
  const int g = lane >> 4;
  if constexpr (KEY_DT == ISB_MXFP4 && Q_DT == ISB_FP8_E4M3) {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      o.data[tt] = k.data[tt];
      o.sa[tt] = (int)((k.scl[tt] >> (8 * g)) & 0xFFu);
    }
  } else if constexpr (KEY_DT == ISB_FP8_E4M3 && Q_DT == ISB_FP8_E4M3) {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const u32x4 c0 = k.t[tt].c[0], c1 = k.t[tt].c[1];
      o.k8[tt] = i32x8{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3], (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
    }
  } else if constexpr (KEY_DT == ISB_MXFP4) {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const float sc = e8m0_to_f32(k.scl[tt] >> (8 * g));
#pragma unroll
      for (int j = 0; j < 4; ++j) o.kb[tt][j] = e2m1x8_to_bf16x8(k.data[tt][j], sc);
    }
  } else {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) tile_operand<KEY_DT>(k.t[tt], o.kb[tt]);
  }
}

// IEEE maximum that propagates NaN (v_maximum3_f32 on gfx950): a NaN
// product among a row's valid keys makes its block maximum NaN with no
// separate test.
__device__ __forceinline__ float nan_max(float x, float y) { return __builtin_elementwise_maximum(x, y); }
__device__ __forceinline__ float nan_max3(float x, float y, float z) { return nan_max(x, nan_max(y, z)); }

// Folds one part's keys into the running maximum `best` of query row n
// (lane (g, m) of a 16-row tile holds keys 4 g + e of row m).  full: every
// row of the tile sees the whole block (wave-uniform); otherwise keys at or
// past nv (the row's causally valid keys in this block) count as -inf.
// qrow: the row as stored.
template <int KEY_DT, int Q_DT>
__device__ __forceinline__ void wide_part_max(const PartOps<KEY_DT, Q_DT>& k, int part, const uint8_t* qrow,
                                              bool full, int nv, int lane, float& best) {
  constexpr int NT = wide_part_tiles<KEY_DT>();
  const int g = lane >> 4;
  f32x4 acc[NT];
  if constexpr (KEY_DT == ISB_MXFP4 && Q_DT == ISB_FP8_E4M3) {
    const u32x4 lo = ld16(qrow + 16 * g);
    const u32x4 hi = ld16(qrow + 64 + 16 * g);
    const i32x8 qb = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const i32x8 ka = {(int)k.data[tt][0], (int)k.data[tt][1], (int)k.data[tt][2], (int)k.data[tt][3], 0, 0, 0, 0};
      acc[tt] = mfma_scale_fp4_e4m3(ka, qb, f32x4{0.f, 0.f, 0.f, 0.f}, k.sa[tt]);
    }
  } else if constexpr (KEY_DT == ISB_FP8_E4M3 && Q_DT == ISB_FP8_E4M3) {
    // the query row's dims 32 g .. 32 g + 31, the bytes the keys hold
    const u32x4 lo = ld16(qrow + 32 * g);
    const u32x4 hi = ld16(qrow + 32 * g + 16);
    const i32x8 qb = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[tt] = mfma_scale_e4m3(k.k8[tt], qb, f32x4{0.f, 0.f, 0.f, 0.f});
  } else {
    bf16x8 qb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) qb[j] = load_q8<Q_DT>(qrow, 32 * g + 8 * j);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[tt] = mfma_16x16x32_bf16(k.kb[tt][j], qb[j], acc[tt]);
    }
  }
  if (full) {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      best = nan_max3(best, acc[tt][0], acc[tt][1]);
      best = nan_max3(best, acc[tt][2], acc[tt][3]);
    }
  } else {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const int key0 = 16 * (part * NT + tt) + 4 * g;
#pragma unroll
      for (int e = 0; e < 4; ++e) best = nan_max(best, key0 + e < nv ? acc[tt][e] : neg_inf());
    }
  }
}

// Tiles that hold tokens of several requests: the tile's 16-row tiles
// against block b of every run of its tokens [k_begin, ntok) after the first,
// folded into best[q] (lane row m of tile q: row n0 + 16 q + m of the tile
// [n0, n1), staged at s_q + (16 q + m) qpitch).  Each run reads its block once,
// a part at a time, and runs it against every 16-row tile with rows in the
// run; the rows' running maxima wait in this wave's LDS slice s_best
// [NQ][64] meanwhile, so the loops stay rolled and the path holds few
// registers (the single-run path keeps its budget).
template <int KEY_DT, int Q_DT, int NQ>
__device__ __forceinline__ void wide_other_runs(const uint8_t* pool, int64_t pool_blocks, const int32_t* bt,
                                                int bt_stride, const int* s_req, const int* s_len,
                                                const uint8_t* s_q, int qpitch, int n0, int n1, int t0, int hsh,
                                                float* s_best, int b, int k_begin, int ntok, float (&best)[NQ]) {
  constexpr int NT = wide_part_tiles<KEY_DT>();
  constexpr int PARTS = 8 / NT;
  constexpr int64_t PB = KEY_DT == ISB_BF16 ? 32768 : KEY_DT == ISB_FP8_E4M3 ? 16384 : kMxPageBytes;
  const int lane = threadIdx.x & 63, m = lane & 15;
#pragma unroll
  for (int q = 0; q < NQ; ++q) s_best[64 * q + lane] = best[q];
  // row n0 + 16 q + m: its token's causally valid keys in block b if the
  // token is in tokens [k0, k1), else 0
  auto row_nv = [&](int q, int k0, int k1) {
    const int n = n0 + 16 * q + m;
    const int k = (n >> hsh) - t0;
    const int v = n < n1 && k >= k0 && k < k1 ? s_len[k] - b * kBlockTokens : 0;
    return v < 0 ? 0 : (v > kBlockTokens ? kBlockTokens : v);
  };
#pragma unroll 1
  for (int k0 = k_begin, k1 = 0; k0 < ntok; k0 = k1) {
    const int rr = __builtin_amdgcn_readfirstlane(s_req[k0]);
    k1 = ntok;
#pragma unroll 1
    for (int base = k0 + 1; base < ntok; base += kWave) {
      const int k = base + lane;
      const uint64_t diff = __ballot(k < ntok && s_req[k] != rr);
      if (diff) {
        k1 = base + __builtin_ctzll(diff);
        break;
      }
    }
    uint32_t has = 0;  // bit q: a row of tile q is in the run and reaches block b
#pragma unroll 1
    for (int q = 0; q < NQ; ++q)
      if (__ballot(row_nv(q, k0, k1) > 0)) has |= 1u << q;
    if (!has) continue;  // wave-uniform
    const int64_t blk = __builtin_amdgcn_readfirstlane(bt[(size_t)rr * bt_stride + b]);
    if (blk < 0 || blk >= pool_blocks) {  // poison block id: nothing is read through it
#pragma unroll 1
      for (int q = 0; q < NQ; ++q)
        if (row_nv(q, k0, k1) > 0) s_best[64 * q + lane] = qnan();
      continue;
    }
    const __amdgpu_buffer_rsrc_t page = page_rsrc(pool + blk * PB, (int)PB);
#pragma unroll 1
    for (int part = 0; part < PARTS; ++part) {
      PartRaw<KEY_DT> raw;
      load_part_raw<KEY_DT>(raw, page, part, lane);
      PartOps<KEY_DT, Q_DT> ops;
      part_operands<KEY_DT, Q_DT>(raw, lane, ops);
#pragma unroll 1
      for (int q = 0; q < NQ; ++q) {
        if (!((has >> q) & 1u)) continue;  // wave-uniform
        const int n = n0 + 16 * q + m;
        const uint8_t* qrow = s_q + ((n < n1 ? n : n0) - n0) * qpitch;
        float bq = s_best[64 * q + lane];
        wide_part_max<KEY_DT, Q_DT>(ops, part, qrow, false, row_nv(q, k0, k1), lane, bq);
        s_best[64 * q + lane] = bq;
      }
    }
  }
#pragma unroll
  for (int q = 0; q < NQ; ++q) best[q] = s_best[64 * q + lane];
}

// Wave-uniform maximum of an int over the wave.
__device__ __forceinline__ int wave_max_int(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off, kWave));
  return __builtin_amdgcn_readfirstlane(x);
}

// grid (ceil(MB / 4), R, tiles a request) for a decode batch (RAGGED false)
// or (ceil(MB / 4), tiles) for a prefill batch, 4 waves a workgroup: wave w
// scores block 4 x + w (x from score_column) for the query rows [n0, n1) of
// the workgroup's tile, which it stages in LDS.  Global query row n = t H_idx
// + h (token t, index head h).  A decode tile is rows [r QR + 128 z, ..) of
// request r (QR = q H_idx): one request, causal lengths from seq_lens.  A
// prefill tile is rows [128 y, 128 y + 128) of the batch, its tokens taken in
// runs of consecutive tokens of one request (one run whenever the tile holds
// one request's tokens); each run scores its request's block b against its
// own rows.  Needs 16 % H_idx == 0, so a 16-row tile holds whole tokens and
// each KV group's index heads sit on adjacent lanes.
template <int KEY_DT, int Q_DT, bool RAGGED>
__global__ __launch_bounds__(256) void index_wide_kernel(ScoreArgs a) {
  constexpr int NT = wide_part_tiles<KEY_DT>();
  constexpr int PARTS = 8 / NT;
  constexpr int QROW = Q_DT == ISB_BF16 ? 2 * kHeadDim : kHeadDim;  // bytes of a query row
  constexpr int TROWS = 16 * kWideTiles;                            // rows of a tile
  constexpr int64_t PB = KEY_DT == ISB_BF16 ? 32768 : KEY_DT == ISB_FP8_E4M3 ? 16384 : kMxPageBytes;
  // LDS pitch of a staged row: 16 bytes past a multiple of 256 puts the 16
  // rows a 16-byte read of a tile touches on distinct banks
  constexpr int QPITCH = QROW + 16;
  __shared__ __attribute__((aligned(16))) uint8_t s_q[TROWS * QPITCH];
  __shared__ int s_req[RAGGED ? TROWS : 1];  // per token of a prefill tile: request and causal length
  __shared__ int s_len[RAGGED ? TROWS : 1];
  __shared__ int s_nb[kScoreWaves];
  __shared__ float s_best[RAGGED ? kScoreWaves * kWideTiles * kWave : 1];  // the later runs' row maxima
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int m = lane & 15;
  int n0, n1;
  if constexpr (RAGGED) {
    n0 = TROWS * blockIdx.y;
    n1 = min(a.T * a.H_idx, n0 + TROWS);
  } else {
    const int QR = a.q_len * a.H_idx;
    n0 = blockIdx.y * QR + TROWS * blockIdx.z;
    n1 = min((int)blockIdx.y * QR + QR, n0 + TROWS);
  }
  const int per = a.H_idx / a.H_kv;  // index heads of a KV group
  // H_idx divides 16 and per divides H_idx: both are powers of two, so the
  // row -> (token, head) and head -> group splits are shifts and masks
  const int hsh = __builtin_ctz(a.H_idx), psh = __builtin_ctz(per);
  const int t0 = n0 >> hsh;                     // first token of the tile
  const int ntok = ((n1 - 1) >> hsh) - t0 + 1;  // its tokens
  // The tile's first request (decode: the tile's request).  Its index also
  // rotates the column -> die map, so that the tiles of one request (and a
  // ragged tile's first run) fetch a block on the same die, where the tiles
  // after the first find it in L2.
  TokenPos tp0{(int)blockIdx.y, 0};
  if constexpr (RAGGED) tp0 = token_pos(a.tm, t0);
  const int col = score_column<kScoreWaves>(blockIdx.x, gridDim.x, tp0.r);
  const int b = col * kScoreWaves + wave;
  // -inf for every token of the tile at block b (none of them reaches it)
  auto write_unreached = [&]() {
    for (int x = lane; x < ntok * a.H_kv; x += kWave) {
      const int k = x / a.H_kv, gg = x % a.H_kv;
      a.scores[((size_t)gg * a.T + t0 + k) * a.MB + b] = neg_inf();
    }
  };
  // The tile's first request and the blocks it has (decode: the request's
  // length bounds every token of the tile, and workgroups past its blocks
  // stop before reading anything else).
  int r0, nreq;
  if constexpr (RAGGED) {
    r0 = tp0.r;
    nreq = (tp0.L + kBlockTokens - 1) / kBlockTokens;  // the first token's: a lower bound
  } else {
    r0 = blockIdx.y;
    nreq = (a.seq_lens[r0] + kBlockTokens - 1) / kBlockTokens;
    if (col * kScoreWaves >= nreq) {  // uniform over the workgroup
      if (b < a.MB) write_unreached();
      return;
    }
  }
  // The first request's block is requested before anything else, so that
  // one round trip covers its keys, the tile's token data and the query rows.
  const bool pre = b < a.MB && b < nreq;
  int64_t blk = 0;
  if (pre) blk = __builtin_amdgcn_readfirstlane(a.bt[(size_t)r0 * a.bt_stride + b]);
  // an out-of-range block id is poison: NaN where the block is causally
  // visible, -inf elsewhere; nothing is read through it
  bool bad = blk < 0 || blk >= a.pool_blocks;
  PartRaw<KEY_DT> raw;
  if (pre) load_part_raw<KEY_DT>(raw, page_rsrc(a.pool + (bad ? 0 : blk) * PB, (int)PB), 0, lane);
  // The tile's query rows, as stored (and a prefill tile's tokens: request,
  // causal length, and the blocks they reach).
  {
    const uint8_t* src = a.q_idx + (size_t)n0 * QROW;
    constexpr int CPR = QROW / 16;  // 16-byte chunks a row
    for (int c = threadIdx.x; c < (n1 - n0) * CPR; c += 256)
      *reinterpret_cast<u32x4*>(s_q + (c / CPR) * QPITCH + (c % CPR) * 16) = ld16(src + (size_t)c * 16);
    if constexpr (RAGGED) {
      int nb = 0;
      for (int k = threadIdx.x; k < ntok; k += 256) {
        const TokenPos tp = token_pos(a.tm, t0 + k);
        s_req[k] = tp.r;
        s_len[k] = tp.L;
        nb = max(nb, (tp.L + kBlockTokens - 1) / kBlockTokens);
      }
      nb = wave_max_int(nb);
      if (lane == 0) s_nb[wave] = nb;
    }
  }
  __syncthreads();
  const int nmax = RAGGED ? max(max(s_nb[0], s_nb[1]), max(s_nb[2], s_nb[3])) : nreq;
  if (b >= a.MB) return;
  if (b >= nmax) {
    write_unreached();
    return;
  }
  // The first run of the tile: its tokens [0, k1) (all of them in a decode
  // tile, and in a prefill tile that holds one request's tokens), which reach
  // nr blocks.
  int k1 = ntok, nr = nreq;
  if constexpr (RAGGED) {
    for (int base = 1; base < ntok; base += kWave) {
      const int k = base + lane;
      const uint64_t diff = __ballot(k < ntok && s_req[k] != r0);
      if (diff) {
        k1 = base + __builtin_ctzll(diff);
        break;
      }
    }
    nr = 0;
    for (int k = lane; k < k1; k += kWave) nr = max(nr, (s_len[k] + kBlockTokens - 1) / kBlockTokens);
    nr = wave_max_int(nr);
    if (!pre && b < nr) {  // a later token of the first run reaches block b
      blk = __builtin_amdgcn_readfirstlane(a.bt[(size_t)r0 * a.bt_stride + b]);
      bad = blk < 0 || blk >= a.pool_blocks;
      if (!bad) load_part_raw<KEY_DT>(raw, page_rsrc(a.pool + blk * PB, (int)PB), 0, lane);
    }
  }
  // row n = n0 + 16 q + m of each tile q: its causally valid keys in this
  // block if its token is in the first run (0 otherwise)
  float best[kWideTiles];
  int nv[kWideTiles];
  const uint8_t* qrow[kWideTiles];  // this lane's staged query row of tile q
  uint32_t full = 0;                // bit q: every row of tile q sees the whole block
  uint32_t act = 0;                 // bit q: tile q has rows in the first run
#pragma unroll
  for (int q = 0; q < kWideTiles; ++q) {
    const int n = n0 + 16 * q + m;
    const int k = (n >> hsh) - t0;
    int v = 0;
    if constexpr (RAGGED) {
      v = n < n1 && k < k1 ? s_len[k] - b * kBlockTokens : 0;
    } else {  // token t = r q + i: length seq_lens[r] - (q - 1 - i)
      const int i = (n >> hsh) - r0 * a.q_len;
      v = n < n1 ? a.seq_lens[r0] - (a.q_len - 1 - i) - b * kBlockTokens : 0;
    }
    nv[q] = v < 0 ? 0 : (v > kBlockTokens ? kBlockTokens : v);
    best[q] = neg_inf();
    qrow[q] = s_q + ((n < n1 ? n : n0) - n0) * QPITCH;
    if (__ballot(nv[q] == kBlockTokens) == ~0ull) full |= 1u << q;
    if (n0 + 16 * q < n1 && ((n0 + 16 * q) >> hsh) - t0 < k1) act |= 1u << q;
  }
  if (b < nr) {
    if (bad) {
#pragma unroll
      for (int q = 0; q < kWideTiles; ++q)
        if (nv[q] > 0) best[q] = qnan();
    } else {
      const __amdgpu_buffer_rsrc_t page = page_rsrc(a.pool + blk * PB, (int)PB);
#pragma unroll
      for (int part = 0; part < PARTS; ++part) {
        PartOps<KEY_DT, Q_DT> ops;
        part_operands<KEY_DT, Q_DT>(raw, lane, ops);
        if (part + 1 < PARTS) load_part_raw<KEY_DT>(raw, page, part + 1, lane);  // in flight during this part
#pragma unroll
        for (int q = 0; q < kWideTiles; ++q)
          if ((act >> q) & 1u)  // wave-uniform
            wide_part_max<KEY_DT, Q_DT>(ops, part, qrow[q], (full >> q) & 1u, nv[q], lane, best[q]);
      }
    }
  }
  if constexpr (RAGGED) {
    if (k1 < ntok)  // tokens of other requests in the tile (wave-uniform)
      wide_other_runs<KEY_DT, Q_DT, kWideTiles>(a.pool, a.pool_blocks, a.bt, a.bt_stride, s_req, s_len, s_q, QPITCH,
                                                n0, n1, t0, hsh, s_best + wave * kWideTiles * kWave, b, k1, ntok,
                                                best);
  }
#pragma unroll
  for (int q = 0; q < kWideTiles; ++q) {
    const int n = n0 + 16 * q + m;
    if (n0 + 16 * q >= n1) continue;  // wave-uniform
    float s = nan_max(best[q], shfl_xor_f32(best[q], 16));  // over the four lane groups
    s = nan_max(s, shfl_xor_f32(s, 32));
    // sum the group's heads: rows n .. n + per - 1 sit on adjacent lanes
    for (int off = 1; off < per; off <<= 1) s += shfl_xor_f32(s, off);
    if (KEY_DT == ISB_FP8_E4M3) s *= a.idx_scale;
    const int h = n & (a.H_idx - 1);
    if (lane < 16 && n < n1 && (h & (per - 1)) == 0) {
      const int gg = h >> psh;
      a.scores[((size_t)gg * a.T + (n >> hsh)) * a.MB + b] = s;
    }
  }
}

// ----------------------------------------------------------------- kernel
// grid (ceil(MB / 4), R), 4 waves a workgroup, wave w scores block 4 x + w.
template <int VARIANT, int KEY_DT, int Q_DT>
__global__ __launch_bounds__(256) void index_score_kernel(ScoreArgs a) {
  __shared__ float s_rowmax[kScoreWaves][kMaxQueryRows];
  __shared__ float s_out[kScoreWaves][kMaxQueryRows];
  __shared__ int s_nvalid[kScoreWaves][16];
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int r = blockIdx.y;
  const int b = score_column<kScoreWaves>(blockIdx.x, gridDim.x, blockIdx.y) * kScoreWaves + wave;
  if (b >= a.MB) return;
  const int L = a.seq_lens[r];
  const int nr = (L + kBlockTokens - 1) / kBlockTokens;
  if (b >= nr) {
    write_scores(a, r, b, lane, nullptr);
    return;
  }
  const int QR = a.q_len * a.H_idx;
  // valid keys of this block for each query token (wave-private LDS)
  for (int i = lane; i < a.q_len; i += kWave) {
    const int v = causal_len(L, a.q_len, i) - b * kBlockTokens;
    s_nvalid[wave][i] = v < 0 ? 0 : (v > kBlockTokens ? kBlockTokens : v);
  }
  const int* nvalid_row = s_nvalid[wave];
  const int64_t blk = __builtin_amdgcn_readfirstlane(a.bt[(size_t)r * a.bt_stride + b]);
  if (blk < 0 || blk >= a.pool_blocks) {
    // An out-of-range block id is poison: NaN where the block is causally
    // visible, -inf elsewhere.  Nothing is read through it.
    for (int x = lane; x < a.q_len * a.H_kv; x += kWave)
      s_out[wave][x] = s_nvalid[wave][x / a.H_kv] > 0 ? qnan() : neg_inf();
    write_scores(a, r, b, lane, s_out[wave]);
    return;
  }
  constexpr int64_t PB = KEY_DT == ISB_BF16 ? 32768 : KEY_DT == ISB_FP8_E4M3 ? 16384 : kMxPageBytes;
  const __amdgpu_buffer_rsrc_t page = page_rsrc(a.pool + blk * PB, (int)PB);
  for (int qt = 0; qt * 16 < QR; ++qt) {
    float best;
    if constexpr (VARIANT == 1) best = tile_block_bf16<KEY_DT, Q_DT>(a, page, r, qt, QR, lane, nvalid_row);
    else best = tile_block_fp4(a, page, r, qt, QR, lane, nvalid_row);
    if (lane < 16 && qt * 16 + lane < QR) s_rowmax[wave][qt * 16 + lane] = best;
  }
  finish<KEY_DT>(a, lane, s_rowmax[wave], s_out[wave]);
  write_scores(a, r, b, lane, s_out[wave]);
}

template <int VARIANT, int KEY_DT, int Q_DT>
static void launch(const ScoreArgs& a, hipStream_t st) {
  if constexpr (VARIANT == 0) {
    const int per = kScoreWaves * stream_blocks<KEY_DT>();
    hipLaunchKernelGGL((index_stream_kernel<KEY_DT, Q_DT>), dim3((a.MB + per - 1) / per, a.R), dim3(256), 0,
                       st, a);
  } else {
    const dim3 grid((a.MB + kScoreWaves - 1) / kScoreWaves, a.R);
    hipLaunchKernelGGL((index_score_kernel<VARIANT, KEY_DT, Q_DT>), grid, dim3(256), 0, st, a);
  }
}

template <int KEY_DT, int Q_DT>
static void launch_wide(const ScoreArgs& a, hipStream_t st) {
  constexpr int TROWS = 16 * kWideTiles;
  const unsigned cols = (a.MB + kScoreWaves - 1) / kScoreWaves;
  dim3 grid;
  if (a.tm.req_id) {
    grid = dim3(cols, (unsigned)(((long long)a.T * a.H_idx + TROWS - 1) / TROWS));
    hipLaunchKernelGGL((index_wide_kernel<KEY_DT, Q_DT, true>), grid, dim3(256), 0, st, a);
  } else {
    const int QR = a.q_len * a.H_idx;
    grid = dim3(cols, a.R, (QR + TROWS - 1) / TROWS);
    hipLaunchKernelGGL((index_wide_kernel<KEY_DT, Q_DT, false>), grid, dim3(256), 0, st, a);
  }
}

template <int KEY_DT, int Q_DT>
static void launch_key(const ScoreArgs& a, bool one_row, bool wide, hipStream_t st) {
  if (wide) {
    launch_wide<KEY_DT, Q_DT>(a, st);
    return;
  }
  if constexpr (KEY_DT == ISB_MXFP4) {
    if constexpr (Q_DT == ISB_FP8_E4M3) launch<2, KEY_DT, Q_DT>(a, st);
    else launch<1, KEY_DT, Q_DT>(a, st);
  } else {
    if (one_row) launch<0, KEY_DT, Q_DT>(a, st);
    else launch<1, KEY_DT, Q_DT>(a, st);
  }
}

}  // namespace isb

namespace isb {

// Dispatch on the key and index-query types.
static void launch_types(const ScoreArgs& a, int q_idx_dtype, int idx_dtype, bool one_row, bool wide,
                         hipStream_t st) {
  const bool qb = q_idx_dtype == ISB_BF16;
  if (idx_dtype == ISB_MXFP4) {
    if (qb) launch_key<ISB_MXFP4, ISB_BF16>(a, one_row, wide, st);
    else launch_key<ISB_MXFP4, ISB_FP8_E4M3>(a, one_row, wide, st);
  } else if (idx_dtype == ISB_FP8_E4M3) {
    if (qb) launch_key<ISB_FP8_E4M3, ISB_BF16>(a, one_row, wide, st);
    else launch_key<ISB_FP8_E4M3, ISB_FP8_E4M3>(a, one_row, wide, st);
  } else {
    if (qb) launch_key<ISB_BF16, ISB_BF16>(a, one_row, wide, st);
    else launch_key<ISB_BF16, ISB_FP8_E4M3>(a, one_row, wide, st);
  }
}

// Checks shared by the two entry points; 0 or an ISB_E_* code.
static int check_score(const void* q_idx, int q_idx_dtype, int num_idx_heads, const void* idx_pool, int idx_dtype,
                       float idx_scale, int64_t idx_pool_blocks, const int32_t* block_table,
                       int block_table_stride, int num_reqs, int num_kv_heads, int max_blocks, float* scores) {
  if (!q_idx || !idx_pool || !block_table || !scores) return ISB_E_INVALID_ARG;
  if (num_idx_heads <= 0 || num_reqs <= 0 || num_kv_heads <= 0 || max_blocks <= 0 || block_table_stride <= 0 ||
      idx_pool_blocks <= 0)
    return ISB_E_INVALID_ARG;
  if (!is_query_dtype(q_idx_dtype) || !is_pool_dtype(idx_dtype)) return ISB_E_UNSUPPORTED_DTYPE;
  if (num_idx_heads % num_kv_heads != 0 || max_blocks > block_table_stride) return ISB_E_SHAPE;
  if (!(idx_scale > 0.f) && idx_dtype == ISB_FP8_E4M3) return ISB_E_INVALID_ARG;
  return ISB_OK;
}

}  // namespace isb

extern "C" int isb_index_score(isb_stream_t stream, const void* q_idx, int q_idx_dtype,
                               int num_idx_heads, const void* idx_pool, int idx_dtype,
                               float idx_scale, int64_t idx_pool_blocks,
                               const int32_t* block_table, int block_table_stride,
                               const int32_t* seq_lens, int num_reqs, int decode_query_len,
                               int num_kv_heads, int max_blocks, float* scores) {
  using namespace isb;
  if (!seq_lens || decode_query_len <= 0) return ISB_E_INVALID_ARG;
  const int err = check_score(q_idx, q_idx_dtype, num_idx_heads, idx_pool, idx_dtype, idx_scale, idx_pool_blocks,
                              block_table, block_table_stride, num_reqs, num_kv_heads, max_blocks, scores);
  if (err) return err;
  // up to 16 tokens and 64 query rows a request: the tile / stream variants;
  // more (a prefill chunk): the wide variant, whose 16-row tiles must hold
  // whole tokens
  const long long QR = (long long)decode_query_len * num_idx_heads;
  const bool wide = decode_query_len > 16 || QR > kMaxQueryRows;
  if (wide && (16 % num_idx_heads != 0 || QR > kMaxWideRows)) return ISB_E_SHAPE;
  if ((long long)num_reqs * decode_query_len > 0x7FFFFFFFLL) return ISB_E_SHAPE;
  if (wide && (long long)num_reqs * QR > 0x7FFFFFFFLL) return ISB_E_SHAPE;
  if (num_reqs > 65535) return ISB_E_SHAPE;
  ScoreArgs a{(const uint8_t*)q_idx, (const uint8_t*)idx_pool, block_table, seq_lens, scores,
              idx_pool_blocks, idx_scale, num_idx_heads, block_table_stride, num_reqs,
              decode_query_len, num_kv_heads, max_blocks, decode_map(seq_lens, decode_query_len),
              num_reqs * decode_query_len};
  launch_types(a, q_idx_dtype, idx_dtype, decode_query_len * num_idx_heads == 1, wide, as_hip(stream));
  return launch_status();
}

extern "C" int isb_index_score_prefill(isb_stream_t stream, const void* q_idx, int q_idx_dtype,
                                       int num_idx_heads, const void* idx_pool, int idx_dtype,
                                       float idx_scale, int64_t idx_pool_blocks,
                                       const int32_t* block_table, int block_table_stride, int num_reqs,
                                       const int32_t* query_req_id, const int32_t* query_abs_pos,
                                       int num_tokens, int num_kv_heads, int max_blocks, float* scores) {
  using namespace isb;
  if (!query_req_id || !query_abs_pos || num_tokens <= 0) return ISB_E_INVALID_ARG;
  const int err = check_score(q_idx, q_idx_dtype, num_idx_heads, idx_pool, idx_dtype, idx_scale, idx_pool_blocks,
                              block_table, block_table_stride, num_reqs, num_kv_heads, max_blocks, scores);
  if (err) return err;
  if (16 % num_idx_heads != 0) return ISB_E_SHAPE;
  const long long rows = (long long)num_tokens * num_idx_heads;
  if (rows > 0x7FFFFFFFLL || (rows + 16 * kWideTiles - 1) / (16 * kWideTiles) > 65535) return ISB_E_SHAPE;
  ScoreArgs a{(const uint8_t*)q_idx, (const uint8_t*)idx_pool, block_table, nullptr, scores,
              idx_pool_blocks, idx_scale, num_idx_heads, block_table_stride, num_reqs,
              1, num_kv_heads, max_blocks, prefill_map(query_req_id, query_abs_pos, num_reqs, max_blocks),
              num_tokens};
  launch_types(a, q_idx_dtype, idx_dtype, false, true, as_hip(stream));
  return launch_status();
}
