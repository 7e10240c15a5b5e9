// isb_sparse_pa_decode: split-K flash decode over the selected pages; the
// last workgroup to finish a row merges the row's splits, in the same launch.
//
// The decode call of the vLLM API page for sparse_attention_msa
// (minimax_m3_sparse_attn_decode_aiter with the emitted sparse_block_table and
// sparse_context_lens): per row (token, KV head) and query head of that KV
// group, softmax(scale q.K) V over the sparse positions.  MXFP4 K/V follow
// ROCm/ATOM PR 2962 (Summary: MXFP4 K and V pages, one row per token and KV
// head).
//
// Work decomposition.  A row's pages are cut into splits; one workgroup of
// four waves attends one split, a round (four runs, one a wave) at a time.  A
// wave issues every load of its run (8 fp8 / 4 bf16 16-token pages, or one
// 128-token MXFP4 page) before any math, computes every logit of the run,
// takes one exact maximum per head, rescales what earlier rounds accumulated
// if that maximum grew, then adds the probabilities' P.V.  The four waves
// merge in LDS, the splits of a row through the workspace.  Small batches
// take several splits a row (every page of the batch in flight in one round);
// batches that fill the chip take one split a row and nothing is merged
// between workgroups.
//   S^T (16 keys x 16 heads) = K_tile . Q^T      v_mfma_f32_16x16x32_bf16, or
//                                                one scaled fp4 x fp8 MFMA
//   O^T (128 dims x 16 heads) += V^T . P^T       v_mfma_f32_16x16x{32,16}_bf16
// The G <= 16 query heads of a KV group fill the MFMA's 16 columns, so K and V
// bytes are read once per row and reused by every head.  K and V are
// dequantised to bf16 in registers (exact for e4m3 and for e2m1 x 2^k); the
// per-tensor fp8 scales and the softmax scale are folded into one logit
// multiplier (k_scale sm_scale log2 e) and the output (v_scale).
//
// Operand layout (lane = 16 g + c):
//   K tile, A of QK:  key c of the tile, dims 32 g .. 32 g + 31 (MFMA j takes
//                     dims 32 g + 8 j .. + 7);  Q^T, B of QK: head c, same dims;
//   S^T result:       lane holds keys 4 g + e (e < 4) of head c;
//   P^T, B of PV:     exactly that: head c, keys 4 g + e;
//   V^T, A of PV:     row r of MFMA dt is one dim, keys 4 g + e;
//   O^T result:       lane holds rows 4 g + e of each dt, head c.
// Every value a lane holds belongs to its head c, so the softmax needs only
// lane-group reductions.
//
// 16-token (bf16 / fp8) pages are stored lane-native: the 16-byte chunk h of
// lane l sits at byte 1024 h + 16 l of the K page and of the V page (K: dims
// 32 g + 16 h .. of key c for fp8; V: dim tiles 4 h .. 4 h + 3, keys 4 g ..
// 4 g + 3 of dim c for fp8), so every load instruction reads one contiguous
// KiB and row r of V^T tile dt is dim 16 dt + r.
// 128-token MXFP4 pages are token-major (the page format of the MXFP4 cache).
// K: lane (g, c) of tile t loads the 16 bytes of token 16 t + c that hold dims
// 32 g .., and their e8m0 scale; with an e4m3 query the scaled MFMA multiplies
// them as stored.  V: lane (g, c) loads, for each of its keys, the 4-byte
// word that holds dims 8 c .. 8 c + 7, and for each tile the 16 bytes of
// scales of its four keys, straight from the page, so row r of V^T tile dt is
// dim 8 r + dt.
//
// Page loads are raw buffer loads from a wave-uniform descriptor of the page
// (one offset register a wave).  When a request has several query tokens (a
// prefill chunk, speculative tokens) its rows share most of their pages, and
// the loads keep the default cache policy so that the rows after the first
// find those pages in L2; with one token a request no page is read twice in a
// launch, and 16-token pages are streamed past the caches (nontemporal
// loads), which raises the rate the memory system delivers them at.
#include <mutex>

#include "grid_maps.h"
#include "isb_device.h"
#include "isb_host.h"
#include "select_device.h"

namespace isb {

struct PaArgs {
  const uint8_t* q;
  const uint8_t* kp;
  const uint8_t* vp;
  const int32_t* sbt;
  const int32_t* sctx;
  float* part_o;
  float* part_ml;
  __bf16* out;
  int64_t num_pages;
  float qk_scale;  // sm_scale * k_scale * log2(e)
  float v_scale;
  int sbt_stride, H_q, H_kv, G, splits, pps;
};

constexpr int kMergeGroup = 8;  // splits whose partials the merging workgroup loads at once

template <int Q_DT>
__device__ __forceinline__ bf16x8 load_q8_t(const uint8_t* row, int dim0) {
  if constexpr (Q_DT == ISB_BF16) {
    return u32x4_as_bf16x8(ld16(row + 2 * dim0));
  } else {
    const u32x2 w = ld8(row + dim0);
    return e4m3x8_to_bf16x8(w[0], w[1]);
  }
}

__device__ __forceinline__ bool page_ok(int64_t id, int64_t n) { return id >= 0 && id < n; }

// Per-workgroup LDS of the merge: each wave's per-head max and sum, and its
// unnormalised output O[head][dim].
template <int NW>
struct alignas(16) WaveParts {
  float m[NW][16];
  float l[NW][16];
  float o[NW][16][kHeadDim + 4];
};

// Split partials in the workspace.  A free slot holds zero in every word; a
// published word holds the bitwise complement of its value, which is never
// zero (NaNs are published as the canonical quiet NaN, and no value has all
// 32 bits set), so every word tells by itself whether it has landed.
__device__ __forceinline__ void publish_word(float* p, float x) {
  const uint32_t bits = x != x ? __float_as_uint(qnan()) : __float_as_uint(x);
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), ~bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void free_word(float* p) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t read_word(const float* p) {
  return __hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool published(uint32_t w) { return w != 0u; }
__device__ __forceinline__ float word_value(uint32_t w) { return __uint_as_float(~w); }

// The workgroup's share of a row, once every wave has written its part: merge
// the waves; a row of one split is finished here.  Otherwise the split
// publishes its partial (agent-coherent stores, thread-interleaved: element x
// of thread i at 256 x + i, so each store covers 256 contiguous bytes), waits
// until its stores are complete, then reads the partials of the row's other
// splits.  A workgroup that finds every word of them published merges the
// row (log-sum-exp weights, in split order, so the result does not depend on
// which workgroup merges), writes it and frees the row's slots for the next
// call.  The split whose stores complete last always finds the others
// published, so every row is merged; two workgroups that both find them
// write the same bytes.  Nothing waits for another workgroup, and only
// coherent (agent-scope) accesses touch the partials, so no cache writeback
// or invalidation is needed between workgroups on different dies.  Thread
// (h, d0) = (tid / 16, 8 (tid % 16)) of the first 256 owns dims d0 .. d0 + 7
// of head h.
template <int NW>
__device__ __forceinline__ void finish_split(const PaArgs& a, WaveParts<NW>& wp, int row, int split, int live,
                                             __bf16* out_row) {
  const int tid = threadIdx.x;
  const int h = (tid >> 4) & 15, d0 = 8 * (tid & 15);
  const bool mine = tid < 256 && h < a.G;
  __syncthreads();
  float M = neg_inf(), L = 0.f, O[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (tid < 256) {
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, wp.m[w][h]);
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = wp.m[w][h];
      const float wt = mw == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L += wp.l[w][h] * wt;
      const f32x4 lo = *reinterpret_cast<const f32x4*>(&wp.o[w][h][d0]);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(&wp.o[w][h][d0 + 4]);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        O[x] += lo[x] * wt;
        O[4 + x] += hi[x] * wt;
      }
    }
  }

  if (live > 1) {
    const size_t rbase = (size_t)row * a.splits;
    if (mine) {
      float* po = a.part_o + (rbase + split) * kPartialO + tid;
#pragma unroll
      for (int x = 0; x < 8; ++x) publish_word(po + 256 * x, O[x]);
      if ((tid & 15) == 0) {
        publish_word(a.part_ml + ((rbase + split) * 16 + h) * 2 + 0, M);
        publish_word(a.part_ml + ((rbase + split) * 16 + h) * 2 + 1, L);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this thread's stores are complete
    __syncthreads();                // ... and every thread's, before any reads back
    // The other live splits, kMergeGroup at a time (every load of a group
    // issued first), merged in split order as they come; whether they were
    // all published is known only at the end, and decides whether this
    // workgroup writes the row.
    bool valid = true;
    const float Mo = M, Lo = L;
    float Oo[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) Oo[x] = O[x];
    M = neg_inf();
    L = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) O[x] = 0.f;
    if (mine) {
      for (int s0 = 0; s0 < live; s0 += kMergeGroup) {
        uint32_t ms[kMergeGroup], ls[kMergeGroup], os[kMergeGroup][8];
#pragma unroll
        for (int k = 0; k < kMergeGroup; ++k) {
          const int sp = s0 + k;
          if (sp < live && sp != split) {  // a wave-uniform branch
            const size_t b = (rbase + sp) * 16 + h;
            ms[k] = read_word(a.part_ml + b * 2 + 0);
            ls[k] = read_word(a.part_ml + b * 2 + 1);
            const float* pk = a.part_o + (rbase + sp) * kPartialO + tid;
#pragma unroll
            for (int x = 0; x < 8; ++x) os[k][x] = read_word(pk + 256 * x);
          }
        }
#pragma unroll
        for (int k = 0; k < kMergeGroup; ++k) {
          const int sp = s0 + k;
          if (sp >= live) break;
          const bool own = sp == split;
          if (!own) {
            bool ok = published(ms[k]) && published(ls[k]);
#pragma unroll
            for (int x = 0; x < 8; ++x) ok = ok && published(os[k][x]);
            valid = valid && ok;
          }
          const float mk = own ? Mo : word_value(ms[k]);
          if (mk == neg_inf()) continue;
          const float Mn = fmaxf(M, mk);
          const float wa = M == neg_inf() ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
          const float wb = __builtin_amdgcn_exp2f(mk - Mn);
          L = L * wa + (own ? Lo : word_value(ls[k])) * wb;
#pragma unroll
          for (int x = 0; x < 8; ++x) O[x] = O[x] * wa + (own ? Oo[x] : word_value(os[k][x])) * wb;
          M = Mn;
        }
      }
    }
    if (!__syncthreads_and(valid)) return;  // another split is still to publish: it merges the row
    if (mine) {  // free the row's slots for the next call
      for (int sp = 0; sp < live; ++sp) {
        float* po = a.part_o + (rbase + sp) * kPartialO + tid;
#pragma unroll
        for (int x = 0; x < 8; ++x) free_word(po + 256 * x);
        if ((tid & 15) == 0) {
          free_word(a.part_ml + ((rbase + sp) * 16 + h) * 2 + 0);
          free_word(a.part_ml + ((rbase + sp) * 16 + h) * 2 + 1);
        }
      }
    }
  }
  // Finished row: normalise and write bf16 (nontemporal: nothing here reads
  // it back).
  if (mine) {
    const float inv = a.v_scale / L;
    bf16x8 ob;
#pragma unroll
    for (int x = 0; x < 8; ++x) ob[x] = (__bf16)(O[x] * inv);
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, ob),
                                reinterpret_cast<u32x4*>(out_row + h * kHeadDim + d0));
  }
}

// A row with nothing to attend outputs zeros (split 0 writes them).
__device__ __forceinline__ void write_empty_row(const PaArgs& a, int split, __bf16* out_row) {
  const int h = threadIdx.x >> 4, d0 = 8 * (threadIdx.x & 15);
  if (split == 0 && threadIdx.x < 256 && h < a.G) {
    bf16x8 z;
#pragma unroll
    for (int x = 0; x < 8; ++x) z[x] = (__bf16)0.f;
    *reinterpret_cast<bf16x8*>(out_row + h * kHeadDim + d0) = z;
  }
}

// A wave's result in LDS; row r of V^T tile dt is dim DIM_MUL r + DT_MUL dt.
template <int DIM_MUL, int DT_MUL, int NW>
__device__ __forceinline__ void wave_to_lds(WaveParts<NW>& wp, int wave, int lane, float m, float l,
                                            const f32x4 (&o)[8]) {
  const int c = lane & 15, g = lane >> 4;
  const float l_tot = sum_over_groups(l);
  if (lane < 16) {
    wp.m[wave][c] = m;
    wp.l[wave][c] = l_tot;
  }
  if constexpr (DIM_MUL == 1) {  // dims 4 g .. 4 g + 3 of tile dt are adjacent: one 16-byte store
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(&wp.o[wave][c][4 * g + DT_MUL * dt]) = o[dt];
  } else {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) wp.o[wave][c][DIM_MUL * (4 * g + e) + DT_MUL * dt] = o[dt][e];
  }
}

// Query columns past the group's G heads are zero (they were loaded from head
// 0 so the load needs no branch).
__device__ __forceinline__ void zero_missing_heads(bf16x8 (&qb)[4], int c, int G) {
  if (c >= G) {
#pragma unroll
    for (int j = 0; j < 4; ++j) qb[j] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
}

// ----------------------------------------------------------------- 16-token pages
// Raw bytes of one page for this lane: NC 16-byte chunks of K and of V.
template <int KV_DT>
struct PageRegs {
  static constexpr int NC = KV_DT == ISB_BF16 ? 4 : 2;
  u32x4 k[NC];
  u32x4 v[NC];
};

template <int KV_DT, bool NT>
__device__ __forceinline__ void load_k16(PageRegs<KV_DT>& pr, __amdgpu_buffer_rsrc_t kpage, int lane) {
#pragma unroll
  for (int h = 0; h < PageRegs<KV_DT>::NC; ++h)
    pr.k[h] = NT ? bl16_nt(kpage, 1024 * h + 16 * lane, 0) : bl16(kpage, 1024 * h + 16 * lane, 0);
}
template <int KV_DT, bool NT>
__device__ __forceinline__ void load_v16(PageRegs<KV_DT>& pr, __amdgpu_buffer_rsrc_t vpage, int lane) {
#pragma unroll
  for (int h = 0; h < PageRegs<KV_DT>::NC; ++h)
    pr.v[h] = NT ? bl16_nt(vpage, 1024 * h + 16 * lane, 0) : bl16(vpage, 1024 * h + 16 * lane, 0);
}

// Keys at or past nvalid in a page may hold anything (0 x NaN would poison
// the sum), so their raw V bytes are cleared before conversion.  Lane
// (g, c) holds keys 4 g .. 4 g + 3: one byte each per fp8 dword, two keys per
// bf16 dword (keys 4 g, 4 g + 1 in dword 2q, 4 g + 2, 4 g + 3 in dword 2q + 1).
template <int KV_DT>
__device__ __forceinline__ void clear_tail_keys(PageRegs<KV_DT>& pr, int nvalid, int g) {
  const int keep = min(4, max(0, nvalid - 4 * g));  // keys of this lane that count
  if constexpr (KV_DT == ISB_BF16) {
    const uint64_t m64 = keep >= 4 ? ~0ull : ((1ull << (16 * keep)) - 1ull);
    const uint32_t lo = (uint32_t)m64, hi = (uint32_t)(m64 >> 32);
#pragma unroll
    for (int h = 0; h < PageRegs<KV_DT>::NC; ++h) {
      pr.v[h][0] &= lo;
      pr.v[h][1] &= hi;
      pr.v[h][2] &= lo;
      pr.v[h][3] &= hi;
    }
  } else {
    const uint32_t m = keep >= 4 ? ~0u : ((1u << (8 * keep)) - 1u);
#pragma unroll
    for (int h = 0; h < PageRegs<KV_DT>::NC; ++h) pr.v[h] &= m;
  }
}

// K operand of one page: fp8 chunk h holds dims 32 g + 16 h .. + 15 (kb[2h],
// kb[2h+1]); bf16 chunk h holds dims 32 g + 8 h .. + 7 (kb[h]).
template <int KV_DT>
__device__ __forceinline__ void k_operand(const PageRegs<KV_DT>& pr, bf16x8 (&kb)[4]) {
  if constexpr (KV_DT == ISB_BF16) {
#pragma unroll
    for (int h = 0; h < 4; ++h) kb[h] = u32x4_as_bf16x8(pr.k[h]);
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int q = 0; q < 2; ++q) kb[2 * h + q] = e4m3x8_to_bf16x8(pr.k[h][2 * q], pr.k[h][2 * q + 1]);
  }
}

// Operand type of P.V: bf16 for bf16 V; f16 for fp8 V, whose e4m3 values
// convert to f16 exactly as well, so the probabilities keep 11 significant
// bits instead of bf16's 8 (a quarter of the rounding error in the output).
template <int KV_DT>
struct PvType {
  using vec = bf16x8;
  using elem = __bf16;
};
template <>
struct PvType<ISB_FP8_E4M3> {
  using vec = f16x8;
  using elem = _Float16;
};
template <int KV_DT>
using pv_vec = typename PvType<KV_DT>::vec;

// v_mfma_f32_16x16x32 of P.V in the operand type of the pages.
template <int KV_DT, bool KEEP>
__device__ __forceinline__ f32x4 pv_mfma(pv_vec<KV_DT> v, pv_vec<KV_DT> p, f32x4 o) {
  if constexpr (KV_DT == ISB_FP8_E4M3) return mfma_16x16x32_f16_k<KEEP>(v, p, o);
  else return mfma_16x16x32_bf16_k<KEEP>(v, p, o);
}

// V^T operand of dim tile dt for a pair of pages (keys 4 g + e of the first
// page, then of the second), as the P.V MFMA wants it.
template <int KV_DT>
__device__ __forceinline__ pv_vec<KV_DT> v_pair_operand(const PageRegs<KV_DT>& a, const PageRegs<KV_DT>& b,
                                                        int dt) {
  if constexpr (KV_DT == ISB_BF16) {
    const int h = dt >> 1, q = dt & 1;
    return __builtin_bit_cast(bf16x8, u32x4{a.v[h][2 * q], a.v[h][2 * q + 1], b.v[h][2 * q], b.v[h][2 * q + 1]});
  } else {
    const int h = dt >> 2, q = dt & 3;
    return e4m3x8_to_f16x8(a.v[h][q], b.v[h][q]);
  }
}

// The pieces of a run for the one-wave-a-row pipeline (attend_row_wave16),
// which issues the next run's loads between this run's passes.  A run of a
// wave: up to RUN consecutive pages of its row, their raw bytes and where they
// come from.
template <int KV_DT, int RUN>
struct RunRegs {
  PageRegs<KV_DT> pr[RUN];
  bool ok[RUN];      // the page id is in range (else page 0 is read and the tile poisoned)
  int64_t use[RUN];  // byte offset of the page's K (and V) in its pool
};

// The run's page ids: lanes ibase .. ibase + cnt - 1 of my_ids (cnt >= 1);
// slots past the run re-read its first page.
template <int KV_DT, int RUN>
__device__ __forceinline__ void run_pages(const PaArgs& a, RunRegs<KV_DT, RUN>& rr, int cnt, int my_ids, int ibase,
                                          int64_t hstride, int64_t hoff) {
#pragma unroll
  for (int j = 0; j < RUN; ++j) {
    const int64_t id = __builtin_amdgcn_readlane(my_ids, ibase + (j < cnt ? j : 0));
    rr.ok[j] = page_ok(id, a.num_pages);
    rr.use[j] = (rr.ok[j] ? id : 0) * hstride + hoff;
  }
}

// Every K load of the run, then (separately) every V load, page by page and
// kept in that order, so the logits of page j wait only for K of pages <= j
// and P.V of page j only for V of pages <= j.  live false: the loads are
// issued against an empty range (they return zeros and read no memory).
template <int KV_DT, int RUN, bool NT>
__device__ __forceinline__ void issue_k_run(const PaArgs& a, RunRegs<KV_DT, RUN>& rr, int lane,
                                            bool live = true) {
  constexpr int PB = KV_DT == ISB_BF16 ? 4096 : 2048;
  __builtin_amdgcn_sched_barrier(0);  // no load of the run moves above what comes before
#pragma unroll
  for (int j = 0; j < RUN; ++j) {
    load_k16<KV_DT, NT>(rr.pr[j], page_rsrc(a.kp + rr.use[j], live ? PB : 0), lane);
    __builtin_amdgcn_sched_barrier(0);
  }
}
template <int KV_DT, int RUN, bool NT>
__device__ __forceinline__ void issue_v_run(const PaArgs& a, RunRegs<KV_DT, RUN>& rr, int lane,
                                            bool live = true) {
  constexpr int PB = KV_DT == ISB_BF16 ? 4096 : 2048;
  __builtin_amdgcn_sched_barrier(0);  // no load of the run moves above what comes before
#pragma unroll
  for (int j = 0; j < RUN; ++j) {
    load_v16<KV_DT, NT>(rr.pr[j], page_rsrc(a.vp + rr.use[j], live ? PB : 0), lane);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Pass 1 of a run (pages wb .. wb + cnt - 1 of the row, raw bytes in pr,
// ok[j]: page j's id was in range): every logit z of the run, then one exact
// max per head, folded into the running max M (rescaling what earlier runs
// accumulated if it grew).  Uses the run's K registers (and clears the V
// bytes of keys past the row's length on its last page).  KEEP: pin MFMA
// operands live (see mfma_16x16x32_bf16_k).
template <int KV_DT, int Q_DT, int RUN, bool KEEP>
__device__ __forceinline__ void run_logits(const PaArgs& a, PageRegs<KV_DT> (&pr)[RUN], const bool (&ok)[RUN],
                                           int lane, int n_tok, int wb, int cnt, const bf16x8 (&qb)[4], bool first,
                                           float& M, float& lsum, f32x4 (&o)[8], float (&z)[RUN][4]) {
  const int g = lane >> 4;
  float mx = neg_inf();
#pragma unroll
  for (int j = 0; j < RUN; ++j) {
    if (j < cnt) {
      bf16x8 kb[4];
      k_operand<KV_DT>(pr[j], kb);
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int x = 0; x < 4; ++x) sacc = mfma_16x16x32_bf16_k<KEEP>(kb[x], qb[x], sacc);
#pragma unroll
      for (int e = 0; e < 4; ++e) z[j][e] = sacc[e] * a.qk_scale;
      const int nv = min(16, n_tok - (wb + j) * 16);
      if (nv < 16) {  // the row's last page: keys past its length do not count
#pragma unroll
        for (int e = 0; e < 4; ++e) z[j][e] = 4 * g + e < nv ? z[j][e] : neg_inf();
        clear_tail_keys<KV_DT>(pr[j], nv, g);
      }
      if (!ok[j]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) z[j][e] = qnan();
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, z[j][e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) z[j][e] = neg_inf();
    }
  }
  mx = max_over_groups(mx);
  const float m_new = fmaxf(M, mx);
  if (!first) {
    const float alpha = M == m_new ? 1.f : __builtin_amdgcn_exp2f(M - m_new);
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
  }
  M = m_new;
}

// Pass 1 for the pipeline, which then holds the run's probabilities rather
// than its logits while the next run's K loads are in flight: keys 4 g + e of
// pages j and j + 1 in pb[j / 2] (in the P.V operand type), their
// fp32 sum into lsum.
template <int KV_DT, int Q_DT, int RUN, bool KEEP>
__device__ __forceinline__ void logits_run(const PaArgs& a, RunRegs<KV_DT, RUN>& rr, int lane, int n_tok, int wb,
                                           int cnt, const bf16x8 (&qb)[4], bool first, float& M, float& lsum,
                                           f32x4 (&o)[8], pv_vec<KV_DT> (&pb)[RUN / 2]) {
  float z[RUN][4];
  run_logits<KV_DT, Q_DT, RUN, KEEP>(a, rr.pr, rr.ok, lane, n_tok, wb, cnt, qb, first, M, lsum, o, z);
#pragma unroll
  for (int j = 0; j < RUN; j += 2) {
    if (j < cnt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0v = __builtin_amdgcn_exp2f(z[j][e] - M);
        const float p1v = __builtin_amdgcn_exp2f(z[j + 1][e] - M);
        lsum += p0v + p1v;
        pb[j / 2][e] = (typename PvType<KV_DT>::elem)p0v;
        pb[j / 2][4 + e] = (typename PvType<KV_DT>::elem)p1v;
      }
    }
  }
}

// Pass 2 of a run: P.V, two pages per MFMA (keys 4 g + e of the first page,
// then of the second, on pv_mfma).  Uses the run's V registers.
template <int KV_DT, int RUN, bool KEEP>
__device__ __forceinline__ void pv_run(RunRegs<KV_DT, RUN>& rr, int lane, int cnt, const pv_vec<KV_DT> (&pb)[RUN / 2],
                                       f32x4 (&o)[8]) {
  const int g = lane >> 4;
#pragma unroll
  for (int j = 0; j < RUN; j += 2) {
    if (j < cnt) {
      if (j + 1 >= cnt) clear_tail_keys<KV_DT>(rr.pr[j + 1], 0, g);  // a run's odd last slot
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        o[dt] = pv_mfma<KV_DT, KEEP>(v_pair_operand<KV_DT>(rr.pr[j], rr.pr[j + 1], dt), pb[j / 2], o[dt]);
    }
  }
}

// One run of a wave: pages wb .. wb + cnt - 1 of its row (cnt >= 1, at most
// RUN), whose ids sit in lanes ibase .. ibase + cnt - 1 of my_ids, folded into
// the wave's running max M (per head), sum share lsum and output o.  Every
// load of the run is issued before any math; its logits give one exact max
// per head, which rescales what earlier runs accumulated if it grew.
// KEEP: pin MFMA operands live (see mfma_16x16x32_bf16_k).
template <int KV_DT, int Q_DT, int RUN, bool NT, bool KEEP>
__device__ __forceinline__ void attend_run16(const PaArgs& a, int lane, int n_tok, int wb, int cnt, int my_ids,
                                             int ibase, int64_t hstride, int64_t hoff, const bf16x8 (&qb)[4],
                                             bool first, float& M, float& lsum, f32x4 (&o)[8]) {
  constexpr int PB = KV_DT == ISB_BF16 ? 4096 : 2048;
  const int g = lane >> 4;
  // Every load of the run, unconditionally: slots past the run re-read its
  // first page, an out-of-range id reads page 0 and poisons its tile.  All
  // K chunks are issued before all V chunks, page by page, and kept in that
  // order, so the logits of page j wait only for K of pages <= j and P.V of
  // page j only for V of pages <= j.
  PageRegs<KV_DT> pr[RUN];
  bool ok[RUN];
  int64_t use[RUN];
#pragma unroll
  for (int j = 0; j < RUN; ++j) {
    const int64_t id = __builtin_amdgcn_readlane(my_ids, ibase + (j < cnt ? j : 0));
    ok[j] = page_ok(id, a.num_pages);
    use[j] = (ok[j] ? id : 0) * hstride + hoff;
    load_k16<KV_DT, NT>(pr[j], page_rsrc(a.kp + use[j], PB), lane);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int j = 0; j < RUN; ++j) {
    load_v16<KV_DT, NT>(pr[j], page_rsrc(a.vp + use[j], PB), lane);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Pass 1: every logit of the run, then one exact max per head.
  float z[RUN][4];
  run_logits<KV_DT, Q_DT, RUN, KEEP>(a, pr, ok, lane, n_tok, wb, cnt, qb, first, M, lsum, o, z);
  // Pass 2: probabilities and P.V, two pages per MFMA (keys 4 g + e of the
  // first page, then of the second, on pv_mfma).
#pragma unroll
  for (int j = 0; j < RUN; j += 2) {
    if (j < cnt) {
      pv_vec<KV_DT> pb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0v = __builtin_amdgcn_exp2f(z[j][e] - M);
        const float p1v = __builtin_amdgcn_exp2f(z[j + 1][e] - M);
        lsum += p0v + p1v;
        pb[e] = (typename PvType<KV_DT>::elem)p0v;
        pb[4 + e] = (typename PvType<KV_DT>::elem)p1v;
      }
      if (j + 1 >= cnt) clear_tail_keys<KV_DT>(pr[j + 1], 0, g);  // a run's odd last slot
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        o[dt] = pv_mfma<KV_DT, KEEP>(v_pair_operand<KV_DT>(pr[j], pr[j + 1], dt), pb, o[dt]);
    }
  }
}

// The attention of one split of row `row` (token t = row / H_kv, KV head kvh),
// given its sparse length, its query operand qb, this lane's page id for the
// first rounds (my_ids = ids(0)) and `ids(r0)`: this lane's page id for round
// r0 + lane / RUN, slot lane % RUN of this wave's run (-1 past the split).
// A split is walked one round (one run a wave) at a time.
template <int KV_DT, int Q_DT, int RUN, bool NT, int NW, typename IdFn>
__device__ __forceinline__ void attend_split16(const PaArgs& a, WaveParts<NW>& wp, int row, int split, int kvh,
                                               int n_tok, bf16x8 (&qb)[4], int my_ids, IdFn ids,
                                               __bf16* out_row) {
  static_assert(RUN % 2 == 0, "P.V takes the pages of a run in pairs");
  constexpr int PB = KV_DT == ISB_BF16 ? 4096 : 2048;
  constexpr int ROUND = NW * RUN;   // pages of a round
  constexpr int IDS = 64 / RUN;     // rounds whose page ids one id fetch holds
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int p0 = split * a.pps;
  if (n_tok <= 0) {
    write_empty_row(a, split, out_row);
    return;
  }
  // a row never lists more pages than its table row holds
  const int npages = min((n_tok + 15) / 16, a.sbt_stride);
  if (p0 >= npages) return;
  const int p1 = min(npages, p0 + a.pps);
  const int live = (npages + a.pps - 1) / a.pps;  // splits of this row that have pages
  const int nrounds = (p1 - p0 + ROUND - 1) / ROUND;
  zero_missing_heads(qb, c, a.G);

  float M = neg_inf(), lsum = 0.f;  // running max (per head) and this lane's share of the sum
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int64_t hstride = (int64_t)a.H_kv * PB;  // bytes per page id (all heads)
  const int64_t hoff = (int64_t)kvh * PB;
  bool first = true;
  for (int r = 0; r < nrounds; ++r) {
    if (r > 0 && r % IDS == 0) my_ids = ids(r);
    const int wb = p0 + r * ROUND + wave * RUN;
    const int cnt = max(0, min(RUN, p1 - wb));
    if (cnt == 0) continue;  // wave-uniform: this wave has nothing left in the split
    attend_run16<KV_DT, Q_DT, RUN, NT, NW == 8>(a, lane, n_tok, wb, cnt, my_ids, (r % IDS) * RUN, hstride, hoff,
                                                qb, first, M, lsum, o);
    first = false;
  }
  wave_to_lds<1, 16, NW>(wp, wave, lane, M, lsum, o);  // row r of tile dt: dim 16 dt + r
  finish_split<NW>(a, wp, row, split, live, out_row);
}

// The whole of row `row` by one wave, its runs one after another (rows that
// fill the chip by themselves: no split, no merge); writes the row's output
// straight from the wave's registers.  my_ids, ids(r0): this lane's page id
// for run r0 + lane / RUN, slot lane % RUN.
template <int KV_DT, int Q_DT, int RUN, bool NT, typename IdFn>
__device__ __forceinline__ void attend_row_wave16(const PaArgs& a, int kvh, int n_tok, bf16x8 (&qb)[4],
                                                  int my_ids, IdFn ids, __bf16* out_row, bf16x8* s_qb) {
  constexpr int PB = KV_DT == ISB_BF16 ? 4096 : 2048;
  constexpr int IDS = 64 / RUN;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const bool mine = c < a.G;
  if (n_tok <= 0) {
    if (mine) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<bf16x4*>(out_row + c * kHeadDim + 16 * dt + 4 * g) = bf16x4{0, 0, 0, 0};
    }
    return;
  }
  const int npages = min((n_tok + 15) / 16, a.sbt_stride);
  const int nruns = (npages + RUN - 1) / RUN;
  zero_missing_heads(qb, c, a.G);
  float M = neg_inf(), lsum = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int64_t hstride = (int64_t)a.H_kv * PB;
  const int64_t hoff = (int64_t)kvh * PB;
  // The runs in a pipeline: the next run's K loads are issued once this
  // run's logits have consumed its K registers, and its V loads once this
  // run's P.V has consumed its V registers, so they are in flight during this
  // run's math without registers of their own.  The query operand waits in
  // this wave's LDS slice s_qb and is read back for each run's logits.
#pragma unroll
  for (int j = 0; j < 4; ++j) s_qb[4 * lane + j] = qb[j];
  RunRegs<KV_DT, RUN> rr;
  run_pages<KV_DT, RUN>(a, rr, min(RUN, npages), my_ids, 0, hstride, hoff);
  issue_k_run<KV_DT, RUN, NT>(a, rr, lane);
  issue_v_run<KV_DT, RUN, NT>(a, rr, lane);
  for (int r = 0; r < nruns; ++r) {
    const int wb = r * RUN, cnt = min(RUN, npages - wb);
    pv_vec<KV_DT> pb[RUN / 2];
    bf16x8 qr[4];
    asm volatile("" ::: "memory");  // read the query back each run, not kept in registers
#pragma unroll
    for (int j = 0; j < 4; ++j) qr[j] = s_qb[4 * lane + j];
    logits_run<KV_DT, Q_DT, RUN, false>(a, rr, lane, n_tok, wb, cnt, qr, r == 0, M, lsum, o, pb);
    // the next run (after the last one: loads of an empty range, so the
    // loop needs no branch around them)
    const bool more = r + 1 < nruns;
    if (more && (r + 1) % IDS == 0) my_ids = ids(r + 1);
    const int nx = more ? r + 1 : r;
    run_pages<KV_DT, RUN>(a, rr, min(RUN, npages - nx * RUN), my_ids, (nx % IDS) * RUN, hstride, hoff);
    issue_k_run<KV_DT, RUN, NT>(a, rr, lane, more);
    pv_run<KV_DT, RUN, false>(rr, lane, cnt, pb, o);
    issue_v_run<KV_DT, RUN, NT>(a, rr, lane, more);
  }
  // lane (g, c): dims 16 dt + 4 g + e of head c
  const float inv = a.v_scale / sum_over_groups(lsum);
  if (mine) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const bf16x4 ob = {(__bf16)(o[dt][0] * inv), (__bf16)(o[dt][1] * inv), (__bf16)(o[dt][2] * inv),
                         (__bf16)(o[dt][3] * inv)};
      __builtin_nontemporal_store(__builtin_bit_cast(u32x2, ob),
                                  reinterpret_cast<u32x2*>(out_row + c * kHeadDim + 16 * dt + 4 * g));
    }
  }
}

// RUN: pages of one wave's run (a power of two); NT: nontemporal page loads;
// NW: waves a workgroup.  grid (rows, splits); page ids come from the sparse
// page table.
template <int KV_DT, int Q_DT, int RUN, bool NT, int NW>
__global__ __launch_bounds__(64 * NW) void pa16_kernel(PaArgs a) {
  constexpr int QB = Q_DT == ISB_BF16 ? 2 : 1;
  constexpr int ROUND = NW * RUN;
  __shared__ WaveParts<NW> wp;
  const int row = grid_row(blockIdx.x, gridDim.x), split = blockIdx.y;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int t = row / a.H_kv, kvh = row % a.H_kv;
  const int32_t* pages = a.sbt + (size_t)row * a.sbt_stride;
  const int p0 = split * a.pps;
  const int pend = min(a.sbt_stride, p0 + a.pps);
  auto load_ids = [&](int r0) {
    const int pidx = p0 + (r0 + lane / RUN) * ROUND + wave * RUN + lane % RUN;
    return pidx < pend ? pages[pidx] : -1;
  };
  // Issued together before anything waits: the first rounds' page ids, the
  // row length and the query, so the K/V gathers start after one round trip.
  const int my_ids = load_ids(0);
  const int n_tok = a.sctx[row];
  // Q^T operand: head kvh * G + c, dims 32 g .. 32 g + 31 (zero past G).
  bf16x8 qb[4];
  {
    const int hc = c < a.G ? c : 0;
    const uint8_t* qrow = a.q + ((size_t)t * a.H_q + kvh * a.G + hc) * kHeadDim * QB;
#pragma unroll
    for (int j = 0; j < 4; ++j) qb[j] = load_q8_t<Q_DT>(qrow, 32 * g + 8 * j);
  }
  __bf16* out_row = a.out + ((size_t)t * a.H_q + kvh * a.G) * kHeadDim;
  attend_split16<KV_DT, Q_DT, RUN, NT, NW>(a, wp, row, split, kvh, n_tok, qb, my_ids, load_ids, out_row);
}

// One wave a row (the row_wave plan): grid (ceil(rows / 4)), wave w of
// workgroup x attends row 4 grid_row(x) + w alone, its runs in order.
template <int KV_DT, int Q_DT, int RUN, bool NT>
__global__ __launch_bounds__(256) void pa16row_kernel(PaArgs a, int rows) {
  constexpr int QB = Q_DT == ISB_BF16 ? 2 : 1;
  __shared__ bf16x8 s_qb[4][4 * kWave];  // each wave's query operand
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int row = 4 * grid_row(blockIdx.x, gridDim.x) + wave;
  if (row >= rows) return;
  const int c = lane & 15, g = lane >> 4;
  const int t = row / a.H_kv, kvh = row % a.H_kv;
  const int32_t* pages = a.sbt + (size_t)row * a.sbt_stride;
  // lane l holds the id of page r0 RUN + l: runs r0 .. r0 + 64 / RUN - 1
  auto load_ids = [&](int r0) {
    const int pidx = r0 * RUN + lane;
    return pidx < a.sbt_stride ? pages[pidx] : -1;
  };
  const int my_ids = load_ids(0);
  const int n_tok = a.sctx[row];
  bf16x8 qb[4];
  {
    const int hc = c < a.G ? c : 0;
    const uint8_t* qrow = a.q + ((size_t)t * a.H_q + kvh * a.G + hc) * kHeadDim * QB;
#pragma unroll
    for (int j = 0; j < 4; ++j) qb[j] = load_q8_t<Q_DT>(qrow, 32 * g + 8 * j);
  }
  __bf16* out_row = a.out + ((size_t)t * a.H_q + kvh * a.G) * kHeadDim;
  attend_row_wave16<KV_DT, Q_DT, RUN, NT>(a, kvh, n_tok, qb, my_ids, load_ids, out_row, s_qb[wave]);
}

// ----------------------------------------------------------------- select + attend
// Top-k selection and the attention of a row in one launch, for 16-token
// pages and rows of up to kSelMaxBlocks blocks.  Every workgroup of a row
// selects the row's blocks itself (the same result in each: the selection is
// a function of the scores) from the scores and the block-table row, both
// read into registers / LDS in one round trip, and takes its page ids from
// LDS; split 0 also writes the selection, the sparse page table and the
// sparse length, as isb_topk_select_emit would.
struct SelArgs {
  const float* scores;      // [H_kv][T][MB]
  TokenMap tm;              // each token's request and causal length
  const int32_t* bt;        // [R][bt_stride]
  int32_t* topk;            // out [H_kv][T][K]
  int32_t* sbt;             // out [T * H_kv][K * ppb]
  int32_t* sctx;            // out [T * H_kv]
  int T, MB, K, bt_stride;
};

constexpr int kSelMaxBlocks = 2048;      // rows whose block-table row is staged in LDS
constexpr int kSelWideMaxBlocks = 8192;  // widest rows selected in the attention launch

// BTL: the request's block-table row is read whole with the scores and kept
// in LDS (rows of up to kSelMaxBlocks blocks); otherwise (wider rows) only the
// selected blocks' entries are read, after the selection.
template <int KV_DT, int Q_DT, int RUN, bool NT, int NW, int E, bool BTL>
__global__ __launch_bounds__(64 * NW) void pa16sel_kernel(PaArgs a, SelArgs sa) {
  constexpr int QB = Q_DT == ISB_BF16 ? 2 : 1;
  constexpr int NT_ = 64 * NW;      // threads a workgroup
  constexpr int ROUND = NW * RUN;
  __shared__ WaveParts<NW> wp;
  __shared__ SelectLds<NT_> sl;
  __shared__ int32_t s_bt[BTL ? kSelMaxBlocks : 1];
  __shared__ int32_t s_sel[kSelMaxBlocks];
  const int row = grid_row(blockIdx.x, gridDim.x), split = blockIdx.y;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int c = lane & 15, g = lane >> 4;
  const int t = row / a.H_kv, kvh = row % a.H_kv;
  const int trow = kvh * sa.T + t;  // the row's index in the score and selection buffers
  // Every global load first: the token's request and length, the row's
  // scores, the request's block-table row and the query.
  const TokenPos tp = token_pos(sa.tm, t);
  float sc[E];
  int32_t btv[BTL ? E : 1];
  load_run<E, true>(sa.scores + (size_t)trow * sa.MB, E * tid, sa.MB, sc);
  if constexpr (BTL) load_run<E, true>(sa.bt + (size_t)tp.r * sa.bt_stride, E * tid, sa.MB, btv);
  bf16x8 qb[4];
  {
    const int hc = c < a.G ? c : 0;
    const uint8_t* qrow = a.q + ((size_t)t * a.H_q + kvh * a.G + hc) * kHeadDim * QB;
#pragma unroll
    for (int j = 0; j < 4; ++j) qb[j] = load_q8_t<Q_DT>(qrow, 32 * g + 8 * j);
  }
  const int Lt = tp.L;
  const int nt = min((Lt + kBlockTokens - 1) / kBlockTokens, sa.MB);
  if constexpr (BTL) {
#pragma unroll
    for (int x = 0; x < E; ++x)
      if (E * tid + x < sa.MB) s_bt[E * tid + x] = btv[x];
  }
  int32_t* o = sa.topk + (size_t)trow * sa.K;
  const int m = select_row<NT_, E>(sc, nt, sa.K, sl, [&](int k, int b) {
    s_sel[k] = b;
    if (split == 0) o[k] = b;
  });
  __syncthreads();  // the selection (and the block-table row) are in LDS
  if constexpr (!BTL) {  // the selected blocks' ids, in place of their indices
    for (int k = tid; k < m; k += NT_) s_sel[k] = sa.bt[(size_t)tp.r * sa.bt_stride + s_sel[k]];
    __syncthreads();
  }
  // block id of the k-th selected block
  auto blk = [&](int k) { return BTL ? s_bt[s_sel[k]] : s_sel[k]; };
  const int n_tok = m > 0 ? (m - 1) * kBlockTokens + (Lt - kBlockTokens * (nt - 1)) : 0;
  if (split == 0) {
    const int slots = sa.K * 8;
    int32_t* so = sa.sbt + (size_t)row * slots;
    for (int x = tid; x < slots; x += NT_) so[x] = (x >> 3) < m ? blk(x >> 3) * 8 + (x & 7) : -1;
    if (tid == 0) sa.sctx[row] = n_tok;
  }
  const int p0 = split * a.pps;
  const int pend = min(a.sbt_stride, p0 + a.pps);
  const int mpages = 8 * m;
  auto ids = [&](int r0) {
    const int pidx = p0 + (r0 + lane / RUN) * ROUND + wave * RUN + lane % RUN;
    return pidx < pend && pidx < mpages ? blk(pidx >> 3) * 8 + (pidx & 7) : -1;
  };
  const int my_ids = ids(0);
  __bf16* out_row = a.out + ((size_t)t * a.H_q + kvh * a.G) * kHeadDim;
  attend_split16<KV_DT, Q_DT, RUN, NT, NW>(a, wp, row, split, kvh, n_tok, qb, my_ids, ids, out_row);
}

// ----------------------------------------------------------------- MXFP4 pages
// The query operand of an MXFP4 row: e4m3 bytes as the scaled MFMA's B
// operand (dims 16 g .. and 64 + 16 g ..), or bf16 operands; zero past the
// group's G heads.
template <int Q_DT>
struct MxQuery {
  i32x8 q8;
  bf16x8 qb[4];
};

template <int Q_DT>
__device__ __forceinline__ MxQuery<Q_DT> load_mx_query(const PaArgs& a, int t, int kvh, int lane) {
  const int c = lane & 15, g = lane >> 4;
  const int hc = c < a.G ? c : 0;
  const uint8_t* qrow = a.q + ((size_t)t * a.H_q + kvh * a.G + hc) * kHeadDim * (Q_DT == ISB_BF16 ? 2 : 1);
  MxQuery<Q_DT> mq;
  if constexpr (Q_DT == ISB_FP8_E4M3) {
    const u32x4 lo = ld16(qrow + 16 * g), hi = ld16(qrow + 64 + 16 * g);
    mq.q8 = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    if (c >= a.G) mq.q8 = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) mq.qb[j] = load_q8_t<Q_DT>(qrow, 32 * g + 8 * j);
    zero_missing_heads(mq.qb, c, a.G);
  }
  return mq;
}

// Page p of a row (one 128-token MXFP4 page: eight 16-key tiles) whose id is
// id (wave-uniform), folded into the wave's running max M (per head), sum
// share lsum and output o.  KEEP: pin MFMA operands live (see
// mfma_16x16x32_bf16_k).
template <int Q_DT, bool KEEP>
__device__ __forceinline__ void attend_page_mx(const PaArgs& a, int lane, int kvh, int n_tok, int p, int64_t id,
                                               const MxQuery<Q_DT>& mq, bool first, float& M, float& lsum,
                                               f32x4 (&o)[8]) {
  const int c = lane & 15, g = lane >> 4;
  const bool ok = page_ok(id, a.num_pages);
  const int64_t pg = ((ok ? id : 0) * a.H_kv + kvh) * kMxPageBytes;
  const __amdgpu_buffer_rsrc_t rk = page_rsrc(a.kp + pg, kMxPageBytes);
  const __amdgpu_buffer_rsrc_t rv = page_rsrc(a.vp + pg, kMxPageBytes);
  u32x4 kd[8];
  uint32_t ks[8];
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
    kd[tt] = bl16(rk, 64 * c + 16 * g, 1024 * tt);
    ks[tt] = bl4(rk, 4 * c, kMxDataBytes + 64 * tt);
  }
  // V: keys 16 tt + 4 g + e of tile tt, the word of dims 8 c .. 8 c + 7,
  // and the four keys' scale words (one 16-byte load a tile)
  uint32_t vw[8][4];
  u32x4 vs[8];
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) vw[tt][e] = bl4(rv, 64 * (4 * g + e) + 4 * c, 1024 * tt);
    vs[tt] = bl16(rv, 16 * g, kMxDataBytes + 64 * tt);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int nvp = min(kBlockTokens, n_tok - p * kBlockTokens);  // keys of the page that count
  // Pass 1: the page's logits and one exact max per head.
  float z[8][4];
  float mx = neg_inf();
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    const uint32_t sbyte = (ks[tt] >> (8 * g)) & 0xFFu;
    if constexpr (Q_DT == ISB_FP8_E4M3) {
      const i32x8 ka = {(int)kd[tt][0], (int)kd[tt][1], (int)kd[tt][2], (int)kd[tt][3], 0, 0, 0, 0};
      s = mfma_scale_fp4_e4m3(ka, mq.q8, s, (int)sbyte);
    } else {
      const float sc = e8m0_to_f32(sbyte);
#pragma unroll
      for (int j = 0; j < 4; ++j) s = mfma_16x16x32_bf16_k<KEEP>(e2m1x8_to_bf16x8(kd[tt][j], sc), mq.qb[j], s);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = ok ? s[e] * a.qk_scale : qnan();
      z[tt][e] = 16 * tt + 4 * g + e < nvp ? v : neg_inf();
      mx = fmaxf(mx, z[tt][e]);
    }
  }
  mx = max_over_groups(mx);
  const float m_new = fmaxf(M, mx);
  if (!first) {
    const float alpha = M == m_new ? 1.f : __builtin_amdgcn_exp2f(M - m_new);
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
  }
  M = m_new;
  // Pass 2: probabilities and P.V.  Lane (g, c) takes keys 4 g + e of the
  // tile and dims 8 c .. 8 c + 7 (one data word, one scale byte per key);
  // MFMA dt gets dim 8 c + dt.
#pragma unroll
  for (int tt = 0; tt < 8; ++tt) {
    float pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pr[e] = __builtin_amdgcn_exp2f(z[tt][e] - M);
      lsum += pr[e];
    }
    const bf16x4 pb = {(__bf16)pr[0], (__bf16)pr[1], (__bf16)pr[2], (__bf16)pr[3]};
    bf16x8 vv[4];  // key e: dims 8 c .. 8 c + 7
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tok = 16 * tt + 4 * g + e;
      const bool on = tok < nvp;  // keys past the length may be poison: zero, unit scale
      const uint32_t w = on ? vw[tt][e] : 0u;
      const uint32_t sw = vs[tt][e];
      const float sc = on ? e8m0_to_f32((sw >> (8 * (c >> 2))) & 0xFFu) : 1.f;
      vv[e] = e2m1x8_to_bf16x8(w, sc);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const bf16x4 vt = {vv[0][dt], vv[1][dt], vv[2][dt], vv[3][dt]};
      o[dt] = mfma_16x16x16_bf16_k<KEEP>(vt, pb, o[dt]);
    }
  }
}

// The attention of one split of an MXFP4 row: page p0 + NW r + wave in round
// r.  ids(r0): this lane's page id for round r0 + lane of this wave (-1 past
// the split), fetched 64 rounds at a time and read out a round at a time.
template <int Q_DT, int NW, typename IdFn>
__device__ __forceinline__ void attend_split_mx(const PaArgs& a, WaveParts<NW>& wp, int row, int split, int t,
                                                int kvh, int n_tok, IdFn ids, __bf16* out_row) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int p0 = split * a.pps;
  if (n_tok <= 0) {
    write_empty_row(a, split, out_row);
    return;
  }
  const int npages = min((n_tok + kBlockTokens - 1) / kBlockTokens, a.sbt_stride);
  if (p0 >= npages) return;
  const int p1 = min(npages, p0 + a.pps);
  const int live = (npages + a.pps - 1) / a.pps;
  float M = neg_inf(), lsum = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (p0 + wave < p1) {  // wave-uniform: this wave has pages in the split
    int32_t my_ids = ids(0);
    const MxQuery<Q_DT> mq = load_mx_query<Q_DT>(a, t, kvh, lane);
    for (int r = 0, p = p0 + wave; p < p1; ++r, p += NW) {
      if (r > 0 && r % kWave == 0) my_ids = ids(r);
      const int64_t id = __builtin_amdgcn_readlane(my_ids, r % kWave);
      attend_page_mx<Q_DT, NW == 8>(a, lane, kvh, n_tok, p, id, mq, r == 0, M, lsum, o);
    }
  }
  wave_to_lds<8, 1, NW>(wp, wave, lane, M, lsum, o);  // row r of tile dt: dim 8 r + dt
  finish_split<NW>(a, wp, row, split, live, out_row);
}

// grid (rows, splits), NW waves a workgroup; page ids come from the sparse
// page table.
template <int Q_DT, int NW>
__global__ __launch_bounds__(64 * NW) void pamx_kernel(PaArgs a) {
  __shared__ WaveParts<NW> wp;
  const int row = grid_row(blockIdx.x, gridDim.x), split = blockIdx.y;
  const int t = row / a.H_kv, kvh = row % a.H_kv;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int n_tok = a.sctx[row];
  const int pend = min(a.sbt_stride, (split + 1) * a.pps);
  const int32_t* pages = a.sbt + (size_t)row * a.sbt_stride;
  auto ids = [&](int r0) {  // this wave's page of round r0 + lane
    const int p = split * a.pps + NW * (r0 + lane) + wave;
    return p < pend ? pages[p] : -1;
  };
  __bf16* out_row = a.out + ((size_t)t * a.H_q + kvh * a.G) * kHeadDim;
  attend_split_mx<Q_DT, NW>(a, wp, row, split, t, kvh, n_tok, ids, out_row);
}

// Selection and attention of a row in one launch for MXFP4 pages (one page a
// block), as pa16sel_kernel does for 16-token pages: every workgroup of a row
// selects the row's blocks from its scores and block-table row, split 0 also
// writes the selection, the page table and the sparse length.
template <int Q_DT, int NW, int E, bool BTL>
__global__ __launch_bounds__(64 * NW) void pamxsel_kernel(PaArgs a, SelArgs sa) {
  constexpr int NT_ = 64 * NW;
  __shared__ WaveParts<NW> wp;
  __shared__ SelectLds<NT_> sl;
  __shared__ int32_t s_bt[BTL ? kSelMaxBlocks : 1];
  __shared__ int32_t s_sel[kSelMaxBlocks];
  const int row = grid_row(blockIdx.x, gridDim.x), split = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int t = row / a.H_kv, kvh = row % a.H_kv;
  const int trow = kvh * sa.T + t;  // the row's index in the score and selection buffers
  const TokenPos tp = token_pos(sa.tm, t);
  float sc[E];
  int32_t btv[BTL ? E : 1];
  load_run<E, true>(sa.scores + (size_t)trow * sa.MB, E * tid, sa.MB, sc);
  if constexpr (BTL) load_run<E, true>(sa.bt + (size_t)tp.r * sa.bt_stride, E * tid, sa.MB, btv);
  const int Lt = tp.L;
  const int nt = min((Lt + kBlockTokens - 1) / kBlockTokens, sa.MB);
  if constexpr (BTL) {
#pragma unroll
    for (int x = 0; x < E; ++x)
      if (E * tid + x < sa.MB) s_bt[E * tid + x] = btv[x];
  }
  int32_t* o = sa.topk + (size_t)trow * sa.K;
  const int m = select_row<NT_, E>(sc, nt, sa.K, sl, [&](int k, int b) {
    s_sel[k] = b;
    if (split == 0) o[k] = b;
  });
  __syncthreads();  // the selection (and the block-table row) are in LDS
  if constexpr (!BTL) {  // the selected blocks' ids, in place of their indices
    for (int k = tid; k < m; k += NT_) s_sel[k] = sa.bt[(size_t)tp.r * sa.bt_stride + s_sel[k]];
    __syncthreads();
  }
  auto blk = [&](int k) { return BTL ? s_bt[s_sel[k]] : s_sel[k]; };
  const int n_tok = m > 0 ? (m - 1) * kBlockTokens + (Lt - kBlockTokens * (nt - 1)) : 0;
  if (split == 0) {  // one page a block: the row's k-th page is its k-th selected block
    int32_t* so = sa.sbt + (size_t)row * sa.K;
    for (int x = tid; x < sa.K; x += NT_) so[x] = x < m ? blk(x) : -1;
    if (tid == 0) sa.sctx[row] = n_tok;
  }
  const int wave = wave_id();
  const int pend = min(m, (split + 1) * a.pps);
  auto ids = [&](int r0) {  // this wave's page of round r0 + lane
    const int p = split * a.pps + NW * (r0 + lane) + wave;
    return p < pend ? blk(p) : -1;
  };
  __bf16* out_row = a.out + ((size_t)t * a.H_q + kvh * a.G) * kHeadDim;
  attend_split_mx<Q_DT, NW>(a, wp, row, split, t, kvh, n_tok, ids, out_row);
}

// nt: one query token a request, so no page is read twice in the launch;
// the plan gives the waves a workgroup.
template <int KV_DT, int Q_DT>
static void launch_decode(const PaArgs& a, dim3 grid, bool nt, const PaPlan& plan, hipStream_t st) {
  const int nw = plan.waves;
  if constexpr (KV_DT == ISB_MXFP4) {  // the plan gives MXFP4 rows four waves a workgroup
    hipLaunchKernelGGL((pamx_kernel<Q_DT, 4>), grid, dim3(256), 0, st, a);
  } else {
    constexpr int RUN = KV_DT == ISB_BF16 ? 4 : 8;
    if (plan.row_wave) {
      const dim3 g((unsigned)((plan.rows + 3) / 4));
      if (nt) hipLaunchKernelGGL((pa16row_kernel<KV_DT, Q_DT, RUN, true>), g, dim3(256), 0, st, a, plan.rows);
      else hipLaunchKernelGGL((pa16row_kernel<KV_DT, Q_DT, RUN, false>), g, dim3(256), 0, st, a, plan.rows);
      return;
    }
    if constexpr (KV_DT == ISB_FP8_E4M3) {  // the plan takes eight waves for fp8 pages only
      if (nw == 8) {
        if (nt) hipLaunchKernelGGL((pa16_kernel<KV_DT, Q_DT, RUN, true, 8>), grid, dim3(512), 0, st, a);
        else hipLaunchKernelGGL((pa16_kernel<KV_DT, Q_DT, RUN, false, 8>), grid, dim3(512), 0, st, a);
        return;
      }
    }
    if (nt) hipLaunchKernelGGL((pa16_kernel<KV_DT, Q_DT, RUN, true, 4>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((pa16_kernel<KV_DT, Q_DT, RUN, false, 4>), grid, dim3(256), 0, st, a);
  }
}

}  // namespace isb

extern "C" size_t isb_sparse_pa_workspace_bytes(int num_tokens, int num_q_heads, int num_kv_heads,
                                                int sparse_bt_stride, int kv_dtype) {
  using namespace isb;
  if (num_tokens <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || sparse_bt_stride <= 0 ||
      !is_pool_dtype(kv_dtype))
    return 0;
  return pa_workspace_bytes(pa_plan(num_tokens, num_kv_heads, sparse_bt_stride, kv_dtype));
}

namespace isb {

// Argument checks and kernel arguments shared by isb_sparse_pa_decode and
// isb_select_attend; 0 or an ISB_E_* code.
static int pa_setup(const void* q, int q_dtype, const void* k_pool, const void* v_pool, int kv_dtype,
                    int64_t num_pages, float k_scale, float v_scale, int sparse_bt_stride,
                    int num_tokens, int num_q_heads, int num_kv_heads, int head_dim, float sm_scale,
                    void* workspace, size_t workspace_bytes, void* out, PaArgs& a, PaPlan& plan) {
  if (!q || !k_pool || !v_pool || !out) return ISB_E_INVALID_ARG;
  if (num_pages <= 0 || sparse_bt_stride <= 0 || num_tokens <= 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0)
    return ISB_E_INVALID_ARG;
  if (!is_query_dtype(q_dtype) || !is_pool_dtype(kv_dtype)) return ISB_E_UNSUPPORTED_DTYPE;
  if (head_dim != kHeadDim || num_q_heads % num_kv_heads != 0 || num_q_heads / num_kv_heads > 16)
    return ISB_E_SHAPE;
  if (!(sm_scale > 0.f) || !(k_scale > 0.f) || !(v_scale > 0.f)) return ISB_E_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return ISB_E_INVALID_ARG;
  const long long rows = (long long)num_tokens * num_kv_heads;
  if (rows > 0x7FFFFFFFLL) return ISB_E_SHAPE;
  plan = pa_plan(num_tokens, num_kv_heads, sparse_bt_stride, kv_dtype);
  if (plan.splits > 65535) return ISB_E_SHAPE;
  const size_t need = pa_workspace_bytes(plan);  // 0: every row one split, nothing published
  if (need > 0 && !workspace) return ISB_E_INVALID_ARG;
  if (workspace_bytes < need) return ISB_E_WORKSPACE;
  const bool fp8 = kv_dtype == ISB_FP8_E4M3;
  a.q = (const uint8_t*)q;
  a.kp = (const uint8_t*)k_pool;
  a.vp = (const uint8_t*)v_pool;
  a.sbt = nullptr;
  a.sctx = nullptr;
  a.part_o = (float*)workspace;
  a.part_ml = a.part_o + (size_t)plan.rows * plan.splits * kPartialO;
  a.out = (__bf16*)out;
  a.num_pages = num_pages;
  a.qk_scale = sm_scale * (fp8 ? k_scale : 1.0f) * 1.4426950408889634f;
  a.v_scale = fp8 ? v_scale : 1.0f;
  a.sbt_stride = sparse_bt_stride;
  a.H_q = num_q_heads;
  a.H_kv = num_kv_heads;
  a.G = num_q_heads / num_kv_heads;
  a.splits = plan.splits;
  a.pps = plan.pages_per_split;
  return ISB_OK;
}

// E: scores a thread holds, E x (64 NW) >= max_blocks; BTL: the block-table
// row goes to LDS with the scores (max_blocks <= kSelMaxBlocks).
template <int KV_DT, int Q_DT, int NW, int E, bool BTL>
static void launch_select_attend_e(const PaArgs& a, const SelArgs& sa, dim3 grid, bool nt, hipStream_t st) {
  if constexpr (KV_DT == ISB_MXFP4) {
    hipLaunchKernelGGL((pamxsel_kernel<Q_DT, NW, E, BTL>), grid, dim3(64 * NW), 0, st, a, sa);
  } else {
    constexpr int RUN = KV_DT == ISB_BF16 ? 4 : 8;
    const dim3 b(64 * NW);
    if (nt) hipLaunchKernelGGL((pa16sel_kernel<KV_DT, Q_DT, RUN, true, NW, E, BTL>), grid, b, 0, st, a, sa);
    else hipLaunchKernelGGL((pa16sel_kernel<KV_DT, Q_DT, RUN, false, NW, E, BTL>), grid, b, 0, st, a, sa);
  }
}

template <int KV_DT, int Q_DT, int NW>
static void launch_select_attend_nw(const PaArgs& a, const SelArgs& sa, dim3 grid, bool nt, hipStream_t st) {
  constexpr int NT = 64 * NW;
  if (sa.MB <= NT) launch_select_attend_e<KV_DT, Q_DT, NW, 1, true>(a, sa, grid, nt, st);
  else if (sa.MB <= 2 * NT) launch_select_attend_e<KV_DT, Q_DT, NW, 2, true>(a, sa, grid, nt, st);
  else if (sa.MB <= 4 * NT) launch_select_attend_e<KV_DT, Q_DT, NW, 4, true>(a, sa, grid, nt, st);
  else if (sa.MB <= kSelMaxBlocks) launch_select_attend_e<KV_DT, Q_DT, NW, 8 * 4 / NW, true>(a, sa, grid, nt, st);
  else if (sa.MB <= 4096) launch_select_attend_e<KV_DT, Q_DT, NW, 16 * 4 / NW, false>(a, sa, grid, nt, st);
  else launch_select_attend_e<KV_DT, Q_DT, NW, 32 * 4 / NW, false>(a, sa, grid, nt, st);
}

template <int KV_DT, int Q_DT>
static void launch_select_attend(const PaArgs& a, const SelArgs& sa, dim3 grid, bool nt, const PaPlan& plan,
                                 hipStream_t st) {
  if constexpr (KV_DT == ISB_FP8_E4M3) {  // the plan takes eight waves for fp8 pages only
    if (plan.waves == 8) {
      launch_select_attend_nw<KV_DT, Q_DT, 8>(a, sa, grid, nt, st);
      return;
    }
  }
  launch_select_attend_nw<KV_DT, Q_DT, 4>(a, sa, grid, nt, st);
}

}  // namespace isb

namespace isb {

// The attention launch for a plan set up by pa_setup; nt: nontemporal page
// loads (one query token a request, so no page is read twice).
static int pa_run(hipStream_t st, const PaArgs& a, const PaPlan& plan, int q_dtype, int kv_dtype, bool nt) {
  const dim3 grid((unsigned)plan.rows, plan.splits);
  const bool qb = q_dtype == ISB_BF16;
  if (kv_dtype == ISB_BF16) {
    if (qb) launch_decode<ISB_BF16, ISB_BF16>(a, grid, nt, plan, st);
    else launch_decode<ISB_BF16, ISB_FP8_E4M3>(a, grid, nt, plan, st);
  } else if (kv_dtype == ISB_FP8_E4M3) {
    if (qb) launch_decode<ISB_FP8_E4M3, ISB_BF16>(a, grid, nt, plan, st);
    else launch_decode<ISB_FP8_E4M3, ISB_FP8_E4M3>(a, grid, nt, plan, st);
  } else {
    if (qb) launch_decode<ISB_MXFP4, ISB_BF16>(a, grid, nt, plan, st);
    else launch_decode<ISB_MXFP4, ISB_FP8_E4M3>(a, grid, nt, plan, st);
  }
  return launch_status();
}

}  // namespace isb

extern "C" int isb_sparse_pa_decode(isb_stream_t stream, const void* q, int q_dtype,
                                    const void* k_pool, const void* v_pool, int kv_dtype,
                                    int64_t num_pages, float k_scale, float v_scale,
                                    const int32_t* sparse_bt, int sparse_bt_stride,
                                    const int32_t* sparse_ctx, int num_tokens, int decode_query_len,
                                    int num_q_heads, int num_kv_heads, int head_dim, float sm_scale,
                                    void* workspace, size_t workspace_bytes, void* out) {
  using namespace isb;
  if (!sparse_bt || !sparse_ctx) return ISB_E_INVALID_ARG;
  if (decode_query_len <= 0) return ISB_E_INVALID_ARG;
  if (num_tokens > 0 && num_tokens % decode_query_len != 0) return ISB_E_SHAPE;
  PaArgs a;
  PaPlan plan;
  const int err = pa_setup(q, q_dtype, k_pool, v_pool, kv_dtype, num_pages, k_scale, v_scale,
                           sparse_bt_stride, num_tokens, num_q_heads, num_kv_heads, head_dim, sm_scale,
                           workspace, workspace_bytes, out, a, plan);
  if (err) return err;
  a.sbt = sparse_bt;
  a.sctx = sparse_ctx;
  return pa_run(as_hip(stream), a, plan, q_dtype, kv_dtype, decode_query_len == 1);
}

extern "C" int isb_sparse_pa_prefill(isb_stream_t stream, const void* q, int q_dtype,
                                     const void* k_pool, const void* v_pool, int kv_dtype,
                                     int64_t num_pages, float k_scale, float v_scale,
                                     const int32_t* sparse_bt, int sparse_bt_stride,
                                     const int32_t* sparse_ctx, int num_tokens, int num_q_heads,
                                     int num_kv_heads, int head_dim, float sm_scale, void* workspace,
                                     size_t workspace_bytes, void* out) {
  using namespace isb;
  if (!sparse_bt || !sparse_ctx) return ISB_E_INVALID_ARG;
  PaArgs a;
  PaPlan plan;
  const int err = pa_setup(q, q_dtype, k_pool, v_pool, kv_dtype, num_pages, k_scale, v_scale,
                           sparse_bt_stride, num_tokens, num_q_heads, num_kv_heads, head_dim, sm_scale,
                           workspace, workspace_bytes, out, a, plan);
  if (err) return err;
  a.sbt = sparse_bt;
  a.sctx = sparse_ctx;
  return pa_run(as_hip(stream), a, plan, q_dtype, kv_dtype, false);
}

// ----------------------------------------------------------------- no allocation
// isb_sparse_pa_decode_noalloc: the same call with the split partials in this
// library's own device memory, for callers that cannot allocate (code under
// HIP graph capture, serving loops, hosts that forbid allocation).  The array
// is zero-initialised when the library's code is loaded on a device, which is
// the free state of every slot, and every completed call leaves it so; each
// device holds its own copy until the process ends.  Calls that overlap in
// time on one device share it and race.
constexpr size_t kNoallocScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // per device: the device address of `scratch`

// The device address of the current device's scratch, looked up once per
// device (with that device current); nullptr if the lookup fails.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" int isb_sparse_pa_decode_noalloc(isb_stream_t stream, const void* q, int q_dtype,
                                            const void* k_pool, const void* v_pool, int kv_dtype,
                                            int64_t num_pages, float k_scale, float v_scale,
                                            const int32_t* sparse_bt, int sparse_bt_stride,
                                            const int32_t* sparse_ctx, int num_tokens, int decode_query_len,
                                            int num_q_heads, int num_kv_heads, int head_dim, float sm_scale,
                                            void* out) {
  using namespace isb;
  // every argument check of isb_sparse_pa_decode first, the scratch standing
  // in as a workspace of its size (nothing is read or written here): errors
  // come back before any device call, and partials beyond the scratch are
  // ISB_E_WORKSPACE
  if (!sparse_bt || !sparse_ctx || decode_query_len <= 0) return ISB_E_INVALID_ARG;
  if (num_tokens > 0 && num_tokens % decode_query_len != 0) return ISB_E_SHAPE;
  {
    PaArgs a;
    PaPlan plan;
    const int err = pa_setup(q, q_dtype, k_pool, v_pool, kv_dtype, num_pages, k_scale, v_scale, sparse_bt_stride,
                             num_tokens, num_q_heads, num_kv_heads, head_dim, sm_scale,
                             reinterpret_cast<void*>(uintptr_t(256)), kNoallocScratchBytes, out, a, plan);
    if (err) return err;
  }
  void* ws = device_scratch();
  if (!ws) return ISB_E_LAUNCH;
  return isb_sparse_pa_decode(stream, q, q_dtype, k_pool, v_pool, kv_dtype, num_pages, k_scale, v_scale, sparse_bt,
                              sparse_bt_stride, sparse_ctx, num_tokens, decode_query_len, num_q_heads, num_kv_heads,
                              head_dim, sm_scale, ws, kNoallocScratchBytes, out);
}

namespace isb {

// isb_select_attend for either batch form; nt as for pa_run.
static int select_attend_run(hipStream_t st, const float* scores, const TokenMap& tm, long long T,
                             int num_kv_heads, int max_blocks, int top_k, const int32_t* block_table,
                             int block_table_stride, const void* q, int q_dtype, const void* k_pool,
                             const void* v_pool, int kv_dtype, int64_t num_pages, float k_scale, float v_scale,
                             int num_q_heads, float sm_scale, void* workspace, size_t workspace_bytes,
                             int32_t* topk_idx, int32_t* sparse_bt, int32_t* sparse_ctx, void* out, bool nt) {
  if (!scores || !block_table || !topk_idx || !sparse_bt || !sparse_ctx) return ISB_E_INVALID_ARG;
  if (T <= 0 || num_kv_heads <= 0 || max_blocks <= 0 || block_table_stride <= 0) return ISB_E_INVALID_ARG;
  if (top_k < 1 || top_k > max_blocks || max_blocks > (1 << 20) || max_blocks > block_table_stride)
    return ISB_E_SHAPE;
  const int ppb = kv_dtype == ISB_MXFP4 ? 1 : 8;
  if (T * num_kv_heads * top_k * ppb > 0x7FFFFFFFLL) return ISB_E_SHAPE;
  PaArgs a;
  PaPlan plan;
  const int err = pa_setup(q, q_dtype, k_pool, v_pool, kv_dtype, num_pages, k_scale, v_scale, top_k * ppb,
                           (int)T, num_q_heads, num_kv_heads, kHeadDim, sm_scale, workspace, workspace_bytes,
                           out, a, plan);
  if (err) return err;
  // rows wider than kSelMaxBlocks keep only their selection in LDS, which
  // holds up to kSelMaxBlocks blocks
  const bool one_launch = max_blocks <= kSelWideMaxBlocks && top_k <= kSelMaxBlocks && max_blocks % 4 == 0 &&
                          block_table_stride % 4 == 0 && reinterpret_cast<uintptr_t>(scores) % 16 == 0 &&
                          reinterpret_cast<uintptr_t>(block_table) % 16 == 0;
  if (!one_launch || plan.row_wave) {
    // wide or unaligned rows, or one wave a row (whose workgroups attend four
    // rows and could not select them together): the two steps as two launches.
    const int e = topk_select_emit_run(st, scores, tm, (int)T, num_kv_heads, max_blocks, top_k, block_table,
                                       block_table_stride, ppb, topk_idx, sparse_bt, sparse_ctx);
    if (e) return e;
    a.sbt = sparse_bt;
    a.sctx = sparse_ctx;
    return pa_run(st, a, plan, q_dtype, kv_dtype, nt);
  }
  SelArgs sa{scores, tm, block_table, topk_idx, sparse_bt, sparse_ctx, (int)T, max_blocks, top_k,
             block_table_stride};
  const dim3 grid((unsigned)plan.rows, plan.splits);
  const bool qb = q_dtype == ISB_BF16;
  if (kv_dtype == ISB_BF16) {
    if (qb) launch_select_attend<ISB_BF16, ISB_BF16>(a, sa, grid, nt, plan, st);
    else launch_select_attend<ISB_BF16, ISB_FP8_E4M3>(a, sa, grid, nt, plan, st);
  } else if (kv_dtype == ISB_FP8_E4M3) {
    if (qb) launch_select_attend<ISB_FP8_E4M3, ISB_BF16>(a, sa, grid, nt, plan, st);
    else launch_select_attend<ISB_FP8_E4M3, ISB_FP8_E4M3>(a, sa, grid, nt, plan, st);
  } else {
    if (qb) launch_select_attend<ISB_MXFP4, ISB_BF16>(a, sa, grid, nt, plan, st);
    else launch_select_attend<ISB_MXFP4, ISB_FP8_E4M3>(a, sa, grid, nt, plan, st);
  }
  return launch_status();
}

}  // namespace isb

extern "C" int isb_select_attend(isb_stream_t stream, const float* scores, const int32_t* seq_lens,
                                 int num_reqs, int decode_query_len, int num_kv_heads, int max_blocks,
                                 int top_k, const int32_t* block_table, int block_table_stride,
                                 const void* q, int q_dtype, const void* k_pool, const void* v_pool,
                                 int kv_dtype, int64_t num_pages, float k_scale, float v_scale,
                                 int num_q_heads, float sm_scale, void* workspace,
                                 size_t workspace_bytes, int32_t* topk_idx, int32_t* sparse_bt,
                                 int32_t* sparse_ctx, void* out) {
  using namespace isb;
  if (!seq_lens || num_reqs <= 0 || decode_query_len <= 0) return ISB_E_INVALID_ARG;
  return select_attend_run(as_hip(stream), scores, decode_map(seq_lens, decode_query_len),
                           (long long)num_reqs * decode_query_len, num_kv_heads, max_blocks, top_k, block_table,
                           block_table_stride, q, q_dtype, k_pool, v_pool, kv_dtype, num_pages, k_scale, v_scale,
                           num_q_heads, sm_scale, workspace, workspace_bytes, topk_idx, sparse_bt, sparse_ctx, out,
                           decode_query_len == 1);
}

extern "C" int isb_select_attend_prefill(isb_stream_t stream, const float* scores, int num_reqs,
                                         const int32_t* query_req_id, const int32_t* query_abs_pos,
                                         int num_tokens, int num_kv_heads, int max_blocks, int top_k,
                                         const int32_t* block_table, int block_table_stride, const void* q,
                                         int q_dtype, const void* k_pool, const void* v_pool, int kv_dtype,
                                         int64_t num_pages, float k_scale, float v_scale, int num_q_heads,
                                         float sm_scale, void* workspace, size_t workspace_bytes,
                                         int32_t* topk_idx, int32_t* sparse_bt, int32_t* sparse_ctx, void* out) {
  using namespace isb;
  if (!query_req_id || !query_abs_pos || num_reqs <= 0) return ISB_E_INVALID_ARG;
  return select_attend_run(as_hip(stream), scores,
                           prefill_map(query_req_id, query_abs_pos, num_reqs, max_blocks), num_tokens,
                           num_kv_heads, max_blocks, top_k, block_table, block_table_stride, q, q_dtype, k_pool,
                           v_pool, kv_dtype, num_pages, k_scale, v_scale, num_q_heads, sm_scale, workspace,
                           workspace_bytes, topk_idx, sparse_bt, sparse_ctx, out, false);
}
