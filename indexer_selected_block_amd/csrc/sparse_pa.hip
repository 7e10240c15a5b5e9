// isb_sparse_pa_decode: split-K flash decode over the selected pages, then a
// reduce launch that merges the splits of rows that needed more than one.
//
// The decode call of the vLLM API page for sparse_attention_msa
// (minimax_m3_sparse_attn_decode_aiter with the emitted sparse_block_table and
// sparse_context_lens): per row (token, KV head) and query head of that KV
// group, softmax(scale q.K) V over the sparse positions.  MXFP4 K/V follow
// ROCm/ATOM PR 2962 (Summary: MXFP4 K and V pages, one row per token and KV
// head).
//
// Work decomposition.  A row's pages are cut into `splits` runs of
// `pages_per_split`; one workgroup of four waves attends one run.  A wave
// takes one 16-token tile at a time:
//   S^T (16 keys x 16 heads) = K_tile . Q^T      4 x v_mfma_f32_16x16x32_bf16
//   online softmax in fp32 (row max over lane groups by lane shuffles)
//   O^T (128 dims x 16 heads) += V^T_tile . P^T   8 x v_mfma_f32_16x16x16_bf16
// The G <= 16 query heads of a KV group fill the MFMA's 16 columns, so K and V
// bytes are read once per row and reused by every head.  K and V are
// dequantised to bf16 in registers (exact for e4m3 and for e2m1 x 2^k); the
// per-tensor fp8 scales and the softmax scale are folded into one logit
// multiplier (k_scale sm_scale log2 e) and the output (v_scale).
//
// Layout of the operands (lane = 16 g + c):
//   K tile, A of QK:  key c of the tile, dims 32 g .. 32 g + 31 (MFMA j takes
//                     dims 32 g + 8 j .. + 7);  Q^T, B of QK: head c, same dims;
//   S^T result:       lane holds keys 4 g + e (e < 4) of head c;
//   P^T, B of PV:     exactly that: head c, keys 4 g + e;
//   V^T, A of PV:     dim 16 dt + c, keys 4 g + e - one dword of an fp8 V page
//                     ([128 dim][16 tok]) per dim tile dt;
//   O^T result:       lane holds dims 16 dt + 4 g + e of head c.
// Every value a lane holds belongs to its head c, so the softmax rescale of
// the output is lane-local.
//
// 16-token (bf16 / fp8) pages go straight from HBM to registers with 16-byte
// (K) and 4-byte (V) loads, the next page's loads issued before the current
// page's math.  128-token MXFP4 pages are token-major, which puts a V tile's
// keys for one dim in four different rows; the workgroup stages each V page in
// LDS and lanes read their nibbles from there.
#include "isb_device.h"
#include "isb_host.h"

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
  int q_dt, sbt_stride, H_q, H_kv, G, splits, pps, ppw;
};

constexpr int kPaWaves = 4;

__device__ __forceinline__ bf16x8 load_q8_pa(const uint8_t* row, int q_dt, int dim0) {
  if (q_dt == ISB_BF16) return u32x4_as_bf16x8(ld16(row + 2 * dim0));
  u32x2 w = ld8(row + dim0);
  bf16x4 a = e4m3x4_to_bf16x4(w[0]);
  bf16x4 b = e4m3x4_to_bf16x4(w[1]);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Running state of one wave: per lane, head c = lane & 15.
struct Softmax {
  float m;      // running max of scaled logits (log2 domain), same in the 4 lane groups
  float l;      // this lane's share of the running sum
  f32x4 o[8];   // O^T: dims 16 dt + 4 g + e of head c
};

// One 16-key tile: kb = K tile as the A operand (4 x bf16x8), vt = V^T tile
// (8 x bf16x4), nvalid = keys of the tile that count (1..16), bad = NaN poison.
__device__ __forceinline__ void attend_tile(Softmax& st, const bf16x8 (&qb)[4], const bf16x8 (&kb)[4],
                                            const bf16x4 (&vt)[8], int nvalid, bool bad,
                                            float qk_scale, int g) {
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) s = mfma_16x16x32_bf16(kb[j], qb[j], s);
  float z[4];
  float tmax = neg_inf();
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float v = bad ? qnan() : s[e] * qk_scale;
    v = (4 * g + e < nvalid) ? v : neg_inf();
    z[e] = v;
    tmax = fmaxf(tmax, v);
  }
  tmax = max_over_groups(tmax);
  const float m_new = fmaxf(st.m, tmax);
  const float alpha = exp2f(st.m - m_new);  // 0 on the first tile (m = -inf)
  float p[4];
  float psum = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    p[e] = exp2f(z[e] - m_new);
    psum += p[e];
  }
  st.l = st.l * alpha + psum;
  st.m = m_new;
  const bf16x4 pb = {(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3]};
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    st.o[dt] *= alpha;
    st.o[dt] = mfma_16x16x16_bf16(vt[dt], pb, st.o[dt]);
  }
}

// Two 16-key tiles under one softmax update.  The PV product runs on
// v_mfma_f32_16x16x32_bf16 with k = 8 g + e: e < 4 are keys 4 g + e of the
// first tile and e >= 4 keys 4 g + e - 4 of the second, which is exactly what
// the two S^T results leave in this lane; V^T is concatenated the same way.
__device__ __forceinline__ void attend_pair(Softmax& st, const bf16x8 (&qb)[4],
                                            const bf16x8 (&kb0)[4], const bf16x8 (&kb1)[4],
                                            const bf16x4 (&vt0)[8], const bf16x4 (&vt1)[8],
                                            int nvalid0, int nvalid1, bool bad0, bool bad1,
                                            float qk_scale, int g) {
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) s0 = mfma_16x16x32_bf16(kb0[j], qb[j], s0);
#pragma unroll
  for (int j = 0; j < 4; ++j) s1 = mfma_16x16x32_bf16(kb1[j], qb[j], s1);
  float z[8];
  float tmax = neg_inf();
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float v0 = bad0 ? qnan() : s0[e] * qk_scale;
    float v1 = bad1 ? qnan() : s1[e] * qk_scale;
    z[e] = (4 * g + e < nvalid0) ? v0 : neg_inf();
    z[4 + e] = (4 * g + e < nvalid1) ? v1 : neg_inf();
    tmax = fmaxf(tmax, fmaxf(z[e], z[4 + e]));
  }
  tmax = max_over_groups(tmax);
  const float m_new = fmaxf(st.m, tmax);
  float psum = 0.f;
  bf16x8 pb;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = exp2f(z[e] - m_new);
    psum += p;
    pb[e] = (__bf16)p;
  }
  // Rescale the output only when some head's running max moved (a wave-uniform
  // branch); after the first pages this is rare.
  if (__ballot(m_new > st.m)) {
    const float alpha = exp2f(st.m - m_new);  // 0 while m = -inf
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[dt] *= alpha;
  }
  st.l += psum;
  st.m = m_new;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const bf16x8 va = {vt0[dt][0], vt0[dt][1], vt0[dt][2], vt0[dt][3],
                       vt1[dt][0], vt1[dt][1], vt1[dt][2], vt1[dt][3]};
    st.o[dt] = mfma_16x16x32_bf16(va, pb, st.o[dt]);
  }
}

// Raw bytes of one 16-token page for this lane.
template <int KV_DT>
struct PageRegs {
  u32x4 k[KV_DT == ISB_BF16 ? 4 : 2];
  uint32_t v[KV_DT == ISB_BF16 ? 16 : 8];
};

template <int KV_DT>
__device__ __forceinline__ void load_page16(PageRegs<KV_DT>& pr, const uint8_t* kpage,
                                            const uint8_t* vpage, int c, int g) {
  if constexpr (KV_DT == ISB_BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) pr.k[j] = ld16(kpage + c * 256 + 64 * g + 16 * j);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      u32x2 w = ld8(vpage + (16 * dt + c) * 32 + 8 * g);
      pr.v[2 * dt] = w[0];
      pr.v[2 * dt + 1] = w[1];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) pr.k[j] = ld16(kpage + c * 128 + 32 * g + 16 * j);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) pr.v[dt] = ld4(vpage + (16 * dt + c) * 16 + 4 * g);
  }
}

template <int KV_DT>
__device__ __forceinline__ void page16_operands(const PageRegs<KV_DT>& pr, int nvalid, int g,
                                                bf16x8 (&kb)[4], bf16x4 (&vt)[8]) {
  if constexpr (KV_DT == ISB_BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) kb[j] = u32x4_as_bf16x8(pr.k[j]);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      bf16x2 a = u32_as_bf16x2(pr.v[2 * dt]);
      bf16x2 b = u32_as_bf16x2(pr.v[2 * dt + 1]);
      vt[dt] = bf16x4{a[0], a[1], b[0], b[1]};
    }
  } else {
    uint32_t w[8] = {pr.k[0][0], pr.k[0][1], pr.k[0][2], pr.k[0][3],
                     pr.k[1][0], pr.k[1][1], pr.k[1][2], pr.k[1][3]};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 lo = e4m3x4_to_bf16x4(w[2 * j]);
      bf16x4 hi = e4m3x4_to_bf16x4(w[2 * j + 1]);
      kb[j] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) vt[dt] = e4m3x4_to_bf16x4(pr.v[dt]);
  }
  if (nvalid < 16) {  // keys past the row's length may hold anything: zero their V
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (4 * g + e >= nvalid) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) vt[dt][e] = (__bf16)0.f;
      }
    }
  }
}

__device__ __forceinline__ bool page_ok(int64_t id, int64_t n) { return id >= 0 && id < n; }

template <int KV_DT>
__global__ __launch_bounds__(256) void pa_decode_kernel(PaArgs a) {
  constexpr int P = KV_DT == ISB_MXFP4 ? 128 : 16;
  constexpr int MAXP = KV_DT == ISB_BF16 ? 4 : 8;  // 16-token pages a wave keeps in flight
  __shared__ float s_m[kPaWaves][16];
  __shared__ float s_l[kPaWaves][16];
  __shared__ float s_o[kPaWaves][16][kHeadDim + 4];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[KV_DT == ISB_MXFP4 ? kMxPageBytes : 16];

  const int row = blockIdx.x, split = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int t = row / a.H_kv, kvh = row % a.H_kv;
  const int32_t* pages = a.sbt + (size_t)row * a.sbt_stride;
  const int p0 = split * a.pps;
  // The page ids of this wave's run are read together with the row length
  // (not after it), so the K/V gathers start one memory round trip sooner.
  const int wb = p0 + wave * a.ppw;
  int my_id = -1;
  if constexpr (KV_DT != ISB_MXFP4) {
    if (lane < a.ppw && wb + lane < a.sbt_stride) my_id = pages[wb + lane];
  }
  const int n_tok = a.sctx[row];
  const int h = threadIdx.x >> 4, d0 = 8 * (threadIdx.x & 15);  // merge / output layout
  __bf16* out_row = a.out + ((size_t)t * a.H_q + kvh * a.G) * kHeadDim;
  if (n_tok <= 0) {  // an empty row attends nothing: split 0 writes its zeros
    if (split == 0 && h < a.G) {
      bf16x8 z;
#pragma unroll
      for (int x = 0; x < 8; ++x) z[x] = (__bf16)0.f;
      *reinterpret_cast<bf16x8*>(out_row + h * kHeadDim + d0) = z;
    }
    return;
  }
  // a row never lists more pages than its table row holds
  const int npages = min((n_tok + P - 1) / P, a.sbt_stride);
  if (p0 >= npages) return;
  const int p1 = min(npages, p0 + a.pps);
  const int live = (npages + a.pps - 1) / a.pps;  // splits of this row that have pages

  // Q^T operand: head kvh * G + c, dims 32 g .. 32 g + 31 (zero past G).
  bf16x8 qb[4];
  {
    const int qbytes = a.q_dt == ISB_BF16 ? 2 : 1;
    if (c < a.G) {
      const uint8_t* qrow = a.q + ((size_t)t * a.H_q + kvh * a.G + c) * kHeadDim * qbytes;
#pragma unroll
      for (int j = 0; j < 4; ++j) qb[j] = load_q8_pa(qrow, a.q_dt, 32 * g + 8 * j);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) qb[j] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  Softmax st;
  st.m = neg_inf();
  st.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if constexpr (KV_DT != ISB_MXFP4) {
    // Each wave owns a run of up to MAXP consecutive pages and issues every
    // load of that run before any math, so a wave keeps its whole share of the
    // row in flight (the split plan sizes runs so ~2048 waves cover a batch).
    constexpr int PB = KV_DT == ISB_BF16 ? 4096 : 2048;
    const int64_t hstride = (int64_t)a.H_kv * PB;  // bytes per page id (all heads)
    const int64_t hoff = (int64_t)kvh * PB;
    const int cnt = max(0, min(a.ppw, p1 - wb));
    PageRegs<KV_DT> pr[MAXP];
    bool ok[MAXP];
#pragma unroll
    for (int j = 0; j < MAXP; ++j) {
      const int64_t id = __builtin_amdgcn_readlane(my_id, j);
      ok[j] = j < cnt && page_ok(id, a.num_pages);
      if (ok[j]) load_page16<KV_DT>(pr[j], a.kp + id * hstride + hoff, a.vp + id * hstride + hoff, c, g);
    }
#pragma unroll
    for (int j = 0; j < MAXP; j += 2) {
      if (j < cnt) {
        const int nv0 = min(16, n_tok - (wb + j) * 16);
        const int nv1 = j + 1 < cnt ? min(16, n_tok - (wb + j + 1) * 16) : 0;
        bf16x8 kb0[4], kb1[4];
        bf16x4 vt0[8], vt1[8];
        if (ok[j]) {
          page16_operands<KV_DT>(pr[j], nv0, g, kb0, vt0);
        } else {
#pragma unroll
          for (int x = 0; x < 4; ++x) kb0[x] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) vt0[dt] = bf16x4{0, 0, 0, 0};
        }
        if (j + 1 < cnt && ok[j + 1]) {
          page16_operands<KV_DT>(pr[j + 1], nv1, g, kb1, vt1);
        } else {
#pragma unroll
          for (int x = 0; x < 4; ++x) kb1[x] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) vt1[dt] = bf16x4{0, 0, 0, 0};
        }
        attend_pair(st, qb, kb0, kb1, vt0, vt1, nv0, nv1, !ok[j], j + 1 < cnt && !ok[j + 1],
                    a.qk_scale, g);
      }
    }
  } else {
    // MXFP4: the workgroup walks its pages together; V is staged in LDS.
    for (int p = p0; p < p1; ++p) {
      const int64_t id = pages[p];
      const bool ok = page_ok(id, a.num_pages);
      __syncthreads();  // previous page's LDS reads are done
      if (ok) {
        const uint8_t* vsrc = a.vp + (id * a.H_kv + kvh) * kMxPageBytes;
        for (int x = threadIdx.x; x < kMxPageBytes / 16; x += 256)
          *reinterpret_cast<u32x4*>(s_v + 16 * x) = ld16(vsrc + 16 * x);
      }
      __syncthreads();
      const uint8_t* kpage = a.kp + ((ok ? id : 0) * a.H_kv + kvh) * kMxPageBytes;
      for (int tile = wave; tile < 8; tile += kPaWaves) {
        const int base = p * P + tile * 16;
        const int nvalid = min(16, n_tok - base);
        if (nvalid <= 0) break;
        bf16x8 kb[4];
        bf16x4 vt[8];
        if (ok) {
          const int tok = tile * 16 + c;
          const u32x4 w = ld16(kpage + tok * 64 + 16 * g);
          const float sc = e8m0_to_f32(ld4(kpage + kMxDataBytes + 4 * tok) >> (8 * g));
#pragma unroll
          for (int j = 0; j < 4; ++j) kb[j] = e2m1x8_to_bf16x8(w[j], sc);
          // V^T: dim 16 dt + c, keys tile*16 + 4 g + e, from the LDS copy.
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int vt_tok = tile * 16 + 4 * g + e;
            const bool on = 4 * g + e < nvalid;
            const uint32_t sw = *reinterpret_cast<const uint32_t*>(s_v + kMxDataBytes + 4 * vt_tok);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
              const int d = 16 * dt + c;
              const uint32_t byte = s_v[vt_tok * 64 + (d >> 1)];
              const uint32_t nib = (d & 1) ? (byte >> 4) : (byte & 0xFu);
              const float sc_v = e8m0_to_f32(sw >> (8 * (d >> 5)));
              const bf16x2 pr2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(nib, sc_v, 0);
              vt[dt][e] = on ? pr2[0] : (__bf16)0.f;
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) kb[j] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) vt[dt] = bf16x4{0, 0, 0, 0};
        }
        attend_tile(st, qb, kb, vt, nvalid, !ok, a.qk_scale, g);
      }
    }
  }

  // Merge the four waves in LDS.
  const float l_tot = sum_over_groups(st.l);
  if (lane < 16) {
    s_m[wave][c] = st.m;
    s_l[wave][c] = l_tot;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_o[wave][c][16 * dt + 4 * g + e] = st.o[dt][e];
  __syncthreads();
  float M = neg_inf();
#pragma unroll
  for (int w = 0; w < kPaWaves; ++w) M = fmaxf(M, s_m[w][h]);
  float L = 0.f, O[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int w = 0; w < kPaWaves; ++w) {
    const float mw = s_m[w][h];
    const float wt = mw == neg_inf() ? 0.f : exp2f(mw - M);
    L += s_l[w][h] * wt;
#pragma unroll
    for (int x = 0; x < 8; ++x) O[x] += s_o[w][h][d0 + x] * wt;
  }

  if (live > 1) {
    // Split-K: publish this split's partial; the reduce launch merges them.
    const size_t base = (size_t)row * a.splits + split;
    float* po = a.part_o + (base * 16 + h) * kHeadDim + d0;
    *reinterpret_cast<f32x4*>(po) = f32x4{O[0], O[1], O[2], O[3]};
    *reinterpret_cast<f32x4*>(po + 4) = f32x4{O[4], O[5], O[6], O[7]};
    if ((threadIdx.x & 15) == 0) {
      a.part_ml[(base * 16 + h) * 2 + 0] = M;
      a.part_ml[(base * 16 + h) * 2 + 1] = L;
    }
    return;
  }
  // A row that fits one split is finished here; the reduce launch skips it.
  if (h < a.G) {
    const float inv = a.v_scale / L;
    bf16x8 ob;
#pragma unroll
    for (int x = 0; x < 8; ++x) ob[x] = (__bf16)(O[x] * inv);
    *reinterpret_cast<bf16x8*>(out_row + h * kHeadDim + d0) = ob;
  }
}

// One workgroup per row with more than one split: merge the row's partial
// results with log-sum-exp weights, normalise and write bf16.  Rows of one
// split (and empty rows) were written by the decode launch.
template <int P>
__global__ __launch_bounds__(256) void pa_reduce_kernel(PaArgs a) {
  const int row = blockIdx.x;
  const int h = threadIdx.x >> 4, d0 = 8 * (threadIdx.x & 15);
  if (h >= a.G) return;
  const int n_tok = a.sctx[row];
  const int npages = n_tok > 0 ? min((n_tok + P - 1) / P, a.sbt_stride) : 0;
  const int live = (npages + a.pps - 1) / a.pps;
  if (live <= 1) return;
  const int t = row / a.H_kv, kvh = row % a.H_kv;
  const size_t b0 = (size_t)row * a.splits * 16 + h;
  float M = neg_inf();
  for (int s = 0; s < live; ++s) M = fmaxf(M, a.part_ml[(b0 + (size_t)s * 16) * 2]);
  float L = 0.f, O[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int s = 0; s < live; ++s) {
    const size_t b = b0 + (size_t)s * 16;
    const float ms = a.part_ml[b * 2];
    const float wt = ms == neg_inf() ? 0.f : exp2f(ms - M);
    L += a.part_ml[b * 2 + 1] * wt;
    const float* po = a.part_o + b * kHeadDim + d0;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(po);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(po + 4);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      O[x] += x0[x] * wt;
      O[4 + x] += x1[x] * wt;
    }
  }
  const float inv = a.v_scale / L;
  bf16x8 ob;
#pragma unroll
  for (int x = 0; x < 8; ++x) ob[x] = (__bf16)(O[x] * inv);
  *reinterpret_cast<bf16x8*>(a.out + ((size_t)t * a.H_q + kvh * a.G + h) * kHeadDim + d0) = ob;
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

extern "C" int isb_sparse_pa_decode(isb_stream_t stream, const void* q, int q_dtype,
                                    const void* k_pool, const void* v_pool, int kv_dtype,
                                    int64_t num_pages, float k_scale, float v_scale,
                                    const int32_t* sparse_bt, int sparse_bt_stride,
                                    const int32_t* sparse_ctx, int num_tokens, int num_q_heads,
                                    int num_kv_heads, int head_dim, float sm_scale,
                                    void* workspace, size_t workspace_bytes, void* out) {
  using namespace isb;
  if (!q || !k_pool || !v_pool || !sparse_bt || !sparse_ctx || !workspace || !out)
    return ISB_E_INVALID_ARG;
  if (num_pages <= 0 || sparse_bt_stride <= 0 || num_tokens <= 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0)
    return ISB_E_INVALID_ARG;
  if (!is_query_dtype(q_dtype) || !is_pool_dtype(kv_dtype)) return ISB_E_UNSUPPORTED_DTYPE;
  if (head_dim != kHeadDim || num_q_heads % num_kv_heads != 0 ||
      num_q_heads / num_kv_heads > 16)
    return ISB_E_SHAPE;
  if (!(sm_scale > 0.f) || !(k_scale > 0.f) || !(v_scale > 0.f)) return ISB_E_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return ISB_E_INVALID_ARG;
  const long long rows = (long long)num_tokens * num_kv_heads;
  if (rows > 0x7FFFFFFFLL) return ISB_E_SHAPE;
  const PaPlan plan = pa_plan(num_tokens, num_kv_heads, sparse_bt_stride, kv_dtype);
  if (plan.splits > 65535) return ISB_E_SHAPE;
  if (workspace_bytes < pa_workspace_bytes(plan)) return ISB_E_WORKSPACE;
  const bool fp8 = kv_dtype == ISB_FP8_E4M3;
  PaArgs a;
  a.q = (const uint8_t*)q;
  a.kp = (const uint8_t*)k_pool;
  a.vp = (const uint8_t*)v_pool;
  a.sbt = sparse_bt;
  a.sctx = sparse_ctx;
  a.part_o = (float*)workspace;
  a.part_ml = a.part_o + (size_t)plan.rows * plan.splits * kPartialO;
  a.out = (__bf16*)out;
  a.num_pages = num_pages;
  a.qk_scale = sm_scale * (fp8 ? k_scale : 1.0f) * 1.4426950408889634f;
  a.v_scale = fp8 ? v_scale : 1.0f;
  a.q_dt = q_dtype;
  a.sbt_stride = sparse_bt_stride;
  a.H_q = num_q_heads;
  a.H_kv = num_kv_heads;
  a.G = num_q_heads / num_kv_heads;
  a.splits = plan.splits;
  a.pps = plan.pages_per_split;
  a.ppw = plan.pages_per_wave;
  hipStream_t st = as_hip(stream);
  dim3 grid((unsigned)rows, plan.splits);
  dim3 rgrid((unsigned)rows);
  if (kv_dtype == ISB_BF16) {
    hipLaunchKernelGGL(pa_decode_kernel<ISB_BF16>, grid, dim3(256), 0, st, a);
    if (plan.splits > 1) hipLaunchKernelGGL(pa_reduce_kernel<16>, rgrid, dim3(256), 0, st, a);
  } else if (kv_dtype == ISB_FP8_E4M3) {
    hipLaunchKernelGGL(pa_decode_kernel<ISB_FP8_E4M3>, grid, dim3(256), 0, st, a);
    if (plan.splits > 1) hipLaunchKernelGGL(pa_reduce_kernel<16>, rgrid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL(pa_decode_kernel<ISB_MXFP4>, grid, dim3(256), 0, st, a);
    if (plan.splits > 1) hipLaunchKernelGGL(pa_reduce_kernel<128>, rgrid, dim3(256), 0, st, a);
  }
  return launch_status();
}
