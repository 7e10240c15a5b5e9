// Device code of the top-k block selection, shared by the selection kernels
// (topk_select.hip) and the attention launch that selects its own rows
// (sparse_pa.hip).
//
// Rule (ROCm/ATOM PR 2962: the decode commit keeps the tail page in every
// selection; the pad-row fix makes a row of causal length 0 compute nothing): a row with n_t
// valid blocks keeps its tail block n_t - 1 and the top_k - 1 best of blocks
// [0, n_t - 1), ties to the lower block index; NaN ranks below every number
// and -0.0 equals +0.0.  The selection is written ascending and padded with -1.
//
// Method: radix select on order-preserving 32-bit keys.  On rows of four or
// more keys a thread, the bits every candidate key shares are found first
// (AND and OR over the row).  Passes of up to 8 bits below them each count,
// per wave, the keys that match the prefix found so far into a 256-bin LDS
// histogram (no contention between waves); the waves' bins are summed and the
// digit where the count of larger keys reaches top_k - 1 is found with a
// wave-wide prefix sum.  With four waves every wave finds the digit itself
// from histograms that alternate between two buffers, so a pass has one
// barrier; with more waves wave 0 finds it and hands it over in LDS (two
// barriers).  The passes stop early once the keys under the prefix found so
// far are exactly the ones still needed.  Keys above the threshold (compared
// under the prefix's mask) are taken, and keys equal to it are taken in block
// order until the count is met.  One scan of packed (greater, equal) counts
// gives each thread its output position, so the output is ascending without
// a sort.
#pragma once

#include "isb_device.h"

namespace isb {

// Order-preserving key: larger score -> larger key; -0.0 == +0.0; every NaN
// maps to 0, below -inf (0x007FFFFF).
__device__ __forceinline__ uint32_t order_key(float s) {
  if (s != s) return 0u;
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts within rows of 16
// lanes, then the totals of rows 0 / 2 broadcast into rows 1 / 3 and the
// total of lanes 0..31 into rows 2 and 3 (DPP; lanes with no source add 0).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Inclusive prefix sum over the NT threads of the workgroup.  REUSE: s_wave
// may be written again (by a later scan) before the caller's next barrier, so
// the scan ends with one.
template <int NT, bool REUSE = true>
__device__ __forceinline__ int block_incl_scan(int v, int* s_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) before += w < wave ? s_wave[w] : 0;
  if constexpr (REUSE) __syncthreads();
  return x + before;
}

// Entries j0 .. j0 + E - 1 of a row of n entries (0 past the end).  VEC: the
// row starts 16-byte aligned and n is a multiple of 4, so the entries arrive
// in 16-byte (E >= 4) or 8-byte (E = 2) loads; per-entry 4-byte loads at a
// stride of E entries would touch E times as many cache lines.
template <int E, bool VEC, typename T>
__device__ __forceinline__ void load_run(const T* row, int j0, int n, T (&v)[E]) {
  if constexpr (VEC && E >= 4) {
#pragma unroll
    for (int x = 0; x < E / 4; ++x) {
      if (j0 + 4 * x < n) {
        const u32x4 w = ld16(row + j0 + 4 * x);
        // each element copied to a scalar first: a bit cast taken straight
        // from a vector element reads element 0 here
        const uint32_t e[4] = {w[0], w[1], w[2], w[3]};
#pragma unroll
        for (int y = 0; y < 4; ++y) v[4 * x + y] = __builtin_bit_cast(T, e[y]);
      } else {
#pragma unroll
        for (int y = 0; y < 4; ++y) v[4 * x + y] = T(0);
      }
    }
  } else if constexpr (VEC && E == 2) {
    if (j0 < n) {
      const u32x2 w = ld8(row + j0);
      const uint32_t e0 = w[0], e1 = w[1];
      v[0] = __builtin_bit_cast(T, e0);
      v[1] = __builtin_bit_cast(T, e1);
    } else {
      v[0] = v[1] = T(0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = j0 + i < n ? row[j0 + i] : T(0);
  }
}

// LDS of select_row: one histogram per wave (two with four waves, used by
// alternate passes), wave totals, the digit found.
template <int NT>
struct alignas(16) SelectLds {
  static constexpr int NB = NT <= 256 ? 2 : 1;
  int hist[NB][NT / 64][256];
  int wave_tot[NT / 64];
  uint32_t wave_and[NT / 64], wave_or[NT / 64];
  int pick[3];
};

// The selection of one row whose scores for blocks E t .. E t + E - 1 are in
// thread t's sc[] (NT threads, all of the workgroup).  put(k, b) receives
// selection slot k < K and its block b (ascending; -1 past the m selected
// blocks).  Returns m = min(K, n_t).  Every thread must call it.
template <int NT, int E, typename PutFn>
__device__ __forceinline__ int select_row(const float (&sc)[E], int nt, int K, SelectLds<NT>& sl, PutFn put) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int W = nt - 1;  // candidates [0, W); block W is the tail
  if (nt == 0 || W <= K - 1) {
    for (int j = tid; j < K; j += NT) put(j, j < nt ? j : -1);
    return nt;
  }
  uint32_t key[E];
#pragma unroll
  for (int i = 0; i < E; ++i) key[i] = E * tid + i < W ? order_key(sc[i]) : 0u;
  const int jlim = W - E * tid;  // my keys i < jlim are candidates
  const int keep = K - 1;        // candidates to select (0 when top_k = 1)
  int need = keep;
  // Rows of four or more keys a thread start below the candidates' common
  // leading bits (AND and OR of every key agree there).  Scores of one row
  // mostly share their sign and leading exponent bits, and a pass over such
  // bits puts nearly every key in one or two bins, whose atomic counts
  // serialize; for narrower rows the extra exchange costs more than it saves.
  uint32_t kand = 0u, kor = ~0u;
  if constexpr (E >= 4) {
    kand = ~0u;
    kor = 0u;
#pragma unroll
    for (int i = 0; i < E; ++i)
      if (i < jlim) {
        kand &= key[i];
        kor |= key[i];
      }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      kand &= (uint32_t)__shfl_xor((int)kand, off, kWave);
      kor |= (uint32_t)__shfl_xor((int)kor, off, kWave);
    }
    if (lane == 0) {
      sl.wave_and[wave] = kand;
      sl.wave_or[wave] = kor;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      kand &= sl.wave_and[w];
      kor |= sl.wave_or[w];
    }
  }
  // bits [0, hi) differ between candidates (all 32 may, for narrow rows); the
  // bits above are the prefix
  int hi = kand == kor ? 0 : 32 - __builtin_clz(kand ^ kor);
  uint32_t pmask = hi == 32 ? 0u : ~((1u << hi) - 1u);
  uint32_t prefix = kand & pmask;
  // With need >= 1 every pass finds its digit (need never exceeds the keys
  // that match the prefix); with top_k = 1 only the tail is selected.
  constexpr int NB = SelectLds<NT>::NB;
  for (int pass = 0; hi > 0 && keep > 0; ++pass) {
    const int lo = hi > 8 ? hi - 8 : 0;  // this pass's digit: bits [lo, hi)
    const uint32_t dmask = (1u << (hi - lo)) - 1u;
    int(&hist)[NW][256] = sl.hist[NB == 2 ? (pass & 1) : 0];
    // this wave's histogram: cleared, then filled (LDS operations of a wave
    // complete in order; no wave still reads it: with two buffers its last
    // reader finished before the previous pass's barrier, with one buffer
    // wave 0 finished before the barrier that ended the previous pass)
#pragma unroll
    for (int x = 0; x < 4; ++x) hist[wave][lane + 64 * x] = 0;
#pragma unroll
    for (int i = 0; i < E; ++i)
      if (i < jlim && (key[i] & pmask) == prefix) atomicAdd(&hist[wave][(key[i] >> lo) & dmask], 1);
    __syncthreads();
    int digit = 0, above = 0, inside = 0;
    if (NB == 2 || wave == 0) {
      // lane l takes digits 255 - 4 l - x (x < 4): descending digit order
      int cnt[4] = {0, 0, 0, 0};
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int4 v = *reinterpret_cast<const int4*>(&hist[w][252 - 4 * lane]);
        cnt[0] += v.w;
        cnt[1] += v.z;
        cnt[2] += v.y;
        cnt[3] += v.x;
      }
      const int tot = cnt[0] + cnt[1] + cnt[2] + cnt[3];
      int run = wave_incl_scan(tot) - tot;  // keys in higher digits
      int fd = -1, fr = 0, fc = 0;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        if (run < need && need <= run + cnt[x]) {
          fd = 255 - 4 * lane - x;
          fr = run;
          fc = cnt[x];
        }
        run += cnt[x];
      }
      // exactly one lane found the digit
      const int src = __builtin_ctzll(__ballot(fd >= 0));
      digit = __builtin_amdgcn_readlane(fd, src);
      above = __builtin_amdgcn_readlane(fr, src);
      inside = __builtin_amdgcn_readlane(fc, src);
    }
    if constexpr (NB == 1) {
      if (tid == 0) {
        sl.pick[0] = digit;
        sl.pick[1] = above;
        sl.pick[2] = inside;
      }
      __syncthreads();
      digit = sl.pick[0];
      above = sl.pick[1];
      inside = sl.pick[2];
    }
    prefix |= (uint32_t)digit << lo;
    pmask |= dmask << lo;
    need -= above;
    hi = lo;
    // Every key under the prefix is taken: the lower digits cannot change
    // the selection, so the passes stop (the keys compare under the mask).
    if (inside == need) break;
  }
  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    if (i < jlim) {
      gt += (key[i] & pmask) > prefix;
      eq += (key[i] & pmask) == prefix;
    }
  }
  const int packed = gt | (eq << 16);
  // one scan a call: its totals are not written again
  const int before = block_incl_scan<NT, false>(packed, sl.wave_tot) - packed;
  int seen = before >> 16;
  int pos = (before & 0xFFFF) + min(seen, need);
#pragma unroll
  for (int i = 0; i < E; ++i) {
    if (i < jlim && keep > 0) {
      const uint32_t mk = key[i] & pmask;
      bool sel = mk > prefix;
      if (mk == prefix) sel = seen++ < need;
      if (sel && pos < keep) put(pos++, E * tid + i);
    }
  }
  if (tid == 0) put(K - 1, W);  // the tail block, larger than every candidate
  return K;
}

}  // namespace isb
