// Device helpers for the gfx950 kernels of libisb: vector types, exact element
// conversions, MFMA wrappers and wave-level reductions.  CDNA4 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "isb.h"

namespace isb {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kHeadDim = 128;
constexpr int kBlockTokens = 128;
constexpr int kPage16Tokens = 16;
constexpr int kMxDataBytes = 128 * 64;
constexpr int kMxPageBytes = kMxDataBytes + 128 * 4;  // 8704
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

// Where query token t stands: the request it belongs to and its causal
// length L_t (positions 0 .. L_t - 1 of that request are visible to it).
//  - decode batches (req_id null): token t = r q + i is one of the last q
//    tokens of request r, L_t = max(0, seq_lens[r] - (q - 1 - i));
//  - prefill batches (the prefill call of the vLLM API page for
//    sparse_attention_msa, MiniMaxM3SparseAiterPAImpl.forward): per-token
//    request ids and 0-based absolute positions, L_t = abs_pos + 1.  A token
//    whose request id is outside [0, num_reqs) or whose position is outside
//    [0, max_len) is an empty row (L_t = 0): nothing is read through it.
struct TokenMap {
  const int32_t* seq_lens;  // decode: [R]
  const int32_t* req_id;    // prefill: [T]; null for a decode batch
  const int32_t* abs_pos;   // prefill: [T]
  int q_len;                // decode
  int num_reqs;             // prefill
  int max_len;              // prefill
};

struct TokenPos {
  int r, L;
};

__device__ __forceinline__ TokenPos token_pos(const TokenMap& m, int t) {
  if (m.req_id) {
    const int r = m.req_id[t], p = m.abs_pos[t];
    const bool ok = r >= 0 && r < m.num_reqs && p >= 0 && p < m.max_len;
    return TokenPos{ok ? r : 0, ok ? p + 1 : 0};
  }
  const int r = t / m.q_len, i = t - r * m.q_len;
  const int L = m.seq_lens[r] - (m.q_len - 1 - i);
  return TokenPos{r, L > 0 ? L : 0};
}

// Index of this thread's wave in the workgroup, as a wave-uniform (scalar)
// value, so that addresses derived from it live in scalar registers.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }
__device__ __forceinline__ float qnan() { return __builtin_nanf(""); }

// ----------------------------------------------------------------- loads
// Plain vector loads that the memory system coalesces.
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 ld8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}
// Raw buffer loads from one cache page.  The page's base address sits in a
// wave-uniform buffer descriptor (scalar registers), so a wave's loads share
// one per-lane offset register and add the rest as scalar and immediate
// offsets, instead of holding a 64-bit address pair per load.  Descriptor
// word 3 is the raw-buffer format of the gfx9 family; `bytes` bounds the page
// (loads past it return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// 16 / 4 bytes at voff + soff, nontemporal (cache policy nt): cache pages
// are read once per launch, and streaming them past the caches raises the
// achieved HBM rate of the index scan by about a tenth.
__device__ __forceinline__ u32x4 bl16_nt(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2));
}
__device__ __forceinline__ uint32_t bl4_nt(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 2);
}
// The same with the default cache policy: pages that several rows of one
// request read (their selections share blocks) stay in L2 and the last-level
// cache between those reads.
__device__ __forceinline__ u32x4 bl16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t bl4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// ----------------------------------------------------------------- conversions
// All exact: e4m3 and e2m1 * 2^k values are representable in bf16 (the
// hardware conversions round only when a value does not fit, which e4m3 and
// in-range e2m1 * scale never do).

// Two e4m3 bytes (bytes 0,1 when hi = false, 2,3 when hi = true) -> two bf16.
__device__ __forceinline__ bf16x2 e4m3x2_to_bf16x2(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
            : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
}

// Eight e4m3 bytes (dword lo: bytes 0..3, then dword hi) -> eight bf16.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                                          __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)});
}

// The same eight e4m3 bytes -> f16 (exact as well: f16 holds every e4m3
// value, subnormals included).
__device__ __forceinline__ f16x8 e4m3x8_to_f16x8(uint32_t lo, uint32_t hi) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return __builtin_bit_cast(f16x8, u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                                         __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)});
}

// Eight e2m1 nibbles of one dword (low nibble of byte 0 first) -> eight bf16,
// each multiplied by `scale` (a power of two from an e8m0 byte).
__device__ __forceinline__ bf16x8 e2m1x8_to_bf16x8(uint32_t w, float scale) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// e8m0 byte -> float 2^(e - 127); 0xFF -> NaN; 0 -> 2^-127 (subnormal).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  e &= 0xFFu;
  if (e == 0xFFu) return qnan();
  if (e == 0u) return __uint_as_float(0x00400000u);
  return __uint_as_float(e << 23);
}

__device__ __forceinline__ bf16x2 u32_as_bf16x2(uint32_t w) {
  return __builtin_bit_cast(bf16x2, w);
}
__device__ __forceinline__ bf16x8 u32x4_as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

// ----------------------------------------------------------------- MFMA
// v_mfma_f32_16x16x32_bf16: lane l = 16 g + r supplies A[r][8 g + i] and
// B[8 g + i][r] (i < 8); the result lane l holds D[4 g + i][r] (i < 4).
__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// The same product with both sources kept live past the instruction (an
// empty asm that takes the result reads them, so it cannot be placed before
// the product), for kernels whose register budget is tight enough that the
// allocator would otherwise place the destination over a source register;
// see mfma_scale_fp4_e4m3.
template <bool KEEP>
__device__ __forceinline__ f32x4 mfma_16x16x32_bf16_k(bf16x8 a, bf16x8 b, f32x4 c) {
  f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  if constexpr (KEEP) asm volatile("" : "+v"(d) : "v"(a), "v"(b));
  return d;
}
// v_mfma_f32_16x16x32_f16: the same lane layout with f16 operands; KEEP as
// for mfma_16x16x32_bf16_k.
template <bool KEEP>
__device__ __forceinline__ f32x4 mfma_16x16x32_f16_k(f16x8 a, f16x8 b, f32x4 c) {
  f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  if constexpr (KEEP) asm volatile("" : "+v"(d) : "v"(a), "v"(b));
  return d;
}
// v_mfma_f32_16x16x16_bf16: lane l = 16 g + r supplies A[r][4 g + i] and
// B[4 g + i][r] (i < 4); result as above.
__device__ __forceinline__ f32x4 mfma_16x16x16_bf16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
template <bool KEEP>
__device__ __forceinline__ f32x4 mfma_16x16x16_bf16_k(bf16x4 a, bf16x4 b, f32x4 c) {
  f32x4 d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  if constexpr (KEEP) asm volatile("" : "+v"(d) : "v"(a), "v"(b));
  return d;
}
// v_mfma_scale_f32_16x16x128_f8f6f4 with A in e2m1 and B in e4m3:
//   A lane l = 16 g + r: row r, k = 32 g .. 32 g + 31 as 32 nibbles in the
//     first four dwords (low nibble first); `scale_a` (e8m0 in bits 0..7)
//     scales exactly those 32 elements;
//   B lane l = 16 g + r: column r, bytes 0..15 are k = 16 g .. 16 g + 15 and
//     bytes 16..31 are k = 64 + 16 g .. 64 + 16 g + 15; unit scale (127).
// The empty asm keeps both sources live past the instruction: without it the
// register allocator may place the destination over a source register, which
// corrupts the product.
__device__ __forceinline__ f32x4 mfma_scale_fp4_e4m3(i32x8 a, i32x8 b, f32x4 c, int scale_a) {
  f32x4 d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, scale_a, 0, 127);
  asm volatile("" ::"v"(a), "v"(b));
  return d;
}

// The same instruction with A and B both in e4m3, unit scales: lane
// l = 16 g + r supplies 32 bytes of row r of A and of column r of B, and byte
// j of a lane group's A lanes meets byte j of the same group's B lanes in
// the sum (the 8-bit layout above is the same for A and B), so any placement
// of the 128 k values over a group's 32 bytes that A and B share gives the
// whole dot product.
__device__ __forceinline__ f32x4 mfma_scale_e4m3(i32x8 a, i32x8 b, f32x4 c) {
  f32x4 d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  asm volatile("" ::"v"(a), "v"(b));
  return d;
}

// ----------------------------------------------------------------- cross-lane
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
// DPP controls: quad_perm [1,0,3,2] (xor 1), [2,3,0,1] (xor 2), row_half_mirror,
// row_mirror.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

__device__ __forceinline__ float shfl_xor_f32(float x, int m) { return __shfl_xor(x, m, kWave); }

// Maximum over the four lanes {r, r+16, r+32, r+48} (the lane groups of an
// MFMA result column).
__device__ __forceinline__ float max_over_groups(float x) {
  x = fmaxf(x, shfl_xor_f32(x, 16));
  x = fmaxf(x, shfl_xor_f32(x, 32));
  return x;
}
__device__ __forceinline__ float sum_over_groups(float x) {
  x += shfl_xor_f32(x, 16);
  x += shfl_xor_f32(x, 32);
  return x;
}

}  // namespace isb
