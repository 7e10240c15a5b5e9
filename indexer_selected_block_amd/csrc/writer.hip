// isb_write_cache: the new tokens' keys, values and index keys quantised into
// the paged caches; isb_quantize_e4m3: the unit-scale e4m3 query cast.
//
// The step in front of the decode path (ROCm/ATOM PR 2962, the commit
// messages under Follow-ups: one fused kernel encodes the new tokens' K and V
// in the MXFP4 / fp8 page format and emits the query in float8_e4m3fn, scale
// 1, clamped at the format's maximum).  Token i of request r's q new tokens sits at position
// seq_lens[r] - q + i; one wave writes one (token, vector) pair, two dims a
// lane: the K and V of every KV head and the token's index key.
//   fp8   - e4m3 of x / scale (formed in fp32): round to nearest, ties to the
//           even code, saturating at +-448, NaN to 0x7F, sign kept;
//   MXFP4 - per 32 dims the e8m0 exponent floor(log2 amax) - 2 (clamped to
//           [-127, 127]), each element's e2m1 code rounded to nearest, ties
//           to the even code, saturating at +-6 (OCP MX v1.0);
//   bf16  - stored as given.
// Before the encoding, K and the index key (and, in isb_prepare_query, the
// query) may take the fused step's QK-norm and rope, with parameters the
// caller gives (isb_norm_rope): y = w x / sqrt(mean(x^2) + eps), then dim
// pairs turned by the table angle of the token's position; computed in fp32.
// Bytes go where the decode kernels read them (the page layouts of isb.h).
// This is not a bandwidth kernel: a decode step writes a few hundred bytes a
// token.
#include "isb_device.h"
#include "isb_host.h"

namespace isb {

// e4m3fn code of y (see above), computed on its binary32 bits.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (!(a == a)) return 0x7Fu;
  if (a >= 448.f) return sign | 0x7Eu;
  if (a < 0.015625f)  // below 2^-6: subnormal steps of 2^-9 (the product is exact)
    return sign | (uint32_t)__builtin_rintf(a * 512.f);  // 8 is the smallest normal, code 0x08
  const uint32_t ua = __float_as_uint(a);
  const uint32_t ex = ((ua >> 23) & 0xFFu) - 127u + 7u;  // biased e4m3 exponent, 1..15
  const uint32_t mant = ua & 0x7FFFFFu;
  uint32_t r = mant >> 20;  // the top three mantissa bits
  const uint32_t rem = mant & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;  // a carry into the exponent is the right code
  return sign | ((ex << 3) + r);
}

// e2m1 code of y (finite), rounding to nearest with ties to the even code and
// saturating: the thresholds are the midpoints between 0, .5, 1, 1.5, 2, 3,
// 4, 6, taken inclusive where the upper neighbour's code is even.
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const float a = fabsf(y);
  const uint32_t m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) +
                     (a > 5.f);
  return ((__float_as_uint(y) >> 28) & 8u) | m;
}

// The device copy of an isb_norm_rope (all zero: nothing to apply).
struct NormRope {
  const float* w;   // [128] or null
  const float* cs;  // [npos][rot / 2] or null
  const float* sn;
  int64_t npos;
  float eps;
  int rot, neox;
};

__device__ __forceinline__ bool applies(const NormRope& f) { return f.w != nullptr || f.cs != nullptr; }

// The QK-norm, then the rope, of one 128-dim vector held two dims a lane
// (x0, x1 = dims 2 lane, 2 lane + 1) at position p < npos.  Wave-uniform.
__device__ __forceinline__ void norm_rope(const NormRope& f, int p, int lane, float& x0, float& x1) {
  if (f.w) {
    float ss = x0 * x0 + x1 * x1;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, kWave);
    const float r = 1.f / sqrtf(ss * (1.f / 128.f) + f.eps);
    x0 = x0 * r * f.w[2 * lane];
    x1 = x1 * r * f.w[2 * lane + 1];
  }
  if (f.cs) {
    const int half = f.rot >> 1, d = 2 * lane;
    const float* c = f.cs + (int64_t)p * half;
    const float* s = f.sn + (int64_t)p * half;
    if (f.neox) {
      // dims d < half pair with d + half, held by the lane half / 2 further on
      const int q = half >> 1;
      const int src = lane < q ? lane + q : lane - q;
      const float y0 = __shfl(x0, src, kWave), y1 = __shfl(x1, src, kWave);
      if (d < half) {
        x0 = x0 * c[d] - y0 * s[d];
        x1 = x1 * c[d + 1] - y1 * s[d + 1];
      } else if (d < f.rot) {
        const int j = d - half;
        x0 = x0 * c[j] + y0 * s[j];
        x1 = x1 * c[j + 1] + y1 * s[j + 1];
      }
    } else if (d < f.rot) {  // the pair (d, d + 1) is this lane's
      const float a = x0, b = x1, cj = c[lane], sj = s[lane];
      x0 = a * cj - b * sj;
      x1 = b * cj + a * sj;
    }
  }
}

// bf16 code of x: round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

struct WriteArgs {
  const uint16_t* k_new;    // bf16 [T][H_kv][128]
  const uint16_t* v_new;
  const uint16_t* idx_new;  // bf16 [T][128]
  const int32_t* bt;
  const int32_t* seq_lens;
  uint8_t* k_pool;
  uint8_t* v_pool;
  uint8_t* idx_pool;
  int64_t num_pages, idx_blocks;
  float k_scale, v_scale, idx_scale;
  int bt_stride, q_len, H_kv, T;
  NormRope ktf, itf;  // the keys' and the index keys' QK-norm / rope
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// One MXFP4 token: dims 2 lane, 2 lane + 1 of the 8704 B page at `page`, slot s.
__device__ __forceinline__ void put_mxfp4(uint8_t* page, int slot, float x0, float x1, int lane) {
  // group maximum over the 16 lanes that hold the group's 32 dims
  float amax = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
  // floor(log2 amax) from the exponent field: exact for normal numbers; zero
  // and binary32 subnormals clamp to the smallest e8m0 exponent
  const int ebits = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  const int e = ebits == 0 ? -127 : max(-127, min(127, ebits - 127 - 2));
  const float inv = __builtin_ldexpf(1.f, -e);  // exact power of two
  const uint32_t code = e2m1_code(x0 * inv) | (e2m1_code(x1 * inv) << 4);
  page[64 * slot + lane] = (uint8_t)code;
  if ((lane & 15) == 0) page[kMxDataBytes + 4 * slot + (lane >> 4)] = (uint8_t)(e + 127);
}

// Dims d, d + 1 (d even) of key c of a 16-token K page (or index tile) at
// `base`: byte 1024 ((d mod 32) div (16/e)) + 256 (d div 32) + 16 c + e (d mod (16/e)),
// so the pair is contiguous.  w holds their bf16 bits (d in the low half).
template <int DT>
__device__ __forceinline__ void put_k16(uint8_t* base, int c, int d, uint32_t w, float x0, float x1, float scale) {
  if constexpr (DT == ISB_BF16) {
    *reinterpret_cast<uint32_t*>(base + 1024 * ((d & 31) >> 3) + 256 * (d >> 5) + 16 * c + 2 * (d & 7)) = w;
  } else {
    const uint32_t q = e4m3_code(x0 / scale) | (e4m3_code(x1 / scale) << 8);
    *reinterpret_cast<uint16_t*>(base + 1024 * ((d & 31) >> 4) + 256 * (d >> 5) + 16 * c + (d & 15)) = (uint16_t)q;
  }
}

// Dims d, d + 1 (d = 16 dt + c, c even) of key t of a 16-token V page at
// `base`: byte 1024 (dt div (4/e)) + 256 (t div 4) + 16 c + 4 e (dt mod (4/e)) + e (t mod 4);
// dim d + 1 is 16 bytes further.
template <int DT>
__device__ __forceinline__ void put_v16(uint8_t* base, int t, int d, uint32_t w, float x0, float x1, float scale) {
  const int dt = d >> 4, c = d & 15;
  if constexpr (DT == ISB_BF16) {
    uint8_t* at = base + 1024 * (dt >> 1) + 256 * (t >> 2) + 16 * c + 8 * (dt & 1) + 2 * (t & 3);
    *reinterpret_cast<uint16_t*>(at) = (uint16_t)(w & 0xFFFFu);
    *reinterpret_cast<uint16_t*>(at + 16) = (uint16_t)(w >> 16);
  } else {
    uint8_t* at = base + 1024 * (dt >> 2) + 256 * (t >> 2) + 16 * c + 4 * (dt & 3) + (t & 3);
    at[0] = (uint8_t)e4m3_code(x0 / scale);
    at[16] = (uint8_t)e4m3_code(x1 / scale);
  }
}

// One wave a (token, vector): vector v < H_kv is K of head v, v < 2 H_kv is V
// of head v - H_kv, v = 2 H_kv the index key (absent when idx_new is null: a
// layer that reuses another layer's top-k keeps no index cache of its own).
// grid ceil(T vecs / 4), four waves a workgroup.  Every test that skips a write is wave-uniform (the
// MXFP4 group maximum is a lane exchange).
template <int KV_DT, int IDX_DT>
__global__ __launch_bounds__(256) void write_cache_kernel(WriteArgs a) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int vecs = 2 * a.H_kv + (a.idx_new != nullptr);
  const long long item = (long long)blockIdx.x * 4 + wave;
  if (item >= (long long)a.T * vecs) return;
  const int t = (int)(item / vecs), v = (int)(item % vecs);
  const int r = t / a.q_len, i = t % a.q_len;
  const int p = a.seq_lens[r] - a.q_len + i;
  if (p < 0 || p / kBlockTokens >= a.bt_stride) return;  // a pad row, or past the table
  // a position past a rope table: the whole token is skipped
  if ((a.ktf.cs && p >= a.ktf.npos) || (a.idx_new && a.itf.cs && p >= a.itf.npos)) return;
  const int64_t blk = a.bt[(size_t)r * a.bt_stride + p / kBlockTokens];
  const int slot = p % kBlockTokens;
  const int d = 2 * lane;  // this lane's dims d, d + 1
  const bool is_idx = v == 2 * a.H_kv, is_v = !is_idx && v >= a.H_kv;
  const int g = is_idx ? 0 : v % a.H_kv;
  const uint16_t* src = is_idx ? a.idx_new + (size_t)t * kHeadDim
                               : (is_v ? a.v_new : a.k_new) + ((size_t)t * a.H_kv + g) * kHeadDim;
  uint32_t w = *reinterpret_cast<const uint32_t*>(src + d);
  float x0 = bf16_bits_to_f32(w & 0xFFFFu), x1 = bf16_bits_to_f32(w >> 16);
  if (!is_v) {
    const NormRope& f = is_idx ? a.itf : a.ktf;
    if (applies(f)) {
      norm_rope(f, p, lane, x0, x1);
      w = bf16_rne(x0) | (bf16_rne(x1) << 16);  // the bf16 pool's bits
    }
  }
  if (is_idx) {  // page id = block id, no head dimension
    if (blk < 0 || blk >= a.idx_blocks) return;
    if constexpr (IDX_DT == ISB_MXFP4) {
      put_mxfp4(a.idx_pool + blk * kMxPageBytes, slot, x0, x1, lane);
    } else {
      constexpr int E = IDX_DT == ISB_BF16 ? 2 : 1;
      uint8_t* tile = a.idx_pool + blk * (16384 * E) + (slot >> 4) * (2048 * E);
      put_k16<IDX_DT>(tile, slot & 15, d, w, x0, x1, a.idx_scale);
    }
    return;
  }
  uint8_t* pool = is_v ? a.v_pool : a.k_pool;
  if constexpr (KV_DT == ISB_MXFP4) {
    if (blk < 0 || blk >= a.num_pages) return;
    put_mxfp4(pool + (blk * a.H_kv + g) * kMxPageBytes, slot, x0, x1, lane);
  } else {
    constexpr int E = KV_DT == ISB_BF16 ? 2 : 1;
    const int64_t page = 8 * blk + (slot >> 4);
    if (blk < 0 || page >= a.num_pages) return;
    uint8_t* base = pool + (page * a.H_kv + g) * (2048 * E);
    if (is_v) put_v16<KV_DT>(base, slot & 15, d, w, x0, x1, a.v_scale);
    else put_k16<KV_DT>(base, slot & 15, d, w, x0, x1, a.k_scale);
  }
}

// The query cast: four elements a thread.
__global__ __launch_bounds__(256) void quantize_e4m3_kernel(const uint16_t* x, int64_t n, uint8_t* out) {
  const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (i0 + k < n) out[i0 + k] = (uint8_t)e4m3_code(bf16_bits_to_f32(x[i0 + k]));
}

// isb_prepare_query: one wave a (token, head) vector of q [T][H][128] bf16;
// out [T][H][128] as bf16 codes (OUT_E = 2) or unit-scale e4m3 (OUT_E = 1).
struct QueryArgs {
  const uint16_t* q;
  const int32_t* seq_lens;
  uint8_t* out;
  NormRope tf;
  int H, q_len, T;
};

template <int OUT_E>
__global__ __launch_bounds__(256) void prepare_query_kernel(QueryArgs a) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const long long item = (long long)blockIdx.x * 4 + wave;
  if (item >= (long long)a.T * a.H) return;
  const int t = (int)(item / a.H);
  const int r = t / a.q_len, i = t % a.q_len;
  const int p = a.seq_lens[r] - a.q_len + i;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(a.q + (size_t)item * kHeadDim + 2 * lane);
  float x0 = bf16_bits_to_f32(w & 0xFFFFu), x1 = bf16_bits_to_f32(w >> 16);
  uint32_t c0, c1;
  if (p < 0) {  // a pad row: zeros
    c0 = c1 = 0u;
  } else if (a.tf.cs && p >= a.tf.npos) {  // past the rope table: NaN
    c0 = c1 = OUT_E == 2 ? 0x7FC0u : 0x7Fu;
  } else {
    norm_rope(a.tf, p, lane, x0, x1);
    c0 = OUT_E == 2 ? bf16_rne(x0) : e4m3_code(x0);
    c1 = OUT_E == 2 ? bf16_rne(x1) : e4m3_code(x1);
  }
  if constexpr (OUT_E == 2)
    *reinterpret_cast<uint32_t*>(a.out + ((size_t)item * kHeadDim + 2 * lane) * 2) = c0 | (c1 << 16);
  else
    *reinterpret_cast<uint16_t*>(a.out + (size_t)item * kHeadDim + 2 * lane) = (uint16_t)(c0 | (c1 << 8));
}

// isb_norm_rope -> NormRope after the host checks; 0 or an ISB_E_* code.
static int read_norm_rope(const isb_norm_rope* h, NormRope& f) {
  f = NormRope{nullptr, nullptr, nullptr, 0, 0.f, 0, 0};
  if (!h) return ISB_OK;
  if (h->norm_weight) {
    if (!(h->eps >= 0.f) || !(h->eps < INFINITY) || reinterpret_cast<uintptr_t>(h->norm_weight) % 4)
      return ISB_E_INVALID_ARG;
    f.w = h->norm_weight;
    f.eps = h->eps;
  }
  if (h->rope_cos || h->rope_sin) {
    if (!h->rope_cos || !h->rope_sin || h->rope_positions <= 0) return ISB_E_INVALID_ARG;
    if (h->rot_dim < 4 || h->rot_dim > kHeadDim || h->rot_dim % 4) return ISB_E_SHAPE;
    if (reinterpret_cast<uintptr_t>(h->rope_cos) % 4 || reinterpret_cast<uintptr_t>(h->rope_sin) % 4)
      return ISB_E_INVALID_ARG;
    f.cs = h->rope_cos;
    f.sn = h->rope_sin;
    f.npos = h->rope_positions;
    f.rot = h->rot_dim;
    f.neox = h->neox != 0;
  }
  return ISB_OK;
}

template <int KV_DT, int IDX_DT>
static void launch_write(const WriteArgs& a, hipStream_t st) {
  const long long items = (long long)a.T * (2 * a.H_kv + (a.idx_new != nullptr));
  hipLaunchKernelGGL((write_cache_kernel<KV_DT, IDX_DT>), dim3((unsigned)((items + 3) / 4)), dim3(256), 0, st, a);
}

template <int KV_DT>
static void launch_write_kv(const WriteArgs& a, int idx_dtype, hipStream_t st) {
  if (idx_dtype == ISB_BF16) launch_write<KV_DT, ISB_BF16>(a, st);
  else if (idx_dtype == ISB_FP8_E4M3) launch_write<KV_DT, ISB_FP8_E4M3>(a, st);
  else launch_write<KV_DT, ISB_MXFP4>(a, st);
}

}  // namespace isb

extern "C" int isb_write_cache(isb_stream_t stream, const void* k_new, const void* v_new,
                               const void* idx_new, const int32_t* block_table, int block_table_stride,
                               const int32_t* seq_lens, int num_reqs, int decode_query_len,
                               int num_kv_heads, void* k_pool, void* v_pool, int kv_dtype, float k_scale,
                               float v_scale, int64_t num_pages, void* idx_pool, int idx_dtype,
                               float idx_scale, int64_t idx_pool_blocks, const isb_norm_rope* k_norm_rope,
                               const isb_norm_rope* idx_norm_rope) {
  using namespace isb;
  if (!k_new || !v_new || !block_table || !seq_lens || !k_pool || !v_pool) return ISB_E_INVALID_ARG;
  const bool with_idx = idx_new != nullptr;
  if (with_idx != (idx_pool != nullptr)) return ISB_E_INVALID_ARG;
  if (block_table_stride <= 0 || num_reqs <= 0 || decode_query_len <= 0 || num_kv_heads <= 0 ||
      num_pages <= 0 || (with_idx && idx_pool_blocks <= 0))
    return ISB_E_INVALID_ARG;
  if (!is_pool_dtype(kv_dtype) || (with_idx && !is_pool_dtype(idx_dtype))) return ISB_E_UNSUPPORTED_DTYPE;
  if ((kv_dtype == ISB_FP8_E4M3 && !(k_scale > 0.f && v_scale > 0.f)) ||
      (with_idx && idx_dtype == ISB_FP8_E4M3 && !(idx_scale > 0.f)))
    return ISB_E_INVALID_ARG;
  const long long T = (long long)num_reqs * decode_query_len;
  if (num_kv_heads > 65535 || T > 0x7FFFFFFFLL || T * (2LL * num_kv_heads + 1) > 4LL * 0x7FFFFFFFLL)
    return ISB_E_SHAPE;
  if (reinterpret_cast<uintptr_t>(k_new) % 4 || reinterpret_cast<uintptr_t>(v_new) % 4 ||
      reinterpret_cast<uintptr_t>(idx_new) % 4 || reinterpret_cast<uintptr_t>(k_pool) % 4 ||
      reinterpret_cast<uintptr_t>(v_pool) % 4 || reinterpret_cast<uintptr_t>(idx_pool) % 4)
    return ISB_E_INVALID_ARG;
  NormRope ktf, itf;
  int e = read_norm_rope(k_norm_rope, ktf);
  if (!e && with_idx) e = read_norm_rope(idx_norm_rope, itf);
  if (e) return e;
  if (!with_idx) itf = NormRope{nullptr, nullptr, nullptr, 0, 0.f, 0, 0};
  WriteArgs a{(const uint16_t*)k_new, (const uint16_t*)v_new, (const uint16_t*)idx_new, block_table, seq_lens,
              (uint8_t*)k_pool, (uint8_t*)v_pool, (uint8_t*)idx_pool, num_pages, idx_pool_blocks,
              k_scale, v_scale, idx_scale, block_table_stride, decode_query_len, num_kv_heads, (int)T,
              ktf, itf};
  if (!with_idx) idx_dtype = ISB_BF16;  // no index vector: any instantiation will do
  hipStream_t st = as_hip(stream);
  if (kv_dtype == ISB_BF16) launch_write_kv<ISB_BF16>(a, idx_dtype, st);
  else if (kv_dtype == ISB_FP8_E4M3) launch_write_kv<ISB_FP8_E4M3>(a, idx_dtype, st);
  else launch_write_kv<ISB_MXFP4>(a, idx_dtype, st);
  return launch_status();
}

extern "C" int isb_quantize_e4m3(isb_stream_t stream, const void* x, int64_t n, void* out) {
  using namespace isb;
  if (!x || !out || n <= 0) return ISB_E_INVALID_ARG;
  if ((n + 1023) / 1024 > 0x7FFFFFFFLL) return ISB_E_SHAPE;
  hipLaunchKernelGGL(quantize_e4m3_kernel, dim3((unsigned)((n + 1023) / 1024)), dim3(256), 0, as_hip(stream),
                     (const uint16_t*)x, n, (uint8_t*)out);
  return launch_status();
}

extern "C" int isb_prepare_query(isb_stream_t stream, const void* q, int num_heads, const int32_t* seq_lens,
                                 int num_reqs, int decode_query_len, const isb_norm_rope* norm_rope,
                                 int out_dtype, void* out) {
  using namespace isb;
  if (!q || !seq_lens || !out || num_heads <= 0 || num_reqs <= 0 || decode_query_len <= 0)
    return ISB_E_INVALID_ARG;
  if (out_dtype != ISB_BF16 && out_dtype != ISB_FP8_E4M3) return ISB_E_UNSUPPORTED_DTYPE;
  const long long T = (long long)num_reqs * decode_query_len;
  if (T > 0x7FFFFFFFLL || num_heads > 65535 || T * num_heads > 4LL * 0x7FFFFFFFLL) return ISB_E_SHAPE;
  if (reinterpret_cast<uintptr_t>(q) % 4 || reinterpret_cast<uintptr_t>(out) % 4) return ISB_E_INVALID_ARG;
  QueryArgs a{(const uint16_t*)q, seq_lens, (uint8_t*)out, {}, num_heads, decode_query_len, (int)T};
  const int e = read_norm_rope(norm_rope, a.tf);
  if (e) return e;
  const dim3 grid((unsigned)((T * num_heads + 3) / 4));
  if (out_dtype == ISB_BF16)
    hipLaunchKernelGGL(prepare_query_kernel<2>, grid, dim3(256), 0, as_hip(stream), a);
  else
    hipLaunchKernelGGL(prepare_query_kernel<1>, grid, dim3(256), 0, as_hip(stream), a);
  return launch_status();
}
