// Decode epilogue ahead of the attention: query concat and latent-cache insert.
//
// "[Perf][Kimi-K3] Cut MLA decode concat/cache epilogue latency" (Purpose):
// one fused kernel joins the absorbed query parts into the 576-wide query and
// writes each new token's latent row (latent | rope(k_pe)) into the cache at
// its slot; its rows are (token, head + 1). Here every lane moves one 16-byte
// chunk (8 elements) of a 576-wide row, 72 lanes per row, so each lane does
// exactly one load, conversion and store whatever the token count.
#include <hip/hip_runtime.h>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(short)))) short i16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

constexpr int kChunksPerRow = kRowDim / 8;     // 72
constexpr int kLatentChunks = kLatentDim / 8;  // 64

struct InsertArgs {
  const uint16_t* ql_nope;  // [T, H, 512]
  const uint16_t* q_pe;     // [T, H, 64]
  const uint16_t* kv_c;     // [T, 512]
  const uint16_t* k_pe;     // [T, 64]
  const int32_t* positions; // [T]
  const float* cos_sin;     // [rope_positions, 64]: cos of the 32 pairs, then sin
  const int64_t* slot_mapping;
  uint16_t* q;              // [T, H, 576]
  uint8_t* cache;           // [num_slots, 576] of 2 (bf16) or 1 (fp8) bytes
  uint32_t* status;         // nullable
  int64_t num_slots;
  int32_t num_tokens, num_heads, rope_positions;
  float kv_scale;
};

__device__ __forceinline__ float lo_bf16(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// e4m3fn of v: nearest even (the converter's rounding), saturated to +-448, NaN -> 0x7f.
__device__ __forceinline__ float fp8_ready(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

template <bool FP8, bool NEOX>
__global__ __launch_bounds__(256) void mla_insert_kernel(InsertArgs a) {
#pragma clang fp contract(off)
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / kChunksPerRow;
  const int chunk = (int)(idx - row * kChunksPerRow);
  const int rows_per_token = a.num_heads + 1;
  if (row >= (int64_t)a.num_tokens * rows_per_token) return;
  const int t = (int)(row / rows_per_token);
  const int h = (int)(row - (int64_t)t * rows_per_token);

  if (h < a.num_heads) {  // query row: ql_nope (64 chunks) then q_pe (8 chunks), bit copy
    const int64_t qrow = (int64_t)t * a.num_heads + h;
    const u32x4_t v = chunk < kLatentChunks
                          ? *(const u32x4_t*)(a.ql_nope + qrow * kLatentDim + 8 * chunk)
                          : *(const u32x4_t*)(a.q_pe + qrow * (kRowDim - kLatentDim) + 8 * (chunk - kLatentChunks));
    *(u32x4_t*)(a.q + qrow * kRowDim + 8 * chunk) = v;
    return;
  }

  // cache row of token t
  const int64_t slot = a.slot_mapping[t];
  if (slot < 0) return;  // padding token
  if (slot >= a.num_slots) {
    if (chunk == 0 && a.status) atomicOr(a.status, MLA_INSERT_SLOT_OUT_OF_RANGE);
    return;
  }
  const int pos = a.positions[t];
  if (pos < 0 || pos >= a.rope_positions) {
    if (chunk == 0 && a.status) atomicOr(a.status, MLA_INSERT_POSITION_OUT_OF_RANGE);
    return;
  }
  const int64_t elem0 = slot * kRowDim + 8 * chunk;  // first element of this lane's 8 in the cache
  float x[8];
  if (chunk < kLatentChunks) {
    const u32x4_t v = *(const u32x4_t*)(a.kv_c + (int64_t)t * kLatentDim + 8 * chunk);
    if constexpr (!FP8) {
      *(u32x4_t*)((uint16_t*)a.cache + elem0) = v;
      return;
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x[2 * w] = lo_bf16(v[w]);
      x[2 * w + 1] = hi_bf16(v[w]);
    }
  } else {
    // rope: output elements 8k .. 8k+7 of the 64; x' = x c - y s, y' = y c + x s with
    // rounded float32 products and sums (no contraction in this function)
    const int k = chunk - kLatentChunks;
    const uint16_t* kp = a.k_pe + (int64_t)t * (kRowDim - kLatentDim);
    const float* cs = a.cos_sin + (int64_t)pos * 64;
    if constexpr (!NEOX) {  // pairs (2i, 2i+1), i = 4k .. 4k+3
      const u32x4_t v = *(const u32x4_t*)(kp + 8 * k);
      const f32x4_t c = *(const f32x4_t*)(cs + 4 * k);
      const f32x4_t s = *(const f32x4_t*)(cs + 32 + 4 * k);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float xe = lo_bf16(v[j]), xo = hi_bf16(v[j]);
        const float p0 = xe * c[j], p1 = xo * s[j], p2 = xo * c[j], p3 = xe * s[j];
        x[2 * j] = p0 - p1;
        x[2 * j + 1] = p2 + p3;
      }
    } else {  // halves (i, i + 32): this lane's 8 outputs are pairs i0 .. i0+7 of one half
      const int i0 = (k & 3) * 8;
      const u32x4_t vf = *(const u32x4_t*)(kp + i0);
      const u32x4_t vs = *(const u32x4_t*)(kp + 32 + i0);
      const f32x4_t c0 = *(const f32x4_t*)(cs + i0), c1 = *(const f32x4_t*)(cs + i0 + 4);
      const f32x4_t s0 = *(const f32x4_t*)(cs + 32 + i0), s1 = *(const f32x4_t*)(cs + 32 + i0 + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float first = (e & 1) ? hi_bf16(vf[e >> 1]) : lo_bf16(vf[e >> 1]);
        const float second = (e & 1) ? hi_bf16(vs[e >> 1]) : lo_bf16(vs[e >> 1]);
        const float c = e < 4 ? c0[e] : c1[e - 4], s = e < 4 ? s0[e] : s1[e - 4];
        if (k < 4) {
          const float p0 = first * c, p1 = second * s;
          x[e] = p0 - p1;
        } else {
          const float p2 = second * c, p3 = first * s;
          x[e] = p2 + p3;
        }
      }
    }
  }

  if constexpr (FP8) {
    unsigned w[2];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = x[4 * d + e] / a.kv_scale;
      i16x2_t p = i16x2_t{0, 0};
      p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, fp8_ready(v[0]), fp8_ready(v[1]), 1.0f, false);
      p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, fp8_ready(v[2]), fp8_ready(v[3]), 1.0f, true);
      unsigned bytes = __builtin_bit_cast(unsigned, p);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (v[e] != v[e]) bytes = (bytes & ~(0xffu << (8 * e))) | (0x7fu << (8 * e));
      w[d] = bytes;
    }
    *(u32x2_t*)(a.cache + elem0) = u32x2_t{w[0], w[1]};
  } else {
    u32x4_t o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x2_t p;
      p[0] = (__bf16)x[2 * j];
      p[1] = (__bf16)x[2 * j + 1];
      o[j] = __builtin_bit_cast(unsigned, p);
    }
    *(u32x4_t*)((uint16_t*)a.cache + elem0) = o;
  }
}

}  // namespace
}  // namespace mla

extern "C" mla_status_t mla_qcat_cache_insert(const mla_insert_params_t* p, const void* d_ql_nope,
                                              const void* d_q_pe, const void* d_kv_c, const void* d_k_pe,
                                              const int32_t* d_positions, const float* d_cos_sin,
                                              const int64_t* d_slot_mapping, void* d_q, void* d_cache,
                                              uint32_t* d_status, void* stream) {
  if (!p) return MLA_ERR_INVALID_ARG;
  if (p->num_tokens < 0 || p->num_heads < 1 || p->num_slots < 1 || p->rope_positions < 1) return MLA_ERR_INVALID_ARG;
  if (p->rope_neox != 0 && p->rope_neox != 1) return MLA_ERR_INVALID_ARG;
  if (p->kv_dtype != MLA_KV_BF16 && p->kv_dtype != MLA_KV_FP8_E4M3FN) return MLA_ERR_INVALID_ARG;
  if (!(p->kv_scale > 0.0f) || !(p->kv_scale < 3.0e38f)) return MLA_ERR_INVALID_ARG;
  if (p->kv_dtype == MLA_KV_BF16 && p->kv_scale != 1.0f) return MLA_ERR_INVALID_ARG;
  if (p->num_tokens == 0) return MLA_OK;
  if (!d_ql_nope || !d_q_pe || !d_kv_c || !d_k_pe || !d_positions || !d_cos_sin || !d_slot_mapping || !d_q ||
      !d_cache)
    return MLA_ERR_INVALID_ARG;
  const int64_t threads = int64_t(p->num_tokens) * (int64_t(p->num_heads) + 1) * mla::kChunksPerRow;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffff) return MLA_ERR_UNSUPPORTED;
  mla::InsertArgs a;
  a.ql_nope = static_cast<const uint16_t*>(d_ql_nope);
  a.q_pe = static_cast<const uint16_t*>(d_q_pe);
  a.kv_c = static_cast<const uint16_t*>(d_kv_c);
  a.k_pe = static_cast<const uint16_t*>(d_k_pe);
  a.positions = d_positions;
  a.cos_sin = d_cos_sin;
  a.slot_mapping = d_slot_mapping;
  a.q = static_cast<uint16_t*>(d_q);
  a.cache = static_cast<uint8_t*>(d_cache);
  a.status = d_status;
  a.num_slots = p->num_slots;
  a.num_tokens = p->num_tokens;
  a.num_heads = p->num_heads;
  a.rope_positions = p->rope_positions;
  a.kv_scale = p->kv_scale;
  const dim3 grid((unsigned)blocks), block(256);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool fp8 = p->kv_dtype == MLA_KV_FP8_E4M3FN;
  if (fp8) {
    if (p->rope_neox) hipLaunchKernelGGL((mla::mla_insert_kernel<true, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((mla::mla_insert_kernel<true, false>), grid, block, 0, st, a);
  } else {
    if (p->rope_neox) hipLaunchKernelGGL((mla::mla_insert_kernel<false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((mla::mla_insert_kernel<false, false>), grid, block, 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}
