// Cached-prefix expansion of the paged latent cache into per-head K and V.
//
// "perf(mla): chunk the non-FP4 gather_kv_b_proj over KV" (description): the
// whole cached context is expanded once per layer, one program per (batch,
// head, KV chunk), a program past its sequence's last chunk exiting at once.
// Here a program is one workgroup of 4 waves that computes, for 128 cached rows
// of one sequence and one head h, the 256 projections W[h] . c (128 K-nope then
// 128 V) on bf16 MFMA (16x16x32), and copies the 64 rope values beside K.
//
//   * The latent (512 wide) streams through LDS in 8 stages of 64 columns,
//     together with the matching 256 x 64 slice of W[h]: global -> registers
//     (the next stage is loaded while the current one is multiplied) ->
//     LDS. An fp8 cache is widened to bf16 on the way (exactly: every e4m3fn
//     value is a bf16 value); kv_scale multiplies the float32 result.
//   * Wave w owns output rows 128 (w & 1) .. +127 of W[h] (so K or V) for the
//     cached rows 64 (w >> 1) .. +63 of the chunk: 8 x 4 accumulator tiles,
//     turned into whole output rows in LDS before they are stored.
//   * Program ids are spread so that each XCD walks a contiguous run of them in
//     (sequence, chunk, head) order: the heads of one chunk run back to back on
//     one XCD and share its L2 copy of the latent rows.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2_t;

#define KVB_LDS(T) __attribute__((address_space(3))) T*

constexpr int kChunkRows = 128;                      // cached rows per program
constexpr int kWRows = 256;                          // rows of W[h]: K nope, then V
constexpr int kNope = 128, kVDim = 128, kRope = 64;  // K is 192 wide: nope then rope
constexpr int kStageCols = 64;                       // latent columns per stage
constexpr int kStages = kLatentDim / kStageCols;     // 8
constexpr int kRowBytes = kStageCols * 2;            // bf16 bytes of one row in a stage
constexpr int kWLdsBytes = kWRows * kRowBytes;       // 32 KB
constexpr int kLatLdsBytes = kChunkRows * kRowBytes; // 16 KB
constexpr int kXcds = 8;
// Epilogue: each wave turns its 128 x 64 tile into bf16 rows of 256 bytes in LDS
// (one row per cached row, 16 bytes of padding against bank conflicts), then
// stores them 16 bytes per lane, 16 lanes per output row.
constexpr int kEpRowBytes = kNope * 2 + 16;
constexpr int kEpWaveBytes = 64 * kEpRowBytes;
constexpr int kLdsBytes = (kWLdsBytes + kLatLdsBytes) > 4 * kEpWaveBytes ? (kWLdsBytes + kLatLdsBytes) : 4 * kEpWaveBytes;

struct KvbArgs {
  const uint8_t* cache;
  const int32_t* kv_indptr;
  const int32_t* kv_page_indices;
  const int32_t* cu_ctx;
  const uint16_t* w;  // bf16 [H, 256, 512]
  uint16_t* k_out;    // bf16 [rows, H, 192]
  uint16_t* v_out;    // bf16 [rows, H, 128]
  uint32_t* status;
  int64_t num_slots;
  int64_t num_out_rows;
  int64_t programs;   // batch * chunks * heads
  int32_t num_heads, page_size, chunks, max_ctx;
  float kv_scale;
};

// Byte offset of 16-byte chunk c (0..7) of LDS row r. The XOR keeps 8 and 16
// consecutive rows read at one chunk on distinct 16-byte bank groups.
__device__ __forceinline__ uint32_t swz(int r, int c) {
  return (uint32_t)(r * kRowBytes + ((c ^ ((r & 7) ^ ((r >> 3) & 1))) << 4));
}

template <bool HI>
__device__ __forceinline__ unsigned fp8x2_bf16x2(unsigned w) {
  bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(unsigned, r);
}

__device__ __forceinline__ unsigned pack2(float a, float b) {
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(unsigned, r);
}

template <bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void mla_kv_b_proj_kernel(KvbArgs a) {
  // program id -> (sequence, chunk, head), XCD-contiguous
  const int64_t per_xcd = (int64_t)gridDim.x / kXcds;
  const int64_t pid = (int64_t)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (pid >= a.programs) return;
  const int h = (int)(pid % a.num_heads);
  const int64_t bc = pid / a.num_heads;
  const int chunk = (int)(bc % a.chunks);
  const int b = (int)(bc / a.chunks);
  const int row0 = a.cu_ctx[b];
  const int ctx = a.cu_ctx[b + 1] - row0;
  const int r0 = chunk * kChunkRows;
  if (row0 < 0 || ctx < 0 || (int64_t)row0 + ctx > a.num_out_rows) {  // rows outside the outputs: none written
    if (chunk == 0 && h == 0 && threadIdx.x == 0 && a.status) atomicOr(a.status, MLA_KVB_ROWS_OUT_OF_RANGE);
    return;
  }
  if (chunk == 0 && h == 0 && threadIdx.x == 0 && ctx > a.max_ctx && a.status)
    atomicOr(a.status, MLA_KVB_CTX_TOO_LONG);  // rows past max_context_len are not written
  const int lim = min(ctx, a.max_ctx);         // rows of this sequence that are expanded
  if (r0 >= lim) return;                       // past this sequence's last chunk
  const int nrows = min(kChunkRows, lim - r0);

  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  KVB_LDS(uint8_t) w_lds = (KVB_LDS(uint8_t))lds;
  KVB_LDS(uint8_t) l_lds = w_lds + kWLdsBytes;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g = lane >> 4;
  const int nh = wave & 1, th = wave >> 1;

  // the cached rows this thread stages: fp8 rows (tid >> 2) + 64 i, bf16 rows (tid >> 3) + 32 i
  constexpr int kMyRows = FP8 ? 2 : 4;
  constexpr int kRowStep = FP8 ? 64 : 32;
  const int my_row0 = FP8 ? (tid >> 2) : (tid >> 3);
  const int my_c = FP8 ? (tid & 3) : (tid & 7);  // 16-byte piece of the row's stage slice
  constexpr int kElem = FP8 ? 1 : 2;
  const uint8_t* src[kMyRows];
  uint32_t bad = 0;
  const int pg_first = max(a.kv_indptr[b], 0), pg_end = a.kv_indptr[b + 1];
#pragma unroll
  for (int i = 0; i < kMyRows; ++i) {
    const int r = r0 + my_row0 + kRowStep * i;
    src[i] = nullptr;
    if (r < lim) {
      const int q = r / a.page_size;
      if (pg_first + q >= pg_end) {
        bad |= MLA_KVB_TOO_FEW_PAGES;
      } else {
        const int64_t slot = (int64_t)a.kv_page_indices[pg_first + q] * a.page_size + (r - q * a.page_size);
        if (slot < 0 || slot >= a.num_slots) bad |= MLA_KVB_SLOT_OUT_OF_RANGE;
        else src[i] = a.cache + slot * (kRowDim * kElem) + my_c * 16;
      }
    }
  }
  if (bad && a.status) atomicOr(a.status, bad);

  // W[h] slice this thread stages: rows (tid >> 3) + 32 i, 16-byte piece tid & 7
  const uint16_t* wsrc = a.w + ((int64_t)h * kWRows + (tid >> 3)) * kLatentDim + (tid & 7) * 8;

  u32x4_t wreg[8];
  u32x4_t lreg[kMyRows];
  auto load_stage = [&](int s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) wreg[i] = *(const u32x4_t*)(wsrc + (int64_t)i * 32 * kLatentDim + s * kStageCols);
#pragma unroll
    for (int i = 0; i < kMyRows; ++i)
      lreg[i] = src[i] ? *(const u32x4_t*)(src[i] + s * kStageCols * kElem) : u32x4_t{0, 0, 0, 0};
  };
  auto store_stage = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) *(KVB_LDS(u32x4_t))(w_lds + swz((tid >> 3) + 32 * i, tid & 7)) = wreg[i];
#pragma unroll
    for (int i = 0; i < kMyRows; ++i) {
      const int r = my_row0 + kRowStep * i;
      if constexpr (FP8) {  // 16 fp8 -> two 16-byte bf16 pieces 2c, 2c+1
        const u32x4_t v = lreg[i];
        const u32x4_t lo = {fp8x2_bf16x2<false>(v[0]), fp8x2_bf16x2<true>(v[0]), fp8x2_bf16x2<false>(v[1]),
                            fp8x2_bf16x2<true>(v[1])};
        const u32x4_t hi = {fp8x2_bf16x2<false>(v[2]), fp8x2_bf16x2<true>(v[2]), fp8x2_bf16x2<false>(v[3]),
                            fp8x2_bf16x2<true>(v[3])};
        *(KVB_LDS(u32x4_t))(l_lds + swz(r, 2 * my_c)) = lo;
        *(KVB_LDS(u32x4_t))(l_lds + swz(r, 2 * my_c + 1)) = hi;
      } else {
        *(KVB_LDS(u32x4_t))(l_lds + swz(r, my_c)) = lreg[i];
      }
    }
  };

  f32x4_t acc[8][4];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[nb][tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  load_stage(0);
  for (int s = 0; s < kStages; ++s) {
    __syncthreads();  // every wave is done reading the previous stage
    store_stage();
    __syncthreads();
    if (s + 1 < kStages) load_stage(s + 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = 4 * ks + g;  // this lane's 8 columns of the 32-column MFMA slab
      bf16x8_t bt[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        bt[tb] = *(KVB_LDS(bf16x8_t))(l_lds + swz(th * 64 + tb * 16 + l16, c));
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const bf16x8_t at = *(KVB_LDS(bf16x8_t))(w_lds + swz(nh * 128 + nb * 16 + l16, c));
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[nb][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(at, bt[tb], acc[nb][tb], 0, 0, 0);
      }
    }
  }

  // acc[nb][tb][i]: W row nh*128 + nb*16 + 4g + i, cached row th*64 + tb*16 + l16
  const int H = a.num_heads;
  __syncthreads();  // every wave is done with the last stage: LDS becomes the epilogue buffer
  KVB_LDS(uint8_t) ep = (KVB_LDS(uint8_t))lds + wave * kEpWaveBytes;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const f32x4_t v = acc[nb][tb];
      *(KVB_LDS(u32x2_t))(ep + (tb * 16 + l16) * kEpRowBytes + (nb * 16 + 4 * g) * 2) =
          u32x2_t{pack2(v[0] * a.kv_scale, v[1] * a.kv_scale), pack2(v[2] * a.kv_scale, v[3] * a.kv_scale)};
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int tr = i * 4 + (lane >> 4), piece = lane & 15;  // wave-local row, 16-byte piece of its 256 bytes
    const int t = th * 64 + tr;
    if (t >= nrows) continue;
    const u32x4_t o = *(KVB_LDS(u32x4_t))(ep + tr * kEpRowBytes + piece * 16);
    const int64_t orow = (int64_t)row0 + r0 + t;
    uint16_t* dst = nh == 0 ? a.k_out + (orow * H + h) * (kNope + kRope) : a.v_out + (orow * H + h) * kVDim;
    *(u32x4_t*)(dst + piece * 8) = o;
  }

  // rope part of K: 128 rows x 8 pieces of 8 values, 4 per thread
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + 256 * i;
    const int t = id >> 3, piece = id & 7;
    if (t >= nrows) continue;
    const int r = r0 + t;
    const int q = r / a.page_size;
    const int64_t slot = pg_first + q < pg_end
                             ? (int64_t)a.kv_page_indices[pg_first + q] * a.page_size + (r - q * a.page_size)
                             : -1;  // no page: the row reads as zeros, like its K-nope and V
    u32x4_t o = {0, 0, 0, 0};
    if (slot >= 0 && slot < a.num_slots) {
      const uint8_t* p = a.cache + slot * (kRowDim * kElem) + (kLatentDim + piece * 8) * kElem;
      if constexpr (FP8) {
        const u32x2_t raw = *(const u32x2_t*)p;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const unsigned lo = fp8x2_bf16x2<false>(raw[j]), hi = fp8x2_bf16x2<true>(raw[j]);
          o[2 * j] = pack2(__uint_as_float(lo << 16) * a.kv_scale, __uint_as_float(lo & 0xffff0000u) * a.kv_scale);
          o[2 * j + 1] = pack2(__uint_as_float(hi << 16) * a.kv_scale, __uint_as_float(hi & 0xffff0000u) * a.kv_scale);
        }
      } else {
        o = *(const u32x4_t*)p;
      }
    }
    *(u32x4_t*)(a.k_out + (((int64_t)row0 + r) * H + h) * (kNope + kRope) + kNope + piece * 8) = o;
  }
}

}  // namespace
}  // namespace mla

extern "C" mla_status_t mla_gather_kv_b_proj(const mla_kv_b_proj_params_t* p, const void* d_kv_cache,
                                             const int32_t* d_kv_indptr, const int32_t* d_kv_page_indices,
                                             const int32_t* d_cu_ctx, const void* d_w_kv_b, void* d_k_out,
                                             void* d_v_out, uint32_t* d_status, void* stream) {
  if (!p) return MLA_ERR_INVALID_ARG;
  if (p->batch < 0 || p->num_heads < 1 || p->page_size < 1 || p->max_context_len < 0 || p->num_slots < 1 ||
      p->num_out_rows < 0)
    return MLA_ERR_INVALID_ARG;
  if (p->kv_dtype != MLA_KV_BF16 && p->kv_dtype != MLA_KV_FP8_E4M3FN) return MLA_ERR_INVALID_ARG;
  if (!(p->kv_scale > 0.0f) || !(p->kv_scale < 3.0e38f)) return MLA_ERR_INVALID_ARG;
  if (p->kv_dtype == MLA_KV_BF16 && p->kv_scale != 1.0f) return MLA_ERR_INVALID_ARG;
  if (p->batch == 0 || p->max_context_len == 0) return MLA_OK;
  if (!d_kv_cache || !d_kv_indptr || !d_kv_page_indices || !d_cu_ctx || !d_w_kv_b || !d_k_out || !d_v_out)
    return MLA_ERR_INVALID_ARG;
  const int64_t chunks = (p->max_context_len + mla::kChunkRows - 1) / mla::kChunkRows;
  const int64_t programs = (int64_t)p->batch * chunks * p->num_heads;
  const int64_t grid = (programs + mla::kXcds - 1) / mla::kXcds * mla::kXcds;
  if (grid > 0x7fffffff) return MLA_ERR_UNSUPPORTED;
  mla::KvbArgs a;
  a.cache = static_cast<const uint8_t*>(d_kv_cache);
  a.kv_indptr = d_kv_indptr;
  a.kv_page_indices = d_kv_page_indices;
  a.cu_ctx = d_cu_ctx;
  a.w = static_cast<const uint16_t*>(d_w_kv_b);
  a.k_out = static_cast<uint16_t*>(d_k_out);
  a.v_out = static_cast<uint16_t*>(d_v_out);
  a.status = d_status;
  a.num_slots = p->num_slots;
  a.num_out_rows = p->num_out_rows;
  a.programs = programs;
  a.num_heads = p->num_heads;
  a.page_size = p->page_size;
  a.chunks = (int32_t)chunks;
  a.max_ctx = p->max_context_len;
  a.kv_scale = p->kv_scale;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 g((unsigned)grid), blk(256);
  if (p->kv_dtype == MLA_KV_FP8_E4M3FN) hipLaunchKernelGGL(mla::mla_kv_b_proj_kernel<true>, g, blk, 0, st, a);
  else hipLaunchKernelGGL(mla::mla_kv_b_proj_kernel<false>, g, blk, 0, st, a);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}
