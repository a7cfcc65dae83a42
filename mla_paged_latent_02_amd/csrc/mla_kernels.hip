// CDNA4 (gfx950) kernels for MLA decode over a paged latent KV cache:
//   mla_plan_kernel    per-sequence chunk counts, partial-record bases, status word
//   mla_decode_kernel  page-gathered HBM->LDS loads, fp8->bf16 in registers,
//                      S^T = K Q^T and O^T = V^T P^T on MFMA, online softmax
//   mla_combine_kernel log-sum-exp merge of split-KV partials
//
// The decode design follows what the pages say about where the time goes and
// what holds on MI355X, redone for gfx950:
//  - "perf(mla): chunk the non-FP4 gather_kv_b_proj over KV" (description): the
//    KV walk is a grid axis of chunks with an early exit past a sequence's end,
//    so the grid fills the 256 CUs instead of 12 workgroups starving HBM.
//  - "HK MLA: MI35x m16x8 retune, new m16x4 kernel, page_size + mask support"
//    (Summary): heads (x draft tokens) stacked as MFMA rows, 64-row KV blocks,
//    transposed LDS reads (ds_read_tr) for the KV operand, cross-lane
//    reductions with v_permlane16/32_swap, and a causal mask for MTP shapes.
// What differs: K and V are the same LDS rows, loaded once per workgroup by
// global_load_lds straight from the gathered cache rows; scores are computed
// transposed (S^T, kv rows as MFMA rows) so that softmax state, the P operand
// and the output accumulator all keep one head per lane column and need no
// data exchange; the fp8 cache is widened to bf16 exactly in registers.
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
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2_t;

#define LDS_PTR(T) __attribute__((address_space(3))) T*

constexpr float kLn2 = 0.6931471805599453f;
// Lazy rescaling: the running reference max of a row moves only when a new
// score exceeds it by more than this (base-2 units), so p <= 2^8 in bf16.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ float wave_max_16x4(float v) {
  // max over the 4 lanes {l, l^16, l^32, l^48} that hold the same head row
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float wave_sum_16x4(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Two fp8 e4m3fn bytes (the low or high 16 bits of w) to two bf16, exactly
// (every e4m3fn value, subnormals included, is a bf16 value).
template <bool HI>
__device__ __forceinline__ unsigned fp8x2_to_bf16x2(unsigned w) {
  bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(unsigned, r);
}

__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(unsigned lo, unsigned hi) {
  u32x4_t r;
  r[0] = fp8x2_to_bf16x2<false>(lo);
  r[1] = fp8x2_to_bf16x2<true>(lo);
  r[2] = fp8x2_to_bf16x2<false>(hi);
  r[3] = fp8x2_to_bf16x2<true>(hi);
  return __builtin_bit_cast(bf16x8_t, r);
}

__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(unsigned, r);
}

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Planner: one workgroup walks the batch in tiles of 256 sequences.
__global__ __launch_bounds__(256) void mla_plan_kernel(PlanArgs a) {
  __shared__ int32_t scan[256];
  __shared__ uint32_t bad_or[256];
  const int tid = threadIdx.x;
  int32_t carry = 0;
  uint32_t bad_acc = 0;
  for (int base = 0; base < a.batch; base += 256) {
    const int b = base + tid;
    int32_t n = 0, contrib = 0;
    if (b < a.batch) {
      const int32_t ctx = a.context_lens[b];
      const int32_t pages = a.kv_indptr[b + 1] - a.kv_indptr[b];
      uint32_t bad = 0;
      if (ctx < a.seqlen_qo) bad |= MLA_DEV_CTX_TOO_SHORT;
      if (ctx > a.max_context_len) bad |= MLA_DEV_CTX_TOO_LONG;
      if (!bad && (int64_t)pages * a.page_size < (int64_t)ctx) bad |= MLA_DEV_TOO_FEW_PAGES;
      bad_acc |= bad;
      n = bad ? 0 : (ctx + a.chunk_len - 1) / a.chunk_len;
      contrib = (n > 1 ? n : 0) * a.num_groups;
    }
    scan[tid] = contrib;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {  // inclusive Hillis-Steele scan
      int32_t v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    if (b < a.batch) {
      a.nchunks[b] = n;
      a.partbase[b] = carry + scan[tid] - contrib;
    }
    carry += scan[255];
    __syncthreads();
  }
  bad_or[tid] = bad_acc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) bad_or[tid] |= bad_or[tid + off];
    __syncthreads();
  }
  if (tid == 0) {
    a.status[0] = bad_or[0];
    a.status[1] = 0;
    a.status[2] = 0;
    a.status[3] = 0;
  }
}

// ---------------------------------------------------------------------------
// Decode. One workgroup = one (chunk, head group, sequence). NW waves; wave w
// owns tile rows [w*HT*16, (w+1)*HT*16) and all 64 cache rows of each block.
//
// LDS block layout (one pipeline stage, 64 cache rows):
//   main region: row r at r*kMainStride holds the 512 latent elements (the V
//                part); the stride is padded by 16 bytes so that consecutive
//                rows start on different banks;
//   tail region: row r at kTailBase + r*kTailBytes holds the 64 rope elements
//                (16-byte slots, physical slot p holds logical slot
//                p ^ (r % kTailSlots)).
// Row permutation: the 16 MFMA rows of a K tile read LDS rows pi(m) =
// (m >> 2) + 4 (m & 3), so score row 4g + r of a tile is cache row g + 4r and
// the four rows that one 16-lane group reads in a transposed V access are 4
// rows apart (distinct banks).
template <bool FP8>
struct RowLayout {
  static constexpr int kElem = FP8 ? 1 : 2;
  static constexpr int kRowBytes = kRowDim * kElem;      // 576 or 1152 in the cache
  static constexpr int kMainBytes = kLatentDim * kElem;  // 512 or 1024
  static constexpr int kMainStride = kMainBytes + 16;
  static constexpr int kTailBytes = 64 * kElem;          // 64 or 128
  static constexpr int kTailSlots = kTailBytes / 16;     // 4 or 8
  static constexpr int kTailBase = kBlockRows * kMainStride;
  static constexpr int kBlockBytes = kTailBase + kBlockRows * kTailBytes;
};

template <bool FP8, int NW>
struct DecodeCfg {
  using L = RowLayout<FP8>;
  static constexpr int kStages = 2;
  static constexpr int kLdsBytes = kStages * L::kBlockBytes;
  static constexpr int kRowsPerWave = kBlockRows / NW;  // rows each wave loads
  static constexpr int kTailRowsPerInst = 64 / L::kTailSlots;
  static constexpr int kTailInsts = (kRowsPerWave + kTailRowsPerInst - 1) / kTailRowsPerInst;
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ u32x4_t lds_b128(LDS_PTR(uint8_t) base, uint32_t off) {
  return *(LDS_PTR(u32x4_t))(base + off);
}

// 16 bytes per lane from global memory straight into LDS at lds_addr + 16*lane
// (global_load_lds_dwordx4; M0 holds the wave's LDS base). Written as inline
// asm so that the compiler does not guard every later LDS read with a wait
// for it: completion is awaited explicitly with s_waitcnt vmcnt(0) before the
// workgroup barrier that publishes a stage.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_addr) : "memory");
}

// One wave = one 16-row head tile: its query rows (72 registers of bf16
// fragments) and its 16 x 512 fp32 output (128 registers) stay in registers
// for the whole chunk, which leaves room for two waves per SIMD. NW waves
// share each 64-row KV block in LDS.
template <bool FP8, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mla_decode_kernel(DecodeArgs a) {
  using Cfg = DecodeCfg<FP8, NW>;
  using L = RowLayout<FP8>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::kLdsBytes];
  LDS_PTR(uint8_t) lds = (LDS_PTR(uint8_t))smem;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  const int chunk = blockIdx.x;
  const int grp = blockIdx.y;
  const int b = blockIdx.z;
  const int n_b = a.nchunks[b];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i16 = lane & 15;  // MFMA column: head row within the wave's 16-row tile
  const int g4 = lane >> 4;   // MFMA k-group

  if (chunk >= n_b) {
    // Early-exit guard. An invalid sequence (n_b == 0) gets NaN rows from chunk 0.
    if (n_b == 0 && chunk == 0) {
      const float nan = __builtin_nanf("");
      for (int rr = wave; rr < a.rows_per_group; rr += NW) {
        const int s = rr / a.heads_per_group;
        const int head = grp * a.heads_per_group + rr % a.heads_per_group;
        if (head >= a.num_heads) continue;
        const int64_t row = ((int64_t)b * a.seqlen_qo + s) * a.num_heads + head;
        for (int c = lane; c < kLatentDim; c += 64) a.out[row * kLatentDim + c] = 0x7fc0;
        if (a.lse && lane == 0) a.lse[row] = nan;
      }
    }
    return;
  }

  const int ctx = a.context_lens[b];
  const int c_start = chunk * a.chunk_len;
  const int c_end = min(c_start + a.chunk_len, ctx);
  const int nblk = (c_end - c_start + kBlockRows - 1) / kBlockRows;
  const int64_t page_base = a.kv_indptr[b];
  const int P = a.page_size;

  // ---- this lane's tile row and its visible limit
  const int rr = wave * 16 + i16;
  const int tok = rr / a.heads_per_group;
  const int head = grp * a.heads_per_group + rr % a.heads_per_group;
  const bool row_ok = rr < a.rows_per_group && head < a.num_heads;
  const int vis_end = min(c_end, a.causal ? ctx - a.seqlen_qo + 1 + tok : ctx);
  const int row_out = row_ok ? (int)(((int64_t)b * a.seqlen_qo + tok) * a.num_heads + head) : 0;

  // ---- query fragments (B operand of S^T = K Q^T), resident for the whole chunk.
  // bf16 cache: fragment t holds d = 32t + 8*g4 .. +7.
  // fp8 cache:  fragment 2p+h holds d = 64p + 16*g4 + 8h .. +7 (one 16-byte LDS read of 16 fp8).
  bf16x8_t qf[18];
  {
    const uint16_t* qrow = a.q + (int64_t)row_out * kRowDim;
#pragma unroll
    for (int t = 0; t < 18; ++t) {
      const int d = FP8 ? (64 * (t >> 1) + 16 * g4 + 8 * (t & 1)) : (32 * t + 8 * g4);
      u32x4_t v = *(const u32x4_t*)(qrow + d);
      if (!row_ok) v = u32x4_t{0, 0, 0, 0};
      qf[t] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // ---- softmax state and output accumulators (O^T tiles: 16 latent cols x 16 heads)
  float m_ref = -__builtin_inff(), l_part = 0.0f;
  f32x4_t o_acc[32];
#pragma unroll
  for (int nt = 0; nt < 32; ++nt) o_acc[nt] = f32x4_t{0, 0, 0, 0};

  // ---- page-gathered block loads. global_load_lds puts lane i of an
  // instruction at LDS base + 16*i; the lane picks which 16-byte piece of
  // which gathered row it fetches.
  const uint8_t* cache = a.cache;
  constexpr int RPW = Cfg::kRowsPerWave;
  // Page ids are fetched one block ahead of their use, so that reading them
  // never waits on the cache rows in flight; validation happens at use.
  auto row_kv = [&](int blk) -> int {  // cache row of this lane (lanes < RPW) in block blk
    const int kv = c_start + blk * kBlockRows + wave * RPW + lane;
    return min(kv, c_end - 1);  // rows past the chunk repeat its last row; they are masked
  };
  auto fetch_page = [&](int blk) -> int { return a.kv_page_indices[page_base + row_kv(blk) / P]; };
  auto page_slot = [&](int blk, int page) -> int {
    if ((uint64_t)(int64_t)page >= (uint64_t)a.num_pages) {
      atomicOr(a.status, MLA_DEV_PAGE_OUT_OF_RANGE);
      page = 0;
    }
    return page * P + row_kv(blk) % P;
  };
  auto issue_block = [&](int blk, int slot_reg) {
    const uint32_t stage_off = (uint32_t)(blk & 1) * L::kBlockBytes;
    const int r_base = wave * RPW;
    // main: one instruction per row; lane l fetches the row's 16-byte slot l
    // (bf16: 64 slots; fp8: 32 slots, upper half of the wave idle)
#pragma unroll
    for (int rl = 0; rl < RPW; ++rl) {
      const int slot = __builtin_amdgcn_readlane(slot_reg, rl);
      const uint8_t* src = cache + (int64_t)slot * L::kRowBytes + (lane << 4);
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_base + stage_off + (uint32_t)((r_base + rl) * L::kMainStride));
      if (FP8 ? lane < 32 : true) dma16(src, dst);
    }
    // tail: kTailRowsPerInst rows x kTailSlots slots per instruction
    const int tslot = lane % L::kTailSlots;
    const int trow = lane / L::kTailSlots;
    const int logical = tslot ^ (trow % L::kTailSlots);  // r % kTailSlots == trow % kTailSlots
#pragma unroll
    for (int m = 0; m < Cfg::kTailInsts; ++m) {
      const int rl = m * Cfg::kTailRowsPerInst + trow;
      const int slot = __shfl(slot_reg, rl & 63);
      const uint8_t* src = cache + (int64_t)slot * L::kRowBytes + L::kMainBytes + (logical << 4);
      const uint32_t dst = __builtin_amdgcn_readfirstlane(
          lds_base + stage_off + (uint32_t)(L::kTailBase + (r_base + m * Cfg::kTailRowsPerInst) * L::kTailBytes));
      if (rl < RPW) dma16(src, dst);
    }
  };

  // Per-lane LDS offsets that do not change over the loop; each access adds a
  // compile-time immediate.
  const int pi16 = (i16 >> 2) + 4 * (i16 & 3);  // LDS row read by MFMA row i16 of a K tile
  const uint32_t k_main_base = (uint32_t)pi16 * L::kMainStride + (uint32_t)g4 * 16;
  const uint32_t k_tail_row = L::kTailBase + (uint32_t)pi16 * L::kTailBytes;
  uint32_t v_base;
  if constexpr (FP8) {
    // supplier lane (k = i16/2, c = i16%2): row g4 + 4(k&3) + 16(k>>2), bytes 8c of the column tile
    const int k = i16 >> 1, c = i16 & 1;
    v_base = (uint32_t)(g4 + 4 * (k & 3) + 16 * (k >> 2)) * L::kMainStride + 8u * c;
  } else {
    // supplier lane (k = i16/4, c = i16%4): row g4 + 4k (and +16), elements 4c of the column tile
    const int k = i16 >> 2, c = i16 & 3;
    v_base = (uint32_t)(g4 + 4 * k) * L::kMainStride + 8u * c;
  }

  int page_next = 0;
  if (lane < RPW) page_next = fetch_page(0);
  issue_block(0, lane < RPW ? page_slot(0, page_next) : 0);
  if (nblk > 1 && lane < RPW) page_next = fetch_page(1);

  const float sscale = a.score_scale_log2;

  for (int blk = 0; blk < nblk; ++blk) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (blk + 1 < nblk) {
      issue_block(blk + 1, lane < RPW ? page_slot(blk + 1, page_next) : 0);
      if (blk + 2 < nblk && lane < RPW) page_next = fetch_page(blk + 2);
    }
    LDS_PTR(uint8_t) stage = lds + (uint32_t)(blk & 1) * L::kBlockBytes;
    const int kv0 = c_start + blk * kBlockRows;

    // ---- S^T[kv, head] = K Q^T for the 64 rows of the block (4 tiles of 16 kv rows).
    // The reads walk (step, tile) with a ring of KD reads in flight; every
    // step ends in a scheduling barrier so the compiler cannot hoist the whole
    // block's reads (which would exhaust the registers).
    f32x4_t sacc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) sacc[nt] = f32x4_t{0, 0, 0, 0};
    {
      constexpr int kSteps = FP8 ? 9 : 18;
      constexpr int kMainSteps = FP8 ? 8 : 16;  // steps whose slots lie in the main region
      constexpr int kReads = kSteps * 4;
      constexpr int KD = 3;
      u32x4_t kb[KD];
      auto kread = [&](int i) -> u32x4_t {
        const int step = i >> 2, nt = i & 3;
        uint32_t off;
        if (step < kMainSteps) {
          off = k_main_base + (uint32_t)(nt * 16 * L::kMainStride + step * 64);
        } else {
          const int s2 = 4 * (step - kMainSteps) + g4;  // logical tail slot of this lane
          off = k_tail_row + (uint32_t)(nt * 16 * L::kTailBytes) +
                ((uint32_t)(s2 ^ (pi16 % L::kTailSlots)) << 4);
        }
        return lds_b128(stage, off);
      };
#pragma unroll
      for (int i = 0; i < KD - 1; ++i) kb[i] = kread(i);
#pragma unroll
      for (int i = 0; i < kReads; ++i) {
        if (i + KD - 1 < kReads) kb[(i + KD - 1) % KD] = kread(i + KD - 1);
        const u32x4_t raw = kb[i % KD];
        const int step = i >> 2, nt = i & 3;
        if constexpr (FP8) {
          // 16 fp8 = d in [64 step + 16 g4, +16): two k-steps of 8
          sacc[nt] = mfma16(fp8x8_to_bf16x8(raw[0], raw[1]), qf[2 * step], sacc[nt]);
          sacc[nt] = mfma16(fp8x8_to_bf16x8(raw[2], raw[3]), qf[2 * step + 1], sacc[nt]);
        } else {
          sacc[nt] = mfma16(__builtin_bit_cast(bf16x8_t, raw), qf[step], sacc[nt]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- mask, online softmax (lane = one head row, 16 kv values per lane)
    bf16x8_t pf[2];
    float alpha;
    bool up;
    {
      float mx = -__builtin_inff();
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kv = kv0 + nt * 16 + g4 + 4 * r;  // score row 4g4+r of tile nt
          float v = sacc[nt][r] * sscale;
          v = kv < vis_end ? v : -__builtin_inff();
          sacc[nt][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = wave_max_16x4(mx);
      const float old = m_ref;
      up = mx > old + kRescaleSlack;
      const float m_new = up ? mx : old;
      alpha = up ? exp2f(old - m_new) : 1.0f;  // old = -inf gives 0
      m_ref = m_new;
      const float m_use = m_new == -__builtin_inff() ? 0.0f : m_new;
      float psum = 0.0f;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = exp2f(sacc[nt][r] - m_use);
          sacc[nt][r] = p;
          psum += p;
        }
      l_part = l_part * alpha + psum;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u32x4_t w;
        w[0] = pack_bf16x2(sacc[2 * u][0], sacc[2 * u][1]);
        w[1] = pack_bf16x2(sacc[2 * u][2], sacc[2 * u][3]);
        w[2] = pack_bf16x2(sacc[2 * u + 1][0], sacc[2 * u + 1][1]);
        w[3] = pack_bf16x2(sacc[2 * u + 1][2], sacc[2 * u + 1][3]);
        pf[u] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
    if (__builtin_amdgcn_ballot_w64(up)) {
#pragma unroll
      for (int nt = 0; nt < 32; ++nt) o_acc[nt] *= alpha;
    }

    // ---- O^T[n, head] += V^T P^T ; V^T fragments by transposed LDS reads.
    // P^T fragment u, lane (head, g4) holds kv rows {32u + g4 + 4r, 32u + 16 + g4 + 4r}, r < 4;
    // the V^T fragment must hold the same kv rows, in the same order, for its latent column.
    {
      constexpr int VD = 4;  // V^T fragments in flight
      u32x4_t vb[VD];
      auto vread = [&](int j) -> u32x4_t {
        const int u = j >> 5, nt = j & 31;
        u32x4_t w;
        if constexpr (FP8) {
          const uint32_t off = v_base + (uint32_t)(32 * u * L::kMainStride + nt * 16);
          const i32x2_t raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_PTR(i32x2_t))(stage + off));
          w[0] = (unsigned)raw[0];
          w[1] = (unsigned)raw[1];
          w[2] = 0;
          w[3] = 0;
        } else {
          const uint32_t off = v_base + (uint32_t)(32 * u * L::kMainStride + nt * 32);
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(i16x4_t))(stage + off));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(i16x4_t))(stage + off + 16 * L::kMainStride));
          const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo);
          const u32x2_t h2 = __builtin_bit_cast(u32x2_t, hi);
          w[0] = l2[0];
          w[1] = l2[1];
          w[2] = h2[0];
          w[3] = h2[1];
        }
        return w;
      };
#pragma unroll
      for (int j = 0; j < VD - 1; ++j) vb[j] = vread(j);
#pragma unroll
      for (int j = 0; j < 64; ++j) {
        if (j + VD - 1 < 64) vb[(j + VD - 1) % VD] = vread(j + VD - 1);
        const u32x4_t w = vb[j % VD];
        const bf16x8_t vf = FP8 ? fp8x8_to_bf16x8(w[0], w[1]) : __builtin_bit_cast(bf16x8_t, w);
        o_acc[j & 31] = mfma16(vf, pf[j >> 5], o_acc[j & 31]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- epilogue: normalise, then the final row (single chunk) or a partial record
  const float l = wave_sum_16x4(l_part);
  const bool empty = !(l > 0.0f);
  const float inv = empty ? 0.0f : a.out_scale / l;
  const float lse2 = empty ? -__builtin_inff() : m_ref + __log2f(l);
  if (!row_ok) return;
  if (n_b == 1) {
    uint16_t* orow = a.out + (int64_t)row_out * kLatentDim;
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) {
      const f32x4_t o = o_acc[nt] * inv;
      u32x2_t w;
      w[0] = pack_bf16x2(o[0], o[1]);
      w[1] = pack_bf16x2(o[2], o[3]);
      *(u32x2_t*)(orow + nt * 16 + 4 * g4) = w;
    }
    if (a.lse && g4 == 0) a.lse[row_out] = lse2 * kLn2;
  } else {
    const int64_t rec = (int64_t)a.partbase[b] + (int64_t)grp * n_b + chunk;
    float* prow = a.part_out + (rec * a.rows_per_group + rr) * kLatentDim;
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) *(f32x4_t*)(prow + nt * 16 + 4 * g4) = o_acc[nt] * inv;
    if (g4 == 0) a.part_lse[rec * a.rows_per_group + rr] = lse2;
  }
}

// ---------------------------------------------------------------------------
// Combine: one workgroup (4 waves) per (column block, tile row, sequence x group).
// Wave w merges chunks w, w+4, ...; the four partial states meet in LDS.
template <int CPL>  // columns per lane: 8 (512-column blocks) or 1 (64-column blocks)
__global__ __launch_bounds__(256) void mla_combine_kernel(CombineArgs a) {
  constexpr int kCols = CPL * 64;
  __shared__ float st_m[4], st_s[4];
  __shared__ float st_acc[4][kCols];
  const int colblk = blockIdx.x;
  const int rr = blockIdx.y;
  const int b = blockIdx.z / a.num_groups;
  const int grp = blockIdx.z % a.num_groups;
  const int n_b = a.nchunks[b];
  if (n_b <= 1 || rr >= a.rows_per_group) return;
  const int s = rr / a.heads_per_group;
  const int head = grp * a.heads_per_group + rr % a.heads_per_group;
  if (head >= a.num_heads) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col0 = colblk * kCols + lane * CPL;
  const int64_t rec0 = (int64_t)a.partbase[b] + (int64_t)grp * n_b;

  float m = -__builtin_inff(), ssum = 0.0f, acc[CPL];
  for (int j = 0; j < CPL; ++j) acc[j] = 0.0f;
  for (int c = wave; c < n_b; c += 4) {
    const int64_t idx = (rec0 + c) * a.rows_per_group + rr;
    const float l = a.part_lse[idx];
    if (l == -__builtin_inff()) continue;
    const float m_new = fmaxf(m, l);
    const float f_old = exp2f(m - m_new);
    const float f_c = exp2f(l - m_new);
    const float* src = a.part_out + idx * kLatentDim + col0;
    ssum = ssum * f_old + f_c;
    if constexpr (CPL == 8) {
      const f32x4_t x0 = *(const f32x4_t*)(src);
      const f32x4_t x1 = *(const f32x4_t*)(src + 4);
      for (int j = 0; j < 4; ++j) {
        acc[j] = acc[j] * f_old + f_c * x0[j];
        acc[4 + j] = acc[4 + j] * f_old + f_c * x1[j];
      }
    } else {
      for (int j = 0; j < CPL; ++j) acc[j] = acc[j] * f_old + f_c * src[j];
    }
    m = m_new;
  }
  if (lane == 0) {
    st_m[wave] = m;
    st_s[wave] = ssum;
  }
  for (int j = 0; j < CPL; ++j) st_acc[wave][lane * CPL + j] = acc[j];
  __syncthreads();
  float M = fmaxf(fmaxf(st_m[0], st_m[1]), fmaxf(st_m[2], st_m[3]));
  const bool empty = M == -__builtin_inff();
  float f[4], total = 0.0f;
  for (int w = 0; w < 4; ++w) {
    f[w] = empty ? 0.0f : exp2f(st_m[w] - M);
    total += f[w] * st_s[w];
  }
  const float inv = total > 0.0f ? 1.0f / total : 0.0f;
  const int64_t orow = ((int64_t)b * a.seqlen_qo + s) * a.num_heads + head;
  for (int c = threadIdx.x; c < kCols; c += 256) {
    const float v = (f[0] * st_acc[0][c] + f[1] * st_acc[1][c] + f[2] * st_acc[2][c] + f[3] * st_acc[3][c]) * inv;
    a.out[orow * kLatentDim + colblk * kCols + c] = __builtin_bit_cast(uint16_t, (__bf16)v);
  }
  if (a.lse && colblk == 0 && threadIdx.x == 0)
    a.lse[orow] = empty ? -__builtin_inff() : (M + __log2f(total)) * kLn2;
}

template <bool FP8, int NW>
int launch_decode_t(const DecodeArgs& a, int gx, int gy, int gz, hipStream_t st) {
  hipLaunchKernelGGL((mla_decode_kernel<FP8, NW>), dim3(gx, gy, gz), dim3(NW * 64), 0, st, a);
  return (int)hipGetLastError();
}

}  // namespace

int launch_plan(const PlanArgs& a, void* stream) {
  hipLaunchKernelGGL(mla_plan_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

// Tile classes: 16, 32, 64, 128 rows -> 1, 2, 4, 8 waves of one 16-row head tile each.
int launch_decode(const DecodeArgs& a, int kv_dtype, int tile_class, int gx, int gy, int gz, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const bool fp8 = kv_dtype == MLA_KV_FP8_E4M3FN;
  switch (tile_class) {
    case 0: return fp8 ? launch_decode_t<true, 1>(a, gx, gy, gz, st) : launch_decode_t<false, 1>(a, gx, gy, gz, st);
    case 1: return fp8 ? launch_decode_t<true, 2>(a, gx, gy, gz, st) : launch_decode_t<false, 2>(a, gx, gy, gz, st);
    case 2: return fp8 ? launch_decode_t<true, 4>(a, gx, gy, gz, st) : launch_decode_t<false, 4>(a, gx, gy, gz, st);
    case 3: return fp8 ? launch_decode_t<true, 8>(a, gx, gy, gz, st) : launch_decode_t<false, 8>(a, gx, gy, gz, st);
  }
  return (int)hipErrorInvalidValue;
}

int launch_combine(const CombineArgs& a, int max_chunks, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int rows = a.rows_per_group;
  const int gz = a.batch * a.num_groups;
  if (max_chunks <= 16) {
    hipLaunchKernelGGL(mla_combine_kernel<8>, dim3(1, rows, gz), dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL(mla_combine_kernel<1>, dim3(kLatentDim / 64, rows, gz), dim3(256), 0, st, a);
  }
  return (int)hipGetLastError();
}

}  // namespace mla
