// Cached-prefix expansion of the paged latent cache into per-head K and V.
//
// "perf(mla): chunk the non-FP4 gather_kv_b_proj over KV" (description): the
// whole cached context is expanded once per layer as a set of (sequence, KV
// chunk, head) programs, none working past its sequence's end. Here a program
// is 256 cached rows of one sequence and one head h: the 256 projections W[h].c
// (128 K-nope then 128 V) on bf16 MFMA (16x16x32), and the 64 rope values
// copied beside K.
//
//   * Persistent: one workgroup per CU walks a static share of the programs
//     (XCD-contiguous, so that the workgroups of one XCD run adjacent programs
//     and share its L2 copy of W[h] and of the latent rows). Reading W[h] once
//     per 256 rows halves the L2 traffic of 128-row programs.
//   * 12 waves, three per SIMD: 8 MFMA waves hold the 256 x 256 output tile
//     (wave w: W rows 128 (w & 1) .. +127 for cached rows 64 (w >> 1) .. +63);
//     4 copy waves, one per SIMD, issue every copy and keep the books. An MFMA
//     wave never issues a copy (it would stall behind the busy vector-memory
//     front end, and its MFMAs with it) and never waits on the memory counter,
//     so its stores complete on their own.
//   * Each cached row is walked in slabs of KC columns (64 for an fp8 cache, 32
//     for bf16): 512 / KC stages multiply a slab of W[h] and of the chunk's 256
//     latent rows (fp8 kept as bytes and widened exactly to bf16 at the operand
//     read; kv_scale multiplies the float32 result), then 64 / KC stages carry
//     only the rope slab, stored as it arrives. The slabs are copied by
//     global_load_lds DMA into a ring of LDS stages (3 for fp8, 4 for bf16) that
//     runs on across program boundaries, so the copy never drains between
//     programs. The copy rate of a CU is set by the number of distinct cache
//     lines it requests: a 64-column W slab reads whole 128-byte lines. Each
//     copy wave waits for its share of a stage with counts of its own; the
//     workgroup barrier then publishes the stage. Each 16-byte piece of a row
//     sits XOR-swizzled by row, so the operand reads hit distinct banks.
//   * Copy wave 0 also copies, ahead of time, each program's page-list window
//     and the sequence bounds of the programs to come (64 at a time), finds the
//     next valid program two programs ahead and works out its row slots, so no
//     wave ever waits on a dependent load. Results are stored straight from
//     registers, 8 consecutive output columns per lane.
//   * Rows past a chunk are copied from a valid row and never stored; rows with
//     no valid slot are zeroed in LDS after they land (such a row reads as
//     zeros) and flag a status bit.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2_t;

#define KVB_LDS(T) __attribute__((address_space(3))) T*

constexpr int kChunkRows = 256;                      // cached rows per program
constexpr int kWRows = 256;                          // rows of W[h]: K nope, then V
constexpr int kNope = 128, kVDim = 128, kRope = 64;  // K is 192 wide: nope then rope
constexpr int kWaves = 8;      // MFMA waves: the 256 x 256 output tile
constexpr int kCopyWaves = 4;  // copy waves: every slab's copies and the bookkeeping
constexpr int kThreads = (kWaves + kCopyWaves) * 64;
constexpr int kXcds = 8;
constexpr int kWindow = 64;     // programs whose sequence bounds one copy fetches
constexpr int kLatSlab = 64;    // bytes of a latent row per stage (64 fp8 or 32 bf16 columns)
constexpr int kPageStages = 4;  // stages that carry a quarter each of the next program's page-list window

template <bool FP8>
struct KvbCfg {
  static constexpr int kElem = FP8 ? 1 : 2;
  static constexpr int kRowBytes = kRowDim * kElem;
  static constexpr int KC = kLatSlab / kElem;                // columns per stage: 64 | 32
  static constexpr int kMfmaStages = kLatentDim / KC;        // 8 | 16
  static constexpr int kStages = kRowDim / KC;               // 9 | 18: the rope is the last 64 / KC
  static constexpr int kKSteps = KC / 32;                    // MFMA k-steps per stage: 2 | 1
  static constexpr int kWRowBytes = KC * 2;                  // bytes of a W row per stage: 128 | 64
  static constexpr int kWSlabBytes = kWRows * kWRowBytes;    // 32 KB | 16 KB
  static constexpr int kWRowsPerInst = 1024 / kWRowBytes;    // 8 | 16
  static constexpr int kWInsts = kWSlabBytes / 1024;         // 32 | 16
  static constexpr int kWPerWave = kWInsts / kCopyWaves;     // 8 | 4
  static constexpr int kLatInsts = kChunkRows * kLatSlab / 1024;  // 16: row 16 j + lane / 4
  static constexpr int kLatPerWave = kLatInsts / kCopyWaves;      // 4
  static constexpr int kRing = FP8 ? 3 : 4;
  static constexpr int kStageBytes = kWSlabBytes + kChunkRows * kLatSlab;
  static constexpr int kPageOff = kRing * kStageBytes;           // one program's page-list window
  static constexpr int kSlotOff = kPageOff + kChunkRows * 4;     // two programs' row slots
  static constexpr int kWinOff = kSlotOff + 2 * kChunkRows * 4;  // two windows of sequence bounds
  static constexpr int kProgOff = kWinOff + 2 * 4 * kWindow * 4;  // four program records of 8 words
  static constexpr int kLdsBytes = kProgOff + 4 * 32;
  // copies a copy wave issues with stage s of a program: its share of the W slab (MFMA stages),
  // of the latent slab and, for copy wave 0 (cls 0) on the first stages, a quarter of the next
  // program's page-list window
  static constexpr int wave_insts(int cls, int s) {
    return (s < kMfmaStages ? kWPerWave : 0) + kLatPerWave + (s < kPageStages && cls == 0 ? 1 : 0);
  }
  // a wave's copies issued after its stage-s copies while stage s is waited for
  static constexpr int wait_after(int cls, int s) {
    int n = 0;
    for (int u = 1; u <= kRing - 2; ++u) n += wave_insts(cls, (s + u) % kStages);
    return n;
  }
  static_assert(kWInsts % kCopyWaves == 0 && kLatInsts % kCopyWaves == 0, "copy shares");
  static_assert(kStages > kPageStages + kRing, "page-list window and slots are ready in time");
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
};

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
  int32_t programs;  // batch * chunks * heads (< 2^31)
  int32_t num_heads, page_size, chunks, max_ctx, head_block;
  uint32_t page_magic;  // floor((2^32 - 1) / page_size): n / page_size = umulhi(n, magic), then one correction
  float kv_scale;
};

// n / page_size for 0 <= n < 2^31
__device__ __forceinline__ int kvb_page_div(int n, const KvbArgs& a) {
  uint32_t q = __umulhi((uint32_t)n, a.page_magic);
  if ((q + 1) * (uint32_t)a.page_size <= (uint32_t)n) ++q;
  return (int)q;
}

// A program as the workgroup's waves see it (8 words in LDS); bad: some row has no valid slot.
struct KvbProg {
  int32_t valid, h, orow, nrows, r0, pg_first, pg_end, bad;
};

// 16-byte piece swizzles (physical piece = logical piece ^ swizzle(row)). W rows are read 16
// at a time in the order that puts 8 consecutive output columns in one lane (rows 0-3, 8-11,
// 16-19, 24-27 of a 32-row block): with 128-byte rows the rows of one parity need distinct
// swizzles, with 64-byte rows distinct (row & 3, swizzle) pairs. Latent rows (64 bytes) are
// read 16 consecutive at a time: distinct (row & 3, swizzle) pairs.
template <bool FP8>
__device__ __forceinline__ int sw_w(int r) {
  if constexpr (FP8) return ((r >> 1) & 1) | ((r >> 2) & 6);
  else return (r >> 3) & 3;
}
__device__ __forceinline__ int sw_lat(int r) { return (r >> 2) & 3; }

// Copies from global memory straight into LDS (M0 = the wave's LDS base, the same in every
// lane): 16 bytes per lane at lds_addr + 16 * lane from a 64-bit address, or from a scalar
// base plus a 32-bit lane offset; 4 bytes per lane at lds_addr + 4 * lane. Inline asm, so
// that the compiler does not guard LDS reads with waits of its own: each wave waits for its
// copies with explicit counts before the barrier that publishes a stage.
__device__ __forceinline__ void kvb_dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}
__device__ __forceinline__ void kvb_dma16s(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}
__device__ __forceinline__ void kvb_dma4(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gptr),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void kvb_wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// wait for a wave's stage-s copies: wait_after(CLS, s) younger copies may still be in flight
template <typename C, int CLS, int S = 0>
__device__ __forceinline__ void kvb_wait_stage(int s) {
  if constexpr (S < C::kStages) {
    if (s == S) kvb_wait_vmcnt<C::wait_after(CLS, S)>();
    else kvb_wait_stage<C, CLS, S + 1>(s);
  }
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

// program id -> (sequence, chunk, head): heads in blocks of head_block, then sequences, then
// chunks, then the heads of the block, so that one XCD's adjacent programs share W[h] and the
// latent rows of a chunk
__device__ __forceinline__ void kvb_decode(const KvbArgs& a, int p, int& b, int& chunk, int& h) {
  const int hb = a.head_block;
  const int per_blk = a.programs / a.num_heads * hb;
  const int blk = p / per_blk;
  const int rem = p - blk * per_blk;
  const int bc = rem / hb;
  h = blk * hb + (rem - bc * hb);
  b = bc / a.chunks;
  chunk = bc - b * a.chunks;
}

template <bool FP8>
__global__ __launch_bounds__(kThreads) void mla_kv_b_proj_kernel(KvbArgs a) {
  using C = KvbCfg<FP8>;
  constexpr int S = C::kStages;
  // The arguments are read from the kernarg segment where they are used, through a pointer
  // the compiler cannot see through: hoisted to the top they would stay live in scalar
  // registers around the whole loop and push the loop's registers into scratch.
  typedef const __attribute__((address_space(4))) KvbArgs* KargPtr;
  auto args = [&]() -> const KvbArgs& {
    KargPtr ap = (KargPtr)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(ap));
    return *(const KvbArgs*)ap;
  };
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::kLdsBytes];
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
  KVB_LDS(uint8_t) L = (KVB_LDS(uint8_t))lds;
  KVB_LDS(int32_t) prog_ring = (KVB_LDS(int32_t))(L + C::kProgOff);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const bool copier = wave >= kWaves;
  const int cw = wave - kWaves;  // copy wave index (copy waves only)

  auto ring_get = [&](int slot) -> KvbProg {  // a program record, as scalars
    KVB_LDS(int32_t) r = prog_ring + slot * 8;
    return KvbProg{__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
                   __builtin_amdgcn_readfirstlane(r[2]), __builtin_amdgcn_readfirstlane(r[3]),
                   __builtin_amdgcn_readfirstlane(r[4]), __builtin_amdgcn_readfirstlane(r[5]),
                   __builtin_amdgcn_readfirstlane(r[6]), __builtin_amdgcn_readfirstlane(r[7])};
  };

  if (copier) {
    // ============================================================ copy waves
    // A copy wave shares its SIMD with two MFMA waves; at the top priority it issues its copies
    // as soon as it may (109,440 rows: 431 -> 421 us, 32,000: 126 -> 121, measured).
    __builtin_amdgcn_s_setprio(3);
    // this workgroup's programs: candidates m = 0 .. count - 1 are programs first + m * step
    // (XCD-contiguous ranges: the workgroups of one XCD take adjacent programs)
    auto cand_first = [&]() -> int {
      const int range = (args().programs + kXcds - 1) / kXcds;
      return (int)(blockIdx.x % kXcds) * range + (int)(blockIdx.x / kXcds);
    };
    const int step = gridDim.x / kXcds;
    int count;
    {
      const int range = (a.programs + kXcds - 1) / kXcds;
      const int xcd = blockIdx.x % kXcds;
      const int first = xcd * range + (int)(blockIdx.x / kXcds);
      const int end = min(a.programs, (xcd + 1) * range);
      count = first < end ? (end - first + step - 1) / step : 0;
    }

    // ---- copy wave 0's bookkeeping. Program records are found two programs ahead from
    // windows of 64 candidates' sequence bounds copied into LDS; the page-list window of a
    // program is copied with the first four stages of the program before it, and its row
    // slots are worked out at that program's stage 4.
    uint32_t bits = 0;  // status bits found by this lane (copy wave 0)
    int cand = 0;       // next candidate to examine
    int win_issued = -1, win_ready = -1;

    auto issue_window = [&](int w) {  // sequence bounds of candidates 64 w .. 64 w + 63
      const KvbArgs& A = args();
      const int m = w * kWindow + lane;
      const int32_t* s0 = A.cu_ctx;
      const int32_t* s1 = A.cu_ctx;
      const int32_t* s2 = A.cu_ctx;
      const int32_t* s3 = A.cu_ctx;
      if (m < count) {
        int b, chunk, h;
        kvb_decode(A, cand_first() + m * step, b, chunk, h);
        s0 = A.cu_ctx + b;
        s1 = A.cu_ctx + b + 1;
        s2 = A.kv_indptr + b;
        s3 = A.kv_indptr + b + 1;
      }
      const uint32_t dst = lds_base + C::kWinOff + (uint32_t)(w & 1) * (4 * kWindow * 4);
      kvb_dma4(s0, dst);
      kvb_dma4(s1, dst + 256);
      kvb_dma4(s2, dst + 512);
      kvb_dma4(s3, dst + 768);
    };
    // the next valid program from candidate `cand` on (all lanes take the same path)
    auto find_next = [&]() -> KvbProg {
      KvbProg r = {};
      while (cand < count) {
        const KvbArgs& A = args();
        const int w = cand / kWindow;
        if (w + 1 > win_issued && (w + 1) * kWindow < count) {
          issue_window(w + 1);
          win_issued = w + 1;
        }
        if (w > win_ready) {  // its copy may be in flight: wait for everything
          kvb_wait_vmcnt<0>();
          win_ready = win_issued;
        }
        KVB_LDS(int32_t) wb = (KVB_LDS(int32_t))(L + C::kWinOff + (w & 1) * (4 * kWindow * 4));
        const int e = cand % kWindow;
        const int32_t row0 = wb[e], row1 = wb[kWindow + e], pg0 = wb[2 * kWindow + e], pg1 = wb[3 * kWindow + e];
        int b, chunk, h;
        kvb_decode(A, cand_first() + cand * step, b, chunk, h);
        ++cand;
        const int ctx = row1 - row0;
        if (row0 < 0 || ctx < 0 || (int64_t)row0 + ctx > A.num_out_rows) {  // rows outside the outputs
          if (chunk == 0 && h == 0) bits |= MLA_KVB_ROWS_OUT_OF_RANGE;
          continue;
        }
        if (chunk == 0 && h == 0 && ctx > A.max_ctx) bits |= MLA_KVB_CTX_TOO_LONG;  // rows past it not written
        const int lim = min(ctx, A.max_ctx);
        const int r0 = chunk * kChunkRows;
        if (r0 >= lim) continue;  // past this sequence's last chunk
        r = KvbProg{1, h, row0 + r0, min(kChunkRows, lim - r0), r0, max(pg0, 0), pg1, 0};
        break;
      }
      return r;
    };
    auto publish = [&](const KvbProg& q, int slot) {  // program record -> LDS ring entry
      if (lane == 0) {
        KVB_LDS(int32_t) r = prog_ring + slot * 8;
        r[0] = q.valid;
        r[1] = q.h;
        r[2] = q.orow;
        r[3] = q.nrows;
        r[4] = q.r0;
        r[5] = q.pg_first;
        r[6] = q.pg_end;
        r[7] = q.bad;
      }
    };
    // page-list window copy j (ids 64 j .. 64 j + 63) of program q
    auto issue_pages = [&](const KvbProg& q, int j) {
      const KvbArgs& A = args();
      const int32_t* src = A.cu_ctx;  // a harmless valid word when the id is not needed
      if (q.valid) {
        const int64_t gi = (int64_t)q.pg_first + kvb_page_div(q.r0, A) + j * 64 + lane;
        if (gi < q.pg_end) src = A.kv_page_indices + gi;
      }
      kvb_dma4(src, lds_base + C::kPageOff + (uint32_t)j * 256);
    };
    // row slots of program q (ring entry `slot`) from its page-list window, 4 rows per lane;
    // records in the entry whether any row has no valid slot
    auto make_slots = [&](int slot, int parity) {
      const KvbProg q = ring_get(slot);
      KVB_LDS(int32_t) pt = (KVB_LDS(int32_t))(L + C::kPageOff);
      KVB_LDS(int32_t) st = (KVB_LDS(int32_t))(L + C::kSlotOff) + parity * kChunkRows;
      const KvbArgs& A = args();
      const int P = A.page_size;
      const int npages = q.pg_end - q.pg_first;
      const int page0 = kvb_page_div(q.r0, A);
      bool any = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = lane + 64 * i;
        const int ra = q.r0 + min(r, q.nrows - 1);
        const int page = kvb_page_div(ra, A);
        int32_t sl = -1;
        if (page < npages) {
          const int64_t v = (int64_t)pt[page - page0] * P + (ra - page * P);
          if (v >= 0 && v < A.num_slots) sl = (int32_t)v;
          else if (r < q.nrows) bits |= MLA_KVB_SLOT_OUT_OF_RANGE;
        } else if (r < q.nrows) {
          bits |= MLA_KVB_TOO_FEW_PAGES;
        }
        any |= sl < 0;
        st[r] = sl;
      }
      const bool bad = __builtin_amdgcn_ballot_w64(any) != 0;  // over all 64 lanes, before the lane-0 store
      if (lane == 0) prog_ring[slot * 8 + 7] = bad;
    };

    // ---- the copies. W copy j: row kWRowsPerInst j + lane / (64 / kWRowsPerInst), place
    // lane % (64 / kWRowsPerInst), holding logical piece place ^ sw_w(row); this wave's are
    // j = kWPerWave cw + i. Latent copy j: row 16 j + lane / 4, place lane % 4 holding logical
    // piece place ^ sw_lat(row) (the same for every j: (lane & 3) ^ ((lane >> 4) & 3)); this
    // wave's are j = kLatPerWave cw + i.
    constexpr int kWLanesPerRow = 64 / C::kWRowsPerInst;  // 8 | 4
    uint32_t w_off[C::kWPerWave];
#pragma unroll
    for (int i = 0; i < C::kWPerWave; ++i) {
      const int j = C::kWPerWave * cw + i;
      const int row = C::kWRowsPerInst * j + lane / kWLanesPerRow;
      const int place = lane % kWLanesPerRow;
      w_off[i] = (uint32_t)(row * (kLatentDim * 2) + ((place ^ sw_w<FP8>(row)) << 4));
    }
    const int lat_logical = (lane & 3) ^ ((lane >> 4) & 3);
    // this wave's copies of stage s of program k (record in ring entry k & 3, slots in table
    // k & 1) and, for copy wave 0 on the first stages, a quarter of program k + 1's page-list window
    auto issue_group = [&](int k, int s) {
      const KvbArgs& A = args();
      const uint32_t stage = lds_base + (uint32_t)(((k * S + s) % C::kRing) * C::kStageBytes);
      if (s < C::kMfmaStages) {
        const int32_t qh = __builtin_amdgcn_readfirstlane(prog_ring[(k & 3) * 8 + 1]);
        const uint8_t* wsrc = (const uint8_t*)(A.w + (int64_t)qh * kWRows * kLatentDim) + s * C::kWRowBytes;
#pragma unroll
        for (int i = 0; i < C::kWPerWave; ++i)
          kvb_dma16s(wsrc, w_off[i], stage + (uint32_t)(C::kWPerWave * cw + i) * 1024);
      }
      KVB_LDS(int32_t) st = (KVB_LDS(int32_t))(L + C::kSlotOff) + (k & 1) * kChunkRows;
#pragma unroll
      for (int i = 0; i < C::kLatPerWave; ++i) {
        const int j = C::kLatPerWave * cw + i;
        const int32_t sl = max(st[16 * j + (lane >> 2)], 0);
        kvb_dma16(A.cache + (int64_t)sl * C::kRowBytes + s * kLatSlab + lat_logical * 16,
                  stage + (uint32_t)(C::kWSlabBytes + j * 1024));
      }
      if (s < kPageStages && cw == 0) issue_pages(ring_get((k + 1) & 3), s);
    };
    // after this wave's stage-s copies of program k have landed: zero the latent pieces of rows
    // with no valid slot
    auto zero_bad = [&](int k, int s) {
      KVB_LDS(int32_t) st = (KVB_LDS(int32_t))(L + C::kSlotOff) + (k & 1) * kChunkRows;
      KVB_LDS(uint8_t) lat = L + ((k * S + s) % C::kRing) * C::kStageBytes + C::kWSlabBytes;
#pragma unroll
      for (int i = 0; i < C::kLatPerWave; ++i) {
        const int j = C::kLatPerWave * cw + i;
        if (st[16 * j + (lane >> 2)] < 0) *(KVB_LDS(u32x4_t))(lat + j * 1024 + lane * 16) = u32x4_t{0, 0, 0, 0};
      }
    };

    // ---- prologue
    if (cw == 0) {
      if (count > 0) {
        issue_window(0);
        win_issued = 0;
        kvb_wait_vmcnt<0>();
        win_ready = 0;
      }
      const KvbProg p0 = find_next();
      const KvbProg p1 = p0.valid ? find_next() : KvbProg{};
      publish(p0, 0);
      publish(p1, 1);
      publish(KvbProg{}, 2);
      if (p0.valid) {
#pragma unroll
        for (int j = 0; j < 4; ++j) issue_pages(p0, j);
        kvb_wait_vmcnt<0>();
        win_ready = win_issued;
        make_slots(0, 0);
      }
    }
    __syncthreads();
    KvbProg cur = ring_get(0);
    if (cur.valid) {
      // stages 0 .. kRing - 2 of program 0 (the first ones carry program 1's page-list window)
#pragma unroll
      for (int s = 0; s < C::kRing - 1; ++s) issue_group(0, s);
    }
    for (int k = 0; cur.valid; ++k) {
      const bool next_valid = __builtin_amdgcn_readfirstlane(prog_ring[((k + 1) & 3) * 8]) != 0;
#pragma unroll 1
      for (int s = 0; s < S; ++s) {
        // this wave's stage-s copies have landed once its younger copies are all that may be in flight
        if (s + C::kRing - 2 >= S && !next_valid) kvb_wait_vmcnt<0>();
        else if (cw == 0) kvb_wait_stage<C, 0>(s);
        else kvb_wait_stage<C, 1>(s);
        if (cur.bad) zero_bad(k, s);
        __syncthreads();  // stage s is in LDS for every wave; every wave is done with stage s - 1
        if (cw == 0 && s == kPageStages && next_valid) make_slots((k + 1) & 3, (k + 1) & 1);  // program k + 1
        if (cw == 0 && s == kPageStages + 1) publish(next_valid ? find_next() : KvbProg{}, (k + 2) & 3);
        // this wave's copies of stage s + kRing - 1 (this program's or the next one's), into the
        // slot of stage s - 1, which every wave is done with
        const int t = s + C::kRing - 1;
        if (t < S) issue_group(k, t);
        else if (next_valid) issue_group(k + 1, t - S);
      }
      cur = ring_get((k + 1) & 3);  // written at stage kPageStages + 1 of the program before this one
    }
    kvb_wait_vmcnt<0>();  // every copy of this wave has landed before the workgroup ends
    if (cw == 0) {
      uint32_t* status = args().status;
      if (bits && status) atomicOr(status, bits);
    }
    return;
  }

  // ============================================================ MFMA waves
  // They issue no copy and wait on no memory counter: they read the published stages,
  // multiply, and store (from registers; the stores complete on their own).
  const int l16 = lane & 15, g = lane >> 4;
  const int nh = wave & 1, th = wave >> 1;
  // LDS byte offsets of the operand reads within a stage, per k-step. Every swizzle involved
  // depends on the lane only: W row nh*128 + 32 (nb / 2) + 8 (l16 / 4) + 4 (nb % 2) + l16 % 4 has
  // sw_w = sw_w(8 (l16 / 4) + l16 % 4), latent row th*64 + 16 tb + l16 has sw_lat = sw_lat(l16), so
  // tile nb and tb only add compile-time row offsets. Opaque, so that the compiler keeps one
  // register per k-step rather than one per tile.
  const int w_row_lane = ((l16 >> 2) << 3) + (l16 & 3);
  uint32_t w_lane[C::kKSteps], l_lane[C::kKSteps];
#pragma unroll
  for (int ks = 0; ks < C::kKSteps; ++ks) {
    w_lane[ks] = (uint32_t)((nh * 128 + w_row_lane) * C::kWRowBytes + (((4 * ks + g) ^ sw_w<FP8>(w_row_lane)) << 4));
    if constexpr (FP8)
      l_lane[ks] = (uint32_t)(C::kWSlabBytes + (th * 64 + l16) * kLatSlab + (((2 * ks + (g >> 1)) ^ sw_lat(l16)) << 4) +
                              ((g & 1) << 3));
    else
      l_lane[ks] = (uint32_t)(C::kWSlabBytes + (th * 64 + l16) * kLatSlab + ((g ^ sw_lat(l16)) << 4));
    asm volatile("" : "+v"(w_lane[ks]), "+v"(l_lane[ks]));
  }
  __syncthreads();  // the prologue's program records
  KvbProg cur = ring_get(0);
  f32x4_t acc[8][4];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[nb][tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; cur.valid; ++k) {
#pragma unroll 1
    for (int s = 0; s < C::kMfmaStages; ++s) {
      __syncthreads();  // stage s is in LDS; every wave is done with stage s - 1
      KVB_LDS(uint8_t) st = L + ((k * S + s) % C::kRing) * C::kStageBytes;
#pragma unroll
      for (int ks = 0; ks < C::kKSteps; ++ks) {
        bf16x8_t bt[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          KVB_LDS(uint8_t) lp = st + l_lane[ks] + tb * 16 * kLatSlab;
          if constexpr (FP8) {
            const u32x2_t raw = *(KVB_LDS(u32x2_t))lp;
            const u32x4_t v = {fp8x2_bf16x2<false>(raw[0]), fp8x2_bf16x2<true>(raw[0]), fp8x2_bf16x2<false>(raw[1]),
                               fp8x2_bf16x2<true>(raw[1])};
            bt[tb] = __builtin_bit_cast(bf16x8_t, v);
          } else {
            bt[tb] = *(KVB_LDS(bf16x8_t))lp;
          }
        }
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          // tile nb's row m holds W row 32 (nb / 2) + 8 (m / 4) + 4 (nb % 2) + m % 4, so that a
          // lane's results of tiles 2i and 2i + 1 are 8 consecutive output columns
          const bf16x8_t at =
              *(KVB_LDS(bf16x8_t))(st + w_lane[ks] + ((nb >> 1) * 32 + (nb & 1) * 4) * C::kWRowBytes);
#pragma unroll
          for (int tb = 0; tb < 4; ++tb)
            acc[nb][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(at, bt[tb], acc[nb][tb], 0, 0, 0);
        }
      }
    }
#pragma unroll 1
    for (int s = C::kMfmaStages; s < S; ++s) {
      __syncthreads();  // stage s is in LDS; every wave is done with stage s - 1
      // a rope slab (rope columns KC (s - kMfmaStages) .. +KC - 1): 256 rows of 4 logical pieces
      // of 16 bytes, stored as bf16 (fp8: 8 output pieces per row, bf16: 4). Thread id handles
      // rows 512 i / kOutPieces + id / kOutPieces: the swizzle of its rows is the same for every i.
      const KvbArgs& A = args();
      const int H = A.num_heads;
      const float scale = A.kv_scale;
      KVB_LDS(uint8_t) ls = L + ((k * S + s) % C::kRing) * C::kStageBytes + C::kWSlabBytes;
      constexpr int kOutPieces = FP8 ? 8 : 4;
      constexpr int kRowsPerPass = kWaves * 64 / kOutPieces;  // 64 | 128
      const int col0 = kNope + C::KC * (s - C::kMfmaStages);
      int id = tid;
      asm volatile("" : "+v"(id));
      const int t0 = id / kOutPieces, piece = id % kOutPieces;
      const uint32_t rope_lane = FP8 ? (uint32_t)(t0 * kLatSlab + (((piece >> 1) ^ sw_lat(t0)) << 4) + ((piece & 1) << 3))
                                     : (uint32_t)(t0 * kLatSlab + ((piece ^ sw_lat(t0)) << 4));
#pragma unroll
      for (int i = 0; i < kChunkRows / kRowsPerPass; ++i) {
        const int t = t0 + i * kRowsPerPass;
        if (t >= cur.nrows) continue;
        u32x4_t o;
        if constexpr (FP8) {
          const u32x2_t raw = *(KVB_LDS(u32x2_t))(ls + rope_lane + i * kRowsPerPass * kLatSlab);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const unsigned lo = fp8x2_bf16x2<false>(raw[j]), hi = fp8x2_bf16x2<true>(raw[j]);
            o[2 * j] = pack2(__uint_as_float(lo << 16) * scale, __uint_as_float(lo & 0xffff0000u) * scale);
            o[2 * j + 1] = pack2(__uint_as_float(hi << 16) * scale, __uint_as_float(hi & 0xffff0000u) * scale);
          }
        } else {
          o = *(KVB_LDS(u32x4_t))(ls + rope_lane + i * kRowsPerPass * kLatSlab);
        }
        *(u32x4_t*)(A.k_out + ((int64_t)(cur.orow + t) * H + cur.h) * (kNope + kRope) + col0 + piece * 8) = o;
      }
      if (s == S - 1) {
        // the results (acc[2i + e][tb][v] is output column 32 i + 8 g + 4 e + v of chunk row
        // th*64 + tb*16 + l16)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const int t = th * 64 + tb * 16 + l16;
          if (t < cur.nrows) {
            const int64_t o = (int64_t)(cur.orow + t) * H + cur.h;
            uint16_t* dst = nh == 0 ? A.k_out + o * (kNope + kRope) : A.v_out + o * kVDim;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const f32x4_t x = acc[2 * i][tb], y = acc[2 * i + 1][tb];
              *(u32x4_t*)(dst + i * 32 + g * 8) =
                  u32x4_t{pack2(x[0] * scale, x[1] * scale), pack2(x[2] * scale, x[3] * scale),
                          pack2(y[0] * scale, y[1] * scale), pack2(y[2] * scale, y[3] * scale)};
            }
          }
        }
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
          for (int tb = 0; tb < 4; ++tb) acc[nb][tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    cur = ring_get((k + 1) & 3);  // written at stage kPageStages + 1 of the program before this one
  }
}

// CUs of the current device, looked up once per device
int kvb_num_cu() {
  static std::mutex mu;
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
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
  if (programs > 0x7fffffff) return MLA_ERR_UNSUPPORTED;
  const int num_cu = mla::kvb_num_cu();
  if (num_cu < 1) return MLA_ERR_HIP;
  // one workgroup per CU (a multiple of the XCD count), no more than there are programs
  int64_t grid = std::max<int64_t>(num_cu / mla::kXcds, 1) * mla::kXcds;
  grid = std::min<int64_t>(grid, (programs + mla::kXcds - 1) / mla::kXcds * mla::kXcds);
  // heads in blocks of up to 4 (a divisor of H): the programs running together on one XCD
  // cover a few heads of several chunks
  int hb = 1;
  for (int d = 1; d <= 4; ++d)
    if (p->num_heads % d == 0) hb = d;
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
  a.programs = (int32_t)programs;
  a.num_heads = p->num_heads;
  a.page_size = p->page_size;
  a.chunks = (int32_t)chunks;
  a.max_ctx = p->max_context_len;
  a.head_block = hb;
  a.page_magic = (uint32_t)(0xFFFFFFFFull / (uint64_t)p->page_size);
  a.kv_scale = p->kv_scale;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 g((unsigned)grid), blk(mla::kThreads);
  if (p->kv_dtype == MLA_KV_FP8_E4M3FN) hipLaunchKernelGGL(mla::mla_kv_b_proj_kernel<true>, g, blk, 0, st, a);
  else hipLaunchKernelGGL(mla::mla_kv_b_proj_kernel<false>, g, blk, 0, st, a);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}
