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
#include <type_traits>

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
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(short)))) short i16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned short)))) unsigned short u16x2_t;

#define LDS_PTR(T) __attribute__((address_space(3))) T*
#ifndef MLA_STEP_BARRIER
#define MLA_STEP_BARRIER() __builtin_amdgcn_sched_barrier(0)
#endif

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
// Planner: one workgroup walks the batch in tiles of 256 sequences, twice.
// Pass 1 counts the work items of each kind; pass 2 writes the per-sequence
// arrays and places every item of the work list: full chunks in (sequence,
// chunk) order, then partial last chunks by length class (longest first,
// ties by sequence), then one NaN-fill item per invalid sequence. Ranks
// within a class follow sequence order (wave ballots plus per-wave counts),
// so the list is deterministic. Last, the status words, with the persistent
// decode grid's task counter at its start W.
constexpr int kLengthClasses = 16;
constexpr int kCats = kLengthClasses + 1;  // length classes, then invalid sequences

struct SeqWork {
  int32_t n;      // chunks (0: invalid sequence)
  int32_t nfull;  // chunks of exactly chunk_len rows
  int32_t cat;    // -1: none; 0..15: length class of the partial last chunk; 16: invalid
  uint32_t bad;   // status bits
  int32_t ctx, page_base;
};

__device__ __forceinline__ SeqWork seq_work(const PlanArgs& a, int b) {
  SeqWork w{0, 0, -1, 0u, 0, 0};
  if (b >= a.batch) return w;
  const int32_t ctx = a.context_lens[b];
  w.ctx = ctx;
  w.page_base = a.kv_indptr[b];
  const int32_t pages = a.kv_indptr[b + 1] - w.page_base;
  if (ctx < a.seqlen_qo) w.bad |= MLA_DEV_CTX_TOO_SHORT;
  if (ctx > a.max_context_len) w.bad |= MLA_DEV_CTX_TOO_LONG;
  if (!w.bad && (int64_t)pages * a.page_size < (int64_t)ctx) w.bad |= MLA_DEV_TOO_FEW_PAGES;
  if (w.bad) {
    w.cat = kLengthClasses;
    return w;
  }
  const int32_t C = a.chunk_len;
  w.n = (ctx + C - 1) / C;
  const int32_t last = ctx - (w.n - 1) * C;  // 1..C
  w.nfull = last == C ? w.n : w.n - 1;
  if (last < C) w.cat = (int32_t)((int64_t)kLengthClasses * last / C);
  return w;
}

// Work item `pos` of the list: the chunk and, so that a decode task needs no
// second round trip for them, its sequence's planned length, page-list start,
// chunk count and first partial record.
__device__ __forceinline__ void store_item(int32_t* work, int64_t pos, int32_t b, int32_t chunk, int32_t ctx,
                                           int32_t page_base, int32_t n, int32_t part_base) {
  u32x4_t lo, hi;
  lo[0] = (uint32_t)b;
  lo[1] = (uint32_t)chunk;
  lo[2] = (uint32_t)ctx;
  lo[3] = (uint32_t)page_base;
  hi[0] = (uint32_t)n;
  hi[1] = (uint32_t)part_base;
  hi[2] = 0;
  hi[3] = 0;
  u32x4_t* dst = (u32x4_t*)(work + pos * kItemWords);
  dst[0] = lo;
  dst[1] = hi;
}

__global__ __launch_bounds__(256) void mla_plan_kernel(PlanArgs a) {
  __shared__ int32_t scan_pb[256], scan_full[256];
  __shared__ int32_t t_ctx[256], t_pb[256], t_n[256], t_base[256];  // the tile's sequence fields
  __shared__ int32_t cat_wave[4][kCats];
  __shared__ int32_t cat_total[kCats], cat_base[kCats], cat_carry[kCats];
  __shared__ int32_t full_total;
  __shared__ int32_t wsum_pb[4], wsum_full[4];  // per-wave totals of the tile's two scans
  __shared__ uint32_t bad_or[256];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  // ---- pass 1: totals of each kind of item
  if (tid < kCats) {
    cat_total[tid] = 0;
    cat_carry[tid] = 0;
  }
  if (tid == 0) full_total = 0;
  __syncthreads();
  uint32_t bad_acc = 0;
  int32_t my_full = 0;
  // the first tile's fields, loaded once for both passes (a batch of at most
  // 256 sequences then costs one round trip for them)
  const SeqWork w_first = seq_work(a, tid);
  for (int base = 0; base < a.batch; base += 256) {
    const SeqWork w = base == 0 ? w_first : seq_work(a, base + tid);
    bad_acc |= w.bad;
    my_full += w.nfull;
    if (w.cat >= 0) atomicAdd(&cat_total[w.cat], 1);
  }
  atomicAdd(&full_total, my_full);
  __syncthreads();
  if (tid == 0) {
    int32_t pos = full_total;
    for (int k = kLengthClasses - 1; k >= 0; --k) {
      cat_base[k] = pos;
      pos += cat_total[k];
    }
    cat_base[kLengthClasses] = pos;
    pos += cat_total[kLengthClasses];
    a.status[1] = (uint32_t)pos;  // work items
  }
  __syncthreads();

  // ---- pass 2: per-sequence arrays and the work list
  int32_t carry_pb = 0, carry_full = 0;
  for (int base = 0; base < a.batch; base += 256) {
    const int b = base + tid;
    const SeqWork w = base == 0 ? w_first : seq_work(a, b);
    const int32_t contrib = (w.n > 1 ? w.n : 0) * a.num_groups;
    int32_t rank = 0;  // among the earlier sequences of this wave with the same class
    for (int k = 0; k < kCats; ++k) {
      const uint64_t m = __builtin_amdgcn_ballot_w64(w.cat == k);
      if (w.cat == k) rank = __popcll(m & ((1ull << lane) - 1));
      if (lane == 0) cat_wave[wave][k] = __popcll(m);
    }
    // inclusive scans of the partial records and the full chunks over the
    // tile: within each wave by lane shifts, then the earlier waves' totals
    int32_t v0 = contrib, v1 = w.nfull;
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t u0 = __shfl_up(v0, off), u1 = __shfl_up(v1, off);
      if (lane >= off) {
        v0 += u0;
        v1 += u1;
      }
    }
    if (lane == 63) {
      wsum_pb[wave] = v0;
      wsum_full[wave] = v1;
    }
    __syncthreads();
    for (int k = 0; k < wave; ++k) {
      v0 += wsum_pb[k];
      v1 += wsum_full[k];
    }
    scan_pb[tid] = v0;
    scan_full[tid] = v1;
    const int32_t my_base = carry_pb + v0 - contrib;
    t_ctx[tid] = w.ctx;
    t_pb[tid] = w.page_base;
    t_n[tid] = w.n;
    t_base[tid] = my_base;
    __syncthreads();
    // the tile's full chunks, spread over all threads: item i of the tile is chunk
    // i - (first item of j) of the tile's sequence j, the first j whose inclusive count
    // exceeds i (a long sequence's chunks are not written by one thread alone)
    const int32_t tile_full = scan_full[255];
    for (int i = tid; i < tile_full; i += 256) {
      int lo = 0, hi = 255;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (scan_full[mid] > i) hi = mid; else lo = mid + 1;
      }
      const int32_t first = lo > 0 ? scan_full[lo - 1] : 0;
      store_item(a.work, carry_full + i, base + lo, i - first, t_ctx[lo], t_pb[lo], t_n[lo], t_base[lo]);
    }
    if (b < a.batch) {
      a.nchunks[b] = w.n;
      a.partbase[b] = my_base;
      if (w.cat >= 0) {
        int32_t pos = cat_base[w.cat] + cat_carry[w.cat] + rank;
        for (int v = 0; v < wave; ++v) pos += cat_wave[v][w.cat];
        store_item(a.work, pos, b, w.cat == kLengthClasses ? -1 : w.n - 1, w.ctx, w.page_base, w.n, my_base);
      }
    }
    carry_pb += scan_pb[255];
    carry_full += scan_full[255];
    __syncthreads();
    if (tid < kCats) cat_carry[tid] += cat_wave[0][tid] + cat_wave[1][tid] + cat_wave[2][tid] + cat_wave[3][tid];
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
    a.status[2] = (uint32_t)a.num_workgroups;  // the task counter: workgroup x's first task is below W
    a.status[3] = 0;                           // reserved
  }
}

// ---------------------------------------------------------------------------
// LDS block layout (one ring stage, BN cache rows; BN is a multiple of 32):
//   main region, bf16: row r at r*kMainStride holds its 512 latent elements
//                (the V part); the 1024-byte row is padded by 32 bytes (8 banks);
//   main region, fp8: the rows come in pairs, rows p and p + 8 of each
//                16-row group g forming pair P = 8g + p at P*kMainStride, the
//                first row in bytes 0..511 of the pair and the second in
//                512..1023, so that one 64-lane copy moves both rows and the
//                rows a wave copies stay within 16-row groups (a page of 16
//                rows holds them). Rows r and r + 16 share banks in transposed
//                V reads, as at any pitch that is a multiple of 16 bytes; those
//                conflicts are off the critical path;
//   tail region: the 64 rope elements of each row, kTailBytes apart from
//                kTailBase in copy order (the row at position pos is
//                row_at(pos): bf16 pos, fp8 the first or second row of pair
//                pos / 2 as pos is even or odd), in 16-byte slots (physical
//                slot j holds logical slot j ^ tail_xor(pos)).
// MFMA row m of K score tile nt is slice row nt*16 + m (fp8: row m / 8 of pair
// m % 8 of the tile's group). Measured on gfx950 with 8 waves: a K fragment
// read (16 rows x 64 bytes) takes 4.6-4.8 clocks per instruction at the bf16
// stride against 4.5 for a contiguous read (8.0 with a 16-byte pad), and the
// transposed V reads stay at 3.2-4.0 clocks.
template <bool FP8, int BN>
struct RowLayout {
  static_assert(BN % 32 == 0, "32-row slices");
  static constexpr int kElem = FP8 ? 1 : 2;
  static constexpr int kRowBytes = kRowDim * kElem;      // 576 or 1152 in the cache
  static constexpr int kMainBytes = kLatentDim * kElem;  // 512 or 1024
  static constexpr int kMainStride = 1024 + 32;          // bf16 row pitch, fp8 pair pitch
  static constexpr int kTileStride = (FP8 ? 8 : 16) * kMainStride;  // main bytes of 16 rows
  static constexpr int kSliceBytes = 2 * kTileStride;                // and of 32
  static constexpr int kTailBytes = 64 * kElem;          // 64 or 128
  static constexpr int kTailSlots = kTailBytes / 16;     // 4 or 8
  static constexpr int kTailBase = BN / 32 * kSliceBytes;
  static constexpr int kBlockBytes = kTailBase + BN * kTailBytes;
  // the tail row stride spans kTailBytes/4 banks; the position bits above that pick the xor
  static __device__ __forceinline__ int tail_xor(int pos) { return FP8 ? ((pos >> 2) & 3) : ((pos >> 1) & 7); }
  // the block row whose copy comes at position pos
  static __device__ __forceinline__ int row_at(int pos) {
    return FP8 ? 16 * (pos >> 4) + ((pos >> 1) & 7) + 8 * (pos & 1) : pos;
  }
};

__device__ __forceinline__ u32x4_t lds_b128(LDS_PTR(uint8_t) base, uint32_t off) {
  return *(LDS_PTR(u32x4_t))(base + off);
}

// 16 bytes per lane from global memory straight into LDS at lds_addr + 16*lane
// (global_load_lds_dwordx4; M0 holds the wave's LDS base). Written as inline
// asm so that the compiler does not guard every later LDS read with a wait
// for it: completion is awaited explicitly (vmcnt) before the workgroup
// barrier that publishes a stage.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_addr) : "memory");
}

// The same from a uniform 64-bit base held in scalar registers plus a 32-bit
// per-lane offset (the lane's address is sbase + voff), so that no per-lane
// 64-bit address has to be formed for a copy whose lanes share one row.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory");
}

// The same for 4 bytes per lane (global_load_lds_dword): lane i lands at lds_addr + 4*lane.
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gptr), "s"(lds_addr) : "memory");
}

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most C + min(k, MAXK) * K vector-memory instructions of this wave are pending.
template <int K, int MAXK, int C>
__device__ __forceinline__ void wait_vmcnt_blocks(int k) {
  if constexpr (MAXK >= 1) {
    if (k >= MAXK) {
      wait_vmcnt<C + MAXK * K>();
      return;
    }
    wait_vmcnt_blocks<K, MAXK - 1, C>(k);
  } else {
    wait_vmcnt<C>();
  }
}

// A lane's byte offset within a cache row's rope tail, made opaque to the
// compiler where the tail DMA's address is formed, so that it is computed there
// as a 32-bit value rather than hoisted out of the block loop and held as a
// 64-bit one (which spilled in the 128-row fp8 kernel, and a reload from
// scratch makes the next wait drain every DMA in flight).
__device__ __forceinline__ uint32_t lane_offset(uint32_t off) {
  asm volatile("" : "+v"(off));
  return off;
}

// Page-gathered loads of one chunk's cache rows, in blocks of BN rows, into
// an LDS ring of NS stages; NW waves of the workgroup (waves 0 .. NW-1) gather
// every block together. Wave w copies the rows at positions w*RPW .. w*RPW +
// RPW - 1 of the block's copy order (RowLayout), the r-th of them being cache
// row min(c_start + blk*BN + row_at(w*RPW + r), c_end - 1): rows past the
// chunk repeat its last row, whose scores are masked. An fp8 row pair (two
// consecutive positions) takes one copy instruction, a bf16 row one.
// Protocol, per block blk of the loop:
//   wait(blk); __syncthreads(); advance(blk); ... read stage blk % NS ...
// (advance(blk) may come later in the iteration: the stage it refills was
// freed by the barrier, and the loads it issues stay ahead of the next wait)
// Page ids never come through scalar loads inside the loop: an outstanding
// scalar load makes the first LDS wait of the block drain everything (the
// counter is shared and scalar loads return out of order).
//  - Ring of more than two stages: the page ids of block j (lane r: row r)
//    are copied by DMA (global_load_lds_dword) into a small LDS ring of NS
//    entries at iteration j - 2NS + 2, ahead of block j - NS + 1's gather in
//    issue order. Loads complete in order, so the wait for block k's gather
//    also covers the ids that iteration k needs; every iteration issues one
//    id copy (block index clamped) and kDmaInsts gather instructions per
//    valid block, and the wait counts both.
//  - Two stages: one vector load per block into a register (lane r: row r),
//    issued right after the previous block's gather: the loop waits for all
//    its loads at the top anyway.
// A page id outside the pool is replaced by page 0 and noted in bad_page.
template <bool FP8, int NW, int BN, int NS>
struct BlockGather {
  using L = RowLayout<FP8, BN>;
  static constexpr int RPW = BN / NW;  // rows each wave gathers per block
  static constexpr int kTailRowsPerInst = 64 / L::kTailSlots;
  static constexpr int kTailInsts = (RPW + kTailRowsPerInst - 1) / kTailRowsPerInst;
  static constexpr int kMainInsts = FP8 ? RPW / 2 : RPW;
  static constexpr int kDmaInsts = kMainInsts + kTailInsts;  // gather instructions per wave per block
  static constexpr bool kVecPages = NS == 2;
  static constexpr int kPidRingBytes = kVecPages ? 0 : NS * BN * 4;
  static_assert(RPW >= 1 && BN % NW == 0, "row split");
  // a wave's fp8 pairs fill part of one 16-row group or whole groups, so that
  // its first and last copies hold its lowest and highest rows
  static_assert(!FP8 || (RPW % 2 == 0 && (16 % RPW == 0 || RPW % 16 == 0)), "fp8 pairs of a wave");
  static_assert(kVecPages || RPW % 4 == 0, "page ids are read four at a time");
  static_assert((NS - 2) * (kDmaInsts + 1) <= 63, "vmcnt range");

  const uint8_t* cache;
  const int32_t* page_ids;
  uint32_t page_lim;  // page ids (int32) at or above this, as unsigned, are outside the pool
  uint32_t magic, lds_base, pid_base;
  int c_start, c_end, nblk, page_base, P, wave, lane, tslot, trow;
  bool bad_page;
  int v_page;  // two stages: lane r < RPW holds the page id of row r of the next block

  // pid_lds: LDS address of kPidRingBytes for the page-id ring (unused with two stages)
  __device__ __forceinline__ BlockGather(const DecodeArgs& a, uint32_t lds_base_, uint32_t pid_lds, int c_start_,
                                         int c_end_, int page_base_, int wave_, int lane_)
      : cache(a.cache),
        page_ids(a.kv_page_indices),
        // min(num_pages, 2^31): a pool of 2^31 pages or more holds every non-negative id
        page_lim((uint32_t)(a.num_pages < 0x80000000LL ? a.num_pages : 0x80000000LL)),
        magic(a.page_div_magic),
        lds_base(lds_base_),
        pid_base(pid_lds),
        c_start(c_start_),
        c_end(c_end_),
        nblk((c_end_ - c_start_ + BN - 1) / BN),
        page_base(page_base_),
        P(a.page_size),
        wave(wave_),
        lane(lane_),
        tslot(lane_ % L::kTailSlots),
        trow(lane_ / L::kTailSlots),
        bad_page(false),
        v_page(0) {}

  __device__ __forceinline__ void page_pos(int kv, int& q, int& rem) const {
    q = (int)__umulhi((uint32_t)kv, magic);
    rem = kv - q * P;
    if (rem >= P) {
      ++q;
      rem -= P;
    }
  }
  __device__ __forceinline__ int row_kv(int blk, int r) const {
    return min(c_start + blk * BN + L::row_at(wave * RPW + r), c_end - 1);
  }
  // the copy whose page id lane l loads: min(l, RPW - 1). For an fp8 cache its
  // row is formed where it is used: held across the block loop instead, it is
  // the value the register allocator spills first in the two-waves-per-SIMD
  // fp8 kernels.
  __device__ __forceinline__ int my_row() const {
    return min(FP8 ? (int)lane_offset((uint32_t)lane) : lane, RPW - 1);
  }
  __device__ __forceinline__ int checked(int pg) {
    if ((uint32_t)pg >= page_lim) {
      bad_page = true;
      pg = 0;
    }
    return pg;
  }
  // main part of the wave's j-th copy, one instruction. bf16: row j of the
  // wave (slot s0, a uniform base), lane l fetches its 16-byte slot l. fp8: the pair of rows
  // 2j and 2j + 1 of the wave (slots s0, s1), lanes 0-31 fetch the first row's
  // 32 slots, lanes 32-63 the second row's.
  __device__ __forceinline__ void issue_main(int blk, int j, int s0, int s1) const {
    const uint32_t stage_off = (uint32_t)(blk % NS) * L::kBlockBytes;
    const uint32_t dst =
        __builtin_amdgcn_readfirstlane(lds_base + stage_off + (uint32_t)((wave * kMainInsts + j) * L::kMainStride));
    if constexpr (FP8)
      dma16(cache + (int64_t)(lane < 32 ? s0 : s1) * L::kRowBytes + ((lane & 31) << 4), dst);
    else
      dma16s(cache + (int64_t)s0 * L::kRowBytes, (uint32_t)lane << 4, dst);
  }
  // rope tails: instruction m covers kTailRowsPerInst rows x kTailSlots slots;
  // sv is the slot of this lane's row
  __device__ __forceinline__ void issue_tail(int blk, int m, int sv) const {
    const uint32_t stage_off = (uint32_t)(blk % NS) * L::kBlockBytes;
    const int r = wave * RPW + m * kTailRowsPerInst + trow;
    const int logical = tslot ^ L::tail_xor(r);
    const uint8_t* src = cache + (int64_t)sv * L::kRowBytes + lane_offset(L::kMainBytes + (logical << 4));
    const uint32_t dst = __builtin_amdgcn_readfirstlane(
        lds_base + stage_off + (uint32_t)(L::kTailBase + (wave * RPW + m * kTailRowsPerInst) * L::kTailBytes));
    if (m * kTailRowsPerInst + trow < RPW) dma16(src, dst);
  }
  // LDS address of this wave's page ids of block j in the ring
  __device__ __forceinline__ uint32_t pid_slot(int j) const {
    return pid_base + (uint32_t)(((j % NS) * BN + wave * RPW) * 4);
  }
  // ring stages: copy the page ids of block j (clamped to the chunk) into the ring
  __device__ __forceinline__ void pid_copy(int j) const {
    int q, rem;
    page_pos(row_kv(min(j, nblk - 1), my_row()), q, rem);
    if (lane < RPW) dma4(page_ids + page_base + q, __builtin_amdgcn_readfirstlane(pid_slot(j)));
  }
  // two stages: load the page ids of block blk into v_page
  __device__ __forceinline__ void fetch_v(int blk) {
    int q, rem;
    page_pos(row_kv(blk, my_row()), q, rem);
    v_page = page_ids[page_base + q];
  }
  __device__ __forceinline__ void issue(int blk) {
    if constexpr (kVecPages) {
      int q, rem;
      page_pos(row_kv(blk, my_row()), q, rem);
      const int slot_v = checked(v_page) * P + rem;
#pragma unroll
      for (int j = 0; j < kMainInsts; ++j) {
        if constexpr (FP8)
          issue_main(blk, j, __builtin_amdgcn_readlane(slot_v, 2 * j), __builtin_amdgcn_readlane(slot_v, 2 * j + 1));
        else
          issue_main(blk, j, __builtin_amdgcn_readlane(slot_v, j), 0);
      }
#pragma unroll
      for (int m = 0; m < kTailInsts; ++m)
        issue_tail(blk, m, __builtin_amdgcn_ds_bpermute((m * kTailRowsPerInst + trow) << 2, slot_v));
    } else {
      // the wave's RPW page ids, four per (uniform-address) LDS read
      int pid[RPW];
      LDS_PTR(uint8_t) ring = (LDS_PTR(uint8_t))(uintptr_t)0;
#pragma unroll
      for (int r4 = 0; r4 < RPW; r4 += 4) {
        const u32x4_t v = *(LDS_PTR(u32x4_t))(ring + pid_slot(blk) + 4 * r4);
#pragma unroll
        for (int k = 0; k < 4; ++k) pid[r4 + k] = __builtin_amdgcn_readfirstlane((int)v[k]);
      }
      // slots of the wave's rows; when one page holds them all (they lie
      // between the rows of its first and last copies, and a page holds
      // consecutive cache rows), one lookup gives them all
      int slot[RPW];
      const int kv_a = __builtin_amdgcn_readfirstlane(row_kv(blk, 0));
      const int kv_b = __builtin_amdgcn_readfirstlane(row_kv(blk, RPW - 1));
      int qa, rema;
      page_pos(kv_a, qa, rema);
      if (rema + (kv_b - kv_a) < P) {
        const int s0 = checked(pid[0]) * P + rema;
#pragma unroll
        for (int r = 0; r < RPW; ++r) slot[r] = s0 + (__builtin_amdgcn_readfirstlane(row_kv(blk, r)) - kv_a);
      } else if (P == 1) {  // a page per row: the slot is the page id
#pragma unroll
        for (int r = 0; r < RPW; ++r) slot[r] = checked(pid[r]);
      } else {
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          int q, rem;
          page_pos(__builtin_amdgcn_readfirstlane(row_kv(blk, r)), q, rem);
          slot[r] = checked(pid[r]) * P + rem;
        }
      }
#pragma unroll
      for (int j = 0; j < kMainInsts; ++j) {
        if constexpr (FP8)
          issue_main(blk, j, slot[2 * j], slot[2 * j + 1]);
        else
          issue_main(blk, j, slot[j], 0);
      }
#pragma unroll
      for (int m = 0; m < kTailInsts; ++m) {
        int sv = slot[m * kTailRowsPerInst];
#pragma unroll
        for (int k = 1; k < kTailRowsPerInst; ++k)
          if (m * kTailRowsPerInst + k < RPW && trow == k) sv = slot[m * kTailRowsPerInst + k];
        issue_tail(blk, m, sv);
      }
    }
  }
  // prologue, first half: the page ids of blocks 0 .. NS-2 (issued before the
  // query loads, so both round trips overlap)
  __device__ __forceinline__ void prefetch_ids() {
    if constexpr (kVecPages) {
      fetch_v(0);
    } else {
#pragma unroll
      for (int j = 0; j < NS - 1; ++j) pid_copy(j);
    }
  }
  // prologue, second half: blocks 0 .. NS-2 in flight
  __device__ __forceinline__ void start() {
    if constexpr (kVecPages) {
      issue(0);
      if (1 < nblk) fetch_v(1);
    } else {
      // then iterations -(NS-1) .. -1 in loop order (id copy of block i + 2NS - 2,
      // gather of block i + NS - 1), so that the loop's wait counts hold from block 0
      wait_vmcnt<0>();
#pragma unroll
      for (int i = -(NS - 1); i < 0; ++i) {
        pid_copy(i + 2 * NS - 2);
        if (i + NS - 1 < nblk) issue(i + NS - 1);
      }
    }
  }
  // this wave's loads of block blk have landed (the caller then synchronises the workgroup)
  __device__ __forceinline__ void wait(int blk) const {
    if constexpr (kVecPages) {
      wait_vmcnt<0>();
    } else {
      // after block blk's gather: NS-2 id copies and the gathers of blocks blk+1 .. min(blk+NS-2, nblk-1)
      wait_vmcnt_blocks<kDmaInsts, NS - 2, NS - 2>(nblk - 1 - blk);
    }
  }
  // after the barrier that publishes block blk: the stage of block blk-1 is free
  __device__ __forceinline__ void advance(int blk) {
    if constexpr (kVecPages) {
      if (blk + 1 < nblk) {
        issue(blk + 1);
        if (blk + 2 < nblk) fetch_v(blk + 2);
      }
    } else {
      pid_copy(blk + 2 * NS - 2);
      if (blk + NS - 1 < nblk) issue(blk + NS - 1);
    }
  }
  __device__ __forceinline__ void report(uint32_t* status) const {
    if (__builtin_amdgcn_ballot_w64(bad_page) && lane == 0) atomicOr(status, MLA_DEV_PAGE_OUT_OF_RANGE);
  }
};

// Rows of an invalid sequence (n_b == 0) are NaN, written by its work item.
__device__ __forceinline__ void fill_invalid_rows(const DecodeArgs& a, int b, int grp, int wave, int nwaves,
                                                  int lane) {
  const float nan = __builtin_nanf("");
  for (int rr = wave; rr < a.rows_per_group; rr += nwaves) {
    const int s = rr / a.heads_per_group;
    const int head = grp * a.heads_per_group + rr % a.heads_per_group;
    if (head >= a.num_heads) continue;
    const int64_t row = ((int64_t)b * a.seqlen_qo + s) * a.num_heads + head;
    for (int c = lane; c < kLatentDim; c += 64) a.out[row * kLatentDim + c] = 0x7fc0;
    if (a.lse && lane == 0) a.lse[row] = nan;
  }
}

// Tile row rr of head group grp: its output row, its visible end in the chunk
// (the causal mask lets token s see ctx - S + 1 + s rows) and whether it exists.
__device__ __forceinline__ void tile_row(const DecodeArgs& a, int b, int grp, int rr, int ctx, int c_end,
                                         int& vis_end, int& row_out, bool& row_ok) {
  const int tok = rr / a.heads_per_group;
  const int head = grp * a.heads_per_group + rr % a.heads_per_group;
  row_ok = rr < a.rows_per_group && head < a.num_heads;
  vis_end = min(c_end, a.causal ? ctx - a.seqlen_qo + 1 + tok : ctx);
  row_out = row_ok ? (int)(((int64_t)b * a.seqlen_qo + tok) * a.num_heads + head) : 0;
}

// One head tile's online softmax over a block of 32 cache rows (two score tiles
// of S^T, lane = one head row, 4 rows per tile per lane): masks rows at or past
// vis_end, moves the reference max lazily, accumulates the row sum and returns
// P^T as one bf16 MFMA operand plus the factor for the output accumulator.
// Score r of tile nt of lane (head, g4) is block row nt*16 + 4*g4 + r; lim is
// vis_end - (first row of the block) - 4*g4.
__device__ __forceinline__ bf16x8_t softmax_block(f32x4_t (&s)[2], float sscale, int lim, float& m_ref,
                                                  float& l_part, float& alpha, bool& up) {
  float mx = -__builtin_inff();
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = s[nt][r] * sscale;
      v = nt * 16 + r < lim ? v : -__builtin_inff();
      s[nt][r] = v;
      mx = fmaxf(mx, v);
    }
  mx = wave_max_16x4(mx);
  const float old = m_ref;
  up = mx > old + kRescaleSlack;
  const float m_new = up ? mx : old;
  alpha = up ? __builtin_amdgcn_exp2f(old - m_new) : 1.0f;  // old = -inf gives 0
  m_ref = m_new;
  const float m_use = m_new == -__builtin_inff() ? 0.0f : m_new;
  float psum = 0.0f;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = __builtin_amdgcn_exp2f(s[nt][r] - m_use);
      s[nt][r] = p;
      psum += p;
    }
  l_part = l_part * alpha + psum;
  u32x4_t w;
  w[0] = pack_bf16x2(s[0][0], s[0][1]);
  w[1] = pack_bf16x2(s[0][2], s[0][3]);
  w[2] = pack_bf16x2(s[1][0], s[1][1]);
  w[3] = pack_bf16x2(s[1][2], s[1][3]);
  return __builtin_bit_cast(bf16x8_t, w);
}

// Final bf16 row (single chunk) or fp32 partial record of 4 latent columns
// [col, col + 4) of one tile row, already divided by the row sum.
__device__ __forceinline__ void store_out4(const DecodeArgs& a, bool final_row, int row_out, int64_t prec_row,
                                           int col, f32x4_t o) {
  if (final_row) {
    u32x2_t w;
    w[0] = pack_bf16x2(o[0], o[1]);
    w[1] = pack_bf16x2(o[2], o[3]);
    *(u32x2_t*)(a.out + (int64_t)row_out * kLatentDim + col) = w;
  } else {
    *(f32x4_t*)(a.part_out + prec_row * kLatentDim + col) = o;
  }
}

// ---------------------------------------------------------------------------
// Decode, row-split form. One workgroup = one (chunk, head group, sequence)
// with HW x KW waves. Wave (hw, kw) owns head tile hw (16 tile rows: its query
// fragments and its 16 x 512 fp32 output stay in registers for the whole
// chunk) and cache rows [32 kw, 32 kw + 32) of every block of BN = 32 KW rows,
// with its own online-softmax state. The KW states of a head tile are merged
// through LDS at the end of the chunk by wave (hw, 0).
template <bool FP8, int HW, int KW, int NS>
struct DecodeCfg {
  static constexpr int kWaves = HW * KW;
  static constexpr int kBlockN = 32 * KW;  // cache rows per block
  // Waves that issue the gather. The 128-row kernels (two waves per SIMD of
  // one workgroup) gather with one wave per SIMD, each taking twice the rows,
  // so that the other wave of each SIMD goes straight from the barrier to its
  // QK^T MFMAs and the pair falls out of step (measured: ragged fp8 decode
  // 832 -> 751 us, dense fp8 171.5 -> 162.2, dense bf16 155.2 -> 153.5; the
  // 64-row kernel, whose two waves per SIMD come from two workgroups, lost).
  static constexpr int kGatherWaves = (HW == 8 && KW == 1) ? kWaves / 2 : kWaves;
  using Gather = BlockGather<FP8, kGatherWaves, kBlockN, NS>;
  using L = typename Gather::L;
  static constexpr int kRingBytes = NS * L::kBlockBytes + Gather::kPidRingBytes;  // stages, then page ids
  // Merge area after the loop: 16 x 512 fp32 outputs, then a max and a sum per head, of every
  // wave when they all fit (each wave then merges a column slice), else of the waves with kw > 0
  // (wave (hw, 0) then merges the whole tile).
  static constexpr int kStateBytes = 32 * 64 * 16 + 2 * 16 * 4;
  static constexpr bool kMergeSpread = KW > 1 && kWaves * kStateBytes <= kRingBytes;
  static constexpr int kMergeWaves = KW == 1 ? 0 : kMergeSpread ? kWaves : (KW - 1) * HW;
  static constexpr int kMergeBytes = kMergeWaves * kStateBytes;
  // then two int32 slots through which the next task's index passes to every wave
  static constexpr int kTaskSlotBase = kRingBytes > kMergeBytes ? kRingBytes : kMergeBytes;
  static constexpr int kLdsBytes = kTaskSlotBase + 16;
  static_assert(kTaskSlotBase % 16 == 0 && kLdsBytes <= 160 * 1024, "LDS budget");
};

// A work item as the planner writes it: the chunk and its sequence's planned fields.
struct TaskItem {
  int32_t b, chunk, ctx, page_base, n_b, rec_base;
};

__device__ __forceinline__ TaskItem load_item(const DecodeArgs& a, int item) {
  const int32_t* w = a.work + (int64_t)item * kItemWords;
  TaskItem t{w[0], w[1], w[2], w[3], w[4], w[5]};
  return t;
}

// The next untaken task of the list: a device-scope vector atomic on the task
// counter (the planner starts it at W, the grid's first tasks being below W).
__device__ __forceinline__ int take_task(const DecodeArgs& a) {
  return (int)__hip_atomic_fetch_add(a.status + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One task: attention of head group grp's tile over KV chunk `chunk` of
// sequence b (a work item of the planner's list); the output for a
// single-chunk sequence, else the chunk's partial record. Lane 0 of wave 0
// takes the workgroup's next task from the counter into nxt as the task's last
// block starts, so that the workgroup takes work when it is about to be free
// and the counter's round trip overlaps that block and the epilogue.
// QF8 (fp8 cache only): the query is e4m3fn bytes; its latent dims go to the
// fp8 MFMA as they are (one term, unit block scale; the per-tensor q scale is
// folded into the softmax scale) and its rope dims are widened exactly to bf16.
template <bool FP8, int HW, int KW, int NS, int WPE, int KD, int VD, int QC, bool QF8>
__device__ __forceinline__ void decode_task(const DecodeArgs& a, LDS_PTR(uint8_t) lds, const TaskItem& it, int grp,
                                            int& nxt) {
  static_assert(FP8 || !QF8, "an fp8 query needs an fp8 cache");
  using Cfg = DecodeCfg<FP8, HW, KW, NS>;
  using L = typename Cfg::L;
  constexpr int NW = Cfg::kWaves;
  constexpr int BN = Cfg::kBlockN;

  // Opaque to the compiler across tasks, so that what is derived from the
  // thread index is computed inside each task rather than kept in registers
  // around the task loop (the gather and MFMA loop needs them all).
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep it scalar
  const int hw = wave % HW;   // head tile
  const int kw = wave / HW;   // row slice of each block
  const int i16 = lane & 15;  // MFMA column: head row within the wave's 16-row tile
  const int g4 = lane >> 4;   // MFMA k-group

  // ---- work item, loaded by the caller with the sequence's planned fields, so
  // that the loads before the first cache row are two batches of cold round
  // trips: the item, then the first page ids together with the query (and the
  // live context length, checked against the planned one).
  const int b = it.b, chunk = it.chunk;
  if (chunk < 0) {  // invalid sequence: NaN rows
    if (wave == 0 && lane == 0) nxt = take_task(a);
    fill_invalid_rows(a, b, grp, wave, NW, lane);
    return;
  }
  const int ctx = it.ctx, page_base = it.page_base, n_b = it.n_b, rec_base = it.rec_base;
  const int live_ctx = a.context_lens[b];

  const int c_start = chunk * a.chunk_len;
  const int c_end = min(c_start + a.chunk_len, ctx);
  int vis_end, row_out;
  bool row_ok;
  tile_row(a, b, grp, hw * 16 + i16, ctx, c_end, vis_end, row_out, row_ok);
  typename Cfg::Gather gather(a, (uint32_t)(uintptr_t)lds, (uint32_t)(uintptr_t)lds + NS * L::kBlockBytes, c_start,
                              c_end, page_base, wave, lane);
  const int nblk = gather.nblk;
  const bool gw = wave < Cfg::kGatherWaves;  // this wave issues gather copies (uniform)
  if (gw) gather.prefetch_ids();  // in flight with the query loads below

  // ---- query fragments (B operand of S^T = K Q^T), resident for the whole chunk.
  // bf16 cache: qf[t] holds d = 32t + 8*g4 .. +7 (18 fragments).
  // fp8 cache: the 512 latent dims run on the fp8 MFMA (16x16x128, 32 k per
  // lane) over the raw cache bytes. For 128-dim block kb the lane's 32 bytes
  // are d = 128kb + 16g4 + (0..15), then 128kb + 64 + 16g4 + (0..15): the dims
  // of its two 16-byte LDS reads of a cache row. The bf16 query is written as
  // 2^e (hi + 2^-4 lo), hi and lo fp8, with one e per head chosen so that the
  // head's largest latent |q| lands in [128, 256); e reaches the MFMA through
  // the E8M0 block scales of the head's column. (A lane's scale applies to a
  // 32-wide k-block made of two lane groups' 16-byte halves, not to its own
  // 32 bytes; one value for all four lanes of a column makes that moot.)
  // hi keeps 4 of a bf16 value's 8 significant bits and the remainder has at
  // most 4, so the split is exact for every element down to 2^-14 of the
  // head's largest. The 64 rope dims stay on the bf16 MFMA: qf[h] holds
  // d = 512 + 16g4 + 8h .. +7.
  bf16x8_t qf[FP8 ? 2 : 18];
  i32x8_t qh[FP8 ? 4 : 1], ql[FP8 ? 4 : 1];
  int q_scale_hi = 127, q_scale_lo = 127;  // E8M0 block scales of the hi and lo terms
  if constexpr (QF8) {
    // qh[kb]: bytes 0..15 = d = 128kb + 16g4 + (0..15), bytes 16..31 = 128kb + 64 + 16g4 + (0..15)
    const uint8_t* qrow8 = reinterpret_cast<const uint8_t*>(a.q) + (int64_t)row_out * kRowDim;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      u32x4_t lo = *(const u32x4_t*)(qrow8 + 128 * kb + 16 * g4);
      u32x4_t hi = *(const u32x4_t*)(qrow8 + 128 * kb + 64 + 16 * g4);
      if (!row_ok) lo = hi = u32x4_t{0, 0, 0, 0};
      qh[kb] = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x2_t w = *(const u32x2_t*)(qrow8 + kLatentDim + 16 * g4 + 8 * h);
      if (!row_ok) w = u32x2_t{0, 0};
      qf[h] = fp8x8_to_bf16x8(w[0], w[1]);
    }
  } else {
    const uint16_t* qrow = a.q + (int64_t)row_out * kRowDim;
    if constexpr (FP8) {
      // raw[4kb + 2h + p] = d = 128kb + 64h + 16g4 + 8p .. +7
      u32x4_t raw[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        u32x4_t v = *(const u32x4_t*)(qrow + 128 * (t >> 2) + 64 * ((t >> 1) & 1) + 16 * g4 + 8 * (t & 1));
        if (!row_ok) v = u32x4_t{0, 0, 0, 0};
        raw[t] = v;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4_t v = *(const u32x4_t*)(qrow + kLatentDim + 16 * g4 + 8 * h);
        if (!row_ok) v = u32x4_t{0, 0, 0, 0};
        qf[h] = __builtin_bit_cast(bf16x8_t, v);
      }
      // largest latent |q| of the lane (bf16 magnitudes order as their bit
      // patterns), then of the head: lanes i16 + 16 {0, 1, 2, 3}
      u16x2_t mx2 = u16x2_t{0, 0};
#pragma unroll
      for (int t = 0; t < 16; ++t)
#pragma unroll
        for (int w = 0; w < 4; ++w)
          mx2 = __builtin_elementwise_max(mx2, __builtin_bit_cast(u16x2_t, raw[t][w] & 0x7fff7fffu));
      const unsigned mx = mx2[0] > mx2[1] ? mx2[0] : mx2[1];
      const float head_max = wave_max_16x4(__uint_as_float(mx << 16));
      // exponent field E of the head's largest: |q| < 2^(E - 126). e = E - 134;
      // E is raised to 11 so the lo scale stays >= 0 (such heads are all below 2^-115).
      const int E = max((int)(__float_as_uint(head_max) >> 23), 11);
      q_scale_hi = E - 7;   // 127 + e
      q_scale_lo = E - 11;  // 127 + e - 4
      const float inv = __uint_as_float((unsigned)(261 - E) << 23);  // 2^-e, exact
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int kbk = t >> 2, dw = 4 * ((t >> 1) & 1) + 2 * (t & 1);
#pragma unroll
        for (int w2 = 0; w2 < 2; ++w2) {
          float xs[4];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const unsigned w = raw[t][2 * w2 + j];
            xs[2 * j] = __uint_as_float(w << 16) * inv;
            xs[2 * j + 1] = __uint_as_float(w & 0xffff0000u) * inv;
          }
          // |xs| < 256: in range of e4m3fn, which the converter does not saturate
          i16x2_t hv = i16x2_t{0, 0};
          hv = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hv, xs[0], xs[1], 1.0f, false);
          hv = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hv, xs[2], xs[3], 1.0f, true);
          const unsigned hw32 = __builtin_bit_cast(unsigned, hv);
          const bf16x2_t h01 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hw32, 1.0f, false);
          const bf16x2_t h23 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hw32, 1.0f, true);
          // remainders times 16: exact, and again below 256 in magnitude
          const float r0 = (xs[0] - (float)h01[0]) * 16.0f, r1 = (xs[1] - (float)h01[1]) * 16.0f;
          const float r2 = (xs[2] - (float)h23[0]) * 16.0f, r3 = (xs[3] - (float)h23[1]) * 16.0f;
          i16x2_t lv = i16x2_t{0, 0};
          lv = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lv, r0, r1, 1.0f, false);
          lv = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lv, r2, r3, 1.0f, true);
          qh[kbk][dw + w2] = (int)hw32;
          ql[kbk][dw + w2] = __builtin_bit_cast(int, lv);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < 18; ++t) {
        u32x4_t v = *(const u32x4_t*)(qrow + 32 * t + 8 * g4);
        if (!row_ok) v = u32x4_t{0, 0, 0, 0};
        qf[t] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
  }

  // ---- softmax state and output accumulators (O^T tiles: 16 latent cols x 16 heads)
  float m_ref = -__builtin_inff(), l_part = 0.0f;
  f32x4_t o_acc[32];
#pragma unroll
  for (int nt = 0; nt < 32; ++nt) o_acc[nt] = f32x4_t{0, 0, 0, 0};

  // Per-lane LDS offsets that do not change over the loop; each access adds a
  // compile-time immediate. K row i16 of score tile nt sits at k_main_base +
  // nt*kTileStride (fp8: row i16 / 8 of pair i16 % 8 of the tile's group).
  const uint32_t k_main_base =
      (FP8 ? (uint32_t)(i16 & 7) * L::kMainStride + (uint32_t)(i16 >> 3) * 512u : (uint32_t)i16 * L::kMainStride) +
      (uint32_t)g4 * 16;
  // V^T reads of the P^T fragment: element e < 4 is row 4g4 + e of the wave's
  // 32, e >= 4 is 16 + 4g4 + e - 4 (the order of the score rows in P^T).
  uint32_t v_base_lo, v_base_hi;
  if constexpr (FP8) {
    // supplier lane (k = i16/2, c = i16%2) reads element k's row, bytes 8c of the column tile
    const int k = i16 >> 1, c = i16 & 1;
    const int row = k < 4 ? 4 * g4 + k : 16 + 4 * g4 + k - 4;
    v_base_lo = (uint32_t)(8 * (row >> 4) + (row & 7)) * L::kMainStride + (uint32_t)((row >> 3) & 1) * 512u + 8u * c;
    v_base_hi = v_base_lo;
  } else {
    // supplier lane (k = i16/4, c = i16%4) reads rows of elements k and 4+k, columns 4c..4c+3
    const int k = i16 >> 2, c = i16 & 3;
    v_base_lo = (uint32_t)(4 * g4 + k) * L::kMainStride + 8u * c;
    v_base_hi = (uint32_t)(16 + 4 * g4 + k) * L::kMainStride + 8u * c;
  }

  // the live context length came with the query: the plan holds for the lengths it was made with
  asm volatile("" ::"s"(live_ctx));
  if (live_ctx != ctx && chunk == 0 && grp == 0 && wave == 0 && lane == 0) atomicOr(a.status, MLA_DEV_STALE_PLAN);
  if (gw) gather.start();
  const float sscale = a.score_scale_log2;
  // Wave priority: two waves share each SIMD, and while one runs its softmax
  // (and, for an fp8 cache, widens V) the other should keep the matrix pipe
  // fed, so a wave raises its priority for its MFMA phases. Measured per
  // configuration: the 128-row fp8 kernel with a bf16 query is fastest with
  // only QK^T raised (its PV phase carries the V widening), the others with
  // both phases raised (no effect on the bf16 kernels).
  constexpr bool kPrioPV = !(FP8 && !QF8 && HW == 8);
  // Where the next block's gather is issued (ring form). Measured per
  // configuration: the 128-row bf16 kernel is fastest issuing it after its
  // QK^T MFMAs, so that both waves of a SIMD start their matrix work as soon
  // as the block is published and the issue overlaps it; the fp8 kernels are
  // fastest issuing it right after the barrier.
  constexpr bool kLateGather = !FP8 && HW == 8 && !Cfg::Gather::kVecPages;

  for (int blk = 0; blk < nblk; ++blk) {
    if (gw) gather.wait(blk);
    __syncthreads();
    if (!kLateGather && gw) gather.advance(blk);
    // the last block issues no gather, so the counter's round trip queues behind no copy
    // (the ring form's page-id copy aside)
    if (blk == nblk - 1 && wave == 0 && lane == 0) nxt = take_task(a);
    LDS_PTR(uint8_t) stage = lds + (uint32_t)(blk % NS) * L::kBlockBytes;
    // this wave's 32 rows of the block: main rows at mstage, rope tails at tstage
    LDS_PTR(uint8_t) mstage = stage + (uint32_t)(kw * L::kSliceBytes);
    LDS_PTR(uint8_t) tstage = stage + (uint32_t)(L::kTailBase + kw * 32 * L::kTailBytes);
    const int kv0 = c_start + blk * BN + kw * 32;

    __builtin_amdgcn_s_setprio(1);
    // ---- S^T[kv, head] = K Q^T for the wave's 32 rows of the block (two tiles of 16 kv rows).
    // The LDS reads run in a ring of KD units in flight. Each tile's sum over
    // the dims is split over QC accumulators (the tile's m-th MFMA goes to chain
    // m % QC) so that consecutive MFMAs do not wait on each other.
    f32x4_t sacc[2];
    {
      f32x4_t sch[2][QC];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int c = 0; c < QC; ++c) sch[nt][c] = f32x4_t{0, 0, 0, 0};
      auto tail_read = [&](int nt, int slot) -> u32x4_t {  // logical 16-byte slot of the row's rope tail
        // copy position of slice row nt*16 + i16
        const int pos = FP8 ? 16 * nt + 2 * (i16 & 7) + (i16 >> 3) : nt * 16 + i16;
        return lds_b128(tstage, (uint32_t)(pos * L::kTailBytes) + ((uint32_t)(slot ^ L::tail_xor(pos)) << 4));
      };
      if constexpr (FP8) {
        // Unit u < 8 = (block kb = u / 2, tile nt = u % 2): the lane's two 16-byte
        // reads of its row for block kb, one fp8 MFMA each for hi and lo.
        // Units 8, 9 = the rope tail of tile 0, 1: one read, widened to bf16.
        constexpr int kUnits = 10;
        i32x8_t ku[KD];
        auto kunit = [&](int u) -> i32x8_t {
          if (u < 8) {
            const uint32_t off = k_main_base + (uint32_t)((u & 1) * L::kTileStride + (u >> 1) * 128);
            const u32x4_t lo = lds_b128(mstage, off), hi = lds_b128(mstage, off + 64);
            return __builtin_bit_cast(i32x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
          const u32x4_t t = tail_read(u - 8, g4);
          return __builtin_bit_cast(i32x8_t, __builtin_shufflevector(t, t, 0, 1, 2, 3, 0, 1, 2, 3));
        };
#pragma unroll
        for (int u = 0; u < KD - 1; ++u) ku[u] = kunit(u);
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
          if (u + KD - 1 < kUnits) ku[(u + KD - 1) % KD] = kunit(u + KD - 1);
          const i32x8_t k = ku[u % KD];
          if (u < 8) {
            const int kbk = u >> 1, nt = u & 1;
            const int c0 = (2 * kbk) % QC, c1 = (2 * kbk + 1) % QC;
            sch[nt][c0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k, qh[kbk], sch[nt][c0], 0, 0, 0, 127, 0,
                                                                            q_scale_hi);
            if constexpr (!QF8)
              sch[nt][c1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k, ql[kbk], sch[nt][c1], 0, 0, 0, 127,
                                                                              0, q_scale_lo);
          } else {
            const int nt = u - 8, c0 = 8 % QC, c1 = 9 % QC;
            sch[nt][c0] = mfma16(fp8x8_to_bf16x8((unsigned)k[0], (unsigned)k[1]), qf[0], sch[nt][c0]);
            sch[nt][c1] = mfma16(fp8x8_to_bf16x8((unsigned)k[2], (unsigned)k[3]), qf[1], sch[nt][c1]);
          }
          MLA_STEP_BARRIER();
        }
      } else {
        constexpr int kReads = 36;  // (step, tile): 16 main steps of 32 dims, then 2 tail steps
        u32x4_t kb[KD];
        auto kread = [&](int i) -> u32x4_t {
          const int step = i / 2, nt = i % 2;
          if (step < 16)
            return lds_b128(mstage, k_main_base + (uint32_t)(nt * L::kTileStride + step * 64));
          return tail_read(nt, 4 * (step - 16) + g4);
        };
#pragma unroll
        for (int i = 0; i < KD - 1; ++i) kb[i] = kread(i);
#pragma unroll
        for (int i = 0; i < kReads; ++i) {
          if (i + KD - 1 < kReads) kb[(i + KD - 1) % KD] = kread(i + KD - 1);
          const int step = i / 2, nt = i % 2;
          sch[nt][step % QC] = mfma16(__builtin_bit_cast(bf16x8_t, kb[i % KD]), qf[step], sch[nt][step % QC]);
          MLA_STEP_BARRIER();
        }
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        sacc[nt] = sch[nt][0];
#pragma unroll
        for (int c = 1; c < QC; ++c) sacc[nt] += sch[nt][c];
      }
    }

    __builtin_amdgcn_s_setprio(0);
    if (kLateGather && gw) gather.advance(blk);
    // ---- mask, online softmax
    float alpha;
    bool up;
    const bf16x8_t pf =
        softmax_block(sacc, sscale, vis_end - kv0 - 4 * g4, m_ref, l_part, alpha, up);
    if (__builtin_amdgcn_ballot_w64(up)) {
#pragma unroll
      for (int nt = 0; nt < 32; ++nt) o_acc[nt] *= alpha;
    }

    if constexpr (kPrioPV) __builtin_amdgcn_s_setprio(1);
    // ---- O^T[n, head] += V^T P^T ; V^T fragments by transposed LDS reads.
    // Lane (head, g4) of P^T holds the wave's rows 4g4 + r (r < 4) then
    // 16 + 4g4 + r; the V^T fragment holds the same rows, in the same order,
    // for its latent column.
    {
      constexpr int kReads = 32;
      u32x4_t vb[VD];
      auto vread = [&](int nt) -> u32x4_t {
        u32x4_t w;
        if constexpr (FP8) {
          const i32x2_t raw =
              __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_PTR(i32x2_t))(mstage + v_base_lo + (uint32_t)(nt * 16)));
          w[0] = (unsigned)raw[0];
          w[1] = (unsigned)raw[1];
          w[2] = 0;
          w[3] = 0;
        } else {
          const uint32_t imm = (uint32_t)(nt * 32);
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(i16x4_t))(mstage + v_base_lo + imm));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(i16x4_t))(mstage + v_base_hi + imm));
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
      for (int j = 0; j < kReads; ++j) {
        if (j + VD - 1 < kReads) vb[(j + VD - 1) % VD] = vread(j + VD - 1);
        const u32x4_t w = vb[j % VD];
        const bf16x8_t vf = FP8 ? fp8x8_to_bf16x8(w[0], w[1]) : __builtin_bit_cast(bf16x8_t, w);
        o_acc[j] = mfma16(vf, pf, o_acc[j]);
        MLA_STEP_BARRIER();
      }
    }
    if constexpr (kPrioPV) __builtin_amdgcn_s_setprio(0);
  }
  if (gw) gather.report(a.status);

  // ---- epilogue. Each head tile has KW partial states (m_ref, l, o_acc) over
  // disjoint row sets, each relative to its own reference max; with KW > 1
  // they are merged through LDS (see DecodeCfg: by column slices over all
  // waves, or by wave (hw, 0) alone). Wave (hw, kw) then stores 16-column
  // output tiles [nt0, nt0 + ntiles) of head tile hw.
  float l_tot = wave_sum_16x4(l_part);
  float m_fin = m_ref;
  int nt0 = 0, ntiles = 32;
  if constexpr (KW > 1) {
    __syncthreads();  // every wave is done with the ring
    LDS_PTR(f32x4_t) ox = (LDS_PTR(f32x4_t))lds;                                     // [slot][32][64]
    LDS_PTR(float) mlx = (LDS_PTR(float))(lds + Cfg::kMergeWaves * 32 * 64 * 16);  // [slot][2][16]
    // LDS slot of wave (hw, k)'s state
    auto slot_of = [&](int k) { return Cfg::kMergeSpread ? k * HW + hw : (k - 1) * HW + hw; };
    if (Cfg::kMergeSpread || kw > 0) {
      const int slot = slot_of(kw);
#pragma unroll
      for (int nt = 0; nt < 32; ++nt) ox[(slot * 32 + nt) * 64 + lane] = o_acc[nt];
      if (g4 == 0) {
        mlx[slot * 32 + i16] = m_ref;
        mlx[slot * 32 + 16 + i16] = l_tot;
      }
    }
    __syncthreads();
    if (!Cfg::kMergeSpread && kw > 0) return;
    float ms[KW], ls[KW], wt[KW];
#pragma unroll
    for (int k = 0; k < KW; ++k) {
      const bool own = !Cfg::kMergeSpread && k == 0;
      ms[k] = own ? m_ref : mlx[slot_of(k) * 32 + i16];
      ls[k] = own ? l_tot : mlx[slot_of(k) * 32 + 16 + i16];
    }
    m_fin = ms[0];
#pragma unroll
    for (int k = 1; k < KW; ++k) m_fin = fmaxf(m_fin, ms[k]);
    l_tot = 0.0f;
#pragma unroll
    for (int k = 0; k < KW; ++k) {
      wt[k] = ms[k] == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(ms[k] - m_fin);
      l_tot += wt[k] * ls[k];
    }
    if (Cfg::kMergeSpread) {
      nt0 = kw * (32 / KW);
      ntiles = 32 / KW;
    }
#pragma unroll
    for (int nt = 0; nt < 32; ++nt) {
      if (Cfg::kMergeSpread && (nt < nt0 || nt >= nt0 + ntiles)) continue;
      f32x4_t acc = f32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int k = 0; k < KW; ++k) {
        const bool own = !Cfg::kMergeSpread && k == 0;
        acc += wt[k] * (own ? o_acc[nt] : ox[(slot_of(k) * 32 + nt) * 64 + lane]);
      }
      o_acc[nt] = acc;
    }
  }
  const bool empty = !(l_tot > 0.0f);
  const float inv = empty ? 0.0f : a.out_scale / l_tot;
  const float lse2 = empty ? -__builtin_inff() : m_fin + __log2f(l_tot);
  if (!row_ok) return;
  const int rr = hw * 16 + i16;
  const int64_t rec = (int64_t)rec_base + (int64_t)grp * n_b + chunk;
  const int64_t prec_row = rec * a.rows_per_group + rr;
#pragma unroll
  for (int nt = 0; nt < 32; ++nt)
    if (nt >= nt0 && nt < nt0 + ntiles) store_out4(a, n_b == 1, row_out, prec_row, nt * 16 + 4 * g4, o_acc[nt] * inv);
  if (kw == 0 && g4 == 0) {
    if (n_b == 1) {
      if (a.lse) a.lse[row_out] = lse2 * kLn2;
    } else {
      a.part_lse[prec_row] = lse2;
    }
  }
}

// The persistent decode kernel: a grid of W = num_cu x occupancy workgroups
// walks the tasks of the planner's list (task t: item t / G, head group t % G).
// Workgroup x first runs task first(x) (consecutive tasks on one XCD: the
// hardware deals consecutive workgroups to the 8 XCDs in turn, so the head
// groups and chunks of one sequence share an L2), then the next untaken task
// of the list from the workspace's task counter (a device-scope vector atomic;
// the planner starts it at W), taken as each task's last block starts, until
// the list is done: the longest work goes first, to whichever workgroup is
// about to be free. The task index passes between waves through two LDS slots
// used in turn. Every finished task takes one value from the counter, so one
// call's values are exactly W .. W + tasks - 1: the workgroup that gets the
// last one knows that every other has taken its last, and sets the counter
// back to W for the next call.
template <bool FP8, int HW, int KW, int NS, int WPE, int KD, int VD, int QC, bool QF8 = false>
__global__ __launch_bounds__(HW * KW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void mla_decode_kernel(DecodeArgs a) {
  using Cfg = DecodeCfg<FP8, HW, KW, NS>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::kLdsBytes];
  LDS_PTR(uint8_t) lds = (LDS_PTR(uint8_t))smem;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = a.num_workgroups;
  const int x = (int)blockIdx.x;
  const int G = a.num_groups;
  int task = W % kNumXcd ? x : (x % kNumXcd) * (W / kNumXcd) + x / kNumXcd;
  // the item count with the first task's item, in one batch (the item index is clamped to
  // the list's capacity, so a workgroup past the list still reads in bounds)
  const int n_items = (int)a.status[1];
  TaskItem cur = load_item(a, min(task / G, a.work_capacity - 1));
  asm volatile("" ::"s"(n_items), "s"(cur.b), "s"(cur.chunk), "s"(cur.ctx), "s"(cur.page_base), "s"(cur.n_b),
               "s"(cur.rec_base));
  const int n_tasks = n_items * G;
  for (int k = 0; task < n_tasks; ++k) {
    int nxt = 0;
    // The kernel arguments are read through a pointer the compiler cannot see
    // across tasks (a is the kernel's only argument: it sits at the start of the
    // kernel-argument segment), so that they are loaded inside each task, as a
    // kernel of one task would: hoisted out of the loop they would all stay live
    // around it and push the registers of the gather and MFMA loop into scratch.
    typedef const __attribute__((address_space(4))) DecodeArgs* KernargPtr;
    KernargPtr ap = (KernargPtr)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(ap));
    const int grp = task - (task / G) * G;
    LDS_PTR(int32_t) slot = (LDS_PTR(int32_t))(lds + Cfg::kTaskSlotBase) + (k & 1);
    decode_task<FP8, HW, KW, NS, WPE, KD, VD, QC, QF8>(*(const DecodeArgs*)ap, lds, cur, grp, nxt);
    if (wave == 0 && lane == 0) {
      *slot = nxt;
      if (nxt == W + n_tasks - 1)  // the call's last value: every workgroup has taken its last
        __hip_atomic_store(a.status + 2, (uint32_t)W, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // every wave is done with the ring, the merge area and this task before the next task's
    // loads land there, and the next task's index is in the slot
    __syncthreads();
    task = __builtin_amdgcn_readfirstlane(*slot);
    if (task < n_tasks) {
      cur = load_item(a, task / G);
      asm volatile("" ::"s"(cur.b), "s"(cur.chunk), "s"(cur.ctx), "s"(cur.page_base), "s"(cur.n_b),
                   "s"(cur.rec_base));
    }
  }
}

// ---------------------------------------------------------------------------
// Combine: one workgroup (256 threads) per (column block of CB columns, tile
// row, sequence x group), in a single pass over the partial records: the
// threads form 1024/CB streams of CB/4 threads (4 columns each); a stream
// walks chunks stream, stream + nstreams, ... keeping a running maximum m,
// weight sum s and weighted column sums, so that the lse and the partial
// output of a chunk are loaded together. The streams are then merged through
// LDS. CB shrinks when there are few rows to merge, so that many workgroups
// share a long list of chunks.
// Split-KV merge of one output row over N chunks (N known at compile time):
// lane l holds columns 4l .. 4l+3 and 256 + 4l .. +3 (each load instruction
// reads 1 KB of a row contiguously), every chunk's loads in flight at once.
// Lane c < N reads chunk c's lse; M = max_c lse_c, w_c = 2^(lse_c - M),
// out = sum_c w_c o_c / sum_c w_c, lse = (M + log2 sum_c w_c) ln 2.
template <int N>
__device__ __forceinline__ void merge_row(const CombineArgs& a, const float* src, int64_t rec_stride,
                                          const float* lse_src, int64_t orow, int lane) {
  f32x4_t x0[N], x1[N];
#pragma unroll
  for (int c = 0; c < N; ++c) {
    x0[c] = *(const f32x4_t*)(src + c * rec_stride);
    x1[c] = *(const f32x4_t*)(src + c * rec_stride + kLatentDim / 2);
  }
  const float lse_l = lane < N ? lse_src[lane * a.rows_per_group] : -__builtin_inff();
  float M = lse_l;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float w_l = lse_l == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(lse_l - M);
  float total = w_l;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) total += __shfl_xor(total, off);
  f32x4_t acc0 = f32x4_t{0, 0, 0, 0}, acc1 = f32x4_t{0, 0, 0, 0};
#pragma unroll
  for (int c = 0; c < N; ++c) {
    const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_l), c));
    acc0 += w * x0[c];
    acc1 += w * x1[c];
  }
  const float inv = total > 0.0f ? 1.0f / total : 0.0f;
  u32x2_t lo, hi;
  lo[0] = pack_bf16x2(acc0[0] * inv, acc0[1] * inv);
  lo[1] = pack_bf16x2(acc0[2] * inv, acc0[3] * inv);
  hi[0] = pack_bf16x2(acc1[0] * inv, acc1[1] * inv);
  hi[1] = pack_bf16x2(acc1[2] * inv, acc1[3] * inv);
  *(u32x2_t*)(a.out + orow * kLatentDim + 4 * lane) = lo;
  *(u32x2_t*)(a.out + orow * kLatentDim + kLatentDim / 2 + 4 * lane) = hi;
  if (a.lse && lane == 0) a.lse[orow] = total > 0.0f ? (M + __log2f(total)) * kLn2 : -__builtin_inff();
}

// The row's merge for its chunk count n (2 <= n <= N), unrolled for each count.
template <int N>
__device__ __forceinline__ void merge_row_upto(int n, const CombineArgs& a, const float* src, int64_t rec_stride,
                                               const float* lse_src, int64_t orow, int lane) {
  if (n == N) {
    merge_row<N>(a, src, rec_stride, lse_src, orow, lane);
  } else if constexpr (N > 2) {
    merge_row_upto<N - 1>(n, a, src, rec_stride, lse_src, orow, lane);
  }
}

// Split-KV merge when no sequence has more than MAXN chunks: one wave per
// output row, dispatched on the row's chunk count, no LDS. Two instances
// (MAXN = 8 and 16) so that the common few-chunk merges keep the register
// count, and the occupancy, of an 8-chunk body.
template <int MAXN>
__global__ __launch_bounds__(256) void mla_combine_rows_kernel(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int rows = a.rows_per_group;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keep the row scalar
  const int64_t r = (int64_t)blockIdx.x * 4 + wave;
  if (r >= (int64_t)a.batch * a.num_groups * rows) return;
  const int bg = (int)(r / rows), rr = (int)(r - (int64_t)bg * rows);
  const int b = bg / a.num_groups, grp = bg - b * a.num_groups;
  const int n_b = a.nchunks[b];
  const int pbase = a.partbase[b];
  asm volatile("" ::"s"(n_b), "s"(pbase));  // one round trip for both
  if (n_b <= 1 || n_b > MAXN) return;  // the launcher picks MAXN >= the plan's chunk count
  const int s = rr / a.heads_per_group;
  const int head = grp * a.heads_per_group + rr % a.heads_per_group;
  if (head >= a.num_heads) return;
  const int64_t rec0 = (int64_t)pbase + (int64_t)grp * n_b;
  const int64_t rec_stride = (int64_t)rows * kLatentDim;
  const float* src = a.part_out + (rec0 * rows + rr) * kLatentDim + 4 * lane;
  const float* lse_src = a.part_lse + rec0 * rows + rr;
  const int64_t orow = ((int64_t)b * a.seqlen_qo + s) * a.num_heads + head;
  merge_row_upto<MAXN>(n_b, a, src, rec_stride, lse_src, orow, lane);
}

// Split-KV merge for any chunk count: column blocks of CB, streams of threads
// walking the chunks with a running max.
template <int CB>
__global__ __launch_bounds__(256) void mla_combine_kernel(CombineArgs a) {
  constexpr int kThreadsPerChunk = CB / 4;
  constexpr int kStreams = 256 / kThreadsPerChunk;
  constexpr int kUnroll = 4;
  __shared__ float m_lds[kStreams], s_lds[kStreams], w_lds[kStreams];
  __shared__ float total_lds;
  __shared__ __attribute__((aligned(16))) float acc_lds[kStreams][CB];
  // blockIdx.x = (sequence x group, tile row, column block), column block fastest
  constexpr int kColBlocks = kLatentDim / CB;
  const int64_t t = blockIdx.x / kColBlocks;
  const int colblk = (int)(blockIdx.x - t * kColBlocks);
  const int rr = (int)(t % a.rows_per_group);
  const int bg = (int)(t / a.rows_per_group);
  const int b = bg / a.num_groups;
  const int grp = bg % a.num_groups;
  const int n_b = a.nchunks[b];
  const int pbase = a.partbase[b];
  asm volatile("" ::"s"(n_b), "s"(pbase));  // one round trip for both
  if (n_b <= 1 || rr >= a.rows_per_group) return;
  const int s = rr / a.heads_per_group;
  const int head = grp * a.heads_per_group + rr % a.heads_per_group;
  if (head >= a.num_heads) return;
  const int tid = threadIdx.x;
  const int stream = tid / kThreadsPerChunk;
  const int quad = tid % kThreadsPerChunk;
  const int64_t rec0 = (int64_t)pbase + (int64_t)grp * n_b;
  const float* lse_base = a.part_lse + rec0 * a.rows_per_group + rr;
  const float* out_base = a.part_out + (rec0 * a.rows_per_group + rr) * kLatentDim + colblk * CB + quad * 4;
  const int64_t rec_stride = (int64_t)a.rows_per_group * kLatentDim;

  // ---- running merge of this stream's chunks (a chunk with lse = -inf has weight 0)
  float m = -__builtin_inff(), ws = 0.0f;
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int c0 = stream; c0 < n_b; c0 += kUnroll * kStreams) {
    float lse[kUnroll];
    f32x4_t x[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const int c = c0 + k * kStreams;
      const bool ok = c < n_b;
      lse[k] = ok ? lse_base[(int64_t)c * a.rows_per_group] : -__builtin_inff();
      x[k] = ok ? *(const f32x4_t*)(out_base + (int64_t)c * rec_stride) : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      if (lse[k] == -__builtin_inff()) continue;
      const float m_new = fmaxf(m, lse[k]);
      const float sc = m == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m - m_new);
      const float w = __builtin_amdgcn_exp2f(lse[k] - m_new);
      acc = acc * sc + w * x[k];
      ws = ws * sc + w;
      m = m_new;
    }
  }

  // ---- merge the streams: weights 2^(m_s - M), then column sums
  *(f32x4_t*)&acc_lds[stream][quad * 4] = acc;
  if (quad == 0) {
    m_lds[stream] = m;
    s_lds[stream] = ws;
  }
  __syncthreads();
  if (tid < 64) {  // one wave: lane st < kStreams holds stream st
    const float ms = tid < kStreams ? m_lds[tid] : -__builtin_inff();
    float M = ms;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float w = ms == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
    float total = tid < kStreams ? w * s_lds[tid] : 0.0f;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) total += __shfl_xor(total, off);
    if (tid < kStreams) w_lds[tid] = w;
    if (tid == 0) {
      total_lds = total;
      const int64_t orow = ((int64_t)b * a.seqlen_qo + s) * a.num_heads + head;
      if (a.lse && colblk == 0) a.lse[orow] = total > 0.0f ? (M + __log2f(total)) * kLn2 : -__builtin_inff();
    }
  }
  __syncthreads();
  const float total = total_lds;
  const float inv = total > 0.0f ? 1.0f / total : 0.0f;
  const int64_t orow = ((int64_t)b * a.seqlen_qo + s) * a.num_heads + head;
  if constexpr (CB < 256) {
    // R consecutive threads per column, each summing every R-th stream, then
    // shuffled together (a serial sum of all the streams per column would be
    // kStreams dependent LDS round trips)
    constexpr int R = 256 / CB;
    const int cc = tid / R, part = tid % R;
    float v = 0.0f;
#pragma unroll
    for (int st = part; st < kStreams; st += R) v += w_lds[st] * acc_lds[st][cc];
#pragma unroll
    for (int off = R / 2; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if (part == 0) a.out[orow * kLatentDim + colblk * CB + cc] = __builtin_bit_cast(uint16_t, (__bf16)(v * inv));
  } else {
    for (int cc = tid; cc < CB; cc += 256) {
      float v = 0.0f;
#pragma unroll 8
      for (int st = 0; st < kStreams; ++st) v += w_lds[st] * acc_lds[st][cc];
      a.out[orow * kLatentDim + colblk * CB + cc] = __builtin_bit_cast(uint16_t, (__bf16)(v * inv));
    }
  }
}

// One decode configuration: the template arguments of a kernel instance and
// FIT, the workgroups of it that one CU holds, which the planner uses as the
// occupancy of the persistent grid. FIT is checked against what the LDS
// footprint and the waves (WPE per SIMD, four SIMDs) allow.
template <bool FP8, int HW, int KW, int NS, int WPE, int KD, int VD, int QC, bool QF8, int FIT>
struct DecodeConfig {
  using Cfg = DecodeCfg<FP8, HW, KW, NS>;
  static constexpr int kLdsPerCu = 160 * 1024;
  static constexpr int kLdsFit = kLdsPerCu / Cfg::kLdsBytes;
  static constexpr int kWaveFit = 4 * WPE / (HW * KW);
  static_assert(FIT >= 1 && FIT == (kLdsFit < kWaveFit ? kLdsFit : kWaveFit),
                "the stated workgroups per CU are what the LDS and the waves allow");
  static constexpr int kFit = FIT;
  static int launch(const DecodeArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((mla_decode_kernel<FP8, HW, KW, NS, WPE, KD, VD, QC, QF8>), dim3(a.num_workgroups),
                       dim3(HW * KW * 64), 0, st, a);
    return (int)hipGetLastError();
  }
};

struct NoConfig {};

// The configuration of each (cache type, query type, tile class), for launches
// and for the planner's occupancy alike. Tile classes (head tiles HW x row
// slices KW, one wave per SIMD unless noted; stages = as many blocks as the LDS
// holds):
//   16 rows:  1 x 4 (fp8, 128-row blocks) or 1 x 2 (bf16, 64-row blocks)
//   32 rows:  2 x 2 (64-row blocks)
//   64 rows:  4 x 1 (fp8, 32-row blocks, two workgroups per CU) or 4 x 2 (bf16,
//             64-row blocks); two waves per SIMD of 256 registers each
//   128 rows: 8 x 1 (32-row blocks, two waves per SIMD, 256 registers each)
// Score sums are split over 4 accumulator chains where registers allow. For
// the two-waves-per-SIMD kernels, ring depths are the deepest that keep every
// register out of scratch inside the loop (measured: a single spill costs more
// than any ring depth gains). For fp8, KD counts 32-byte units (two reads).
template <typename F>
int dispatch_decode(int kv_dtype, bool q_fp8, int tile_class, F&& f) {
  const bool fp8 = kv_dtype == MLA_KV_FP8_E4M3FN;
  if (q_fp8) {  // fp8 query x fp8 cache: the fp8-cache configurations
    if (!fp8) return f(NoConfig{});
    switch (tile_class) {
      case 0: return f(DecodeConfig<true, 1, 4, 2, 1, 4, 8, 4, true, 1>{});
      case 1: return f(DecodeConfig<true, 2, 2, 4, 1, 4, 8, 4, true, 1>{});
      case 2: return f(DecodeConfig<true, 4, 1, 4, 2, 3, 3, 1, true, 2>{});
      case 3: return f(DecodeConfig<true, 8, 1, 8, 2, 3, 3, 1, true, 1>{});
    }
    return f(NoConfig{});
  }
  switch (tile_class) {
    case 0: return fp8 ? f(DecodeConfig<true, 1, 4, 2, 1, 4, 8, 4, false, 1>{})
                       : f(DecodeConfig<false, 1, 2, 2, 1, 8, 8, 4, false, 1>{});
    case 1: return fp8 ? f(DecodeConfig<true, 2, 2, 4, 1, 4, 8, 4, false, 1>{})
                       : f(DecodeConfig<false, 2, 2, 2, 1, 8, 8, 4, false, 1>{});
    case 2: return fp8 ? f(DecodeConfig<true, 4, 1, 4, 2, 3, 3, 1, false, 2>{})
                       : f(DecodeConfig<false, 4, 2, 2, 2, 3, 3, 2, false, 1>{});
    case 3: return fp8 ? f(DecodeConfig<true, 8, 1, 8, 2, 3, 3, 1, false, 1>{})
                       : f(DecodeConfig<false, 8, 1, 4, 2, 4, 3, 1, false, 1>{});
  }
  return f(NoConfig{});
}

}  // namespace

int launch_plan(const PlanArgs& a, void* stream) {
  hipLaunchKernelGGL(mla_plan_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int decode_wg_per_cu_fit(int kv_dtype, bool q_fp8, int tile_class) {
  return dispatch_decode(kv_dtype, q_fp8, tile_class, [](auto c) -> int {
    if constexpr (std::is_same_v<decltype(c), NoConfig>) {
      return 1;
    } else {
      return decltype(c)::kFit;
    }
  });
}

int launch_decode(const DecodeArgs& a, int kv_dtype, bool q_fp8, int tile_class, void* stream) {
  return dispatch_decode(kv_dtype, q_fp8, tile_class, [&](auto c) -> int {
    if constexpr (std::is_same_v<decltype(c), NoConfig>) {
      return (int)hipErrorInvalidValue;
    } else {
      return decltype(c)::launch(a, (hipStream_t)stream);
    }
  });
}

int launch_combine(const CombineArgs& a, int max_chunks, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  const int64_t row_count = (int64_t)a.batch * a.num_groups * a.rows_per_group;
  if (max_chunks <= 16) {
    const int64_t wgs = (row_count + 3) / 4;
    if (wgs > 0x7fffffff) return (int)hipErrorInvalidValue;
    if (max_chunks <= 8)
      hipLaunchKernelGGL(mla_combine_rows_kernel<8>, dim3((unsigned)wgs), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(mla_combine_rows_kernel<16>, dim3((unsigned)wgs), dim3(256), 0, st, a);
    return (int)hipGetLastError();
  }
  // Narrow column blocks when few rows carry long chunk lists; one grid dimension of
  // (rows x column blocks) workgroups.
  const int cb = row_count >= 1024 ? 512 : row_count >= 128 ? 128 : 16;
  const int64_t wgs = row_count * (kLatentDim / cb);
  if (wgs > 0x7fffffff) return (int)hipErrorInvalidValue;
  if (cb == 512) {
    hipLaunchKernelGGL(mla_combine_kernel<512>, dim3((unsigned)wgs), dim3(256), 0, st, a);
  } else if (cb == 128) {
    hipLaunchKernelGGL(mla_combine_kernel<128>, dim3((unsigned)wgs), dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL(mla_combine_kernel<16>, dim3((unsigned)wgs), dim3(256), 0, st, a);
  }
  return (int)hipGetLastError();
}

}  // namespace mla
