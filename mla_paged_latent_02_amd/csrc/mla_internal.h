// Internal declarations shared by the host planner, the C-ABI layer and the kernels.
#pragma once

#include <cstdint>

#include "mla_decode.h"

namespace mla {

constexpr int kRowDim = MLA_ROW_DIM;       // 576
constexpr int kLatentDim = MLA_LATENT_DIM; // 512
constexpr int kBlockRows = 64;             // chunks are multiples of this many cache rows
constexpr int kMaxTileRows = 128;
constexpr int kMaxSeqlenQo = MLA_MAX_SEQLEN_QO;
constexpr int kNumXcd = 8;                 // the hardware deals consecutive workgroups to 8 XCDs in turn
constexpr int kItemWords = 8;              // work item: b, chunk, ctx, page start, n_b, first record, 0, 0

// Everything one decode launch needs, passed by value.
struct DecodeArgs {
  const uint16_t* q;            // [B, S, H, 576]: bf16, or e4m3fn bytes (fp8 query)
  const uint8_t* cache;         // [num_slots, 576] elements of 2 (bf16) or 1 (fp8) bytes
  const int32_t* kv_indptr;     // [B+1]
  const int32_t* kv_page_indices;
  const int32_t* context_lens;  // [B]
  const int32_t* nchunks;       // [B] from the planner
  const int32_t* partbase;      // [B] from the planner
  const int32_t* work;          // [capacity][8] work items from the planner
  uint32_t* status;             // [0] status bits, [1] item count, [2] task counter, [3] finished workgroups
  uint16_t* out;                // bf16 [B, S, H, 512]
  float* lse;                   // [B, S, H] or null
  float* part_out;              // [records][rows][512]
  float* part_lse;              // [records][rows]
  int64_t num_pages;            // num_slots / page_size
  uint32_t page_div_magic;      // floor((2^32 - 1) / page_size): q = umulhi(n, magic), then one correction
  int32_t batch, seqlen_qo, num_heads, page_size;
  int32_t heads_per_group, num_groups, rows_per_group, chunk_len;
  int32_t num_workgroups;       // W: the persistent grid
  int32_t work_capacity;        // entries of the work list
  int32_t causal;
  float score_scale_log2;       // softmax_scale * kv_scale * q_scale * log2(e)
  float out_scale;              // kv_scale
};

struct CombineArgs {
  const int32_t* nchunks;
  const int32_t* partbase;
  const float* part_out;
  const float* part_lse;
  uint16_t* out;
  float* lse;
  int32_t batch, seqlen_qo, num_heads, heads_per_group, num_groups, rows_per_group;
};

struct PlanArgs {
  const int32_t* context_lens;
  const int32_t* kv_indptr;
  int32_t* nchunks;
  int32_t* partbase;
  int32_t* work;
  uint32_t* status;
  int32_t batch, seqlen_qo, max_context_len, page_size, chunk_len, num_groups, num_workgroups;
};

// Launchers (mla_kernels.hip). Return hipError_t as int.
int launch_plan(const PlanArgs& a, void* stream);
int launch_decode(const DecodeArgs& a, int kv_dtype, bool q_fp8, int tile_class, void* stream);
int launch_combine(const CombineArgs& a, int max_chunks, void* stream);

// Workgroups per CU that the decode kernel of this cache type, query type and
// tile class holds (its LDS and its waves): the occupancy the planner can ask for.
int decode_wg_per_cu_fit(int kv_dtype, bool q_fp8, int tile_class);

}  // namespace mla
