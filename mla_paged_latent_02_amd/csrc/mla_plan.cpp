// Host half of the work planner: argument validation, the persistent grid, the
// chunk rule and the workspace layout. Pure integer arithmetic, no device work.
//
// Rule sources: "HK MLA: MI35x m16x8 retune, new m16x4 kernel, page_size +
// mask support" (Summary and file table: a persistent decode kernel whose
// device-built metadata is sized for num_cu clusters, doubled when the 64-row
// kernel runs at occupancy 2; heads x query tokens stacked into 64- or 128-row
// tiles) and "perf(mla): chunk the non-FP4 gather_kv_b_proj over KV"
// (description: a long context split over KV chunks so that the whole device
// streams; 12 programs on 256 CUs starve HBM).
#include <cmath>
#include <cstring>

#include <hip/hip_runtime_api.h>

#include "mla_internal.h"

namespace {

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
uint64_t align256(uint64_t x) { return (x + 255u) & ~uint64_t(255u); }

bool valid_options(const mla_plan_options_t& o) {
  for (int c = 0; c < 4; ++c) {
    if (o.wg_per_cu[c] < 1 || o.wg_per_cu[c] > 64) return false;
    if (o.chunk_min[c] < mla::kBlockRows || o.chunk_min[c] % mla::kBlockRows) return false;
    if (o.chunk_max[c] < o.chunk_min[c] || o.chunk_max[c] % mla::kBlockRows) return false;
  }
  if (o.force_chunk < 0 || o.force_chunk % mla::kBlockRows) return false;
  return true;
}

mla_status_t validate_params(const mla_decode_params_t& p) {
  if (p.batch < 1 || p.num_heads < 1 || p.page_size < 1) return MLA_ERR_INVALID_ARG;
  if (p.seqlen_qo < 1) return MLA_ERR_INVALID_ARG;
  if (p.seqlen_qo > mla::kMaxSeqlenQo) return MLA_ERR_UNSUPPORTED;
  if (p.max_context_len < p.seqlen_qo) return MLA_ERR_INVALID_ARG;
  if (p.causal != 0 && p.causal != 1) return MLA_ERR_INVALID_ARG;
  if (p.kv_dtype != MLA_KV_BF16 && p.kv_dtype != MLA_KV_FP8_E4M3FN) return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(p.softmax_scale) || p.softmax_scale == 0.0f) return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(p.kv_scale) || !(p.kv_scale > 0.0f)) return MLA_ERR_INVALID_ARG;
  if (p.kv_dtype == MLA_KV_BF16 && p.kv_scale != 1.0f) return MLA_ERR_INVALID_ARG;
  if (p.num_slots < 1 || p.num_slots % p.page_size) return MLA_ERR_INVALID_ARG;
  if (p.q_dtype != MLA_Q_BF16 && p.q_dtype != MLA_Q_FP8_E4M3FN) return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(p.q_scale) || !(p.q_scale > 0.0f)) return MLA_ERR_INVALID_ARG;
  if (p.q_dtype == MLA_Q_BF16 && p.q_scale != 1.0f) return MLA_ERR_INVALID_ARG;
  if (p.q_dtype == MLA_Q_FP8_E4M3FN && p.kv_dtype != MLA_KV_FP8_E4M3FN) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

}  // namespace

extern "C" {

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_status_string(mla_status_t s) {
  switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MLA_ERR_HIP: return "HIP runtime error";
    case MLA_ERR_BAD_PLAN: return "plan not made by mla_decode_plan";
    case MLA_ERR_SCRATCH_TOO_SMALL: return "the call needs more workspace than the static scratch holds";
  }
  return "unknown status";
}

void mla_plan_options_default(mla_plan_options_t* out) {
  if (!out) return;
  static const int32_t wg[4] = {1, 1, 2, 1};
  static const int32_t cmin[4] = {256, 256, 256, 64};
  static const int32_t cmax[4] = {8192, 8192, 4096, 6144};
  for (int c = 0; c < 4; ++c) {
    out->wg_per_cu[c] = wg[c];
    out->chunk_min[c] = cmin[c];
    out->chunk_max[c] = cmax[c];
  }
  out->force_chunk = 0;
}

mla_status_t mla_decode_plan_host(const mla_decode_params_t* params, const mla_plan_options_t* options,
                                  int32_t num_cu, mla_plan_t* out_plan) {
  if (!params || !out_plan) return MLA_ERR_INVALID_ARG;
  mla_status_t st = validate_params(*params);
  if (st != MLA_OK) return st;
  mla_plan_options_t opt;
  if (options) {
    opt = *options;
  } else {
    mla_plan_options_default(&opt);
  }
  if (!valid_options(opt)) return MLA_ERR_INVALID_ARG;
  if (num_cu <= 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return MLA_ERR_HIP;
    num_cu = n;
  }
  if (num_cu <= 0 || num_cu > 65536) return MLA_ERR_UNSUPPORTED;

  const mla_decode_params_t& p = *params;
  const int64_t B = p.batch, S = p.seqlen_qo, H = p.num_heads, L = p.max_context_len;
  const int64_t hpg = H < mla::kMaxTileRows / S ? H : mla::kMaxTileRows / S;
  const int64_t G = cdiv(H, hpg);
  const int64_t rows = hpg * S;
  int cls = 0;
  int64_t TR = 16;
  while (TR < rows) {
    TR *= 2;
    ++cls;
  }
  // the persistent grid: the requested workgroups per CU, capped at what the class's decode
  // kernel holds (its LDS and waves)
  const int32_t fit = mla::decode_wg_per_cu_fit(p.kv_dtype, p.q_dtype == MLA_Q_FP8_E4M3FN, cls);
  const int64_t occ = opt.wg_per_cu[cls] < fit ? opt.wg_per_cu[cls] : fit;
  const int64_t W = int64_t(num_cu) * occ;
  int64_t C;
  if (opt.force_chunk) {
    C = opt.force_chunk;
  } else {
    int64_t want = W / (B * G);
    if (want < 1) want = 1;
    C = cdiv(cdiv(L, want), mla::kBlockRows) * mla::kBlockRows;
    if (C < opt.chunk_min[cls]) C = opt.chunk_min[cls];
    if (C > opt.chunk_max[cls]) C = opt.chunk_max[cls];
  }
  const int64_t max_chunks = cdiv(L, C);
  // The device counts tasks (items x groups) and partial rows in 32 bits.
  if (B * max_chunks * G > 0x7fffffff || B * G * max_chunks * rows > 0x7fffffff || W > 0x7fffffff)
    return MLA_ERR_UNSUPPORTED;

  mla_plan_t plan;
  std::memset(&plan, 0, sizeof(plan));
  plan.magic = MLA_PLAN_MAGIC;
  plan.num_cu = num_cu;
  plan.params = p;
  plan.options = opt;
  plan.heads_per_group = int32_t(hpg);
  plan.num_groups = int32_t(G);
  plan.rows_per_group = int32_t(rows);
  plan.tile_rows = int32_t(TR);
  plan.tile_class = cls;
  plan.chunk_len = int32_t(C);
  plan.max_chunks = int32_t(max_chunks);
  plan.wg_per_cu = int32_t(occ);
  plan.num_workgroups = int32_t(W);
  plan.work_capacity = B * max_chunks;
  plan.partial_capacity_records = B * G * max_chunks;
  uint64_t off = 0;
  plan.ws_status_offset = off;
  off = align256(off + 16);
  plan.ws_nchunks_offset = off;
  off = align256(off + uint64_t(B) * 4);
  plan.ws_partbase_offset = off;
  off = align256(off + uint64_t(B) * 4);
  plan.ws_part_out_offset = off;
  off = align256(off + uint64_t(plan.partial_capacity_records) * uint64_t(rows) * mla::kLatentDim * 4);
  plan.ws_part_lse_offset = off;
  off = align256(off + uint64_t(plan.partial_capacity_records) * uint64_t(rows) * 4);
  plan.ws_work_offset = off;
  off = align256(off + uint64_t(plan.work_capacity) * mla::kItemWords * 4);
  plan.ws_bytes = off;
  *out_plan = plan;
  return MLA_OK;
}

size_t mla_decode_workspace_size(const mla_decode_params_t* params, const mla_plan_options_t* options,
                                 int32_t num_cu) {
  mla_plan_t plan;
  if (mla_decode_plan_host(params, options, num_cu, &plan) != MLA_OK) return 0;
  return size_t(plan.ws_bytes);
}

}  // extern "C"
