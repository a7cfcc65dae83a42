// extern "C" entry points: argument checks, then kernel launches on the caller's stream.
#include <cmath>
#include <cstring>

#include <hip/hip_runtime_api.h>

#include "mla_internal.h"

namespace {

bool plan_ok(const mla_plan_t* p) { return p && p->magic == MLA_PLAN_MAGIC; }

uint8_t* ws_at(void* ws, uint64_t off) { return static_cast<uint8_t*>(ws) + off; }

}  // namespace

extern "C" {

mla_status_t mla_decode_plan(const mla_decode_params_t* params, const mla_plan_options_t* options,
                             int32_t num_cu, const int32_t* d_context_lens, const int32_t* d_kv_indptr,
                             void* d_workspace, size_t workspace_bytes, void* stream, mla_plan_t* out_plan) {
  if (!params || !out_plan || !d_context_lens || !d_kv_indptr || !d_workspace) return MLA_ERR_INVALID_ARG;
  mla_plan_t plan;
  mla_status_t st = mla_decode_plan_host(params, options, num_cu, &plan);
  if (st != MLA_OK) return st;
  if (plan.params.num_slots >= (int64_t(1) << 31)) return MLA_ERR_UNSUPPORTED;
  if (workspace_bytes < plan.ws_bytes) return MLA_ERR_WORKSPACE_TOO_SMALL;
  mla::PlanArgs a;
  a.context_lens = d_context_lens;
  a.kv_indptr = d_kv_indptr;
  a.nchunks = reinterpret_cast<int32_t*>(ws_at(d_workspace, plan.ws_nchunks_offset));
  a.partbase = reinterpret_cast<int32_t*>(ws_at(d_workspace, plan.ws_partbase_offset));
  a.work = reinterpret_cast<int32_t*>(ws_at(d_workspace, plan.ws_work_offset));
  a.status = reinterpret_cast<uint32_t*>(ws_at(d_workspace, plan.ws_status_offset));
  a.batch = plan.params.batch;
  a.seqlen_qo = plan.params.seqlen_qo;
  a.max_context_len = plan.params.max_context_len;
  a.page_size = plan.params.page_size;
  a.chunk_len = plan.chunk_len;
  a.num_groups = plan.num_groups;
  a.num_workgroups = plan.num_workgroups;
  if (mla::launch_plan(a, stream) != 0) return MLA_ERR_HIP;
  *out_plan = plan;
  return MLA_OK;
}

mla_status_t mla_decode(const mla_plan_t* plan, const void* d_q, const void* d_kv_cache,
                        const int32_t* d_kv_indptr, const int32_t* d_kv_page_indices,
                        const int32_t* d_context_lens, void* d_out, float* d_lse, void* d_workspace,
                        size_t workspace_bytes, void* stream) {
  if (!plan_ok(plan)) return MLA_ERR_BAD_PLAN;
  if (!d_q || !d_kv_cache || !d_kv_indptr || !d_kv_page_indices || !d_context_lens || !d_out || !d_workspace)
    return MLA_ERR_INVALID_ARG;
  if (workspace_bytes < plan->ws_bytes) return MLA_ERR_WORKSPACE_TOO_SMALL;
  const mla_decode_params_t& p = plan->params;
  mla::DecodeArgs a;
  a.q = static_cast<const uint16_t*>(d_q);
  a.cache = static_cast<const uint8_t*>(d_kv_cache);
  a.kv_indptr = d_kv_indptr;
  a.kv_page_indices = d_kv_page_indices;
  a.context_lens = d_context_lens;
  a.nchunks = reinterpret_cast<const int32_t*>(ws_at(d_workspace, plan->ws_nchunks_offset));
  a.partbase = reinterpret_cast<const int32_t*>(ws_at(d_workspace, plan->ws_partbase_offset));
  a.work = reinterpret_cast<const int32_t*>(ws_at(d_workspace, plan->ws_work_offset));
  a.status = reinterpret_cast<uint32_t*>(ws_at(d_workspace, plan->ws_status_offset));
  a.out = static_cast<uint16_t*>(d_out);
  a.lse = d_lse;
  a.part_out = reinterpret_cast<float*>(ws_at(d_workspace, plan->ws_part_out_offset));
  a.part_lse = reinterpret_cast<float*>(ws_at(d_workspace, plan->ws_part_lse_offset));
  a.num_pages = p.num_slots / p.page_size;
  a.page_div_magic = uint32_t(0xFFFFFFFFull / uint64_t(p.page_size));
  a.batch = p.batch;
  a.seqlen_qo = p.seqlen_qo;
  a.num_heads = p.num_heads;
  a.page_size = p.page_size;
  a.heads_per_group = plan->heads_per_group;
  a.num_groups = plan->num_groups;
  a.rows_per_group = plan->rows_per_group;
  a.chunk_len = plan->chunk_len;
  a.num_workgroups = plan->num_workgroups;
  a.work_capacity = int32_t(plan->work_capacity);
  a.causal = p.causal;
  // both per-tensor scales multiply every score: folded into the softmax scale
  a.score_scale_log2 =
      float(double(p.softmax_scale) * double(p.kv_scale) * double(p.q_scale) * 1.4426950408889634);
  a.out_scale = p.kv_scale;
  if (mla::launch_decode(a, p.kv_dtype, p.q_dtype == MLA_Q_FP8_E4M3FN, plan->tile_class, stream) != 0)
    return MLA_ERR_HIP;
  return MLA_OK;
}

mla_status_t mla_split_combine(const mla_plan_t* plan, void* d_workspace, size_t workspace_bytes, void* d_out,
                               float* d_lse, void* stream) {
  if (!plan_ok(plan)) return MLA_ERR_BAD_PLAN;
  if (!d_workspace || !d_out) return MLA_ERR_INVALID_ARG;
  if (workspace_bytes < plan->ws_bytes) return MLA_ERR_WORKSPACE_TOO_SMALL;
  if (plan->max_chunks <= 1) return MLA_OK;  // no sequence can have been split
  mla::CombineArgs a;
  a.nchunks = reinterpret_cast<const int32_t*>(ws_at(d_workspace, plan->ws_nchunks_offset));
  a.partbase = reinterpret_cast<const int32_t*>(ws_at(d_workspace, plan->ws_partbase_offset));
  a.part_out = reinterpret_cast<const float*>(ws_at(d_workspace, plan->ws_part_out_offset));
  a.part_lse = reinterpret_cast<const float*>(ws_at(d_workspace, plan->ws_part_lse_offset));
  a.out = static_cast<uint16_t*>(d_out);
  a.lse = d_lse;
  a.batch = plan->params.batch;
  a.seqlen_qo = plan->params.seqlen_qo;
  a.num_heads = plan->params.num_heads;
  a.heads_per_group = plan->heads_per_group;
  a.num_groups = plan->num_groups;
  a.rows_per_group = plan->rows_per_group;
  if (mla::launch_combine(a, plan->max_chunks, stream) != 0) return MLA_ERR_HIP;
  return MLA_OK;
}

mla_status_t mla_debug_read_plan_arrays(const mla_plan_t* plan, const void* d_workspace, int32_t* h_nchunks,
                                        int32_t* h_partbase, uint32_t* h_status) {
  if (!plan_ok(plan)) return MLA_ERR_BAD_PLAN;
  if (!d_workspace) return MLA_ERR_INVALID_ARG;
  const uint8_t* ws = static_cast<const uint8_t*>(d_workspace);
  const size_t nb = size_t(plan->params.batch) * 4;
  if (hipDeviceSynchronize() != hipSuccess) return MLA_ERR_HIP;
  if (h_nchunks && hipMemcpy(h_nchunks, ws + plan->ws_nchunks_offset, nb, hipMemcpyDeviceToHost) != hipSuccess)
    return MLA_ERR_HIP;
  if (h_partbase && hipMemcpy(h_partbase, ws + plan->ws_partbase_offset, nb, hipMemcpyDeviceToHost) != hipSuccess)
    return MLA_ERR_HIP;
  if (h_status && hipMemcpy(h_status, ws + plan->ws_status_offset, 16, hipMemcpyDeviceToHost) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

mla_status_t mla_debug_read_work_list(const mla_plan_t* plan, const void* d_workspace, int32_t* h_count,
                                      int32_t* h_items) {
  if (!plan_ok(plan)) return MLA_ERR_BAD_PLAN;
  if (!d_workspace || !h_count) return MLA_ERR_INVALID_ARG;
  const uint8_t* ws = static_cast<const uint8_t*>(d_workspace);
  uint32_t words[2];
  if (hipDeviceSynchronize() != hipSuccess) return MLA_ERR_HIP;
  if (hipMemcpy(words, ws + plan->ws_status_offset, 8, hipMemcpyDeviceToHost) != hipSuccess) return MLA_ERR_HIP;
  if (int64_t(words[1]) > plan->work_capacity) return MLA_ERR_BAD_PLAN;
  *h_count = int32_t(words[1]);
  if (h_items && words[1] > 0 &&
      hipMemcpy(h_items, ws + plan->ws_work_offset, size_t(words[1]) * mla::kItemWords * 4, hipMemcpyDeviceToHost) !=
          hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

}  // extern "C"
