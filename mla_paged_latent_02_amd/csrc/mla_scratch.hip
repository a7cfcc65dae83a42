// The decode call for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// plan, decode and merge in one call, with the workspace in a file-scope
// device array of fixed size instead of a caller-provided buffer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mla_internal.h"

namespace {

// The workspace of every mla_decode_scratch call on a device: each device that
// loads this library holds its own copy until the process ends. In host code
// this name is only a stand-in for the device array, never its address: the
// address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) uint8_t scratch[MLA_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device with
// that device current (each device holds its own copy at its own address).
mla_status_t scratch_for_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MLA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status_t mla_decode_scratch(const mla_decode_params_t* params, const mla_plan_options_t* options, int32_t num_cu,
                                const void* d_q, const void* d_kv_cache, const int32_t* d_kv_indptr,
                                const int32_t* d_kv_page_indices, const int32_t* d_context_lens, void* d_out,
                                float* d_lse, void* stream, mla_plan_t* out_plan) {
  if (!params || !d_q || !d_kv_cache || !d_kv_indptr || !d_kv_page_indices || !d_context_lens || !d_out)
    return MLA_ERR_INVALID_ARG;
  // the host half first: its size check rejects an oversized call before any device work
  mla_plan_t plan;
  mla_status_t st = mla_decode_plan_host(params, options, num_cu, &plan);
  if (st != MLA_OK) return st;
  if (plan.ws_bytes > MLA_SCRATCH_BYTES) return MLA_ERR_SCRATCH_TOO_SMALL;
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != MLA_OK) return st;
  // the planner writes every array and status word the decode reads (the task counter
  // included), so nothing left by an earlier call needs clearing
  st = mla_decode_plan(params, options, plan.num_cu, d_context_lens, d_kv_indptr, ws, MLA_SCRATCH_BYTES, stream,
                       &plan);
  if (st != MLA_OK) return st;
  st = mla_decode(&plan, d_q, d_kv_cache, d_kv_indptr, d_kv_page_indices, d_context_lens, d_out, d_lse, ws,
                  MLA_SCRATCH_BYTES, stream);
  if (st != MLA_OK) return st;
  st = mla_split_combine(&plan, ws, MLA_SCRATCH_BYTES, d_out, d_lse, stream);
  if (st != MLA_OK) return st;
  if (out_plan) *out_plan = plan;
  return MLA_OK;
}

}  // extern "C"
