// mrr_entry.hip -- the C entry points of the MoE re-routing operator
// (MoeReRoutingV2; page "CANN ops-transformer MoeReRoutingV2": the moves of
// "计算公式" with the inputs, outputs and attributes of "参数说明"). Each runs
// the host checks and planning of mrr_validate.cpp, then the launchers of the
// kernel files.
#include <atomic>
#include <mutex>

#include "mrr_device.h"

// The workspace of moe_rerouting_v2_noalloc(), for callers that cannot
// allocate: one copy per GPU, held until the process ends. In host code the
// name `scratch` is a host-side stand-in, not a device address: host code
// takes the address hipGetSymbolAddress gives for the current device and
// never passes the name itself to a kernel or a copy.
static __device__ __align__(256) uint8_t scratch[MRR_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch[kMaxScratchDevices];
std::mutex g_scratch_mu;

// The device address of the current device's copy of `scratch`, looked up on
// the first call on that device (with that device current) and kept.
mrr_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return MRR_ERROR_HIP;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MRR_ERROR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MRR_SUCCESS;
}

}  // namespace

extern "C" mrr_status moe_rerouting_v2_offsets(const mrr_args* args, void* workspace, size_t workspace_bytes,
                                               struct ihipStream_t* stream) {
  mrr::Plan plan;
  const mrr_status st = mrr::make_plan(args, workspace, workspace_bytes, &plan);
  if (st != MRR_SUCCESS) return st;
  return mrr::launch_offsets(plan, args, workspace, stream);
}

extern "C" mrr_status moe_rerouting_v2_gather(const mrr_args* args, void* workspace, size_t workspace_bytes,
                                              struct ihipStream_t* stream) {
  mrr::Plan plan;
  const mrr_status st = mrr::make_plan(args, workspace, workspace_bytes, &plan);
  if (st != MRR_SUCCESS) return st;
  return mrr::launch_gather(plan, args, workspace, stream);
}

extern "C" mrr_status moe_rerouting_v2(const mrr_args* args, void* workspace, size_t workspace_bytes,
                                       struct ihipStream_t* stream) {
  mrr::Plan plan;
  mrr_status st = mrr::make_plan(args, workspace, workspace_bytes, &plan);
  if (st != MRR_SUCCESS) return st;
  if (plan.fused) return mrr::launch_fused(plan, args, workspace, stream);
  if (plan.stream_fused) return mrr::launch_stream_fused(plan, args, workspace, stream);
  st = mrr::launch_offsets(plan, args, workspace, stream);
  if (st != MRR_SUCCESS) return st;
  return mrr::launch_gather(plan, args, workspace, stream);
}

extern "C" mrr_status mrr_get_device_status(const void* workspace, struct ihipStream_t* stream) {
  if (workspace == nullptr) return MRR_ERROR_INVALID_VALUE;
  mrr::WsHeader h{};
  if (hipMemcpyAsync(&h, workspace, sizeof(h), hipMemcpyDeviceToHost, stream) != hipSuccess) return MRR_ERROR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return MRR_ERROR_HIP;
  if (h.status == mrr::kTablesValid || h.status == mrr::kCountsValid) return MRR_SUCCESS;
  if (h.status == mrr::kTablesBad) return MRR_ERROR_BAD_COUNTS;
  return MRR_ERROR_INVALID_VALUE;
}


// The whole call with the library's own scratch as the workspace: the same
// checks, kernels and results as moe_rerouting_v2, with no allocation (the
// workspace needs no clearing: every kernel reads only what the offsets phase
// of the same call wrote, after checking the header it wrote).
extern "C" mrr_status moe_rerouting_v2_noalloc(const mrr_args* args, struct ihipStream_t* stream) {
  if (args == nullptr) return MRR_ERROR_INVALID_VALUE;
  const size_t need = mrr_workspace_size(args->A, args->N, args->E);  // 0 for shapes the checks refuse
  if (need > MRR_NOALLOC_SCRATCH_BYTES) return MRR_ERROR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  const mrr_status st = scratch_address(&ws);
  if (st != MRR_SUCCESS) return st;
  return moe_rerouting_v2(args, ws, MRR_NOALLOC_SCRATCH_BYTES, stream);
}
