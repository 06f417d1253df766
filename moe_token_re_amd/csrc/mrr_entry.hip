// mrr_entry.hip -- the C entry points of the MoE re-routing operator
// (MoeReRoutingV2; page "CANN ops-transformer MoeReRoutingV2": the moves of
// "计算公式" with the inputs, outputs and attributes of "参数说明"). Each runs
// the host checks and planning of mrr_validate.cpp, then the launchers of the
// kernel files.
#include "mrr_device.h"

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

