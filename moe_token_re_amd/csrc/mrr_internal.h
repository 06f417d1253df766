// mrr_internal.h -- shared between the host validation/planning code
// (mrr_validate.cpp, which includes no HIP header) and the kernels and
// launchers (mrr_kernels.hip). Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "moe_rerouting_v2.h"

namespace mrr {

// Workspace layout (all offsets from the workspace base):
//   [0, 256)                 WsHeader: validity of the counts the tables were built from
//   [256, 256 + T1)          dst_off[M + 1] int32, cells in column-major (expert, rank)
//                            order m = j*N + i; dst_off[M] = A
//   [256 + T1, 256 + T1+T2)  src_off[M] int32, same cell order
// with M = N*E, T1 = round_up(4*(M+1), 256), T2 = round_up(4*M, 256).
constexpr size_t kHeaderBytes = 256;
constexpr uint32_t kTablesValid = 0x4D525256u;  // "VRRM": tables valid for (A, N, E)
constexpr uint32_t kTablesBad = 0x4D525242u;    // "BRRM": the counts were rejected

// Flags the offsets kernel sets when it rejects the counts.
constexpr uint32_t kFlagNegative = 1u;      // some count < 0
constexpr uint32_t kFlagSumMismatch = 2u;   // sum of counts != A
constexpr uint32_t kFlagTooLarge = 4u;      // some count > INT32_MAX

struct WsHeader {
  uint32_t status;  // kTablesValid or kTablesBad; anything else: no tables yet
  uint32_t flags;
  int64_t A;
  int64_t N;
  int64_t E;
  int64_t total;    // sum of the counts, each clamped to [0, INT32_MAX]
};

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Threads of the gather kernel's workgroup and the number of 16-byte (or
// narrower) vectors each thread keeps in flight.
constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 8;
constexpr int kMaxRowsPerWg = 256;

// Everything the launchers need, derived on the host from mrr_args.
struct Plan {
  int64_t A, N, E, M;
  int64_t row_bytes;        // R: bytes of one token row
  int token_vec;            // bytes per access of the token copy: 16, 8, 4, 2 or 1
  int64_t vecs_per_row;     // R / token_vec
  int64_t scale_row_bytes;  // Rs, 0 when there is nothing to move
  int scale_vec;            // bytes per access of the scale copy
  int count_bytes;          // 4 or 8
  bool has_weight;
  bool scatter;             // idx_type == 1
  bool cumsum;              // expert_token_num_type == 0
  int rows_per_wg;
  int64_t grid;             // gather workgroups
  size_t dst_off_bytes;     // offset of dst_off in the workspace
  size_t src_off_bytes;     // offset of src_off in the workspace
};

// Host-only: fills `plan` from validated arguments. Returns MRR_SUCCESS or an error.
mrr_status make_plan(const mrr_args* args, const void* workspace, size_t workspace_bytes,
                     Plan* plan);

}  // namespace mrr
