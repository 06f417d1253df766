// mrr_validate.cpp -- host-side argument checks, workspace sizing and launch
// planning of the MoE re-routing operator. This file includes no HIP header
// and makes no HIP call, so every check runs (and is tested) without a GPU.
//
// The contract checked here is the operator's (page "CANN ops-transformer
// MoeReRoutingV2", nlpx.cn article): the parameter table "参数说明" (dtypes,
// shapes, optional inputs, the pairing of expert_topk_weight and
// permute_topk_weight), "约束说明" (0 < H < 16384, Sum(counts) == A, the
// attributes) and the InferShape rules (output shapes follow the inputs).
// Count values live on the device and are checked there by the offsets kernel.
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>

#include "mrr_internal.h"

namespace {

using mrr::round_up;

constexpr int64_t kMaxCells = int64_t(1) << 30;
constexpr int64_t kMaxH = 16384;  // exclusive bound of the contract

int token_bits(int32_t dt) {
  switch (dt) {
    case MRR_F16:
    case MRR_BF16:
      return 16;
    case MRR_I8:
    case MRR_F8_E5M2:
    case MRR_F8_E4M3FN:
    case MRR_HIF8:
      return 8;
    case MRR_F4_E2M1:
    case MRR_F4_E1M2:
      return 4;
    default:
      return 0;
  }
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
  bool is_output;
};

bool overlaps(const Range& x, const Range& y) { return x.lo < y.hi && y.lo < x.hi; }

int env_int(const char* name, int fallback) {
  const char* s = getenv(name);
  if (s == nullptr || *s == '\0') return fallback;
  return atoi(s);
}

// Tuning overrides, read once per process. They change the launch shape only,
// never a result.
struct Tuning {
  int rows_per_wg;  // 0 = automatic
  int offsets;      // 0 = automatic, 1 = single-workgroup offsets kernel, 2 = banded where it applies
  int stream;       // 1 (default): the stream gather kernel for the two-kernel path; 0: row workgroups
  int band_split;   // 0 = automatic; else workgroups per band of the banded offsets kernel (1..16)
  bool fused;       // allow the single-kernel path (MRR_FUSED=0 turns it off)
  bool byte_rows;   // rows that are no multiple of 16 bytes stream as aligned 16-byte blocks
  bool stream_fused;  // allow the one-launch stream kernel (MRR_STREAM_FUSED=0 turns it off)
  int sf_bytes;       // its byte form: 0 off, 1 rows that are no multiple of 16 bytes, 2 (default) also
                      // rows of 16-byte vectors that are no multiple of 64 bytes (MRR_SF_BYTES)
  int sf_bytes16_min; // the shortest such row of 16-byte vectors it takes (MRR_SF_BYTES16_MIN)
  int sf_min_row;     // its smallest token row in bytes (MRR_SF_MIN_ROW, at least 32)
  int64_t sf_small;   // rows under 1 KiB: token bytes below which the fused kernel stays (MRR_SF_SMALL_KIB)
  bool log;
  Tuning()
      : rows_per_wg(env_int("MRR_ROWS_PER_WG", 0)),
        offsets(env_int("MRR_OFFSETS", 0)),
        stream(env_int("MRR_STREAM", 1)),
        band_split(env_int("MRR_BAND_SPLIT", 0)),
        fused(env_int("MRR_FUSED", 1) != 0),
        byte_rows(env_int("MRR_BYTE_ROWS", 1) != 0),
        stream_fused(env_int("MRR_STREAM_FUSED", 1) != 0),
        sf_bytes(env_int("MRR_SF_BYTES", 2)),
        sf_bytes16_min(env_int("MRR_SF_BYTES16_MIN", 1000)),
        sf_min_row(std::max(32, env_int("MRR_SF_MIN_ROW", 32))),
        sf_small(int64_t(1024) * env_int("MRR_SF_SMALL_KIB", static_cast<int>(mrr::kStreamFusedSmallRowMinBytes >> 10))),
        log(env_int("MRR_LOG", 0) != 0) {}
};

const Tuning& tuning() {
  static const Tuning t;
  return t;
}

int widest_vec(int64_t bytes, const void* a, const void* b) {
  for (int v = 16; v > 1; v /= 2)
    if (bytes % v == 0 && aligned(a, v) && aligned(b, v)) return v;
  return 1;
}

}  // namespace

extern "C" size_t mrr_workspace_size(int64_t A, int64_t N, int64_t E) {
  if (A < 0 || A > INT32_MAX || N < 0 || E < 0) return 0;
  if (N != 0 && E > kMaxCells / N) return 0;
  const size_t M = static_cast<size_t>(N * E);
  return mrr::kHeaderBytes + round_up(8 * (M + 1), 256) + round_up(4 * static_cast<size_t>(A), 256);
}

#ifndef MRR_SOURCE_HASH
#define MRR_SOURCE_HASH "unknown"
#endif

extern "C" const char* mrr_source_hash(void) { return MRR_SOURCE_HASH; }

extern "C" const char* mrr_status_string(mrr_status s) {
  switch (s) {
    case MRR_SUCCESS: return "MRR_SUCCESS";
    case MRR_ERROR_INVALID_VALUE: return "MRR_ERROR_INVALID_VALUE";
    case MRR_ERROR_INVALID_SHAPE: return "MRR_ERROR_INVALID_SHAPE";
    case MRR_ERROR_UNSUPPORTED_DTYPE: return "MRR_ERROR_UNSUPPORTED_DTYPE";
    case MRR_ERROR_MISALIGNED: return "MRR_ERROR_MISALIGNED";
    case MRR_ERROR_WORKSPACE_TOO_SMALL: return "MRR_ERROR_WORKSPACE_TOO_SMALL";
    case MRR_ERROR_BAD_COUNTS: return "MRR_ERROR_BAD_COUNTS";
    case MRR_ERROR_HIP: return "MRR_ERROR_HIP";
  }
  return "MRR_ERROR_UNKNOWN";
}

namespace mrr {

mrr_status make_plan(const mrr_args* a, const void* ws, size_t ws_bytes, Plan* p) {
  if (a == nullptr || p == nullptr) return MRR_ERROR_INVALID_VALUE;

  // dtypes (parameter table and the REG_OP prototype)
  const int bits = token_bits(a->tokens_dtype);
  if (bits == 0) return MRR_ERROR_UNSUPPORTED_DTYPE;
  if (a->counts_dtype != MRR_I32 && a->counts_dtype != MRR_I64) return MRR_ERROR_UNSUPPORTED_DTYPE;
  const int cb = a->counts_dtype == MRR_I64 ? 8 : 4;

  // attributes
  if (a->expert_token_num_type != 0 && a->expert_token_num_type != 1) return MRR_ERROR_INVALID_VALUE;
  if (a->idx_type != 0 && a->idx_type != 1) return MRR_ERROR_INVALID_VALUE;
  if (a->direction != MRR_FORWARD && a->direction != MRR_INVERSE) return MRR_ERROR_INVALID_VALUE;

  // shapes ("约束说明": 0 < H < 16384; Sum(counts) == A, with int32 indices)
  if (a->A < 0 || a->A > INT32_MAX) return MRR_ERROR_INVALID_SHAPE;
  if (a->H <= 0 || a->H >= kMaxH) return MRR_ERROR_INVALID_SHAPE;
  if (bits == 4 && (a->H % 2) != 0) return MRR_ERROR_INVALID_SHAPE;
  if (a->N < 0 || a->E < 0) return MRR_ERROR_INVALID_SHAPE;
  if (a->N != 0 && a->E > kMaxCells / a->N) return MRR_ERROR_INVALID_SHAPE;
  const int64_t M = a->N * a->E;
  if (M == 0 && a->A != 0) return MRR_ERROR_INVALID_SHAPE;
  const int64_t R = a->H * bits / 8;

  // optional scales: [A] f32, [A, S] f32, or [A, ceil(H/64), 2] e8m0
  int64_t Rs = 0;
  if (a->per_token_scales != nullptr) {
    if (a->scales_dtype == MRR_F32) {
      if (a->scales_ndim == 1) {
        if (a->scales_dims[0] != a->A) return MRR_ERROR_INVALID_SHAPE;
        Rs = 4;
      } else if (a->scales_ndim == 2) {
        if (a->scales_dims[0] != a->A || a->scales_dims[1] < 1 || a->scales_dims[1] > (1 << 24))
          return MRR_ERROR_INVALID_SHAPE;
        Rs = 4 * a->scales_dims[1];
      } else {
        return MRR_ERROR_INVALID_SHAPE;
      }
    } else if (a->scales_dtype == MRR_F8_E8M0) {
      if (a->scales_ndim != 3 || a->scales_dims[0] != a->A || a->scales_dims[1] != (a->H + 63) / 64 ||
          a->scales_dims[2] != 2)
        return MRR_ERROR_INVALID_SHAPE;
      Rs = 2 * a->scales_dims[1];
    } else {
      return MRR_ERROR_UNSUPPORTED_DTYPE;
    }
    if (a->A > 0 && a->permute_per_token_scales == nullptr) return MRR_ERROR_INVALID_VALUE;
  }

  // expert_topk_weight and permute_topk_weight come together or not at all
  const bool has_w = a->expert_topk_weight != nullptr;
  if (has_w != (a->permute_topk_weight != nullptr)) return MRR_ERROR_INVALID_VALUE;

  // required pointers
  if (ws == nullptr) return MRR_ERROR_INVALID_VALUE;
  if (a->A > 0 && (a->tokens == nullptr || a->permute_tokens == nullptr || a->permute_token_idx == nullptr))
    return MRR_ERROR_INVALID_VALUE;
  if (M > 0 && a->expert_token_num_per_rank == nullptr) return MRR_ERROR_INVALID_VALUE;
  if (a->E > 0 && a->expert_token_num == nullptr) return MRR_ERROR_INVALID_VALUE;

  // alignment of typed elements
  if (!aligned(ws, 16)) return MRR_ERROR_MISALIGNED;
  if (!aligned(a->expert_token_num_per_rank, cb) || !aligned(a->expert_token_num, cb)) return MRR_ERROR_MISALIGNED;
  if (!aligned(a->permute_token_idx, 4)) return MRR_ERROR_MISALIGNED;
  if (has_w && (!aligned(a->expert_topk_weight, 4) || !aligned(a->permute_topk_weight, 4)))
    return MRR_ERROR_MISALIGNED;
  if (Rs > 0 && a->scales_dtype == MRR_F32 &&
      (!aligned(a->per_token_scales, 4) || !aligned(a->permute_per_token_scales, 4)))
    return MRR_ERROR_MISALIGNED;

  // workspace size
  const size_t need = mrr_workspace_size(a->A, a->N, a->E);
  if (need == 0 || ws_bytes < need) return MRR_ERROR_WORKSPACE_TOO_SMALL;

  // no output may overlap any other buffer
  Range r[10];
  int nr = 0;
  auto add = [&](const void* ptr, int64_t bytes, bool out) {
    if (ptr != nullptr && bytes > 0) {
      uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
      r[nr++] = Range{lo, lo + static_cast<uintptr_t>(bytes), out};
    }
  };
  add(a->tokens, a->A * R, false);
  add(a->expert_token_num_per_rank, M * cb, false);
  if (Rs > 0) add(a->per_token_scales, a->A * Rs, false);
  if (has_w) add(a->expert_topk_weight, a->A * 4, false);
  add(a->permute_tokens, a->A * R, true);
  if (Rs > 0) add(a->permute_per_token_scales, a->A * Rs, true);
  add(a->permute_token_idx, a->A * 4, true);
  add(a->expert_token_num, a->E * cb, true);
  if (has_w) add(a->permute_topk_weight, a->A * 4, true);
  add(ws, static_cast<int64_t>(need), true);
  for (int x = 0; x < nr; ++x)
    for (int y = x + 1; y < nr; ++y)
      if ((r[x].is_output || r[y].is_output) && overlaps(r[x], r[y])) return MRR_ERROR_INVALID_VALUE;

  // the launch plan
  Plan q{};
  q.A = a->A;
  q.N = a->N;
  q.E = a->E;
  q.M = M;
  q.row_bytes = R;
  q.token_vec = widest_vec(R, a->tokens, a->permute_tokens);
  q.vecs_per_row = R / q.token_vec;
  q.scale_row_bytes = Rs;
  q.scale_vec = Rs > 0 ? widest_vec(Rs, a->per_token_scales, a->permute_per_token_scales) : 1;
  q.count_bytes = cb;
  q.has_weight = has_w;
  q.scatter = a->idx_type == 1;
  q.inverse = a->direction == MRR_INVERSE;
  q.cumsum = a->expert_token_num_type == 0;
  int64_t rows = int64_t(kGatherThreads) * kGatherUnroll / q.vecs_per_row;
  if (tuning().rows_per_wg > 0) rows = tuning().rows_per_wg;
  q.rows_per_wg = static_cast<int>(std::min<int64_t>(std::max<int64_t>(rows, 1), kMaxRowsPerWg));
  q.grid = (q.A + q.rows_per_wg - 1) / q.rows_per_wg;
  q.scale_inline = 0;
  if (Rs > 0 && q.token_vec == 16) {
    if (q.scale_vec == 16 && q.rows_per_wg * (Rs / 16) <= kGatherThreads)
      q.scale_inline = 16;
    else if (q.scale_vec >= 4 && q.rows_per_wg * (Rs / 4) <= kGatherThreads)
      q.scale_inline = 4;
  }
  q.fused = tuning().fused && q.A > 0 && M <= kGatherThreads;
  q.band_grid = 0;
  q.band_rows = 0;
  q.band_lanes = 0;
  q.band_split = 1;
  const bool band_fits = M > 0 && q.E <= kOffsetThreads && M <= kBandMaxCells;
  if (band_fits && (tuning().offsets == 2 || (tuning().offsets == 0 && M > kOffsetThreads))) {
    q.band_rows = static_cast<int>(std::min<int64_t>(q.N, kOffsetThreads / q.E));
    int lanes = 1;
    while (lanes * 2 * q.E <= kOffsetThreads) lanes *= 2;
    q.band_lanes = lanes;
    q.band_grid = (q.N + q.band_rows - 1) / q.band_rows;
  }
  // The stream gather reads the row map, which the single-workgroup kernel
  // with one cell per thread and the banded kernel write.
  q.stream = tuning().stream != 0 && (q.band_grid > 0 || M <= kOffsetThreads);
  // With the row map, several workgroups per band, so that each writes about
  // one row per two threads (measured at 65536 rows in 16 bands: 8 workgroups
  // per band 0.26 us per call faster than 4, 16 no faster than 8).
  if (q.stream && q.band_grid > 0)
    q.band_split = static_cast<int>(
        std::min<int64_t>(16, std::max<int64_t>(1, 2 * q.A / (q.band_grid * kOffsetThreads))));
  if (q.stream && q.band_grid > 0 && tuning().band_split > 0)
    q.band_split = std::min(16, tuning().band_split);
  q.tok_chunks = q.sc_chunks = q.item_chunks = q.stream_grid = 0;
  q.byte_rows = false;
  q.fold_scales = false;
  if (q.stream) {
    q.byte_rows = tuning().byte_rows && q.token_vec < 16 && q.row_bytes >= 16 && aligned(a->tokens, 16) &&
                  aligned(a->permute_tokens, 16);
    q.tok_chunks = q.byte_rows ? (q.A * q.row_bytes + 1023) / 1024 : (q.A * q.vecs_per_row + 63) / 64;
    q.fold_scales = Rs == 4 && q.scale_vec == 4;
    q.sc_chunks = Rs > 0 && !q.fold_scales ? (q.A * (Rs / q.scale_vec) + 63) / 64 : 0;
    q.item_chunks = (q.A + kItemRows - 1) / kItemRows;
    q.stream_grid = q.tok_chunks + q.sc_chunks + q.item_chunks;
    if (q.stream_grid >= kMaxStreamGrid) q.stream = false;  // 32-bit chunk numbers and grid
  }
  // The single-kernel path saves a launch; the two-kernel path's stream
  // gather streams faster. The launch matters less than the rate from a few
  // tens of MiB of rows on.
  if (q.fused && q.stream && q.A * q.row_bytes >= (M <= 64 ? kFusedMaxTokenBytesFewCells : kFusedMaxTokenBytes))
    q.fused = false;
  if (q.fused && q.byte_rows && q.A * q.row_bytes >= kFusedMaxByteRowBytes) q.fused = false;
  // The single kernel is one launch: never more workgroups than a launch holds.
  if (q.fused && q.grid > max_launch_grid(kGatherThreads)) q.fused = false;
  // The one-launch stream kernel runs in place of both the fused kernel and
  // the two kernels whenever its shape fits: at most 512 cells, token rows of
  // 16-byte vectors (both buffers aligned) and at least 32 bytes, scale rows
  // of at most 4 KiB, A < 2^30 (its exact-sum check), fewer than 2^32 token
  // vectors in all, and one launch of at most 2^31 workgroups; rows under
  // 1 KiB leave calls of under 2 MiB of token rows to the fused kernel where
  // it applies. (16x16 counts with 7168-byte rows, whole call: 1.8 MiB 4.7
  // against 5.7 us for the fused kernel, 27 MiB 11.2 against 14.1, 46 MiB
  // 17.6 against 21.4; at 112 MiB 37 against 41 us for the two kernels.
  // 512-byte rows: 1 MiB 5.34 against 5.37, 16 MiB 8.33 against 10.73 (fused),
  // 131 MiB 43.5 against 50.0 (two kernels); 32-byte rows at 64 MiB 32.3
  // against 45.6; the 42-row tiny call 4.64 against 3.73 for the fused kernel.)
  // Rows that are no multiple of 16 bytes, and rows of 16-byte vectors from
  // 1000 bytes that are no multiple of 64, take the kernel's byte form: at
  // least 17 bytes and below 2^16 (its row division), both token buffers
  // 16-byte aligned, and fewer than 2^31 token bytes (32-bit byte offsets).
  // (Its waves write whole 64-byte pieces of the output where 16-byte vectors
  // of such rows would write parts of them from two waves. 16x16 counts,
  // whole call: 7184-byte rows, 112 MiB, 40.0 against 44.8 us; 1040-byte rows,
  // 64 MiB, 24.5 against 25.9; 1008-byte rows 24.6 against 25.9; below 1000
  // bytes the 16-byte vectors measured faster (720-byte rows 14.3 against
  // 14.7, 32-byte rows 18.1 against 18.9). Against the two kernels, rows that
  // are no multiple of 16 bytes: 7169-byte rows 40.5 against 46.0 us, 1000
  // bytes 25.0 against 28.8, 158 bytes (16 MiB) 10.0 against 13.2, 42 bytes
  // (32 MiB) 18.7 against 26.0.)
  q.stream_fused = false;
  q.sf_bytes = false;
  q.sf_item_waves = q.sf_grid = 0;
  q.sf_rows_per_lane = 1;
  q.sf_cells_per_lane = M > 256 ? 8 : 4;
  const bool sf_vec_rows = q.token_vec == 16 && q.row_bytes >= tuning().sf_min_row &&
                           q.A * (q.row_bytes / 16) < (int64_t(1) << 32);
  const bool sf_byte_rows = (q.row_bytes % 16 != 0 ? tuning().sf_bytes >= 1
                                                   : tuning().sf_bytes >= 2 && q.row_bytes % 64 != 0 &&
                                                         q.row_bytes >= tuning().sf_bytes16_min) &&
                            q.row_bytes >= 17 &&
                            q.row_bytes < 65536 && aligned(a->tokens, 16) && aligned(a->permute_tokens, 16) &&
                            q.A * q.row_bytes < (int64_t(1) << 31);
  if (tuning().stream_fused && q.A > 0 && M <= kStreamFusedMaxCells && (sf_vec_rows || sf_byte_rows) &&
      q.scale_row_bytes <= kStreamFusedMaxScaleRow && q.A < (int64_t(1) << 30)) {
    // item waves of 256 output rows (64 for scale rows of more than 16 bytes,
    // so that more waves carry their traffic)
    q.sf_rows_per_lane = q.scale_row_bytes > 16 ? 1 : 4;
    const int64_t waves = (q.A + 64 * q.sf_rows_per_lane - 1) / (64 * q.sf_rows_per_lane);
    // token waves: 1 KiB of the rows each
    const int64_t grid = waves + (q.A * q.row_bytes + 1023) / 1024;
    // Small calls of short rows stay with the fused kernel where it applies:
    // rows of 16-byte vectors under 1 KiB below 2 MiB of rows, rows that are
    // no multiple of 16 bytes (the fused kernel moves them in narrower
    // vectors) under 512 bytes below 256 KiB (there a wave's KiB spans
    // several cells and walks them one by one). (158-byte rows, 16x16 counts:
    // 0.11 MiB 8.5 against 6.7 us for the fused kernel, 0.23 MiB 5.5-6.4
    // against 6.2, 0.47 MiB 4.9-5.8 against 6.3; 1000-byte rows: 0.24 MiB 4.3
    // against 6.8, 0.5 MiB 4.6 against 6.9; 1001-byte rows, 4x4 counts, 15
    // rows: 4.1 against 6.1.)
    const bool small_fused =
        q.fused && (q.row_bytes % 16 != 0
                        ? q.row_bytes < 512 && q.A * q.row_bytes < kStreamFusedSmallByteRowMinBytes
                        : q.row_bytes < 1024 && q.A * q.row_bytes < tuning().sf_small);
    if (grid < kMaxStreamGrid && grid <= max_launch_grid(64) && !small_fused) {
      q.stream_fused = true;
      q.sf_bytes = sf_byte_rows;
      q.fused = false;
      q.sf_item_waves = waves;
      q.sf_grid = grid;
    }
  }
  q.gather_launches = q.A == 0 || q.fused ? (q.A == 0 ? 0 : 1)
                    : q.stream ? (q.stream_grid + max_launch_grid(64) - 1) / max_launch_grid(64)
                               : (q.grid + max_launch_grid(kGatherThreads) - 1) / max_launch_grid(kGatherThreads);
  q.table_bytes = kHeaderBytes;
  q.rowmap_bytes = kHeaderBytes + round_up(8 * (static_cast<size_t>(M) + 1), 256);
  *p = q;

  if (tuning().log)
    fprintf(stderr,
            "[mrr] A=%lld N=%lld E=%lld R=%lld vec=%d rows/wg=%d grid=%lld Rs=%lld svec=%d w=%d scatter=%d "
            "fused=%d bands=%lld\n",
            (long long)q.A, (long long)q.N, (long long)q.E, (long long)q.row_bytes, q.token_vec,
            q.rows_per_wg, (long long)q.grid, (long long)q.scale_row_bytes, q.scale_vec,
            (int)q.has_weight, (int)q.scatter, (int)q.fused, (long long)q.band_grid);
  return MRR_SUCCESS;
}

}  // namespace mrr

extern "C" mrr_status mrr_validate(const mrr_args* args, const void* workspace, size_t workspace_bytes) {
  mrr::Plan plan;
  return mrr::make_plan(args, workspace, workspace_bytes, &plan);
}

extern "C" mrr_status mrr_describe_plan(const mrr_args* args, const void* workspace, size_t workspace_bytes,
                                        mrr_plan_info* info) {
  if (info == nullptr) return MRR_ERROR_INVALID_VALUE;
  mrr::Plan plan;
  const mrr_status st = mrr::make_plan(args, workspace, workspace_bytes, &plan);
  if (st != MRR_SUCCESS) return st;
  info->fused = plan.fused ? 1 : plan.stream_fused ? 2 : 0;
  info->token_vec_bytes = (plan.byte_rows || plan.sf_bytes) && !plan.fused ? 16 : plan.token_vec;
  info->scale_vec_bytes = plan.scale_row_bytes > 0 ? plan.scale_vec : 0;
  info->rows_per_workgroup = plan.rows_per_wg;
  info->threads_per_workgroup = plan.fused || !plan.stream ? mrr::kGatherThreads : 64;
  info->gather_workgroups = plan.fused || !plan.stream ? plan.grid : plan.stream_grid;
  info->one_launch_workgroups = plan.fused ? plan.grid : plan.stream_fused ? plan.sf_grid : 0;
  info->token_row_bytes = plan.row_bytes;
  info->scale_row_bytes = plan.scale_row_bytes;
  info->scale_inline_bytes = plan.scale_inline;
  info->offsets_workgroups = plan.band_grid > 0 ? plan.band_grid * plan.band_split
                           : plan.M == 0 ? 0
                           : !plan.stream ? 1
                           : plan.M <= mrr::kSmallOffsetCells
                               ? std::max<int64_t>(1, (plan.A + mrr::kSmallOffsetCells - 1) / mrr::kSmallOffsetCells)
                           : plan.M <= mrr::kMidOffsetCells
                               ? std::max<int64_t>(1, (plan.A + mrr::kMidOffsetCells - 1) / mrr::kMidOffsetCells)
                               : std::max<int64_t>(1, (plan.A + mrr::kOffsetThreads - 1) / mrr::kOffsetThreads);
  info->gather_kernel = plan.stream ? 1 : 0;
  info->gather_launches = plan.gather_launches;
  return MRR_SUCCESS;
}
