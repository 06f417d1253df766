// mrr_internal.h -- shared between the host validation/planning code
// (mrr_validate.cpp, which includes no HIP header) and the kernels and
// launchers (the .hip files, through mrr_device.h). Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "moe_rerouting_v2.h"

namespace mrr {

// Workspace layout (all offsets from the workspace base):
//   [0, 256)              WsHeader: validity of the counts the table was built from
//   [256, 256 + T)        table[M + 1] of int32 pairs (output offset, input offset) in
//                         output order (written only when the gather searches it, i.e.
//                         without a row map), so that the first member is non-decreasing in m:
//                         forward: (DstOffset, SrcOffset) of cell m = j*N + i (column-major);
//                         inverse: (SrcOffset, DstOffset) of cell m = i*E + j (row-major);
//                         table[M] = (A, A)
//   [256 + T, ... + Rm)   rowmap[A] int32: the input row of every output row (written by
//                         the offsets kernels that can, see Plan::rowmap)
// with M = N*E, T = round_up(8*(M+1), 256) and Rm = round_up(4*A, 256). The
// gather kernels only see the table or the row map, so one kernel serves both
// directions.
constexpr size_t kHeaderBytes = 256;
constexpr uint32_t kTablesValid = 0x4D525256u;  // "VRRM": counts valid, table built for (A, N, E)
constexpr uint32_t kCountsValid = 0x4D525243u;  // "CRRM": counts valid, no table (single-kernel path)
constexpr uint32_t kTablesBad = 0x4D525242u;    // "BRRM": the counts were rejected

// Flags the offsets kernel sets when it rejects the counts.
constexpr uint32_t kFlagNegative = 1u;      // some count < 0
constexpr uint32_t kFlagSumMismatch = 2u;   // sum of counts != A
constexpr uint32_t kFlagTooLarge = 4u;      // some count > INT32_MAX

struct WsHeader {
  uint32_t status;  // kTablesValid or kTablesBad; anything else: no tables yet
  uint32_t flags;
  uint32_t inverse;  // the table's direction (1: inverse)
  uint32_t pad;
  int64_t A;
  int64_t N;
  int64_t E;
  int64_t total;    // sum of the counts (diagnostic only when the counts are rejected)
};

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Shape of the gather kernel's workgroups: threads, and vectors (16 bytes or
// narrower) each thread keeps in flight. A workgroup owns
// rows_per_wg = max(1, threads * unroll / vectors_per_row) adjacent output rows.
#ifndef MRR_GATHER_THREADS
#define MRR_GATHER_THREADS 256
#endif
#ifndef MRR_GATHER_UNROLL
#define MRR_GATHER_UNROLL 8
#endif
constexpr int kGatherThreads = MRR_GATHER_THREADS;

constexpr int kGatherUnroll = MRR_GATHER_UNROLL;
constexpr int kMaxRowsPerWg = 256;

// The offsets kernels run workgroups of kOffsetThreads threads. Count
// matrices with kOffsetThreads < M <= kBandMaxCells and E <= kOffsetThreads
// take the banded kernel: one workgroup per band of band_rows ranks, each of
// which reads the whole matrix once (so its L2 reads grow as M^2 /
// kOffsetThreads); the others take one workgroup.
constexpr int kOffsetThreads = 1024;
// Matrices of at most this many cells, when the row map is written, take
// workgroups of this many threads (one per that many rows).
constexpr int kSmallOffsetCells = 256;
constexpr int kMidOffsetCells = 512;  // 256 < N*E <= 512: the same kernel with 512 threads
constexpr int64_t kBandMaxCells = int64_t(1) << 17;

// The stream gather kernel has one workgroup per chunk and numbers chunks in
// 32 bits; calls with more chunks than this take the row-workgroup gather
// kernel instead.
constexpr int64_t kMaxStreamGrid = int64_t(1) << 31;

// The stream gather's per-row items (index, weight, and scale rows of one
// 4-byte word) move in chunks of kItemRows rows, four per lane.
constexpr int kItemRowsPerLane = 4;
constexpr int kItemRows = 64 * kItemRowsPerLane;

// A launch may hold at most 2^32 - 1 threads (grid x workgroup size), so a
// gather with more workgroups than that is launched in pieces, each taking
// the next workgroups in order.
constexpr int64_t kMaxLaunchThreads = (int64_t(1) << 32) - 1;
inline int64_t max_launch_grid(int64_t threads) { return kMaxLaunchThreads / threads; }

// Calls whose token rows total at least this many bytes take the two-kernel
// path (offsets, then the stream gather) even when the single-kernel path
// could run them (measured with 7168-byte rows: the single kernel is 1 us
// faster at 17 MB, 0.2 us at 36 MB, 1.1 us slower at 54 MB).
constexpr int64_t kFusedMaxTokenBytes = int64_t(48) << 20;
// The same for count matrices of at most 64 cells, whose two-kernel path has
// the cheaper register offsets kernel (8x8 counts, 7168-byte rows: the single
// kernel is 0.7 us faster at 16 MB, 0.3 us at 23 MB, 0.75 us slower at 32 MB).
constexpr int64_t kFusedMaxTokenBytesFewCells = int64_t(28) << 20;
// The same for rows the stream gather moves as aligned 16-byte blocks while
// the single kernel would move them in narrow vectors.
constexpr int64_t kFusedMaxByteRowBytes = int64_t(4) << 20;

// The one-launch stream kernel (count matrices of at most 512 cells, 4 or 8
// a lane, token rows of 16-byte vectors and at least 32 bytes, or rows of at
// least 17 bytes that are no multiple of 64 in its byte form): its item waves
// move 64 scale rows each, so scale rows are limited to this many bytes
// (larger ones take two kernels).
constexpr int kStreamFusedMaxCells = 512;
constexpr int64_t kStreamFusedMaxScaleRow = 4096;
// Below this many bytes of token rows, rows under 1 KiB stay with the fused
// kernel where it applies (it measured as fast or faster there).
constexpr int64_t kStreamFusedSmallRowMinBytes = int64_t(2) << 20;
// The same for byte-form rows under 512 bytes (its slow path walks the cells
// of a wave one by one): the fused kernel below this many bytes.
constexpr int64_t kStreamFusedSmallByteRowMinBytes = int64_t(256) << 10;

// Offsets computed in one workgroup's LDS (the single-workgroup offsets
// kernel, and every workgroup of the fused kernel) use one of two layouts:
//  * one cell per thread (M <= threads): counts and source offsets in
//    column-major cell order, [M] int32 each;
//  * chunks of cells per thread (M > threads): counts (overwritten by the
//    destination offsets) and source offsets as [E][NS] int32 matrices, the
//    column stride NS = N rounded up to odd so that lanes walking odd-length
//    chunks hit distinct LDS banks;
// plus the expert starts [E + 1]. 16 bytes of slack keep the first-cell reads
// of an empty matrix inside the allocation.
inline int64_t lds_col_stride(int64_t N) { return N | 1; }
inline int64_t offsets_lds_bytes(int64_t N, int64_t E, int64_t threads) {
  const int64_t M = N * E;
  const int64_t mats = M <= threads ? 2 * M : 2 * E * lds_col_stride(N);
  return 4 * (mats + E + 1) + 16;
}

// The whole call runs as one kernel (each gather workgroup recomputes the
// offsets in LDS, one cell per thread) when the count matrix has at most as
// many cells as a gather workgroup has threads.
inline int64_t fused_lds_bytes(int64_t N, int64_t E) {
  return 8 * (N * E + 1) + offsets_lds_bytes(N, E, MRR_GATHER_THREADS);
}

// Everything the launchers need, derived on the host from mrr_args.
struct Plan {
  int64_t A, N, E, M;
  int64_t row_bytes;        // R: bytes of one token row
  int token_vec;            // bytes per access of the token copy: 16, 8, 4, 2 or 1
  int64_t vecs_per_row;     // R / token_vec
  int64_t scale_row_bytes;  // Rs, 0 when there is nothing to move
  int scale_vec;            // bytes per access of the scale copy
  int scale_inline;         // 16 or 4: scale rows moved in pieces of that many bytes, at most one
                            // piece per thread, loaded together with the token rows; 0: a
                            // separate pass after the token rows
  int count_bytes;          // 4 or 8
  bool has_weight;
  bool scatter;             // idx_type == 1
  bool cumsum;              // expert_token_num_type == 0
  bool inverse;             // direction == MRR_INVERSE: the table in row-major cell order
  bool fused;               // moe_rerouting_v2 runs the single fused kernel
  bool stream_fused;        // moe_rerouting_v2 runs the one-launch stream kernel instead (64-lane
                            // workgroups: item waves of 256 (or 64) output rows, then one 1 KiB chunk of
                            // the input token rows each)
  int64_t sf_item_waves;    // its item waves: ceil(A / (64 sf_rows_per_lane))
  int sf_rows_per_lane;     // output rows per lane of an item wave: 4, or 1 for scale rows over 16 bytes
  int sf_cells_per_lane;    // cells of the count matrix per lane: 4 (at most 256 cells) or 8 (at most 512)
  int64_t sf_grid;          // its workgroups: item waves + ceil(A * R / 1024)
  bool sf_bytes;            // its byte form: rows that are no multiple of 64 bytes as one byte stream
  int rows_per_wg;
  int64_t grid;             // gather workgroups
  bool stream;              // the gather kernel is the stream kernel: 64-lane workgroups, one chunk of
                            // 64 vectors (token or scale rows) or 64 rows (items) each
  int64_t tok_chunks, sc_chunks, item_chunks;  // the stream kernel's chunks
  bool fold_scales;         // scale rows of one 4-byte word move with the items (no scale chunks)
  bool byte_rows;           // token rows stream as bytes in 1 KiB chunks of aligned 16-byte blocks
                            // (rows of 16 bytes or more that are no multiple of 16, both buffers
                            // 16-byte aligned)
  int64_t stream_grid;      // its workgroups: the total number of chunks
  int64_t gather_launches;  // launches of the gather phase (pieces of at most max_launch_grid)
  int64_t band_grid;        // banded offsets kernel: workgroups (bands); 0 = single-workgroup kernel
  int band_rows;            // ranks per band: min(N, kOffsetThreads / E)
  int band_lanes;           // threads per column in the banded kernel's first step (a power of two)
  int band_split;           // workgroups per band (they share the band's row map writes)
  size_t table_bytes;       // offset of the (dst_off, src_off) table in the workspace
  size_t rowmap_bytes;      // offset of the row map in the workspace
};

// Host-only: fills `plan` from validated arguments. Returns MRR_SUCCESS or an error.
mrr_status make_plan(const mrr_args* args, const void* workspace, size_t workspace_bytes,
                     Plan* plan);

}  // namespace mrr
