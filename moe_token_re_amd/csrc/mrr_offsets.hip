// mrr_offsets.hip -- the offsets phase of the MoE re-routing operator
// (MoeReRoutingV2): page "CANN ops-transformer MoeReRoutingV2", section
// "计算公式" (SrcOffset and DstOffset, the two double sums), "参数说明"
// (expert_token_num) and "约束说明" (Sum(counts) == A).
//
// Every kernel validates the counts, writes the status header and
// expert_token_num, and then what the gather kernel of the plan reads: the row
// map (the input row of every output row, one int32 per row) for the stream
// gather, or else a table of int32 pairs in output order (forward: cell
// j*N + i holds (dst_off, src_off); inverse: cell i*E + j holds (src_off,
// dst_off)) for the row-workgroup gather.
//   * offsets_regs_kernel (at most 64 cells): every wave computes the
//     offsets in its registers and writes 64 rows of the row map, with no
//     LDS and no barrier.
//   * offsets_small_kernel (at most 256 or 512 cells) and offsets_staged_kernel (at
//     most 1024): each workgroup stages the counts in LDS and scans them
//     row-major then column-major; workgroup 0 writes the header,
//     expert_token_num and any table, and every workgroup writes its slice of
//     the row map, one row per thread: each cell marks where its rows start
//     and a wave running maximum gives every row its cell.
//   * offsets_banded_kernel (up to 2^17 cells, E <= 1024): the ranks are cut
//     into bands; every workgroup sweeps the whole count matrix once for the
//     validity flags and the column totals, then scans its own band and,
//     split over a few workgroups per band, writes the row map cell by cell
//     (by a thread, a wave or the workgroups of the band, by cell size), or
//     its band's rows of the table.
//   * offsets_staged_kernel with chunks of cells per thread, and
//     offsets_global_kernel (one workgroup scanning through global memory):
//     the table for count matrices the others do not take.
#include <algorithm>
#include <mutex>

#include "mrr_device.h"

namespace mrr {
namespace {

constexpr int kOffsetItems = 4;  // counts per thread per tile (global path)
constexpr int kOffsetTile = kOffsetThreads * kOffsetItems;

// The same for larger matrices (kThreads < M <= kThreads * kC), with chunks of
// kC consecutive cells per thread (kC odd). lds holds two [E][NS] int32
// matrices, NS = N rounded up to odd: the counts (overwritten by DstOffset)
// and SrcOffset. Chunk loops are unrolled, so a thread's loads are all in
// flight together; a chunk walk along a column touches consecutive LDS words,
// and with kC and NS both odd the 64 lanes of a wave start in distinct banks.
template <int kThreads, int kC, typename CountT>
__device__ uint32_t offsets_chunks(const CountT* __restrict__ counts, int N, int E, int64_t A, int inverse,
                                   int32_t* lds, int32_t* col, pair_t* tab, ScanShared<kThreads>* sh,
                                   int64_t* total_out) {
  const int tid = threadIdx.x;
  const int M = N * E;
  const int NS = N | 1;
  int32_t* s_c = lds;           // [E][NS]: counts, then DstOffset
  int32_t* s_s = lds + E * NS;  // [E][NS]: SrcOffset
  if (tid == 0) sh->flags = 0;
  for (int j = tid; j <= E; j += kThreads) col[j] = 0;
  uint32_t flags = 0;
  const int m0 = tid * kC;

  // Stage the counts with coalesced loads, all in flight: cell m = i*E + j
  // (m = tid + k * kThreads) goes to s_c[j][i].
  {
    CountT raw[kC];
#pragma unroll
    for (int k = 0; k < kC; ++k) {
      const int m = tid + k * kThreads;
      raw[k] = counts[m < M ? m : M - 1];
    }
    int i = tid / E, j = tid - (tid / E) * E;
    const int di = kThreads / E, dj = kThreads - (kThreads / E) * E;
#pragma unroll
    for (int k = 0; k < kC; ++k) {
      if (tid + k * kThreads < M) s_c[j * NS + i] = clamp_count(raw[k], &flags);
      i += di;
      j += dj;
      const bool wrap = j >= E;
      j = wrap ? j - E : j;
      i += wrap ? 1 : 0;
    }
  }
  __syncthreads();

  // Pass 1: SrcOffset over my row-major chunk [m0, m0 + kC).
  uint64_t total;
  {
    int addr[kC];
    int i = m0 / E, j = m0 - (m0 / E) * E;
#pragma unroll
    for (int k = 0; k < kC; ++k) {
      addr[k] = m0 + k < M ? j * NS + i : 0;
      ++j;
      const bool wrap = j == E;
      j = wrap ? 0 : j;
      i += wrap ? 1 : 0;
    }
    uint32_t c[kC];
    uint32_t local = 0;
    uint64_t exact = 0;
#pragma unroll
    for (int k = 0; k < kC; ++k) {
      c[k] = m0 + k < M ? static_cast<uint32_t>(s_c[addr[k]]) : 0u;
      local += c[k];
      exact += c[k];
    }
    uint32_t run = block_scan_u32<kThreads, true>(local, exact, sh->w[0], sh->t[0], &total);
#pragma unroll
    for (int k = 0; k < kC; ++k) {
      if (m0 + k < M) s_s[addr[k]] = static_cast<int32_t>(run);
      run += c[k];
    }
  }
  *total_out = static_cast<int64_t>(total);
  flags = block_or(flags, &sh->flags);  // also orders pass 1's writes before pass 2's reads
  if (total != static_cast<uint64_t>(A)) flags |= kFlagSumMismatch;
  if (flags != 0) return flags;

  // Pass 2: DstOffset over my column-major chunk, in place of the counts.
  {
    int addr[kC];
    uint32_t c[kC];
    uint32_t top = 0;  // bit k: the chunk's k-th cell is rank 0 of its expert
    int j = m0 / N, i = m0 - (m0 / N) * N;
#pragma unroll
    for (int k = 0; k < kC; ++k) {
      addr[k] = m0 + k < M ? j * NS + i : 0;
      top |= (m0 + k < M && i == 0 ? 1u : 0u) << k;
      ++i;
      const bool wrap = i == N;
      i = wrap ? 0 : i;
      j += wrap ? 1 : 0;
    }
    uint32_t local = 0;
#pragma unroll
    for (int k = 0; k < kC; ++k) {
      c[k] = m0 + k < M ? static_cast<uint32_t>(s_c[addr[k]]) : 0u;
      local += c[k];
    }
    uint64_t unused;
    uint32_t run = block_scan_u32<kThreads, false>(local, 0, sh->w[1], sh->t[1], &unused);
#pragma unroll
    for (int k = 0; k < kC; ++k) {
      if (m0 + k < M) {
        s_c[addr[k]] = static_cast<int32_t>(run);
        if ((top >> k) & 1u) col[(m0 + k) / N] = static_cast<int32_t>(run);
      }
      run += c[k];
    }
  }
  __syncthreads();

  // The table, with coalesced stores, in output order: forward, cell m =
  // j*N + i; inverse, cell m = i*E + j with the pair's members swapped.
  if (inverse) {
    int i = tid / E, j = tid - (tid / E) * E;
    const int di = kThreads / E, dj = kThreads - (kThreads / E) * E;
#pragma unroll
    for (int k = 0; k < kC; ++k) {
      const int m = tid + k * kThreads;
      if (m < M) {
        pair_t t;
        t.x = s_s[j * NS + i];
        t.y = s_c[j * NS + i];
        tab[m] = t;
      }
      i += di;
      j += dj;
      const bool wrap = j >= E;
      j = wrap ? j - E : j;
      i += wrap ? 1 : 0;
    }
  } else {
    int j = tid / N, i = tid - (tid / N) * N;
    const int dj = kThreads / N, di = kThreads - (kThreads / N) * N;
#pragma unroll
    for (int k = 0; k < kC; ++k) {
      const int m = tid + k * kThreads;
      if (m < M) {
        pair_t t;
        t.x = s_c[j * NS + i];
        t.y = s_s[j * NS + i];
        tab[m] = t;
      }
      i += di;
      j += dj;
      const bool wrap = i >= N;
      i = wrap ? i - N : i;
      j += wrap ? 1 : 0;
    }
  }
  finish_offsets(tab, col, M, E, A);
  return 0;
}

// ---------------------------------------------------------------------------
// Offsets kernels
// ---------------------------------------------------------------------------

// kC == 1: one cell per thread (M <= kOffsetThreads); otherwise chunks of kC.
template <typename CountT, int kC>
__global__ __launch_bounds__(kOffsetThreads) void offsets_staged_kernel(
    const CountT* __restrict__ counts, int32_t N, int32_t E, int64_t A, int cumsum, int inverse,
    CountT* __restrict__ etn, WsHeader* __restrict__ hdr, pair_t* __restrict__ table, int32_t mats_ints,
    int32_t* __restrict__ rowmap) {
  extern __shared__ int32_t s_dyn[];
  __shared__ ScanShared<kOffsetThreads> sh;
  int32_t* col = s_dyn + mats_ints;  // [E + 1], after the offset matrices
  int64_t total = 0;
  uint32_t flags;
  // With a row map (one cell per thread only), workgroup b also writes the
  // row map's rows [1024 b, 1024 b + 1024); workgroup 0 alone writes
  // expert_token_num, the status and, without a row map, the table.
  const bool lead = blockIdx.x == 0;
  if (kC == 1)
    flags = offsets_cells<kOffsetThreads>(load_count(counts, N * E), N, E, A, inverse, s_dyn, col,
                                          lead && rowmap == nullptr ? table : nullptr, &sh, &total,
                                          rowmap, static_cast<int>(blockIdx.x) * kOffsetThreads,
                                          col + E + 1);  // row marks after col (the launch sizes them)
  else
    flags = offsets_chunks<kOffsetThreads, kC>(counts, N, E, A, inverse, s_dyn, col, table, &sh, &total);
  if (!lead) return;
  if (flags == 0) write_etn<kOffsetThreads>(col, E, cumsum, etn);
  if (threadIdx.x == 0) write_header(hdr, A, N, E, total, flags, kTablesValid, inverse);
}

// Offsets and the row map for count matrices of at most kT cells (kT = 256
// or 512): the same work as offsets_staged_kernel<CountT, 1> in workgroups of
// kT threads (shorter workgroup scans and barriers than its 1024), one per
// kT rows of the row map; workgroup 0 also writes expert_token_num and the
// status. No table: the gather that follows reads the row map only.
constexpr int kSmallCells = kSmallOffsetCells;

template <typename CountT, int kT>
__global__ __launch_bounds__(kT) void offsets_small_kernel(
    const CountT* __restrict__ counts, int32_t N, int32_t E, int64_t A, int cumsum, int inverse,
    CountT* __restrict__ etn, WsHeader* __restrict__ hdr, int32_t* __restrict__ rowmap) {
  __shared__ int32_t s_mats[2 * kT];
  __shared__ int32_t s_col[kT + 1];
  __shared__ ScanShared<kT> sh;
  __shared__ int32_t s_mark[kT];  // row marks
  const bool lead = blockIdx.x == 0;
  int64_t total = 0;
  const uint32_t flags =
      offsets_cells<kT>(load_count(counts, N * E), N, E, A, inverse, s_mats, s_col, nullptr, &sh, &total, rowmap,
                        static_cast<int>(blockIdx.x) * kT, s_mark);
  if (!lead) return;
  if (flags == 0) write_etn<kT>(s_col, E, cumsum, etn);
  if (threadIdx.x == 0) write_header(hdr, A, N, E, total, flags, kTablesValid, inverse);
}

// For count matrices too large for LDS: the same two scans in tiles of
// kOffsetTile cells, reading the counts from global memory (the column-major
// pass reads them transposed) and writing each pass's offsets straight into
// their slot of the table (output order; see the workspace layout).
template <typename CountT>
__global__ __launch_bounds__(kOffsetThreads) void offsets_global_kernel(
    const CountT* __restrict__ counts, int32_t N, int32_t E, int64_t A, int cumsum, int inverse,
    CountT* __restrict__ etn, WsHeader* __restrict__ hdr, int32_t* __restrict__ table) {
  __shared__ int64_t s_scan[2 * kOffsetThreads / 64 + 1];
  __shared__ uint32_t s_flags;
  const int tid = threadIdx.x;
  const int M = N * E;
  if (tid == 0) s_flags = 0;
  uint32_t flags = 0;

  // Pass 1: SrcOffset (row-major): forward, the second member of cell (i, j)'s
  // pair at j*N + i; inverse, the first member at i*E + j.
  int64_t carry = 0;
  for (int base = 0; base < M; base += kOffsetTile) {
    CountT raw[kOffsetItems];
#pragma unroll
    for (int k = 0; k < kOffsetItems; ++k) {
      const int m = base + tid * kOffsetItems + k;
      raw[k] = counts[m < M ? m : M - 1];
    }
    int32_t c[kOffsetItems];
    int64_t local = 0;
#pragma unroll
    for (int k = 0; k < kOffsetItems; ++k) {
      const int m = base + tid * kOffsetItems + k;
      c[k] = m < M ? clamp_count(raw[k], &flags) : 0;
      local += c[k];
    }
    int64_t tile_total;
    int64_t run = carry + block_exclusive_scan<kOffsetThreads>(local, s_scan, &tile_total);
#pragma unroll
    for (int k = 0; k < kOffsetItems; ++k) {
      const int m = base + tid * kOffsetItems + k;
      if (m < M) {
        const int i = m / E;
        const int j = m - i * E;
        table[inverse ? 2 * m : 2 * (j * N + i) + 1] = static_cast<int32_t>(run);
      }
      run += c[k];
    }
    carry += tile_total;
  }
  flags = block_or(flags, &s_flags);
  if (carry != A) flags |= kFlagSumMismatch;
  if (flags != 0) {
    if (tid == 0) write_header(hdr, A, N, E, carry, flags, kTablesValid, inverse);
    return;
  }

  // Pass 2: DstOffset (column-major): forward, the first member at j*N + i;
  // inverse, the second member at i*E + j.
  carry = 0;
  for (int base = 0; base < M; base += kOffsetTile) {
    CountT raw[kOffsetItems];
#pragma unroll
    for (int k = 0; k < kOffsetItems; ++k) {
      const int mc = base + tid * kOffsetItems + k;
      const int mcc = mc < M ? mc : M - 1;
      const int j = mcc / N;
      raw[k] = counts[(mcc - j * N) * E + j];
    }
    int32_t c[kOffsetItems];
    int64_t local = 0;
#pragma unroll
    for (int k = 0; k < kOffsetItems; ++k) {
      const int mc = base + tid * kOffsetItems + k;
      c[k] = mc < M ? clamp_count(raw[k], &flags) : 0;
      local += c[k];
    }
    int64_t tile_total;
    int64_t run = carry + block_exclusive_scan<kOffsetThreads>(local, s_scan, &tile_total);
#pragma unroll
    for (int k = 0; k < kOffsetItems; ++k) {
      const int mc = base + tid * kOffsetItems + k;
      if (mc < M) {
        const int j = mc / N;
        const int i = mc - j * N;
        table[inverse ? 2 * (i * E + j) + 1 : 2 * mc] = static_cast<int32_t>(run);
      }
      run += c[k];
    }
    carry += tile_total;
  }
  if (tid == 0) {  // the end entry, indexed in 64 bits (2 * M reaches 2^31 at the largest M)
    table[2 * int64_t(M)] = static_cast<int32_t>(A);
    table[2 * int64_t(M) + 1] = static_cast<int32_t>(A);
  }
  __threadfence_block();
  __syncthreads();

  // expert_token_num from the expert starts DstOffset(0, j) in the table.
  for (int j = tid; j < E; j += kOffsetThreads) {
    int64_t start, end;
    if (inverse) {
      start = N > 0 ? table[2 * j + 1] : 0;
      end = N > 0 && j + 1 < E ? table[2 * (j + 1) + 1] : A;
    } else {
      start = table[2 * int64_t(j * N)];
      end = table[2 * int64_t((j + 1) * N)];  // (j + 1) * N reaches M
    }
    etn[j] = static_cast<CountT>(cumsum ? end : end - start);
  }
  if (tid == 0) write_header(hdr, A, N, E, carry, 0, kTablesValid, inverse);
}

// Banded offsets for larger count matrices (kOffsetThreads < M, E <=
// kOffsetThreads): the workgroups of a band of ranks [i0, i0 + band_rows)
// write that band's share of the row map (or its table entries); no
// workgroup waits for another.
//  1. Every workgroup reads the whole count matrix (from L2 after the first
//     reader): thread t takes expert column j = t % E and every lanes-th rank
//     from t / E (lanes * E <= kOffsetThreads, a power of two), with all its
//     loads in flight together, and sums the column over all ranks (T_j) and
//     over the ranks above the band (B_j); the thread of column j then adds up
//     the lanes' sums from LDS. Reading every cell also tells each workgroup
//     whether the counts are valid. The band's own cells come from one more
//     load per thread, issued first.
//  2. Column scans: expert j's rows start at DstOffset(0, j) = sum of T_j'
//     over j' < j, and the band's first source offset is sum_j B_j. With at
//     most 64 experts, wave 0 alone does this.
//  3. The band's cells are scanned in row-major order for SrcOffset (after
//     sum_j B_j) and in column-major order for DstOffset: a cell of column j
//     gets DstOffset(0, j) + B_j plus the band's counts above it in its
//     column (the column-major scan minus its value at the column's first
//     band cell). These scans start before step 2 ends (they need only the
//     band's counts). Without a row map, each order's threads write their
//     half of the cell's (DstOffset, SrcOffset) pair.
//  4. With a row map, the workgroups of a band split its cells, taken in
//     output order: a group of threads (the workgroup's threads over its
//     cells, up to kBandCellRows) writes the rows of a cell of at most
//     kBandCellRows rows, a wave those of a cell of at most kOffsetThreads
//     rows, and every workgroup of the band its share of a larger cell's
//     rows.
// Every workgroup repeats step 1 over all M cells, which is why the per-cell
// work is kept to a few instructions, and why the L2 reads grow as
// M * (number of bands); the planner bounds M for this path.
constexpr int kBandCellRows = 16;  // row-map rows of a cell written by a group of threads; larger cells take a wave
constexpr int kBandUnroll = 16;  // count loads in flight per thread in step 1
constexpr int kBandFanIn = 16;   // lanes' sums a column's thread adds up; more take a first LDS pass

struct BandShared {
  uint64_t tot[kOffsetThreads];      // per-lane sums over all ranks,
  uint32_t bef[kOffsetThreads];      // and over the ranks above the band
  int32_t band[2 * kOffsetThreads];  // the band's counts, [rows][E | 1]
  int32_t col[kOffsetThreads + 1];   // DstOffset(0, j), col[E] = A
  uint32_t above[kOffsetThreads];    // B_j
  uint32_t cstart[kOffsetThreads];   // column-major band scan at each column's first band cell
  int32_t src_q[kOffsetThreads + 1]; // the band's cells by row-major index: SrcOffset (+ end),
  int32_t dst_q[kOffsetThreads];     // and DstOffset (for the row map)
  uint32_t w[4][kOffsetThreads / 64];
  uint64_t t[4][kOffsetThreads / 64];
  uint32_t flags;
  uint32_t above_all;
  uint64_t grand;
  int32_t mid[kOffsetThreads];  // the workgroup's cells of (kBandCellRows, kOffsetThreads] rows
  int32_t big[kOffsetThreads];  // and of more rows
  int32_t nmid;
  int32_t nbig;
};


// One count of the main sweep: the running sums, and what validity needs.
// int32 counts: the OR of the raw words keeps the sign bits (a negative
// count), and the 64-bit sum is exact. int64 counts are checked one by one.
template <typename CountT>
struct CountAcc {
  uint64_t tot = 0;
  uint32_t bef = 0;
  uint32_t orv = 0;
  uint32_t flags = 0;
  __device__ __forceinline__ void add(CountT raw, bool above) {
    uint32_t c;
    if (sizeof(CountT) == 4) {
      c = static_cast<uint32_t>(raw);
      orv |= c;
    } else {
      c = static_cast<uint32_t>(clamp_count(raw, &flags));
    }
    tot += c;
    bef += above ? c : 0u;
  }
  __device__ __forceinline__ uint32_t final_flags() const {
    return flags | ((orv >> 31) != 0 ? kFlagNegative : 0u);
  }
};

template <typename CountT>
__global__ __launch_bounds__(kOffsetThreads) void offsets_banded_kernel(
    const CountT* __restrict__ counts, int32_t N, int32_t E, int32_t band_rows, int32_t lanes, int64_t A,
    int cumsum, int inverse, CountT* __restrict__ etn, WsHeader* __restrict__ hdr, pair_t* __restrict__ table,
    int32_t* __restrict__ rowmap, int32_t split) {
  __shared__ BandShared s;
  const int tid = threadIdx.x;
  // `split` workgroups share a band: each computes its offsets and writes
  // 1/split of its rows' row map; without a row map, slice 0 writes the
  // band's table entries.
  const int band = blockIdx.x / split;
  const int slice = blockIdx.x - band * split;
  const int i0 = band * band_rows;
  const int rows = min(band_rows, N - i0);  // ranks in this band
  const int cells = rows * E;               // <= kOffsetThreads
  const int ES = E | 1;                     // LDS row stride of the band's counts
  const float inv_e = 1.0f / static_cast<float>(E);
  const float inv_rows = 1.0f / static_cast<float>(rows);
  if (tid == 0) {
    s.flags = 0;
    s.nmid = 0;
    s.nbig = 0;
  }

  // Step 1: per-lane column sums, and the band's counts.
  const int qi = div_small(tid, inv_e);  // row-major band cell q = tid: (qi, qj)
  const int qj = tid - qi * E;
  const CountT band_raw = counts[i0 * E + (tid < cells ? tid : cells - 1)];  // row-major: cell q of the band
  CountAcc<CountT> acc;
  {
    const int r = qi;  // lane r of column j = qj
    const int j = qj;
    if (r < lanes) {
      // Bounds and strides are uniform scalars and each thread walks one pointer: per-load
      // addresses of the form (ib + k * lanes) * E made the compiler use 64-bit multiply-adds
      // whose unused high half shares a register with band_raw's load, so the sweep waited for
      // that load before issuing its own.
      const int lim = N - (kBandUnroll - 1) * lanes;  // uniform
      const int stride = lanes * E;                    // uniform: elements between a thread's loads
      int ib = r;
      const CountT* p = counts + (j + r * E);          // M <= kBandMaxCells: 32-bit element offsets
      for (; ib < lim; ib += kBandUnroll * lanes, p += kBandUnroll * stride) {
        CountT raw[kBandUnroll];
#pragma unroll
        for (int k = 0; k < kBandUnroll; ++k) raw[k] = p[k * stride];
#pragma unroll
        for (int k = 0; k < kBandUnroll; ++k) acc.add(raw[k], ib + k * lanes < i0);
      }
      if (ib < N) {  // the last, partial chunk: clamped loads, predicated sums
        CountT raw[kBandUnroll];
#pragma unroll
        for (int k = 0; k < kBandUnroll; ++k) {
          const int i = ib + k * lanes;
          raw[k] = counts[j + (i < N ? i : N - 1) * E];
        }
#pragma unroll
        for (int k = 0; k < kBandUnroll; ++k)
          if (ib + k * lanes < N) acc.add(raw[k], ib + k * lanes < i0);
      }
      s.tot[tid] = acc.tot;
      s.bef[tid] = acc.bef;
    }
    uint32_t f = acc.final_flags();
    if (tid < cells) s.band[qi * ES + qj] = clamp_count(band_raw, &f);
    if (f != 0) atomicOr(&s.flags, f);
    __syncthreads();
    if (lanes > kBandFanIn) {  // uniform: fold lanes r + 16k into lane r < 16
      if (r < kBandFanIn) {
        uint64_t tot = s.tot[tid];
        uint32_t bef = s.bef[tid];
        for (int k = r + kBandFanIn; k < lanes; k += kBandFanIn) {
          tot += s.tot[k * E + j];
          bef += s.bef[k * E + j];
        }
        s.tot[tid] = tot;
        s.bef[tid] = bef;
      }
      __syncthreads();
    }
  }

  // Step 2: column scans and validity. A column total at or above 2^32
  // already rules the counts out; otherwise the 32-bit running sum over the
  // columns is exact unless it wraps, which shows as an inclusive value
  // below the exclusive one.
  const bool is_col = tid < E;
  uint64_t tot_j = 0;
  uint32_t bef_j = 0;
  if (is_col) {
    // all kBandFanIn reads issued before the sums (k < fan <= lanes keeps k * E + tid
    // below lanes * E <= kOffsetThreads; unused slots read lane 0's and add nothing)
    const int fan = lanes < kBandFanIn ? lanes : kBandFanIn;
    uint64_t t[kBandFanIn];
    uint32_t f[kBandFanIn];
#pragma unroll
    for (int k = 0; k < kBandFanIn; ++k) {
      const int kk = k < fan ? k : 0;
      t[k] = s.tot[kk * E + tid];
      f[k] = s.bef[kk * E + tid];
    }
#pragma unroll
    for (int k = 0; k < kBandFanIn; ++k) {
      tot_j += k < fan ? t[k] : 0;
      bef_j += k < fan ? f[k] : 0u;
    }
  }
  const uint32_t t32 = static_cast<uint32_t>(tot_j);
  if (E <= 64) {  // uniform: wave 0 holds every column
    if (tid < 64) {
      const uint32_t incl = wave_scan_u32(t32);
      const uint32_t excl = incl - t32;
      const bool bad = (tot_j >> 32) != 0 || incl < excl;
      const uint32_t above_all = __builtin_amdgcn_readlane(wave_scan_u32(bef_j), 63);
      const uint32_t grand = __builtin_amdgcn_readlane(incl, 63);
      const bool any_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
      if (is_col) {
        s.col[tid] = static_cast<int32_t>(excl);
        s.above[tid] = bef_j;
      }
      if (tid == 0) {
        if (any_bad || grand != static_cast<uint64_t>(A)) s.flags |= kFlagSumMismatch;
        s.col[E] = static_cast<int32_t>(A);
        s.above_all = above_all;
        s.grand = grand;
      }
    }
  } else {
    const uint64_t tot_c = tot_j < (uint64_t(1) << 32) ? tot_j : (uint64_t(1) << 32);
    uint32_t ex2[2];
    uint64_t sum2[2];
    block_scan_k<kOffsetThreads, 2, 3u>({t32, 0u}, {tot_c, bef_j}, ex2, sum2, s.w, s.t);
    if (is_col) {
      s.col[tid] = static_cast<int32_t>(ex2[0]);
      s.above[tid] = bef_j;
    }
    if (tid == 0) {
      s.col[E] = static_cast<int32_t>(A);
      s.above_all = static_cast<uint32_t>(sum2[1]);
      s.grand = sum2[0];
      if (sum2[0] != static_cast<uint64_t>(A)) atomicOr(&s.flags, kFlagSumMismatch);
    }
  }

  // Step 3: the band's cells in row-major (q = qi * E + qj) and column-major
  // (u = uj * rows + ui) order. These scans need only the band's counts, so
  // they start without waiting for step 2; their barrier also publishes step
  // 2's results and flags.
  const int uj = div_small(tid, inv_rows);
  const int ui = tid - uj * rows;
  const bool in = tid < cells;
  const uint32_t cq = in ? static_cast<uint32_t>(s.band[qi * ES + qj]) : 0u;
  const uint32_t cu = in ? static_cast<uint32_t>(s.band[ui * ES + uj]) : 0u;
  uint32_t ex3[2];
  uint64_t unused[2];
  block_scan_k<kOffsetThreads, 2, 0u>({cq, cu}, {0, 0}, ex3, unused, s.w + 2, s.t + 2);
  const uint32_t flags = s.flags;
  if (flags != 0) {  // uniform: every workgroup saw every count
    if (blockIdx.x == 0 && tid == 0)
      write_header(hdr, A, N, E, static_cast<int64_t>(s.grand), flags, kTablesValid, inverse);
    return;
  }
  if (in && ui == 0) s.cstart[uj] = ex3[1];
  __syncthreads();
  int32_t* words = reinterpret_cast<int32_t*>(table);
  // The table only for a gather that searches it (no row map); output order:
  // forward, cell j*N + i as (dst, src); inverse, cell i*E + j as (src, dst).
  if (in && slice == 0 && rowmap == nullptr) {
    const int32_t src = static_cast<int32_t>(s.above_all + ex3[0]);
    const int32_t dst =
        static_cast<int32_t>(static_cast<uint32_t>(s.col[uj]) + s.above[uj] + (ex3[1] - s.cstart[uj]));
    if (inverse) {
      words[2 * ((i0 + qi) * E + qj)] = src;
      words[2 * ((i0 + ui) * E + uj) + 1] = dst;
    } else {
      words[2 * (qj * N + i0 + qi) + 1] = src;
      words[2 * (uj * N + i0 + ui)] = dst;
    }
  }
  if (in) {
    s.src_q[tid] = static_cast<int32_t>(s.above_all + ex3[0]);
    s.dst_q[ui * E + uj] =
        static_cast<int32_t>(static_cast<uint32_t>(s.col[uj]) + s.above[uj] + (ex3[1] - s.cstart[uj]));
    if (tid == cells - 1) s.src_q[cells] = static_cast<int32_t>(s.above_all + ex3[0] + cq);  // the band's end
  }
  if (rowmap != nullptr) {
    // The row map for the band's cells: the workgroups of the band split its
    // cells; a group of threads writes the rows of a cell with at most
    // kBandCellRows rows, and the workgroup writes each larger cell's rows
    // together, strided over all its threads. Forward: output row DstOffset +
    // k takes source row SrcOffset + k; inverse: the reverse.
    __syncthreads();
    {
      // The slice's cells in output order (forward: column-major, so that
      // neighbouring cells' rows are neighbours in the row map), tpc threads
      // per cell (a power of two, the workgroup's threads over its cells):
      // thread sub of a cell writes its rows sub, sub + tpc, ...
      const int per = (cells + split - 1) / split;
      int tpc = 1;
      while (tpc < kBandCellRows && tpc * 2 * per <= kOffsetThreads) tpc *= 2;
      const int o = slice * per + tid / tpc;  // output-order index of the cell
      const int sub = tid & (tpc - 1);
      if (tid / tpc < per && o < cells) {
        const int oj = div_small(o, inv_rows);  // forward: o = oj * rows + oi
        const int q = inverse ? o : (o - oj * rows) * E + oj;
        const int sq = s.src_q[q], dq = s.dst_q[q], n = s.src_q[q + 1] - sq;
        if (n <= kBandCellRows) {
          for (int k = sub; k < n; k += tpc) {
            if (inverse)
              rowmap[sq + k] = dq + k;
            else
              rowmap[dq + k] = sq + k;
          }
        } else if (n <= kOffsetThreads && sub == 0) {
          s.mid[atomicAdd(&s.nmid, 1)] = q;
        }
      }
      // cells of more than kOffsetThreads rows: every workgroup of the band
      // takes its share of their rows
      if (tid < cells && s.src_q[tid + 1] - s.src_q[tid] > kOffsetThreads) s.big[atomicAdd(&s.nbig, 1)] = tid;
      __syncthreads();
      const int nmid = s.nmid;
      const int lane = tid & 63;
      for (int b = tid >> 6; b < nmid; b += kOffsetThreads / 64) {  // one wave per cell
        const int q2 = s.mid[b];
        const int sq = s.src_q[q2], dq = s.dst_q[q2], n = s.src_q[q2 + 1] - sq;
        for (int k = lane; k < n; k += 64) {
          if (inverse)
            rowmap[sq + k] = dq + k;
          else
            rowmap[dq + k] = sq + k;
        }
      }
      const int nbig = s.nbig;
      for (int b = 0; b < nbig; ++b) {  // uniform
        const int q2 = s.big[b];
        const int sq = s.src_q[q2], dq = s.dst_q[q2], n = s.src_q[q2 + 1] - sq;
        const int share = (n + split - 1) / split;
        const int k1 = min(n, (slice + 1) * share);
        for (int k = slice * share + tid; k < k1; k += kOffsetThreads) {
          if (inverse)
            rowmap[sq + k] = dq + k;
          else
            rowmap[dq + k] = sq + k;
        }
      }
    }
  }
  if (blockIdx.x == 0) {
    write_etn<kOffsetThreads>(s.col, E, cumsum, etn);
    if (tid == 0) {
      pair_t t;
      t.x = static_cast<int32_t>(A);
      t.y = static_cast<int32_t>(A);
      if (rowmap == nullptr) table[N * E] = t;
      write_header(hdr, A, N, E, static_cast<int64_t>(s.grand), 0, kTablesValid, inverse);
    }
  }
}

// Offsets and the row map for count matrices of at most 64 cells, in
// registers: every wave computes the offsets itself (wave_offsets64) and maps
// its 64 output rows to their input rows with wave_map_row (the row map of a
// direction is the input-to-output map of the other), with no LDS and no
// barrier. Workgroups of 256 threads own 256 rows of the row map; wave 0 of
// workgroup 0 also writes expert_token_num and the status.
template <typename CountT>
__global__ __launch_bounds__(256) void offsets_regs_kernel(
    const CountT* __restrict__ counts, int32_t N, int32_t E, int64_t A, int cumsum, int inverse,
    CountT* __restrict__ etn, WsHeader* __restrict__ hdr, int32_t* __restrict__ rowmap) {
  const int lane = threadIdx.x & 63;
  const bool lead = blockIdx.x == 0 && threadIdx.x < 64;
  WaveCells w;
  int64_t total = 0;
  const uint32_t flags = wave_offsets64<CountT>(load_count64(counts, N * E), N, E, A, &w, &total);
  if (flags != 0) {  // the same in every wave: no row map
    if (lead && lane == 0) write_header(hdr, A, N, E, total, flags, kTablesValid, inverse);
    return;
  }
  const int M = N * E;
  const int64_t d = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int32_t v = wave_map_row(w, M, inverse ? 0 : 1, d < A ? static_cast<int32_t>(d) : 0);
  if (d < A) rowmap[d] = v;
  if (lead) {
    // expert j starts at the DstOffset of column-major cell j * N (rank 0)
    for (int j0 = 0; j0 < E; j0 += 64) {
      const int j = j0 + lane;
      const int32_t cs = __shfl(static_cast<int>(w.dst_cm), j < E ? j * N : 0);
      const int32_t cs1 = __shfl(static_cast<int>(w.dst_cm), j + 1 < E ? (j + 1) * N : 0);
      const int32_t next = j + 1 < E ? cs1 : static_cast<int32_t>(A);
      if (j < E) etn[j] = static_cast<CountT>(cumsum ? next : next - cs);
    }
    if (lane == 0) write_header(hdr, A, N, E, total, 0, kTablesValid, inverse);
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

// Chunk lengths of the single-workgroup offsets kernel (1: one cell per
// thread); the launcher takes the smallest that covers the count matrix.
constexpr int kChunkSizes[] = {1, 3, 5, 9, 17};

template <typename CountT>
const void* staged_kernel_fn(int kc) {
  switch (kc) {
    case 1: return reinterpret_cast<const void*>(&offsets_staged_kernel<CountT, 1>);
    case 3: return reinterpret_cast<const void*>(&offsets_staged_kernel<CountT, 3>);
    case 5: return reinterpret_cast<const void*>(&offsets_staged_kernel<CountT, 5>);
    case 9: return reinterpret_cast<const void*>(&offsets_staged_kernel<CountT, 9>);
    default: return reinterpret_cast<const void*>(&offsets_staged_kernel<CountT, 17>);
  }
}

// Per-device facts, read once per device.
struct DeviceInfo {
  int lds_limit = 0;  // dynamic LDS the staged offsets kernel may take
};

constexpr int kMaxDevices = 64;
constexpr int kStaticLdsReserve = 1024;  // the offsets kernels' own static LDS, rounded up
std::once_flag g_dev_once[kMaxDevices];
DeviceInfo g_dev[kMaxDevices];

mrr_status device_info(const DeviceInfo** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MRR_ERROR_HIP;
  std::call_once(g_dev_once[dev], [&] {
    // Up to 64 KiB needs no opt-in; gfx950 lets one workgroup opt in to up
    // to 160 KiB.
    int optin = 0;
    if (hipDeviceGetAttribute(&optin, hipDeviceAttributeSharedMemPerBlockOptin, dev) != hipSuccess) optin = 0;
    int plain = 0;
    if (hipDeviceGetAttribute(&plain, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) plain = 0;
    int limit = (plain < 65536 ? plain : 65536) - kStaticLdsReserve;
    const int want = optin - kStaticLdsReserve;
    if (want > limit) {
      bool ok = true;
      for (int kc : kChunkSizes) {
        ok = ok && hipFuncSetAttribute(staged_kernel_fn<int32_t>(kc), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       want) == hipSuccess;
        ok = ok && hipFuncSetAttribute(staged_kernel_fn<int64_t>(kc), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       want) == hipSuccess;
      }
      if (ok) limit = want;
    }
    (void)hipGetLastError();  // a refused opt-in only keeps the smaller limit
    g_dev[dev].lds_limit = limit > 0 ? limit : 0;
  });
  *out = &g_dev[dev];
  return MRR_SUCCESS;
}

template <typename CountT, int kC>
void launch_staged(const Plan& pl, const mrr_args* a, uint8_t* base, size_t lds, hipStream_t stream) {
  const int32_t mats = static_cast<int32_t>((static_cast<int64_t>(lds) - 16) / 4 - (pl.E + 1));
  const unsigned grid =
      kC == 1 && pl.stream ? static_cast<unsigned>(std::max<int64_t>(1, (pl.A + kOffsetThreads - 1) / kOffsetThreads))
                           : 1u;
  // one cell per thread with a row map: the row marks after col
  const size_t dyn = lds + (kC == 1 && pl.stream ? 4 * static_cast<size_t>(kOffsetThreads) : 0);
  hipLaunchKernelGGL((offsets_staged_kernel<CountT, kC>), dim3(grid), dim3(kOffsetThreads), dyn, stream,
                     static_cast<const CountT*>(a->expert_token_num_per_rank), static_cast<int32_t>(pl.N),
                     static_cast<int32_t>(pl.E), pl.A, pl.cumsum ? 1 : 0, pl.inverse ? 1 : 0,
                     static_cast<CountT*>(a->expert_token_num), reinterpret_cast<WsHeader*>(base),
                     reinterpret_cast<pair_t*>(base + pl.table_bytes), mats,
                     pl.stream ? reinterpret_cast<int32_t*>(base + pl.rowmap_bytes) : nullptr);
}

template <typename CountT>
mrr_status launch_offsets_t(const Plan& pl, const mrr_args* a, void* ws, hipStream_t stream) {
  auto* base = static_cast<uint8_t*>(ws);
  if (pl.band_grid > 0) {
    hipLaunchKernelGGL((offsets_banded_kernel<CountT>), dim3(static_cast<unsigned>(pl.band_grid * pl.band_split)),
                       dim3(kOffsetThreads), 0, stream, static_cast<const CountT*>(a->expert_token_num_per_rank),
                       static_cast<int32_t>(pl.N), static_cast<int32_t>(pl.E), pl.band_rows, pl.band_lanes, pl.A,
                       pl.cumsum ? 1 : 0, pl.inverse ? 1 : 0, static_cast<CountT*>(a->expert_token_num),
                       reinterpret_cast<WsHeader*>(base), reinterpret_cast<pair_t*>(base + pl.table_bytes),
                       pl.stream ? reinterpret_cast<int32_t*>(base + pl.rowmap_bytes) : nullptr, pl.band_split);
    return hipGetLastError() == hipSuccess ? MRR_SUCCESS : MRR_ERROR_HIP;
  }
  if (pl.stream && pl.M <= 64) {
    const unsigned grid = static_cast<unsigned>(std::max<int64_t>(1, (pl.A + kSmallCells - 1) / kSmallCells));
    hipLaunchKernelGGL((offsets_regs_kernel<CountT>), dim3(grid), dim3(256), 0, stream,
                       static_cast<const CountT*>(a->expert_token_num_per_rank), static_cast<int32_t>(pl.N),
                       static_cast<int32_t>(pl.E), pl.A, pl.cumsum ? 1 : 0, pl.inverse ? 1 : 0,
                       static_cast<CountT*>(a->expert_token_num), reinterpret_cast<WsHeader*>(base),
                       reinterpret_cast<int32_t*>(base + pl.rowmap_bytes));
    return hipGetLastError() == hipSuccess ? MRR_SUCCESS : MRR_ERROR_HIP;
  }
  if (pl.stream && pl.M <= kSmallCells) {
    const unsigned grid = static_cast<unsigned>(std::max<int64_t>(1, (pl.A + kSmallCells - 1) / kSmallCells));
    hipLaunchKernelGGL((offsets_small_kernel<CountT, kSmallCells>), dim3(grid), dim3(kSmallCells), 0, stream,
                       static_cast<const CountT*>(a->expert_token_num_per_rank), static_cast<int32_t>(pl.N),
                       static_cast<int32_t>(pl.E), pl.A, pl.cumsum ? 1 : 0, pl.inverse ? 1 : 0,
                       static_cast<CountT*>(a->expert_token_num), reinterpret_cast<WsHeader*>(base),
                       reinterpret_cast<int32_t*>(base + pl.rowmap_bytes));
    return hipGetLastError() == hipSuccess ? MRR_SUCCESS : MRR_ERROR_HIP;
  }
  if (pl.stream && pl.M <= kMidOffsetCells) {
    const unsigned grid =
        static_cast<unsigned>(std::max<int64_t>(1, (pl.A + kMidOffsetCells - 1) / kMidOffsetCells));
    hipLaunchKernelGGL((offsets_small_kernel<CountT, kMidOffsetCells>), dim3(grid), dim3(kMidOffsetCells), 0, stream,
                       static_cast<const CountT*>(a->expert_token_num_per_rank), static_cast<int32_t>(pl.N),
                       static_cast<int32_t>(pl.E), pl.A, pl.cumsum ? 1 : 0, pl.inverse ? 1 : 0,
                       static_cast<CountT*>(a->expert_token_num), reinterpret_cast<WsHeader*>(base),
                       reinterpret_cast<int32_t*>(base + pl.rowmap_bytes));
    return hipGetLastError() == hipSuccess ? MRR_SUCCESS : MRR_ERROR_HIP;
  }
  const DeviceInfo* di = nullptr;
  if (device_info(&di) != MRR_SUCCESS) return MRR_ERROR_HIP;
  const int64_t lds = offsets_lds_bytes(pl.N, pl.E, kOffsetThreads);
  int kc = 0;
  for (int c : kChunkSizes)
    if (kc == 0 && int64_t(kOffsetThreads) * c >= pl.M) kc = c;
  if (kc != 0 && lds <= di->lds_limit) {
    const size_t l = static_cast<size_t>(lds);
    switch (kc) {
      case 1: launch_staged<CountT, 1>(pl, a, base, l, stream); break;
      case 3: launch_staged<CountT, 3>(pl, a, base, l, stream); break;
      case 5: launch_staged<CountT, 5>(pl, a, base, l, stream); break;
      case 9: launch_staged<CountT, 9>(pl, a, base, l, stream); break;
      default: launch_staged<CountT, 17>(pl, a, base, l, stream); break;
    }
  } else {
    hipLaunchKernelGGL((offsets_global_kernel<CountT>), dim3(1), dim3(kOffsetThreads), 0, stream,
                       static_cast<const CountT*>(a->expert_token_num_per_rank), static_cast<int32_t>(pl.N),
                       static_cast<int32_t>(pl.E), pl.A, pl.cumsum ? 1 : 0, pl.inverse ? 1 : 0,
                       static_cast<CountT*>(a->expert_token_num), reinterpret_cast<WsHeader*>(base),
                       reinterpret_cast<int32_t*>(base + pl.table_bytes));
  }
  return hipGetLastError() == hipSuccess ? MRR_SUCCESS : MRR_ERROR_HIP;
}

}  // namespace

mrr_status launch_offsets(const Plan& pl, const mrr_args* a, void* ws, hipStream_t stream) {
  return pl.count_bytes == 8 ? launch_offsets_t<int64_t>(pl, a, ws, stream)
                             : launch_offsets_t<int32_t>(pl, a, ws, stream);
}

}  // namespace mrr
