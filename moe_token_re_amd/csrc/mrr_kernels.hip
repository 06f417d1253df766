// mrr_kernels.hip -- HIP kernels and launchers of the MoE re-routing operator
// (MoeReRoutingV2) for MI355X (gfx950, CDNA4: 64-lane waves, 256 CUs).
//
// Page: "CANN ops-transformer MoeReRoutingV2" (nlpx.cn article).
//   offsets          -- section "计算公式", the two double sums: SrcOffset is the
//                       exclusive prefix of the count matrix in row-major (rank,
//                       expert) order, DstOffset in column-major (expert, rank)
//                       order; plus expert_token_num ("参数说明") and the
//                       Sum(counts) == A constraint ("约束说明").
//   row moves        -- section "计算公式", the moves
//                       permute_X[DstOffset + k] = X[SrcOffset + k] for tokens,
//                       per_token_scales and expert_topk_weight, and
//                       permute_token_idx ("参数说明"; gather or scatter form).
//
// Kernels (the design is ours, not the Ascend tiling the article sketches).
// Offsets phase: every kernel validates the counts, writes the status header
// and expert_token_num, and then what the gather kernel of the plan reads:
// the row map (the input row of every output row, one int32 per row) for the
// stream gather, or else a table of int32 pairs in output order (forward:
// cell j*N + i holds (dst_off, src_off); inverse: cell i*E + j holds
// (src_off, dst_off)) for the row-workgroup gather.
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
//   * offsets_global_kernel: one workgroup scans through global memory, for
//     count matrices too large for the others (no row map).
// Gather phase:
//   * stream_gather_kernel (when a row map exists): one 64-lane wave per
//     chunk of 64 16-byte vectors of token rows, 64 vectors of scale rows or
//     64 rows of 4-byte items (index, weight); each lane finds its row's input
//     row with one row-map load, then copies with non-temporal loads and
//     stores. A chunk that covers whole rows finds its first row with a
//     multiply-high by a precomputed reciprocal, so all its lanes share one
//     row-map word. The grid is the plain copy's, which measures fastest.
//     Token rows that are no multiple of 16 bytes stream as bytes instead:
//     each lane builds one aligned 16-byte block of the output from at most
//     two input rows with aligned loads and byte funnel shifts.
//   * gather_kernel (no row map): each workgroup owns a few adjacent output
//     rows; every wave maps 64 of them to their input rows with a 64-way
//     search over the table (a ballot over 64 pivots, then a shuffle search in
//     a 64-cell window), then the workgroup moves the items, one lane per
//     row, and streams the row bytes with all loads of a thread issued before
//     its stores (clamped, branch-free loads; predicated stores).
//   * fused_kernel: for small count matrices, the whole call in one launch,
//     in input order: every workgroup loads its own input rows first, then
//     recomputes the offsets in its own LDS (a few KiB, read from L2) with
//     the output row of each of its input rows, and stores the rows there;
//     workgroup 0 also writes expert_token_num and the status. Up to 64
//     cells, every wave computes the offsets in its registers (DPP scans,
//     lane shuffles, a six-step search) with no barrier.
// No atomics on global memory; every output element is written exactly once,
// so results are deterministic.
#include <hip/hip_runtime.h>

#include <limits.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "mrr_internal.h"

namespace mrr {
namespace {

using pair_t = int32_t __attribute__((ext_vector_type(2)));  // (dst_off, src_off)

constexpr int kOffsetItems = 4;  // counts per thread per tile (global path)
constexpr int kOffsetTile = kOffsetThreads * kOffsetItems;


// ---------------------------------------------------------------------------
// Workgroup scans
// ---------------------------------------------------------------------------

__device__ __forceinline__ int64_t wave_inclusive_scan(int64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive prefix of `v` over the workgroup (thread order), and the total.
// s holds 2 * kThreads / 64 + 1 entries.
template <int kThreads>
__device__ __forceinline__ int64_t block_exclusive_scan(int64_t v, int64_t* s, int64_t* total) {
  constexpr int kW = kThreads / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t inc = wave_inclusive_scan(v);
  if (lane == 63) s[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int64_t w = lane < kW ? s[lane] : 0;
    const int64_t wi = wave_inclusive_scan(w);
    if (lane < kW) s[kW + lane] = wi - w;
    if (lane == kW - 1) s[2 * kW] = wi;
  }
  __syncthreads();
  const int64_t res = s[kW + wave] + inc - v;
  *total = s[2 * kW];
  __syncthreads();  // s is reused by the next call
  return res;
}

// OR of `flags` over the workgroup (every thread gets the result).
__device__ __forceinline__ uint32_t block_or(uint32_t flags, uint32_t* s_flags) {
  if (flags != 0) atomicOr(s_flags, flags);
  __syncthreads();
  return *s_flags;
}

// Inclusive scan over the 64 lanes of a wave (wrapping 32-bit adds), with no
// LDS traffic: DPP row shifts by 1, 2, 4 and 8 scan each row of 16 lanes, then
// the row totals (read with readlane) are added to the later rows. Every lane
// of the wave must be active.
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t v) {
  constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kRowShr1, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kRowShr2, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kRowShr4, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kRowShr8, 0xf, 0xf, false));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 15);
  const uint32_t r1 = __builtin_amdgcn_readlane(v, 31);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Exact sum over the 64 lanes of a wave of values below 2^36, without LDS:
// the low 16 and the high 20 bits are summed apart with the DPP scan (each sum
// fits in 32 bits) and recombined.
__device__ __forceinline__ uint64_t wave_sum_u36(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readlane(wave_scan_u32(static_cast<uint32_t>(v & 0xffffu)), 63);
  const uint32_t hi = __builtin_amdgcn_readlane(wave_scan_u32(static_cast<uint32_t>(v >> 16)), 63);
  return (uint64_t(hi) << 16) + lo;
}

// Exact sum over the 64 lanes of a wave of values below 2^42 (the low 16 and
// the high 26 bits summed apart, each sum fitting in 32 bits).
__device__ __forceinline__ uint64_t wave_sum_u42(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readlane(wave_scan_u32(static_cast<uint32_t>(v & 0xffffu)), 63);
  const uint32_t hi = __builtin_amdgcn_readlane(wave_scan_u32(static_cast<uint32_t>(v >> 16)), 63);
  return (uint64_t(hi) << 16) + lo;
}

// kK exclusive scans over the workgroup (thread order, wrapping 32-bit adds)
// behind one barrier; for each k in kExactMask also the exact workgroup sum of
// exact[k] (each term < 2^36) in tot[k]. Each wave scans its lanes with DPP and
// publishes its total; after the barrier every wave reads the kThreads / 64
// wave totals one per lane and scans them the same way. LDS the caller writes
// before the call is visible to every thread after it. s_w and s_t must not
// be reused before a later barrier.
template <int kThreads, int kK, unsigned kExactMask>
__device__ __forceinline__ void block_scan_k(const uint32_t (&v)[kK], const uint64_t (&exact)[kK],
                                             uint32_t (&out)[kK], uint64_t (&tot)[kK],
                                             uint32_t (*s_w)[kThreads / 64], uint64_t (*s_t)[kThreads / 64]) {
  constexpr int kW = kThreads / 64;
  static_assert(kW <= 64, "one lane per wave total");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t incl[kK];
#pragma unroll
  for (int k = 0; k < kK; ++k) {
    incl[k] = wave_scan_u32(v[k]);
    if (lane == 63) s_w[k][wave] = incl[k];
    if ((kExactMask >> k) & 1u) {
      const uint64_t ws = wave_sum_u36(exact[k]);
      if (lane == 63) s_t[k][wave] = ws;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kK; ++k) {
    const uint32_t wi = wave_scan_u32(lane < kW ? s_w[k][lane] : 0u);
    const uint32_t base = wave > 0 ? __builtin_amdgcn_readlane(wi, wave - 1) : 0u;
    out[k] = base + incl[k] - v[k];
    tot[k] = 0;
    if ((kExactMask >> k) & 1u) tot[k] = wave_sum_u42(lane < kW ? s_t[k][lane] : 0);
  }
}

// Exclusive scan of v over the workgroup (thread order) with wrapping 32-bit
// adds. With kExact, also the exact workgroup sum of `exact` (each < 2^36)
// in *total: a caller that finds *total == A (<= INT32_MAX) with every term
// >= 0 knows that no partial sum wrapped. s_w and s_t hold kThreads / 64
// entries each and must not be reused before a later barrier.
template <int kThreads, bool kExact>
__device__ __forceinline__ uint32_t block_scan_u32(uint32_t v, uint64_t exact, uint32_t* s_w, uint64_t* s_t,
                                                   uint64_t* total) {
  uint32_t out[1];
  uint64_t tot[1];
  block_scan_k<kThreads, 1, kExact ? 1u : 0u>({v}, {exact}, out, tot,
                                              reinterpret_cast<uint32_t(*)[kThreads / 64]>(s_w),
                                              reinterpret_cast<uint64_t(*)[kThreads / 64]>(s_t));
  if (kExact) *total = tot[0];
  return out[0];
}

template <typename CountT>
__device__ __forceinline__ int32_t clamp_count(CountT raw, uint32_t* flags) {
  const int64_t v = static_cast<int64_t>(raw);
  if (v < 0) {
    *flags |= kFlagNegative;
    return 0;
  }
  if (v > INT32_MAX) {
    *flags |= kFlagTooLarge;
    return INT32_MAX;
  }
  return static_cast<int32_t>(v);
}

__device__ __forceinline__ void write_header(WsHeader* hdr, int64_t A, int64_t N, int64_t E, int64_t total,
                                             uint32_t flags, uint32_t valid_status, int inverse) {
  hdr->inverse = static_cast<uint32_t>(inverse);
  hdr->A = A;
  hdr->N = N;
  hdr->E = E;
  hdr->total = total;
  hdr->flags = flags;
  hdr->status = flags == 0 ? valid_status : kTablesBad;
}

// ---------------------------------------------------------------------------
// Offsets in a workgroup's LDS
// ---------------------------------------------------------------------------

// Scratch a workgroup needs to exchange wave results while computing offsets.
template <int kThreads>
struct ScanShared {
  uint32_t w[2][kThreads / 64];
  uint64_t t[2][kThreads / 64];
  uint32_t flags;
};

// floor(t / d) for 0 <= t < 2^12 and 1 <= d <= 2^12, with inv = 1.0f / d:
// (t + 1/2) / d lies at least 1 / (2d) from an integer, far more than the
// float error of the product.
__device__ __forceinline__ int div_small(int t, float inv) {
  return static_cast<int>((static_cast<float>(t) + 0.5f) * inv);
}

// Inclusive running maximum of v over the 64 lanes of a wave (values >= -1),
// with no LDS. Every lane must be active.
__device__ __forceinline__ int32_t wave_max_scan(int32_t v) {
  constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
  v = max(v, __builtin_amdgcn_update_dpp(-1, v, kRowShr1, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(-1, v, kRowShr2, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(-1, v, kRowShr4, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(-1, v, kRowShr8, 0xf, 0xf, false));
  const int row = (threadIdx.x & 63) >> 4;
  const int32_t r0 = __builtin_amdgcn_readlane(v, 15);
  const int32_t r1 = __builtin_amdgcn_readlane(v, 31);
  const int32_t r2 = __builtin_amdgcn_readlane(v, 47);
  v = max(v, row >= 1 ? r0 : -1);
  v = max(v, row >= 2 ? r1 : -1);
  return max(v, row >= 3 ? r2 : -1);
}

// Writes the end-of-table entries and finishes: tab[M] = (A, A), col[E] = A.
__device__ __forceinline__ void finish_offsets(pair_t* tab, int32_t* col, int M, int E, int64_t A) {
  if (threadIdx.x == 0) {
    pair_t t;
    t.x = static_cast<int32_t>(A);
    t.y = static_cast<int32_t>(A);
    if (tab != nullptr) tab[M] = t;
    col[E] = static_cast<int32_t>(A);
  }
  __syncthreads();
}

// Both offset tables of counts[N][E] with one cell per thread (M <= kThreads),
// in a workgroup's LDS. lds holds the counts and the source offsets in
// column-major cell order ([M] int32 each); the counts are then replaced by
// the destination offsets. Writes the table (in LDS or global memory; none
// when tab is null) in output order: forward, tab[j*N + i] = (DstOffset,
// SrcOffset) (coalesced); inverse, tab[i*E + j] = (SrcOffset, DstOffset);
// then tab[M] = (A, A), and the expert starts col[j] = DstOffset(0, j),
// col[E] = A. With a row map, also rowmap[d] for d = row0 + thread (one row
// per thread, coalesced); with s_map instead, s_map[thread] = that value in
// LDS (-1 past A).
// Returns 0, or the rejection flags (the same in every thread; then tab and
// col are not written).
template <int kThreads, typename CountT>
__device__ uint32_t offsets_cells(const CountT* __restrict__ counts, int N, int E, int64_t A, int inverse,
                                  int32_t* lds, int32_t* col, pair_t* tab, ScanShared<kThreads>* sh,
                                  int64_t* total_out, int32_t* __restrict__ rowmap = nullptr, int row0 = 0,
                                  int32_t* s_mark = nullptr, int32_t* s_map = nullptr) {
  const bool mapping = rowmap != nullptr || s_map != nullptr;
  const int tid = threadIdx.x;
  const int M = N * E;
  int32_t* s_c = lds;      // counts, column-major
  int32_t* s_s = lds + M;  // SrcOffset, column-major
  if (tid == 0) sh->flags = 0;
  for (int j = tid; j <= E; j += kThreads) col[j] = 0;
  if (mapping) s_mark[tid] = -1;
  uint32_t flags = 0;
  // Thread t holds cell t in row-major (rank i, expert j) order.
  const bool in = tid < M;
  uint32_t c = 0;
  if (in) c = static_cast<uint32_t>(clamp_count(counts[tid], &flags));
  uint64_t total;
  const uint32_t src = block_scan_u32<kThreads, true>(c, c, sh->w[0], sh->t[0], &total);
  if (in) {
    const int i = tid / E;
    const int j = tid - i * E;
    s_c[j * N + i] = static_cast<int32_t>(c);
    s_s[j * N + i] = static_cast<int32_t>(src);
  }
  *total_out = static_cast<int64_t>(total);
  flags = block_or(flags, &sh->flags);  // also orders the writes above before the reads below
  if (total != static_cast<uint64_t>(A)) flags |= kFlagSumMismatch;
  if (flags != 0) return flags;
  // Thread u now holds cell u in column-major (expert j, rank i) order.
  const uint32_t c2 = in ? static_cast<uint32_t>(s_c[tid]) : 0u;
  uint64_t unused;
  const uint32_t dst = block_scan_u32<kThreads, false>(c2, 0, sh->w[1], sh->t[1], &unused);
  if (in) {
    const int j = tid / N;
    const int i = tid - j * N;
    pair_t t;
    if (inverse) {
      t.x = s_s[tid];
      t.y = static_cast<int32_t>(dst);
      if (tab != nullptr) tab[i * E + j] = t;
    } else {
      t.x = static_cast<int32_t>(dst);
      t.y = s_s[tid];
      if (tab != nullptr) tab[tid] = t;
    }
    if (i == 0) col[j] = static_cast<int32_t>(dst);
    s_c[tid] = static_cast<int32_t>(dst);  // this thread's own count was read before the scan
    if (mapping && c2 > 0) {
      // Mark where this cell's rows start among the workgroup's output rows
      // [row0, row0 + kThreads), by its output-order index (forward: this
      // column-major index; inverse: the row-major one). Each wave's 64 rows
      // are marked on their own: the cell that covers a wave's first row from
      // before marks that row. Output-order indices rise with the output
      // offset, so a running maximum over each wave's marks gives each row
      // its cell, with no exchange between waves.
      const int32_t out_off = inverse ? s_s[tid] : static_cast<int32_t>(dst);
      const int lo = out_off - row0;
      const int o = inverse ? i * E + j : tid;
      if (lo >= 0 && lo < kThreads) s_mark[lo] = o;
      const int32_t end = out_off + static_cast<int32_t>(c2);
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) {
        const int first = row0 + 64 * w;  // wave w's first row
        if (out_off < first && end > first) s_mark[64 * w] = o;
      }
    }
  }
  finish_offsets(tab, col, M, E, A);
  if (mapping) {
    const int o = wave_max_scan(s_mark[tid]);
    const int d = row0 + tid;
    int32_t v = -1;
    if (d < A) {
      int u = o;  // the cell's column-major index
      if (inverse) {
        const int i = div_small(o, 1.0f / static_cast<float>(E));
        u = (o - i * E) * N + i;
      }
      // forward: s_s holds the input (source) offsets, s_c the output ones; inverse: the reverse
      v = inverse ? s_c[u] + (d - s_s[u]) : s_s[u] + (d - s_c[u]);
      if (s_map == nullptr) rowmap[d] = v;
    }
    if (s_map != nullptr) s_map[tid] = v;
  }
  return 0;
}

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

// expert_token_num from the expert starts col[0..E]: expert j's rows are
// [col[j], col[j+1]); the cumsum form is the inclusive total col[j+1].
template <int kThreads, typename CountT>
__device__ __forceinline__ void write_etn(const int32_t* col, int E, int cumsum, CountT* __restrict__ etn) {
  for (int j = threadIdx.x; j < E; j += kThreads)
    etn[j] = static_cast<CountT>(cumsum ? col[j + 1] : col[j + 1] - col[j]);
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
    flags = offsets_cells<kOffsetThreads>(counts, N, E, A, inverse, s_dyn, col,
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
      offsets_cells<kT>(counts, N, E, A, inverse, s_mats, s_col, nullptr, &sh, &total, rowmap,
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
  if (tid == 0) {
    table[2 * M] = static_cast<int32_t>(A);
    table[2 * M + 1] = static_cast<int32_t>(A);
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
      start = table[2 * (j * N)];
      end = table[2 * ((j + 1) * N)];
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
//  4. With a row map, the workgroups of a band split its cells: a thread
//     writes the rows of a cell of at most kBandCellRows rows, a wave those
//     of a cell of at most kOffsetThreads rows, and every workgroup of the
//     band its share of a larger cell's rows.
// Every workgroup repeats step 1 over all M cells, which is why the per-cell
// work is kept to a few instructions, and why the L2 reads grow as
// M * (number of bands); the planner bounds M for this path.
constexpr int kBandCellRows = 16;  // row-map rows a thread writes for one cell; larger cells take the workgroup
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
      const CountT* p = counts + j;
      int ib = r;
      for (; ib + (kBandUnroll - 1) * lanes < N; ib += kBandUnroll * lanes) {
        CountT raw[kBandUnroll];
#pragma unroll
        for (int k = 0; k < kBandUnroll; ++k) raw[k] = p[(ib + k * lanes) * E];
#pragma unroll
        for (int k = 0; k < kBandUnroll; ++k) acc.add(raw[k], ib + k * lanes < i0);
      }
      if (ib < N) {  // the last, partial chunk: clamped loads, predicated sums
        CountT raw[kBandUnroll];
#pragma unroll
        for (int k = 0; k < kBandUnroll; ++k) {
          const int i = ib + k * lanes;
          raw[k] = p[(i < N ? i : N - 1) * E];
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
    const int fan = lanes < kBandFanIn ? lanes : kBandFanIn;
    for (int k = 0; k < fan; ++k) {
      tot_j += s.tot[k * E + tid];
      bef_j += s.bef[k * E + tid];
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
    // cells; a thread writes the rows of a cell with at most kBandCellRows
    // rows itself, and the workgroup writes each larger cell's rows together,
    // strided over all its threads. Forward: output row DstOffset + k takes
    // source row SrcOffset + k; inverse: the reverse.
    __syncthreads();
    {
      const int per = (cells + split - 1) / split;
      const int q = slice * per + tid;
      if (tid < per && q < cells) {
        const int sq = s.src_q[q], dq = s.dst_q[q], n = s.src_q[q + 1] - sq;
        if (n <= kBandCellRows) {
          for (int k = 0; k < n; ++k) {
            if (inverse)
              rowmap[sq + k] = dq + k;
            else
              rowmap[dq + k] = sq + k;
          }
        } else if (n <= kOffsetThreads) {
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

// ---------------------------------------------------------------------------
// Row moves
// ---------------------------------------------------------------------------

template <int V>
struct VecT;
template <>
struct VecT<16> {
  using type = uint32_t __attribute__((ext_vector_type(4)));
};
template <>
struct VecT<8> {
  using type = uint32_t __attribute__((ext_vector_type(2)));
};
template <>
struct VecT<4> {
  using type = uint32_t;
};
template <>
struct VecT<2> {
  using type = uint16_t;
};
template <>
struct VecT<1> {
  using type = uint8_t;
};

struct GatherArgs {
  const uint8_t* tokens;
  uint8_t* out_tokens;
  const uint8_t* scales;
  uint8_t* out_scales;
  const uint32_t* weight;  // fp32 weights moved as raw 4-byte words
  uint32_t* out_weight;
  int32_t* idx;
  const pair_t* table;     // in the workspace (gather_kernel)
  const int32_t* rowmap;   // in the workspace (stream_gather_kernel): input row of every output row
  WsHeader* hdr;
  int64_t row_bytes;
  int64_t scale_row_bytes;
  int64_t N;
  int64_t E;
  int32_t vecs_per_row;
  int32_t scale_vecs_per_row;
  int32_t scale_vec;
  int32_t A;
  int32_t M;
  int32_t rows_per_wg;
  int32_t inverse;         // the direction the table must have been built for
};

// Source row of output row d, from a table of M + 1 (output offset, input
// offset) pairs sorted by output offset, in LDS or global memory. All 64 lanes of a wave call it together, with
// their rows d in [d_lo, d_lo + 63]; d_lo is the same for the whole wave.
// Whatever the table holds, every read stays inside its M + 1 entries.
__device__ __forceinline__ int32_t source_row(const pair_t* table, int M, int d_lo, int d) {
  const int lane = threadIdx.x & 63;
  // 64-way search for the cell of d_lo: the largest m with dst_off[m] <= d_lo.
  // Invariant: dst_off[lo] <= d_lo and that cell lies in [lo, hi).
  int lo = 0;
  int hi = M;
  while (hi - lo > 64) {
    const int stride = (hi - lo + 63) >> 6;
    const int pos = lo + lane * stride;
    const int v = pos < hi ? table[pos].x : INT_MAX;
    const uint64_t below = __ballot(v <= d_lo);  // a prefix of the lanes
    const int k = max(static_cast<int>(__popcll(below)) - 1, 0);
    lo += k * stride;
    hi = min(hi, lo + stride);
  }
  // The 64-cell window [lo, lo + 64) with both offsets of each cell: a
  // shuffle binary search per lane for the largest l with dst_off <= d.
  pair_t w;
  w.x = INT_MAX;
  w.y = 0;
  if (lo + lane <= M) w = table[lo + lane];
  int l = 0;
#pragma unroll
  for (int step = 32; step > 0; step >>= 1) {
    const int cand = l + step;
    if (__shfl(w.x, cand, 64) <= d) l = cand;
  }
  int dm = __shfl(w.x, l, 64);
  int sm = __shfl(w.y, l, 64);
  if (l == 63 && lo + 63 < M) {
    // d lies past the window (many empty cells in between): finish alone.
    int a = lo + 63;
    int b = M;  // dst_off[a] <= d < dst_off[b] == A
    while (b - a > 1) {
      const int mid = (a + b) >> 1;
      if (table[mid].x <= d)
        a = mid;
      else
        b = mid;
    }
    const pair_t t = table[a];
    dm = t.x;
    sm = t.y;
  }
  return sm + (d - dm);
}

// Fills s_src[0, rows) with the source rows of output rows row0 + [0, rows),
// or -1 for a row whose mapped source lies outside [0, A).
__device__ __forceinline__ void map_rows(const pair_t* table, int M, int A, int row0, int rows, int32_t* s_src) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int b = wave * 64; b < rows; b += kGatherThreads) {
    const int lr = b + lane;
    const bool mine = lr < rows;
    const int d_lo = row0 + b;
    const int d = mine ? row0 + lr : d_lo;
    const int32_t s = source_row(table, M, d_lo, d);
    const bool ok = mine && static_cast<unsigned>(s) < static_cast<unsigned>(A);
    if (mine) s_src[lr] = ok ? s : -1;
  }
}

// Copies `rows` rows of row_bytes = vpr * V bytes: source row s_src[r] to the
// r-th row of dst_chunk (rows adjacent). Rows with s_src[r] < 0 are skipped.
// The (row, vector) space is flattened and walked in steps of the workgroup
// size; each thread issues kGatherUnroll loads before their stores.
template <int V>
__device__ __forceinline__ void copy_rows(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst_chunk,
                                          int64_t row_bytes, int vpr, int rows,
                                          const int32_t* __restrict__ s_src) {
  using T = typename VecT<V>::type;
  const int total = rows * vpr;
  const int tid = threadIdx.x;
  int r = tid / vpr;
  int c = tid - r * vpr;
  const int dr = kGatherThreads / vpr;
  const int dc = kGatherThreads - dr * vpr;
  for (int e0 = 0; e0 < total; e0 += kGatherThreads * kGatherUnroll) {
    // First every item's (row, column) and source row (LDS reads, all issued
    // together), then all the loads, then all the stores.
    int32_t srow[kGatherUnroll];
    int col[kGatherUnroll];
#pragma unroll
    for (int k = 0; k < kGatherUnroll; ++k) {
      const bool in = e0 + tid + k * kGatherThreads < total;
      srow[k] = s_src[in ? r : 0];
      col[k] = in ? c : -1;
      r += dr;
      c += dc;
      if (c >= vpr) {
        c -= vpr;
        ++r;
      }
    }
    T v[kGatherUnroll];
#pragma unroll
    for (int k = 0; k < kGatherUnroll; ++k) {
      // Branch-free load: items out of range read row 0, column 0 (always
      // valid, since A > 0 here) and are not stored.
      const bool ok = col[k] >= 0 && srow[k] >= 0;
      const int64_t off = ok ? int64_t(srow[k]) * row_bytes + int64_t(col[k]) * V : 0;
      v[k] = __builtin_nontemporal_load(reinterpret_cast<const T*>(src + off));
    }
#pragma unroll
    for (int k = 0; k < kGatherUnroll; ++k) {
      const int e = e0 + tid + k * kGatherThreads;
      if (col[k] >= 0 && srow[k] >= 0)
        __builtin_nontemporal_store(v[k], reinterpret_cast<T*>(dst_chunk + int64_t(e) * V));
    }
  }
}

// Everything a workgroup writes for its output rows row0 + [0, rows), once
// s_src holds their source rows: the index and weight (one lane per row), the
// token rows and the scale rows. The small loads (the weight, and with kSV > 0
// this thread's kSV-byte piece of the scale rows) are issued before the token
// copy so that they are in flight with it, and stored after it; with kSV == 0
// the scale rows take a separate pass after the token rows.
template <int V, int kSV, bool kScatter, bool kWeight>
__device__ __forceinline__ void move_rows(const GatherArgs& p, int row0, int rows, const int32_t* s_src) {
  const int tid = threadIdx.x;
  const int64_t Rs = p.scale_row_bytes;

  // This thread's row for the per-row words (first round; more rows than
  // threads only happen for tiny rows and are handled below).
  const int32_t my_s = tid < rows ? s_src[tid] : -1;
  uint32_t wv = 0;
  if (kWeight) wv = p.weight[my_s >= 0 ? my_s : 0];  // branch-free: row 0 when unused

  using ST = typename VecT<(kSV > 0 ? kSV : 4)>::type;
  ST piece{};
  int32_t sc_src = -1;
  int sc_row = 0, sc_off = 0;
  if (kSV > 0) {
    const int spr = static_cast<int>(Rs / kSV);  // pieces per scale row
    sc_row = tid / spr;
    sc_off = (tid - sc_row * spr) * kSV;
    sc_src = tid < rows * spr ? s_src[sc_row] : -1;
    const int64_t off = sc_src >= 0 ? int64_t(sc_src) * Rs + sc_off : 0;  // branch-free
    piece = __builtin_nontemporal_load(reinterpret_cast<const ST*>(p.scales + off));
  }

  copy_rows<V>(p.tokens, p.out_tokens + int64_t(row0) * p.row_bytes, p.row_bytes, p.vecs_per_row, rows, s_src);

  if (kSV > 0 && sc_src >= 0)
    __builtin_nontemporal_store(piece, reinterpret_cast<ST*>(p.out_scales + int64_t(row0 + sc_row) * Rs + sc_off));
  for (int lr = tid; lr < rows; lr += kGatherThreads) {
    const int32_t s = lr == tid ? my_s : s_src[lr];
    if (s < 0) continue;
    const int d = row0 + lr;
    if (kScatter)
      p.idx[s] = d;
    else
      p.idx[d] = s;
    if (kWeight) p.out_weight[d] = lr == tid ? wv : p.weight[s];
  }

  if (kSV == 0 && Rs > 0) {
    uint8_t* out = p.out_scales + int64_t(row0) * Rs;
    const int spr = p.scale_vecs_per_row;
    switch (p.scale_vec) {
      case 16: copy_rows<16>(p.scales, out, Rs, spr, rows, s_src); break;
      case 8: copy_rows<8>(p.scales, out, Rs, spr, rows, s_src); break;
      case 4: copy_rows<4>(p.scales, out, Rs, spr, rows, s_src); break;
      case 2: copy_rows<2>(p.scales, out, Rs, spr, rows, s_src); break;
      default: copy_rows<1>(p.scales, out, Rs, spr, rows, s_src); break;
    }
  }
}

template <int V, int kSV, bool kScatter, bool kWeight>
__global__ __launch_bounds__(kGatherThreads) void gather_kernel(GatherArgs p) {
  __shared__ int32_t s_src[kMaxRowsPerWg];
  const int row0 = blockIdx.x * p.rows_per_wg;
  const int rows = min(p.rows_per_wg, p.A - row0);
  // The table is searched before the header is checked, so that the two
  // reads overlap; nothing is written unless the header says the table was
  // built from valid counts for this (A, N, E) and direction.
  const WsHeader* h = p.hdr;
  const bool valid_table = h->status == kTablesValid && h->A == p.A && h->N == p.N && h->E == p.E &&
                           h->inverse == static_cast<uint32_t>(p.inverse);
  map_rows(p.table, p.M, p.A, row0, rows, s_src);
  if (!valid_table) return;  // uniform over the workgroup
  __syncthreads();
  move_rows<V, kSV, kScatter, kWeight>(p, row0, rows, s_src);
}

// ---------------------------------------------------------------------------
// Stream gather: one-wave workgroups, one vector per lane
// ---------------------------------------------------------------------------

// The output of the two-kernel path is three byte streams in output order:
// the token rows (A * vpr vectors of V bytes), the scale rows (A * svpr
// vectors of SV bytes) and the per-row items (A rows: index and weight).
// Each is cut into chunks of 64 consecutive vectors (rows, for the items),
// and one 64-lane workgroup moves one chunk: every lane finds its vector's
// output row, looks up that row's source in the offsets table (a 64-way
// search shared by the wave), and issues one load and one store. Small
// one-shot workgroups keep the CU's wave slots full while each wave's short
// search is in flight, which streams closer to the copy ceiling than large
// workgroups with many loads per lane.
struct StreamGrid {
  uint32_t tok_chunks;   // ceil(A * vpr / 64)
  uint32_t small;        // scale and item chunks, which take the grid's first workgroups
  uint32_t sc_end;       // tok_chunks + ceil(A * svpr / 64) (no scale chunks without scales)
  uint32_t cpr;          // token chunks per row when whole (vpr % 64 == 0), else 0
  uint32_t cpr_magic;    // ceil(2^32 / cpr): chunk / cpr by a multiply-high and one correction
  float inv_vpr;         // 1 / vpr and 1 / svpr, for rows shorter than a chunk
  float inv_svpr;
  uint32_t byte_rows;    // token rows stream as bytes: aligned 16-byte blocks of the output
  float inv_row;         // 1 / row bytes, for byte_rows with rows under 1 KiB
  uint32_t rows8;        // byte_rows with R >= 147 and A >= 8: a 1 KiB chunk spans at most
                         // floor(1023 / R) + 2 <= 8 rows
};

// The workspace header's verdict, read through the scalar cache: it was
// written by an earlier kernel and this kernel does not write it.
__device__ __forceinline__ bool header_valid(const WsHeader* hdr, const GatherArgs& p) {
  using CHdr = const WsHeader __attribute__((address_space(4)))*;
  const CHdr h = reinterpret_cast<CHdr>(reinterpret_cast<uintptr_t>(hdr));
  // all fields loaded together (no short-circuit between the loads)
  const uint32_t status = h->status, inverse = h->inverse;
  const int64_t A = h->A, N = h->N, E = h->E;
  return (status == kTablesValid) & (A == p.A) & (N == p.N) & (E == p.E) &
         (inverse == static_cast<uint32_t>(p.inverse));
}

// A token chunk that lies in one row (the row is a whole number of chunks):
// chunk c is part c % cpr of row c / cpr. The row's row-map word and the
// workspace header are read through the scalar cache and waited for
// together, so each wave's chain is one scalar round trip, the token load and
// the store (the row map was written by an earlier kernel; this one does not
// write it).
template <int V>
__device__ __forceinline__ void stream_whole_row_chunk(const GatherArgs& p, const StreamGrid& g, uint32_t c) {
  using T = typename VecT<V>::type;
  using CInt = const int32_t __attribute__((address_space(4)))*;
  uint32_t d = c;
  if (g.cpr != 1) {  // uniform
    d = __umulhi(c, g.cpr_magic);
    d -= d * g.cpr > c ? 1u : 0u;
  }
  d = __builtin_amdgcn_readfirstlane(d);
  const int32_t s = reinterpret_cast<CInt>(reinterpret_cast<uintptr_t>(p.rowmap))[d];
  const uint32_t col = (c - d * g.cpr) * 64u + (threadIdx.x & 63);  // vector within the row
  // `&`, not `&&`: the header loads issue beside the row-map load
  const bool ok = header_valid(p.hdr, p) & (static_cast<unsigned>(s) < static_cast<unsigned>(p.A));
  const int64_t so = ok ? int64_t(s) * p.row_bytes + int64_t(col) * V : 0;
  const T v = __builtin_nontemporal_load(reinterpret_cast<const T*>(p.tokens + so));
  if (ok) __builtin_nontemporal_store(v, reinterpret_cast<T*>(p.out_tokens + int64_t(d) * p.row_bytes + int64_t(col) * V));
}

// Chunk `chunk` of a row stream: vectors [64 chunk, 64 chunk + 64) of the
// rows [0, A) of vpr vectors of V bytes each, output row d taken from
// source row rowmap[d]. The header check of p is computed after the row-map
// load is issued (and without short-circuit), so its scalar loads overlap
// that load instead of preceding it; the same holds in every chunk kind.
template <int V>
__device__ __forceinline__ void stream_rows(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                            int64_t row_bytes, int vpr, float inv_vpr, int64_t chunk,
                                            const int32_t* __restrict__ rowmap, int A, const GatherArgs& p) {
  using T = typename VecT<V>::type;
  const int lane = threadIdx.x & 63;
  const int64_t g0 = chunk * 64;
  const int64_t total = int64_t(A) * vpr;
  const int64_t d0 = g0 / vpr;  // the chunk's first row (uniform)
  const int off = static_cast<int>(g0 - d0 * vpr) + lane;  // < vpr + 64
  // Row within the chunk: at most one row boundary when vpr >= 64; below
  // that, a small exact division (off < 128).
  const int dd = vpr >= 64 ? (off >= vpr ? 1 : 0) : div_small(off, inv_vpr);
  const int col = off - dd * vpr;
  const bool in = g0 + lane < total;
  const int d = static_cast<int>(d0) + (in ? dd : 0);  // in [d0, d0 + 63]
  const int32_t s = rowmap[d];
  const bool ok = in & header_valid(p.hdr, p) & (static_cast<unsigned>(s) < static_cast<unsigned>(A));
  // Branch-free load (row 0, column 0 when not moving: always valid here).
  const int64_t so = ok ? int64_t(s) * row_bytes + int64_t(col) * V : 0;
  const T v = __builtin_nontemporal_load(reinterpret_cast<const T*>(src + so));
  if (ok) __builtin_nontemporal_store(v, reinterpret_cast<T*>(dst + (g0 + lane) * V));
}

// Bytes [w, w + 16) of `base`, of which [n0, n1) are needed (w <= n0 < n1 <=
// w + 16): two aligned 16-byte loads, each of a block that holds a needed
// byte (a block with none takes the other's address, so no load leaves the
// 16-byte blocks the needed bytes lie in), then a byte funnel shift.
__device__ __forceinline__ VecT<16>::type window16(const uint8_t* __restrict__ base, int64_t w, int64_t n0,
                                                   int64_t n1) {
  using T = VecT<16>::type;
  const int64_t a = w & ~int64_t(15);
  const bool need_a = a + 16 > n0;
  const bool need_b = a + 16 < n1;
  const T lo = *reinterpret_cast<const T*>(base + (need_a ? a : a + 16));
  const T hi = *reinterpret_cast<const T*>(base + (need_b ? a + 16 : a));
  const uint32_t wd[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  const int sh = static_cast<int>(w - a);  // 0..15
  const int q = sh >> 2;
  const uint32_t r = static_cast<uint32_t>(sh & 3);
  uint32_t x[5];  // wd[q .. q + 4]
#pragma unroll
  for (int i = 0; i < 5; ++i) x[i] = q == 0 ? wd[i] : q == 1 ? wd[i + 1] : q == 2 ? wd[i + 2] : wd[i + 3];
  T out;
  out.x = __builtin_amdgcn_alignbyte(x[1], x[0], r);
  out.y = __builtin_amdgcn_alignbyte(x[2], x[1], r);
  out.z = __builtin_amdgcn_alignbyte(x[3], x[2], r);
  out.w = __builtin_amdgcn_alignbyte(x[4], x[3], r);
  return out;
}

// Token rows that are no multiple of 16 bytes (but at least 16 bytes, with
// both buffers 16-byte aligned), as one byte stream: lane l of chunk c builds
// the aligned 16-byte block of the dense output at byte 1024 c + 16 l from at
// most two output rows, i.e. two input rows (row map), with window16 each,
// and stores it whole (the last, partial block byte by byte).
__device__ __forceinline__ void stream_bytes_chunk(const GatherArgs& p, const StreamGrid& g, uint32_t chunk) {
  using T = VecT<16>::type;
  const int lane = threadIdx.x & 63;
  const int64_t R = p.row_bytes;
  const int64_t total = int64_t(p.A) * R;
  const int64_t o0 = int64_t(chunk) * 1024;
  const int64_t d_base = o0 / R;  // the chunk's first row (uniform)
  const int64_t o = o0 + 16 * lane;
  if (o >= total) return;
  // Row within the chunk: at most one boundary for rows of 1 KiB or more;
  // below that, a small exact division (off < 2048).
  const int off = static_cast<int>(o0 - d_base * R) + 16 * lane;  // < R + 1024
  const int Ri = static_cast<int>(R);
  const int dd = Ri >= 1024 ? (off >= Ri ? 1 : 0) : div_small(off, g.inv_row);
  const int col1 = off - dd * Ri;
  const int d1 = static_cast<int>(d_base) + dd;
  const int len1 = min(16, Ri - col1);  // bytes from row d1; the rest from row d1 + 1
  const bool has2 = len1 < 16;
  const int d2 = has2 ? min(d1 + 1, p.A - 1) : d1;
  const bool hv = header_valid(p.hdr, p);  // its loads go out first, beside the row-map loads
  int32_t s1, s2;
  if (g.rows8) {  // uniform: the chunk's rows lie in 8 consecutive row-map words, read through the
                  // scalar cache (beside the header loads) starting at min(d_base, A - 8)
    using CInt = const int32_t __attribute__((address_space(4)))*;
    const int base = min(static_cast<int>(d_base), p.A - 8);
    const CInt m = reinterpret_cast<CInt>(reinterpret_cast<uintptr_t>(p.rowmap + base));
    int32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = m[k];
    const int k1 = d1 - base, k2 = d2 - base;  // in [0, 8)
    s1 = w[0];
    s2 = w[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) {
      s1 = k1 == k ? w[k] : s1;
      s2 = k2 == k ? w[k] : s2;
    }
  } else {
    s1 = p.rowmap[d1];
    s2 = p.rowmap[d2];
  }
  const bool ok = hv & (static_cast<unsigned>(s1) < static_cast<unsigned>(p.A)) &
                  (static_cast<unsigned>(s2) < static_cast<unsigned>(p.A));
  s1 = ok ? s1 : 0;  // input row 0 when not moving: always valid here
  s2 = ok ? s2 : 0;
  const int64_t w1 = int64_t(s1) * R + col1;
  T v = window16(p.tokens, w1, w1, w1 + len1);
  if (has2) {  // the block crosses into the next row (a few lanes of a wave)
    const int64_t r2 = int64_t(s2) * R;  // output byte b >= len1 is input byte r2 + b - len1
    const T x2 = window16(p.tokens, r2 - len1, r2, r2 + (16 - len1));
    uint32_t m[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int nb = min(max(len1 - 4 * k, 0), 4);  // bytes of dword k taken from the first row
      m[k] = nb >= 4 ? 0xffffffffu : (1u << (8 * nb)) - 1u;
    }
    v.x = (v.x & m[0]) | (x2.x & ~m[0]);
    v.y = (v.y & m[1]) | (x2.y & ~m[1]);
    v.z = (v.z & m[2]) | (x2.z & ~m[2]);
    v.w = (v.w & m[3]) | (x2.w & ~m[3]);
  }
  if (!ok) return;
  if (o + 16 <= total) {
    __builtin_nontemporal_store(v, reinterpret_cast<T*>(p.out_tokens + o));
  } else {
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
    for (int b = 0; b < static_cast<int>(total - o); ++b)
      p.out_tokens[o + b] = static_cast<uint8_t>(wv[b >> 2] >> (8 * (b & 3)));
  }
}

// One chunk per workgroup. Chunk numbers: token chunks [0, tok_chunks), scale
// chunks [tok_chunks, sc_end), then item chunks; the workgroups take the scale
// and item chunks first (with the token chunks' scalar row-map read, this
// order measured faster than token chunks first). Branches are uniform.
template <int V, bool kScatter, bool kWeight>
__global__ __launch_bounds__(64) void stream_gather_kernel(GatherArgs p, StreamGrid g) {
  const uint32_t bx = blockIdx.x;
  const uint32_t b = bx >= g.small ? bx - g.small : bx + g.tok_chunks;
  if (b < g.tok_chunks && g.cpr != 0) {  // cpr is 0 for byte rows
    stream_whole_row_chunk<V>(p, g, b);
    return;
  }
  if (b < g.tok_chunks) {
    if (V < 16 && g.byte_rows != 0)
      stream_bytes_chunk(p, g, b);
    else
      stream_rows<V>(p.tokens, p.out_tokens, p.row_bytes, p.vecs_per_row, g.inv_vpr, b, p.rowmap, p.A, p);
  } else if (b < g.sc_end) {
    const int64_t c = b - g.tok_chunks;
    const int spr = p.scale_vecs_per_row;
    const int64_t Rs = p.scale_row_bytes;
    const float inv = g.inv_svpr;
    switch (p.scale_vec) {
      case 16: stream_rows<16>(p.scales, p.out_scales, Rs, spr, inv, c, p.rowmap, p.A, p); break;
      case 8: stream_rows<8>(p.scales, p.out_scales, Rs, spr, inv, c, p.rowmap, p.A, p); break;
      case 4: stream_rows<4>(p.scales, p.out_scales, Rs, spr, inv, c, p.rowmap, p.A, p); break;
      case 2: stream_rows<2>(p.scales, p.out_scales, Rs, spr, inv, c, p.rowmap, p.A, p); break;
      default: stream_rows<1>(p.scales, p.out_scales, Rs, spr, inv, c, p.rowmap, p.A, p); break;
    }
  } else {
    const int r0 = static_cast<int>(b - g.sc_end) * 64;
    const int d = r0 + static_cast<int>(threadIdx.x & 63);
    const bool in = d < p.A;
    const int32_t s = p.rowmap[in ? d : r0];
    const bool ok = in & header_valid(p.hdr, p) & (static_cast<unsigned>(s) < static_cast<unsigned>(p.A));
    if (kWeight) {
      const uint32_t wv = p.weight[ok ? s : 0];
      if (ok) p.out_weight[d] = wv;
    }
    if (ok) {
      if (kScatter)
        p.idx[s] = d;
      else
        p.idx[d] = s;
    }
  }
}

struct FusedArgs {
  const void* counts;
  void* etn;
  int32_t cumsum;
};

// Offsets of a count matrix of at most 64 cells inside one wave, with no LDS
// and no barrier (every wave of a workgroup computes them alike). Lane q
// holds row-major cell q = i*E + j; lane u holds column-major cell u = j*N + i.
struct WaveCells {
  uint32_t src;     // lane q: SrcOffset of cell q
  uint32_t dst;     // lane q: DstOffset of cell q
  uint32_t dst_cm;  // lane u: DstOffset of cell u
  uint32_t src_cm;  // lane u: SrcOffset of cell u
  int first_row;    // lane u: 1 when cell u is in rank 0 (DstOffset(0, j) is an expert's start)
  int expert;       // lane u: its expert j
};

// Returns the rejection flags (the same in every lane) and, in *total, the
// exact sum of the clamped counts. All 64 lanes must be active.
template <typename CountT>
__device__ __forceinline__ uint32_t wave_offsets64(const CountT* __restrict__ counts, int N, int E, int64_t A,
                                                   WaveCells* w, int64_t* total) {
  const int lane = threadIdx.x & 63;
  const int M = N * E;
  uint32_t f = 0;
  const uint32_t c = lane < M ? static_cast<uint32_t>(clamp_count(counts[lane], &f)) : 0u;
  const uint64_t tot = wave_sum_u36(c);
  uint32_t flags = tot != static_cast<uint64_t>(A) ? kFlagSumMismatch : 0u;
  if (__builtin_amdgcn_ballot_w64((f & kFlagNegative) != 0) != 0) flags |= kFlagNegative;
  if (__builtin_amdgcn_ballot_w64((f & kFlagTooLarge) != 0) != 0) flags |= kFlagTooLarge;
  *total = static_cast<int64_t>(tot);
  // Exact when flags == 0: the total is A <= INT32_MAX and no count is negative.
  w->src = wave_scan_u32(c) - c;
  const bool in = lane < M;
  const int ju = div_small(lane, 1.0f / static_cast<float>(max(N, 1)));  // lane u = ju * N + iu
  const int iu = lane - ju * N;
  const int q_of_u = in ? iu * E + ju : lane;
  const uint32_t c_u = static_cast<uint32_t>(__shfl(static_cast<int>(c), q_of_u));  // every lane takes part
  const uint32_t cu = in ? c_u : 0u;
  w->dst_cm = wave_scan_u32(cu) - cu;
  w->src_cm = static_cast<uint32_t>(__shfl(static_cast<int>(w->src), q_of_u));
  w->first_row = in && iu == 0;
  w->expert = ju;
  const int iq = div_small(lane, 1.0f / static_cast<float>(max(E, 1)));  // lane q = iq * E + jq
  const int jq = lane - iq * E;
  w->dst = static_cast<uint32_t>(__shfl(static_cast<int>(w->dst_cm), in ? jq * N + iq : lane));
  return flags;
}

// Output row of input row s (< A) from the wave's cells: the last cell of the
// input order that starts at or before s (empty cells share their start with
// the next cell, so it is the one holding s). A branch-free six-step search
// over the lanes; all 64 lanes must be active.
__device__ __forceinline__ int32_t wave_map_row(const WaveCells& w, int M, int inverse, int32_t s) {
  const uint32_t in_start = inverse ? w.dst_cm : w.src;   // input order: column-major when inverse
  const uint32_t out_start = inverse ? w.src_cm : w.dst;
  int k = 0;
#pragma unroll
  for (int b = 32; b >= 1; b >>= 1) {
    const int cand = k + b;
    const uint32_t v = static_cast<uint32_t>(__shfl(static_cast<int>(in_start), cand < M ? cand : 0));
    if (cand < M && v <= static_cast<uint32_t>(s)) k = cand;
  }
  const uint32_t i0 = static_cast<uint32_t>(__shfl(static_cast<int>(in_start), k));
  const uint32_t o0 = static_cast<uint32_t>(__shfl(static_cast<int>(out_start), k));
  return static_cast<int32_t>(o0 + (static_cast<uint32_t>(s) - i0));
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
  const uint32_t flags = wave_offsets64<CountT>(counts, N, E, A, &w, &total);
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

// Items [e0, e0 + kGatherThreads * kGatherUnroll) of `rows` input rows of
// vpr vectors each, starting at input row row0, kGatherUnroll per thread
// (item e is vector e % vpr of row e / vpr): the loads, and where each item
// goes (c = -1: none). Items past the end load row row0, vector 0.
template <int V>
struct RowRound {
  typename VecT<V>::type v[kGatherUnroll];
  int r[kGatherUnroll];
  int c[kGatherUnroll];
};

template <int V>
__device__ __forceinline__ void load_round(RowRound<V>& q, const uint8_t* __restrict__ src, int64_t row_bytes,
                                           int vpr, int rows, int row0, int e0) {
  using T = typename VecT<V>::type;
  const int total = rows * vpr;
  const int e = e0 + static_cast<int>(threadIdx.x);
  int r = e / vpr;
  int c = e - r * vpr;
  const int dr = kGatherThreads / vpr;
  const int dc = kGatherThreads - dr * vpr;
#pragma unroll
  for (int k = 0; k < kGatherUnroll; ++k) {
    const bool in = e + k * kGatherThreads < total;
    q.r[k] = in ? r : 0;
    q.c[k] = in ? c : -1;
    const int64_t off = in ? int64_t(row0 + r) * row_bytes + int64_t(c) * V : int64_t(row0) * row_bytes;
    q.v[k] = __builtin_nontemporal_load(reinterpret_cast<const T*>(src + off));
    r += dr;
    c += dc;
    if (c >= vpr) {
      c -= vpr;
      ++r;
    }
  }
}

// Stores a round: item (r, c) to output row s_dst[r] (skipped when outside
// [0, A)).
template <int V>
__device__ __forceinline__ void store_round(const RowRound<V>& q, uint8_t* __restrict__ dst, int64_t row_bytes,
                                            int A, const int32_t* s_dst) {
  using T = typename VecT<V>::type;
#pragma unroll
  for (int k = 0; k < kGatherUnroll; ++k) {
    const int32_t d = s_dst[q.r[k]];
    if (q.c[k] >= 0 && static_cast<unsigned>(d) < static_cast<unsigned>(A))
      __builtin_nontemporal_store(q.v[k],
                                  reinterpret_cast<T*>(dst + int64_t(d) * row_bytes + int64_t(q.c[k]) * V));
  }
}

// All `rows` input rows from row0 on, vpr vectors each, to their output rows.
template <int V>
__device__ __forceinline__ void scatter_rows(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                             int64_t row_bytes, int vpr, int rows, int row0, int A,
                                             const int32_t* s_dst, int e_start = 0) {
  for (int e0 = e_start; e0 < rows * vpr; e0 += kGatherThreads * kGatherUnroll) {
    RowRound<V> q;
    load_round<V>(q, src, row_bytes, vpr, rows, row0, e0);
    store_round<V>(q, dst, row_bytes, A, s_dst);
  }
}

// The whole call for small count matrices, in input order: workgroup b owns
// the input rows [b * rows_per_wg, ...). It issues the loads of its first
// round of token vectors (and its scale pieces and weights) before anything
// else, then computes the offsets of the whole matrix in its LDS, with the
// output row of each of its input rows (the row map of the other direction),
// and stores everything there. The row loads and the count loads are in
// flight together, so a small call waits for one memory round trip before
// its offsets rather than two.
template <int V, int kSV, bool kScatter, bool kWeight, typename CountT>
__global__ __launch_bounds__(kGatherThreads) void fused_kernel(GatherArgs p, FusedArgs f) {
  extern __shared__ int32_t s_dyn[];
  __shared__ int32_t s_dst[kGatherThreads];                       // output row of input row row0 + t
  __shared__ int32_t s_mark[kGatherThreads];  // row marks
  __shared__ ScanShared<kGatherThreads> sh;
  const int tid = threadIdx.x;
  const int N = static_cast<int>(p.N);
  const int E = static_cast<int>(p.E);
  const int row0 = blockIdx.x * p.rows_per_wg;
  const int rows = min(p.rows_per_wg, p.A - row0);  // >= 1: the grid covers [0, A) exactly
  const int64_t Rs = p.scale_row_bytes;

  RowRound<V> q;
  load_round<V>(q, p.tokens, p.row_bytes, p.vecs_per_row, rows, row0, 0);
  using ST = typename VecT<(kSV > 0 ? kSV : 4)>::type;
  ST piece{};
  int sc_row = 0, sc_off = 0;
  bool sc_in = false;
  if (kSV > 0) {
    const int spr = static_cast<int>(Rs / kSV);  // pieces per scale row
    sc_row = tid / spr;
    sc_off = (tid - sc_row * spr) * kSV;
    sc_in = tid < rows * spr;
    const int64_t off = sc_in ? int64_t(row0 + sc_row) * Rs + sc_off : 0;
    piece = __builtin_nontemporal_load(reinterpret_cast<const ST*>(p.scales + off));
  }
  uint32_t wv = 0;
  if (kWeight) wv = p.weight[tid < rows ? row0 + tid : row0];

  int32_t* mats = s_dyn + 2 * (p.M + 1);  // counts and source offsets, [M] each
  int32_t* col = mats + 2 * p.M;          // [E + 1]
  int64_t total = 0;
  uint32_t flags;
  if (p.M <= 64) {  // uniform: every wave computes the offsets by itself and maps its 64 rows
    WaveCells w;
    flags = wave_offsets64<CountT>(static_cast<const CountT*>(f.counts), N, E, p.A, &w, &total);
    if (flags == 0) {
      const int32_t s = row0 + tid;
      const int32_t d = wave_map_row(w, p.M, p.inverse, s < p.A ? s : 0);
      s_dst[tid] = s < p.A ? d : -1;
      if (tid < 64) {
        if (w.first_row) col[w.expert] = static_cast<int32_t>(w.dst_cm);
        if (tid == 0) col[E] = static_cast<int32_t>(p.A);
      }
    }
  } else {
    flags = offsets_cells<kGatherThreads>(static_cast<const CountT*>(f.counts), N, E, p.A, p.inverse ? 0 : 1,
                                          mats, col, nullptr, &sh, &total, nullptr, row0, s_mark, s_dst);
  }
  if (flags != 0) {  // uniform: nothing is written for rejected counts
    if (blockIdx.x == 0 && tid == 0) write_header(p.hdr, p.A, p.N, p.E, total, flags, kCountsValid, p.inverse);
    return;
  }
  __syncthreads();  // every thread's s_dst entry, and the expert starts
  if (blockIdx.x == 0) {
    write_etn<kGatherThreads>(col, E, f.cumsum, static_cast<CountT*>(f.etn));
    if (tid == 0) write_header(p.hdr, p.A, p.N, p.E, total, 0, kCountsValid, p.inverse);
  }

  store_round<V>(q, p.out_tokens, p.row_bytes, p.A, s_dst);
  scatter_rows<V>(p.tokens, p.out_tokens, p.row_bytes, p.vecs_per_row, rows, row0, p.A, s_dst,
                  kGatherThreads * kGatherUnroll);
  if (kSV > 0 && sc_in) {
    const int32_t d = s_dst[sc_row];
    if (static_cast<unsigned>(d) < static_cast<unsigned>(p.A))
      __builtin_nontemporal_store(piece, reinterpret_cast<ST*>(p.out_scales + int64_t(d) * Rs + sc_off));
  }
  if (tid < rows) {
    const int32_t d = s_dst[tid];
    const int s = row0 + tid;
    if (static_cast<unsigned>(d) < static_cast<unsigned>(p.A)) {
      if (kScatter)
        p.idx[s] = d;
      else
        p.idx[d] = s;
      if (kWeight) p.out_weight[d] = wv;
    }
  }
  if (kSV == 0 && Rs > 0) {
    const int spr = p.scale_vecs_per_row;
    switch (p.scale_vec) {
      case 16: scatter_rows<16>(p.scales, p.out_scales, Rs, spr, rows, row0, p.A, s_dst); break;
      case 8: scatter_rows<8>(p.scales, p.out_scales, Rs, spr, rows, row0, p.A, s_dst); break;
      case 4: scatter_rows<4>(p.scales, p.out_scales, Rs, spr, rows, row0, p.A, s_dst); break;
      case 2: scatter_rows<2>(p.scales, p.out_scales, Rs, spr, rows, row0, p.A, s_dst); break;
      default: scatter_rows<1>(p.scales, p.out_scales, Rs, spr, rows, row0, p.A, s_dst); break;
    }
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

mrr_status launch_offsets(const Plan& pl, const mrr_args* a, void* ws, hipStream_t stream) {
  return pl.count_bytes == 8 ? launch_offsets_t<int64_t>(pl, a, ws, stream)
                             : launch_offsets_t<int32_t>(pl, a, ws, stream);
}

GatherArgs gather_args(const Plan& pl, const mrr_args* a, void* ws) {
  auto* base = static_cast<uint8_t*>(ws);
  GatherArgs g{};
  g.tokens = static_cast<const uint8_t*>(a->tokens);
  g.out_tokens = static_cast<uint8_t*>(a->permute_tokens);
  g.scales = static_cast<const uint8_t*>(a->per_token_scales);
  g.out_scales = static_cast<uint8_t*>(a->permute_per_token_scales);
  g.weight = reinterpret_cast<const uint32_t*>(a->expert_topk_weight);
  g.out_weight = reinterpret_cast<uint32_t*>(a->permute_topk_weight);
  g.idx = a->permute_token_idx;
  g.table = reinterpret_cast<const pair_t*>(base + pl.table_bytes);
  g.rowmap = reinterpret_cast<const int32_t*>(base + pl.rowmap_bytes);
  g.hdr = reinterpret_cast<WsHeader*>(base);
  g.row_bytes = pl.row_bytes;
  g.scale_row_bytes = pl.scale_row_bytes;
  g.N = pl.N;
  g.E = pl.E;
  g.vecs_per_row = static_cast<int32_t>(pl.vecs_per_row);
  g.scale_vecs_per_row = pl.scale_row_bytes > 0 ? static_cast<int32_t>(pl.scale_row_bytes / pl.scale_vec) : 0;
  g.scale_vec = pl.scale_vec;
  g.A = static_cast<int32_t>(pl.A);
  g.M = static_cast<int32_t>(pl.M);
  g.rows_per_wg = pl.rows_per_wg;
  g.inverse = pl.inverse ? 1 : 0;
  return g;
}

// Launches kernel K<V, SV, scatter, weight> (gather or fused) for the plan's
// token vector width, inline scale piece width and flags; `launch` receives a
// pointer to the instance. Inline scale pieces are only planned with 16-byte
// token vectors.
template <template <int, int, bool, bool> class K, typename Launch>
void dispatch(const Plan& pl, Launch&& launch) {
  auto flags = [&](auto vtag, auto stag) {
    constexpr int V = decltype(vtag)::value;
    constexpr int SV = decltype(stag)::value;
    if (pl.scatter) {
      if (pl.has_weight)
        launch(K<V, SV, true, true>::fn());
      else
        launch(K<V, SV, true, false>::fn());
    } else {
      if (pl.has_weight)
        launch(K<V, SV, false, true>::fn());
      else
        launch(K<V, SV, false, false>::fn());
    }
  };
  using I16 = std::integral_constant<int, 16>;
  using I0 = std::integral_constant<int, 0>;
  switch (pl.token_vec) {
    case 16:
      if (pl.scale_inline == 16)
        flags(I16{}, I16{});
      else if (pl.scale_inline == 4)
        flags(I16{}, std::integral_constant<int, 4>{});
      else
        flags(I16{}, I0{});
      break;
    case 8: flags(std::integral_constant<int, 8>{}, I0{}); break;
    case 4: flags(std::integral_constant<int, 4>{}, I0{}); break;
    case 2: flags(std::integral_constant<int, 2>{}, I0{}); break;
    default: flags(std::integral_constant<int, 1>{}, I0{}); break;
  }
}

template <int V, int SV, bool S, bool W>
struct GatherK {
  static auto fn() { return &gather_kernel<V, SV, S, W>; }
};
template <int V, int SV, bool S, bool W>
struct FusedK32 {
  static auto fn() { return &fused_kernel<V, SV, S, W, int32_t>; }
};
template <int V, int SV, bool S, bool W>
struct FusedK64 {
  static auto fn() { return &fused_kernel<V, SV, S, W, int64_t>; }
};

StreamGrid stream_grid(const Plan& pl) {
  StreamGrid sg;
  sg.tok_chunks = static_cast<uint32_t>(pl.tok_chunks);
  sg.sc_end = static_cast<uint32_t>(pl.tok_chunks + pl.sc_chunks);
  sg.small = static_cast<uint32_t>(pl.sc_chunks + pl.item_chunks);
  sg.inv_vpr = 1.0f / static_cast<float>(pl.vecs_per_row);
  sg.inv_svpr = pl.scale_row_bytes > 0 ? 1.0f / static_cast<float>(pl.scale_row_bytes / pl.scale_vec) : 0.0f;
  // cpr_magic = ceil(2^32 / cpr) puts umulhi(c, magic) at c / cpr or one above.
  sg.cpr = 0;
  sg.cpr_magic = 0;
  sg.byte_rows = pl.byte_rows ? 1u : 0u;
  sg.inv_row = 1.0f / static_cast<float>(pl.row_bytes);
  sg.rows8 = pl.byte_rows && pl.row_bytes >= 147 && pl.A >= 8 ? 1u : 0u;
  if (!pl.byte_rows && pl.vecs_per_row % 64 == 0) {
    sg.cpr = static_cast<uint32_t>(pl.vecs_per_row / 64);
    sg.cpr_magic = sg.cpr == 1 ? 0u : static_cast<uint32_t>(((uint64_t(1) << 32) + sg.cpr - 1) / sg.cpr);
  }
  return sg;
}

template <bool S, bool W>
void launch_stream_sw(const Plan& pl, const GatherArgs& g, hipStream_t stream) {
  const StreamGrid sg = stream_grid(pl);
  const dim3 grid(static_cast<unsigned>(pl.stream_grid)), block(64);
  switch (pl.token_vec) {
    case 16: hipLaunchKernelGGL((stream_gather_kernel<16, S, W>), grid, block, 0, stream, g, sg); break;
    case 8: hipLaunchKernelGGL((stream_gather_kernel<8, S, W>), grid, block, 0, stream, g, sg); break;
    case 4: hipLaunchKernelGGL((stream_gather_kernel<4, S, W>), grid, block, 0, stream, g, sg); break;
    case 2: hipLaunchKernelGGL((stream_gather_kernel<2, S, W>), grid, block, 0, stream, g, sg); break;
    default: hipLaunchKernelGGL((stream_gather_kernel<1, S, W>), grid, block, 0, stream, g, sg); break;
  }
}

mrr_status launch_gather(const Plan& pl, const mrr_args* a, void* ws, hipStream_t stream) {
  if (pl.A == 0) return MRR_SUCCESS;
  const GatherArgs g = gather_args(pl, a, ws);
  if (pl.stream) {
    if (pl.scatter)
      pl.has_weight ? launch_stream_sw<true, true>(pl, g, stream) : launch_stream_sw<true, false>(pl, g, stream);
    else
      pl.has_weight ? launch_stream_sw<false, true>(pl, g, stream) : launch_stream_sw<false, false>(pl, g, stream);
    return hipGetLastError() == hipSuccess ? MRR_SUCCESS : MRR_ERROR_HIP;
  }
  dispatch<GatherK>(pl, [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(pl.grid)), dim3(kGatherThreads), 0, stream, g);
  });
  return hipGetLastError() == hipSuccess ? MRR_SUCCESS : MRR_ERROR_HIP;
}

mrr_status launch_fused(const Plan& pl, const mrr_args* a, void* ws, hipStream_t stream) {
  const GatherArgs g = gather_args(pl, a, ws);
  FusedArgs f{};
  f.counts = a->expert_token_num_per_rank;
  f.etn = a->expert_token_num;
  f.cumsum = pl.cumsum ? 1 : 0;
  const size_t lds = static_cast<size_t>(fused_lds_bytes(pl.N, pl.E));
  auto launch = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(pl.grid)), dim3(kGatherThreads), lds, stream, g, f);
  };
  if (pl.count_bytes == 8)
    dispatch<FusedK64>(pl, launch);
  else
    dispatch<FusedK32>(pl, launch);
  return hipGetLastError() == hipSuccess ? MRR_SUCCESS : MRR_ERROR_HIP;
}

}  // namespace
}  // namespace mrr

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
