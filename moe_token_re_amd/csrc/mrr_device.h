// mrr_device.h -- the pieces the kernel files of the MoE re-routing operator
// (MoeReRoutingV2) share, for MI355X (gfx950, CDNA4: 64-lane waves, 256 CUs).
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
// The kernels (the design is ours, not the Ascend tiling the article sketches):
//   mrr_offsets.hip  the offsets phase: every kernel validates the counts,
//                    writes the status header and expert_token_num, and then
//                    what the plan's gather reads: the row map (the input row
//                    of every output row) or the (output offset, input offset)
//                    table in output order;
//   mrr_gather.hip   the gather phase: the stream gather (one 64-lane wave per
//                    chunk of 64 vectors of one output stream, row map) and the
//                    row-workgroup gather (table search);
//   mrr_fused.hip    the whole call in one launch for small count matrices;
//   mrr_one_launch.hip  the whole call in one launch of one-wave workgroups
//                    for count matrices of at most 512 cells and token rows
//                    of 16-byte vectors from 32 bytes, at any size;
//   mrr_entry.hip    the C entry points.
// This header holds the workgroup and wave scans, the count checks and the
// workspace header, the offsets of a count matrix in a workgroup's LDS (one
// cell per thread) and in one wave's registers (at most 64 cells), the gather
// arguments, and the launchers' declarations.
// No atomics on global memory; every output element is written exactly once,
// so results are deterministic.
#pragma once

#include <hip/hip_runtime.h>

#include <limits.h>
#include <stdint.h>

#include <type_traits>

#include "mrr_internal.h"

namespace mrr {

using pair_t = int32_t __attribute__((ext_vector_type(2)));  // (dst_off, src_off)

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

// A 16-byte store of streaming data written through the L2 (system scope sc1,
// non-temporal nt), where __builtin_nontemporal_store writes nt alone. On
// this chip it drains 1 KiB rows scattered over the output about 4% faster
// (a plain permuted copy of 7 KiB rows in 16x16 balanced cells: 37.2 against
// 38.8 us) and rows in order a little faster (35.8 against 36.0 us).
__device__ __forceinline__ void store16_through(void* p, VecT<16>::type v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1 nt" ::"v"(p), "v"(v) : "memory");
}

// The same at a uniform base plus a 32-bit offset.
__device__ __forceinline__ void store16_through(void* base, uint32_t off, VecT<16>::type v) {
  asm volatile("global_store_dwordx4 %0, %1, %2 sc1 nt" ::"v"(off), "v"(v), "s"(base) : "memory");
}

// A streaming store of a V-byte vector: 16-byte vectors written through the
// L2 as above, narrower ones non-temporal.
template <int V>
__device__ __forceinline__ void store_stream(typename VecT<V>::type* p, typename VecT<V>::type v) {
  if constexpr (V == 16)
    store16_through(p, v);
  else
    __builtin_nontemporal_store(v, p);
}

// floor(n / d) for n < 2^31 and 2 <= d < 2^16, with magic = ceil(2^32 / d):
// the multiply-high is the quotient or one more.
__device__ __forceinline__ uint32_t div_magic(uint32_t n, uint32_t d, uint32_t magic) {
  const uint32_t q = __umulhi(n, magic);
  return q - (q * d > n ? 1u : 0u);
}

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
  int64_t block_base;      // gather_kernel: workgroups of earlier launches of the same call
};

struct FusedArgs {
  const void* counts;
  void* etn;
  int32_t cumsum;
};

// The one-launch stream kernel's own arguments (count matrices of at most 512
// cells, token rows of whole 16-byte vectors, at least 32 bytes).
struct StreamFusedArgs {
  const void* counts;
  void* etn;
  int32_t cumsum;
  int32_t item_waves;  // workgroups [0, item_waves) move the per-row items, 64 rpl output rows each
  int32_t rpl;         // output rows per lane of an item wave: 4, or 1 for scale rows over 16 bytes
  int32_t idx16;       // permute_token_idx is 16-byte aligned (four rows' indices in one store)
  int32_t w16;         // permute_topk_weight is 16-byte aligned (the same for the weights)
  uint32_t vpr;        // 16-byte vectors per token row (at least 2)
  uint32_t vpr_magic;  // ceil(2^32 / vpr): n / vpr by a multiply-high and one correction (n < 2^32)
  uint32_t vectors;    // A * vpr: the token vectors of the call
  int32_t minor;       // cells per major index in input order: E forward, N inverse
  int32_t major;       // N forward, E inverse
  float inv_minor;     // 1 / minor
  float inv_spr;       // 1 / (scale vectors per row), when there are scales
  float inv_vpr;       // 1 / vpr
  // Token rows that are no multiple of 16 bytes (0 otherwise): the row
  // length in bytes (at least 17), ceil(2^32 / rbytes), and A * rbytes
  // (below 2^31).
  uint32_t rbytes;
  uint32_t rb_magic;
  uint32_t tbytes;
  // The output-order position of each input-order cell: it depends on N, E
  // and the direction alone, so the host computes it once instead of every
  // wave. With 4 cells a lane (at most 256 cells), cell m = 4 l + k in byte k
  // of outpos[l]; with 8 (at most 512), cell m = 8 l + k in bits
  // [16 (k % 2), 16 (k % 2) + 16) of outpos[4 l + k / 2]. 0 past the matrix.
  alignas(16) uint32_t outpos[256];
};

namespace {

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

// Inclusive scan over the 64 lanes of a wave (wrapping 32-bit adds) in DPP
// alone, with no LDS: row shifts by 1, 2, 4 and 8 scan each row of 16 lanes,
// then row_bcast:15 adds lane 15's total to row 1 and lane 47's to row 3, and
// row_bcast:31 adds lane 31's (rows 0-1) to rows 2 and 3; rows outside a
// step's row mask keep their value. Every lane of the wave must be active.
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t v) {
  constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
  constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kRowShr1, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kRowShr2, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kRowShr4, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kRowShr8, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kRowBcast15, 0xa, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kRowBcast31, 0xc, 0xf, false));
  return v;
}

// Sum over the 64 lanes of a wave (wrapping 32-bit adds), in every lane.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return __builtin_amdgcn_readlane(wave_scan_u32(v), 63);
}

// Exact sum over the 64 lanes of a wave of values below 2^42, without LDS:
// the low 16 and the high 26 bits are summed apart with the DPP scan (64
// terms below 2^26 sum below 2^32) and recombined.
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
      const uint64_t ws = wave_sum_u42(exact[k]);
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
  uint32_t wflags[kThreads / 64];  // each wave's rejection flags, published with its scan totals
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
// raw is the thread's count (row-major cell tid; anything past the matrix),
// loaded by the caller ahead of its other loads so that the offsets wait for
// it alone. Returns 0, or the rejection flags (the same in every thread; then
// tab and col are not written).
template <int kThreads, typename CountT>
__device__ uint32_t offsets_cells(CountT raw, int N, int E, int64_t A, int inverse,
                                  int32_t* lds, int32_t* col, pair_t* tab, ScanShared<kThreads>* sh,
                                  int64_t* total_out, int32_t* __restrict__ rowmap = nullptr, int row0 = 0,
                                  int32_t* s_mark = nullptr, int32_t* s_map = nullptr) {
  const bool mapping = rowmap != nullptr || s_map != nullptr;
  const int tid = threadIdx.x;
  const int M = N * E;
  int32_t* s_c = lds;      // counts, column-major
  int32_t* s_s = lds + M;  // SrcOffset, column-major
  for (int j = tid; j <= E; j += kThreads) col[j] = 0;
  if (mapping) s_mark[tid] = -1;
  uint32_t flags = 0;
  // Thread t holds cell t in row-major (rank i, expert j) order.
  const bool in = tid < M;
  uint32_t c = 0;
  if (in) c = static_cast<uint32_t>(clamp_count(raw, &flags));
  const int ci = in ? tid / E : 0;
  const int cj = tid - ci * E;
  if (in) s_c[cj * N + ci] = static_cast<int32_t>(c);  // column-major, ordered by the scan's barrier
  // The wave's rejection flags go out with its scan totals: the scan's barrier
  // publishes both.
  {
    uint32_t wf = 0;
    if (__builtin_amdgcn_ballot_w64((flags & kFlagNegative) != 0) != 0) wf |= kFlagNegative;
    if (__builtin_amdgcn_ballot_w64((flags & kFlagTooLarge) != 0) != 0) wf |= kFlagTooLarge;
    if ((tid & 63) == 0) sh->wflags[tid >> 6] = wf;
  }
  uint64_t total;
  const uint32_t src = block_scan_u32<kThreads, true>(c, c, sh->w[0], sh->t[0], &total);
  flags = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) flags |= sh->wflags[w];
  if (in) s_s[cj * N + ci] = static_cast<int32_t>(src);
  *total_out = static_cast<int64_t>(total);
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

// expert_token_num from the expert starts col[0..E]: expert j's rows are
// [col[j], col[j+1]); the cumsum form is the inclusive total col[j+1].
template <int kThreads, typename CountT>
__device__ __forceinline__ void write_etn(const int32_t* col, int E, int cumsum, CountT* __restrict__ etn) {
  for (int j = threadIdx.x; j < E; j += kThreads)
    etn[j] = static_cast<CountT>(cumsum ? col[j + 1] : col[j + 1] - col[j]);
}





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

// The raw count of row-major cell threadIdx.x, 0 past the matrix (no load:
// the count pointer may be null when the matrix has no cells).
template <typename CountT>
__device__ __forceinline__ CountT load_count(const CountT* __restrict__ counts, int M) {
  return static_cast<int>(threadIdx.x) < M ? counts[threadIdx.x] : CountT(0);
}

// The raw count of the cell a lane of a wave holds in wave_offsets64 (lane q:
// row-major cell q), 0 past the matrix. Loaded by the caller ahead of other
// loads, so that the offsets wait for it alone.
template <typename CountT>
__device__ __forceinline__ CountT load_count64(const CountT* __restrict__ counts, int M) {
  const int lane = threadIdx.x & 63;
  return lane < M ? counts[lane] : CountT(0);
}

// Returns the rejection flags (the same in every lane) and, in *total, the
// exact sum of the clamped counts; raw is load_count64's value. All 64 lanes
// must be active.
template <typename CountT>
__device__ __forceinline__ uint32_t wave_offsets64(CountT raw, int N, int E, int64_t A, WaveCells* w,
                                                   int64_t* total) {
  const int lane = threadIdx.x & 63;
  const int M = N * E;
  uint32_t f = 0;
  const uint32_t c = lane < M ? static_cast<uint32_t>(clamp_count(raw, &f)) : 0u;
  const uint64_t tot = wave_sum_u42(c);
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

}  // namespace

// ---------------------------------------------------------------------------
// Launchers (host), one per kernel file
// ---------------------------------------------------------------------------

mrr_status launch_offsets(const Plan& pl, const mrr_args* a, void* ws, hipStream_t stream);
mrr_status launch_gather(const Plan& pl, const mrr_args* a, void* ws, hipStream_t stream);
mrr_status launch_fused(const Plan& pl, const mrr_args* a, void* ws, hipStream_t stream);
mrr_status launch_stream_fused(const Plan& pl, const mrr_args* a, void* ws, hipStream_t stream);
GatherArgs gather_args(const Plan& pl, const mrr_args* a, void* ws);

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

}  // namespace mrr
