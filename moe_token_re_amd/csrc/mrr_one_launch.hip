// mrr_one_launch.hip -- the whole MoE re-routing call (MoeReRoutingV2, page
// "CANN ops-transformer MoeReRoutingV2": the offsets and moves of "计算公式",
// permute_token_idx and expert_token_num of "参数说明") in one launch of
// 64-lane workgroups, for count matrices of at most 512 cells, token rows of
// 16-byte vectors and at least 32 bytes (or, in the byte form, of any length
// from 17 bytes), and scale rows of at most 4 KiB, at any size. Workgroups
// [0, item_waves) move the per-row items and scale rows of 64 rpl output rows
// each; every later workgroup moves one 1 KiB chunk of the input token rows,
// in input order, so that its token load goes out at once (beside the count
// load); it then works out where the chunk's rows go from the counts while
// the load is in flight. Every wave checks the counts itself and writes
// nothing when they are rejected; workgroup 0 writes expert_token_num and the
// status. A lane holds kC cells of the matrix: 4 up to 256 cells, 8 up to 512.
#include "mrr_device.h"

namespace mrr {
namespace {

constexpr int kItemWaveRows = 4 * 64;  // the most output rows of an item wave (four per lane)
constexpr int kScaleRound = 4;         // scale vectors per lane loaded before they are stored

// The host's output-position table: with kC = 4 one word a lane, a byte a
// cell; with kC = 8 four words a lane, 16 bits a cell (positions reach 511).
// Cell m = kC l + k of lane l sits in word kWords l + k kBits / 32, from bit
// (k kBits) % 32.
template <int kC>
struct PosFmt {
  static constexpr int kBits = kC == 4 ? 8 : 16;
  static constexpr int kWords = kC * kBits / 32;
  static constexpr uint32_t kMask = (1u << kBits) - 1u;
};

// The raw counts of this lane's cells m = kC lane + k in input order
// (forward: row-major (rank, expert), the order of SrcOffset; inverse:
// column-major); past the matrix, the matrix's first counts, until mask_cells
// or order_cells sets them to 0. Every wave reads the whole matrix, so the
// number of load instructions matters: with kVec (the counts 16-byte aligned,
// M a multiple of 4) each group of four counts comes in one 16-byte load (two
// for int64) in matrix order, and the inverse puts them in column-major order
// afterwards through LDS (order_cells); else in one load a cell. kVec is a
// template choice, not a branch: at a join of two load paths the compiler
// would wait for the counts before the token load goes out.
template <typename CountT, int kC>
struct RawCells {
  CountT r[kC];
  uint32_t pos[PosFmt<kC>::kWords];  // this lane's words of the output-position table
};

// kCalc (eight cells a lane, the minor dimension a multiple of 8): the
// lane's words of the position table computed instead of loaded. Its eight
// cells m = 8 lane + k then share one major index a = 8 lane / minor, and
// cell m's position is (8 lane - a minor + k) major + a (0 past the matrix).
template <typename CountT, int kC, bool kVec, bool kInv, bool kCalc>
__device__ __forceinline__ void load_cells(const CountT* __restrict__ counts, int M, const StreamFusedArgs& f,
                                           RawCells<CountT, kC>& rc) {
  using PF = PosFmt<kC>;
  const int lane = threadIdx.x & 63;
  if constexpr (kCalc) {
    static_assert(kC == 8, "computed positions: eight cells a lane");
    const int m0 = kC * lane;
    const int a = div_small(m0, f.inv_minor);
    const uint32_t b0 = static_cast<uint32_t>(m0 - a * f.minor);
#pragma unroll
    for (int j = 0; j < PF::kWords; ++j) {
      const uint32_t lo = m0 + 2 * j < M ? (b0 + 2 * j) * f.major + a : 0u;
      const uint32_t hi = m0 + 2 * j + 1 < M ? (b0 + 2 * j + 1) * f.major + a : 0u;
      rc.pos[j] = lo | (hi << 16);
    }
  } else {
#pragma unroll
    for (int j = 0; j < PF::kWords; ++j) rc.pos[j] = f.outpos[PF::kWords * lane + j];
  }
  if (kVec) {
#pragma unroll
    for (int g = 0; g < kC / 4; ++g) {
      const int m0 = kC * lane + 4 * g;
      const bool in = m0 < M;  // then all four cells are (M % 4 == 0)
      const CountT* q = counts + (in ? m0 : 0);
      CountT r[4];
      if (sizeof(CountT) == 4) {
        using I4 = int32_t __attribute__((ext_vector_type(4)));
        const I4 v = *reinterpret_cast<const I4*>(q);
        r[0] = static_cast<CountT>(v.x);
        r[1] = static_cast<CountT>(v.y);
        r[2] = static_cast<CountT>(v.z);
        r[3] = static_cast<CountT>(v.w);
      } else {
        using L2 = int64_t __attribute__((ext_vector_type(2)));
        const L2 v0 = reinterpret_cast<const L2*>(q)[0];
        const L2 v1 = reinterpret_cast<const L2*>(q)[1];
        r[0] = static_cast<CountT>(v0.x);
        r[1] = static_cast<CountT>(v0.y);
        r[2] = static_cast<CountT>(v1.x);
        r[3] = static_cast<CountT>(v1.y);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) rc.r[4 * g + k] = r[k];
    }
    return;
  }
  // Addresses first (no branch between the loads: at its join the compiler
  // would wait for the earlier ones). Inverse, cell (rank b, expert a) of the
  // column-major order sits at b * E + a.
  int at[kC];
#pragma unroll
  for (int k = 0; k < kC; ++k) {
    const int m = kC * lane + k;
    int cm = m;
    if (kInv) {
      const int a = div_small(m, f.inv_minor);
      cm = (m - a * f.minor) * f.major + a;
    }
    at[k] = m < M ? cm : 0;  // M >= 1 here
  }
#pragma unroll
  for (int k = 0; k < kC; ++k) rc.r[k] = counts[at[k]];
}

// The loaded counts past the matrix (read from its start) set to 0; not
// needed after order_cells, which does the same.
template <typename CountT, int kC, bool kVec, bool kInv>
__device__ __forceinline__ void mask_cells(RawCells<CountT, kC>& rc, int M) {
  if (kVec && kInv) return;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < kC; ++k) rc.r[k] = kC * lane + k < M ? rc.r[k] : CountT(0);
}

// The position of each of this lane's cells in output order, from the host's
// table (cell (major a, minor b) of the input order is cell b * major + a of
// the output order). Past the matrix the table holds 0 (those cells count 0
// and are never looked up or written).
template <int kC>
__device__ __forceinline__ void cell_positions(const uint32_t (&pos)[PosFmt<kC>::kWords], uint32_t (&out)[kC]) {
  using PF = PosFmt<kC>;
#pragma unroll
  for (int k = 0; k < kC; ++k) out[k] = (pos[k * PF::kBits / 32] >> ((k * PF::kBits) % 32)) & PF::kMask;
}

// The position of cell m in output order, in every lane (pos: this lane's
// words of the table). The word is chosen by the bits of m (named values,
// not an index into the array, which would put it in scratch memory).
template <int kC>
__device__ __forceinline__ uint32_t cell_position(const uint32_t (&pos)[PosFmt<kC>::kWords], int m) {
  if constexpr (kC == 4) {
    return (__builtin_amdgcn_readlane(pos[0], m >> 2) >> (8 * (m & 3))) & 0xffu;
  } else {
    const uint32_t lo = (m & 2) ? pos[1] : pos[0], hi = (m & 2) ? pos[3] : pos[2];
    return (__builtin_amdgcn_readlane((m & 4) ? hi : lo, m >> 3) >> (16 * (m & 1))) & 0xffffu;
  }
}

// With kVec and the inverse direction: the counts loaded in matrix order
// (row-major) rearranged into column-major order through s_c (M counts), one
// LDS write a group of four and one read a cell. Called after the token load
// is issued. The LDS operations of one wave complete in order, so the reads
// see the writes; the compiler barriers keep the LDS accesses of the callers
// (other types, same words) on their side.
template <typename CountT, int kC, bool kVec, bool kInv>
__device__ __forceinline__ void order_cells(RawCells<CountT, kC>& rc, CountT* s_c, int M) {
  if (!kVec || !kInv) return;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int g = 0; g < kC / 4; ++g)
    if (kC * lane + 4 * g < M) {
#pragma unroll
      for (int k = 0; k < 4; ++k) s_c[kC * lane + 4 * g + k] = rc.r[4 * g + k];
    }
  __builtin_amdgcn_wave_barrier();
  // Inverse, the output order is the matrix order: the output position of
  // input-order cell m is its matrix index (rank * E + expert).
  uint32_t p[kC];
  cell_positions<kC>(rc.pos, p);
#pragma unroll
  for (int k = 0; k < kC; ++k) {
    const CountT v = s_c[p[k]];  // s_c[0] past the matrix
    rc.r[k] = kC * lane + k < M ? v : CountT(0);
  }
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// What every wave derives from its cells: the counts, each cell's input
// offset (the exclusive prefix in input order: SrcOffset forward, DstOffset
// inverse), and the verdict on the whole matrix. Exactness: each count is
// below 2^31 (larger ones are flagged). While every count is below 2^22 the
// at most 512 of them sum below 2^31, so the wrapping 32-bit sum is exact.
// Otherwise (rare: a cell of 4M rows or more), with H the sum of the counts'
// bits from 2^20 up, the true sum lies below H 2^20 + 2^29; while H < 1024 it
// is below 2^32 and the wrapping sum is exact, and a valid matrix sums to
// A < 2^30 (the plan sends only A < 2^30 here), so its H is below 1024.
template <int kC>
struct InCells {
  int32_t c[kC];
  uint32_t start[kC];
  uint32_t total;  // uniform: the wrapping 32-bit sum
  uint32_t flags;  // uniform: kFlag* of the whole matrix (0: valid)
};

// kFlags: the flags say why the counts are rejected (item waves: workgroup 0
// writes them to the header); without it (token waves) any rejection shows
// as kFlagNegative, which is enough to write nothing and costs fewer
// instructions (a count is in [0, 2^31) when its bits from 31 up are 0; the
// sums and scans over a rejected matrix are never used).
template <typename CountT, int kC, bool kFlags>
__device__ __forceinline__ void finish_cells(const RawCells<CountT, kC>& rc, int A, InCells<kC>& w) {
  uint32_t fl = 0;
  uint32_t own = 0;
  uint32_t any = 0;  // the OR of the counts (>= 0 here)
#pragma unroll
  for (int k = 0; k < kC; ++k) {
    if (kFlags) {
      w.c[k] = clamp_count(rc.r[k], &fl);
    } else {
      // the low word as the count; an int64 count's high word must be 0
      const uint64_t u = static_cast<uint64_t>(static_cast<int64_t>(rc.r[k]));
      w.c[k] = static_cast<int32_t>(static_cast<uint32_t>(u));
      if (sizeof(CountT) == 8) fl |= static_cast<uint32_t>(u >> 32);
    }
    own += static_cast<uint32_t>(w.c[k]);
    any |= static_cast<uint32_t>(w.c[k]);
  }
  // Without kFlags, a count outside [0, 2^31) sets bit 31 of the OR of the
  // low words or a bit of an int64 high word.
  if (!kFlags) fl |= any >> 31;
  const uint32_t incl = wave_scan_u32(own);
  w.total = __builtin_amdgcn_readlane(incl, 63);
  w.start[0] = incl - own;
#pragma unroll
  for (int k = 1; k < kC; ++k) w.start[k] = w.start[k - 1] + static_cast<uint32_t>(w.c[k - 1]);
  uint32_t flags = kFlags ? (__ballot(fl & kFlagNegative) != 0 ? kFlagNegative : 0u) |
                                (__ballot(fl & kFlagTooLarge) != 0 ? kFlagTooLarge : 0u)
                          : (__ballot(fl != 0) != 0 ? kFlagNegative : 0u);
  if (__ballot(any >= (1u << 22)) != 0) {  // uniform and rare
    uint32_t hi = 0;
#pragma unroll
    for (int k = 0; k < kC; ++k) hi += static_cast<uint32_t>(w.c[k]) >> 20;
    if (wave_sum_u32(hi) >= 1024u) flags |= kFlagSumMismatch;
  }
  if (w.total != static_cast<uint32_t>(A)) flags |= kFlagSumMismatch;
  w.flags = flags;
}

// v[k] of the lane holding cell m (k = m % kC), in every lane: every lane
// selects its own v[k] by the bits of k (named values, not an index into the
// array, which would put it in scratch memory), then that lane is read.
template <int kC>
__device__ __forceinline__ uint32_t cell_value(const uint32_t (&v)[kC], int m) {
  const bool b0 = (m & 1) != 0, b1 = (m & 2) != 0;
  const uint32_t v0 = v[0], v1 = v[1], v2 = v[2], v3 = v[3];
  const uint32_t lo = b0 ? v1 : v0, hi = b0 ? v3 : v2;
  const uint32_t q0 = b1 ? hi : lo;  // v[m % 4]
  if constexpr (kC == 4) {
    return __builtin_amdgcn_readlane(q0, m >> 2);
  } else {
    const uint32_t v4 = v[4], v5 = v[5], v6 = v[6], v7 = v[7];
    const uint32_t lo1 = b0 ? v5 : v4, hi1 = b0 ? v7 : v6;
    const uint32_t q1 = b1 ? hi1 : lo1;  // v[4 + m % 4]
    return __builtin_amdgcn_readlane((m & 4) ? q1 : q0, m >> 3);
  }
}

// The cell holding input row s (the last one that starts at or before it),
// in every lane; 0 when the counts are rejected and no cell qualifies.
template <int kC>
__device__ __forceinline__ int cell_of(uint32_t s, const InCells<kC>& w) {
  int m = -1;
#pragma unroll
  for (int k = 0; k < kC; ++k) m += __popcll(__ballot(w.start[k] <= s));
  return max(m, 0);
}

// The output row of input row s in cell m: the cell's output offset (the
// counts of the cells before it in output order) plus s's place in the cell.
template <int kC>
__device__ __forceinline__ uint32_t dest_row(uint32_t s, int m, const InCells<kC>& w,
                                             const uint32_t (&pos)[PosFmt<kC>::kWords], const uint32_t (&outp)[kC]) {
  const uint32_t out_m = cell_position<kC>(pos, m);
  uint32_t before = 0;
#pragma unroll
  for (int k = 0; k < kC; ++k) before += outp[k] < out_m ? static_cast<uint32_t>(w.c[k]) : 0u;
  return wave_sum_u32(before) + (s - cell_value<kC>(w.start, m));
}

// Token wave c: the 16-byte vectors [64 c, 64 c + 64) of the input token rows
// taken as one stream (input order, vpr >= 2 vectors a row), one load and
// store per lane: this chip streams fastest with one-wave workgroups of one
// load each (two chunks a wave measured slower). The load needs no offsets.
// The chunk covers rows s0 .. s_last. When they all lie in one cell (always
// for a single row), they go to consecutive output rows, so the chunk's 1 KiB
// lands contiguous from output row d0 on. Otherwise each lane finds its row,
// and a walk over the cells the chunk touches gives each row its output row.
template <typename CountT, int kC, bool kVec, bool kInv, bool kCalc>
__device__ __forceinline__ void stream_fused_tokens(const GatherArgs& p, const StreamFusedArgs& f, uint32_t c,
                                                    uint32_t* s_lds) {
  using T = VecT<16>::type;
  const int lane = threadIdx.x & 63;
  const uint32_t n0 = c * 64u;  // the chunk's first vector; A * vpr < 2^32 (the plan checks)
  // s0 = n0 / vpr: the multiply-high is the quotient or one above
  const uint32_t q = __umulhi(n0, f.vpr_magic);
  const uint32_t s0 = __builtin_amdgcn_readfirstlane(q - (q * f.vpr > n0 ? 1u : 0u));
  const uint32_t v = n0 + static_cast<uint32_t>(lane);
  const bool in = v < f.vectors;  // the last chunk may be partial
  const uint32_t lane16 = static_cast<uint32_t>(lane) * 16u;
  RawCells<CountT, kC> rc;
  load_cells<CountT, kC, kVec, kInv, kCalc>(static_cast<const CountT*>(f.counts), p.M, f, rc);
  // a uniform base and a 32-bit lane offset (a lane past the end reads the chunk's first vector)
  const uint8_t* tok = p.tokens + static_cast<uint64_t>(n0) * 16u;
  const T x = __builtin_nontemporal_load(reinterpret_cast<const T*>(tok + (in ? lane16 : 0u)));
  // The offsets below wait for the counts alone (loads return in issue
  // order). The compiler would otherwise sink the token load below them, next
  // to its store: this barrier names the token buffer, so the load stays here.
  // The count and position registers then pass through empty statements after
  // it, so no arithmetic on them (and no wait for them) is scheduled ahead of
  // the token load either.
  asm volatile("" ::"s"(p.tokens) : "memory");
#pragma unroll
  for (int k = 0; k < kC; ++k) asm volatile("" : "+v"(rc.r[k]));
#pragma unroll
  for (int j = 0; j < PosFmt<kC>::kWords; ++j) asm volatile("" : "+v"(rc.pos[j]));
  mask_cells<CountT, kC, kVec, kInv>(rc, p.M);
  order_cells<CountT, kC, kVec, kInv>(rc, reinterpret_cast<CountT*>(s_lds), p.M);
  InCells<kC> w;
  finish_cells<CountT, kC, false>(rc, p.A, w);
  uint32_t outp[kC];
  cell_positions<kC>(rc.pos, outp);
  const int m0 = cell_of<kC>(s0, w);
  const uint32_t d0 = dest_row<kC>(s0, m0, w, rc.pos, outp);
  // the chunk's last row (s0 when the rows are whole KiB), and its cell
  uint32_t s_last = s0;
  if (f.vpr % 64u != 0) {  // uniform
    const uint32_t n_last = min(n0 + 63u, f.vectors - 1u);
    const uint32_t ql = __umulhi(n_last, f.vpr_magic);
    s_last = __builtin_amdgcn_readfirstlane(ql - (ql * f.vpr > n_last ? 1u : 0u));
  }
  const int m_last = s_last == s0 ? m0 : cell_of<kC>(s_last, w);
  if (m_last == m0) {  // uniform (every chunk when the rows are whole KiB; most of them otherwise)
    uint8_t* out = p.out_tokens + static_cast<uint64_t>(d0) * static_cast<uint64_t>(p.row_bytes) +
                   static_cast<uint64_t>(n0 - s0 * f.vpr) * 16u;
    if (w.flags == 0 && in && d0 + (s_last - s0) < static_cast<uint32_t>(p.A))
      store16_through(out, lane16, x);
    return;
  }
  if (w.flags != 0) return;  // uniform: rejected counts
  // this lane's row: t < 64 + vpr vectors past the start of row s0 (div_small is exact below 2^12)
  const uint32_t t = v - s0 * f.vpr;
  const uint32_t r = s0 + (f.vpr >= 64 ? (t >= f.vpr ? 1u : 0u) : static_cast<uint32_t>(div_small(t, f.inv_vpr)));
  uint32_t cnt[kC];
#pragma unroll
  for (int k = 0; k < kC; ++k) cnt[k] = static_cast<uint32_t>(w.c[k]);
  uint32_t d = 0xffffffffu;  // (stays out of range, so unstored, if no cell held the row)
  for (int m = m0; m <= m_last; ++m) {  // uniform: the cells of rows s0 .. s_last, in input order
    const uint32_t n = cell_value<kC>(cnt, m);
    if (n == 0) continue;
    const uint32_t st = cell_value<kC>(w.start, m);
    const uint32_t om = dest_row<kC>(st, m, w, rc.pos, outp);  // the cell's output offset
    if (r - st < n) d = om + (r - st);
  }
  if (in && d < static_cast<uint32_t>(p.A))
    store16_through(p.out_tokens + int64_t(d) * p.row_bytes + int64_t(v - r * f.vpr) * 16, x);
}

// Bytes [0, n) of v (n <= 16) to dst, one byte store each: the output
// blocks that hold bytes of two cells, whose other bytes another wave writes.
__device__ __forceinline__ void store_bytes(uint8_t* dst, const VecT<16>::type& v, uint32_t n) {
  const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (uint32_t k = 0; k < 16; ++k)
    if (k < n) dst[k] = static_cast<uint8_t>(wd[k >> 2] >> (8 * (k & 3)));
}

// Token wave c for token rows that are no multiple of 64 bytes (R >= 17, both
// token buffers 16-byte aligned, A R < 2^31): the rows taken as one byte
// stream, the wave owns the bytes [base, base + 1 KiB), base = 1024 c, and
// loads the 68 aligned 16-byte blocks from base (64 and then 4 more, before
// the offsets, as above). A cell's rows are one byte range on both sides,
// moved by delta = (output row - input row) R bytes. Stores are grouped by
// aligned 64-byte segments of the output: every block of a cell in a segment
// is written by the wave that owns the first of the cell's input bytes in that
// segment, so no two waves write parts of one segment except where two cells
// meet in the output. (This chip streams a permuted copy fastest when each
// wave writes a whole 1 KiB: waves whose 1 KiB of output starts at 16 bytes
// past a 64-byte boundary ran 13-22% slower, at 64 bytes past it 1-3%, and
// waves of fewer bytes slower still: 960-byte waves 17%, under a permutation
// of 256 cells.) An aligned output block whose bytes all come from one cell
// is input bytes [x, x + 16), x = 16 o - delta, the blocks (x - base) / 16 and
// the next funnel-shifted by sh = -delta mod 16: the lanes read them from the
// blocks staged in LDS. With the wave inside one cell it writes the 1 KiB of
// output from the first segment whose input starts at or after base, block j
// by lane j. A cell's first block, when it also holds bytes of the output
// row before (its head), and its last, when it holds bytes of the row after
// (its tail), are written byte by byte; the other cell's wave writes the rest
// of them.
constexpr int kByteBlocks = 68;  // blocks staged per wave: a segment starting at byte 1023 ends before 1088

// Stages this wave's blocks in LDS (after the values u, v, b that the stores
// need are computed: the empty statement takes them and hands x on, so that
// the compiler computes them before it waits for the token loads).
__device__ __forceinline__ void stage_blocks(VecT<16>::type* s_blk, VecT<16>::type& x, VecT<16>::type& xb,
                                             uint32_t u, uint32_t v, bool b) {
  asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w), "+v"(xb.x), "+v"(xb.y), "+v"(xb.z), "+v"(xb.w)
               : "s"(u), "v"(v), "v"(static_cast<uint32_t>(b)));
  const int lane = threadIdx.x & 63;
  s_blk[lane] = x;
  if (lane < kByteBlocks - 64) s_blk[64 + lane] = xb;
  __builtin_amdgcn_wave_barrier();
}

// The 16 staged bytes from byte k of the wave's stream: five words from LDS
// from word k / 4 on, then byte funnel shifts (no branch on the shift). For a
// tail block near the end of the staged bytes the last words lie past them,
// inside the LDS array; their bytes are never stored.
__device__ __forceinline__ VecT<16>::type staged16(const VecT<16>::type* s_blk, uint32_t k) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(s_blk) + (k >> 2);
  const uint32_t r = k & 3u;
  const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3], w4 = w[4];
  VecT<16>::type o;
  o.x = __builtin_amdgcn_alignbyte(w1, w0, r);
  o.y = __builtin_amdgcn_alignbyte(w2, w1, r);
  o.z = __builtin_amdgcn_alignbyte(w3, w2, r);
  o.w = __builtin_amdgcn_alignbyte(w4, w3, r);
  return o;
}

template <typename CountT, int kC, bool kVec, bool kInv, bool kCalc>
__device__ __forceinline__ void stream_fused_bytes(const GatherArgs& p, const StreamFusedArgs& f, uint32_t c,
                                                   uint32_t* s_lds) {
  using T = VecT<16>::type;
  const int lane = threadIdx.x & 63;
  const uint32_t base = c * 1024u;  // < A R < 2^31
  const uint32_t tb = f.tbytes, rb = f.rbytes;
  const uint32_t lane16 = static_cast<uint32_t>(lane) * 16u;
  RawCells<CountT, kC> rc;
  load_cells<CountT, kC, kVec, kInv, kCalc>(static_cast<const CountT*>(f.counts), p.M, f, rc);
  // Only blocks that hold bytes of the stream are loaded (a lane past the end
  // reads the chunk's first block): such a block never crosses a page. Lane l
  // also loads block 64 + l % 4, the next wave's first bytes. Plain loads,
  // which the cache then often serves to the other wave (16x16 counts,
  // 7169-byte rows, 112 MiB: 40.2 us per call against 42.3 with
  // non-temporal loads, 39.1 with no extra load at all (wrong results); both
  // loads plain 39.9).
  const uint8_t* tok = p.tokens + base;
  const uint32_t lb = 1024u + 16u * static_cast<uint32_t>(lane & 3);
  T x = *reinterpret_cast<const T*>(tok + (base + lane16 < tb ? lane16 : 0u));
  T xb = *reinterpret_cast<const T*>(tok + (base + lb < tb ? lb : 0u));
  // as in stream_fused_tokens: the loads stay ahead of the offsets arithmetic
  asm volatile("" ::"s"(p.tokens) : "memory");
#pragma unroll
  for (int k = 0; k < kC; ++k) asm volatile("" : "+v"(rc.r[k]));
#pragma unroll
  for (int j = 0; j < PosFmt<kC>::kWords; ++j) asm volatile("" : "+v"(rc.pos[j]));
  mask_cells<CountT, kC, kVec, kInv>(rc, p.M);
  order_cells<CountT, kC, kVec, kInv>(rc, reinterpret_cast<CountT*>(s_lds), p.M);
  InCells<kC> w;
  finish_cells<CountT, kC, false>(rc, p.A, w);
  if (w.flags != 0) return;  // uniform: rejected counts
  uint32_t outp[kC];
  cell_positions<kC>(rc.pos, outp);
  T* s_blk = reinterpret_cast<T*>(s_lds);  // the counts in LDS (order_cells) are in registers by now
  const uint32_t s0 = __builtin_amdgcn_readfirstlane(div_magic(base, rb, f.rb_magic));
  const int m0 = cell_of<kC>(s0, w);
  const uint32_t d0 = dest_row<kC>(s0, m0, w, rc.pos, outp);
  // Fast path: the cell of row s0 holds the input of the 1 KiB of output from
  // the first segment whose input starts at base + sh64 (sh64 = -delta mod
  // 64), [base + sh64, base + sh64 + 1024), and starts before base (or sh64
  // == 0: no head segment).
  const uint32_t delta = (d0 - s0) * rb;  // mod 2^32: output byte = input byte + delta
  const uint32_t sh64 = (0u - delta) & 63u;
  const uint32_t reach = base + sh64 + 1024u;
  bool fast = false;
  if (reach <= tb) {  // uniform
    const uint32_t s_e = __builtin_amdgcn_readfirstlane(div_magic(reach - 1u, rb, f.rb_magic));
    fast = s_e == s0 || cell_of<kC>(s_e, w) == m0;
    if (fast && sh64 != 0 && s0 * rb == base) fast = cell_value<kC>(w.start, m0) != s0;
  }
  if (fast) {
    const uint32_t o = base + sh64 + delta + lane16;  // 64-byte aligned from lane 0
    const bool ok = o <= tb - 16u;
    stage_blocks(s_blk, x, xb, sh64, o, ok);
    const T y = staged16(s_blk, 16u * static_cast<uint32_t>(lane) + sh64);
    if (ok) store16_through(p.out_tokens + o, y);
    return;
  }
  // Otherwise each cell the owned bytes touch in turn (rows s0 .. s_last), for
  // the blocks of lanes v = lane and v = 64 + lane (lanes 0..3).
  const uint32_t own_end = min(base + 1024u, tb);
  const uint32_t s_last = __builtin_amdgcn_readfirstlane(div_magic(own_end - 1u, rb, f.rb_magic));
  const int m_last = s_last == s0 ? m0 : cell_of<kC>(s_last, w);
  uint32_t cnt[kC];
#pragma unroll
  for (int k = 0; k < kC; ++k) cnt[k] = static_cast<uint32_t>(w.c[k]);
  stage_blocks(s_blk, x, xb, s_last, own_end, true);
  for (int m = m0; m <= m_last; ++m) {  // uniform
    const uint32_t n = cell_value<kC>(cnt, m);
    if (n == 0) continue;
    const uint32_t st = cell_value<kC>(w.start, m);
    const uint32_t om = dest_row<kC>(st, m, w, rc.pos, outp);
    if (om + n > static_cast<uint32_t>(p.A)) continue;  // (valid counts keep every cell in range)
    const uint32_t cs = st * rb, ce = cs + n * rb;  // the cell's input bytes
    const uint32_t dl = (om - st) * rb;
    const uint32_t shm = (0u - dl) & 15u;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int v = lane + 64 * pass;
      if (v >= kByteBlocks) break;
      const uint32_t xl = base + shm + 16u * static_cast<uint32_t>(v);  // this block's first input byte
      // the first of the cell's input bytes in the block's segment (signed:
      // the segment may start before byte 0; every byte offset is below 2^31)
      const int32_t xf =
          max(static_cast<int32_t>(xl) - static_cast<int32_t>((xl + dl) & 63u), static_cast<int32_t>(cs));
      if (xl >= cs && xl < ce && xf >= static_cast<int32_t>(base) && xf < static_cast<int32_t>(own_end)) {
        const T y = staged16(s_blk, xl - base);
        if (xl + 16u <= ce)
          store16_through(p.out_tokens + (xl + dl), y);
        else
          store_bytes(p.out_tokens + (xl + dl), y, ce - xl);  // the tail block
      }
    }
    if (cs >= base && cs < own_end && ((cs + dl) & 15u) != 0) {  // uniform: the head block
      const uint32_t at = cs - base;
      if (static_cast<uint32_t>(lane) == at >> 4) {
        const T z = staged16(s_blk, at);  // input bytes [cs, cs + 16)
        store_bytes(p.out_tokens + (cs + dl), z, min(16u - ((cs + dl) & 15u), ce - cs));
      }
    }
  }
}

// The scale rows of output rows [d0, d0 + rows), output row d0 + r taken
// from input row s_src[r] (LDS); kScaleRound vectors per lane are loaded
// before they are stored.
template <int SV>
__device__ __forceinline__ void stream_fused_scales(const GatherArgs& p, const StreamFusedArgs& f, int d0, int rows,
                                                    const uint32_t* s_src) {
  using T = typename VecT<SV>::type;
  const int lane = threadIdx.x & 63;
  const int spr = p.scale_vecs_per_row;
  const int64_t Rs = p.scale_row_bytes;
  const int total = rows * spr;  // < 2^22 (Rs is at most 4 KiB here): div_small is exact
  for (int e0 = 0; e0 < total; e0 += 64 * kScaleRound) {
    T v[kScaleRound];
    int64_t to[kScaleRound];
    bool in[kScaleRound];
#pragma unroll
    for (int k = 0; k < kScaleRound; ++k) {
      const int e = e0 + 64 * k + lane;
      in[k] = e < total;
      const int r = in[k] ? div_small(e, f.inv_spr) : 0;
      const int cv = e - r * spr;
      v[k] = __builtin_nontemporal_load(
          reinterpret_cast<const T*>(p.scales + (in[k] ? int64_t(s_src[r]) * Rs + int64_t(cv) * SV : 0)));
      to[k] = int64_t(d0 + r) * Rs + int64_t(cv) * SV;
    }
#pragma unroll
    for (int k = 0; k < kScaleRound; ++k)
      if (in[k]) store_stream<SV>(reinterpret_cast<T*>(p.out_scales + to[k]), v[k]);
  }
}

// Four 4-byte words of four adjacent rows: one 16-byte store when all four are
// live and the address is 16-byte aligned, else a store per live word.
__device__ __forceinline__ void store_word_quad(uint32_t* dst, const uint32_t (&v)[4], const bool (&live)[4],
                                               bool aligned16) {
  using U4 = uint32_t __attribute__((ext_vector_type(4)));
  if (aligned16 && live[0] && live[1] && live[2] && live[3]) {
    U4 q;
    q.x = v[0];
    q.y = v[1];
    q.z = v[2];
    q.w = v[3];
    *reinterpret_cast<U4*>(dst) = q;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (live[r]) dst[r] = v[r];
  }
}

// LDS of a workgroup: the item waves' two tables of 64 kC cells (by output
// position: the count, later the output offset; the input offset) and 256
// row marks (later the rows' source rows); the token waves use its first M
// counts (inverse, kVec: at most 2 64 kC words).
template <int kC>
constexpr int stream_fused_lds_words() {
  return 2 * kC * 64 + kItemWaveRows;
}

// Item wave iw: output rows [64 rpl iw, 64 rpl (iw + 1)), rpl = f.rpl rows a
// lane (lane l: rows 64 rpl iw + rpl l + r, r < rpl). The offsets in output
// order come from one exchange of the counts through LDS; each row finds its
// cell by a mark at every cell start within the wave's rows and a running
// maximum (within the lane's rows, then over the lanes). Four rows a lane
// where the scale rows are small: a quarter of the item waves (at 16384 rows
// of 7 KiB, 256 item waves at the head of the grid cost ~1 us per call, 128
// ~0.1); one where they are larger, so that more waves carry the scale
// traffic.
template <bool kScatter, bool kWeight, typename CountT, int kC, bool kVec, bool kInv, bool kCalc>
__device__ __forceinline__ void stream_fused_items(const GatherArgs& p, const StreamFusedArgs& f, int iw,
                                                   uint32_t* s_lds) {
  // By output position: the count, overwritten by the output offset (each
  // lane reads its own cells' counts before it writes their offsets), and the
  // input offset; then the row marks, overwritten by the rows' source rows
  // (each lane reads its own rows' marks before it writes their sources).
  uint32_t* s_cnt = s_lds;
  uint32_t* s_out = s_lds;
  uint32_t* s_in = s_lds + kC * 64;
  int32_t* s_mark = reinterpret_cast<int32_t*>(s_lds + 2 * kC * 64);
  const int lane = threadIdx.x & 63;
  const int M = p.M, A = p.A;
  RawCells<CountT, kC> rc;
  load_cells<CountT, kC, kVec, kInv, kCalc>(static_cast<const CountT*>(f.counts), M, f, rc);
  mask_cells<CountT, kC, kVec, kInv>(rc, M);
  order_cells<CountT, kC, kVec, kInv>(rc, reinterpret_cast<CountT*>(s_lds), M);
  InCells<kC> w;
  finish_cells<CountT, kC, true>(rc, A, w);
  uint32_t outp[kC];
  cell_positions<kC>(rc.pos, outp);
  const int rpl = f.rpl;  // 1 or 4
  const int rows_w = 64 * rpl;
  const int d0 = iw * rows_w;
#pragma unroll
  for (int r = 0; r < 4; ++r) s_mark[4 * lane + r] = -1;
#pragma unroll
  for (int k = 0; k < kC; ++k)
    if (kC * lane + k < M) {
      s_cnt[outp[k]] = static_cast<uint32_t>(w.c[k]);
      s_in[outp[k]] = w.start[k];
    }
  __syncthreads();
  uint32_t co[kC], ostart[kC];
  uint32_t own = 0;
#pragma unroll
  for (int k = 0; k < kC; ++k) {
    co[k] = kC * lane + k < M ? s_cnt[kC * lane + k] : 0u;
    own += co[k];
  }
  ostart[0] = wave_scan_u32(own) - own;
#pragma unroll
  for (int k = 1; k < kC; ++k) ostart[k] = ostart[k - 1] + co[k - 1];
  // the cell holding row d0 (the last one starting at or before it) marks the
  // first row; every later cell starting within the wave's rows marks its start
  int u0 = -1;
#pragma unroll
  for (int k = 0; k < kC; ++k) {
    const int u = kC * lane + k;
    if (u < M) {
      s_out[u] = ostart[k];
      if (co[k] > 0 && ostart[k] > static_cast<uint32_t>(d0) && ostart[k] < static_cast<uint32_t>(d0 + rows_w))
        s_mark[ostart[k] - d0] = u;
    }
    u0 += __popcll(__ballot(u < M && ostart[k] <= static_cast<uint32_t>(d0)));
  }
  if (lane == 0) s_mark[0] = u0;
  __syncthreads();
  // running maximum: within the lane's rows, then the lanes before it
  int cell[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) cell[r] = r < rpl ? s_mark[rpl * lane + r] : -1;
#pragma unroll
  for (int r = 1; r < 4; ++r) cell[r] = max(cell[r], cell[r - 1]);
  const int before = __shfl_up(wave_max_scan(cell[3]), 1);  // the lanes before this one
  const bool valid = w.flags == 0;
  uint32_t src[4], dv[4];
  bool live[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int u = max(lane == 0 ? cell[r] : max(cell[r], before), 0);  // -1 only for rejected counts
    const int d = d0 + rpl * lane + r;
    live[r] = valid && r < rpl && d < A;
    dv[r] = static_cast<uint32_t>(d);
    src[r] = live[r] ? s_in[u] + (static_cast<uint32_t>(d) - s_out[u]) : 0u;
  }
  if (kScatter) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (live[r]) p.idx[src[r]] = static_cast<int32_t>(dv[r]);
  } else {
    store_word_quad(reinterpret_cast<uint32_t*>(p.idx) + d0 + rpl * lane, src, live, rpl == 4 && f.idx16 != 0);
  }
  if (kWeight) {
    uint32_t wv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[r] = p.weight[src[r]];  // src is 0 when not live
    store_word_quad(p.out_weight + d0 + rpl * lane, wv, live, rpl == 4 && f.w16 != 0);
  }
  if (valid && p.scale_row_bytes > 0) {  // uniform
    // the rows' source rows to LDS, for the scale vectors' lanes
    uint32_t* s_src = reinterpret_cast<uint32_t*>(s_mark);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (r < rpl) s_src[rpl * lane + r] = src[r];
    __builtin_amdgcn_wave_barrier();
    const int rows = min(rows_w, A - d0);
    switch (p.scale_vec) {
      case 16: stream_fused_scales<16>(p, f, d0, rows, s_src); break;
      case 8: stream_fused_scales<8>(p, f, d0, rows, s_src); break;
      case 4: stream_fused_scales<4>(p, f, d0, rows, s_src); break;
      case 2: stream_fused_scales<2>(p, f, d0, rows, s_src); break;
      default: stream_fused_scales<1>(p, f, d0, rows, s_src); break;
    }
  }
  if (iw == 0) {
    // expert j's rows start at the output offset of output position j * N
    // forward (expert-major output), at the input offset of output position j
    // inverse (expert-major input; output position j is cell (0, j))
    const int E = static_cast<int>(p.E), N = static_cast<int>(p.N);
    if (valid)
      for (int j = lane; j < E; j += 64) {
        const uint32_t a0 = kInv ? s_in[j] : s_out[j * N];
        const uint32_t a1 = j + 1 < E ? (kInv ? s_in[j + 1] : s_out[(j + 1) * N]) : static_cast<uint32_t>(A);
        static_cast<CountT*>(f.etn)[j] = static_cast<CountT>(f.cumsum ? a1 : a1 - a0);
      }
    // the exact sum for the header: the bits from 2^20 up and the low 20
    // bits summed apart (each sum exact in 32 bits)
    uint32_t hi = 0, lo = 0;
#pragma unroll
    for (int k = 0; k < kC; ++k) {
      hi += static_cast<uint32_t>(w.c[k]) >> 20;
      lo += static_cast<uint32_t>(w.c[k]) & 0xfffffu;
    }
    const int64_t total = (int64_t(wave_sum_u32(hi)) << 20) + wave_sum_u32(lo);
    if (lane == 0) write_header(p.hdr, p.A, p.N, p.E, total, w.flags, kCountsValid, p.inverse);
  }
}

// kBytes: token rows that are no multiple of 16 bytes (stream_fused_bytes).
template <bool kScatter, bool kWeight, typename CountT, int kC, bool kVec, bool kInv, bool kBytes, bool kCalc>
__global__ __launch_bounds__(64) void stream_fused_kernel(GatherArgs p, StreamFusedArgs f) {
  __shared__ uint32_t s_lds[stream_fused_lds_words<kC>()];
  const int b = static_cast<int>(blockIdx.x);
  // The scalars a token wave needs before its loads, fetched together with the
  // first kernel arguments (the compiler would fetch them one after the
  // other inside the branch, each a scalar-cache round trip).
  if constexpr (kBytes)
    asm volatile("" ::"s"(p.tokens), "s"(f.counts), "s"(f.tbytes), "s"(f.rbytes), "s"(f.rb_magic), "s"(p.M));
  else
    asm volatile("" ::"s"(p.tokens), "s"(f.counts), "s"(f.vpr), "s"(f.vpr_magic), "s"(f.vectors), "s"(p.M));
  if (b < f.item_waves) {  // uniform
    stream_fused_items<kScatter, kWeight, CountT, kC, kVec, kInv, kCalc>(p, f, b, s_lds);
    return;
  }
  if constexpr (kBytes)
    stream_fused_bytes<CountT, kC, kVec, kInv, kCalc>(p, f, static_cast<uint32_t>(b - f.item_waves), s_lds);
  else
    stream_fused_tokens<CountT, kC, kVec, kInv, kCalc>(p, f, static_cast<uint32_t>(b - f.item_waves), s_lds);
}

template <typename CountT, int kC, bool kVec, bool kInv, bool kBytes, bool kCalc>
void launch_stream_fused_c(const Plan& pl, const GatherArgs& g, const StreamFusedArgs& f, unsigned grid,
                           hipStream_t stream) {
  const dim3 block(64);
  if (pl.scatter) {
    if (pl.has_weight)
      hipLaunchKernelGGL((stream_fused_kernel<true, true, CountT, kC, kVec, kInv, kBytes, kCalc>), dim3(grid), block,
                         0, stream, g, f);
    else
      hipLaunchKernelGGL((stream_fused_kernel<true, false, CountT, kC, kVec, kInv, kBytes, kCalc>), dim3(grid), block,
                         0, stream, g, f);
  } else {
    if (pl.has_weight)
      hipLaunchKernelGGL((stream_fused_kernel<false, true, CountT, kC, kVec, kInv, kBytes, kCalc>), dim3(grid), block,
                         0, stream, g, f);
    else
      hipLaunchKernelGGL((stream_fused_kernel<false, false, CountT, kC, kVec, kInv, kBytes, kCalc>), dim3(grid),
                         block, 0, stream, g, f);
  }
}

template <typename CountT, int kC, bool kBytes, bool kCalc>
void launch_stream_fused_v(const Plan& pl, const GatherArgs& g, const StreamFusedArgs& f, unsigned grid, bool vec,
                           hipStream_t stream) {
  if (vec)
    pl.inverse ? launch_stream_fused_c<CountT, kC, true, true, kBytes, kCalc>(pl, g, f, grid, stream)
               : launch_stream_fused_c<CountT, kC, true, false, kBytes, kCalc>(pl, g, f, grid, stream);
  else
    pl.inverse ? launch_stream_fused_c<CountT, kC, false, true, kBytes, kCalc>(pl, g, f, grid, stream)
               : launch_stream_fused_c<CountT, kC, false, false, kBytes, kCalc>(pl, g, f, grid, stream);
}

// Four cells a lane up to 256 cells; eight up to 512, their output positions
// computed where the minor dimension is a multiple of 8, else from the table.
template <typename CountT, bool kBytes>
void launch_stream_fused_b(const Plan& pl, const GatherArgs& g, const StreamFusedArgs& f, unsigned grid, bool vec,
                           hipStream_t stream) {
  if (pl.sf_cells_per_lane != 8)
    launch_stream_fused_v<CountT, 4, kBytes, false>(pl, g, f, grid, vec, stream);
  else if (f.minor % 8 == 0)
    launch_stream_fused_v<CountT, 8, kBytes, true>(pl, g, f, grid, vec, stream);
  else
    launch_stream_fused_v<CountT, 8, kBytes, false>(pl, g, f, grid, vec, stream);
}

template <typename CountT>
void launch_stream_fused_t(const Plan& pl, const GatherArgs& g, const StreamFusedArgs& f, unsigned grid, bool vec,
                           hipStream_t stream) {
  if (pl.sf_bytes)
    launch_stream_fused_b<CountT, true>(pl, g, f, grid, vec, stream);
  else
    launch_stream_fused_b<CountT, false>(pl, g, f, grid, vec, stream);
}

}  // namespace

mrr_status launch_stream_fused(const Plan& pl, const mrr_args* a, void* ws, hipStream_t stream) {
  const GatherArgs g = gather_args(pl, a, ws);
  StreamFusedArgs f{};
  f.counts = a->expert_token_num_per_rank;
  f.etn = a->expert_token_num;
  f.cumsum = pl.cumsum ? 1 : 0;
  f.item_waves = static_cast<int32_t>(pl.sf_item_waves);
  f.rpl = pl.sf_rows_per_lane;
  f.idx16 = reinterpret_cast<uintptr_t>(g.idx) % 16 == 0 ? 1 : 0;
  f.w16 = reinterpret_cast<uintptr_t>(g.out_weight) % 16 == 0 ? 1 : 0;
  if (pl.sf_bytes) {
    f.rbytes = static_cast<uint32_t>(pl.row_bytes);  // in [17, 2^16), no multiple of 16
    f.rb_magic = static_cast<uint32_t>(((uint64_t(1) << 32) + f.rbytes - 1) / f.rbytes);
    f.tbytes = static_cast<uint32_t>(pl.A * pl.row_bytes);  // < 2^31 (the plan checks)
  } else {
    f.vpr = static_cast<uint32_t>(pl.row_bytes / 16);  // >= 2
    f.vpr_magic = static_cast<uint32_t>(((uint64_t(1) << 32) + f.vpr - 1) / f.vpr);
    f.inv_vpr = 1.0f / static_cast<float>(f.vpr);
    f.vectors = static_cast<uint32_t>(pl.A * f.vpr);   // < 2^32 (the plan checks)
  }
  f.minor = static_cast<int32_t>(pl.inverse ? pl.N : pl.E);
  f.major = static_cast<int32_t>(pl.inverse ? pl.E : pl.N);
  f.inv_minor = 1.0f / static_cast<float>(f.minor);
  f.inv_spr = g.scale_vecs_per_row > 0 ? 1.0f / static_cast<float>(g.scale_vecs_per_row) : 0.0f;
  // output positions: 8 bits a cell with 4 cells a lane, 16 with 8
  const int kc = pl.sf_cells_per_lane;
  const int bits = kc == 4 ? 8 : 16;
  const int words = kc * bits / 32;
  for (int l = 0; l < 64; ++l)
    for (int k = 0; k < kc; ++k) {
      const int m = kc * l + k;  // input-order cell (major m / minor, minor m % minor)
      if (m < pl.M)
        f.outpos[words * l + k * bits / 32] |= static_cast<uint32_t>((m % f.minor) * f.major + m / f.minor)
                                               << ((k * bits) % 32);
    }
  const unsigned grid = static_cast<unsigned>(pl.sf_grid);
  // each group of four counts in one or two 16-byte loads: aligned, whole groups of four cells
  const bool vec = reinterpret_cast<uintptr_t>(a->expert_token_num_per_rank) % 16 == 0 && pl.M % 4 == 0;
  if (pl.count_bytes == 8)
    launch_stream_fused_t<int64_t>(pl, g, f, grid, vec, stream);
  else
    launch_stream_fused_t<int32_t>(pl, g, f, grid, vec, stream);
  return hipGetLastError() == hipSuccess ? MRR_SUCCESS : MRR_ERROR_HIP;
}

}  // namespace mrr
