// mrr_fused.hip -- the whole MoE re-routing call (MoeReRoutingV2, page
// "CANN ops-transformer MoeReRoutingV2": the offsets and moves of "计算公式",
// permute_token_idx and expert_token_num of "参数说明") in one launch, for
// small count matrices, in input order: every workgroup loads its own input
// rows first, then recomputes the offsets in its own LDS (a few KiB, read
// from L2) with the output row of each of its input rows, and stores the rows
// there; workgroup 0 also writes expert_token_num and the status. Up to 64
// cells, every wave computes the offsets in its registers (DPP scans, lane
// shuffles, a six-step search) with no barrier.
#include "mrr_device.h"

namespace mrr {
namespace {

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

  // The count first: its load is the oldest in flight, so the offsets below
  // wait for it alone while the row loads issued next are still under way.
  const CountT* counts = static_cast<const CountT*>(f.counts);
  const CountT craw = p.M <= 64 ? load_count64(counts, p.M) : load_count(counts, p.M);
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
    flags = wave_offsets64<CountT>(craw, N, E, p.A, &w, &total);
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
    flags = offsets_cells<kGatherThreads>(craw, N, E, p.A, p.inverse ? 0 : 1,
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
// The whole call in one launch of 64-lane workgroups, for count matrices of at
// most 256 cells and token rows of 16-byte vectors and at least 1 KiB.
// Workgroups [0, item_waves) move the per-row items and scale rows of 64
// output rows each; every later workgroup moves one 1 KiB chunk of the input
// token rows, in input order, so that its token load goes out at once (beside
// the count load); it then works out where its row (or two rows) go from the
// counts while the load is in flight. Every wave checks the counts itself and writes nothing when they
// are rejected; workgroup 0 writes expert_token_num and the status.
// ---------------------------------------------------------------------------

constexpr int kCellsPerLane = 4;  // 64 lanes x 4 = 256 cells
constexpr int kItemWaveRows = 4 * 64;  // the most output rows of an item wave (four per lane)
constexpr int kScaleRound = 4;    // scale vectors per lane loaded before they are stored

// The raw counts of this lane's cells m = 4 lane + k in input order (forward:
// row-major (rank, expert), the order of SrcOffset; inverse: column-major), 0
// past the matrix. Every wave reads the whole matrix, so the number of load
// instructions matters: with kVec (the counts 16-byte aligned, M a multiple of
// 4) a lane's four counts come in one 16-byte load (two for int64) in matrix
// order, and the inverse puts them in column-major order afterwards through
// LDS (order_cells); else in four loads. kVec is a template choice, not a
// branch: at a join of two load paths the compiler would wait for the counts
// before the token load goes out.
template <typename CountT>
struct RawCells {
  CountT r[kCellsPerLane];
  uint32_t pos;  // this lane's word of the host's output-position table (loaded with the counts)
};

template <typename CountT, bool kVec, bool kInv>
__device__ __forceinline__ void load_cells(const CountT* __restrict__ counts, int M, const StreamFusedArgs& f,
                                           RawCells<CountT>& rc) {
  const int lane = threadIdx.x & 63;
  rc.pos = f.outpos[lane];
  if (kVec) {
    const bool in = kCellsPerLane * lane < M;  // then all four cells are (M % 4 == 0)
    const CountT* q = counts + (in ? kCellsPerLane * lane : 0);
    CountT r[kCellsPerLane];
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
    for (int k = 0; k < kCellsPerLane; ++k) rc.r[k] = in ? r[k] : CountT(0);
    return;
  }
  // Addresses first (no branch between the loads: at its join the compiler
  // would wait for the earlier ones). Inverse, cell (rank b, expert a) of the
  // column-major order sits at b * E + a.
  int at[kCellsPerLane];
#pragma unroll
  for (int k = 0; k < kCellsPerLane; ++k) {
    const int m = kCellsPerLane * lane + k;
    int cm = m;
    if (kInv) {
      const int a = div_small(m, f.inv_minor);
      cm = (m - a * f.minor) * f.major + a;
    }
    at[k] = m < M ? cm : 0;  // M >= 1 here
  }
#pragma unroll
  for (int k = 0; k < kCellsPerLane; ++k) {
    const CountT raw = counts[at[k]];
    rc.r[k] = kCellsPerLane * lane + k < M ? raw : CountT(0);
  }
}

// With kVec and the inverse direction: the counts loaded in matrix order
// (row-major) rearranged into column-major order through s_c (M counts), one
// LDS write and four reads per lane. Called after the token load is issued.
// The LDS operations of one wave complete in order, so the reads see the
// writes.
template <typename CountT, bool kVec, bool kInv>
__device__ __forceinline__ void order_cells(RawCells<CountT>& rc, CountT* s_c, int M) {
  if (!kVec || !kInv) return;
  const int lane = threadIdx.x & 63;
  if (kCellsPerLane * lane < M) {
#pragma unroll
    for (int k = 0; k < kCellsPerLane; ++k) s_c[kCellsPerLane * lane + k] = rc.r[k];
  }
  __builtin_amdgcn_wave_barrier();
  // Inverse, the output order is the matrix order: the output position of
  // input-order cell m is its matrix index (rank * E + expert).
#pragma unroll
  for (int k = 0; k < kCellsPerLane; ++k) {
    const CountT v = s_c[(rc.pos >> (8 * k)) & 0xffu];  // 0 past the matrix
    rc.r[k] = kCellsPerLane * lane + k < M ? v : CountT(0);
  }
  __builtin_amdgcn_wave_barrier();
}

// The position of each of this lane's cells in output order, from the
// host's table (cell (major a, minor b) of the input order is cell
// b * major + a of the output order). Past the matrix the value means nothing
// (those cells count 0 and are never looked up or written).
__device__ __forceinline__ void cell_positions(uint32_t word, uint32_t (&out)[kCellsPerLane]) {
#pragma unroll
  for (int k = 0; k < kCellsPerLane; ++k) out[k] = (word >> (8 * k)) & 0xffu;
}

// The position of cell m in output order, in every lane (word: this lane's
// cell_positions word).
__device__ __forceinline__ uint32_t cell_position(uint32_t word, int m) {
  return (__builtin_amdgcn_readlane(word, m >> 2) >> (8 * (m & 3))) & 0xffu;
}

// What every wave derives from its cells: the counts, each cell's input
// offset (the exclusive prefix in input order: SrcOffset forward, DstOffset
// inverse), and the verdict on the whole matrix. Exactness: each count is
// below 2^31 (larger ones are flagged). While every count is below 2^22 the
// 256 of them sum below 2^30, so the wrapping 32-bit sum is exact. Otherwise
// (rare: a cell of 4M rows or more), with H the sum of the counts' bits from
// 2^20 up, the true sum lies below H 2^20 + 2^28; while H < 1024 it is below
// 2^32 and the wrapping sum is exact, and a valid matrix sums to A < 2^30
// (the plan sends only A < 2^30 here), so its H is below 1024.
struct InCells {
  int32_t c[kCellsPerLane];
  uint32_t start[kCellsPerLane];
  uint32_t total;  // uniform: the wrapping 32-bit sum
  uint32_t flags;  // uniform: kFlag* of the whole matrix (0: valid)
};

// kFlags: the flags say why the counts are rejected (item waves: workgroup 0
// writes them to the header); without it (token waves) any rejection shows
// as kFlagNegative, which is enough to write nothing and costs fewer
// instructions (a count is in [0, 2^31) when its bits from 31 up are 0).
template <typename CountT, bool kFlags>
__device__ __forceinline__ void finish_cells(const RawCells<CountT>& rc, int A, InCells& w) {
  uint32_t fl = 0;
  uint32_t own = 0;
#pragma unroll
  for (int k = 0; k < kCellsPerLane; ++k) {
    if (kFlags) {
      w.c[k] = clamp_count(rc.r[k], &fl);
    } else {
      const uint64_t u = static_cast<uint64_t>(static_cast<int64_t>(rc.r[k]));
      w.c[k] = static_cast<int32_t>(u & 0x7fffffffu);
      fl |= static_cast<uint32_t>(u >> 31);  // 0 for counts in [0, 2^31)
    }
    own += static_cast<uint32_t>(w.c[k]);
  }
  const uint32_t incl = wave_scan_u32(own);
  w.total = __builtin_amdgcn_readlane(incl, 63);
  w.start[0] = incl - own;
#pragma unroll
  for (int k = 1; k < kCellsPerLane; ++k) w.start[k] = w.start[k - 1] + static_cast<uint32_t>(w.c[k - 1]);
  uint32_t flags = kFlags ? (__ballot(fl & kFlagNegative) != 0 ? kFlagNegative : 0u) |
                               (__ballot(fl & kFlagTooLarge) != 0 ? kFlagTooLarge : 0u)
                         : (__ballot(fl != 0) != 0 ? kFlagNegative : 0u);
  const uint32_t any = static_cast<uint32_t>(w.c[0] | w.c[1] | w.c[2] | w.c[3]);  // counts are >= 0 here
  if (__ballot(any >= (1u << 22)) != 0) {  // uniform and rare
    uint32_t hi = 0;
#pragma unroll
    for (int k = 0; k < kCellsPerLane; ++k) hi += static_cast<uint32_t>(w.c[k]) >> 20;
    if (wave_sum_u32(hi) >= 1024u) flags |= kFlagSumMismatch;
  }
  if (w.total != static_cast<uint32_t>(A)) flags |= kFlagSumMismatch;
  w.flags = flags;
}

// v[k] of the lane holding cell m (k = m % 4), in every lane: every lane
// selects its own v[k] by the bits of k (named values, not an index into the
// array, which would put it in scratch memory), then that lane is read.
__device__ __forceinline__ uint32_t cell_value(const uint32_t (&v)[kCellsPerLane], int m) {
  const uint32_t v0 = v[0], v1 = v[1], v2 = v[2], v3 = v[3];
  const uint32_t lo = (m & 1) ? v1 : v0, hi = (m & 1) ? v3 : v2;
  return __builtin_amdgcn_readlane((m & 2) ? hi : lo, m >> 2);
}

// The cell holding input row s (the last one that starts at or before it),
// in every lane; 0 when the counts are rejected and no cell qualifies.
__device__ __forceinline__ int cell_of(uint32_t s, const InCells& w) {
  int m = -1;
#pragma unroll
  for (int k = 0; k < kCellsPerLane; ++k) m += __popcll(__ballot(w.start[k] <= s));
  return max(m, 0);
}

// The output row of input row s in cell m: the cell's output offset (the
// counts of the cells before it in output order) plus s's place in the cell.
__device__ __forceinline__ uint32_t dest_row(uint32_t s, int m, const InCells& w, uint32_t pos,
                                             const uint32_t (&outp)[kCellsPerLane]) {
  const uint32_t out_m = cell_position(pos, m);
  uint32_t before = 0;
#pragma unroll
  for (int k = 0; k < kCellsPerLane; ++k) before += outp[k] < out_m ? static_cast<uint32_t>(w.c[k]) : 0u;
  return wave_sum_u32(before) + (s - cell_value(w.start, m));
}

// Token wave c: the 16-byte vectors [64 c, 64 c + 64) of the input token rows
// taken as one stream (input order, vpr >= 64 vectors a row), one load and
// store per lane: this chip streams fastest with one-wave workgroups of one
// load each (two chunks a wave measured slower). The load needs no offsets.
// The chunk lies in row s0, or reaches into row s0 + 1 when the rows are no
// whole number of KiB; then the wave also works out where row s0 + 1 goes
// (the next output row when it is in the same cell).
template <typename CountT, bool kVec, bool kInv>
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
  RawCells<CountT> rc;
  load_cells<CountT, kVec, kInv>(static_cast<const CountT*>(f.counts), p.M, f, rc);
  const T x = __builtin_nontemporal_load(reinterpret_cast<const T*>(p.tokens + (in ? int64_t(v) * 16 : 0)));
  // The offsets below wait for the counts alone (loads return in issue
  // order). The compiler would otherwise sink the token load below them, next
  // to its store: this barrier names the token buffer, so the load stays here.
  asm volatile("" ::"s"(p.tokens) : "memory");
  order_cells<CountT, kVec, kInv>(rc, reinterpret_cast<CountT*>(s_lds), p.M);
  InCells w;
  finish_cells<CountT, false>(rc, p.A, w);
  uint32_t outp[kCellsPerLane];
  cell_positions(rc.pos, outp);
  const int m0 = cell_of(s0, w);
  const uint32_t d0 = dest_row(s0, m0, w, rc.pos, outp);
  const uint32_t b = (s0 + 1) * f.vpr;  // the first vector of row s0 + 1 (<= A * vpr)
  uint32_t d1 = d0 + 1;
  if (b < n0 + 64u && s0 + 1 < static_cast<uint32_t>(p.A)) {  // uniform: the chunk reaches row s0 + 1
    const int m1 = cell_of(s0 + 1, w);
    if (m1 != m0) d1 = dest_row(s0 + 1, m1, w, rc.pos, outp);  // uniform
  }
  const bool second = v >= b;
  const uint32_t d = second ? d1 : d0;
  const uint32_t col = v - (second ? s0 + 1 : s0) * f.vpr;  // the vector within its row
  if (w.flags == 0 && in && d < static_cast<uint32_t>(p.A))
    __builtin_nontemporal_store(x, reinterpret_cast<T*>(p.out_tokens + int64_t(d) * p.row_bytes + int64_t(col) * 16));
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
      if (in[k]) __builtin_nontemporal_store(v[k], reinterpret_cast<T*>(p.out_scales + to[k]));
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

// Item wave iw: output rows [64 rpl iw, 64 rpl (iw + 1)), rpl = f.rpl rows a
// lane (lane l: rows 64 rpl iw + rpl l + r, r < rpl). The offsets in output
// order come from one exchange of the counts through LDS; each row finds its
// cell by a mark at every cell start within the wave's rows and a running
// maximum (within the lane's rows, then over the lanes). Four rows a lane
// where the scale rows are small: a quarter of the item waves (at pages_shape,
// 256 item waves at the head of the grid cost ~1 us per call, 128 ~0.1); one
// where they are larger, so that more waves carry the scale traffic.
template <bool kScatter, bool kWeight, typename CountT, bool kVec, bool kInv>
__device__ __forceinline__ void stream_fused_items(const GatherArgs& p, const StreamFusedArgs& f, int iw,
                                                   uint32_t* s_lds) {
  uint32_t* s_cnt = s_lds;                                 // by output position: the count (later the
                                                           // rows' source rows),
  uint32_t* s_in = s_lds + kCellsPerLane * 64;             // the input offset,
  uint32_t* s_out = s_lds + 2 * kCellsPerLane * 64;        // the output offset;
  int32_t* s_mark = reinterpret_cast<int32_t*>(s_lds + 3 * kCellsPerLane * 64);  // row marks [256]
  const int lane = threadIdx.x & 63;
  const int M = p.M, A = p.A;
  RawCells<CountT> rc;
  load_cells<CountT, kVec, kInv>(static_cast<const CountT*>(f.counts), M, f, rc);
  order_cells<CountT, kVec, kInv>(rc, reinterpret_cast<CountT*>(s_lds), M);
  InCells w;
  finish_cells<CountT, true>(rc, A, w);
  uint32_t outp[kCellsPerLane];
  cell_positions(rc.pos, outp);
  const int rpl = f.rpl;  // 1 or 4
  const int rows_w = 64 * rpl;
  const int d0 = iw * rows_w;
#pragma unroll
  for (int r = 0; r < 4; ++r) s_mark[4 * lane + r] = -1;
#pragma unroll
  for (int k = 0; k < kCellsPerLane; ++k)
    if (kCellsPerLane * lane + k < M) {
      s_cnt[outp[k]] = static_cast<uint32_t>(w.c[k]);
      s_in[outp[k]] = w.start[k];
    }
  __syncthreads();
  uint32_t co[kCellsPerLane], ostart[kCellsPerLane];
  uint32_t own = 0;
#pragma unroll
  for (int k = 0; k < kCellsPerLane; ++k) {
    co[k] = kCellsPerLane * lane + k < M ? s_cnt[kCellsPerLane * lane + k] : 0u;
    own += co[k];
  }
  ostart[0] = wave_scan_u32(own) - own;
#pragma unroll
  for (int k = 1; k < kCellsPerLane; ++k) ostart[k] = ostart[k - 1] + co[k - 1];
  // the cell holding row d0 (the last one starting at or before it) marks the
  // first row; every later cell starting within the 256 rows marks its start
  int u0 = -1;
#pragma unroll
  for (int k = 0; k < kCellsPerLane; ++k) {
    const int u = kCellsPerLane * lane + k;
    if (u < M) {
      s_out[u] = ostart[k];
      if (co[k] > 0 && ostart[k] > static_cast<uint32_t>(d0) && ostart[k] < static_cast<uint32_t>(d0 + rows_w))
        s_mark[ostart[k] - d0] = u;
    }
    u0 += __popcll(__ballot(u < M && ostart[k] <= static_cast<uint32_t>(d0)));
  }
  if (lane == 0) s_mark[0] = u0;
  __syncthreads();
  // running maximum: within the lane's four rows, then the lanes before it
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
    // the rows' source rows to LDS (over the counts, no longer read), for the
    // scale vectors' lanes
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (r < rpl) s_cnt[rpl * lane + r] = src[r];
    __builtin_amdgcn_wave_barrier();
    const int rows = min(rows_w, A - d0);
    switch (p.scale_vec) {
      case 16: stream_fused_scales<16>(p, f, d0, rows, s_cnt); break;
      case 8: stream_fused_scales<8>(p, f, d0, rows, s_cnt); break;
      case 4: stream_fused_scales<4>(p, f, d0, rows, s_cnt); break;
      case 2: stream_fused_scales<2>(p, f, d0, rows, s_cnt); break;
      default: stream_fused_scales<1>(p, f, d0, rows, s_cnt); break;
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
    for (int k = 0; k < kCellsPerLane; ++k) {
      hi += static_cast<uint32_t>(w.c[k]) >> 20;
      lo += static_cast<uint32_t>(w.c[k]) & 0xfffffu;
    }
    const int64_t total = (int64_t(wave_sum_u32(hi)) << 20) + wave_sum_u32(lo);
    if (lane == 0) write_header(p.hdr, p.A, p.N, p.E, total, w.flags, kCountsValid, p.inverse);
  }
}

// LDS of a workgroup: the item waves' three tables of 256 cells and 256 row
// marks; the token waves use its first 256 counts (inverse, kVec).
constexpr int kStreamFusedLdsWords = 3 * kCellsPerLane * 64 + kItemWaveRows;

template <bool kScatter, bool kWeight, typename CountT, bool kVec, bool kInv>
__global__ __launch_bounds__(64) void stream_fused_kernel(GatherArgs p, StreamFusedArgs f) {
  __shared__ uint32_t s_lds[kStreamFusedLdsWords];
  const int b = static_cast<int>(blockIdx.x);
  // The scalars a token wave needs before its loads, fetched together with the
  // first kernel arguments (the compiler would fetch them one after the
  // other inside the branch, each a scalar-cache round trip).
  asm volatile("" ::"s"(p.tokens), "s"(f.counts), "s"(f.vpr), "s"(f.vpr_magic), "s"(f.vectors), "s"(p.M));
  if (b < f.item_waves) {  // uniform
    stream_fused_items<kScatter, kWeight, CountT, kVec, kInv>(p, f, b, s_lds);
    return;
  }
  stream_fused_tokens<CountT, kVec, kInv>(p, f, static_cast<uint32_t>(b - f.item_waves), s_lds);
}

template <int V, int SV, bool S, bool W>
struct FusedK32 {
  static auto fn() { return &fused_kernel<V, SV, S, W, int32_t>; }
};
template <int V, int SV, bool S, bool W>
struct FusedK64 {
  static auto fn() { return &fused_kernel<V, SV, S, W, int64_t>; }
};

template <typename CountT, bool kVec, bool kInv>
void launch_stream_fused_c(const Plan& pl, const GatherArgs& g, const StreamFusedArgs& f, unsigned grid,
                           hipStream_t stream) {
  const dim3 block(64);
  if (pl.scatter) {
    if (pl.has_weight)
      hipLaunchKernelGGL((stream_fused_kernel<true, true, CountT, kVec, kInv>), dim3(grid), block, 0, stream, g, f);
    else
      hipLaunchKernelGGL((stream_fused_kernel<true, false, CountT, kVec, kInv>), dim3(grid), block, 0, stream, g, f);
  } else {
    if (pl.has_weight)
      hipLaunchKernelGGL((stream_fused_kernel<false, true, CountT, kVec, kInv>), dim3(grid), block, 0, stream, g, f);
    else
      hipLaunchKernelGGL((stream_fused_kernel<false, false, CountT, kVec, kInv>), dim3(grid), block, 0, stream, g, f);
  }
}

template <typename CountT>
void launch_stream_fused_v(const Plan& pl, const GatherArgs& g, const StreamFusedArgs& f, unsigned grid, bool vec,
                           hipStream_t stream) {
  if (vec)
    pl.inverse ? launch_stream_fused_c<CountT, true, true>(pl, g, f, grid, stream)
               : launch_stream_fused_c<CountT, true, false>(pl, g, f, grid, stream);
  else
    pl.inverse ? launch_stream_fused_c<CountT, false, true>(pl, g, f, grid, stream)
               : launch_stream_fused_c<CountT, false, false>(pl, g, f, grid, stream);
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
  f.vpr = static_cast<uint32_t>(pl.row_bytes / 16);  // >= 64
  f.vpr_magic = static_cast<uint32_t>(((uint64_t(1) << 32) + f.vpr - 1) / f.vpr);
  f.vectors = static_cast<uint32_t>(pl.A * f.vpr);   // < 2^32 (the plan checks)
  f.minor = static_cast<int32_t>(pl.inverse ? pl.N : pl.E);
  f.major = static_cast<int32_t>(pl.inverse ? pl.E : pl.N);
  f.inv_minor = 1.0f / static_cast<float>(f.minor);
  f.inv_spr = g.scale_vecs_per_row > 0 ? 1.0f / static_cast<float>(g.scale_vecs_per_row) : 0.0f;
  for (int l = 0; l < 64; ++l) {
    uint32_t word = 0;
    for (int k = 0; k < kCellsPerLane; ++k) {
      const int m = kCellsPerLane * l + k;  // input-order cell (major m / minor, minor m % minor)
      if (m < pl.M) word |= static_cast<uint32_t>((m % f.minor) * f.major + m / f.minor) << (8 * k);
    }
    f.outpos[l] = word;
  }
  const unsigned grid = static_cast<unsigned>(pl.sf_grid);
  // a lane's four counts in one or two 16-byte loads: aligned, whole groups of four cells
  const bool vec = reinterpret_cast<uintptr_t>(a->expert_token_num_per_rank) % 16 == 0 && pl.M % kCellsPerLane == 0;
  if (pl.count_bytes == 8)
    launch_stream_fused_v<int64_t>(pl, g, f, grid, vec, stream);
  else
    launch_stream_fused_v<int32_t>(pl, g, f, grid, vec, stream);
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

}  // namespace mrr
