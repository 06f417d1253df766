// mrr_gather.hip -- the gather phase of the MoE re-routing operator
// (MoeReRoutingV2): page "CANN ops-transformer MoeReRoutingV2", section
// "计算公式" (the moves permute_X[DstOffset + k] = X[SrcOffset + k] for the
// tokens, per_token_scales and expert_topk_weight) and "参数说明"
// (permute_token_idx, gather or scatter form).
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
#include <algorithm>

#include "mrr_device.h"

namespace mrr {
namespace {

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
        store_stream<V>(reinterpret_cast<T*>(dst_chunk + int64_t(e) * V), v[k]);
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
    store_stream<(kSV > 0 ? kSV : 4)>(reinterpret_cast<ST*>(p.out_scales + int64_t(row0 + sc_row) * Rs + sc_off), piece);
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
  const int row0 = static_cast<int>((p.block_base + blockIdx.x) * p.rows_per_wg);  // < A
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
  uint32_t row_magic;    // ceil(2^32 / row bytes): quotients by the row length (byte_rows)
  uint32_t rows8;        // byte_rows with R >= 147 and A >= 8: a 1 KiB chunk spans at most
                         // floor(1023 / R) + 2 <= 8 rows
  uint32_t fold_scales;  // scale rows of one 4-byte word move in the item chunks
  uint32_t idx16;        // permute_token_idx is 16-byte aligned (a lane's four indices in one store)
  uint32_t w16;          // permute_topk_weight is 16-byte aligned (the same for its weights)
  uint32_t sc16;         // permute_per_token_scales is 16-byte aligned (the same for folded scales)
  uint32_t base;         // workgroups of earlier launches of the same call
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
  if (ok) store_stream<V>(reinterpret_cast<T*>(p.out_tokens + int64_t(d) * p.row_bytes + int64_t(col) * V), v);
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
  if (ok) store_stream<V>(reinterpret_cast<T*>(dst + (g0 + lane) * V), v);
}

// The 16 bytes at byte sh (0..15) of the 32-byte concatenation lo:hi, by
// byte funnel shifts (cheapest when sh is the same in every lane).
__device__ __forceinline__ VecT<16>::type funnel16(const VecT<16>::type& lo, const VecT<16>::type& hi, int sh) {
  const uint32_t wd[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  const int q = sh >> 2;
  const uint32_t r = static_cast<uint32_t>(sh & 3);
  uint32_t x[5];  // wd[q .. q + 4]
#pragma unroll
  for (int i = 0; i < 5; ++i) x[i] = q == 0 ? wd[i] : q == 1 ? wd[i + 1] : q == 2 ? wd[i + 2] : wd[i + 3];
  VecT<16>::type out;
  out.x = __builtin_amdgcn_alignbyte(x[1], x[0], r);
  out.y = __builtin_amdgcn_alignbyte(x[2], x[1], r);
  out.z = __builtin_amdgcn_alignbyte(x[3], x[2], r);
  out.w = __builtin_amdgcn_alignbyte(x[4], x[3], r);
  return out;
}

// funnel16 for a shift that is the same in every lane: a branch on q = sh / 4
// picks the four byte-aligned word pairs.
__device__ __forceinline__ VecT<16>::type funnel16_uniform(const VecT<16>::type& lo, const VecT<16>::type& hi,
                                                           int sh) {
  const uint32_t r = static_cast<uint32_t>(sh & 3);
  VecT<16>::type o;
  switch (sh >> 2) {
    case 0:
      o.x = __builtin_amdgcn_alignbyte(lo.y, lo.x, r);
      o.y = __builtin_amdgcn_alignbyte(lo.z, lo.y, r);
      o.z = __builtin_amdgcn_alignbyte(lo.w, lo.z, r);
      o.w = __builtin_amdgcn_alignbyte(hi.x, lo.w, r);
      break;
    case 1:
      o.x = __builtin_amdgcn_alignbyte(lo.z, lo.y, r);
      o.y = __builtin_amdgcn_alignbyte(lo.w, lo.z, r);
      o.z = __builtin_amdgcn_alignbyte(hi.x, lo.w, r);
      o.w = __builtin_amdgcn_alignbyte(hi.y, hi.x, r);
      break;
    case 2:
      o.x = __builtin_amdgcn_alignbyte(lo.w, lo.z, r);
      o.y = __builtin_amdgcn_alignbyte(hi.x, lo.w, r);
      o.z = __builtin_amdgcn_alignbyte(hi.y, hi.x, r);
      o.w = __builtin_amdgcn_alignbyte(hi.z, hi.y, r);
      break;
    default:
      o.x = __builtin_amdgcn_alignbyte(hi.x, lo.w, r);
      o.y = __builtin_amdgcn_alignbyte(hi.y, hi.x, r);
      o.z = __builtin_amdgcn_alignbyte(hi.z, hi.y, r);
      o.w = __builtin_amdgcn_alignbyte(hi.w, hi.z, r);
      break;
  }
  return o;
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
  return funnel16(lo, hi, static_cast<int>(w - a));
}

// One aligned 16-byte block of a run copy: output byte o takes input byte
// o + delta for the whole chunk (sh = delta & 15, the same in every lane).
// Loads the aligned input block holding byte o + delta, and the next one when
// sh != 0 (both then hold some of the 16 bytes), and funnel-shifts them. The
// two loads of neighbouring lanes overlap, so they are plain loads: the second
// one then finds the block in the cache (with non-temporal loads a shifted
// 41 MB copy measured 15.95 us against 14.40 us with plain loads and 13.88
// us for an aligned copy).
__device__ __forceinline__ VecT<16>::type run_block(const uint8_t* __restrict__ tokens, int64_t o, int64_t delta,
                                                    int sh) {
  using T = VecT<16>::type;
  const int64_t a = o + (delta - sh);
  if (sh == 0)  // uniform
    return __builtin_nontemporal_load(reinterpret_cast<const T*>(tokens + a));
  const T lo = *reinterpret_cast<const T*>(tokens + a);
  const T hi = *reinterpret_cast<const T*>(tokens + a + 16);
  return funnel16_uniform(lo, hi, sh);
}

// One aligned 16-byte block o of the dense output of byte rows, in general:
// its bytes come from output rows d1 (from byte col1, len1 bytes) and, when
// has2, the next one, i.e. from input rows s1 and s2, each with window16; a
// byte mask merges the two parts. The last, partial block of the output is
// stored byte by byte. Nothing is stored unless hv and both input rows lie in
// [0, A).
__device__ __forceinline__ void byte_block(const GatherArgs& p, int64_t o, int64_t total, int col1, int len1,
                                           bool has2, int32_t s1, int32_t s2, bool hv) {
  using T = VecT<16>::type;
  const int64_t R = p.row_bytes;
  const bool ok = hv & (static_cast<unsigned>(s1) < static_cast<unsigned>(p.A)) &
                  (static_cast<unsigned>(s2) < static_cast<unsigned>(p.A));
  s1 = ok ? s1 : 0;  // input row 0 when not moving: always valid here
  s2 = ok ? s2 : 0;
  const int64_t w1 = int64_t(s1) * R + col1;
  T v = window16(p.tokens, w1, w1, w1 + len1);
  if (has2) {  // the block crosses into the next row (a few lanes of a wave)
    const int64_t r2b = int64_t(s2) * R;  // output byte b >= len1 is input byte r2b + b - len1
    const T x2 = window16(p.tokens, r2b - len1, r2b, r2b + (16 - len1));
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
    store16_through(p.out_tokens + o, v);
  } else {
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
    for (int b = 0; b < static_cast<int>(total - o); ++b)
      p.out_tokens[o + b] = static_cast<uint8_t>(wv[b >> 2] >> (8 * (b & 3)));
  }
}

// Token rows that are no multiple of 16 bytes (at least 17 bytes, both
// buffers 16-byte aligned), as one byte stream: lane l of chunk c builds the
// aligned 16-byte block of the dense output at byte 1024 c + 16 l, from the
// chunk's output rows.
//  * Run copy: when those rows come from consecutive input rows (one segment,
//    or segments that continue each other) and the chunk is whole, its 1 KiB
//    is one byte range of the input at a fixed distance (the pages' moves copy
//    a segment's rows in order, so a segment is contiguous on both sides):
//    run_block.
//  * Otherwise byte_block.
// With rows of 147 bytes or more (rows8) a chunk spans at most 8 rows, whose
// row-map words the wave reads through the scalar cache beside the header, and
// the run check is scalar; with shorter rows (at most 1024 / 17 + 2 < 64 of
// them) lane k loads the k-th row's word and a ballot checks the run. The
// chunk's first row and its offset there come from 32-bit scalar quotients by
// R. (2 KiB chunks of 16 scalar words, amortizing this prologue, measured no
// faster at odd_rows.)
__device__ __forceinline__ void stream_bytes_chunk(const GatherArgs& p, const StreamGrid& g, uint32_t chunk) {
  using T = VecT<16>::type;
  const int lane = threadIdx.x & 63;
  const int64_t R = p.row_bytes;
  const uint32_t R32 = static_cast<uint32_t>(R);
  const int Ri = static_cast<int>(R32);
  const int64_t total = int64_t(p.A) * R;
  const int64_t o0 = int64_t(chunk) * 1024;
  // d_base = floor(1024 c / R) and off0 = 1024 c - d_base R: with c = qc R +
  // rc, 1024 c / R = 1024 qc + 1024 rc / R, and 1024 rc < 2^25.
  const uint32_t qc = div_magic(chunk, R32, g.row_magic);
  const uint32_t rc = chunk - qc * R32;
  const uint32_t r2 = div_magic(1024u * rc, R32, g.row_magic);
  const int d_base = static_cast<int>(1024u * qc + r2);  // < A
  const uint32_t off0 = 1024u * rc - r2 * R32;           // < R
  const bool whole = o0 + 1024 <= total;
  // rows the chunk touches: up to the one holding its last byte
  const uint32_t last = whole ? 1023u : static_cast<uint32_t>(total - 1 - o0);
  const int span = static_cast<int>(div_magic(off0 + last, R32, g.row_magic)) + 1;
  const int64_t o = o0 + 16 * lane;
  // this lane's block: from output row d_base + dd, byte col1, len1 bytes, the rest from the next row
  const int off = static_cast<int>(off0) + 16 * lane;  // < R + 1024
  int32_t s1, s2;
  bool hv;
  int dd;
  if (g.rows8) {  // uniform: the chunk's rows lie in 8 consecutive row-map words from
                  // min(d_base, A - 8) on, read through the scalar cache
    using CInt = const int32_t __attribute__((address_space(4)))*;
    const int base = min(d_base, p.A - 8);
    const CInt m = reinterpret_cast<CInt>(reinterpret_cast<uintptr_t>(p.rowmap + base));
    int32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = m[k];
    hv = header_valid(p.hdr, p);  // its loads go out after the row-map loads, both waited for once
    // a run: w[k] == w[0] + k for the chunk's rows k < span
    uint32_t diff = 0;
#pragma unroll
    for (int k = 1; k < 8; ++k) diff |= k < span ? static_cast<uint32_t>(w[k] - w[0] - k) : 0u;
    if (whole & (base == d_base) & (diff == 0)) {  // uniform: run copy
      const bool ok = hv & (w[0] >= 0) & (int64_t(w[0]) + span <= p.A);
      const int64_t delta = ok ? (int64_t(w[0]) - d_base) * R : -o0;  // not moving: input bytes [0, 1024)
      const T v = run_block(p.tokens, o, delta, static_cast<int>(delta & 15));
      if (ok) store16_through(p.out_tokens + o, v);
      return;
    }
    // row within the chunk: at most one boundary for rows of 1 KiB or more; below that,
    // a small exact division (off < 2048)
    dd = Ri >= 1024 ? (off >= Ri ? 1 : 0) : div_small(off, g.inv_row);
    const int k1 = d_base + dd - base;
    const int k2 = min(d_base + dd + 1, p.A - 1) - base;  // in [0, 8) for lanes inside the output
    s1 = w[0];
    s2 = w[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) {
      s1 = k1 == k ? w[k] : s1;
      s2 = k2 == k ? w[k] : s2;
    }
  } else {
    const int32_t word = p.rowmap[min(d_base + lane, p.A - 1)];
    hv = header_valid(p.hdr, p);  // its loads go out beside the row-map load
    const int32_t s0 = __builtin_amdgcn_readfirstlane(word);
    const bool brk = lane < span && word != s0 + lane;
    if (__builtin_amdgcn_ballot_w64(brk) == 0 && whole) {  // uniform: run copy
      const bool ok = hv & (s0 >= 0) & (int64_t(s0) + span <= p.A);
      const int64_t delta = ok ? (int64_t(s0) - d_base) * R : -o0;  // not moving: input bytes [0, 1024)
      const int sh = __builtin_amdgcn_readfirstlane(static_cast<int>(delta & 15));
      const T v = run_block(p.tokens, o, delta, sh);
      if (ok) store16_through(p.out_tokens + o, v);
      return;
    }
    dd = Ri >= 1024 ? (off >= Ri ? 1 : 0) : div_small(off, g.inv_row);
    // the rows' words from the lanes that loaded them (every lane takes part)
    s1 = __shfl(word, min(dd, 63), 64);
    s2 = __shfl(word, min(min(d_base + dd + 1, p.A - 1) - d_base, 63), 64);
  }
  const int col1 = off - dd * Ri;
  const int len1 = min(16, Ri - col1);
  const bool has2 = len1 < 16;
  if (o < total) byte_block(p, o, total, col1, len1, has2, s1, has2 ? s2 : s1, hv);
}

// Four words to dst[0..3]: one 16-byte store when `whole` (all four move and
// dst is 16-byte aligned), else the words of the rows that move.
__device__ __forceinline__ void store_words4(uint32_t* dst, const uint32_t (&v)[kItemRowsPerLane],
                                             const bool (&ok)[kItemRowsPerLane], bool whole) {
  using U4 = uint32_t __attribute__((ext_vector_type(4)));
  if (whole) {
    U4 x;
    x.x = v[0];
    x.y = v[1];
    x.z = v[2];
    x.w = v[3];
    *reinterpret_cast<U4*>(dst) = x;
  } else {
#pragma unroll
    for (int k = 0; k < kItemRowsPerLane; ++k)
      if (ok[k]) dst[k] = v[k];
  }
}

// Item chunk c: output rows [c * kItemRows, (c + 1) * kItemRows), four per
// lane (lane l: rows d0 = c * kItemRows + 4 l to d0 + 3): their index and
// weight and, with fold_scales, their one-word scale rows. The four row-map
// words come in one 16-byte load; the four rows' indices (gather form),
// weights and scale words are adjacent in the output and go out in one
// 16-byte store each when aligned.
template <bool kScatter, bool kWeight>
__device__ __forceinline__ void stream_items_chunk(const GatherArgs& p, const StreamGrid& g, uint32_t c) {
  using I4 = int32_t __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int d0 = static_cast<int>(c) * kItemRows + kItemRowsPerLane * lane;
  int32_t s[kItemRowsPerLane];
  if (d0 + kItemRowsPerLane <= p.A) {  // the row map sits 16-byte aligned in the workspace, d0 % 4 == 0
    const I4 w = *reinterpret_cast<const I4*>(p.rowmap + d0);
    s[0] = w.x;
    s[1] = w.y;
    s[2] = w.z;
    s[3] = w.w;
  } else {
#pragma unroll
    for (int k = 0; k < kItemRowsPerLane; ++k) s[k] = p.rowmap[min(d0 + k, p.A - 1)];
  }
  const bool hv = header_valid(p.hdr, p);
  bool ok[kItemRowsPerLane];
  bool all = true;
#pragma unroll
  for (int k = 0; k < kItemRowsPerLane; ++k) {
    ok[k] = hv & (d0 + k < p.A) & (static_cast<unsigned>(s[k]) < static_cast<unsigned>(p.A));
    all &= ok[k];
  }
  uint32_t wv[kItemRowsPerLane], sv[kItemRowsPerLane];
  if (kWeight) {
#pragma unroll
    for (int k = 0; k < kItemRowsPerLane; ++k) wv[k] = p.weight[ok[k] ? s[k] : 0];  // branch-free
  }
  const uint32_t* sc = reinterpret_cast<const uint32_t*>(p.scales);
  if (g.fold_scales) {  // uniform
#pragma unroll
    for (int k = 0; k < kItemRowsPerLane; ++k) sv[k] = sc[ok[k] ? s[k] : 0];
  }
  if (kScatter) {
#pragma unroll
    for (int k = 0; k < kItemRowsPerLane; ++k)
      if (ok[k]) p.idx[s[k]] = d0 + k;
  } else if (all && g.idx16) {
    I4 v;
    v.x = s[0];
    v.y = s[1];
    v.z = s[2];
    v.w = s[3];
    *reinterpret_cast<I4*>(p.idx + d0) = v;
  } else {
#pragma unroll
    for (int k = 0; k < kItemRowsPerLane; ++k)
      if (ok[k]) p.idx[d0 + k] = s[k];
  }
  if (kWeight) store_words4(p.out_weight + d0, wv, ok, all && g.w16);
  if (g.fold_scales) store_words4(reinterpret_cast<uint32_t*>(p.out_scales) + d0, sv, ok, all && g.sc16);
}

// One chunk per workgroup. Chunk numbers: token chunks [0, tok_chunks), scale
// chunks [tok_chunks, sc_end), then item chunks; the workgroups take the scale
// and item chunks first (with the token chunks' scalar row-map read, this
// order measured faster than token chunks first). Branches are uniform.
template <int V, bool kScatter, bool kWeight>
__global__ __launch_bounds__(64) void stream_gather_kernel(GatherArgs p, StreamGrid g) {
  const uint32_t bx = g.base + blockIdx.x;
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
    stream_items_chunk<kScatter, kWeight>(p, g, b - g.sc_end);
  }
}

template <int V, int SV, bool S, bool W>
struct GatherK {
  static auto fn() { return &gather_kernel<V, SV, S, W>; }
};

StreamGrid stream_grid(const Plan& pl) {
  StreamGrid sg;
  sg.base = 0;
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
  sg.row_magic = pl.byte_rows ? static_cast<uint32_t>(((uint64_t(1) << 32) + pl.row_bytes - 1) / pl.row_bytes) : 0u;
  sg.rows8 = pl.byte_rows && pl.row_bytes >= 147 && pl.A >= 8 ? 1u : 0u;
  sg.fold_scales = pl.fold_scales ? 1u : 0u;
  sg.idx16 = 0;
  sg.w16 = 0;
  sg.sc16 = 0;
  if (!pl.byte_rows && pl.vecs_per_row % 64 == 0) {
    sg.cpr = static_cast<uint32_t>(pl.vecs_per_row / 64);
    sg.cpr_magic = sg.cpr == 1 ? 0u : static_cast<uint32_t>(((uint64_t(1) << 32) + sg.cpr - 1) / sg.cpr);
  }
  return sg;
}

// Launches the stream gather's workgroups in pieces of at most
// max_launch_grid(64) (normally one piece).
template <bool S, bool W>
void launch_stream_sw(const Plan& pl, const GatherArgs& g, hipStream_t stream) {
  StreamGrid sg = stream_grid(pl);
  sg.idx16 = reinterpret_cast<uintptr_t>(g.idx) % 16 == 0 ? 1u : 0u;
  sg.w16 = reinterpret_cast<uintptr_t>(g.out_weight) % 16 == 0 ? 1u : 0u;
  sg.sc16 = reinterpret_cast<uintptr_t>(g.out_scales) % 16 == 0 ? 1u : 0u;
  const int64_t piece = max_launch_grid(64);
  for (int64_t base = 0; base < pl.stream_grid; base += piece) {
    sg.base = static_cast<uint32_t>(base);  // < kMaxStreamGrid
    const dim3 grid(static_cast<unsigned>(std::min(piece, pl.stream_grid - base))), block(64);
    switch (pl.token_vec) {
      case 16: hipLaunchKernelGGL((stream_gather_kernel<16, S, W>), grid, block, 0, stream, g, sg); break;
      case 8: hipLaunchKernelGGL((stream_gather_kernel<8, S, W>), grid, block, 0, stream, g, sg); break;
      case 4: hipLaunchKernelGGL((stream_gather_kernel<4, S, W>), grid, block, 0, stream, g, sg); break;
      case 2: hipLaunchKernelGGL((stream_gather_kernel<2, S, W>), grid, block, 0, stream, g, sg); break;
      default: hipLaunchKernelGGL((stream_gather_kernel<1, S, W>), grid, block, 0, stream, g, sg); break;
    }
  }
}

}  // namespace

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
  // in pieces of at most max_launch_grid(kGatherThreads) workgroups (normally one)
  const int64_t piece = max_launch_grid(kGatherThreads);
  for (int64_t base = 0; base < pl.grid; base += piece) {
    GatherArgs gp = g;
    gp.block_base = base;
    const unsigned n = static_cast<unsigned>(std::min(piece, pl.grid - base));
    dispatch<GatherK>(pl, [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(n), dim3(kGatherThreads), 0, stream, gp);
    });
  }
  return hipGetLastError() == hipSuccess ? MRR_SUCCESS : MRR_ERROR_HIP;
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

}  // namespace mrr
