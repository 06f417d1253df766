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
      store_stream<V>(reinterpret_cast<T*>(dst + int64_t(d) * row_bytes + int64_t(q.c[k]) * V), q.v[k]);
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
      store_stream<(kSV > 0 ? kSV : 4)>(reinterpret_cast<ST*>(p.out_scales + int64_t(d) * Rs + sc_off), piece);
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

template <int V, int SV, bool S, bool W>
struct FusedK32 {
  static auto fn() { return &fused_kernel<V, SV, S, W, int32_t>; }
};
template <int V, int SV, bool S, bool W>
struct FusedK64 {
  static auto fn() { return &fused_kernel<V, SV, S, W, int64_t>; }
};

}  // namespace

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
