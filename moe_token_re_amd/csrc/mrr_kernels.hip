// mrr_kernels.hip -- HIP kernels and launchers of the MoE re-routing operator
// (MoeReRoutingV2) for MI355X (gfx950, CDNA4: 64-lane waves, 256 CUs).
//
// Page: "CANN ops-transformer MoeReRoutingV2" (nlpx.cn article).
//   offsets_kernel  -- section "计算公式", the two double sums: SrcOffset is the
//                      exclusive prefix of the count matrix in row-major (rank,
//                      expert) order, DstOffset in column-major (expert, rank)
//                      order; plus expert_token_num ("参数说明") and the
//                      Sum(counts) == A constraint ("约束说明").
//   gather_kernel   -- section "计算公式", the moves
//                      permute_X[DstOffset + k] = X[SrcOffset + k] for tokens,
//                      per_token_scales and expert_topk_weight, and
//                      permute_token_idx ("参数说明"; gather or scatter form).
//
// Design (not the Ascend tiling of the article, which targets another chip):
//   * One workgroup of 1024 threads scans the counts twice (row-major, then
//     column-major) with wave shuffles and LDS, and writes per-cell tables
//     ordered by destination: dst_off[m], src_off[m] for m = j*N + i.
//   * The gather kernel works in destination order. Each workgroup owns a
//     contiguous run of output rows; every wave maps 64 of those rows to their
//     source rows with a cooperative 64-way search over dst_off (ballot over
//     64 pivots per round, then a 6-step shuffle search inside a 64-cell
//     window), and moves the 4-byte per-row items (index, weight) with one
//     lane per row. Then the whole workgroup streams the token bytes: the
//     (row, 16-byte vector) space of its rows is flattened, every thread keeps
//     8 vector loads in flight, and the stores are non-temporal and fully
//     contiguous, since the workgroup's output rows are adjacent.
//   * No atomics anywhere; every output element is written exactly once, so
//     results are deterministic.
#include <hip/hip_runtime.h>

#include <limits.h>
#include <stdint.h>

#include <mutex>

#include "mrr_internal.h"

namespace mrr {
namespace {

// ---------------------------------------------------------------------------
// Offsets
// ---------------------------------------------------------------------------

constexpr int kOffsetThreads = 1024;
constexpr int kOffsetItems = 4;  // counts per thread per tile
constexpr int64_t kOffsetTile = int64_t(kOffsetThreads) * kOffsetItems;
constexpr int kWaves = kOffsetThreads / 64;

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
// s holds 2*kWaves + 1 entries.
__device__ __forceinline__ int64_t block_exclusive_scan(int64_t v, int64_t* s, int64_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t inc = wave_inclusive_scan(v);
  if (lane == 63) s[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int64_t w = lane < kWaves ? s[lane] : 0;
    const int64_t wi = wave_inclusive_scan(w);
    if (lane < kWaves) s[kWaves + lane] = wi - w;
    if (lane == kWaves - 1) s[2 * kWaves] = wi;
  }
  __syncthreads();
  const int64_t res = s[kWaves + wave] + inc - v;
  *total = s[2 * kWaves];
  __syncthreads();  // s is reused by the next call
  return res;
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

// One workgroup. counts[N*E] row-major. Writes src_off/dst_off (cells in
// column-major order), expert_token_num and the workspace header. When
// `staged`, the clamped counts are kept in dynamic LDS between the passes.
template <typename CountT>
__global__ __launch_bounds__(kOffsetThreads) void offsets_kernel(
    const CountT* __restrict__ counts, int64_t N, int64_t E, int64_t A, int cumsum,
    CountT* __restrict__ etn, WsHeader* __restrict__ hdr, int32_t* __restrict__ dst_off,
    int32_t* __restrict__ src_off, int staged) {
  extern __shared__ int32_t s_counts[];
  __shared__ int64_t s_scan[2 * kWaves + 1];
  __shared__ uint32_t s_flags;
  const int tid = threadIdx.x;
  const int64_t M = N * E;
  if (tid == 0) s_flags = 0;
  uint32_t flags = 0;

  // Pass 1: SrcOffset = exclusive prefix in row-major (rank i, expert j) order.
  int64_t carry = 0;
  for (int64_t base = 0; base < M; base += kOffsetTile) {
    int32_t c[kOffsetItems];
    int64_t local = 0;
#pragma unroll
    for (int k = 0; k < kOffsetItems; ++k) {
      const int64_t m = base + int64_t(tid) * kOffsetItems + k;
      c[k] = m < M ? clamp_count(counts[m], &flags) : 0;
      if (staged && m < M) s_counts[m] = c[k];
      local += c[k];
    }
    int64_t tile_total;
    int64_t run = carry + block_exclusive_scan(local, s_scan, &tile_total);
#pragma unroll
    for (int k = 0; k < kOffsetItems; ++k) {
      const int64_t m = base + int64_t(tid) * kOffsetItems + k;
      if (m < M) {
        const int64_t i = m / E;
        const int64_t j = m - i * E;
        src_off[j * N + i] = static_cast<int32_t>(run);
      }
      run += c[k];
    }
    carry += tile_total;
  }

  if (flags != 0) atomicOr(&s_flags, flags);
  __syncthreads();
  flags = s_flags;
  if (carry != A) flags |= kFlagSumMismatch;
  if (flags != 0) {
    if (tid == 0) {
      hdr->A = A;
      hdr->N = N;
      hdr->E = E;
      hdr->total = carry;
      hdr->flags = flags;
      hdr->status = kTablesBad;
    }
    return;  // uniform: every thread sees the same flags
  }

  // Pass 2: DstOffset = exclusive prefix in column-major (expert j, rank i) order.
  carry = 0;
  for (int64_t base = 0; base < M; base += kOffsetTile) {
    int32_t c[kOffsetItems];
    int64_t local = 0;
#pragma unroll
    for (int k = 0; k < kOffsetItems; ++k) {
      const int64_t mc = base + int64_t(tid) * kOffsetItems + k;
      int32_t v = 0;
      if (mc < M) {
        const int64_t j = mc / N;
        const int64_t i = mc - j * N;
        v = staged ? s_counts[i * E + j] : clamp_count(counts[i * E + j], &flags);
      }
      c[k] = v;
      local += v;
    }
    int64_t tile_total;
    int64_t run = carry + block_exclusive_scan(local, s_scan, &tile_total);
#pragma unroll
    for (int k = 0; k < kOffsetItems; ++k) {
      const int64_t mc = base + int64_t(tid) * kOffsetItems + k;
      if (mc < M) dst_off[mc] = static_cast<int32_t>(run);
      run += c[k];
    }
    carry += tile_total;
  }
  if (tid == 0) dst_off[M] = static_cast<int32_t>(A);
  __threadfence_block();
  __syncthreads();

  // expert_token_num: column j covers cells [j*N, (j+1)*N) of the column-major
  // table, so its rows are dst_off[(j+1)*N] - dst_off[j*N]; the cumsum form is
  // the inclusive running total dst_off[(j+1)*N].
  for (int64_t j = tid; j < E; j += kOffsetThreads) {
    const int64_t end = dst_off[(j + 1) * N];
    const int64_t start = dst_off[j * N];
    etn[j] = static_cast<CountT>(cumsum ? end : end - start);
  }
  if (tid == 0) {
    hdr->A = A;
    hdr->N = N;
    hdr->E = E;
    hdr->total = carry;
    hdr->flags = 0;
    hdr->status = kTablesValid;
  }
}

// ---------------------------------------------------------------------------
// Gather
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
  const int32_t* dst_off;
  const int32_t* src_off;
  const WsHeader* hdr;
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
};

// The cell (in column-major order) holding output row d: the largest m with
// dst_off[m] <= d. All 64 lanes call it together; their rows d lie in
// [d_lo, d_lo + 63]. Returns m and dst_off[m].
__device__ __forceinline__ void locate(const int32_t* __restrict__ dst_off, int M, int d_lo, int d,
                                       int* m_out, int* dm_out) {
  const int lane = threadIdx.x & 63;
  // 64-way search for the cell of d_lo; invariant: dst_off[lo] <= d_lo and
  // that cell lies in [lo, hi).
  int lo = 0;
  int hi = M;
  while (hi - lo > 64) {
    const int stride = (hi - lo + 63) >> 6;
    const int pos = lo + lane * stride;
    const int v = pos < hi ? dst_off[pos] : INT_MAX;
    const uint64_t below = __ballot(v <= d_lo);  // a prefix of the lanes
    const int k = max(__popcll(below) - 1, 0);
    lo += k * stride;
    hi = min(hi, lo + stride);
  }
  // The 64-cell window [lo, lo + 64): a shuffle binary search per lane.
  const int piv = (lo + lane <= M) ? dst_off[lo + lane] : INT_MAX;
  int l = 0;
#pragma unroll
  for (int step = 32; step > 0; step >>= 1) {
    const int cand = l + step;
    const int pv = __shfl(piv, cand, 64);
    if (pv <= d) l = cand;
  }
  int m = lo + l;
  int dm = __shfl(piv, l, 64);
  if (l == 63 && lo + 63 < M) {
    // d lies past the window (many empty cells in between): finish alone.
    int a = lo + 63;
    int b = M;  // dst_off[a] <= d < dst_off[b] == A
    while (b - a > 1) {
      const int mid = (a + b) >> 1;
      if (dst_off[mid] <= d)
        a = mid;
      else
        b = mid;
    }
    m = a;
    dm = dst_off[a];
  }
  *m_out = min(m, M - 1);  // a no-op on tables the offsets kernel wrote
  *dm_out = dm;
}

// Copies `rows` rows of row_bytes = vpr * V bytes: source row s_src[r] to the
// r-th row of dst_chunk (rows adjacent). Rows with s_src[r] < 0 are skipped.
// The (row, vector) space is flattened and walked in steps of the workgroup
// size, kGatherUnroll loads in flight per thread before their stores.
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
    T v[kGatherUnroll];
    bool ok[kGatherUnroll];
#pragma unroll
    for (int k = 0; k < kGatherUnroll; ++k) {
      const int e = e0 + tid + k * kGatherThreads;
      ok[k] = false;
      if (e < total) {
        const int32_t srow = s_src[r];
        if (srow >= 0) {
          ok[k] = true;
          v[k] = __builtin_nontemporal_load(
              reinterpret_cast<const T*>(src + int64_t(srow) * row_bytes + int64_t(c) * V));
        }
      }
      r += dr;
      c += dc;
      if (c >= vpr) {
        c -= vpr;
        ++r;
      }
    }
#pragma unroll
    for (int k = 0; k < kGatherUnroll; ++k) {
      const int e = e0 + tid + k * kGatherThreads;
      if (ok[k]) __builtin_nontemporal_store(v[k], reinterpret_cast<T*>(dst_chunk + int64_t(e) * V));
    }
  }
}

template <int V, bool kScatter, bool kWeight>
__global__ __launch_bounds__(kGatherThreads) void gather_kernel(GatherArgs p) {
  __shared__ int32_t s_src[kMaxRowsPerWg];
  const WsHeader* h = p.hdr;
  if (h->status != kTablesValid || h->A != p.A || h->N != p.N || h->E != p.E) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int row0 = blockIdx.x * p.rows_per_wg;
  const int rows = min(p.rows_per_wg, p.A - row0);

  // Map this workgroup's output rows to source rows; move the per-row words.
  for (int b = wave * 64; b < rows; b += kGatherThreads) {
    const int lr = b + lane;
    const bool valid = lr < rows;
    const int d_lo = row0 + b;
    const int d = valid ? row0 + lr : d_lo;
    int m, dm;
    locate(p.dst_off, p.M, d_lo, d, &m, &dm);
    const int s = p.src_off[m] + (d - dm);
    const bool ok = valid && static_cast<unsigned>(s) < static_cast<unsigned>(p.A);
    if (valid) s_src[lr] = ok ? s : -1;
    if (ok) {
      if (kScatter)
        p.idx[s] = d;
      else
        p.idx[d] = s;
      if (kWeight) p.out_weight[d] = p.weight[s];
    }
  }
  __syncthreads();

  copy_rows<V>(p.tokens, p.out_tokens + int64_t(row0) * p.row_bytes, p.row_bytes, p.vecs_per_row, rows,
               s_src);

  if (p.scale_row_bytes > 0) {
    uint8_t* out = p.out_scales + int64_t(row0) * p.scale_row_bytes;
    switch (p.scale_vec) {
      case 16: copy_rows<16>(p.scales, out, p.scale_row_bytes, p.scale_vecs_per_row, rows, s_src); break;
      case 8: copy_rows<8>(p.scales, out, p.scale_row_bytes, p.scale_vecs_per_row, rows, s_src); break;
      case 4: copy_rows<4>(p.scales, out, p.scale_row_bytes, p.scale_vecs_per_row, rows, s_src); break;
      case 2: copy_rows<2>(p.scales, out, p.scale_row_bytes, p.scale_vecs_per_row, rows, s_src); break;
      default: copy_rows<1>(p.scales, out, p.scale_row_bytes, p.scale_vecs_per_row, rows, s_src); break;
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

// Per-device facts, read once per device.
struct DeviceInfo {
  int max_lds_per_block = 0;
};

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
DeviceInfo g_dev[kMaxDevices];

mrr_status device_info(const DeviceInfo** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MRR_ERROR_HIP;
  mrr_status st = MRR_SUCCESS;
  std::call_once(g_dev_once[dev], [&] {
    int lds = 0;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) lds = 0;
    g_dev[dev].max_lds_per_block = lds;
  });
  *out = &g_dev[dev];
  return st;
}

template <typename CountT>
mrr_status launch_offsets_t(const Plan& pl, const mrr_args* a, void* ws, hipStream_t stream) {
  const DeviceInfo* di = nullptr;
  if (device_info(&di) != MRR_SUCCESS) return MRR_ERROR_HIP;
  auto* base = static_cast<uint8_t*>(ws);
  // Keep the counts in LDS between the two passes when they fit in the
  // 64 KiB a launch may take without opting in to more (leaving room for the
  // kernel's static LDS).
  const int64_t stage_bytes = pl.M * 4;
  const int64_t lds_limit = di->max_lds_per_block < 65536 ? di->max_lds_per_block : 65536;
  const bool staged = pl.M > 0 && stage_bytes + 1024 <= lds_limit;
  hipLaunchKernelGGL((offsets_kernel<CountT>), dim3(1), dim3(kOffsetThreads),
                     staged ? static_cast<size_t>(stage_bytes) : 0, stream,
                     static_cast<const CountT*>(a->expert_token_num_per_rank), pl.N, pl.E, pl.A,
                     pl.cumsum ? 1 : 0, static_cast<CountT*>(a->expert_token_num),
                     reinterpret_cast<WsHeader*>(base), reinterpret_cast<int32_t*>(base + pl.dst_off_bytes),
                     reinterpret_cast<int32_t*>(base + pl.src_off_bytes), staged ? 1 : 0);
  return hipGetLastError() == hipSuccess ? MRR_SUCCESS : MRR_ERROR_HIP;
}

mrr_status launch_offsets(const Plan& pl, const mrr_args* a, void* ws, hipStream_t stream) {
  return pl.count_bytes == 8 ? launch_offsets_t<int64_t>(pl, a, ws, stream)
                             : launch_offsets_t<int32_t>(pl, a, ws, stream);
}

template <int V, bool kScatter, bool kWeight>
void launch_gather_vsw(const Plan& pl, const GatherArgs& g, hipStream_t stream) {
  hipLaunchKernelGGL((gather_kernel<V, kScatter, kWeight>), dim3(static_cast<unsigned>(pl.grid)),
                     dim3(kGatherThreads), 0, stream, g);
}

template <int V>
void launch_gather_v(const Plan& pl, const GatherArgs& g, hipStream_t stream) {
  if (pl.scatter) {
    if (pl.has_weight)
      launch_gather_vsw<V, true, true>(pl, g, stream);
    else
      launch_gather_vsw<V, true, false>(pl, g, stream);
  } else {
    if (pl.has_weight)
      launch_gather_vsw<V, false, true>(pl, g, stream);
    else
      launch_gather_vsw<V, false, false>(pl, g, stream);
  }
}

mrr_status launch_gather(const Plan& pl, const mrr_args* a, void* ws, hipStream_t stream) {
  if (pl.A == 0) return MRR_SUCCESS;
  auto* base = static_cast<uint8_t*>(ws);
  GatherArgs g{};
  g.tokens = static_cast<const uint8_t*>(a->tokens);
  g.out_tokens = static_cast<uint8_t*>(a->permute_tokens);
  g.scales = static_cast<const uint8_t*>(a->per_token_scales);
  g.out_scales = static_cast<uint8_t*>(a->permute_per_token_scales);
  g.weight = reinterpret_cast<const uint32_t*>(a->expert_topk_weight);
  g.out_weight = reinterpret_cast<uint32_t*>(a->permute_topk_weight);
  g.idx = a->permute_token_idx;
  g.dst_off = reinterpret_cast<const int32_t*>(base + pl.dst_off_bytes);
  g.src_off = reinterpret_cast<const int32_t*>(base + pl.src_off_bytes);
  g.hdr = reinterpret_cast<const WsHeader*>(base);
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
  switch (pl.token_vec) {
    case 16: launch_gather_v<16>(pl, g, stream); break;
    case 8: launch_gather_v<8>(pl, g, stream); break;
    case 4: launch_gather_v<4>(pl, g, stream); break;
    case 2: launch_gather_v<2>(pl, g, stream); break;
    default: launch_gather_v<1>(pl, g, stream); break;
  }
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
  st = mrr::launch_offsets(plan, args, workspace, stream);
  if (st != MRR_SUCCESS) return st;
  return mrr::launch_gather(plan, args, workspace, stream);
}

extern "C" mrr_status mrr_get_device_status(const void* workspace, struct ihipStream_t* stream) {
  if (workspace == nullptr) return MRR_ERROR_INVALID_VALUE;
  mrr::WsHeader h{};
  if (hipMemcpyAsync(&h, workspace, sizeof(h), hipMemcpyDeviceToHost, stream) != hipSuccess) return MRR_ERROR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return MRR_ERROR_HIP;
  if (h.status == mrr::kTablesValid) return MRR_SUCCESS;
  if (h.status == mrr::kTablesBad) return MRR_ERROR_BAD_COUNTS;
  return MRR_ERROR_INVALID_VALUE;
}
