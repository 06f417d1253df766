// host_fuzz.cpp -- randomised and extreme-value driver for the host-side
// argument checks and launch planning of the MoE re-routing library
// (mrr_validate, mrr_describe_plan, mrr_workspace_size, mrr_status_string).
// Built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitized.py; links mrr_validate.cpp only (no HIP code, no
// device). Every pointer is a fake address: nothing is dereferenced.
//
// Checks, for every generated argument set:
//   * mrr_validate and mrr_describe_plan agree on the status;
//   * an accepted call has a sane plan: workgroup sizes 64 or 256, grids in
//     [0, 2^31), the token row size H * bits / 8, a workspace size that fits;
//   * consistent argument sets built to be valid are accepted;
//   * no sanitizer report (signed overflow, out-of-bounds access, ...).
// Usage: host_fuzz <seed> <iterations>; exit status 0 when every check held.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <limits>

#include "moe_rerouting_v2.h"

namespace {

uint64_t g_state = 1;

uint64_t next() {  // xorshift64*
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return g_state * 0x2545F4914F6CDD1DULL;
}

int64_t pick_int() {
  static const int64_t kEdge[] = {0,       1,          2,          3,           7,
                                  63,      64,         65,         255,         256,
                                  257,     1023,       1024,       1025,        16383,
                                  16384,   65536,      131072,     131073,      (1LL << 24),
                                  INT32_MAX, (1LL << 31), (1LL << 32), (1LL << 62), std::numeric_limits<int64_t>::max(),
                                  -1,      -2,         INT32_MIN,  std::numeric_limits<int64_t>::min()};
  const uint64_t r = next();
  if (r % 3 == 0) return kEdge[(r >> 8) % (sizeof(kEdge) / sizeof(kEdge[0]))];
  if (r % 3 == 1) return static_cast<int64_t>((r >> 8) % 2000);
  return static_cast<int64_t>((r >> 8) % 5000000) - 1000;
}

// Fake device addresses: null, or one of several regions far apart, at a
// random small misalignment.
const void* pick_ptr(int slot) {
  const uint64_t r = next();
  if (r % 11 == 0) return nullptr;
  uint64_t base = (static_cast<uint64_t>(slot) + 1) << 40;
  if (r % 13 == 0) base = 1ULL << 40;  // sometimes the same region as another buffer
  const uint64_t mis = (r >> 8) % 7 == 0 ? (r >> 16) % 16 : 0;
  return reinterpret_cast<const void*>(base + mis);
}

int token_bits(int32_t dt) {
  switch (dt) {
    case MRR_F16: case MRR_BF16: return 16;
    case MRR_I8: case MRR_F8_E5M2: case MRR_F8_E4M3FN: case MRR_HIF8: return 8;
    case MRR_F4_E2M1: case MRR_F4_E1M2: return 4;
    default: return 0;
  }
}

int g_fail = 0;
long g_random_ok = 0;
long g_paths[3][2] = {{0, 0}, {0, 0}, {0, 0}};  // [fused: 0, 1, 2][stream gather] among accepted sets

void fail(const char* what, const mrr_args& a) {
  if (g_fail++ < 20)
    fprintf(stderr, "FAIL %s: A=%lld H=%lld N=%lld E=%lld tok=%d cnt=%d sc=%d/%d\n", what, (long long)a.A,
            (long long)a.H, (long long)a.N, (long long)a.E, a.tokens_dtype, a.counts_dtype, a.scales_dtype,
            a.scales_ndim);
}

void check(const mrr_args& a, const void* ws, size_t ws_bytes, bool must_pass) {
  const mrr_status v = mrr_validate(&a, ws, ws_bytes);
  mrr_plan_info info;
  const mrr_status d = mrr_describe_plan(&a, ws, ws_bytes, &info);
  (void)mrr_status_string(v);
  if (v != d) fail("validate and describe_plan disagree", a);
  if (must_pass && v != MRR_SUCCESS) fail("a consistent argument set was rejected", a);
  if (v != MRR_SUCCESS) return;
  if (!must_pass) ++g_random_ok;
  if (info.fused < 0 || info.fused > 2) fail("fused", a);
  if (must_pass) ++g_paths[info.fused][info.gather_kernel ? 1 : 0];
  const int bits = token_bits(a.tokens_dtype);
  if (info.threads_per_workgroup != 64 && info.threads_per_workgroup != 256) fail("threads per workgroup", a);
  if (info.gather_workgroups < 0 || info.gather_workgroups >= (1LL << 31)) fail("gather grid", a);
  if (info.offsets_workgroups < 0 || info.offsets_workgroups >= (1LL << 31)) fail("offsets grid", a);
  // every launch holds at most 2^32 - 1 threads: the gather in gather_launches pieces, the
  // fused kernel and the offsets kernels (workgroups of at most 1024 threads) in one
  const long long max_threads = (1LL << 32) - 1;
  const long long per_launch = info.gather_launches > 0
                                   ? (info.gather_workgroups + info.gather_launches - 1) / info.gather_launches
                                   : 0;
  if (a.A > 0 && info.gather_launches < 1) fail("no gather launch", a);
  if (per_launch * info.threads_per_workgroup > max_threads) fail("gather launch too large", a);
  if (info.fused == 1 && info.gather_launches != 1) fail("fused kernel in several launches", a);
  // moe_rerouting_v2's single launch: 256-thread workgroups (fused 1) or 64-lane ones (fused 2)
  if ((info.fused != 0) != (info.one_launch_workgroups > 0)) fail("one-launch workgroups", a);
  if (info.one_launch_workgroups * (info.fused == 1 ? 256 : 64) > max_threads) fail("one launch too large", a);
  if (info.offsets_workgroups * 1024 > max_threads) fail("offsets launch too large", a);
  if (info.token_row_bytes != a.H * bits / 8) fail("token row bytes", a);
  const size_t need = mrr_workspace_size(a.A, a.N, a.E);
  if (need == 0 || need > ws_bytes) fail("workspace size", a);
}

// A consistent argument set: sizes within every documented limit, distinct
// aligned buffers, a workspace large enough.
mrr_args consistent(size_t* ws_bytes) {
  mrr_args a{};
  const uint64_t r = next();
  a.tokens_dtype = static_cast<int32_t>(r % 8);
  a.counts_dtype = (r >> 4) % 2 ? MRR_I64 : MRR_I32;
  a.N = 1 + static_cast<int64_t>((r >> 8) % 700);
  a.E = 1 + static_cast<int64_t>((r >> 20) % 1200);
  if ((r >> 32) % 5 == 0) a.N = 1 + (a.N % 8);
  if (a.N * a.E > (1 << 20)) a.E = (1 << 20) / a.N;
  a.A = static_cast<int64_t>(next() % 3000000);
  if ((r >> 40) % 4 == 0) a.A = static_cast<int64_t>(next() % 300);
  a.H = 2 * (1 + static_cast<int64_t>(next() % 8191));
  const int cb = a.counts_dtype == MRR_I64 ? 8 : 4;
  auto addr = [](int slot) { return reinterpret_cast<void*>((static_cast<uint64_t>(slot) + 1) << 44); };
  a.tokens = addr(0);
  a.expert_token_num_per_rank = addr(1);
  a.permute_tokens = addr(2);
  a.permute_token_idx = static_cast<int32_t*>(addr(3));
  a.expert_token_num = addr(4);
  const uint64_t s = next();
  if (s % 3 == 1) {
    a.per_token_scales = addr(5);
    a.permute_per_token_scales = addr(6);
    a.scales_dtype = MRR_F32;
    a.scales_ndim = (s >> 4) % 2 ? 2 : 1;
    a.scales_dims[0] = a.A;
    a.scales_dims[1] = 1 + static_cast<int64_t>((s >> 8) % 64);
  } else if (s % 3 == 2) {
    a.per_token_scales = addr(5);
    a.permute_per_token_scales = addr(6);
    a.scales_dtype = MRR_F8_E8M0;
    a.scales_ndim = 3;
    a.scales_dims[0] = a.A;
    a.scales_dims[1] = (a.H + 63) / 64;
    a.scales_dims[2] = 2;
  }
  if ((s >> 16) % 2) {
    a.expert_topk_weight = static_cast<const float*>(addr(7));
    a.permute_topk_weight = static_cast<float*>(addr(8));
  }
  a.expert_token_num_type = (s >> 20) % 2;
  a.idx_type = (s >> 21) % 2;
  a.direction = (s >> 22) % 2;
  (void)cb;
  *ws_bytes = mrr_workspace_size(a.A, a.N, a.E);
  return a;
}

}  // namespace

int main(int argc, char** argv) {
  g_state = argc > 1 ? strtoull(argv[1], nullptr, 10) * 0x9E3779B97F4A7C15ULL + 1 : 1;
  const long iters = argc > 2 ? strtol(argv[2], nullptr, 10) : 100000;
  const void* ws_addr = reinterpret_cast<const void*>(15ULL << 44);
  long accepted = 0;
  for (long it = 0; it < iters; ++it) {
    // fully random arguments
    mrr_args a{};
    a.tokens_dtype = static_cast<int32_t>(next() % 14) - 1;
    a.counts_dtype = static_cast<int32_t>(next() % 14) - 1;
    a.A = pick_int();
    a.H = pick_int();
    a.N = pick_int();
    a.E = pick_int();
    a.tokens = pick_ptr(0);
    a.expert_token_num_per_rank = pick_ptr(1);
    a.per_token_scales = next() % 2 ? pick_ptr(2) : nullptr;
    a.scales_dtype = static_cast<int32_t>(next() % 14) - 1;
    a.scales_ndim = static_cast<int32_t>(next() % 5) - 1;
    for (int k = 0; k < 3; ++k) a.scales_dims[k] = next() % 2 ? pick_int() : a.A;
    a.expert_topk_weight = static_cast<const float*>(next() % 2 ? pick_ptr(3) : nullptr);
    a.permute_tokens = const_cast<void*>(pick_ptr(4));
    a.permute_per_token_scales = const_cast<void*>(pick_ptr(5));
    a.permute_token_idx = static_cast<int32_t*>(const_cast<void*>(pick_ptr(6)));
    a.expert_token_num = const_cast<void*>(pick_ptr(7));
    a.permute_topk_weight = static_cast<float*>(next() % 2 ? const_cast<void*>(pick_ptr(8)) : nullptr);
    a.expert_token_num_type = pick_int() % 3;
    a.idx_type = pick_int() % 3;
    a.direction = pick_int() % 3;
    const size_t ws_bytes = next() % 2 ? static_cast<size_t>(next()) : static_cast<size_t>(next() % (1 << 26));
    check(a, next() % 17 ? ws_addr : nullptr, ws_bytes, false);

    // a consistent set, which must be accepted
    size_t wb = 0;
    const mrr_args c = consistent(&wb);
    check(c, ws_addr, wb, true);
    ++accepted;
    (void)mrr_workspace_size(pick_int(), pick_int(), pick_int());
  }
  printf("host_fuzz: %ld iterations, %ld random sets accepted, %ld consistent sets (fused %ld, one-launch stream "
         "%ld, row workgroups %ld, stream %ld), %d failures\n",
         iters, g_random_ok, accepted, g_paths[1][0] + g_paths[1][1], g_paths[2][0] + g_paths[2][1], g_paths[0][0],
         g_paths[0][1], g_fail);
  return g_fail == 0 ? 0 : 1;
}
