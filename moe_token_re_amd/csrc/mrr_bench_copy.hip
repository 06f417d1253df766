// mrr_bench_copy.hip -- the copy-ceiling kernel of the benchmark: each
// workgroup copies one contiguous 32 KiB chunk (256 threads x 8 x 16 bytes),
// all 8 loads of a thread in flight before its stores, non-temporal both ways.
// The same access pattern as the re-routing gather's token copy, minus the
// row mapping.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "mrr_bench_copy.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr size_t kChunk = size_t(kThreads) * kUnroll * 16;

using v4u = uint32_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void copy_kernel(v4u* __restrict__ dst, const v4u* __restrict__ src,
                                                        size_t n_vec) {
  const size_t base = size_t(blockIdx.x) * (kThreads * kUnroll) + threadIdx.x;
  v4u v[kUnroll];
#pragma unroll
  for (int k = 0; k < kUnroll; ++k) {
    const size_t i = base + size_t(k) * kThreads;
    if (i < n_vec) v[k] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int k = 0; k < kUnroll; ++k) {
    const size_t i = base + size_t(k) * kThreads;
    if (i < n_vec) __builtin_nontemporal_store(v[k], dst + i);
  }
}

}  // namespace

extern "C" int mrr_bench_copy(void* dst, const void* src, size_t bytes, struct ihipStream_t* stream) {
  if (dst == nullptr || src == nullptr || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return 1;
  if (bytes == 0) return 0;
  const size_t blocks = (bytes + kChunk - 1) / kChunk;
  if (blocks > 0x7fffffffu) return 1;
  hipLaunchKernelGGL(copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                     static_cast<v4u*>(dst), static_cast<const v4u*>(src), bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
