// mrr_bench_copy.hip -- the copy-ceiling kernel of the benchmark: a plain
// streaming copy in the fastest form measured on MI355X for this job: one
// 64-lane wave per workgroup, each lane moving one 16-byte vector (1 KiB per
// workgroup), non-temporal loads, stores written through the L2 as streaming
// data (sc1 nt, ~0.5% faster than nt alone, the same store the re-routing
// kernels use). Same byte count as the re-routing gather's token rows, no
// index work.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "mrr_bench_copy.h"

namespace {

constexpr int kThreads = 64;

using v4u = uint32_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void copy_kernel(v4u* __restrict__ dst, const v4u* __restrict__ src,
                                                        size_t n_vec) {
  const size_t i = size_t(blockIdx.x) * kThreads + threadIdx.x;
  // Branch-free load (a clamped index), predicated store.
  const v4u v = __builtin_nontemporal_load(src + (i < n_vec ? i : n_vec - 1));
  if (i < n_vec) asm volatile("global_store_dwordx4 %0, %1, off sc1 nt" ::"v"(dst + i), "v"(v) : "memory");
}

}  // namespace

extern "C" int mrr_bench_copy(void* dst, const void* src, size_t bytes, struct ihipStream_t* stream) {
  if (dst == nullptr || src == nullptr || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return 1;
  if (bytes == 0) return 0;
  const size_t n_vec = bytes / 16;
  const size_t blocks = (n_vec + kThreads - 1) / kThreads;
  if (blocks > 0x7fffffffu) return 1;
  hipLaunchKernelGGL(copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                     static_cast<v4u*>(dst), static_cast<const v4u*>(src), n_vec);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int mrr_bench_device_facts(int device, long long out[7]) {
  const hipDeviceAttribute_t attrs[7] = {
      hipDeviceAttributeMultiprocessorCount,        hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
      hipDeviceAttributeSharedMemPerBlockOptin,     hipDeviceAttributeClockRate,
      hipDeviceAttributeMemoryClockRate,            hipDeviceAttributeMemoryBusWidth,
      hipDeviceAttributeL2CacheSize};
  for (int k = 0; k < 7; ++k) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, attrs[k], device) != hipSuccess) return 2;
    out[k] = v;
  }
  return 0;
}
