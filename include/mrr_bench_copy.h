/*
 * mrr_bench_copy.h -- a plain streaming device-to-device copy, used only to
 * measure the copy ceiling the re-routing gather is compared with (same byte
 * count, same 16-byte non-temporal loads and stores, no index work). Lives in
 * its own library, libmrr_bench_copy.so; not part of the operator.
 */
#ifndef MRR_BENCH_COPY_H
#define MRR_BENCH_COPY_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;

/*
 * Copies `bytes` bytes from device pointer `src` to device pointer `dst`
 * (non-overlapping, both 16-byte aligned, bytes a multiple of 16) on
 * `stream`, asynchronously. Returns 0 on success, 1 on bad arguments (nothing
 * launched), 2 if the launch failed.
 */
int mrr_bench_copy(void* dst, const void* src, size_t bytes, struct ihipStream_t* stream);

#ifdef __cplusplus
}
#endif
#endif /* MRR_BENCH_COPY_H */
