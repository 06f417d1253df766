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

/*
 * Facts about device `device` that the benchmark report states beside its
 * figures, written to out[0..6]: compute units, LDS bytes per compute unit,
 * largest LDS bytes one workgroup may use, peak shader clock (kHz), memory
 * clock (kHz), memory bus width (bits), L2 cache bytes. Host-side queries
 * only. Returns 0, or 2 if a query failed (out is then partly written).
 */
int mrr_bench_device_facts(int device, long long out[7]);

#ifdef __cplusplus
}
#endif
#endif /* MRR_BENCH_COPY_H */
