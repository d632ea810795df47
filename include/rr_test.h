/*
 * rr_test.h -- test hooks of librr.  Not part of the product interface.
 */
#ifndef RR_TEST_H
#define RR_TEST_H

#include <stddef.h>
#include <stdint.h>

#include "rr.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Arrival-order skew for the split-K tier of rr_reduce_rows and for the
 * partitions of rr_splitk_attention.  With a value k > 0, the workgroup
 * folding slice g of a row sleeps about (G - 1 - g) * k short periods before
 * it publishes its partial (the attention: partition p of a query tile,
 * (P - 1 - p) * k before it takes the tile's ticket), so slices tend to
 * arrive in descending rank order.  The cross-workgroup fold of
 * "cluster_allreduce" (description) visits ranks in ascending order
 * regardless of arrival, so the output bits must not change.  0 (the
 * default) turns the skew off; negative values count as 0.  Process-wide;
 * affects launches made after the call.
 */
void rr_test_set_splitk_skew(int32_t sleeps_per_rank);

/*
 * Reference streams of known size, the achievable HBM bandwidth against which
 * the row kernels' rooflines are read (the published peak is not reachable):
 *   RR_TEST_STREAM_READ   reads `bytes` of x (y is not used and may be NULL);
 *   RR_TEST_STREAM_WRITE  writes `bytes` of y with a fixed pattern (x may be NULL);
 *   RR_TEST_STREAM_COPY   copies `bytes` from x to y (the ranges must not overlap).
 * Device pointers, 16-byte aligned; `bytes` a multiple of 16.  128-bit
 * non-temporal loads and stores, no arithmetic on the data; each workgroup
 * streams one contiguous run.  blocks_per_cu workgroups of 256 threads per
 * compute unit (1..16; 0 picks 2).  Asynchronous on `stream` (a hipStream_t,
 * NULL for the default stream); nothing is allocated.
 * Errors (nothing launched): RR_ERR_SHAPE for an unknown mode, misaligned
 * pointers or size, or blocks_per_cu out of range; RR_ERR_NULL for a missing
 * pointer the mode uses; RR_ERR_HIP if the launch fails.
 */
enum { RR_TEST_STREAM_READ = 0, RR_TEST_STREAM_WRITE = 1, RR_TEST_STREAM_COPY = 2 };
rr_status rr_test_stream(int32_t mode, const void* x, void* y, size_t bytes,
                         int32_t blocks_per_cu, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RR_TEST_H */
