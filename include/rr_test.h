/*
 * rr_test.h -- test hooks of librr.  Not part of the product interface.
 */
#ifndef RR_TEST_H
#define RR_TEST_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Arrival-order skew for the split-K tier of rr_reduce_rows.  With a value
 * k > 0, the workgroup folding slice g of a row sleeps about (G - 1 - g) * k
 * short periods before it publishes its partial, so slices tend to arrive in
 * descending rank order.  The cross-workgroup fold of "cluster_allreduce"
 * (description) visits ranks in ascending order regardless of arrival, so the
 * output bits must not change.  0 (the default) turns the skew off; negative
 * values count as 0.  Process-wide; affects launches made after the call.
 */
void rr_test_set_splitk_skew(int32_t sleeps_per_rank);

#ifdef __cplusplus
}
#endif

#endif /* RR_TEST_H */
