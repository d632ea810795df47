// rr_plan.hpp -- host-side validation and planning (no HIP).
#pragma once

#include "../../include/rr.h"
#include "rr_config.hpp"

namespace rr {

// Shared by the ABI entry points and the planner queries.
rr_status plan_reduce(int64_t rows, int64_t cols, int64_t ld, rr_dtype dtype, rr_op op,
                      rr_tier tier, int32_t cu_count, bool vec, rr_plan* out);
// The block tier's persistent-row shape for a row reduction (nt == 0: one
// workgroup per row): element-aligned rows that fit row_pf_shape and at least
// kReducePfMinRowsPerCU rows per CU.
RowPfShape reduce_pf_shape(int64_t rows, int64_t cols, rr_op op, int32_t cu_count, bool vec);
// Lanes per row of that shape when a wavefront takes several rows (rows of
// up to 64 chunks: 16; up to 128: 32), else 0 (the workgroup's threads; also
// when a step's rows, ld elements apart, would span 2^31 bytes).
int reduce_pf_lanes(int64_t cols, int64_t ld);
// vec: x (and y) are aligned to their element size, so the block and split-K
// tiers take each row's body from its first 16-byte boundary in 128-bit
// chunks; rows16: every row of x and y starts 16-byte aligned (the wave tier
// and the layernorm's persistent rows need that for 128-bit chunks).
rr_status plan_softmax(int64_t rows, int64_t cols, rr_dtype x_dtype, rr_dtype y_dtype,
                       rr_tier tier, int32_t cu_count, bool vec, bool rows16, rr_plan* out);
rr_status plan_layernorm(int64_t rows, int64_t cols, rr_dtype x_dtype, rr_dtype y_dtype,
                         rr_dtype w_dtype, rr_tier tier, int32_t cu_count, bool vec,
                         bool rows16, rr_plan* out);
rr_status plan_axis(int64_t outer, int64_t axis, int64_t inner, rr_dtype dtype, rr_op op,
                    rr_tier tier, int32_t cu_count, bool vec, rr_plan* out);
uint64_t splitk_workspace_bytes(int64_t rows, int32_t slices, int partial_bytes);
uint64_t softmax_splitk_workspace_bytes(int64_t rows, int32_t slices);

}  // namespace rr
