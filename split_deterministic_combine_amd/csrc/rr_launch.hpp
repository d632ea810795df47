// rr_launch.hpp -- internal interface between the ABI entry points and the
// kernel launchers (one launcher per operation, in its own translation unit).
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/rr.h"

namespace rr {

struct ReduceLaunch {
    const void* x;
    void* y;              // single statistic
    int64_t rows, cols, ld;
    rr_dtype dtype;
    rr_op op;
    bool multi;           // sum, max and min over one read into ys (NULL: not written)
    void* ys[3];
    bool vec;             // element-aligned x: block, wave and split-K tiers load each
                          // row's body from its first 16-byte boundary in 128 bits
    bool rows16;          // every row starts 16-byte aligned: tiled and serial tiers
                          // load 128 bits per step
    void* workspace;      // split-K only
    int skew;             // test hook: split-K arrival skew (0 = off)
    hipStream_t stream;
    int32_t cu = 0;       // compute units the plan was made for (block tier: persistent rows)
};

struct SoftmaxLaunch {
    const void* x;
    void* y;
    int64_t rows, cols, ld_x, ld_y;
    rr_dtype x_dtype, y_dtype;
    bool vec;             // x and y element-aligned: block and split-K tiers take each
                          // row's body from its first 16-byte boundary in 128 bits
    bool rows16;          // every row of x and y 16-byte aligned (wave tier, and the
                          // persistent rows without a head or tail)
    void* workspace;      // split-K only
    int32_t cu;           // compute units of the current device
    hipStream_t stream;
};

struct AxisLaunch {
    const void* x;        // [outer][axis][inner]
    void* y;              // [outer][inner]
    int64_t outer, axis, inner;
    rr_dtype dtype;
    rr_op op;
    bool vec;             // 4 adjacent outputs per thread, 16-byte loads
    void* workspace;      // split-K only
    hipStream_t stream;
};

struct LayernormLaunch {
    const void* x;
    void* y;
    const void* gamma;    // [cols] of w_dtype, or NULL (1)
    const void* beta;     // [cols] of w_dtype, or NULL (0)
    float* mean_out;      // [rows] or NULL
    float* rstd_out;      // [rows] or NULL
    int64_t rows, cols, ld_x, ld_y;
    rr_dtype x_dtype, y_dtype, w_dtype;
    float eps;
    bool vec;             // x, y, gamma, beta element-aligned: block tier chunks from each
                          // row's first 16-byte boundary
    bool rows16;          // every row of x and y 16-byte aligned, gamma / beta too
                          // (persistent rows, wave tier)
    bool same_phase;      // every row of x at one offset from a 16-byte boundary
                          // (split-K tier with chunks)
    void* workspace;      // split-K only
    int32_t cu;           // compute units of the current device
    hipStream_t stream;
};

struct MergeLaunch {
    const float* o;
    const float* m;
    const float* l;
    void* out;
    int32_t P;
    int64_t rows;
    int32_t depth;
    float scale;
    rr_dtype out_dtype;
    bool vec;
    hipStream_t stream;
};

struct AttentionLaunch {
    const uint16_t* q;    // [batch*heads][q_rows][depth] bf16
    const uint16_t* k;    // [batch*kv_heads][kv_len][depth] bf16
    const uint16_t* v;
    float* o;             // [P][rows][depth]
    float* m;             // [P][rows]
    float* l;             // [P][rows]
    int64_t batch, heads, kv_heads, q_rows, kv_len;
    int32_t depth, P;
    float scale;
    void* out;            // fused: [rows][depth] of out_dtype; NULL: the partials are the output
    rr_dtype out_dtype;
    uint32_t* tickets;    // fused: one per (head, query tile), zero on entry and on exit
    int skew;             // fused, test hook: partition arrival skew (0 = off)
    hipStream_t stream;
    // packed variable-length sequences (NULL: the dense layout): q [total_q]
    // [heads][depth], k, v [kv_len][kv_heads][depth], token offsets of batch
    // sequences; q_rows is then the longest sequence's query count
    const int32_t* cu_q = nullptr;
    const int32_t* cu_k = nullptr;
    int64_t total_q = 0;
};

rr_status launch_reduce(const rr_plan& plan, const ReduceLaunch& a);
rr_status launch_reduce_identity(const ReduceLaunch& a);  // cols == 0
rr_status launch_softmax(const rr_plan& plan, const SoftmaxLaunch& a);
rr_status launch_merge(const MergeLaunch& a);
rr_status launch_attention(const AttentionLaunch& a);
rr_status launch_layernorm(const rr_plan& plan, const LayernormLaunch& a);
rr_status launch_reduce_axis(const rr_plan& plan, const AxisLaunch& a);
rr_status launch_fill_zero(void* p, size_t bytes, hipStream_t stream);
// Device address of this GPU's copy of the library's scratch array
// (RR_NOALLOC_SCRATCH_BYTES, rr_reduce.hip), looked up once per device.
rr_status noalloc_scratch(void** out);

}  // namespace rr
