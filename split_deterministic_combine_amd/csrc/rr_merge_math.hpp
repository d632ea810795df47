// rr_merge_math.hpp -- the per-row arithmetic of the split-K LSE merge, shared
// by the merge kernels and the fused split-K attention, so that both give the
// same bits for the same partials.
//
// "fa4_splitk_reduce_scatter_write", per-band steps: each partition's output
// is weighted by exp(m_p - M) * l_p and the partitions are accumulated.
// Partition p of a row is empty when l_p <= 0 or m_p == -inf; M is the
// largest m_p of the non-empty ones; w_p = exp(scale * (m_p - M)) * l_p (0 for
// an empty p); W = sum of w_p in ascending p; the coefficient is c_p = w_p / W,
// or -1 for an empty p, which the accumulation skips (an empty partition's
// O_p, possibly NaN, never enters the sum).  Double precision throughout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rr_device.hpp"

namespace rr {

__device__ __forceinline__ bool merge_live(float2 st)
{
    return st.y > 0.0f && st.x > -__builtin_inff();
}

// M over a row's P statistics (m_p, l_p), `stride` cells apart; 0 when no
// partition is live (then no weight uses it).
__device__ __forceinline__ double merge_row_max(const float2* rs, int32_t P, int32_t stride = 1)
{
    bool any = false;
    double M = 0.0;
    for (int32_t p = 0; p < P; ++p) {
        const float2 s = rs[(int64_t)p * stride];
        if (merge_live(s)) {
            if (!any || (double)s.x > M)
                M = (double)s.x;
            any = true;
        }
    }
    return M;
}

__device__ __forceinline__ double merge_weight(float2 st, double M, float scale)
{
    return merge_live(st) ? exp((double)scale * ((double)st.x - M)) * (double)st.y : 0.0;
}

// W: the row's P weights (`stride` cells apart) added in ascending partition
// order.
__device__ __forceinline__ double merge_total(const double* wrow, int32_t P, int32_t stride = 1)
{
    double W = 0.0;
    for (int32_t p = 0; p < P; ++p)
        W += wrow[(int64_t)p * stride];
    return W;
}

__device__ __forceinline__ double merge_coef(float2 st, double w, double W)
{
    return merge_live(st) ? w / W : -1.0;
}

// acc += c_p * O_p over n values, skipped for an empty partition.
template <int N>
__device__ __forceinline__ void merge_accumulate(double* acc, double cp, const float* v)
{
    if (cp >= 0.0) {
#pragma unroll
        for (int e = 0; e < N; ++e)
            acc[e] = fma(cp, (double)v[e], acc[e]);
    }
}

// Four accumulated values of an output row, rounded once to YT (bf16 bits
// or float) and stored together.  bf16: the double goes to float rounded to
// odd, then to bf16 rounded to nearest even -- one correct rounding of the
// double (f32_round_odd).
template <class YT>
struct MergeOut;
template <>
struct MergeOut<uint16_t> {
    __device__ static void four(uint16_t* p, const double* a)
    {
        uint2 u;
        u.x = pack_bf16x2_from_double(a[0], a[1]);
        u.y = pack_bf16x2_from_double(a[2], a[3]);
        store8_nt(p, u);
    }
    __device__ static void one(uint16_t* p, double a) { *p = bf16_bits_from_double(a); }
};
template <>
struct MergeOut<float> {
    __device__ static void four(float* p, const double* a)
    {
        store16_nt(p, make_uint4(__float_as_uint((float)a[0]), __float_as_uint((float)a[1]),
                                 __float_as_uint((float)a[2]), __float_as_uint((float)a[3])));
    }
    __device__ static void one(float* p, double a) { *p = (float)a; }
};

}  // namespace rr
