// rr_axis.hip -- reduction over a non-last axis, gfx950.
//
// "reduce" (algorithm.gpu.rowwise), Args: ctx.axis is the reduce axis and the
// other dims are pinned; tier semantics: the tiled tier's thread owns
// emit_tile_width adjacent output rows, issues one tile per axis step and
// sends each lane of the tile to its own state.  x is [outer][axis][inner]
// (contiguous), y is [outer][inner]:
//   y[o][i] = fold over a = 0 .. axis-1 of x[o][a][i].
// With adjacent outputs in adjacent threads, each axis step of a wavefront
// reads one contiguous run of memory (the inner dimension is the contiguous
// one), so the strided reduction stays coalesced.
//
// Tiers:
//   TILED   a thread owns VEC (4, or 1 on the scalar path) adjacent outputs
//           and walks the whole axis in order, kAxisUnroll 16-byte loads in
//           flight; the fold order is the index order of the axis.
//   SPLITK  (few or narrow outputs, long axis) the axis is cut into G
//           slices, in two launches: a workgroup tile of GW output groups by
//           AL axis lanes folds slice g (lanes interleaved along the axis,
//           their partials folded in lane order) and stores the partials;
//           then the fold pass folds each output's G partials in ascending
//           g over a fixed tree ("cluster_allreduce", description: rank
//           order) and writes y.
//           The kernel boundary makes the partials visible; no counters.
#include <hip/hip_runtime.h>

#include "rr_config.hpp"
#include "rr_device.hpp"
#include "rr_launch.hpp"
#include "rr_launch_util.hpp"

namespace rr {

namespace {

template <class T, int VEC>
__device__ __forceinline__ Vec<T, VEC> load_group(const T* p)
{
    if constexpr (VEC == 4) {
        return load4<T, true>(p);
    } else {
        Vec<T, 1> v;
        v.v[0] = *p;
        return v;
    }
}

// Fold x[a0 .. a1) of the VEC adjacent columns at p (p points at x[o][0][i0]).
template <class M, int VEC>
__device__ __forceinline__ void fold_axis(const typename M::in_t* p, int64_t inner, int64_t a0,
                                          int64_t a1, typename M::acc_t* acc)
{
    using T = typename M::in_t;
    constexpr int U = kAxisUnroll;
    int64_t a = a0;
    for (; a + U <= a1; a += U) {
        Vec<T, VEC> v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = load_group<T, VEC>(p + (a + u) * inner);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < VEC; ++k)
                acc[k] = M::combine(acc[k], M::lift(v[u].v[k]));
    }
    for (; a < a1; ++a) {
        const Vec<T, VEC> v = load_group<T, VEC>(p + a * inner);
#pragma unroll
        for (int k = 0; k < VEC; ++k)
            acc[k] = M::combine(acc[k], M::lift(v.v[k]));
    }
}

}  // namespace

template <class M, int VEC>
__global__ __launch_bounds__(kBlockThreads) void k_reduce_axis_tiled(
    const typename M::in_t* __restrict__ x, typename M::out_t y, int64_t outer, int64_t axis,
    int64_t inner)
{
    using A = typename M::acc_t;
    const int64_t gpo = inner / VEC;  // output groups per outer index
    const int64_t ngroups = outer * gpo;
    for (int64_t q = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; q < ngroups;
         q += (int64_t)gridDim.x * kBlockThreads) {
        const int64_t o = q / gpo;
        const int64_t i0 = (q - o * gpo) * VEC;
        A acc[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k)
            acc[k] = M::identity();
        fold_axis<M, VEC>(x + o * axis * inner + i0, inner, 0, axis, acc);
#pragma unroll
        for (int k = 0; k < VEC; ++k)
            M::store(y, o * inner + i0 + k, acc[k]);
    }
}

// Fold the axis steps start, start + AL, ... below a1 of the VEC adjacent
// columns at p, in that order (AL axis lanes share a slice).
template <class M, int VEC>
__device__ __forceinline__ void fold_axis_lanes(const typename M::in_t* p, int64_t inner,
                                                int64_t start, int64_t a1, int64_t AL,
                                                typename M::acc_t* acc)
{
    using T = typename M::in_t;
    constexpr int U = kAxisSplitKUnroll;
    int64_t a = start;
    for (; a + (U - 1) * AL < a1; a += U * AL) {
        Vec<T, VEC> v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = load_group<T, VEC>(p + (a + u * AL) * inner);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < VEC; ++k)
                acc[k] = M::combine(acc[k], M::lift(v[u].v[k]));
    }
    for (; a < a1; a += AL) {
        const Vec<T, VEC> v = load_group<T, VEC>(p + a * inner);
#pragma unroll
        for (int k = 0; k < VEC; ++k)
            acc[k] = M::combine(acc[k], M::lift(v.v[k]));
    }
}

// Split-K partial pass.  A workgroup is a 2-D tile: GW = 2^gw_log2 output
// groups (of VEC adjacent outputs, one outer index) by AL = 256 / GW axis
// lanes.  Lane l of slice g folds steps a0 + l, a0 + l + AL, ..., so at each
// step the AL lanes read AL consecutive rows of the inner dimension -- one
// contiguous block when the inner dimension is narrow.  The AL lane partials
// of an output are then folded in lane order through LDS and stored to
// part[g][output]; part is [G][outer * inner] of acc_t.
template <class M, int VEC>
__global__ __launch_bounds__(kBlockThreads) void k_reduce_axis_partial(
    const typename M::in_t* __restrict__ x, int64_t outer, int64_t axis, int64_t inner, int32_t G,
    int32_t gw_log2, typename M::acc_t* __restrict__ part)
{
    using A = typename M::acc_t;
    __shared__ A red[kBlockThreads * VEC];
    const int GW = 1 << gw_log2;
    const int AL = kBlockThreads >> gw_log2;
    const int gl = (int)threadIdx.x & (GW - 1);
    const int al = (int)threadIdx.x >> gw_log2;
    const int64_t gpo = inner / VEC;          // output groups per outer index
    const int64_t bpo = ceil_div(gpo, (int64_t)GW);  // tiles per outer index
    const int64_t ntile = outer * bpo;
    const int64_t nout = outer * inner;
    const int64_t slice = ceil_div(axis, (int64_t)G);
    for (int64_t b = blockIdx.x; b < ntile * G; b += gridDim.x) {
        const int64_t w = b / G;
        const int32_t g = (int32_t)(b - w * G);
        const int64_t o = w / bpo;
        const int64_t grp = (w - o * bpo) * GW + gl;
        const bool valid = grp < gpo;
        const int64_t i0 = grp * VEC;
        const int64_t a0 = (int64_t)g * slice;
        const int64_t a1 = a0 + slice < axis ? a0 + slice : axis;
        A acc[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k)
            acc[k] = M::identity();
        if (valid)
            fold_axis_lanes<M, VEC>(x + o * axis * inner + i0, inner, a0 + al, a1, AL, acc);
#pragma unroll
        for (int k = 0; k < VEC; ++k)
            red[((int)threadIdx.x) * VEC + k] = acc[k];  // = [al][gl][k]
        __syncthreads();
        if (al == 0 && valid) {
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                A r = red[gl * VEC + k];
                for (int l = 1; l < AL; ++l)
                    r = M::combine(r, red[(l * GW + gl) * VEC + k]);
                part[(int64_t)g * nout + o * inner + i0 + k] = r;
            }
        }
        __syncthreads();  // red is rewritten by the next tile
    }
}

// Fold pass.  A workgroup is FO = 256 >> gl_log2 outputs by GL = 2^gl_log2
// slice lanes; lane l folds the contiguous slices l*G/GL .. (l+1)*G/GL - 1
// in ascending order, and the GL lane results of an output are folded in
// lane order through LDS: ascending slice order over a fixed tree.
template <class M>
__global__ __launch_bounds__(kBlockThreads) void k_reduce_axis_fold(
    typename M::out_t y, int64_t nout, int32_t G, int32_t gl_log2,
    const typename M::acc_t* __restrict__ part)
{
    using A = typename M::acc_t;
    __shared__ A red[kBlockThreads];
    const int GL = 1 << gl_log2;
    const int FO = kBlockThreads >> gl_log2;
    const int lane = (int)threadIdx.x & (GL - 1);
    const int fo = (int)threadIdx.x >> gl_log2;
    const int32_t s0 = (int32_t)(((int64_t)G * lane) / GL);
    const int32_t s1 = (int32_t)(((int64_t)G * (lane + 1)) / GL);
    for (int64_t j0 = (int64_t)blockIdx.x * FO; j0 < nout; j0 += (int64_t)gridDim.x * FO) {
        const int64_t j = j0 + fo;
        A a = M::identity();
        if (j < nout)
            for (int32_t s = s0; s < s1; ++s)
                a = M::combine(a, part[(int64_t)s * nout + j]);
        red[threadIdx.x] = a;  // [fo][lane]
        __syncthreads();
        if (lane == 0 && j < nout) {
            A r = red[fo * GL];
            for (int l = 1; l < GL; ++l)
                r = M::combine(r, red[fo * GL + l]);
            M::store(y, j, r);
        }
        __syncthreads();
    }
}

template <class M>
static rr_status launch_axis_monoid(const rr_plan& p, const AxisLaunch& a)
{
    using T = typename M::in_t;
    using A = typename M::acc_t;
    const T* x = static_cast<const T*>(a.x);
    const typename M::out_t y = static_cast<typename M::out_t>(a.y);
    const dim3 grid((unsigned)(p.grid > kMaxGrid ? kMaxGrid : p.grid)), block(kBlockThreads);
    if (p.tier == RR_TIER_TILED || p.tier == RR_TIER_SERIAL)  // SERIAL: a.vec is false
        return a.vec ? launch_kernel(k_reduce_axis_tiled<M, 4>, grid, block, 0, a.stream, x, y,
                                     a.outer, a.axis, a.inner)
                     : launch_kernel(k_reduce_axis_tiled<M, 1>, grid, block, 0, a.stream, x, y,
                                     a.outer, a.axis, a.inner);
    if (p.tier == RR_TIER_SPLITK) {
        A* part = static_cast<A*>(a.workspace);
        const int32_t gwl = axis_tile_log2(a.inner / (a.vec ? 4 : 1));
        rr_status st =
            a.vec ? launch_kernel(k_reduce_axis_partial<M, 4>, grid, block, 0, a.stream, x,
                                  a.outer, a.axis, a.inner, p.slices, gwl, part)
                  : launch_kernel(k_reduce_axis_partial<M, 1>, grid, block, 0, a.stream, x,
                                  a.outer, a.axis, a.inner, p.slices, gwl, part);
        if (st != RR_OK)
            return st;
        const int64_t nout = a.outer * a.inner;
        const int32_t gll = axis_fold_lanes_log2(p.slices);
        int64_t fg = ceil_div(nout, (int64_t)(kBlockThreads >> gll));
        if (fg > kMaxGrid)
            fg = kMaxGrid;
        return launch_kernel(k_reduce_axis_fold<M>, dim3((unsigned)fg), block, 0, a.stream, y,
                             nout, p.slices, gll, (const A*)part);
    }
    return RR_ERR_TIER;
}

rr_status launch_reduce_axis(const rr_plan& p, const AxisLaunch& a)
{
    if (a.dtype == RR_F32) {
        switch (a.op) {
        case RR_SUM: return launch_axis_monoid<SumF32>(p, a);
        case RR_MAX: return launch_axis_monoid<MaxF32>(p, a);
        case RR_MIN: return launch_axis_monoid<MinF32>(p, a);
        default: break;
        }
    } else if (a.dtype == RR_I32) {
        switch (a.op) {
        case RR_SUM: return launch_axis_monoid<SumI32>(p, a);
        case RR_MAX: return launch_axis_monoid<MaxI32>(p, a);
        case RR_MIN: return launch_axis_monoid<MinI32>(p, a);
        default: break;
        }
    }
    return RR_ERR_DTYPE;
}

}  // namespace rr
