// rr_merge.hip -- split-K log-sum-exp merge of partial attention outputs.
//
// "fa4_splitk_reduce_scatter_write", per-band steps: each partition's output
// is scaled by its weight w[b], the other partitions' outputs are
// accumulated onto it, and the result is packed to bf16; every partition
// joins, and an empty one contributes nothing.  The pages' statistics are the
// row max and row sum of each partition (own_max, own_sum).
//
// Per row: partition p is empty when l_p <= 0 or m_p == -inf; M is the
// largest m_p of the non-empty ones; w_p = exp(scale * (m_p - M)) * l_p;
// W = sum w_p; out = sum over non-empty p (ascending) of (w_p / W) * O_p.
// Weights and the accumulation are double precision with fused multiply-add
// (rr_merge_math.hpp, shared with the fused split-K attention).
//
// One workgroup takes `rw` rows.  Phase 1 stages (m_p, l_p) of those rows in
// LDS, phase 2 forms w_p, phase 3 the coefficients c_p = w_p / W (or -1 for
// an empty partition, which is then skipped -- a NaN O_p of an empty
// partition never enters the sum).  The depth axis is spread over LPR lanes
// per row with 128-bit loads; the first batch of partial outputs is loaded
// before the weight phases so its latency overlaps them.
#include <hip/hip_runtime.h>

#include "rr_config.hpp"
#include "rr_device.hpp"
#include "rr_launch.hpp"
#include "rr_launch_util.hpp"
#include "rr_merge_math.hpp"
#include "rr_rowio.hpp"

namespace rr {

template <int VE>
struct OChunk {
    float v[VE];
};

template <int VE>
__device__ __forceinline__ OChunk<VE> load_o(const float* p)
{
    OChunk<VE> c;
    if constexpr (VE == 4) {
        uint4 u = load16_nt(p);
        c.v[0] = __uint_as_float(u.x); c.v[1] = __uint_as_float(u.y);
        c.v[2] = __uint_as_float(u.z); c.v[3] = __uint_as_float(u.w);
    } else {
        c.v[0] = *p;
    }
    return c;
}

// LDS per workgroup: per (row, partition) one double w and one 8-byte cell
// that first holds (m_p, l_p) as two floats and then the coefficient c_p
// (the cell array has at least one entry per thread).
template <class YT, int VE, int LPR>
__global__ __launch_bounds__(kBlockThreads) void k_lse_merge(const float* __restrict__ o,
                                                             const float* __restrict__ m,
                                                             const float* __restrict__ l,
                                                             YT* __restrict__ out, int32_t P,
                                                             int64_t rows, int32_t depth,
                                                             float scale, int32_t rw)
{
    constexpr int B = kMergeBatch;
    extern __shared__ double lds[];
    const int32_t npairs = rw * P;
    double* wd = lds;                                      // [npairs]
    double* cell = lds + npairs;                           // [max(npairs, block)]
    float2* stat = reinterpret_cast<float2*>(cell);        // same cells as (m, l)

    const int q = threadIdx.x / LPR;       // row of this lane within the workgroup
    const int li = threadIdx.x % LPR;      // lane within the row
    const int64_t nblocks = ceil_div(rows, rw);

    for (int64_t blk = blockIdx.x; blk < nblocks; blk += gridDim.x) {
        const int64_t row_base = blk * rw;
        const int64_t r = row_base + q;
        const bool row_ok = q < rw && r < rows;
        const int64_t d_first = (int64_t)li * VE;
        const bool lane_ok = row_ok && d_first < depth;

        // (m_p, l_p) of this thread's first (row, partition) pair ...  The
        // loads below are unconditional at clamped, always valid addresses
        // (branch-free code keeps the later waits partial); values loaded
        // for lanes without work are discarded.
        const int32_t i0 = (int32_t)threadIdx.x < npairs ? (int32_t)threadIdx.x : npairs - 1;
        const int32_t q0 = i0 / P, p0i = i0 - q0 * P;
        const int64_t r0 = row_base + q0 < rows ? row_base + q0 : rows - 1;
        const float m0 = m[(int64_t)p0i * rows + r0];
        const float l0 = l[(int64_t)p0i * rows + r0];
        __builtin_amdgcn_sched_barrier(0);  // issue (m, l) before the partial outputs
        // ... then the first batch of partial outputs, consumed after the
        // weight phases, so the HBM latency of both overlaps them.
        const int64_t rc = r < rows ? r : rows - 1;
        const int64_t dc = lane_ok ? d_first : 0;
        OChunk<VE> ch[B];
#pragma unroll
        for (int b = 0; b < B; ++b)
            ch[b] = load_o<VE>(o + ((int64_t)(b < P ? b : P - 1) * rows + rc) * depth + dc);
        const bool st0_ok = (int32_t)threadIdx.x < npairs && row_base + q0 < rows;

        // Phase 1: stage (m_p, l_p) in LDS.  Every thread writes its cell
        // (cells past npairs are never read), so no branch separates the
        // loads above from this use.
        stat[threadIdx.x] = make_float2(st0_ok ? m0 : -__builtin_inff(), st0_ok ? l0 : 0.0f);
        for (int32_t i = threadIdx.x + kBlockThreads; i < npairs; i += kBlockThreads) {
            const int32_t qq = i / P, p = i - qq * P;
            float2 st = make_float2(-__builtin_inff(), 0.0f);
            if (row_base + qq < rows)
                st = make_float2(m[(int64_t)p * rows + row_base + qq],
                                 l[(int64_t)p * rows + row_base + qq]);
            stat[i] = st;
        }
        __syncthreads();
        // Phase 2: M over the non-empty partitions of the row, then w_p.
        for (int32_t i = threadIdx.x; i < npairs; i += kBlockThreads) {
            const int32_t qq = i / P;
            const double M = merge_row_max(stat + (int64_t)qq * P, P);
            wd[i] = merge_weight(stat[i], M, scale);
        }
        __syncthreads();
        // Phase 3: W in ascending partition order, then c_p (or -1 if empty).
        for (int32_t i = threadIdx.x; i < npairs; i += kBlockThreads) {
            const int32_t qq = i / P;
            const double W = merge_total(wd + (int64_t)qq * P, P);
            cell[i] = merge_coef(stat[i], wd[i], W);
        }
        __syncthreads();

        // Accumulate: out[d] = sum_p c_p * O_p[d], ascending p, empty p skipped.
        if (row_ok) {
            const double* c = cell + (int64_t)q * P;
            for (int64_t d0 = d_first; d0 < depth; d0 += (int64_t)LPR * VE) {
                double acc[VE];
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    acc[e] = 0.0;
                for (int32_t p0 = 0; p0 < P; p0 += B) {
                    if (d0 != d_first || p0 != 0) {
#pragma unroll
                        for (int b = 0; b < B; ++b)
                            ch[b] = load_o<VE>(o + ((int64_t)(p0 + b < P ? p0 + b : P - 1) * rows + r) * depth + d0);
                    }
#pragma unroll
                    for (int b = 0; b < B; ++b)
                        if (p0 + b < P)
                            merge_accumulate<VE>(acc, c[p0 + b], ch[b].v);
                }
                YT* orow = out + r * depth + d0;
                if (VE == 4 && d0 + 4 <= depth) {
                    MergeOut<YT>::four(orow, acc);
                } else {
#pragma unroll
                    for (int e = 0; e < VE; ++e)
                        if (d0 + e < depth)
                            MergeOut<YT>::one(orow + e, acc[e]);
                }
            }
        }
        __syncthreads();  // LDS is reused by the next row block
    }
}

// ------------------------------------------- partition-outer fast path
// depth == LPR * 4 (one 128-bit chunk per lane per row), P <= kMergePOuterMaxP.
// A workgroup takes RW = (256 / LPR) * K rows; lane group q owns rows
// q, q + 256/LPR, ... (K of them).  After the weight phases it walks the
// partitions in ascending order and, for each, reads that partition's chunk
// of its K rows -- so the workgroup reads K * 4 KiB (LPR = 32) of one
// partition at a time instead of one row of all partitions -- with the next
// partition's loads in flight (two alternating buffers, clamped look-ahead).
// Per output element the arithmetic and its order are those of k_lse_merge.
template <int K>
struct Chunks {
    OChunk<4> c[K];
};

// Partition p's chunks of the K rows rk.  BUF (a partition of at most 2^31
// bytes): buffer loads over partition p's range, which is empty when live
// is false, so a look-ahead past the last partition reads zeros and no
// memory (a clamped one would read the last partition again); else plain
// non-temporal loads, the look-ahead clamped by the caller.
template <int LPR, int K, bool BUF>
__device__ __forceinline__ void po_load(const float* __restrict__ o, int64_t rows, int32_t depth,
                                        int32_t p, const int64_t* rk, Chunks<K>& dst,
                                        bool live = true)
{
    const int64_t d = (int64_t)(threadIdx.x % LPR) * 4;
    if constexpr (BUF) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(o + (int64_t)p * rows * depth), 0,
            live ? (int)(rows * depth * 4) : 0, kBufferWord3);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const rr_u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(
                rs, (int)((rk[k] * depth + d) * 4), 0, kBufferNonTemporal);
            dst.c[k].v[0] = __uint_as_float(u.x);
            dst.c[k].v[1] = __uint_as_float(u.y);
            dst.c[k].v[2] = __uint_as_float(u.z);
            dst.c[k].v[3] = __uint_as_float(u.w);
        }
    } else {
#pragma unroll
        for (int k = 0; k < K; ++k)
            dst.c[k] = load_o<4>(o + ((int64_t)p * rows + rk[k]) * depth + d);
    }
}

// The coefficient of (row q, partition p) is cell[p * RW + q].
template <int K, int RW>
__device__ __forceinline__ void po_fold(double (*acc)[4], const Chunks<K>& ch, const double* cell,
                                        const int* qk, int32_t p)
{
#pragma unroll
    for (int k = 0; k < K; ++k) {
        merge_accumulate<4>(acc[k], cell[p * RW + qk[k]], ch.c[k].v);
    }
}

template <class YT, int LPR, int K, bool BUF>
__global__ __launch_bounds__(kBlockThreads) void k_lse_merge_po(const float* __restrict__ o,
                                                                const float* __restrict__ m,
                                                                const float* __restrict__ l,
                                                                YT* __restrict__ out, int32_t P,
                                                                int64_t rows, int32_t depth,
                                                                float scale)
{
    constexpr int GR = kBlockThreads / LPR;  // rows per lane-group pass
    constexpr int RW = GR * K;                // rows per workgroup
    extern __shared__ double lds[];
    const int32_t npairs = RW * P;
    double* wd = lds;                                  // [npairs]
    double* cell = lds + npairs;                       // [max(npairs, block)]
    float2* stat = reinterpret_cast<float2*>(cell);
    const int q = threadIdx.x / LPR;
    const int64_t nblocks = ceil_div(rows, RW);

    for (int64_t blk = blockIdx.x; blk < nblocks; blk += gridDim.x) {
        const int64_t row_base = blk * RW;
        int qk[K];
        int64_t rk[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            qk[k] = q + GR * k;
            const int64_t r = row_base + qk[k];
            rk[k] = r < rows ? r : rows - 1;
        }
        // Statistics of this thread's first pair, then partition 0's chunks.
        // Pairs are partition-major, cell i = p * RW + q (row fastest): a
        // wavefront reads whole 128-byte lines of m and l (32 rows of one
        // partition), and consecutive lanes touch consecutive LDS cells.
        const int32_t i0 = (int32_t)threadIdx.x < npairs ? (int32_t)threadIdx.x : npairs - 1;
        const int32_t p0i = i0 / RW, q0 = i0 - p0i * RW;
        const int64_t r0 = row_base + q0 < rows ? row_base + q0 : rows - 1;
        const float m0 = m[(int64_t)p0i * rows + r0];
        const float l0 = l[(int64_t)p0i * rows + r0];
        __builtin_amdgcn_sched_barrier(0);
        Chunks<K> A, B;
        po_load<LPR, K, BUF>(o, rows, depth, 0, rk, A);
        const bool st0_ok = (int32_t)threadIdx.x < npairs && row_base + q0 < rows;

        // Phase 1: stage (m_p, l_p) (cells past npairs are never read).
        stat[threadIdx.x] = make_float2(st0_ok ? m0 : -__builtin_inff(), st0_ok ? l0 : 0.0f);
        for (int32_t i = threadIdx.x + kBlockThreads; i < npairs; i += kBlockThreads) {
            const int32_t p = i / RW, qq = i - p * RW;
            float2 st = make_float2(-__builtin_inff(), 0.0f);
            if (row_base + qq < rows)
                st = make_float2(m[(int64_t)p * rows + row_base + qq],
                                 l[(int64_t)p * rows + row_base + qq]);
            stat[i] = st;
        }
        __syncthreads();
        // Phase 2: M over the non-empty partitions of the row, then w_p.
        for (int32_t i = threadIdx.x; i < npairs; i += kBlockThreads) {
            const int32_t qq = i % RW;
            const double M = merge_row_max(stat + qq, P, RW);
            wd[i] = merge_weight(stat[i], M, scale);
        }
        __syncthreads();
        // Phase 3: W in ascending partition order, then c_p (or -1 if empty).
        for (int32_t i = threadIdx.x; i < npairs; i += kBlockThreads) {
            const int32_t qq = i % RW;
            const double W = merge_total(wd + qq, P, RW);
            cell[i] = merge_coef(stat[i], wd[i], W);
        }
        __syncthreads();

        // Accumulate partition by partition, ascending p.
        double acc[K][4];
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc[k][e] = 0.0;
        for (int32_t p = 0;;) {
            const int32_t pn = p + 1 < P ? p + 1 : p;
            po_load<LPR, K, BUF>(o, rows, depth, pn, rk, B, p + 1 < P);
            po_fold<K, RW>(acc, A, cell, qk, p);
            if (++p >= P)
                break;
            const int32_t pn2 = p + 1 < P ? p + 1 : p;
            po_load<LPR, K, BUF>(o, rows, depth, pn2, rk, A, p + 1 < P);
            po_fold<K, RW>(acc, B, cell, qk, p);
            if (++p >= P)
                break;
        }
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (row_base + qk[k] < rows)
                MergeOut<YT>::four(out + (row_base + qk[k]) * depth +
                                       (int64_t)(threadIdx.x % LPR) * 4, acc[k]);
        __syncthreads();  // LDS is reused by the next row block
    }
}

// The partition-outer path holds 16 bytes of LDS per (row, partition) of a
// workgroup; it is taken when that fits in 32 KiB.
template <int LPR>
static bool po_fits(int32_t P)
{
    constexpr int RW = (kBlockThreads / LPR) * kMergePOuterRowsPerLane;
    return (int64_t)RW * P * 16 <= 32768;
}

template <class YT, int LPR>
static rr_status launch_po(const MergeLaunch& a)
{
    constexpr int K = kMergePOuterRowsPerLane;
    constexpr int RW = (kBlockThreads / LPR) * K;
    int64_t grid = ceil_div(a.rows, RW);
    if (grid > kMaxGrid) grid = kMaxGrid;
    const int64_t npairs = (int64_t)RW * a.P;
    const size_t lds = (size_t)8 * npairs + (size_t)8 * (npairs > kBlockThreads ? npairs : kBlockThreads);
    // buffer loads when one partition's bytes fit a 31-bit offset
    auto kernel = a.rows * (int64_t)a.depth * 4 <= (int64_t)INT32_MAX ? k_lse_merge_po<YT, LPR, K, true>
                                                                      : k_lse_merge_po<YT, LPR, K, false>;
    return launch_kernel(kernel, dim3((unsigned)grid), dim3(kBlockThreads), lds, a.stream, a.o,
                         a.m, a.l, static_cast<YT*>(a.out), a.P, a.rows, a.depth, a.scale);
}

static int lanes_per_row(int32_t depth, int ve)
{
    const int64_t chunks = ceil_div(depth, ve);
    int lpr = 4;
    while (lpr < 64 && lpr < chunks)
        lpr *= 2;
    return lpr;
}

template <class YT, int VE, int LPR>
static rr_status launch_lpr(const MergeLaunch& a)
{
    constexpr int RW = kBlockThreads / LPR;
    // 16 bytes of LDS per (row, partition); keep a workgroup within 32 KiB.
    int32_t rw = (int32_t)(32768 / (16 * (int64_t)a.P));
    if (rw > RW) rw = RW;
    if (rw < 1) rw = 1;
    int64_t grid = ceil_div(a.rows, rw);
    if (grid > kMaxGrid) grid = kMaxGrid;
    const int64_t npairs = (int64_t)rw * a.P;
    const size_t lds = (size_t)8 * npairs + (size_t)8 * (npairs > kBlockThreads ? npairs : kBlockThreads);
    return launch_kernel(k_lse_merge<YT, VE, LPR>, dim3((unsigned)grid), dim3(kBlockThreads), lds,
                         a.stream, a.o, a.m, a.l, static_cast<YT*>(a.out), a.P, a.rows, a.depth,
                         a.scale, rw);
}

template <class YT, int VE>
static rr_status launch_ve(const MergeLaunch& a)
{
    if constexpr (VE == 4) {
        if (a.P <= kMergePOuterMaxP) {
            switch (a.depth) {  // one 128-bit chunk per lane
            case 16: if (po_fits<4>(a.P)) return launch_po<YT, 4>(a); break;
            case 32: if (po_fits<8>(a.P)) return launch_po<YT, 8>(a); break;
            case 64: if (po_fits<16>(a.P)) return launch_po<YT, 16>(a); break;
            case 128: if (po_fits<32>(a.P)) return launch_po<YT, 32>(a); break;
            case 256: if (po_fits<64>(a.P)) return launch_po<YT, 64>(a); break;
            default: break;
            }
        }
    }
    switch (lanes_per_row(a.depth, VE)) {
    case 4: return launch_lpr<YT, VE, 4>(a);
    case 8: return launch_lpr<YT, VE, 8>(a);
    case 16: return launch_lpr<YT, VE, 16>(a);
    case 32: return launch_lpr<YT, VE, 32>(a);
    default: return launch_lpr<YT, VE, 64>(a);
    }
}

rr_status launch_merge(const MergeLaunch& a)
{
    if (a.out_dtype == RR_BF16)
        return a.vec ? launch_ve<uint16_t, 4>(a) : launch_ve<uint16_t, 1>(a);
    return a.vec ? launch_ve<float, 4>(a) : launch_ve<float, 1>(a);
}

}  // namespace rr
