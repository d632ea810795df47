// rr_softmax.hip -- two-pass row softmax over the last axis, gfx950.
//
// "reduce" (algorithm.gpu.rowwise), description: softmax is two passes;
// pass 1 folds a monoid over the row -- here the online (max, sum) pair --
// and pass 2 is a pure map that writes y = exp(x - max) / sum.  The tiers
// reuse the row-reduce shapes (wave / block / tiled / serial).
//
// Block tier, row held in registers: each thread keeps its chunks of the row
// in VGPRs through both passes, so x is read from HBM once.  Pass 1 takes the
// thread's own maximum m_t, turns every element into p = exp(x - m_t) and sums
// them (one exponential per element); the (m_t, s_t) pairs are then combined
// across the workgroup, and pass 2 writes p * exp(m_t - M) / S.
// Exponentials are exp2 of (x - m) * log2(e).
#include <hip/hip_runtime.h>

#include "rr_config.hpp"
#include "rr_device.hpp"
#include "rr_launch.hpp"
#include "rr_launch_util.hpp"
#include "rr_rowio.hpp"

namespace rr {

constexpr float kNegInf = -__builtin_inff();

// Pass 1 on values held by one thread: m = max, v <- exp(v - m), s = sum v.
// With m == -inf (nothing but -inf / padding) every p is 0.
// The exponent argument is (x - m) * log2(e): the difference first, so its
// error is relative to the (small) argument whatever the size of m.  A
// fused x*log2(e) - m*log2(e) would carry the rounding of m*log2(e), half an
// ulp of |m|*1.44, into every exponent (a relative error of 4e-5 at m = 1000,
// different in every thread).  The hardware exponential is exact for normal
// results; when any argument falls below -126 (a subnormal or vanishing
// result, or a -inf entry) the thread takes exp2_sub, which scales such
// arguments into the normal range.  m is the thread's maximum.  live(i, t):
// whether value i is a row element; the others (-inf padding, whose
// exponential the hardware gives as 0 exactly) leave the range check alone,
// so padding alone does not send a thread to the slow path.  It is given
// i and the exponent argument t of value i.
struct AllLive {
    __device__ bool operator()(int, float) const { return true; }
};
// Every -inf value treated as padding: both exponentials give exactly 0 for
// it, and on arguments down to -126 they agree bit for bit, so a thread
// whose only low arguments are -inf may take the hardware path.  A test on
// the value, where a test on the position would cost 64-bit index
// arithmetic per element.
struct FiniteLive {
    __device__ bool operator()(int, float t) const { return t != kNegInf; }
};
template <int N, class Live = AllLive>
__device__ __forceinline__ MS exp_sum_from(float* v, float m, Live live = Live())
{
    float s = 0.0f;
    if (m != kNegInf) {
        float tmin = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            v[i] = (v[i] - m) * kLog2e;
            tmin = fminf(tmin, live(i, v[i]) ? v[i] : 0.0f);
        }
        if (tmin >= -126.0f) {
#pragma unroll
            for (int i = 0; i < N; ++i)
                v[i] = exp2_hw(v[i]);
        } else {
            keep_branch();
#pragma unroll
            for (int i = 0; i < N; ++i)
                v[i] = exp2_sub(v[i]);
        }
#pragma unroll
        for (int i = 0; i < N; ++i)
            s += v[i];
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i)
            v[i] = 0.0f;
    }
    return MS{m, s};
}

template <int N, class Live = AllLive>
__device__ __forceinline__ MS local_exp_sum(float* v, Live live = Live())
{
    float m = kNegInf;
#pragma unroll
    for (int i = 0; i < N; ++i)
        m = fmaxf(m, v[i]);
    return exp_sum_from<N>(v, m, live);
}

// Pass 1 on a thread's N values plus one more element e (a misaligned row's
// head or tail element, or -inf for none): the maximum covers both; e's
// exponential (exp2_sub, any range) is added after the others' sum and
// returned in *pe for pass 2.
template <int N, class Live = AllLive>
__device__ __forceinline__ MS local_exp_sum_plus(float* v, float e, float* pe,
                                                 Live live = Live())
{
    float m = e;
#pragma unroll
    for (int i = 0; i < N; ++i)
        m = fmaxf(m, v[i]);
    MS own = exp_sum_from<N>(v, m, live);
    const float p = e == kNegInf ? 0.0f : exp2_sub((e - m) * kLog2e);
    own.s += p;
    *pe = p;
    return own;
}

// Row statistics (M, S) over the workgroup from each thread's (m_t, s_t),
// identical bits in every thread, and the thread's own factor
// e_t = exp(m_t - M).  Inside a wavefront only the cheap monoids run: a max
// of m_t, one exponential per lane to bring s_t to the wavefront max, and a
// sum; the per-wavefront pairs are then folded in wave order with the online
// (max, sum) combine.  Fixed shapes throughout, so the bits do not change
// from run to run.
template <int NT>
__device__ __forceinline__ MS block_softmax_stats(MS own, MS* slot, float* e_t)
{
    constexpr int NW = NT / kWave;
    const float mw = wave_reduce<MaxFloat>(own.m);
    const float ew = mw == kNegInf ? 0.0f : exp2_hw((own.m - mw) * kLog2e);
    const float sw = wave_reduce<SumFloat>(own.s * ew);
    MS tot = MS{mw, sw};
    if constexpr (NW > 1) {
        if (lane_id() == 0)
            slot[threadIdx.x / kWave] = tot;
        __syncthreads();
        tot = slot[0];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            tot = SoftmaxMS::combine(tot, slot[w]);
    }
    *e_t = exp2_f32((own.m - tot.m) * kLog2e);
    return tot;
}

// ------------------------------------------- block tier, row in registers
// VEC: each row's body from its first 16-byte boundary goes in chunks (the
// tail chunk element by element); the head, h < E elements before that
// boundary, one element to each of the first threads.  y's chunks are stored
// whole when y + h is aligned for them, else element by element.
template <class XT, class YT, int NCH, bool VEC, int NT>
__global__ __launch_bounds__(NT) void k_softmax_block(const XT* __restrict__ x,
                                                      YT* __restrict__ y, int64_t rows,
                                                      int64_t cols, int64_t ldx, int64_t ldy)
{
    constexpr int E = VEC ? XIn<XT>::kChunk : 1;
    __shared__ MS slot[2][NT / kWave];
    int par = 0;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const XT* xr = x + r * ldx;
        YT* yr = y + r * ldy;
        const int64_t h = VEC ? head_elems(xr, cols) : 0;
        const int64_t cb = cols - h;
        const bool yvec = VEC && chunk_aligned<YT, E>(yr + h);
        float v[NCH * E];
#pragma unroll
        for (int k = 0; k < NCH; ++k)
            load_padded<XT, E, VEC>(xr + h, ((int64_t)threadIdx.x + (int64_t)k * NT) * E, cb,
                                    v + k * E);
        const bool has_e = (int64_t)threadIdx.x < h;
        const float e = has_e ? XIn<XT>::one(xr + threadIdx.x) : kNegInf;
        float pe;
        const MS own = local_exp_sum_plus<NCH * E>(v, e, &pe, FiniteLive());
        float e_t;
        const MS tot = block_softmax_stats<NT>(own, slot[par], &e_t);
        par ^= 1;
        const float sc = e_t / tot.s;
#pragma unroll
        for (int i = 0; i < NCH * E; ++i)
            v[i] *= sc;
#pragma unroll
        for (int k = 0; k < NCH; ++k)
            store_masked_rt<YT, E>(yr + h, ((int64_t)threadIdx.x + (int64_t)k * NT) * E, cb,
                                   v + k * E, yvec);
        if (has_e)
            YOut<YT>::one(yr + threadIdx.x, pe * sc);
    }
}

// ------------------------- block tier, persistent rows with prefetch
// Workgroup b takes rows b, b + grid, b + 2*grid, ... and loads the next
// row's chunks while it computes the current one, so each workgroup keeps a
// row's worth of loads in flight through its compute phase.  Two register
// buffers alternate; when there is no next row the prefetch goes out with no
// bytes to read and is dropped, so no load sits behind a branch.
// EXACT: cols == NT * NCH * chunk and every row 16-byte aligned, so every
// chunk of every thread is in the row and no per-chunk bound check is
// emitted.  PEEL: rows at any element offset or length -- each row's body
// of whole chunks from its first 16-byte boundary, and one head or tail
// element per thread (PeelGeom); y's chunks are stored whole when y + h is
// aligned for them.  Neither: 16-byte aligned rows of whole chunks.
template <class XT, class YT, int NCH, int NT, bool EXACT, bool PEEL, bool ROT>
__device__ __forceinline__ void softmax_row_from_chunks(const RowBuf<NCH>& buf, const XT* xr,
                                                        YT* yr, int64_t cols, MS* slot)
{
    constexpr int E = XIn<XT>::kChunk;
    int64_t h = 0, nbe = cols, idx = -1;
    if constexpr (PEEL) {
        const PeelGeom<XT> pg(xr, cols);
        h = pg.h;
        nbe = pg.nbe;
        idx = pg.idx;
    }
    const int q = ROT ? line_phase(xr + h) : 0;  // as the row's loads
    float v[NCH * E];
    bool ok[NCH];  // the slot holds a chunk of the row's body
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int64_t j0 = (int64_t)slot_chunk<NCH, NT, ROT>(k, q) * E;
        ok[k] = EXACT || j0 < nbe;
        if (ok[k]) {
            unpack_chunk<XT>(buf.c[k], v + k * E);
        } else {
#pragma unroll
            for (int i = 0; i < E; ++i)
                v[k * E + i] = kNegInf;
        }
    }
    float pe = 0.0f;
    const auto live = [&](int i, float) { return ok[i / E]; };
    const MS own = PEEL ? local_exp_sum_plus<NCH * E>(v, buf.e, &pe, live)
                        : local_exp_sum<NCH * E>(v, live);
    float e_t;
    const MS tot = block_softmax_stats<NT>(own, slot, &e_t);
    const float sc = e_t / tot.s;
#pragma unroll
    for (int i = 0; i < NCH * E; ++i)
        v[i] *= sc;
    if constexpr (EXACT) {
#pragma unroll
        for (int k = 0; k < NCH; ++k)
            YOut<YT>::template chunk<E>(yr + (int64_t)slot_chunk<NCH, NT, ROT>(k, q) * E, v + k * E);
    } else {
        store_row_peeled<YT, E, NCH, NT, ROT>(yr, cols, h, nbe, idx, v, pe * sc, q);
    }
}

// PEEL rows are always rotated; ROT rotates whole-chunk rows that do not all
// start on a 128-byte line.
template <class XT, class YT, int NCH, int NT, bool EXACT, bool PEEL, bool ROT>
__global__ __launch_bounds__(NT) void k_softmax_rows_pf(const XT* __restrict__ x,
                                                        YT* __restrict__ y, int64_t rows,
                                                        int64_t cols, int64_t ldx, int64_t ldy)
{
    __shared__ MS slot[2][NT / kWave];
    if ((int64_t)blockIdx.x >= rows)
        return;
    persistent_rows<RowBuf<NCH>>(
        blockIdx.x, gridDim.x, rows,
        [&](int64_t r, bool live, RowBuf<NCH>& buf) {
            if constexpr (PEEL)
                load_row_peeled<XT, NCH, NT>(x + r * ldx, cols, live, buf);
            else
                load_row_raw<NCH, NT, ROT>(x + r * ldx, live ? cols * (int64_t)sizeof(XT) : 0,
                                           buf.c);
        },
        [] {},
        [&](const RowBuf<NCH>& buf, int64_t r, int par) {
            softmax_row_from_chunks<XT, YT, NCH, NT, EXACT, PEEL, PEEL || ROT>(buf, x + r * ldx,
                                                                               y + r * ldy,
                                                                  cols, slot[par]);
        });
}

// ---------------------------------------- block tier, streaming long rows
// Pass 1 folds (m, s) chunk by chunk; pass 2 reads x again.  VEC: the row's
// body from its first 16-byte boundary in chunks, the head (h < E elements)
// first, one element to each of the first threads.
template <class XT, class YT, bool VEC, int NT>
__global__ __launch_bounds__(NT) void k_softmax_stream(const XT* __restrict__ x,
                                                       YT* __restrict__ y, int64_t rows,
                                                       int64_t cols, int64_t ldx, int64_t ldy)
{
    constexpr int E = VEC ? XIn<XT>::kChunk : 1;
    __shared__ MS slot[2][NT / kWave];
    int par = 0;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const XT* xr0 = x + r * ldx;
        YT* yr0 = y + r * ldy;
        const int64_t h = VEC ? head_elems(xr0, cols) : 0;
        const bool has_e = (int64_t)threadIdx.x < h;
        const XT* xr = xr0 + h;
        YT* yr = yr0 + h;
        const int64_t cb = cols - h;
        const bool yvec = VEC && chunk_aligned<YT, E>(yr);
        // per-thread running (m, s); s is kept in double because a thread
        // adds many terms in sequence on long rows
        float tm = kNegInf;
        double ts = 0.0;
        if (has_e) {
            tm = XIn<XT>::one(xr0 + threadIdx.x);
            ts = tm == kNegInf ? 0.0 : 1.0;
        }
        for (int64_t j0 = (int64_t)threadIdx.x * E; j0 < cb; j0 += (int64_t)NT * E) {
            float v[E];
            load_padded<XT, E, VEC>(xr, j0, cb, v);
            float cm = kNegInf;
#pragma unroll
            for (int i = 0; i < E; ++i)
                cm = fmaxf(cm, v[i]);
            const float M = fmaxf(tm, cm);
            if (M != kNegInf) {
                double s = ts * (double)exp2_f32((tm - M) * kLog2e);
#pragma unroll
                for (int i = 0; i < E; ++i)
                    s += (double)exp2_f32((v[i] - M) * kLog2e);
                tm = M;
                ts = s;
            }
        }
        const MS tot = block_reduce<SoftmaxMS, NT>(MS{tm, (float)ts}, slot[par]);
        par ^= 1;
        const float inv = 1.0f / tot.s;
        if (has_e)
            YOut<YT>::one(yr0 + threadIdx.x,
                          exp2_f32((XIn<XT>::one(xr0 + threadIdx.x) - tot.m) * kLog2e) * inv);
        for (int64_t j0 = (int64_t)threadIdx.x * E; j0 < cb; j0 += (int64_t)NT * E) {
            float v[E];
            load_padded<XT, E, VEC>(xr, j0, cb, v);
#pragma unroll
            for (int i = 0; i < E; ++i)
                v[i] = exp2_f32((v[i] - tot.m) * kLog2e) * inv;
            store_masked_rt<YT, E>(yr, j0, cb, v, yvec);
        }
    }
}

// -------------------------------------------------------------- wave tier
// S lanes per row, one chunk per lane (S * E >= cols).
template <class XT, class YT, bool VEC, int S>
__global__ __launch_bounds__(kBlockThreads) void k_softmax_wave(const XT* __restrict__ x,
                                                                YT* __restrict__ y, int64_t rows,
                                                                int64_t cols, int64_t ldx,
                                                                int64_t ldy)
{
    constexpr int E = VEC ? XIn<XT>::kChunk : 1;
    constexpr int RPG = kWave / S;
    constexpr int U = kWaveRowGroups;
    const int lane = lane_id();
    const int seg = lane / S;
    const int64_t j0 = (int64_t)(lane % S) * E;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
         w * RPG * U < rows; w += nwaves) {
        const int64_t row0 = w * RPG * U;
        float v[U][E];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t r = row0 + (int64_t)u * RPG + seg;
            if (r < rows) {
                load_padded<XT, E, VEC>(x + r * ldx, j0, cols, v[u]);
            } else {
#pragma unroll
                for (int i = 0; i < E; ++i)
                    v[u][i] = kNegInf;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const MS own = local_exp_sum<E>(v[u], [&](int i, float) { return j0 + i < cols; });
            const MS tot = segment_reduce<SoftmaxMS, S>(own);
            const float sc = exp2_f32((own.m - tot.m) * kLog2e) / tot.s;
#pragma unroll
            for (int i = 0; i < E; ++i)
                v[u][i] *= sc;
            const int64_t r = row0 + (int64_t)u * RPG + seg;
            if (r < rows)
                store_masked<YT, E, VEC>(y + r * ldy, j0, cols, v[u]);
        }
    }
}

// ---------------------------------------------- tiled and serial tiers
// Thread owns R adjacent rows and walks each row element by element:
// max, then sum of exp, then the map.  R == 1 is the serial tier.
template <class XT, class YT, int R>
__global__ __launch_bounds__(kBlockThreads) void k_softmax_tiled(const XT* __restrict__ x,
                                                                 YT* __restrict__ y,
                                                                 int64_t rows, int64_t cols,
                                                                 int64_t ldx, int64_t ldy)
{
    const int64_t nthreads = (int64_t)gridDim.x * kBlockThreads;
    for (int64_t tid = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; tid * R < rows;
         tid += nthreads) {
        for (int k = 0; k < R; ++k) {
            const int64_t r = tid * R + k;
            if (r >= rows)
                break;
            const XT* xr = x + r * ldx;
            YT* yr = y + r * ldy;
            float m = kNegInf;
            for (int64_t j = 0; j < cols; ++j)
                m = fmaxf(m, XIn<XT>::one(xr + j));
            // one thread adds every term of the row in sequence: accumulate
            // in double so the sum stays accurate for long rows
            double s = 0.0;
            if (m != kNegInf)
                for (int64_t j = 0; j < cols; ++j)
                    s += (double)exp2_f32((XIn<XT>::one(xr + j) - m) * kLog2e);
            const float inv = (float)(1.0 / s);
            for (int64_t j = 0; j < cols; ++j)
                YOut<YT>::one(yr + j, exp2_f32((XIn<XT>::one(xr + j) - m) * kLog2e) * inv);
        }
    }
}

// ----------------------------------------------------------- split-K tier
// For fewer rows than compute units, with long rows: G workgroups per row
// ("reduce", tier semantics), each owning tiles g, g + G, ... of the row.
// Two launches on one stream:
//   statistics: workgroup (r, g) folds (max, sum) over its tiles and stores
//     the pair to part[r * G + g];
//   map: every workgroup of row r reads the row's G pairs and folds them in
//     rank order into (M, S) -- the same inputs in the same order, so every
//     workgroup of the row holds the same bits ("cluster_allreduce",
//     description: the all-gather variant, where every block needs the
//     result) -- then writes exp(x - M) / S over its tiles.
// The kernel boundary makes the statistics pass's stores visible to the map
// pass; no atomics and no counters are needed.  A tile is
// kSoftmaxSplitKUnroll 16-byte chunks per thread.

// Exponentials of a thread's map arguments t: the hardware instruction when
// every t >= -126 (exact there), else exp2_sub (subnormal results).
template <int N>
__device__ __forceinline__ void exp2_values(float* t)
{
    float tmin = 0.0f;
#pragma unroll
    for (int i = 0; i < N; ++i)
        tmin = fminf(tmin, t[i]);
    if (tmin >= -126.0f) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            t[i] = exp2_hw(t[i]);
    } else {
        keep_branch();
#pragma unroll
        for (int i = 0; i < N; ++i)
            t[i] = exp2_sub(t[i]);
    }
}

// Fold one tile's N values into the thread's running (tm, ts): exponentials
// relative to the new running maximum, summed pairwise in float (N is a
// power of two), added to the running sum in double.  The hardware
// exponential is used without a range check: the running sum always holds
// the 1 of its own maximum, so a term it flushes (below 2^-126) lies far
// below the double's resolution there and the sum comes out the same.
template <int N>
__device__ __forceinline__ void stats_fold_tile(float* v, float& tm, double& ts)
{
    static_assert((N & (N - 1)) == 0, "pairwise sum over a power of two");
    float cm = kNegInf;
#pragma unroll
    for (int i = 0; i < N; ++i)
        cm = fmaxf(cm, v[i]);
    const float M = fmaxf(tm, cm);
    if (M == kNegInf)
        return;
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] = exp2_hw((v[i] - M) * kLog2e);
#pragma unroll
    for (int w = N / 2; w >= 1; w /= 2)
#pragma unroll
        for (int i = 0; i < w; ++i)
            v[i] += v[i + w];
    ts = ts * (double)exp2_f32((tm - M) * kLog2e) + (double)v[0];
    tm = M;
}

template <int N, class R>
__device__ __forceinline__ void stats_fold_raw(const R& raw, float& tm, double& ts)
{
    float v[N];
    raw.unpack(v);
    stats_fold_tile<N>(v, tm, ts);
}

template <class XT, bool VEC>
__global__ __launch_bounds__(kBlockThreads) void k_softmax_splitk_stats(
    const XT* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, int32_t G,
    uint64_t* __restrict__ part)
{
    constexpr int E = VEC ? XIn<XT>::kChunk : 1;
    constexpr int U = kSoftmaxSplitKUnroll;
    constexpr int N = U * E;
    constexpr int64_t kTile = (int64_t)N * kBlockThreads;
    __shared__ MS slot[2][kWavesPerBlock];
    int par = 0;
    const int64_t total = rows * G;
    for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
        const int64_t r = b / G;
        const int32_t g = (int32_t)(b - r * G);
        // Tiles cover the row's body from its first 16-byte boundary (VEC);
        // workgroup 0 also takes the head, h < E elements, one element to
        // each of its first threads.
        const XT* xr0 = x + r * ldx;
        const int64_t h = VEC ? head_elems(xr0, cols) : 0;
        const XT* xr = xr0 + h;
        const int64_t cb = cols - h;
        const int64_t ntiles = ceil_div(cb, kTile);
        const int64_t nfull = cb / kTile;
        float tm = kNegInf;
        double ts = 0.0;
        if (VEC && g == 0 && (int64_t)threadIdx.x < h) {
            tm = XIn<XT>::one(xr0 + threadIdx.x);
            ts = tm == kNegInf ? 0.0 : 1.0;
        }
        // Whole tiles g, g + G, ...: n of them.  Two register buffers; the
        // next tile's loads are issued before the current one is folded.
        // Trip counts are uniform over the workgroup (scalar branches).
        const int64_t n = g < nfull ? (nfull - 1 - g) / G + 1 : 0;
        if (n > 0) {
            const int64_t step = (int64_t)G * kTile;
            const XT* tp = xr + (int64_t)g * kTile;
            RawTile<XT, VEC, U> A, B;
            A.load(tp);
            int64_t k = 0;
            // sched_barrier: keep the folds' first uses of the older buffer
            // below the younger loads, so those are issued without waiting
            for (; k + 2 < n; k += 2) {
                B.load(tp + (k + 1) * step);
                __builtin_amdgcn_sched_barrier(0);
                stats_fold_raw<N>(A, tm, ts);
                A.load(tp + (k + 2) * step);
                __builtin_amdgcn_sched_barrier(0);
                stats_fold_raw<N>(B, tm, ts);
            }
            if (k + 1 < n) {
                B.load(tp + (k + 1) * step);
                __builtin_amdgcn_sched_barrier(0);
                stats_fold_raw<N>(A, tm, ts);
                stats_fold_raw<N>(B, tm, ts);
            } else {
                stats_fold_raw<N>(A, tm, ts);
            }
        }
        for (int64_t t = g + n * G; t < ntiles; t += G) {  // ragged last tile, -inf padded
            float v[N];
            load_tile_padded<XT, E, VEC, U>(xr, t * kTile, cb, v);
            stats_fold_tile<N>(v, tm, ts);
        }
        float e_t;
        const MS tot = block_softmax_stats<kBlockThreads>(MS{tm, (float)ts}, slot[par], &e_t);
        par ^= 1;
        if (threadIdx.x == 0)
            part[r * G + g] = pack_ms(tot);
    }
}

// y = exp(x - M) / S on the tile's values, in place.
template <int N>
__device__ __forceinline__ void map_tile(float* v, float M, float inv)
{
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] = (v[i] - M) * kLog2e;
    exp2_values<N>(v);
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] *= inv;
}

// Row statistics from the row's G pairs (p: this thread's pair, the
// identity for threads >= G), in rank order: M = max over g of m_g (exact,
// so the order does not matter), then S = sum over g of s_g * exp(m_g - M),
// the G terms taken in parallel and added in double over a fixed tree whose
// leaves are the ranks in order.  Every workgroup computing it from the same
// pairs gets the same bits.
__device__ __forceinline__ MS fold_row_partials(MS p, float* fslot, double* dslot)
{
    const float M = block_reduce<MaxFloat, kBlockThreads>(p.m, fslot);
    const double w = p.m == kNegInf ? 0.0 : (double)p.s * (double)exp2_f32((p.m - M) * kLog2e);
    const double S = block_reduce<SumF32, kBlockThreads>(w, dslot);
    return MS{M, (float)S};
}

template <class XT, class YT, bool VEC>
__global__ __launch_bounds__(kBlockThreads) void k_softmax_splitk_map(
    const XT* __restrict__ x, YT* __restrict__ y, int64_t rows, int64_t cols, int64_t ldx,
    int64_t ldy, int32_t G, const uint64_t* __restrict__ part)
{
    constexpr int E = VEC ? XIn<XT>::kChunk : 1;
    constexpr int U = kSoftmaxSplitKUnroll;
    constexpr int64_t kTile = (int64_t)U * kBlockThreads * E;
    static_assert(kSplitKMaxSlices <= kBlockThreads, "one pair per thread in the row fold");
    __shared__ float fslot[kWavesPerBlock];
    __shared__ double dslot[kWavesPerBlock];
    const int64_t total = rows * G;
    for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
        const int64_t r = b / G;
        const int32_t g = (int32_t)(b - r * G);
        // the statistics pass's tiles (from the row's first 16-byte
        // boundary); y's chunks are stored whole when y + h is aligned
        const XT* xr0 = x + r * ldx;
        YT* yr0 = y + r * ldy;
        const int64_t h = VEC ? head_elems(xr0, cols) : 0;
        const XT* xr = xr0 + h;
        YT* yr = yr0 + h;
        const int64_t cb = cols - h;
        const int64_t ntiles = ceil_div(cb, kTile);
        const int64_t nfull = cb / kTile;
        const bool yvec = VEC && chunk_aligned<YT, E>(yr);
        // the row's pairs first, then the first tile: the fold waits only
        // for the pairs while the tile is in flight
        MS p = MS{kNegInf, 0.0f};
        if ((int32_t)threadIdx.x < G)
            p = unpack_ms(part[r * G + threadIdx.x]);
        int64_t t = g;
        float v[U * E];
        if (t < nfull)
            load_tile_full<XT, E, VEC, U>(xr + t * kTile, v);
        const MS st = fold_row_partials(p, fslot, dslot);
        const float inv = 1.0f / st.s;
        if (VEC && g == 0 && (int64_t)threadIdx.x < h)
            YOut<YT>::one(yr0 + threadIdx.x,
                          exp2_f32((XIn<XT>::one(xr0 + threadIdx.x) - st.m) * kLog2e) * inv);
        for (; t < nfull; t += G) {
            map_tile<U * E>(v, st.m, inv);
            if (!VEC || yvec)
                store_tile_full<YT, E, VEC, U>(yr + t * kTile, v);
            else
                store_tile_full_rt<YT, E, U>(yr + t * kTile, v, false);
            if (t + G < nfull)
                load_tile_full<XT, E, VEC, U>(xr + (t + G) * kTile, v);
        }
        for (; t < ntiles; t += G) {
            load_tile_padded<XT, E, VEC, U>(xr, t * kTile, cb, v);
            map_tile<U * E>(v, st.m, inv);
            if (!VEC)
                store_tile_masked<YT, E, VEC, U>(yr, t * kTile, cb, v);
            else
                store_tile_masked_rt<YT, E, U>(yr, t * kTile, cb, v, yvec);
        }
        __syncthreads();  // the fold's LDS slots are reused by the next row
    }
}

template <class XT, class YT, bool VEC>
static rr_status launch_splitk(const rr_plan& p, const SoftmaxLaunch& a)
{
    const XT* x = static_cast<const XT*>(a.x);
    YT* y = static_cast<YT*>(a.y);
    uint64_t* part = static_cast<uint64_t*>(a.workspace);
    const dim3 grid((unsigned)(p.grid > kMaxGrid ? kMaxGrid : p.grid)), block(kBlockThreads);
    rr_status st = launch_kernel(k_softmax_splitk_stats<XT, VEC>, grid, block, 0, a.stream, x,
                                 a.rows, a.cols, a.ld_x, p.slices, part);
    if (st != RR_OK)
        return st;
    return launch_kernel(k_softmax_splitk_map<XT, YT, VEC>, grid, block, 0, a.stream, x, y, a.rows,
                         a.cols, a.ld_x, a.ld_y, p.slices, (const uint64_t*)part);
}

// ---------------------------------------------------------------- launch
// Persistent rows: the plan's grid, lowered to the workgroups that can be
// resident at once (occupancy times CUs), so no workgroup of the persistent
// grid waits for another to finish before it starts.
template <class XT, class YT, int NCH, int NT>
static rr_status launch_pf(const XT* x, YT* y, const rr_plan& p, const SoftmaxLaunch& a)
{
    constexpr int E = XIn<XT>::kChunk;
    constexpr int64_t kExactCols = (int64_t)NT * NCH * E;
    // rows that start 16-byte aligned and end on a chunk need no head or tail;
    // those that also all start on a 128-byte line need no rotation
    const bool whole = a.rows16 && a.cols % E == 0;
    const bool lines = (uintptr_t)a.x % 128 == 0 && (a.ld_x * (int64_t)sizeof(XT)) % 128 == 0;
    const bool exact = a.cols == kExactCols;
    auto kernel = !whole ? k_softmax_rows_pf<XT, YT, NCH, NT, false, true, true>
                  : lines ? (exact ? k_softmax_rows_pf<XT, YT, NCH, NT, true, false, false>
                                   : k_softmax_rows_pf<XT, YT, NCH, NT, false, false, false>)
                          : (exact ? k_softmax_rows_pf<XT, YT, NCH, NT, true, false, true>
                                   : k_softmax_rows_pf<XT, YT, NCH, NT, false, false, true>);
    int per_cu = 0;
    if (blocks_per_cu(kernel, NT, &per_cu) != RR_OK)
        return RR_ERR_HIP;
    const int64_t cap = (int64_t)per_cu * a.cu;
    const dim3 grid((unsigned)(p.grid < cap ? p.grid : cap));
    return launch_kernel(kernel, grid, dim3(NT), 0, a.stream, x, y, a.rows, a.cols, a.ld_x,
                         a.ld_y);
}

// Block tier, one row per workgroup: the row stays in registers when each of
// the NT threads holds at most kSoftmaxMaxChunks chunks; longer rows stream
// twice.
template <class XT, class YT, bool VEC, int NT>
static rr_status launch_block(const rr_plan& p, const SoftmaxLaunch& a)
{
    const XT* x = static_cast<const XT*>(a.x);
    YT* y = static_cast<YT*>(a.y);
    const dim3 grid((unsigned)p.grid), block(NT);
    const hipStream_t s = a.stream;
    constexpr int E = VEC ? XIn<XT>::kChunk : 1;
    const int64_t nch = ceil_div(ceil_div(a.cols, E), NT);
    if (nch <= 1)
        return launch_kernel(k_softmax_block<XT, YT, 1, VEC, NT>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld_x, a.ld_y);
    if (nch <= 2)
        return launch_kernel(k_softmax_block<XT, YT, 2, VEC, NT>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld_x, a.ld_y);
    if (nch <= 4)
        return launch_kernel(k_softmax_block<XT, YT, 4, VEC, NT>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld_x, a.ld_y);
    if (nch <= kSoftmaxMaxChunks)
        return launch_kernel(k_softmax_block<XT, YT, kSoftmaxMaxChunks, VEC, NT>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld_x, a.ld_y);
    return launch_kernel(k_softmax_stream<XT, YT, VEC, NT>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld_x, a.ld_y);
}

// Block tier: persistent rows when the plan chose them, else one row per
// workgroup.
template <class XT, class YT, bool VEC>
static rr_status launch_block_tier(const rr_plan& p, const SoftmaxLaunch& a)
{
    if constexpr (VEC) {
        constexpr int E = XIn<XT>::kChunk;
        {
            const RowPfShape sh = row_pf_shape(ceil_div(a.cols, E));
            if (sh.nt > 0) {
                if (sh.nt != p.block)
                    return RR_ERR_TIER;  // plan and launch disagree: refuse, launch nothing
                const XT* x = static_cast<const XT*>(a.x);
                YT* y = static_cast<YT*>(a.y);
                switch (sh.nt * 16 + sh.nch) {
                case 64 * 16 + 1: return launch_pf<XT, YT, 1, 64>(x, y, p, a);
                case 64 * 16 + 2: return launch_pf<XT, YT, 2, 64>(x, y, p, a);
                case 64 * 16 + 4: return launch_pf<XT, YT, 4, 64>(x, y, p, a);
                case 128 * 16 + 4: return launch_pf<XT, YT, 4, 128>(x, y, p, a);
                case 256 * 16 + 4: return launch_pf<XT, YT, 4, 256>(x, y, p, a);
                case 512 * 16 + 4: return launch_pf<XT, YT, 4, 512>(x, y, p, a);
                default: return RR_ERR_TIER;
                }
            }
        }
    }
    return p.block == kSoftmaxWideThreads ? launch_block<XT, YT, VEC, kSoftmaxWideThreads>(p, a)
                                          : launch_block<XT, YT, VEC, kBlockThreads>(p, a);
}

template <class XT, class YT, bool VEC>
static rr_status launch_wave(const rr_plan& p, const SoftmaxLaunch& a)
{
    const XT* x = static_cast<const XT*>(a.x);
    YT* y = static_cast<YT*>(a.y);
    const dim3 grid((unsigned)p.grid), block(kBlockThreads);
    const hipStream_t s = a.stream;
    switch (p.lanes_per_row) {
    case 4: return launch_kernel(k_softmax_wave<XT, YT, VEC, 4>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld_x, a.ld_y);
    case 16: return launch_kernel(k_softmax_wave<XT, YT, VEC, 16>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld_x, a.ld_y);
    case 64: return launch_kernel(k_softmax_wave<XT, YT, VEC, 64>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld_x, a.ld_y);
    default: return RR_ERR_TIER;
    }
}

// VEC (element-aligned x and y): the block and split-K tiers; the wave tier
// takes 128-bit chunks only when every row is 16-byte aligned (rows16).
template <class XT, class YT, bool VEC>
static rr_status launch_typed(const rr_plan& p, const SoftmaxLaunch& a)
{
    const XT* x = static_cast<const XT*>(a.x);
    YT* y = static_cast<YT*>(a.y);
    const dim3 grid((unsigned)p.grid), block(kBlockThreads);
    const hipStream_t s = a.stream;
    switch (p.tier) {
    case RR_TIER_BLOCK:
        return launch_block_tier<XT, YT, VEC>(p, a);
    case RR_TIER_WAVE:
        return VEC && a.rows16 ? launch_wave<XT, YT, true>(p, a) : launch_wave<XT, YT, false>(p, a);
    case RR_TIER_SPLITK:
        return launch_splitk<XT, YT, VEC>(p, a);
    case RR_TIER_TILED:
        return launch_kernel(k_softmax_tiled<XT, YT, kTiledRows>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld_x, a.ld_y);
    case RR_TIER_SERIAL:
        return launch_kernel(k_softmax_tiled<XT, YT, 1>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld_x, a.ld_y);
    default:
        return RR_ERR_TIER;
    }
}

template <class XT, class YT>
static rr_status launch_xy(const rr_plan& p, const SoftmaxLaunch& a)
{
    return a.vec ? launch_typed<XT, YT, true>(p, a) : launch_typed<XT, YT, false>(p, a);
}

rr_status launch_softmax(const rr_plan& p, const SoftmaxLaunch& a)
{
    const bool xb = a.x_dtype == RR_BF16, yb = a.y_dtype == RR_BF16;
    if (xb && yb) return launch_xy<uint16_t, uint16_t>(p, a);
    if (xb) return launch_xy<uint16_t, float>(p, a);
    if (yb) return launch_xy<float, uint16_t>(p, a);
    return launch_xy<float, float>(p, a);
}

}  // namespace rr
