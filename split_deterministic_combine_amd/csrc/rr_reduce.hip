// rr_reduce.hip -- row reductions over the last axis, five tiers, gfx950.
//
// Tier shapes follow "reduce" (algorithm.gpu.rowwise), tier semantics:
//   wave    a group of lanes of one wavefront owns a short row (cols <= 64);
//   block   one workgroup strides along a row with 128-bit loads, scalar tail;
//   tiled   one thread owns kTiledRows adjacent rows, no cross-thread combine;
//   serial  one thread per row, element by element;
//   split-K several workgroups per row; the cross-workgroup combine follows
//           "cluster_allreduce" (description): each group reduces inside
//           itself first, then the groups' values are folded in rank order,
//           so the bits do not depend on which group finishes first.
// The monoids (sum / max / min on 32-bit values) are the page's combine_fn.
#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>

#include "rr_config.hpp"
#include "rr_device.hpp"
#include "rr_launch.hpp"
#include "rr_launch_util.hpp"

namespace rr {

// Fold row[begin, end) into acc, thread t of NT.  With VEC == 4 the thread
// visits 128-bit chunks t, t+NT, t+2NT, ... (U chunks in flight), then the
// scalar tail; begin must then be a multiple of 4 elements from a 16-byte
// aligned row start.  Elements are folded in ascending index order per
// thread.
template <class M, int VEC, int NT, int U>
__device__ __forceinline__ typename M::acc_t thread_fold(const typename M::in_t* __restrict__ row,
                                                         int64_t begin, int64_t end, int t,
                                                         typename M::acc_t acc)
{
    using T = typename M::in_t;
    const T* base = row + begin;
    const int64_t n = end - begin;
    if constexpr (VEC == 4) {
        const int64_t nchunks = n >> 2;
        int64_t c = t;
        for (; c + (int64_t)(U - 1) * NT < nchunks; c += (int64_t)U * NT) {
            Vec<T, 4> v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = load4<T, true>(base + (c + (int64_t)u * NT) * 4);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc = M::combine(acc, M::lift(v[u].v[i]));
        }
        for (; c < nchunks; c += NT) {
            Vec<T, 4> v = load4<T, true>(base + c * 4);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc = M::combine(acc, M::lift(v.v[i]));
        }
        for (int64_t j = nchunks * 4 + t; j < n; j += NT)
            acc = M::combine(acc, M::lift(base[j]));
    } else {
        int64_t j = t;
        for (; j + (int64_t)(U - 1) * NT < n; j += (int64_t)U * NT) {
            T v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = base[j + (int64_t)u * NT];
#pragma unroll
            for (int u = 0; u < U; ++u)
                acc = M::combine(acc, M::lift(v[u]));
        }
        for (; j < n; j += NT)
            acc = M::combine(acc, M::lift(base[j]));
    }
    return acc;
}

// ------------------------------------------------------------ block tier
// VEC == 4: each row's body from its first 16-byte boundary goes in 128-bit
// loads; its head (h <= 3 elements before that boundary) and its tail (at
// most 3 elements after the last whole chunk) one element to each of the
// first h + tl threads, loaded before the body so that every load of the row
// is in flight at once.
// VEC == 4 and not PEEL: every row starts 16-byte aligned (only the tail
// chunk of a row goes element by element, after the body).
template <class M, int VEC, bool PEEL>
__global__ __launch_bounds__(kBlockThreads) void k_reduce_block(
    const typename M::in_t* __restrict__ x, typename M::out_t y, int64_t rows,
    int64_t cols, int64_t ld)
{
    using A = typename M::acc_t;
    __shared__ A slot[2][kWavesPerBlock];
    int par = 0;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const typename M::in_t* row = x + r * ld;
        A acc;
        if constexpr (VEC == 4 && !PEEL) {
            acc = thread_fold<M, 4, kBlockThreads, kBlockUnroll>(row, 0, cols, threadIdx.x,
                                                                  M::identity());
        } else if constexpr (VEC == 4) {
            const int64_t h = head_elems(row, cols);
            const int64_t nbe = (cols - h) & ~(int64_t)3;
            const int64_t t = threadIdx.x;
            const int64_t e = t < h ? t : t < cols - nbe ? nbe + t : -1;  // extra's column
            const typename M::in_t xe = row[e >= 0 ? e : 0];
            acc = thread_fold<M, 4, kBlockThreads, kBlockUnroll>(row + h, 0, nbe, threadIdx.x,
                                                                  M::identity());
            if (e >= 0)
                acc = M::combine(acc, M::lift(xe));
        } else {
            acc = thread_fold<M, 1, kBlockThreads, kBlockUnroll>(row, 0, cols, threadIdx.x,
                                                                 M::identity());
        }
        acc = block_reduce<M, kBlockThreads>(acc, slot[par]);
        par ^= 1;
        if (threadIdx.x == 0)
            M::store(y, r, acc);
    }
}

// ------------------------------------------------------------- wave tier
// S lanes per row (S >= ceil(cols / VEC)); 64 / S rows per group and
// kWaveRowGroups groups per wavefront task.  VEC == 4 (rows of at least 7
// elements, so every row has a whole chunk): a row's body starts at its
// first 16-byte boundary, h = 0..3 elements in; lane l < nb (nb = whole body
// chunks) owns columns [h + 4l, h + 4l + 4), and the head and the tail
// (h + tl <= 6 elements) go one element to lanes 0, 1, ... (NX per lane).
// VEC == 1: lane l owns column l.  (Fewer lanes per row with several chunks
// each -- a shorter cross-lane combine -- measured slower: 38.5 against
// 32.5 us for f32 sums of [1048576, 48].)  All loads of a task are issued
// before any is folded, at clamped addresses that stay inside the row (rows
// past the end read the last row, lanes without a chunk or an element the
// first ones; those values are masked off), so the wavefront has all of them
// in flight without branches between.
// PEEL false: every row starts 16-byte aligned and is whole chunks (no head
// or tail elements).
template <class M, int VEC, int S, bool PEEL>
__global__ __launch_bounds__(kBlockThreads) void k_reduce_wave(
    const typename M::in_t* __restrict__ x, typename M::out_t y, int64_t rows,
    int64_t cols, int64_t ld)
{
    using T = typename M::in_t;
    using A = typename M::acc_t;
    constexpr int RPG = kWave / S;
    constexpr int U = kWaveRowGroups;
    constexpr int NX = VEC == 4 && PEEL ? (6 + S - 1) / S : 0;  // head / tail elements per lane
    const int lane = lane_id();
    const int seg = lane / S;
    const int li = lane % S;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
         w * RPG * U < rows; w += nwaves) {
        const int64_t row0 = w * RPG * U;
        Vec<T, VEC> v[U];
        T xe[U][NX > 0 ? NX : 1];
        bool full[U], has[U][NX > 0 ? NX : 1];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t r = row0 + (int64_t)u * RPG + seg;
            r = r < rows ? r : rows - 1;
            const T* rp = x + r * ld;
            if constexpr (VEC == 4) {
                // 32-bit column arithmetic: a wave-tier row has at most 64 columns
                const int c = (int)cols;
                const int h = PEEL ? (int)head_elems(rp, cols) : 0;
                const int nbe = (c - h) & ~3;
                full[u] = li * 4 < nbe;
                v[u] = load4<T, true>(rp + h + (full[u] ? li * 4 : 0));
#pragma unroll
                for (int k = 0; k < NX; ++k) {
                    // head or tail element ex of h + tl = cols - nbe: column ex
                    // of the head, or nbe + ex (= h + nbe + (ex - h)) of the tail
                    const int ex = li + k * S;
                    has[u][k] = ex < c - nbe;
                    xe[u][k] = rp[has[u][k] ? (ex < h ? ex : nbe + ex) : 0];
                }
            } else {
                full[u] = li < cols;
                v[u].v[0] = rp[full[u] ? li : 0];
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // every load of the task goes out before any fold
        A acc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            acc[u] = M::identity();
#pragma unroll
            for (int i = 0; i < VEC; ++i)
                acc[u] = full[u] ? M::combine(acc[u], M::lift(v[u].v[i])) : acc[u];
#pragma unroll
            for (int k = 0; k < NX; ++k)
                acc[u] = has[u][k] ? M::combine(acc[u], M::lift(xe[u][k])) : acc[u];
        }
        // Every lane of a segment holds the row's result after the combine,
        // so all of them store it (the same bits to one address), and rows
        // past the end store their clamped row's result -- the last row's,
        // computed the same way -- to that row.  No store is predicated: a
        // predicated store between two groups makes the memory-counter wait
        // before the next group's fold also hold for a load it does not need.
#pragma unroll
        for (int u = 0; u < U; ++u) {
            A t = segment_reduce<M, S>(acc[u]);
            const int64_t r = row0 + (int64_t)u * RPG + seg;
            M::store(y, r < rows ? r : rows - 1, t);
        }
    }
}

// ------------------------------------------------- tiled and serial tiers
// Thread owns R adjacent rows; each axis step loads the step's element (or
// 128-bit chunk) of all R rows and folds each into its own state.  R == 1 is
// the serial tier.  No cross-thread combine.  Rows past the end are clamped
// to the last row (loads stay in bounds, results are not stored).
template <class M, int VEC, int R>
__global__ __launch_bounds__(kBlockThreads) void k_reduce_tiled(
    const typename M::in_t* __restrict__ x, typename M::out_t y, int64_t rows,
    int64_t cols, int64_t ld)
{
    using T = typename M::in_t;
    using A = typename M::acc_t;
    const int64_t nthreads = (int64_t)gridDim.x * kBlockThreads;
    for (int64_t tid = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; tid * R < rows;
         tid += nthreads) {
        const int64_t r0 = tid * R;
        const T* rp[R];
        A acc[R];
#pragma unroll
        for (int k = 0; k < R; ++k) {
            rp[k] = x + (r0 + k < rows ? r0 + k : rows - 1) * ld;
            acc[k] = M::identity();
        }
        const int64_t nfull = VEC == 4 ? (cols >> 2) : 0;
        for (int64_t c = 0; c < nfull; ++c) {
            Vec<T, 4> v[R];
#pragma unroll
            for (int k = 0; k < R; ++k)
                v[k] = load4(rp[k] + c * 4);
#pragma unroll
            for (int k = 0; k < R; ++k)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[k] = M::combine(acc[k], M::lift(v[k].v[i]));
        }
        for (int64_t j = nfull * 4; j < cols; ++j) {
            T v[R];
#pragma unroll
            for (int k = 0; k < R; ++k)
                v[k] = rp[k][j];
#pragma unroll
            for (int k = 0; k < R; ++k)
                acc[k] = M::combine(acc[k], M::lift(v[k]));
        }
#pragma unroll
        for (int k = 0; k < R; ++k)
            if (r0 + k < rows)
                M::store(y, r0 + k, acc[k]);
    }
}

// One unrolled load round of a thread: chunks p, p + NT*VEC, ... (U of them).
template <int VEC, int NT, int U, class T>
__device__ __forceinline__ void load_tile(const T* p, Vec<T, VEC>* v)
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if constexpr (VEC == 4) {
            v[u] = load4<T, true>(p + (int64_t)u * NT * 4);
        } else {
            v[u].v[0] = p[(int64_t)u * NT];
        }
    }
}

// Fold a load round in ascending index order.
template <class M, int VEC, int U>
__device__ __forceinline__ typename M::acc_t fold_tile(typename M::acc_t acc,
                                                       const Vec<typename M::in_t, VEC>* v)
{
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < VEC; ++i)
            acc = M::combine(acc, M::lift(v[u].v[i]));
    return acc;
}

// ----------------------------------------------------------- split-K tier
// A row is cut into tiles of kSplitKUnroll * kBlockThreads * VEC columns
// (one unrolled load round of the workgroup); workgroup (r, g) folds the
// contiguous run of tiles [g * T / G, (g + 1) * T / G) of row r (T tiles in
// the row, the ragged last one included), in ascending order.  One long
// sequential stream per workgroup reads faster on MI355X than tiles dealt
// round-robin (measured on a 1 GiB read at 2 workgroups per CU: 88% against
// 84% of peak).  It then publishes its partial to part[r * G + g]
// and takes a ticket on row r.  The workgroup that draws ticket G - 1 is the
// last to arrive: it folds part[r * G + 0 .. G - 1] in ascending g, writes
// y[r] and resets the ticket and the row's partial slots to zero for the
// next call.  `skew` (a test hook, normally 0) makes
// workgroup g wait about (G - 1 - g) * skew sleep periods before publishing,
// so arrival order runs against rank order.
template <class M, int VEC>
__global__ __launch_bounds__(kBlockThreads) void k_reduce_splitk(
    const typename M::in_t* __restrict__ x, typename M::out_t y, int64_t rows,
    int64_t cols, int64_t ld, int32_t G, typename M::acc_t* part, uint32_t* ticket, int32_t skew)
{
    using A = typename M::acc_t;
    constexpr int64_t kTile = (int64_t)kSplitKUnroll * kBlockThreads * VEC;
    static_assert(kSplitKMaxSlices <= kBlockThreads, "one partial per thread when gathering");
    __shared__ A slot[2][kWavesPerBlock];
    __shared__ A gathered[kSplitKMaxSlices];
    __shared__ bool last;
    int par = 0;
    if (threadIdx.x == 0)
        last = false;
    const int64_t total = rows * G;
    for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
        const int64_t r = b / G;
        const int32_t g = (int32_t)(b - r * G);
        // Tiles cover the row's body from its first 16-byte boundary (h
        // elements in, VEC == 4); workgroup 0 also folds the head [0, h),
        // one element to each of its first threads.
        const typename M::in_t* row0 = x + r * ld;
        const int64_t h = VEC == 4 ? head_elems(row0, cols) : 0;
        const typename M::in_t* row = row0 + h;
        const int64_t body = cols - h;
        const int64_t ntiles = ceil_div(body, kTile);
        A acc = M::identity();
        if (VEC == 4 && g == 0 && (int64_t)threadIdx.x < h)
            acc = M::lift(row0[threadIdx.x]);
        // Whole tiles: each round issues the thread's kSplitKUnroll loads of
        // one tile, then folds them.  Tile indices are uniform across the
        // workgroup, so the loop branch is scalar.
        const int64_t nfull = body / kTile;
        const int64_t t_end = (int64_t)(g + 1) * ntiles / G;
        const int64_t t_full = t_end < nfull ? t_end : nfull;
        int64_t t = (int64_t)g * ntiles / G;
        {
            using T = typename M::in_t;
            const T* p = row + (int64_t)threadIdx.x * VEC;
            for (; t < t_full; ++t) {
                Vec<T, VEC> v[kSplitKUnroll];
                load_tile<VEC, kBlockThreads, kSplitKUnroll>(p + t * kTile, v);
                acc = fold_tile<M, VEC, kSplitKUnroll>(acc, v);
            }
        }
        // The partial last tile, if this workgroup owns it.
        for (; t < t_end; ++t) {
            const int64_t begin = t * kTile;
            const int64_t end = begin + kTile < body ? begin + kTile : body;
            acc = thread_fold<M, VEC, kBlockThreads, kSplitKUnroll>(row, begin, end, threadIdx.x, acc);
        }
        acc = block_reduce<M, kBlockThreads>(acc, slot[par]);
        par ^= 1;
        if (threadIdx.x == 0) {
            if (skew > 0) {
                const int n = (G - 1 - g) * skew;
                for (int i = 0; i < n; ++i)
                    __builtin_amdgcn_s_sleep(8);
            }
            publish_partial(&part[r * G + g], acc);
            const uint32_t t = __hip_atomic_fetch_add(&ticket[r], 1u, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
            last = t == (uint32_t)(G - 1);
        }
        __syncthreads();
        if (last) {
            // The whole workgroup gathers the G partials at once (G <= the
            // block size), then thread 0 folds them in ascending rank order.
            // Each slot is cleared once read, so a completed call leaves
            // every workspace byte it used zero: a later call with more rows
            // keeps its tickets where this one kept partials.
            for (int32_t k = threadIdx.x; k < G; k += kBlockThreads) {
                gathered[k] = read_partial(&part[r * G + k]);
                clear_partial(&part[r * G + k]);
            }
            __syncthreads();
            if (threadIdx.x == 0) {
                A a = gathered[0];
                for (int32_t k = 1; k < G; ++k)
                    a = M::combine(a, gathered[k]);
                M::store(y, r, a);
                last = false;
                __hip_atomic_store(&ticket[r], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------- small utilities
__global__ __launch_bounds__(kBlockThreads) void k_fill_u32(uint32_t* __restrict__ p, int64_t n,
                                                             uint32_t v)
{
    for (int64_t i = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kBlockThreads)
        p[i] = v;
}

__global__ __launch_bounds__(kBlockThreads) void k_fill_zero_bytes(uint8_t* __restrict__ p,
                                                                    int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kBlockThreads)
        p[i] = 0;
}

static unsigned grid_for(int64_t n)
{
    int64_t g = ceil_div(n, kBlockThreads);
    if (g > 4096) g = 4096;
    return (unsigned)(g < 1 ? 1 : g);
}

rr_status launch_fill_zero(void* p, size_t bytes, hipStream_t stream)
{
    if (bytes == 0) return RR_OK;
    return launch_kernel(k_fill_zero_bytes, dim3(grid_for((int64_t)bytes)), dim3(kBlockThreads),
                         0, stream, (uint8_t*)p, (int64_t)bytes);
}

// ------------------------------------------------ library-owned scratch
// The split-K workspace of rr_reduce_rows_noalloc, for callers that cannot
// allocate: a file-scope device array, one copy per GPU, held until the
// process ends.  On the host the name `scratch` only stands for the symbol;
// the device address of the current GPU's copy comes from
// hipGetSymbolAddress, looked up once per device with that device current and
// kept per device, and only that address is ever passed to a kernel or a
// fill.
static __device__ __align__(256) uint8_t scratch[RR_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch[kScratchDevices];
}  // namespace

rr_status noalloc_scratch(void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices)
        return RR_ERR_HIP;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return RR_ERR_HIP;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return RR_OK;
}

// ---------------------------------------------------------------- launch
// The output argument of monoid M's kernels.
template <class M>
static typename M::out_t outputs_of(const ReduceLaunch& a)
{
    using O = typename M::out_t;
    if constexpr (std::is_pointer<O>::value) {
        return static_cast<O>(a.y);
    } else {
        using T = typename M::in_t;
        return O{static_cast<T*>(a.ys[0]), static_cast<T*>(a.ys[1]), static_cast<T*>(a.ys[2])};
    }
}

template <class M>
static rr_status launch_monoid(const rr_plan& p, const ReduceLaunch& a)
{
    using T = typename M::in_t;
    using A = typename M::acc_t;
    const T* x = static_cast<const T*>(a.x);
    const typename M::out_t y = outputs_of<M>(a);
    const dim3 grid((unsigned)p.grid), block(kBlockThreads);
    const hipStream_t s = a.stream;
    switch (p.tier) {
    case RR_TIER_BLOCK:
        return !a.vec ? launch_kernel(k_reduce_block<M, 1, false>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld)
               : a.rows16 ? launch_kernel(k_reduce_block<M, 4, false>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld)
                          : launch_kernel(k_reduce_block<M, 4, true>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld);
    case RR_TIER_WAVE: {
        // 128-bit chunks for rows of at least 7 elements (as the plan's
        // lanes); head and tail elements unless every row is aligned whole chunks
        const bool v4 = a.vec && a.cols >= 7;
        const bool peel = !(a.rows16 && a.cols % 4 == 0);
        switch (p.lanes_per_row) {
        case 4:
            return !v4 ? launch_kernel(k_reduce_wave<M, 1, 4, false>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld)
                   : peel ? launch_kernel(k_reduce_wave<M, 4, 4, true>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld)
                          : launch_kernel(k_reduce_wave<M, 4, 4, false>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld);
        case 16:
            return !v4 ? launch_kernel(k_reduce_wave<M, 1, 16, false>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld)
                   : peel ? launch_kernel(k_reduce_wave<M, 4, 16, true>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld)
                          : launch_kernel(k_reduce_wave<M, 4, 16, false>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld);
        case 64:
            return !v4 ? launch_kernel(k_reduce_wave<M, 1, 64, false>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld)
                   : peel ? launch_kernel(k_reduce_wave<M, 4, 64, true>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld)
                          : launch_kernel(k_reduce_wave<M, 4, 64, false>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld);
        default:
            return RR_ERR_TIER;
        }
    }
    case RR_TIER_TILED:
        return a.rows16 ? launch_kernel(k_reduce_tiled<M, 4, kTiledRows>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld)
                        : launch_kernel(k_reduce_tiled<M, 1, kTiledRows>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld);
    case RR_TIER_SERIAL:
        return a.rows16 ? launch_kernel(k_reduce_tiled<M, 4, 1>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld)
                        : launch_kernel(k_reduce_tiled<M, 1, 1>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld);
    case RR_TIER_SPLITK: {
        uint32_t* ticket = static_cast<uint32_t*>(a.workspace);
        A* part = reinterpret_cast<A*>(static_cast<char*>(a.workspace) +
                                       round_up(a.rows * 4, kWorkspaceAlign));
        const dim3 g2((unsigned)(p.grid > kMaxGrid ? kMaxGrid : p.grid));
        return a.vec ? launch_kernel(k_reduce_splitk<M, 4>, g2, block, 0, s, x, y, a.rows, a.cols, a.ld,
                                     p.slices, part, ticket, a.skew)
                     : launch_kernel(k_reduce_splitk<M, 1>, g2, block, 0, s, x, y, a.rows, a.cols, a.ld,
                                     p.slices, part, ticket, a.skew);
    }
    default:
        return RR_ERR_TIER;
    }
}

rr_status launch_reduce(const rr_plan& p, const ReduceLaunch& a)
{
    if (a.multi)
        return a.dtype == RR_F32 ? launch_monoid<MultiF32>(p, a)
                                 : a.dtype == RR_I32 ? launch_monoid<MultiI32>(p, a) : RR_ERR_DTYPE;
    if (a.dtype == RR_F32) {
        switch (a.op) {
        case RR_SUM: return launch_monoid<SumF32>(p, a);
        case RR_MAX: return launch_monoid<MaxF32>(p, a);
        case RR_MIN: return launch_monoid<MinF32>(p, a);
        }
    } else if (a.dtype == RR_I32) {
        switch (a.op) {
        case RR_SUM: return launch_monoid<SumI32>(p, a);
        case RR_MAX: return launch_monoid<MaxI32>(p, a);
        case RR_MIN: return launch_monoid<MinI32>(p, a);
        }
    }
    return RR_ERR_DTYPE;
}

// cols == 0: every row gets the monoid identity (each requested output of a
// tuple reduction its own).
static uint32_t identity_bits(rr_dtype dtype, rr_op op)
{
    if (dtype == RR_F32)
        return op == RR_SUM ? 0u : op == RR_MAX ? 0xFF800000u : 0x7F800000u;
    return op == RR_SUM ? 0u : op == RR_MAX ? 0x80000000u : 0x7FFFFFFFu;
}

rr_status launch_reduce_identity(const ReduceLaunch& a)
{
    const dim3 grid(grid_for(a.rows)), block(kBlockThreads);
    if (!a.multi)
        return launch_kernel(k_fill_u32, grid, block, 0, a.stream, static_cast<uint32_t*>(a.y),
                             a.rows, identity_bits(a.dtype, a.op));
    const rr_op ops[3] = {RR_SUM, RR_MAX, RR_MIN};
    for (int i = 0; i < 3; ++i) {
        if (!a.ys[i])
            continue;
        const rr_status st = launch_kernel(k_fill_u32, grid, block, 0, a.stream,
                                           static_cast<uint32_t*>(a.ys[i]), a.rows,
                                           identity_bits(a.dtype, ops[i]));
        if (st != RR_OK)
            return st;
    }
    return RR_OK;
}

}  // namespace rr
