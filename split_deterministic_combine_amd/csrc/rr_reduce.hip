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
#include "rr_plan.hpp"
#include "rr_rowio.hpp"

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

// ------------------------------------- block tier, persistent rows
// Rows that fit a workgroup's registers (row_pf_shape: NT threads, NCH
// 16-byte chunks each), on a persistent grid: workgroup b takes rows b,
// b + grid, ... and loads the next row while it folds the current one
// (persistent_rows).  Each row's body, from its first 16-byte boundary, sits
// in chunk slots rotated onto 128-byte lines (slot_chunk), so every load
// instruction covers whole lines; PEEL: the head and tail elements (rows that
// do not all start 16-byte aligned or do not end on a chunk) one to each of
// the first threads, in their own element load through the same buffer
// descriptor.  Chunks past the body read nothing (an offset past the
// descriptor's range) and are dropped from the fold as a whole.
template <int NCH>
struct ReduceRowBuf {
    uint4 c[NCH];
    uint32_t e;
};

template <class M>
__device__ __forceinline__ typename M::acc_t lift_bits(uint32_t u)
{
    if constexpr (std::is_same<typename M::in_t, float>::value)
        return M::lift(__uint_as_float(u));
    else
        return M::lift((typename M::in_t)u);
}

// The results of a step's rows r0 .. r0 + nr - 1, row r0 + seg's by the
// first lane of its segment: every thread issues the stores, through one
// descriptor per output over the step's nr results, and the others' go past
// the range (a store behind a branch would make the persistent loop's waits
// count it); the three statistics' outputs may be NULL (range 0).
__device__ __forceinline__ void store_word(void* p, int nr, uint32_t bits, int seg, bool first)
{
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(p, 0, nr * 4,
                                                                        kBufferWord3);
    __builtin_amdgcn_raw_buffer_store_b32(bits, rs, first && seg < nr ? seg * 4 : nr * 4 + 16,
                                          0, 0);
}
template <class M>
__device__ __forceinline__ void store_row_results(typename M::out_t y, int64_t r0, int nr,
                                                  int seg, bool first, typename M::acc_t a)
{
    using T = typename M::in_t;
    uint32_t bits;
    if constexpr (std::is_pointer<typename M::out_t>::value) {
        const T res = M::finish(a);
        __builtin_memcpy(&bits, &res, 4);
        store_word(y + r0, nr, bits, seg, first);
    } else {
        T res[3];
        M::finish3(a, res);
        T* outs[3] = {y.sum, y.max, y.min};
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            __builtin_memcpy(&bits, &res[i], 4);
            store_word(outs[i] ? outs[i] + r0 : nullptr, outs[i] ? nr : 0, bits, seg, first);
        }
    }
}

template <class M, int NCH, int NT, bool PEEL, int S = NT>
__global__ __launch_bounds__(NT) void k_reduce_rows_pf(const typename M::in_t* __restrict__ x,
                                                       typename M::out_t y, int64_t rows,
                                                       int64_t cols, int64_t ld)
{
    using T = typename M::in_t;
    using A = typename M::acc_t;
    static_assert(sizeof(T) == 4, "4-byte elements");
    static_assert(S == NT || (NT == kWave && (S == 16 || S == 32)), "row segments of a wavefront");
    constexpr int RPS = NT / S;     // rows per step
    constexpr int NS = S * NCH;     // chunk slots per row
    static_assert((NS & (NS - 1)) == 0, "a power-of-two slot count");
    __shared__ A slot[2][NT / kWave > 1 ? NT / kWave : 1];
    const int64_t steps = (rows + RPS - 1) / RPS;
    if ((int64_t)blockIdx.x >= steps)
        return;
    const int ls = (int)threadIdx.x % S;        // lane within the row's segment
    const int seg = (int)threadIdx.x / S;       // the segment's row within the step
    auto slot_of = [&](int k, int q) { return (ls + k * S - q) & (NS - 1); };
    auto live_rows = [&](int64_t g) {           // rows of step g inside the call
        const int64_t n = rows - g * RPS;
        return (int)(n < RPS ? n : RPS);
    };
    persistent_rows<ReduceRowBuf<NCH>>(
        blockIdx.x, gridDim.x, steps,
        [&](int64_t g, bool live, ReduceRowBuf<NCH>& buf) {
            const int nr = live ? live_rows(g) : 0;
            const T* x0 = x + g * RPS * ld;
            const int range = nr > 0 ? (int)(((int64_t)nr - 1) * ld * 4 + cols * 4) : 0;
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<T*>(x0), 0, range, kBufferWord3);
            const T* xr = x0 + (int64_t)seg * ld;
            const int64_t h = PEEL ? head_elems(xr, cols) : 0;
            const int nbe = seg < nr ? (int)((cols - h) & ~(int64_t)3) : 0;
            const int base = (int)((int64_t)seg * ld * 4 + h * 4);
            const int q = line_phase(xr + h);
#pragma unroll
            for (int k = 0; k < NCH; ++k) {
                const int off = slot_of(k, q) * 16;
                const int o = off + 16 <= nbe * 4 ? base + off : range + 16;
                const rr_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0,
                                                                          kBufferNonTemporal);
                buf.c[k] = make_uint4(v.x, v.y, v.z, v.w);
            }
            if constexpr (PEEL) {
                // lane l < h: head element l; h <= l < h + tail: element nbe + l
                const int64_t t = ls, tl = cols - h - nbe;
                const int64_t idx = seg >= nr ? -1 : t < h ? t : t < h + tl ? nbe + t : -1;
                const int eo = idx >= 0 ? (int)((int64_t)seg * ld * 4 + idx * 4) : range + 16;
                buf.e = __builtin_amdgcn_raw_buffer_load_b32(rs, eo, 0, kBufferNonTemporal);
            }
        },
        [] {},
        [&](const ReduceRowBuf<NCH>& buf, int64_t g, int par) {
            const int nr = live_rows(g);
            const T* xr = x + (g * RPS + seg) * ld;
            const int64_t h = PEEL ? head_elems(xr, cols) : 0;
            const int64_t nb = (cols - h) >> 2;
            const int q = line_phase(xr + h);
            A acc = M::identity();
#pragma unroll
            for (int k = 0; k < NCH; ++k) {
                const uint4 u = buf.c[k];
                A ck = lift_bits<M>(u.x);
                ck = M::combine(ck, lift_bits<M>(u.y));
                ck = M::combine(ck, lift_bits<M>(u.z));
                ck = M::combine(ck, lift_bits<M>(u.w));
                acc = (int64_t)slot_of(k, q) < nb ? M::combine(acc, ck) : acc;
            }
            if constexpr (PEEL) {
                const int64_t tl = cols - h - (nb << 2);
                if (ls < h + tl)
                    acc = M::combine(acc, lift_bits<M>(buf.e));
            }
            if constexpr (S == NT)
                acc = block_reduce<M, NT>(acc, slot[par]);
            else
                acc = segment_reduce<M, S>(acc);
            store_row_results<M>(y, g * RPS, nr, seg, ls == 0, acc);
        });
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
// PEEL (kPeelNone): every row starts 16-byte aligned and is whole chunks (no
// head or tail elements).  kPeelQuads, when a segment has two lanes past the
// body (nb + 2 <= S): lane nb reads the row's first four elements and lane
// nb + 1 its last four, each in one 128-bit load of the same instruction
// as the body, and folds the head's h (the tail's tl) of them; with no
// separate instruction for the head and tail, no memory line of the row is
// asked for twice.  kPeelElements: the head and tail one element per lane
// as above, in their own loads.
//
// Tasks start at multiples of 4 * 64 / S rows, so with 4-byte elements the
// row a lane reads in group u of any task sits at the same offset from a
// 16-byte boundary as row u * 64 / S + (its segment): the lane's column
// split is worked out once per group before the first task (once in all
// when 64 / S is a multiple of 4) and reused by every task that has all
// its rows.  Only the last task of a ragged row count works it out per row.
enum WavePeel { kPeelNone = 0, kPeelElements = 1, kPeelQuads = 2 };

template <class M, int VEC, int S, int PEEL>
__global__ __launch_bounds__(kBlockThreads) void k_reduce_wave(
    const typename M::in_t* __restrict__ x, typename M::out_t y, int64_t rows,
    int64_t cols, int64_t ld)
{
    using T = typename M::in_t;
    using A = typename M::acc_t;
    static_assert(sizeof(T) == 4, "the wave tier reads 4-byte elements");
    constexpr int RPG = kWave / S;
    constexpr int U = kWaveRowGroups;
    constexpr int NX = VEC == 4 && PEEL == kPeelElements ? (6 + S - 1) / S : 0;  // per lane
    constexpr int NXA = NX > 0 ? NX : 1;
    constexpr int NG = VEC == 4 && PEEL != kPeelNone && RPG % 4 != 0 ? U : 1;  // distinct splits
    const int lane = lane_id();
    const int seg = lane / S;
    const int li = lane % S;
    const int c = (int)cols;  // a wave-tier row has at most 64 * VEC columns

    // The column split of a row starting at p: the lane's body chunk (or
    // element) offset and which of its VEC values are in the row (all or
    // none, except for the quads), its head / tail element offsets (0 when
    // it has none) and whether each is in the row.
    struct Split {
        int body;
        uint32_t on;  // bit i: value i of the lane's chunk is folded
        int xo[NXA];
        bool has[NXA];
    };
    auto split_of = [&](const T* p) {
        Split g;
        if constexpr (VEC == 4) {
            const int h = PEEL != kPeelNone ? (int)head_elems(p, cols) : 0;
            const int nbe = (c - h) & ~3;
            const int nb = nbe / 4;
            const bool full = li < nb;
            g.on = full ? 0xFu : 0u;
            g.body = h + (full ? li * 4 : 0);
            if constexpr (PEEL == kPeelQuads) {
                const int tl = c - h - nbe;                  // 0..3 tail elements
                if (li == nb) {                              // the first four: h of them
                    g.body = 0;
                    g.on = (1u << h) - 1u;
                } else if (li == nb + 1) {                   // the last four: tl of them
                    g.body = c - 4;
                    g.on = (0xFu << (4 - tl)) & 0xFu;
                }
            }
#pragma unroll
            for (int k = 0; k < NXA; ++k) {
                // head or tail element ex of h + tl = cols - nbe: column ex
                // of the head, or nbe + ex (= h + nbe + (ex - h)) of the tail
                const int ex = li + k * S;
                g.has[k] = NX > 0 && ex < c - nbe;
                g.xo[k] = g.has[k] ? (ex < h ? ex : nbe + ex) : 0;
            }
        } else {
            g.on = li < c ? 1u : 0u;
            g.body = li < c ? li : 0;
#pragma unroll
            for (int k = 0; k < NXA; ++k) {
                g.has[k] = false;
                g.xo[k] = 0;
            }
        }
        return g;
    };
    Split pre[NG];
#pragma unroll
    for (int u = 0; u < NG; ++u) {
        // row u * RPG + seg's offset from a 16-byte boundary, from integers
        // (the row need not exist)
        const uintptr_t a = (uintptr_t)x + (uintptr_t)(((int64_t)u * RPG + seg) * ld) * sizeof(T);
        pre[u] = split_of(reinterpret_cast<const T*>(a));
    }
    // one task: loads of all U groups, then the folds, the combines and the
    // stores.  WHOLE: every row of the task exists, group u's row is RPG * ld
    // elements after group u - 1's and its split is pre[u]; otherwise rows
    // are clamped and each split is worked out from its row.
    auto task = [&](int64_t row0, auto whole) {
        constexpr bool WHOLE = decltype(whole)::value;
        Vec<T, VEC> v[U];
        T xe[U][NXA];
        uint32_t on[U];
        bool has[U][NXA];
        const T* base = x + (row0 + seg) * ld;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const T* rp;
            Split g;
            if constexpr (WHOLE) {
                rp = base + (int64_t)u * RPG * ld;
                g = pre[NG == 1 ? 0 : u];
            } else {
                int64_t r = row0 + (int64_t)u * RPG + seg;
                r = r < rows ? r : rows - 1;
                rp = x + r * ld;
                g = split_of(rp);
            }
            on[u] = g.on;
            if constexpr (VEC == 4)
                v[u] = PEEL == kPeelQuads ? load4_unaligned<T, true>(rp + g.body)
                                          : load4<T, true>(rp + g.body);
            else
                v[u].v[0] = rp[g.body];
#pragma unroll
            for (int k = 0; k < NX; ++k) {
                // non-temporal like the body: a plain load of a line that a
                // streaming load of the body also asks for costs a refetch
                has[u][k] = g.has[k];
                xe[u][k] = __builtin_nontemporal_load(rp + g.xo[k]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // every load of the task goes out before any fold
        A acc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            acc[u] = M::identity();
#pragma unroll
            for (int i = 0; i < VEC; ++i)
                acc[u] = fold_if<M>(acc[u], v[u].v[i], (on[u] >> i) & 1u);
#pragma unroll
            for (int k = 0; k < NX; ++k)
                acc[u] = fold_if<M>(acc[u], xe[u][k], has[u][k]);
        }
        segment_reduce_n<M, S, U>(acc);
        // Every lane of a segment holds the row's result after the combine,
        // so all of them store it (the same bits to one address), and rows
        // past the end store their clamped row's result -- the last row's,
        // computed the same way -- to that row.  No store is predicated: a
        // predicated store between two groups makes the memory-counter wait
        // before the next group's fold also hold for a load it does not need.
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t r = row0 + (int64_t)u * RPG + seg;
            M::store(y, WHOLE || r < rows ? r : rows - 1, acc[u]);
        }
    };

    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
         w * RPG * U < rows; w += nwaves) {
        const int64_t row0 = w * RPG * U;
        if (row0 + RPG * U <= rows)  // wave-uniform: every row of the task exists
            task(row0, std::true_type{});
        else
            task(row0, std::false_type{});
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

// The wave tier with S lanes per row: 128-bit chunks for rows of at least
// 7 elements (as the plan's lanes); head and tail elements unless every row
// is aligned whole chunks, as quads when two lanes of every segment are
// past the body (a body has at most cols / 4 chunks).
template <class M, int S>
static rr_status launch_wave(dim3 grid, dim3 block, hipStream_t s, const typename M::in_t* x,
                             typename M::out_t y, const ReduceLaunch& a)
{
    if (!(a.vec && a.cols >= 7))
        return launch_kernel(k_reduce_wave<M, 1, S, kPeelNone>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld);
    if (a.rows16 && a.cols % 4 == 0)
        return launch_kernel(k_reduce_wave<M, 4, S, kPeelNone>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld);
    if (a.cols / 4 + 2 <= S)
        return launch_kernel(k_reduce_wave<M, 4, S, kPeelQuads>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld);
    return launch_kernel(k_reduce_wave<M, 4, S, kPeelElements>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld);
}

// Block tier, persistent rows: the plan's grid, lowered to the workgroups
// that can be resident at once.
template <class M>
static typename M::out_t outputs_of(const ReduceLaunch& a);

template <class M, int NCH, int NT, int S = NT>
static rr_status launch_rows_pf(const rr_plan& p, const ReduceLaunch& a)
{
    const auto* x = static_cast<const typename M::in_t*>(a.x);
    const typename M::out_t y = outputs_of<M>(a);
    auto kernel = a.rows16 && a.cols % 4 == 0 ? k_reduce_rows_pf<M, NCH, NT, false, S>
                                              : k_reduce_rows_pf<M, NCH, NT, true, S>;
    int per_cu = 0;
    if (blocks_per_cu(kernel, NT, &per_cu) != RR_OK)
        return RR_ERR_HIP;
    const int64_t cap = (int64_t)per_cu * a.cu;
    const dim3 grid((unsigned)(p.grid < cap ? p.grid : cap));
    return launch_kernel(kernel, grid, dim3(NT), 0, a.stream, x, y, a.rows, a.cols, a.ld);
}

template <class M>
static rr_status launch_rows_pf_shape(const rr_plan& p, const ReduceLaunch& a, RowPfShape sh)
{
    if (sh.nt != p.block)
        return RR_ERR_TIER;  // plan and launch disagree: refuse, launch nothing
    const int lanes = reduce_pf_lanes(a.cols, a.ld);
    if (lanes != p.lanes_per_row)
        return RR_ERR_TIER;
    switch (sh.nt * 16 + sh.nch) {
    case 64 * 16 + 4:
        return lanes == 16   ? launch_rows_pf<M, 4, 64, 16>(p, a)
               : lanes == 32 ? launch_rows_pf<M, 4, 64, 32>(p, a)
                             : launch_rows_pf<M, 4, 64>(p, a);
    case 128 * 16 + 4: return launch_rows_pf<M, 4, 128>(p, a);
    case 256 * 16 + 4: return launch_rows_pf<M, 4, 256>(p, a);
    case 512 * 16 + 4: return launch_rows_pf<M, 4, 512>(p, a);
    default: return RR_ERR_TIER;
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
    case RR_TIER_BLOCK: {
        const RowPfShape sh =
            reduce_pf_shape(a.rows, a.cols, a.multi ? RR_SUM_MAX_MIN : a.op, a.cu, a.vec);
        if (sh.nt > 0 && a.cu > 0)
            return launch_rows_pf_shape<M>(p, a, sh);
    }
        return !a.vec ? launch_kernel(k_reduce_block<M, 1, false>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld)
               : a.rows16 ? launch_kernel(k_reduce_block<M, 4, false>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld)
                          : launch_kernel(k_reduce_block<M, 4, true>, grid, block, 0, s, x, y, a.rows, a.cols, a.ld);
    case RR_TIER_WAVE:
        switch (p.lanes_per_row) {
        case 4: return launch_wave<M, 4>(grid, block, s, x, y, a);
        case 16: return launch_wave<M, 16>(grid, block, s, x, y, a);
        case 64: return launch_wave<M, 64>(grid, block, s, x, y, a);
        default: return RR_ERR_TIER;
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
        default: return RR_ERR_OP;  // the three statistics take the multi path above
        }
    } else if (a.dtype == RR_I32) {
        switch (a.op) {
        case RR_SUM: return launch_monoid<SumI32>(p, a);
        case RR_MAX: return launch_monoid<MaxI32>(p, a);
        case RR_MIN: return launch_monoid<MinI32>(p, a);
        default: return RR_ERR_OP;
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
