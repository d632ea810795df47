// rr_device.hpp -- device building blocks for the gfx950 row-reduce kernels.
//
// Monoid states, 64-lane wavefront combines (DPP within 16-lane rows, then a
// fixed-order fold of the four rows), the cross-wavefront LDS combine with a
// broadcast result, 128-bit loads and bf16 packing.
//
// Every combine here has a fixed shape that depends only on the launch
// geometry, never on timing, so a kernel built from these pieces returns the
// same bits on every run.  Every combine function is commutative bit for bit
// (a+b == b+a in IEEE arithmetic, max/min are symmetric, and the online
// softmax pair below is written symmetrically), which the mirror-pattern DPP
// steps rely on: after each step all lanes of a group hold the same bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rr {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// ------------------------------------------------------------------ DPP
// DPP16 controls (GCN/CDNA): quad_perm selects within groups of 4 lanes;
// row_half_mirror reverses each 8-lane half row; row_mirror reverses each
// 16-lane row.
enum : int {
    kDppQuadSwap1 = 0xB1,  // quad_perm [1,0,3,2]
    kDppQuadSwap2 = 0x4E,  // quad_perm [2,3,0,1]
    kDppHalfMirror = 0x141,
    kDppMirror = 0x140,
};

// Every lane reads a lane of its own row (all row and bank masks on), so no
// lane keeps an old value: mov_dpp, with no old operand to materialise.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// A trivially copyable value as 32-bit words (for cross-lane moves).
template <class T>
struct Words {
    static_assert(sizeof(T) % 4 == 0, "values move as whole 32-bit words");
    uint32_t w[sizeof(T) / 4];
};

// DPP move of any trivially copyable value of whole 32-bit words, word by
// word (a tuple state moves each of its states on its own).
template <int CTRL, class T>
__device__ __forceinline__ T dpp(T v)
{
    Words<T> p = __builtin_bit_cast(Words<T>, v);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 4); ++i)
        p.w[i] = dpp_u32<CTRL>(p.w[i]);
    return __builtin_bit_cast(T, p);
}

template <class T>
__device__ __forceinline__ T readlane(T v, int lane)
{
    Words<T> p = __builtin_bit_cast(Words<T>, v);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 4); ++i)
        p.w[i] = (uint32_t)__builtin_amdgcn_readlane((int)p.w[i], lane);
    return __builtin_bit_cast(T, p);
}

// ------------------------------------------------------------- monoids
// IEEE 754 totalOrder as a signed-integer key: non-negative patterns keep
// their order, negative patterns reverse their magnitude bits.  The map is
// its own inverse and puts -0 below +0 and NaNs by sign and payload.
__device__ __forceinline__ int32_t f32_order_key(float x)
{
    int32_t b = __float_as_int(x);
    return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float f32_from_order_key(int32_t k)
{
    return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF));
}

// Every monoid writes its result with store(out, r, acc); out_t is the
// output pointer (a tuple of pointers for the tuple monoids below).  A
// single-statistic monoid also names an input whose lift leaves every state
// as it is (neutral_in), which masked lanes fold instead of selecting their
// state; the tuple monoids have none.
// float SUM: double accumulator, one rounding at the end.
struct SumF32 {
    using in_t = float;
    using acc_t = double;
    using out_t = float*;
    __device__ static acc_t identity() { return 0.0; }
    // -0 adds nothing to any sum (also to -0)
    __device__ static float neutral_in() { return -0.0f; }
    __device__ static acc_t lift(float x) { return (double)x; }
    __device__ static acc_t combine(acc_t a, acc_t b) { return a + b; }
    __device__ static float finish(acc_t a) { return (float)a; }
    __device__ static void store(out_t y, int64_t r, acc_t a) { y[r] = finish(a); }
};
// float MAX / MIN over totalOrder keys (identities are the extreme keys).
struct MaxF32 {
    using in_t = float;
    using acc_t = int32_t;
    using out_t = float*;
    __device__ static acc_t identity() { return INT32_MIN; }
    // the negative NaN of largest payload has the smallest key
    __device__ static float neutral_in() { return __int_as_float(-1); }
    __device__ static acc_t lift(float x) { return f32_order_key(x); }
    __device__ static acc_t combine(acc_t a, acc_t b) { return a > b ? a : b; }
    __device__ static float finish(acc_t a) { return f32_from_order_key(a); }
    __device__ static void store(out_t y, int64_t r, acc_t a) { y[r] = finish(a); }
};
struct MinF32 {
    using in_t = float;
    using acc_t = int32_t;
    using out_t = float*;
    __device__ static acc_t identity() { return INT32_MAX; }
    // the positive NaN of largest payload has the largest key
    __device__ static float neutral_in() { return __int_as_float(INT32_MAX); }
    __device__ static acc_t lift(float x) { return f32_order_key(x); }
    __device__ static acc_t combine(acc_t a, acc_t b) { return a < b ? a : b; }
    __device__ static float finish(acc_t a) { return f32_from_order_key(a); }
    __device__ static void store(out_t y, int64_t r, acc_t a) { y[r] = finish(a); }
};
// int32 SUM wraps modulo 2^32 (unsigned arithmetic), so order never matters.
struct SumI32 {
    using in_t = int32_t;
    using acc_t = uint32_t;
    using out_t = int32_t*;
    __device__ static acc_t identity() { return 0u; }
    __device__ static int32_t neutral_in() { return 0; }
    __device__ static acc_t lift(int32_t x) { return (uint32_t)x; }
    __device__ static acc_t combine(acc_t a, acc_t b) { return a + b; }
    __device__ static int32_t finish(acc_t a) { return (int32_t)a; }
    __device__ static void store(out_t y, int64_t r, acc_t a) { y[r] = finish(a); }
};
struct MaxI32 {
    using in_t = int32_t;
    using acc_t = int32_t;
    using out_t = int32_t*;
    __device__ static acc_t identity() { return INT32_MIN; }
    __device__ static int32_t neutral_in() { return INT32_MIN; }
    __device__ static acc_t lift(int32_t x) { return x; }
    __device__ static acc_t combine(acc_t a, acc_t b) { return a > b ? a : b; }
    __device__ static int32_t finish(acc_t a) { return a; }
    __device__ static void store(out_t y, int64_t r, acc_t a) { y[r] = finish(a); }
};
struct MinI32 {
    using in_t = int32_t;
    using acc_t = int32_t;
    using out_t = int32_t*;
    __device__ static acc_t identity() { return INT32_MAX; }
    __device__ static int32_t neutral_in() { return INT32_MAX; }
    __device__ static acc_t lift(int32_t x) { return x; }
    __device__ static acc_t combine(acc_t a, acc_t b) { return a < b ? a : b; }
    __device__ static int32_t finish(acc_t a) { return a; }
    __device__ static void store(out_t y, int64_t r, acc_t a) { y[r] = finish(a); }
};

// Several statistics over one read ("reduce", algorithm.gpu.rowwise: the body
// combines each state needing a cross-thread combine on its own): the tuple
// of the SUM, MAX and MIN states, each folded and combined by its own
// operation, so the tuple combine is bit-commutative because each part is.
// Outputs may be NULL (that statistic is not written).
template <class T>
struct Outs3 {
    T* sum;
    T* max;
    T* min;
};
struct MultiF32 {
    using in_t = float;
    struct acc_t {
        double sum;
        int32_t maxk, mink;  // totalOrder keys
    };
    using out_t = Outs3<float>;
    __device__ static acc_t identity() { return acc_t{0.0, INT32_MIN, INT32_MAX}; }
    __device__ static acc_t lift(float x)
    {
        const int32_t k = f32_order_key(x);
        return acc_t{(double)x, k, k};
    }
    __device__ static acc_t combine(acc_t a, acc_t b)
    {
        return acc_t{a.sum + b.sum, a.maxk > b.maxk ? a.maxk : b.maxk,
                     a.mink < b.mink ? a.mink : b.mink};
    }
    // the three results, in the order sum, max, min
    __device__ static void finish3(acc_t a, float* o)
    {
        o[0] = (float)a.sum;
        o[1] = f32_from_order_key(a.maxk);
        o[2] = f32_from_order_key(a.mink);
    }
    __device__ static void store(out_t y, int64_t r, acc_t a)
    {
        if (y.sum) y.sum[r] = (float)a.sum;
        if (y.max) y.max[r] = f32_from_order_key(a.maxk);
        if (y.min) y.min[r] = f32_from_order_key(a.mink);
    }
};
struct MultiI32 {
    using in_t = int32_t;
    struct acc_t {
        uint32_t sum;  // wraps modulo 2^32
        int32_t max, min;
    };
    using out_t = Outs3<int32_t>;
    __device__ static acc_t identity() { return acc_t{0u, INT32_MIN, INT32_MAX}; }
    __device__ static acc_t lift(int32_t x) { return acc_t{(uint32_t)x, x, x}; }
    __device__ static acc_t combine(acc_t a, acc_t b)
    {
        return acc_t{a.sum + b.sum, a.max > b.max ? a.max : b.max, a.min < b.min ? a.min : b.min};
    }
    __device__ static void finish3(acc_t a, int32_t* o)
    {
        o[0] = (int32_t)a.sum;
        o[1] = a.max;
        o[2] = a.min;
    }
    __device__ static void store(out_t y, int64_t r, acc_t a)
    {
        if (y.sum) y.sum[r] = (int32_t)a.sum;
        if (y.max) y.max[r] = a.max;
        if (y.min) y.min[r] = a.min;
    }
};

// Online softmax state (m, s): m the largest value seen, s = sum exp(x - m).
// (m1, s1) + (m2, s2) = (M, s1 exp(m1 - M) + s2 exp(m2 - M)), M = max(m1, m2);
// the identity is (-inf, 0) and two identities combine without evaluating
// exp(-inf - -inf).  Exponentials are base 2 on pre-scaled differences.
constexpr float kLog2e = 1.4426950408889634f;

struct MS {
    float m;
    float s;
};

// exp2 with correct subnormal results (the library function scales the
// argument range itself).
__device__ __forceinline__ float exp2_f32(float t) { return exp2f(t); }

// The hardware instruction v_exp_f32 alone: equal to exp2f wherever the
// result is a normal number (checked on MI355X over the whole normal range
// boundary), but it flushes results below 2^-126 to zero.  Used where such
// a result cannot change anything, or behind a check for that range.
__device__ __forceinline__ float exp2_hw(float t) { return __builtin_amdgcn_exp2f(t); }

// exp2 over the whole range from the hardware instruction: below -126 the
// argument is raised by 64 (a normal result, exact as above) and the result
// scaled by 2^-64, which rounds it once onto the subnormal grid.
__device__ __forceinline__ float exp2_sub(float t)
{
    const bool low = t < -126.0f;  // one exponential either way
    return exp2_hw(low ? t + 64.0f : t) * (low ? 0x1p-64f : 1.0f);
}

// Marks the rarely taken side of a branch between a fast and a
// subnormal-safe computation: an empty statement the compiler must keep, so
// that it does not turn the branch into both computations and a select
// (which ran every element through both).
__device__ __forceinline__ void keep_branch() { __asm__ volatile(""); }

struct SoftmaxMS {
    using acc_t = MS;
    __device__ static acc_t identity() { return MS{-__builtin_inff(), 0.0f}; }
    // Every non-identity state has s >= 1 (its own maximum contributes
    // exp(0) = 1), so a term flushed by exp2_hw -- below 2^-126 times s <=
    // 2^24 -- lies far under half an ulp of the other term and the hardware
    // exponential gives the same sum.
    __device__ static acc_t combine(acc_t a, acc_t b)
    {
        float M = fmaxf(a.m, b.m);
        if (M == -__builtin_inff())
            return MS{M, 0.0f};
        float s = a.s * exp2_hw((a.m - M) * kLog2e) + b.s * exp2_hw((b.m - M) * kLog2e);
        return MS{M, s};
    }
};

// Plain float max / sum monoids for the cheap wave-level steps of the
// softmax statistics (both are commutative bit for bit).
struct MaxFloat {
    using acc_t = float;
    __device__ static acc_t combine(acc_t a, acc_t b) { return fmaxf(a, b); }
};
struct SumFloat {
    using acc_t = float;
    __device__ static acc_t combine(acc_t a, acc_t b) { return a + b; }
};

// ----------------------------------------------------- wavefront combines

// Combine within aligned groups of S lanes (S in {1, 2, 4, 8, 16}); every
// lane of a group ends with the group's result.
template <class M, int S>
__device__ __forceinline__ typename M::acc_t group_reduce(typename M::acc_t v)
{
    static_assert(S == 1 || S == 2 || S == 4 || S == 8 || S == 16, "group of 1..16 lanes");
    if constexpr (S >= 2) v = M::combine(v, dpp<kDppQuadSwap1>(v));
    if constexpr (S >= 4) v = M::combine(v, dpp<kDppQuadSwap2>(v));
    if constexpr (S >= 8) v = M::combine(v, dpp<kDppHalfMirror>(v));
    if constexpr (S >= 16) v = M::combine(v, dpp<kDppMirror>(v));
    return v;
}

// Combine all 64 lanes; the result is wave-uniform.  The four 16-lane rows
// are folded in ascending row order.
template <class M>
__device__ __forceinline__ typename M::acc_t wave_reduce(typename M::acc_t v)
{
    v = group_reduce<M, 16>(v);
    typename M::acc_t r = readlane(v, 0);
    r = M::combine(r, readlane(v, 16));
    r = M::combine(r, readlane(v, 32));
    r = M::combine(r, readlane(v, 48));
    return r;
}

// Groups of S in {32, 64}: two or four rows folded in ascending order via
// cross-lane reads; every lane of a group gets the group's result.
template <class M, int S>
__device__ __forceinline__ typename M::acc_t group_reduce_wide(typename M::acc_t v)
{
    static_assert(S == 32 || S == 64, "wide group");
    using A = typename M::acc_t;
    if constexpr (S == 64) {
        return wave_reduce<M>(v);
    } else {
        v = group_reduce<M, 16>(v);
        A r0 = readlane(v, 0), r1 = readlane(v, 16), r2 = readlane(v, 32), r3 = readlane(v, 48);
        A lo = M::combine(r0, r1), hi = M::combine(r2, r3);
        return lane_id() < 32 ? lo : hi;
    }
}

template <class M, int S>
__device__ __forceinline__ typename M::acc_t segment_reduce(typename M::acc_t v)
{
    if constexpr (S <= 16)
        return group_reduce<M, S>(v);
    else
        return group_reduce_wide<M, S>(v);
}

// segment_reduce of N independent values, one combine step at a time over
// all of them, so that the DPP moves of one value fill the wait states of
// another.  Each value gets exactly the combines segment_reduce gives it.
template <class M, int S, int N>
__device__ __forceinline__ void segment_reduce_n(typename M::acc_t (&v)[N])
{
    using A = typename M::acc_t;
    if constexpr (S >= 2) {
        A t[N];
#pragma unroll
        for (int i = 0; i < N; ++i) t[i] = dpp<kDppQuadSwap1>(v[i]);
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = M::combine(v[i], t[i]);
    }
    if constexpr (S >= 4) {
        A t[N];
#pragma unroll
        for (int i = 0; i < N; ++i) t[i] = dpp<kDppQuadSwap2>(v[i]);
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = M::combine(v[i], t[i]);
    }
    if constexpr (S >= 8) {
        A t[N];
#pragma unroll
        for (int i = 0; i < N; ++i) t[i] = dpp<kDppHalfMirror>(v[i]);
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = M::combine(v[i], t[i]);
    }
    if constexpr (S >= 16) {
        A t[N];
#pragma unroll
        for (int i = 0; i < N; ++i) t[i] = dpp<kDppMirror>(v[i]);
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = M::combine(v[i], t[i]);
    }
    if constexpr (S > 16) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            // the 16-lane rows folded in ascending order, as group_reduce_wide
            const A r0 = readlane(v[i], 0), r1 = readlane(v[i], 16);
            const A r2 = readlane(v[i], 32), r3 = readlane(v[i], 48);
            if constexpr (S == 64) {
                v[i] = M::combine(M::combine(M::combine(r0, r1), r2), r3);
            } else {
                const A lo = M::combine(r0, r1), hi = M::combine(r2, r3);
                v[i] = lane_id() < 32 ? lo : hi;
            }
        }
    }
}

// Whether M names a neutral input (see the monoids above).
template <class M, class = void>
struct HasNeutralIn {
    static constexpr bool value = false;
};
template <class M>
struct HasNeutralIn<M, decltype((void)M::neutral_in())> {
    static constexpr bool value = true;
};

// acc combined with x when `on`, else left as it is: through the neutral
// input where M has one (a 32-bit select before the lift), else by
// selecting the state.
template <class M>
__device__ __forceinline__ typename M::acc_t fold_if(typename M::acc_t acc, typename M::in_t x,
                                                     bool on)
{
    if constexpr (HasNeutralIn<M>::value)
        return M::combine(acc, M::lift(on ? x : M::neutral_in()));
    else
        return on ? M::combine(acc, M::lift(x)) : acc;
}

// Workgroup combine of NT threads: wave combine, then each wave's lane 0
// writes its result to an LDS slot and every thread folds the slots in wave
// order after one barrier, so all threads return identical bits.  The caller
// alternates between two slot arrays from one call to the next: a wave that
// runs ahead can then only write the array its peers are not reading.
template <class M, int NT>
__device__ __forceinline__ typename M::acc_t block_reduce(typename M::acc_t v,
                                                          typename M::acc_t* slot)
{
    constexpr int NW = NT / kWave;
    v = wave_reduce<M>(v);
    if constexpr (NW == 1) {
        return v;
    } else {
        if (lane_id() == 0)
            slot[threadIdx.x / kWave] = v;
        __syncthreads();
        typename M::acc_t r = slot[0];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            r = M::combine(r, slot[w]);
        return r;
    }
}

// ---------------------------------------------------------------- memory

template <class T, int N>
struct Vec {
    T v[N];
};

typedef uint32_t rr_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t rr_u32x2 __attribute__((ext_vector_type(2)));

// 128-bit loads and stores.  The streaming kernels read every input byte
// once, so they use the non-temporal forms (global_load/store ... nt): on
// MI355X a plain stream of 128-bit nt loads sustains about 7 TB/s where the
// cached form stays near 6.2 TB/s.
__device__ __forceinline__ uint4 load16_nt(const void* p)
{
    rr_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const rr_u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store16_nt(void* p, uint4 u)
{
    rr_u32x4 v = {u.x, u.y, u.z, u.w};
    __builtin_nontemporal_store(v, reinterpret_cast<rr_u32x4*>(p));
}
__device__ __forceinline__ void store8_nt(void* p, uint2 u)
{
    rr_u32x2 v = {u.x, u.y};
    __builtin_nontemporal_store(v, reinterpret_cast<rr_u32x2*>(p));
}

// Elements of a row before its first 16-byte boundary (its head), at most
// cols: the row's 128-bit body starts at p + head_elems(p, cols).  p must be
// aligned to its element size.  "reduce" (algorithm.gpu.rowwise), tier
// semantics: the full-width tile function runs on the aligned chunks and the
// one-element tile function on the rest.
template <class T>
__device__ __forceinline__ int64_t head_elems(const T* p, int64_t cols)
{
    const int64_t h = (int64_t)((0u - (uint32_t)(uintptr_t)p) & 15u) / (int64_t)sizeof(T);
    return h < cols ? h : cols;
}

// One 128-bit load of 4 elements of 4 bytes at any 4-byte aligned address
// (the chip serves unaligned vector loads; NT: non-temporal).
typedef uint32_t rr_u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
template <class T, bool NT = false>
__device__ __forceinline__ Vec<T, 4> load4_unaligned(const T* p)
{
    static_assert(sizeof(T) == 4, "4-byte elements");
    const rr_u32x4_a4* q = reinterpret_cast<const rr_u32x4_a4*>(p);
    const rr_u32x4_a4 u = NT ? __builtin_nontemporal_load(q) : *q;
    // the words as plain values first: this compiler reads every element of
    // an under-aligned vector as element 0 when __builtin_bit_cast takes it
    // directly
    const uint32_t w0 = u.x, w1 = u.y, w2 = u.z, w3 = u.w;
    Vec<T, 4> r;
    r.v[0] = __builtin_bit_cast(T, w0);
    r.v[1] = __builtin_bit_cast(T, w1);
    r.v[2] = __builtin_bit_cast(T, w2);
    r.v[3] = __builtin_bit_cast(T, w3);
    return r;
}

// 16 and 8 bytes from any address with the alignment of the elements they
// hold (2 or 4 bytes), through the cache: one vector load each.  The words go
// through plain values first, as in load4_unaligned.
typedef uint32_t rr_u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
typedef uint32_t rr_u32x2_a2 __attribute__((ext_vector_type(2), aligned(2)));
__device__ __forceinline__ uint4 load16_any(const void* p)
{
    const rr_u32x4_a2 u = *reinterpret_cast<const rr_u32x4_a2*>(p);
    const uint32_t w0 = u.x, w1 = u.y, w2 = u.z, w3 = u.w;
    return make_uint4(w0, w1, w2, w3);
}
__device__ __forceinline__ uint2 load8_any(const void* p)
{
    const rr_u32x2_a2 u = *reinterpret_cast<const rr_u32x2_a2*>(p);
    const uint32_t w0 = u.x, w1 = u.y;
    return make_uint2(w0, w1);
}

// One 128-bit load of 4 elements of 4 bytes (NT: non-temporal).
template <class T, bool NT = false>
__device__ __forceinline__ Vec<T, 4> load4(const T* p)
{
    static_assert(sizeof(T) == 4, "4-byte elements");
    uint4 u = NT ? load16_nt(p) : *reinterpret_cast<const uint4*>(p);
    Vec<T, 4> r;
    r.v[0] = __builtin_bit_cast(T, u.x);
    r.v[1] = __builtin_bit_cast(T, u.y);
    r.v[2] = __builtin_bit_cast(T, u.z);
    r.v[3] = __builtin_bit_cast(T, u.w);
    return r;
}

// bf16 <-> f32.  bf16 is the top half of a binary32, so widening is a shift;
// narrowing rounds to nearest even in hardware (v_cvt_pk_bf16_f32).
typedef float rr_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 rr_bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    rr_f32x2 f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, rr_bf16x2));
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float a)
{
    return __builtin_bit_cast(uint16_t, (__bf16)a);
}

// double -> float rounded to odd: truncate toward zero and, if anything was
// dropped, set the last fraction bit.  Boldo and Melquiond ("Emulation of FMA
// and correctly rounded sums: proved algorithms using rounding to odd", IEEE
// Trans. Computers 57(4), 2008) show that a rounding to odd into a format
// with at least two more bits, followed by a rounding to nearest even into
// the narrower format, equals one rounding to nearest even.  float carries 16
// more fraction bits than bf16, so the pair below rounds a double to bf16
// once, where (float)a followed by the bf16 conversion can round twice (a
// value just above a bf16 tie becomes the tie in float and then rounds to
// even, one bf16 ulp low).  NaN stays NaN.
__device__ __forceinline__ float f32_round_odd(double a)
{
    float f = (float)a;  // nearest even
    if ((double)f != a) {
        uint32_t u = __float_as_uint(f);
        if (fabs((double)f) > fabs(a))
            u -= 1u;     // rounded away from zero (incl. overflow to inf): one step back
        f = __uint_as_float(u | 1u);
    }
    return f;
}
// The same bf16 through the plain float rounding, cheaper where most values
// are not near a bf16 halfway point: the double rounded to the nearest
// float, which the bf16 store's round to nearest even then takes to the
// double's correct bf16 -- except where that float lands exactly on a bf16
// halfway point (low 16 bits 0x8000) without being the double.  The double
// then lies to one side of the halfway point, and one float ulp toward it
// makes the store round that way.
__device__ __forceinline__ float f32_for_bf16(double a)
{
    const float f = (float)a;
    const uint32_t u = __float_as_uint(f);
    const double fd = (double)f;
    const uint32_t toward = fabs(a) > fabs(fd) ? u + 1u : u - 1u;
    return __uint_as_float((u & 0xFFFFu) == 0x8000u && fd != a ? toward : u);
}

__device__ __forceinline__ uint32_t pack_bf16x2_from_double(double a, double b)
{
    return pack_bf16x2(f32_round_odd(a), f32_round_odd(b));
}
__device__ __forceinline__ uint16_t bf16_bits_from_double(double a)
{
    return f32_to_bf16_bits(f32_round_odd(a));
}

// ------------------------------------------ cross-workgroup publishing
// Publishing a partial across workgroups (and across the eight XCDs, whose
// L2 caches are not coherent with each other).  The partial is written with a
// device-scope atomic store, which writes through the XCD's L2 to the
// device-coherent level, and s_waitcnt vmcnt(0) holds the wave until that
// store is acknowledged; only then is the ticket incremented.  This is the
// agent-scope release of the AMDGPU memory model without its L2 writeback
// (buffer_wbl2), which exists to push data written by ordinary stores and
// costs tens of microseconds when a thousand workgroups issue it at the end
// of a streaming pass.  The last workgroup reads the partials with
// device-scope atomic loads, which are served coherently without an L2
// invalidate.  The signal fences keep the compiler from moving the memory
// operations across the wait.
template <class A>
__device__ __forceinline__ void publish_partial(A* slot, A v)
{
    if constexpr (sizeof(A) == 4 || sizeof(A) == 8) {
        __hip_atomic_store(slot, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {  // a tuple state: word by word, all acknowledged before the ticket
        const Words<A> p = __builtin_bit_cast(Words<A>, v);
        uint32_t* s = reinterpret_cast<uint32_t*>(slot);
#pragma unroll
        for (int i = 0; i < (int)(sizeof(A) / 4); ++i)
            __hip_atomic_store(s + i, p.w[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
template <class A>
__device__ __forceinline__ A read_partial(const A* slot)
{
    if constexpr (sizeof(A) == 4 || sizeof(A) == 8) {
        return __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        Words<A> p;
        const uint32_t* s = reinterpret_cast<const uint32_t*>(slot);
#pragma unroll
        for (int i = 0; i < (int)(sizeof(A) / 4); ++i)
            p.w[i] = __hip_atomic_load(s + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return __builtin_bit_cast(A, p);
    }
}

// Zero a partial slot (plain stores, word by word; the next kernel on the
// stream sees them).
template <class A>
__device__ __forceinline__ void clear_partial(A* slot)
{
    uint32_t* s = reinterpret_cast<uint32_t*>(slot);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(A) / 4); ++i)
        s[i] = 0u;
}

// An (m, s) pair travels as one 64-bit word.
__device__ __forceinline__ uint64_t pack_ms(MS v) { return __builtin_bit_cast(uint64_t, v); }
__device__ __forceinline__ MS unpack_ms(uint64_t u) { return __builtin_bit_cast(MS, u); }

}  // namespace rr
