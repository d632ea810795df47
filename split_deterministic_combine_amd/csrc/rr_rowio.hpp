// rr_rowio.hpp -- row element access shared by the softmax and layernorm
// kernels: bf16 (as uint16_t bits) or float rows, moved in 16-byte chunks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rr_config.hpp"
#include "rr_device.hpp"

namespace rr {

// Element access: XT is uint16_t (bf16 bits) or float.  Whole 16-byte chunks
// move with non-temporal loads and stores (every byte is touched once).
template <class XT>
struct XIn;
template <>
struct XIn<uint16_t> {
    static constexpr int kChunk = 8;  // elements per 128-bit load
    __device__ static void chunk(const uint16_t* p, float* v)
    {
        uint4 u = load16_nt(p);
        v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x);
        v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
        v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z);
        v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
    }
    __device__ static float one(const uint16_t* p) { return bf16_bits_to_f32(*p); }
};
template <>
struct XIn<float> {
    static constexpr int kChunk = 4;
    __device__ static void chunk(const float* p, float* v)
    {
        uint4 u = load16_nt(p);
        v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
        v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
    }
    __device__ static float one(const float* p) { return *p; }
};

template <class YT>
struct YOut;
template <>
struct YOut<uint16_t> {
    template <int E>
    __device__ static void chunk(uint16_t* p, const float* v)
    {
        if constexpr (E == 8) {
            uint4 u;
            u.x = pack_bf16x2(v[0], v[1]); u.y = pack_bf16x2(v[2], v[3]);
            u.z = pack_bf16x2(v[4], v[5]); u.w = pack_bf16x2(v[6], v[7]);
            store16_nt(p, u);
        } else {
            static_assert(E == 4, "chunk of 4 or 8");
            uint2 u;
            u.x = pack_bf16x2(v[0], v[1]); u.y = pack_bf16x2(v[2], v[3]);
            store8_nt(p, u);
        }
    }
    __device__ static void one(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
};
template <>
struct YOut<float> {
    template <int E>
    __device__ static void chunk(float* p, const float* v)
    {
#pragma unroll
        for (int i = 0; i < E; i += 4)
            store16_nt(p + i, make_uint4(__float_as_uint(v[i]), __float_as_uint(v[i + 1]),
                                         __float_as_uint(v[i + 2]), __float_as_uint(v[i + 3])));
    }
    __device__ static void one(float* p, float v) { *p = v; }
};

// Load chunk j0 .. j0+E-1 of a row (E == 1 for the scalar variant), padding
// past `cols` with `pad` (-inf unless given).
template <class XT, int E, bool VEC>
__device__ __forceinline__ void load_padded(const XT* row, int64_t j0, int64_t cols, float* v,
                                            float pad = -__builtin_inff())
{
    if constexpr (VEC) {
        if (j0 + E <= cols) {
            XIn<XT>::chunk(row + j0, v);
            return;
        }
    }
    {
#pragma unroll
        for (int i = 0; i < E; ++i)
            v[i] = j0 + i < cols ? XIn<XT>::one(row + j0 + i) : pad;
    }
}

// Whether a chunk of E output elements can be stored at p with one (or two)
// vector stores: 16-byte alignment, 8 bytes for a bf16 chunk of 4.
template <class YT, int E>
__device__ __forceinline__ bool chunk_aligned(const YT* p)
{
    constexpr int kAlign = E * (int)sizeof(YT) < 16 ? E * (int)sizeof(YT) : 16;
    return ((uint32_t)(uintptr_t)p & (uint32_t)(kAlign - 1)) == 0;
}

// store_masked with the vector form chosen at run time (yvec: the row's
// chunks are chunk_aligned).
template <class YT, int E>
__device__ __forceinline__ void store_masked_rt(YT* row, int64_t j0, int64_t cols, const float* v,
                                                bool yvec)
{
    if constexpr (E > 1) {
        if (yvec && j0 + E <= cols) {
            YOut<YT>::template chunk<E>(row + j0, v);
            return;
        }
    }
#pragma unroll
    for (int i = 0; i < E; ++i)
        if (j0 + i < cols)
            YOut<YT>::one(row + j0 + i, v[i]);
}

template <class YT, int E, bool VEC>
__device__ __forceinline__ void store_masked(YT* row, int64_t j0, int64_t cols, const float* v)
{
    if constexpr (VEC) {
        if (j0 + E <= cols) {
            YOut<YT>::template chunk<E>(row + j0, v);
            return;
        }
    }
    {
#pragma unroll
        for (int i = 0; i < E; ++i)
            if (j0 + i < cols)
                YOut<YT>::one(row + j0 + i, v[i]);
    }
}

template <class XT>
__device__ __forceinline__ void unpack_chunk(uint4 u, float* v)
{
    if constexpr (sizeof(XT) == 2) {
        v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x);
        v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
        v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z);
        v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
    } else {
        v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
        v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
    }
}

// ------------------------------------------------ split-K tiles of a row
// One split-K tile of a thread: U chunks of E elements, chunk u at element
// offset (u * kBlockThreads + threadIdx.x) * E of the tile.
template <class XT, int E, bool VEC, int U>
__device__ __forceinline__ void load_tile_full(const XT* tile, float* v)
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const XT* p = tile + ((int64_t)u * kBlockThreads + threadIdx.x) * E;
        if constexpr (VEC)
            XIn<XT>::chunk(p, v + u * E);
        else
            v[u] = XIn<XT>::one(p);
    }
}

template <class XT, int E, bool VEC, int U>
__device__ __forceinline__ void load_tile_padded(const XT* row, int64_t begin, int64_t cols, float* v,
                                                 float pad = -__builtin_inff())
{
#pragma unroll
    for (int u = 0; u < U; ++u)
        load_padded<XT, E, VEC>(row, begin + ((int64_t)u * kBlockThreads + threadIdx.x) * E, cols,
                                v + u * E, pad);
}

template <class YT, int E, bool VEC, int U>
__device__ __forceinline__ void store_tile_full(YT* tile, const float* v)
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        YT* p = tile + ((int64_t)u * kBlockThreads + threadIdx.x) * E;
        if constexpr (VEC)
            YOut<YT>::template chunk<E>(p, v + u * E);
        else
            YOut<YT>::one(p, v[u]);
    }
}

template <class YT, int E, bool VEC, int U>
__device__ __forceinline__ void store_tile_masked(YT* row, int64_t begin, int64_t cols, const float* v)
{
#pragma unroll
    for (int u = 0; u < U; ++u)
        store_masked<YT, E, VEC>(row, begin + ((int64_t)u * kBlockThreads + threadIdx.x) * E, cols,
                                 v + u * E);
}

// Tile stores with the vector form chosen at run time (yvec: the row's chunks
// are chunk_aligned; else element by element).
template <class YT, int E, int U>
__device__ __forceinline__ void store_tile_full_rt(YT* tile, const float* v, bool yvec)
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        YT* p = tile + ((int64_t)u * kBlockThreads + threadIdx.x) * E;
        if (E > 1 && yvec) {
            if constexpr (E > 1)
                YOut<YT>::template chunk<E>(p, v + u * E);
        } else {
#pragma unroll
            for (int i = 0; i < E; ++i)
                YOut<YT>::one(p + i, v[u * E + i]);
        }
    }
}

template <class YT, int E, int U>
__device__ __forceinline__ void store_tile_masked_rt(YT* row, int64_t begin, int64_t cols,
                                                     const float* v, bool yvec)
{
#pragma unroll
    for (int u = 0; u < U; ++u)
        store_masked_rt<YT, E>(row, begin + ((int64_t)u * kBlockThreads + threadIdx.x) * E, cols,
                               v + u * E, yvec);
}

// A thread's share of one whole tile as loaded, before conversion to float,
// so that the next tile's loads can be in flight while this one is folded.
// Plain (cached) loads: split-K statistics passes are followed by a map pass
// that re-reads the same rows soon after.
template <class XT, bool VEC, int U>
struct RawTile;
template <class XT, int U>
struct RawTile<XT, true, U> {
    uint4 c[U];
    __device__ void load(const XT* tile)
    {
#pragma unroll
        for (int u = 0; u < U; ++u)
            c[u] = *reinterpret_cast<const uint4*>(
                tile + ((int64_t)u * kBlockThreads + threadIdx.x) * XIn<XT>::kChunk);
    }
    __device__ void unpack(float* v) const
    {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (sizeof(XT) == 2) {
                float* o = v + u * 8;
                o[0] = bf16_lo(c[u].x); o[1] = bf16_hi(c[u].x);
                o[2] = bf16_lo(c[u].y); o[3] = bf16_hi(c[u].y);
                o[4] = bf16_lo(c[u].z); o[5] = bf16_hi(c[u].z);
                o[6] = bf16_lo(c[u].w); o[7] = bf16_hi(c[u].w);
            } else {
                float* o = v + u * 4;
                o[0] = __uint_as_float(c[u].x); o[1] = __uint_as_float(c[u].y);
                o[2] = __uint_as_float(c[u].z); o[3] = __uint_as_float(c[u].w);
            }
        }
    }
};
template <class XT, int U>
struct RawTile<XT, false, U> {
    float c[U];
    __device__ void load(const XT* tile)
    {
#pragma unroll
        for (int u = 0; u < U; ++u)
            c[u] = XIn<XT>::one(tile + (int64_t)u * kBlockThreads + threadIdx.x);
    }
    __device__ void unpack(float* v) const
    {
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = c[u];
    }
};

// The 16-byte chunks k = 0 .. NCH-1 of a row held in registers by NT threads,
// at byte offsets (threadIdx.x + k * NT) * 16 from the row's start, as
// non-temporal buffer loads.  The row's start and length go into a buffer
// descriptor (scalar registers) and each chunk's offset is a loop-invariant
// 32-bit VGPR, so issuing a row takes no vector instruction.  The descriptor
// covers row_bytes: a chunk past the row end reads as zero (never stored).
// Word 3 sets the 32-bit data format, which untyped buffer loads on this
// architecture family expect to be non-zero.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kBufferNonTemporal = 2;  // cache-policy bits of the buffer builtins: nt
constexpr int kBufferDeviceScope = 16;  // sc1: device-coherent (write-through / L2-bypassing)

// Which chunk of a row's body slot k of a thread holds.  Unrotated, slot k
// of thread t holds chunk t + k * NT, so a wavefront's 64 slots of one k are
// 1 KiB of consecutive chunks.  Rotated by q (the body start's 16-byte index
// within its 128-byte memory line), slot s holds chunk (s - q) mod NS (NS =
// NCH * NT slots, a power of two): every wavefront's load or store of one k
// then covers whole lines from a line boundary, instead of touching nine
// lines, two of them partly, when rows do not start on a line (16 KiB bf16
// rows at a 16-byte row phase: 51 against 47 us for the whole softmax).
// Which chunks a row's sum folds in which thread changes with q; the result
// is still a function of the row's bytes and address.
template <int NCH, int NT, bool ROT>
__device__ __forceinline__ int slot_chunk(int k, int q)
{
    constexpr int NS = NCH * NT;
    static_assert((NS & (NS - 1)) == 0, "a power-of-two slot count");
    return ROT ? (((int)threadIdx.x + k * NT - q) & (NS - 1)) : (int)threadIdx.x + k * NT;
}
__device__ __forceinline__ int line_phase(const void* p)
{
    return (int)(((uintptr_t)p >> 4) & 7);
}

template <int NCH, int NT, bool ROT = false>
__device__ __forceinline__ void load_row_raw(const void* row, int64_t row_bytes, uint4* raw)
{
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(row), 0, (int)row_bytes, kBufferWord3);
    const int q = ROT ? line_phase(row) : 0;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int off = slot_chunk<NCH, NT, ROT>(k, q) * 16;
        const rr_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kBufferNonTemporal);
        raw[k] = make_uint4(v.x, v.y, v.z, v.w);
    }
}

// A persistent row as loaded: the thread's NCH 16-byte chunks of the row's
// body and, for rows that do not start 16-byte aligned or do not end on a
// chunk, one element of the head or the tail (PeelGeom).
template <int NCH>
struct RowBuf {
    uint4 c[NCH];
    float e;
};

// Where a row's elements go when its body is whole 16-byte chunks from its
// first 16-byte boundary ("reduce", algorithm.gpu.rowwise, tier semantics:
// full-width tiles on the aligned chunks, one-element tiles on the rest): h
// head elements, nbe body elements (a multiple of E), tl tail elements.
// Thread t < h holds head element t; thread h <= t < h + tl holds tail
// element h + nbe + (t - h) (h + tl <= 2E - 2, fewer than any workgroup's
// threads); `idx` is that element's column, or -1.
template <class XT>
struct PeelGeom {
    int64_t h, nbe, idx;
    __device__ PeelGeom(const XT* xr, int64_t cols)
    {
        constexpr int E = XIn<XT>::kChunk;
        h = head_elems(xr, cols);
        nbe = (cols - h) / E * E;
        const int64_t tl = cols - h - nbe;
        const int64_t t = threadIdx.x;
        idx = t < h ? t : t < h + tl ? nbe + t : -1;
    }
};

// Load a row's body chunks and the thread's head or tail element through one
// buffer descriptor over the row (bytes 0 when the row is not live: nothing
// is read, every value comes back as zero; the element is then -inf).
template <class XT, int NCH, int NT>
__device__ __forceinline__ void load_row_peeled(const XT* xr, int64_t cols, bool live,
                                                RowBuf<NCH>& buf)
{
    const PeelGeom<XT> pg(xr, cols);
    const int64_t row_bytes = live ? cols * (int64_t)sizeof(XT) : 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<XT*>(xr), 0, (int)row_bytes, kBufferWord3);
    const int body = (int)(pg.h * (int64_t)sizeof(XT));
    const int body_end = live ? (int)((pg.h + pg.nbe) * (int64_t)sizeof(XT)) : 0;
    const int q = line_phase(xr + pg.h);
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int off = slot_chunk<NCH, NT, true>(k, q) * 16;
        // chunks past the body read as zero (never used): clamp them to an
        // offset past the descriptor's range
        const int o = off + 16 <= body_end - body ? body + off : row_bytes + 16;
        const rr_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, kBufferNonTemporal);
        buf.c[k] = make_uint4(v.x, v.y, v.z, v.w);
    }
    const int eo = pg.idx >= 0 ? (int)(pg.idx * (int64_t)sizeof(XT)) : row_bytes + 16;
    float e;
    if constexpr (sizeof(XT) == 2)
        e = bf16_bits_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rs, eo, 0, kBufferNonTemporal));
    else
        e = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, eo, 0, kBufferNonTemporal));
    buf.e = (live && pg.idx >= 0) ? e : -__builtin_inff();
}

// The stores of one row held as NCH chunks of E values per thread (slot k
// of thread t: row elements h + slot_chunk(k, q) * E onwards, the layout
// load_row_peeled reads) plus one head or tail value (element idx, or none
// when idx < 0), as non-temporal buffer stores: a chunk's E outputs in one
// 8-, 16- or 32-byte store at whatever 2-byte offset the output row gives
// them, the extra value in a 16- or 32-bit one.  Chunks past the body
// (element h + nbe on) and threads without an extra value store at an
// offset past the descriptor's range, which the hardware drops, so every
// thread issues the same stores with no branch between them: the waits of
// persistent_rows then count a fixed number of stores.
template <class YT, int E, int NCH, int NT, bool ROT>
__device__ __forceinline__ void store_row_peeled(YT* yr, int64_t cols, int64_t h, int64_t nbe,
                                                 int64_t idx, const float* v, float ev, int q)
{
    constexpr int S = (int)sizeof(YT);
    const int row_bytes = (int)(cols * S);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(yr, 0, row_bytes, kBufferWord3);
    const int past = row_bytes + 32;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int j0 = slot_chunk<NCH, NT, ROT>(k, q) * E;
        const int o = j0 + E <= nbe ? (int)(h + j0) * S : past;
        const float* c = v + k * E;
        if constexpr (S == 2) {
            if constexpr (E == 8) {
                const rr_u32x4 u = {pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3]),
                                    pack_bf16x2(c[4], c[5]), pack_bf16x2(c[6], c[7])};
                __builtin_amdgcn_raw_buffer_store_b128(u, rs, o, 0, kBufferNonTemporal);
            } else {
                static_assert(E == 4, "chunks of 4 or 8 elements");
                const rr_u32x2 u = {pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3])};
                __builtin_amdgcn_raw_buffer_store_b64(u, rs, o, 0, kBufferNonTemporal);
            }
        } else {
#pragma unroll
            for (int q = 0; q < E; q += 4) {
                const rr_u32x4 u = {__float_as_uint(c[q]), __float_as_uint(c[q + 1]),
                                    __float_as_uint(c[q + 2]), __float_as_uint(c[q + 3])};
                __builtin_amdgcn_raw_buffer_store_b128(u, rs, o + q * 4, 0, kBufferNonTemporal);
            }
        }
    }
    const int eo = idx >= 0 ? (int)idx * S : past;
    if constexpr (S == 2)
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)f32_to_bf16_bits(ev), rs, eo, 0,
                                              kBufferNonTemporal);
    else
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ev), rs, eo, 0, kBufferNonTemporal);
}

// Persistent rows with a one-row prefetch.  Workgroup b takes rows b, b + step,
// ... < rows; the loads of the next row go out before the current row is
// computed, into the other of two register buffers.  On gfx9 one in-order
// counter (vmcnt) covers loads and stores, and the compiler places each wait
// before the first use of a row's data, so two things keep that wait from
// retiring the next row's loads too:
//   * a scheduling barrier after each prefetch keeps the first uses of the
//     current row below those loads;
//   * the first row is peeled, so the loop is entered with the same memory
//     operations in flight as on its back edge (the next row's loads, then
//     the current row's stores).  Otherwise the wait at the loop head is the
//     stricter of the two paths, and on the back edge it also waits for the
//     previous row's stores.
// Loads the caller issues before this (a row's weights) retire with the first
// row.  With no next row the prefetch still goes out, with no bytes to read
// (the buffer loads then read zeros and touch no memory), so no load sits
// behind a branch.  load(r, live, buf) issues row r's loads (none of its
// bytes when live is false); start() runs once, after the first two rows'
// loads are out (to unpack what the caller loaded before); row(buf, r,
// parity) computes and stores row r (parity alternates, for double-buffered
// shared memory).
template <class Buf, class Load, class Start, class Row>
__device__ __forceinline__ void persistent_rows(int64_t r, int64_t step, int64_t rows, Load load,
                                                Start start, Row row)
{
    // Rows after the current one; the loop tests it against zero only (a
    // 64-bit less-than has no scalar form and would put a VGPR write, and
    // with it a wait, ahead of the prefetch).
    int64_t left = (rows - 1 - r) / step;
    Buf a, c;
    load(r, true, a);
    __builtin_amdgcn_sched_barrier(0);  // the first row's loads go out first
    load(r + step, left != 0, c);
    __builtin_amdgcn_sched_barrier(0);
    start();
    row(a, r, 0);
    for (;;) {
        if (left == 0)
            return;
        r += step;
        --left;
        load(r + step, left != 0, a);
        __builtin_amdgcn_sched_barrier(0);
        row(c, r, 1);
        if (left == 0)
            return;
        r += step;
        --left;
        load(r + step, left != 0, c);
        __builtin_amdgcn_sched_barrier(0);
        row(a, r, 0);
    }
}

}  // namespace rr
