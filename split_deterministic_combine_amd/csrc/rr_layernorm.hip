// rr_layernorm.hip -- two-pass layer normalisation over the last axis, gfx950.
//
// "reduce" (algorithm.gpu.rowwise), description: layernorm is one of the
// two-pass algorithms -- pass 1 reduces the row's statistics, each state
// combined across threads on its own, and pass 2 is a pure map:
//   mean = sum x / n,  var = sum (x - mean)^2 / n,  rstd = 1 / sqrt(var + eps)
//   y = (x - mean) * rstd * gamma + beta      (gamma / beta per column)
//
// Statistics, by how much of the row a thread holds:
//   * rows in registers (block tier: persistent workgroups of 64 to 512
//     threads holding up to 4 chunks each, or up to kLnMaxChunks chunks per
//     thread of 256 for unaligned rows; wave tier): the exact two-pass form.  The sum of x is taken in
//     double; then every thread forms d = (x - mean_f) - c, with mean_f the
//     float mean and c = (float)(mean - mean_f), and the sum of d^2 is taken
//     (float inside a chunk, double across chunks and threads).  d stays in
//     registers for the map.
//   * rows streamed from memory (long rows, split-K): one statistics read with
//     sums shifted by the row's first element K: s1 = sum (x - K),
//     s2 = sum (x - K)^2, in double.  Then mean = K + s1/n and
//     n var = s2 - s1^2/n.  Since K is an element of the row,
//     |K - mean| <= sqrt(n - 1) * sd (Samuelson's inequality), so the
//     cancellation costs at most log2(n) bits of the double's 53.
// Each state is combined across threads by its own fixed-shape sum
// (wave DPP tree, then waves in order), so every run gives the same bits.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "rr_config.hpp"
#include "rr_device.hpp"
#include "rr_launch.hpp"
#include "rr_launch_util.hpp"
#include "rr_rowio.hpp"

namespace rr {

// Per-column weights: gamma (default 1) or beta (default 0), float or bf16.
struct Weights {
    const void* p;  // NULL: every column takes `dflt`
    bool bf16;
    float dflt;
};

// Row statistics from the two reduced states.
struct LnRow {
    double mean;
    double rstd;
};

namespace {

__device__ __forceinline__ float weight_one(const Weights& w, int64_t j)
{
    if (!w.p)
        return w.dflt;
    return w.bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(w.p)[j])
                  : static_cast<const float*>(w.p)[j];
}

// The weights of a row's body that starts h columns in: the same vector,
// offset by h elements (a NULL vector stays NULL).
__device__ __forceinline__ Weights shifted(const Weights& w, int64_t h)
{
    return Weights{w.p ? static_cast<const char*>(w.p) + h * (w.bf16 ? 2 : 4) : nullptr, w.bf16,
                   w.dflt};
}

// E weights of columns j0 .. j0+E-1 (past `cols`: the default).  With VEC a
// whole chunk inside the row is one vector load at whatever element
// alignment the vector gives it (cached: every row reads the same weights);
// the rest element by element.
template <int E, bool VEC>
__device__ __forceinline__ void load_weights(const Weights& w, int64_t j0, int64_t cols, float* o)
{
    if (!w.p) {
#pragma unroll
        for (int i = 0; i < E; ++i)
            o[i] = w.dflt;
        return;
    }
    if constexpr (VEC) {
        if (j0 + E <= cols) {
            if (w.bf16) {
                const uint16_t* p = static_cast<const uint16_t*>(w.p) + j0;
                if constexpr (E == 8) {
                    const uint4 u = load16_any(p);
                    o[0] = bf16_lo(u.x); o[1] = bf16_hi(u.x);
                    o[2] = bf16_lo(u.y); o[3] = bf16_hi(u.y);
                    o[4] = bf16_lo(u.z); o[5] = bf16_hi(u.z);
                    o[6] = bf16_lo(u.w); o[7] = bf16_hi(u.w);
                } else {
                    static_assert(E == 4, "chunks of 4 or 8 elements");
                    const uint2 u = load8_any(p);
                    o[0] = bf16_lo(u.x); o[1] = bf16_hi(u.x);
                    o[2] = bf16_lo(u.y); o[3] = bf16_hi(u.y);
                }
            } else {
                const float* p = static_cast<const float*>(w.p) + j0;
#pragma unroll
                for (int k = 0; k < E; k += 4) {
                    const uint4 u = load16_any(p + k);
                    o[k] = __uint_as_float(u.x); o[k + 1] = __uint_as_float(u.y);
                    o[k + 2] = __uint_as_float(u.z); o[k + 3] = __uint_as_float(u.w);
                }
            }
            return;
        }
    }
#pragma unroll
    for (int i = 0; i < E; ++i)
        o[i] = j0 + i < cols ? weight_one(w, j0 + i) : w.dflt;
}

// One output, y = (x - mean) * rstd * gamma + beta, formed in double (x -
// mean is exact there) and rounded once to the output type: a float output
// directly; a bf16 one through the float that the bf16 store then rounds to
// the double's correct bf16 (f32_for_bf16).  Without weights gamma is 1 and
// beta 0, which leave the product as it is.
template <class YT>
struct LnMap {
    double mean, rstd;
    __device__ double exact(float x, float g, float b) const
    {
        return __builtin_fma(((double)x - mean) * rstd, (double)g, (double)b);
    }
    __device__ float operator()(float x, float g, float b) const
    {
        const double y = exact(x, g, b);
        if constexpr (sizeof(YT) == 2)
            return f32_for_bf16(y);
        else
            return (float)y;
    }
    // E values in place: for bf16, the plain float roundings first and the
    // halfway-point check of f32_for_bf16 only for a chunk that has a float
    // on a bf16 halfway point (one branch per chunk, rarely taken).
    template <int E>
    __device__ void chunk(float* v, const float* g, const float* b) const
    {
        double y[E];
#pragma unroll
        for (int i = 0; i < E; ++i)
            y[i] = exact(v[i], g[i], b[i]);
        if constexpr (sizeof(YT) == 2) {
            bool half = false;
#pragma unroll
            for (int i = 0; i < E; ++i) {
                v[i] = (float)y[i];
                half |= (__float_as_uint(v[i]) & 0xFFFFu) == 0x8000u;
            }
            if (half) {
#pragma unroll
                for (int i = 0; i < E; ++i)
                    v[i] = f32_for_bf16(y[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < E; ++i)
                v[i] = (float)y[i];
        }
    }
};

// The map on E values x of columns j0.. (in place), with their weights.
template <class YT, int E, bool VEC>
__device__ __forceinline__ void ln_affine(float* v, const LnMap<YT>& map, const Weights& g,
                                          const Weights& b, int64_t j0, int64_t cols)
{
    float gw[E], bw[E];
    load_weights<E, VEC>(g, j0, cols, gw);
    load_weights<E, VEC>(b, j0, cols, bw);
    map.template chunk<E>(v, gw, bw);
}

__device__ __forceinline__ double rstd_of(double m2, int64_t n, float eps)
{
    const double var = (m2 > 0.0 ? m2 : 0.0) / (double)n;
    return 1.0 / sqrt(var + (double)eps);
}

// Shifted sums (s1 = sum (x - K), s2 = sum (x - K)^2) to (mean, rstd).
__device__ __forceinline__ LnRow row_from_shifted(double K, double s1, double s2, int64_t n,
                                                  float eps)
{
    const double dn = (double)n;
    return LnRow{K + s1 / dn, rstd_of(s2 - s1 * (s1 / dn), n, eps)};
}

// Per-row statistics written by every thread of a persistent row loop (the
// same bits to one address): buffer stores whose range is empty for a NULL
// output, so no store of the loop sits behind a branch and the prefetch's
// memory-counter waits count a fixed number of them.
struct StatsOut {
    __amdgpu_buffer_rsrc_t m, s;
    __device__ StatsOut(float* mean_out, float* rstd_out, int64_t rows)
        : m(__builtin_amdgcn_make_buffer_rsrc(mean_out, 0, mean_out ? (int)(rows * 4) : 0,
                                              kBufferWord3)),
          s(__builtin_amdgcn_make_buffer_rsrc(rstd_out, 0, rstd_out ? (int)(rows * 4) : 0,
                                              kBufferWord3))
    {
    }
    __device__ void write(int64_t r, const LnRow& st) const
    {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((float)st.mean), m, (int)(r * 4), 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((float)st.rstd), s, (int)(r * 4), 0, 0);
    }
};

__device__ __forceinline__ void write_stats(float* mean_out, float* rstd_out, int64_t r,
                                            const LnRow& st)
{
    if (mean_out)
        mean_out[r] = (float)st.mean;
    if (rstd_out)
        rstd_out[r] = (float)st.rstd;
}

// The weights of a thread's NCH chunks of E columns as raw pieces of 2E bytes
// (a bf16 chunk; a float chunk is two pieces, a bf16 one reads its piece
// twice).  Chunks past the row end load chunk 0 and are never stored.  No
// branch depends on a loaded value, so all the loads go out together and the
// unpack, later, waits for nothing else.
template <int NCH, int NT, int E>
struct RawWeights {
    using Piece = typename std::conditional<E == 8, uint4, uint2>::type;
    Piece lo[NCH], hi[NCH];
    __device__ void load(const Weights& w, int64_t cols)
    {
        if (!w.p)
            return;
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            int64_t j0 = ((int64_t)threadIdx.x + (int64_t)k * NT) * E;
            j0 = j0 < cols ? j0 : 0;
            const Piece* q = reinterpret_cast<const Piece*>(static_cast<const char*>(w.p) +
                                                            j0 * (w.bf16 ? 2 : 4));
            lo[k] = q[0];
            hi[k] = q[w.bf16 ? 0 : 1];
        }
    }
    __device__ void unpack(const Weights& w, float* o) const
    {
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            float* ok = o + k * E;
            if (!w.p) {
#pragma unroll
                for (int i = 0; i < E; ++i)
                    ok[i] = w.dflt;
            } else if (w.bf16) {
                const uint32_t* u = reinterpret_cast<const uint32_t*>(&lo[k]);
#pragma unroll
                for (int i = 0; i < E / 2; ++i) {
                    ok[2 * i] = bf16_lo(u[i]);
                    ok[2 * i + 1] = bf16_hi(u[i]);
                }
            } else {
                const uint32_t* u0 = reinterpret_cast<const uint32_t*>(&lo[k]);
                const uint32_t* u1 = reinterpret_cast<const uint32_t*>(&hi[k]);
#pragma unroll
                for (int i = 0; i < E / 2; ++i) {
                    ok[i] = __uint_as_float(u0[i]);
                    ok[E / 2 + i] = __uint_as_float(u1[i]);
                }
            }
        }
    }
};

// ------------------------------------------------ block tier, row in registers
// One row at a time per workgroup; the thread's chunks are k = 0 .. NCH-1 at
// columns (threadIdx.x + k * NT) * E.  `valid(k, i)` says whether element i
// of chunk k lies in the row; invalid elements hold 0 and are left out.
// *e: one more element of the row held by this thread (a misaligned row's
// head element) when has_e; else unused.  The values stay as they are: the
// sum of squared deviations takes x - mean in double, element by element.
// CHUNKWISE: validity is per chunk (valid(k, 0) speaks for the chunk), so
// each chunk's squared deviations are summed unconditionally and the chunk
// is kept or dropped once.
template <int NCH, int E, int NT, bool CHUNKWISE = false, class Valid>
__device__ __forceinline__ LnRow row_stats_in_registers(const float* v, int64_t cols, float eps,
                                                        double* slot_a, double* slot_b,
                                                        Valid valid, const float* e = nullptr,
                                                        bool has_e = false)
{
    double s = 0.0;  // invalid elements hold 0
#pragma unroll
    for (int i = 0; i < NCH * E; ++i)
        s += (double)v[i];
    if (has_e)
        s += (double)*e;
    const double mean = block_reduce<SumF32, NT>(s, slot_a) / (double)cols;
    double q = 0.0;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        if constexpr (CHUNKWISE) {
            double qk = 0.0;
#pragma unroll
            for (int i = 0; i < E; ++i) {
                const double d = (double)v[k * E + i] - mean;
                qk = __builtin_fma(d, d, qk);
            }
            q = valid(k, 0) ? q + qk : q;
        } else {
#pragma unroll
            for (int i = 0; i < E; ++i) {
                const double d = (double)v[k * E + i] - mean;
                q = valid(k, i) ? __builtin_fma(d, d, q) : q;
            }
        }
    }
    if (has_e) {
        const double d = (double)*e - mean;
        q = __builtin_fma(d, d, q);
    }
    const double Q = block_reduce<SumF32, NT>(q, slot_b);
    return LnRow{mean, rstd_of(Q, cols, eps)};
}

}  // namespace

// One row from its raw chunks; gw / bw hold this thread's gamma / beta
// (AFF), loaded once per workgroup.
template <class XT, class YT, int NCH, int NT, bool EXACT, bool AFF>
__device__ __forceinline__ void ln_row_from_chunks(const uint4* raw, YT* yr, int64_t r,
                                                   int64_t cols, float eps, const float* gw,
                                                   const float* bw, const StatsOut& so,
                                                   double* slot_a, double* slot_b)
{
    constexpr int E = XIn<XT>::kChunk;
    float v[NCH * E];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int64_t j0 = ((int64_t)threadIdx.x + (int64_t)k * NT) * E;
        if (EXACT || j0 < cols) {
            unpack_chunk<XT>(raw[k], v + k * E);
        } else {
#pragma unroll
            for (int i = 0; i < E; ++i)
                v[k * E + i] = 0.0f;
        }
    }
    const LnRow st = row_stats_in_registers<NCH, E, NT, true>(
        v, cols, eps, slot_a, slot_b, [&](int k, int) {
            return EXACT || ((int64_t)threadIdx.x + (int64_t)k * NT) * E < cols;
        });
    so.write(r, st);
    const LnMap<YT> map{st.mean, st.rstd};
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        if constexpr (AFF) {
            // the weights pass through an empty asm per row, so that their
            // conversions to double are not hoisted out of the row loop
            // (that kept 2 x NCH x E doubles live: spills at 512 threads)
            float gl[E], bl[E];
#pragma unroll
            for (int i = 0; i < E; ++i) {
                gl[i] = gw[k * E + i];
                bl[i] = bw[k * E + i];
                __asm__ volatile("" : "+v"(gl[i]), "+v"(bl[i]));
            }
            map.template chunk<E>(v + k * E, gl, bl);
        } else {
            float ones[E], zeros[E];
#pragma unroll
            for (int i = 0; i < E; ++i) {
                ones[i] = 1.0f;
                zeros[i] = 0.0f;
            }
            map.template chunk<E>(v + k * E, ones, zeros);
        }
        if constexpr (EXACT)
            YOut<YT>::template chunk<E>(yr + ((int64_t)threadIdx.x + (int64_t)k * NT) * E, v + k * E);
    }
    if constexpr (!EXACT)  // chunks past the row go past the buffer range: dropped
        store_row_peeled<YT, E, NCH, NT, false>(yr, cols, 0, cols, -1, v, 0.0f, 0);
}

// Persistent rows (persistent_rows: one-row prefetch, two register buffers).
// A thread's columns are the same in every row, so its gamma / beta are loaded
// into registers once: issued before the first row's loads, unpacked after
// the first two rows' loads are out.  Rows are whole 16-byte chunks, 16-byte
// aligned.
template <class XT, class YT, int NCH, int NT, bool EXACT, bool AFF>
__global__ __launch_bounds__(NT) void k_layernorm_rows_pf(
    const XT* __restrict__ x, YT* __restrict__ y, Weights g, Weights b, float* mean_out,
    float* rstd_out, int64_t rows, int64_t cols, int64_t ldx, int64_t ldy, float eps)
{
    constexpr int E = XIn<XT>::kChunk;
    __shared__ double slot[2][NT / kWave];
    if ((int64_t)blockIdx.x >= rows)
        return;
    const StatsOut so(mean_out, rstd_out, rows);
    float gw[AFF ? NCH * E : 1], bw[AFF ? NCH * E : 1];
    RawWeights<AFF ? NCH : 1, NT, E> graw, braw;
    if constexpr (AFF) {
        graw.load(g, cols);
        braw.load(b, cols);
    }
    persistent_rows<RowBuf<NCH>>(
        blockIdx.x, gridDim.x, rows,
        [&](int64_t r, bool live, RowBuf<NCH>& buf) {
            load_row_raw<NCH, NT>(x + r * ldx, live ? cols * (int64_t)sizeof(XT) : 0, buf.c);
        },
        [&] {
            if constexpr (AFF) {
                graw.unpack(g, gw);
                braw.unpack(b, bw);
            }
        },
        [&](const RowBuf<NCH>& buf, int64_t r, int) {
            ln_row_from_chunks<XT, YT, NCH, NT, EXACT, AFF>(buf.c, y + r * ldy, r, cols, eps, gw,
                                                            bw, so, slot[0], slot[1]);
        });
}

// Persistent rows at any alignment and any column count (rows that do not
// all start 16-byte aligned or do not end on a chunk): the softmax's row
// layout (load_row_peeled: each row's body from its first 16-byte boundary
// in chunk slots rotated onto 128-byte lines, one head or tail element per
// thread).  A thread's columns then move with the row's phase, so gamma and
// beta are read per row at the body's columns.  LDSW: the workgroup first
// copies them, as float, into LDS, column c's (gamma, beta) pair at pair
// c + c / E -- one pad pair after every E columns, so that the lanes of a
// chunk read (E columns apart) fall in distinct banks -- and each row reads
// its columns there, one 8-byte read per column; else from global memory
// (whole 16-byte words at any element alignment; every row reads the same
// vectors, which stay in the caches).  AFF false: the call has neither
// gamma nor beta, and the kernel holds no weight code.
template <class XT, class YT, int NCH, int NT, bool LDSW, bool AFF>
__global__ __launch_bounds__(NT) void k_layernorm_rows_peel(
    const XT* __restrict__ x, YT* __restrict__ y, Weights g, Weights b, float* mean_out,
    float* rstd_out, int64_t rows, int64_t cols, int64_t ldx, int64_t ldy, float eps)
{
    constexpr int E = XIn<XT>::kChunk;
    __shared__ double slot[2][NT / kWave];
    extern __shared__ float2 ldsw[];
    if ((int64_t)blockIdx.x >= rows)
        return;
    const StatsOut so(mean_out, rstd_out, rows);
    if constexpr (LDSW) {
        for (uint32_t j = threadIdx.x; j < (uint32_t)cols; j += NT) {
            ldsw[j + j / E] = make_float2(weight_one(g, j), weight_one(b, j));
        }
        __syncthreads();
    }
    persistent_rows<RowBuf<NCH>>(
        blockIdx.x, gridDim.x, rows,
        [&](int64_t r, bool live, RowBuf<NCH>& buf) {
            load_row_peeled<XT, NCH, NT>(x + r * ldx, cols, live, buf);
        },
        [] {},
        [&](const RowBuf<NCH>& buf, int64_t r, int) {
            const XT* xr = x + r * ldx;
            const PeelGeom<XT> pg(xr, cols);
            const int q = line_phase(xr + pg.h);  // as the row's loads
            bool ok[NCH];  // the slot holds a chunk of the row's body
            float gw[NCH * E], bw[NCH * E];
            const int64_t we = pg.idx >= 0 ? pg.idx : 0;
            float ge, be;
#pragma unroll
            for (int k = 0; k < NCH; ++k)
                ok[k] = (int64_t)slot_chunk<NCH, NT, true>(k, q) * E < pg.nbe;
            if constexpr (!AFF) {
                // no gamma or beta: 1 and 0, and no weight code in the kernel
                // (the dispatch over weight types and alignments, compiled in
                // and skipped, had cost 13 us at [16384, 4095])
                (void)we;
#pragma unroll
                for (int i = 0; i < NCH * E; ++i) {
                    gw[i] = 1.0f;
                    bw[i] = 0.0f;
                }
                ge = 1.0f;
                be = 0.0f;
            } else if constexpr (!LDSW) {
                // the row's weights first, so that their loads are in flight
                // while the statistics are formed
                const Weights gh = shifted(g, pg.h), bh = shifted(b, pg.h);
#pragma unroll
                for (int k = 0; k < NCH; ++k) {
                    // slots past the body take chunk 0's weights (never stored)
                    const int64_t j0 = ok[k] ? (int64_t)slot_chunk<NCH, NT, true>(k, q) * E : 0;
                    load_weights<E, true>(gh, j0, pg.nbe, gw + k * E);
                    load_weights<E, true>(bh, j0, pg.nbe, bw + k * E);
                }
                ge = weight_one(g, we);
                be = weight_one(b, we);
            }
            float v[NCH * E];
#pragma unroll
            for (int k = 0; k < NCH; ++k) {
                if (ok[k]) {
                    unpack_chunk<XT>(buf.c[k], v + k * E);
                } else {
#pragma unroll
                    for (int i = 0; i < E; ++i)
                        v[k * E + i] = 0.0f;
                }
            }
            const bool has_e = pg.idx >= 0;
            float e = has_e ? buf.e : 0.0f;
            const LnRow st = row_stats_in_registers<NCH, E, NT, true>(
                v, cols, eps, slot[0], slot[1], [&](int k, int) { return ok[k]; }, &e, has_e);
            so.write(r, st);
            if constexpr (LDSW) {
                // columns h + j0 + i of the body's chunks (j0 = m E): pairs
                // h + j0 + m + i, plus one where h + i passes E (the same
                // for every chunk of the row); slots past the body read
                // from pair 0 (never stored); then the head or tail element
                const uint32_t h = (uint32_t)pg.h;
#pragma unroll
                for (int k = 0; k < NCH; ++k) {
                    const uint32_t m = (uint32_t)slot_chunk<NCH, NT, true>(k, q);
                    const uint32_t w0 = ok[k] ? h + m * (E + 1) : 0u;
#pragma unroll
                    for (int i = 0; i < E; ++i) {
                        const uint32_t w = w0 + i + (h + i >= (uint32_t)E ? 1u : 0u);
                        const float2 gb = ldsw[w];
                        gw[k * E + i] = gb.x;
                        bw[k * E + i] = gb.y;
                    }
                }
                const uint32_t wc = (uint32_t)we + (uint32_t)we / E;
                const float2 gbe = ldsw[wc];
                ge = gbe.x;
                be = gbe.y;
            }
            const LnMap<YT> map{st.mean, st.rstd};
#pragma unroll
            for (int k = 0; k < NCH; ++k)
                map.template chunk<E>(v + k * E, gw + k * E, bw + k * E);
            const float ev = map(e, ge, be);
            store_row_peeled<YT, E, NCH, NT, true>(y + r * ldy, cols, pg.h, pg.nbe,
                                                   has_e ? pg.idx : -1, v, ev, q);
        });
}

// Any alignment and any column count (masked chunks), one row per workgroup
// at a time, the row in registers.  VEC (element-aligned x and y): each row's
// body from its first 16-byte boundary in chunks (the tail chunk element by
// element), the head (h < E elements) one element to each of the first
// threads; y's chunks are stored whole, and gamma / beta loaded whole, where
// they are aligned at the body's first column.
template <class XT, class YT, int NCH, bool VEC, int NT>
__global__ __launch_bounds__(NT) void k_layernorm_block(
    const XT* __restrict__ x, YT* __restrict__ y, Weights g, Weights b, float* mean_out,
    float* rstd_out, int64_t rows, int64_t cols, int64_t ldx, int64_t ldy, float eps)
{
    constexpr int E = VEC ? XIn<XT>::kChunk : 1;
    __shared__ double slot[2][NT / kWave];
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const XT* xr0 = x + r * ldx;
        YT* yr0 = y + r * ldy;
        const int64_t h = VEC ? head_elems(xr0, cols) : 0;
        const XT* xr = xr0 + h;
        YT* yr = yr0 + h;
        const int64_t cb = cols - h;
        const Weights gh = shifted(g, h), bh = shifted(b, h);
        const bool yvec = VEC && chunk_aligned<YT, E>(yr);
        float v[NCH * E];
#pragma unroll
        for (int k = 0; k < NCH; ++k)
            load_padded<XT, E, VEC>(xr, ((int64_t)threadIdx.x + (int64_t)k * NT) * E, cb,
                                    v + k * E, 0.0f);
        const bool has_e = (int64_t)threadIdx.x < h;
        float e = has_e ? XIn<XT>::one(xr0 + threadIdx.x) : 0.0f;
        const LnRow st = row_stats_in_registers<NCH, E, NT>(
            v, cols, eps, slot[0], slot[1],
            [&](int k, int i) { return ((int64_t)threadIdx.x + (int64_t)k * NT) * E + i < cb; },
            &e, has_e);
        if (threadIdx.x == 0)
            write_stats(mean_out, rstd_out, r, st);
        const LnMap<YT> map{st.mean, st.rstd};
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int64_t j0 = ((int64_t)threadIdx.x + (int64_t)k * NT) * E;
            ln_affine<YT, E, VEC>(v + k * E, map, gh, bh, j0, cb);
            store_masked_rt<YT, E>(yr, j0, cb, v + k * E, yvec);
        }
        if (has_e)
            YOut<YT>::one(yr0 + threadIdx.x,
                          map(e, weight_one(g, threadIdx.x), weight_one(b, threadIdx.x)));
    }
}

// ---------------------------------------- block tier, streaming long rows
// Statistics read with shifted sums (padding with K adds nothing), then a
// second read for the map.
template <class XT, class YT, bool VEC, int NT>
__global__ __launch_bounds__(NT) void k_layernorm_stream(
    const XT* __restrict__ x, YT* __restrict__ y, Weights g, Weights b, float* mean_out,
    float* rstd_out, int64_t rows, int64_t cols, int64_t ldx, int64_t ldy, float eps)
{
    constexpr int E = VEC ? XIn<XT>::kChunk : 1;
    __shared__ double slot[2][NT / kWave];
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        // VEC: the body from the row's first 16-byte boundary in chunks, the
        // head (h < E elements) one element to each of the first threads
        const XT* xr0 = x + r * ldx;
        YT* yr0 = y + r * ldy;
        const int64_t h = VEC ? head_elems(xr0, cols) : 0;
        const XT* xr = xr0 + h;
        YT* yr = yr0 + h;
        const int64_t cb = cols - h;
        const Weights gh = shifted(g, h), bh = shifted(b, h);
        const bool yvec = VEC && chunk_aligned<YT, E>(yr);
        const bool has_e = (int64_t)threadIdx.x < h;
        const float kf = XIn<XT>::one(xr0);
        const double K = (double)kf;
        double s1 = 0.0, s2 = 0.0;
        if (has_e) {
            const double d = (double)XIn<XT>::one(xr0 + threadIdx.x) - K;
            s1 = d;
            s2 = d * d;
        }
        for (int64_t j0 = (int64_t)threadIdx.x * E; j0 < cb; j0 += (int64_t)NT * E) {
            float v[E];
            load_padded<XT, E, VEC>(xr, j0, cb, v, kf);
#pragma unroll
            for (int i = 0; i < E; ++i) {
                const double d = (double)v[i] - K;
                s1 += d;
                s2 = __builtin_fma(d, d, s2);
            }
        }
        const double S1 = block_reduce<SumF32, NT>(s1, slot[0]);
        const double S2 = block_reduce<SumF32, NT>(s2, slot[1]);
        const LnRow st = row_from_shifted(K, S1, S2, cols, eps);
        if (threadIdx.x == 0)
            write_stats(mean_out, rstd_out, r, st);
        const LnMap<YT> map{st.mean, st.rstd};
        if (has_e)
            YOut<YT>::one(yr0 + threadIdx.x, map(XIn<XT>::one(xr0 + threadIdx.x),
                                                 weight_one(g, threadIdx.x),
                                                 weight_one(b, threadIdx.x)));
        for (int64_t j0 = (int64_t)threadIdx.x * E; j0 < cb; j0 += (int64_t)NT * E) {
            float v[E];
            load_padded<XT, E, VEC>(xr, j0, cb, v, 0.0f);
            ln_affine<YT, E, VEC>(v, map, gh, bh, j0, cb);
            store_masked_rt<YT, E>(yr, j0, cb, v, yvec);
        }
        __syncthreads();  // slot reuse by the next row
    }
}

// -------------------------------------------------------------- wave tier
// S lanes per row, one chunk per lane (S * E >= cols), kWaveRowGroups row
// groups per wavefront step.
template <class XT, class YT, bool VEC, int S>
__global__ __launch_bounds__(kBlockThreads) void k_layernorm_wave(
    const XT* __restrict__ x, YT* __restrict__ y, Weights g, Weights b, float* mean_out,
    float* rstd_out, int64_t rows, int64_t cols, int64_t ldx, int64_t ldy, float eps)
{
    constexpr int E = VEC ? XIn<XT>::kChunk : 1;
    constexpr int RPG = kWave / S;
    constexpr int U = kWaveRowGroups;
    const int lane = lane_id();
    const int seg = lane / S;
    const int64_t j0 = (int64_t)(lane % S) * E;
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
    // the weights of this lane's columns are the same for every row
    float gw[E], bw[E];
    load_weights<E, VEC>(g, j0, cols, gw);
    load_weights<E, VEC>(b, j0, cols, bw);
    for (int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
         w * RPG * U < rows; w += nwaves) {
        const int64_t row0 = w * RPG * U;
        float v[U][E];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t r = row0 + (int64_t)u * RPG + seg;
            if (r < rows) {
                load_padded<XT, E, VEC>(x + r * ldx, j0, cols, v[u], 0.0f);
            } else {
#pragma unroll
                for (int i = 0; i < E; ++i)
                    v[u][i] = 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            double s = 0.0;
#pragma unroll
            for (int i = 0; i < E; ++i)
                s += (double)v[u][i];
            const double mean = segment_reduce<SumF32, S>(s) / (double)cols;
            double q = 0.0;
#pragma unroll
            for (int i = 0; i < E; ++i) {
                const double d = (double)v[u][i] - mean;
                q = j0 + i < cols ? __builtin_fma(d, d, q) : q;
            }
            const double Q = segment_reduce<SumF32, S>(q);
            const LnRow st{mean, rstd_of(Q, cols, eps)};
            const LnMap<YT> map{st.mean, st.rstd};
            const int64_t r = row0 + (int64_t)u * RPG + seg;
            if (r < rows) {
                if (lane % S == 0)
                    write_stats(mean_out, rstd_out, r, st);
                map.template chunk<E>(v[u], gw, bw);
                store_masked<YT, E, VEC>(y + r * ldy, j0, cols, v[u]);
            }
        }
    }
}

// ---------------------------------------------- tiled and serial tiers
// A thread owns R adjacent rows and walks each row three times (sum, sum of
// squared deviations, map), in double.  R == 1 is the serial tier.
template <class XT, class YT, int R>
__global__ __launch_bounds__(kBlockThreads) void k_layernorm_tiled(
    const XT* __restrict__ x, YT* __restrict__ y, Weights g, Weights b, float* mean_out,
    float* rstd_out, int64_t rows, int64_t cols, int64_t ldx, int64_t ldy, float eps)
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
            double s = 0.0;
            for (int64_t j = 0; j < cols; ++j)
                s += (double)XIn<XT>::one(xr + j);
            const double mean = s / (double)cols;
            double q = 0.0;
            for (int64_t j = 0; j < cols; ++j) {
                const double d = (double)XIn<XT>::one(xr + j) - mean;
                q = __builtin_fma(d, d, q);
            }
            const LnRow st{mean, rstd_of(q, cols, eps)};
            write_stats(mean_out, rstd_out, r, st);
            const LnMap<YT> map{st.mean, st.rstd};
            for (int64_t j = 0; j < cols; ++j)
                YOut<YT>::one(yr + j, map(XIn<XT>::one(xr + j), weight_one(g, j), weight_one(b, j)));
        }
    }
}

// ----------------------------------------------------------- split-K tier
// G workgroups per row own tiles g, g + G, ... (kLnSplitKUnroll 16-byte
// chunks per thread).  Statistics pass: workgroup (r, g) stores its shifted
// sums (s1, s2) to part[(r * G + g) * 2 + {0, 1}].  Map pass, tile-major: a
// work item is one column tile of a chunk of rows; its workgroup sums each
// of the chunk's rows' G pairs over a fixed tree (the same in every
// workgroup: "cluster_allreduce", description, the all-gather variant),
// loads the tile's gamma / beta once and maps that tile of every row of the
// chunk, the next row's tile in flight.

// Shifted sums of one tile's N values in double, into 4 interleaved
// accumulator pairs (element i goes to pair i % 4; fixed order).
template <int N, class R>
__device__ __forceinline__ void ln_fold_raw(const R& raw, double K, double* s1, double* s2)
{
    float v[N];
    raw.unpack(v);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const double d = (double)v[i] - K;
        s1[i & 3] += d;
        s2[i & 3] = __builtin_fma(d, d, s2[i & 3]);
    }
}

template <class XT, bool VEC>
__global__ __launch_bounds__(kBlockThreads) void k_layernorm_splitk_stats(
    const XT* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, int32_t G,
    double* __restrict__ part)
{
    constexpr int E = VEC ? XIn<XT>::kChunk : 1;
    constexpr int U = kLnSplitKUnroll;
    constexpr int N = U * E;
    constexpr int64_t kTile = (int64_t)N * kBlockThreads;
    __shared__ double slot[2][kWavesPerBlock];
    const int64_t total = rows * G;
    for (int64_t blk = blockIdx.x; blk < total; blk += gridDim.x) {
        const int64_t r = blk / G;
        const int32_t gi = (int32_t)(blk - r * G);
        // Tiles cover the row's body from its first 16-byte boundary (VEC);
        // workgroup 0 also takes the head, h < E elements, one element to
        // each of its first threads.
        const XT* xr0 = x + r * ldx;
        const int64_t h = VEC ? head_elems(xr0, cols) : 0;
        const XT* xr = xr0 + h;
        const int64_t cb = cols - h;
        const int64_t ntiles = ceil_div(cb, kTile);
        const int64_t nfull = cb / kTile;
        const float kf = XIn<XT>::one(xr0);
        const double K = (double)kf;
        double s1[4] = {0.0, 0.0, 0.0, 0.0}, s2[4] = {0.0, 0.0, 0.0, 0.0};
        if (VEC && gi == 0 && (int64_t)threadIdx.x < h) {
            const double d = (double)XIn<XT>::one(xr0 + threadIdx.x) - K;
            s1[0] = d;
            s2[0] = d * d;
        }
        // whole tiles, double-buffered (next tile's loads issued before the
        // current one is folded; trip counts uniform over the workgroup)
        const int64_t n = gi < nfull ? (nfull - 1 - gi) / G + 1 : 0;
        if (n > 0) {
            const int64_t step = (int64_t)G * kTile;
            const XT* tp = xr + (int64_t)gi * kTile;
            RawTile<XT, VEC, U> A, B;
            A.load(tp);
            int64_t k = 0;
            for (; k + 2 < n; k += 2) {
                B.load(tp + (k + 1) * step);
                __builtin_amdgcn_sched_barrier(0);
                ln_fold_raw<N>(A, K, s1, s2);
                A.load(tp + (k + 2) * step);
                __builtin_amdgcn_sched_barrier(0);
                ln_fold_raw<N>(B, K, s1, s2);
            }
            if (k + 1 < n) {
                B.load(tp + (k + 1) * step);
                __builtin_amdgcn_sched_barrier(0);
                ln_fold_raw<N>(A, K, s1, s2);
                ln_fold_raw<N>(B, K, s1, s2);
            } else {
                ln_fold_raw<N>(A, K, s1, s2);
            }
        }
        for (int64_t t = gi + n * G; t < ntiles; t += G) {  // ragged tile, padded with K
            float v[N];
            load_tile_padded<XT, E, VEC, U>(xr, t * kTile, cb, v, kf);
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const double d = (double)v[i] - K;
                s1[i & 3] += d;
                s2[i & 3] = __builtin_fma(d, d, s2[i & 3]);
            }
        }
        const double t1 = (s1[0] + s1[1]) + (s1[2] + s1[3]);
        const double t2 = (s2[0] + s2[1]) + (s2[2] + s2[3]);
        const double S1 = block_reduce<SumF32, kBlockThreads>(t1, slot[0]);
        const double S2 = block_reduce<SumF32, kBlockThreads>(t2, slot[1]);
        if (threadIdx.x == 0) {
            part[(r * G + gi) * 2] = S1;
            part[(r * G + gi) * 2 + 1] = S2;
        }
        __syncthreads();  // slot reuse by the next (row, slice)
    }
}

// Row statistics of rows r0 .. r0+nr-1 (nr <= kBlockThreads) from their G
// pairs, into LDS.  TPR = threads per row (a power of two, at most 64):
// lane l of a row sums the pairs g = l, l + TPR, ... in order, then the TPR
// lane sums are added over the fixed DPP tree.
template <class XT>
__device__ __forceinline__ void ln_row_stats_lds(const XT* x, int64_t ldx, int64_t r0, int nr,
                                                 int64_t cols, float eps, int32_t G,
                                                 const double* part, double* smean, double* srstd)
{
    int tpr = 1;
    while (tpr < 64 && tpr * 2 * nr <= kBlockThreads)
        tpr *= 2;
    const int row = (int)threadIdx.x / tpr;
    const int lane = (int)threadIdx.x % tpr;
    double s1 = 0.0, s2 = 0.0;
    if (row < nr) {
        const double* pr = part + (r0 + row) * (int64_t)G * 2;
        for (int32_t g = lane; g < G; g += tpr) {
            s1 += pr[g * 2];
            s2 += pr[g * 2 + 1];
        }
    }
    double S1 = s1, S2 = s2;
    switch (tpr) {
    case 2: S1 = segment_reduce<SumF32, 2>(s1); S2 = segment_reduce<SumF32, 2>(s2); break;
    case 4: S1 = segment_reduce<SumF32, 4>(s1); S2 = segment_reduce<SumF32, 4>(s2); break;
    case 8: S1 = segment_reduce<SumF32, 8>(s1); S2 = segment_reduce<SumF32, 8>(s2); break;
    case 16: S1 = segment_reduce<SumF32, 16>(s1); S2 = segment_reduce<SumF32, 16>(s2); break;
    case 32: S1 = segment_reduce<SumF32, 32>(s1); S2 = segment_reduce<SumF32, 32>(s2); break;
    case 64: S1 = segment_reduce<SumF32, 64>(s1); S2 = segment_reduce<SumF32, 64>(s2); break;
    default: break;
    }
    if (row < nr && lane == 0) {
        const double K = (double)XIn<XT>::one(x + (r0 + row) * ldx);
        const LnRow st = row_from_shifted(K, S1, S2, cols, eps);
        smean[row] = st.mean;
        srstd[row] = st.rstd;
    }
}

// Work item b of the map pass: column tile t = b % ntiles of the row chunk
// b / ntiles (rows chunk * rc .. + rc - 1, rc <= kBlockThreads).  The
// workgroup of tile 0 of a chunk writes that chunk's mean / rstd.  VEC: every
// row of x starts at the same offset from a 16-byte boundary (the host checks
// the row stride), so the tiles of all rows cover the same columns from the
// first row's head h on, and share one load of their gamma / beta; the
// workgroup of tile 0 also maps the head columns of its rows.
template <class XT, class YT, bool VEC, bool AFF>
__global__ __launch_bounds__(kBlockThreads) void k_layernorm_splitk_map(
    const XT* __restrict__ x, YT* __restrict__ y, Weights g, Weights b, float* mean_out,
    float* rstd_out, int64_t rows, int64_t cols, int64_t ldx, int64_t ldy, float eps, int32_t G,
    const double* __restrict__ part, int32_t rc)
{
    constexpr int E = VEC ? XIn<XT>::kChunk : 1;
    constexpr int U = kLnSplitKUnroll;
    constexpr int N = U * E;
    constexpr int64_t kTile = (int64_t)N * kBlockThreads;
    __shared__ double smean[kBlockThreads];
    __shared__ double srstd[kBlockThreads];
    const int64_t h = VEC ? head_elems(x, cols) : 0;
    const int64_t cb = cols - h;
    const Weights gh = shifted(g, h), bh = shifted(b, h);
    // at least one tile, so that the work items of tile 0 also map the head
    // when it is the whole row (a row shorter than its offset to the next
    // 16-byte boundary: the tile itself is then empty)
    const int64_t ntiles = cb > 0 ? ceil_div(cb, kTile) : 1;
    const int64_t nfull = cb / kTile;
    const int64_t nchunk = ceil_div(rows, (int64_t)rc);
    int64_t have = -1;  // row chunk whose statistics are in LDS
    for (int64_t item = blockIdx.x; item < ntiles * nchunk; item += gridDim.x) {
        const int64_t chunk = item / ntiles;
        const int64_t t = item - chunk * ntiles;
        const int64_t r0 = chunk * rc;
        const int nr = (int)(rows - r0 < rc ? rows - r0 : rc);
        if (chunk != have) {  // uniform over the workgroup
            __syncthreads();  // the previous chunk is done with the LDS statistics
            ln_row_stats_lds<XT>(x, ldx, r0, nr, cols, eps, G, part, smean, srstd);
            __syncthreads();
            have = chunk;
        }
        if (t == 0 && (int)threadIdx.x < nr)
            write_stats(mean_out, rstd_out, r0 + threadIdx.x,
                        LnRow{smean[threadIdx.x], srstd[threadIdx.x]});
        if (VEC && t == 0 && (int64_t)threadIdx.x < h) {  // head columns of the chunk's rows
            const float gj = weight_one(g, threadIdx.x), bj = weight_one(b, threadIdx.x);
            for (int i = 0; i < nr; ++i) {
                const LnMap<YT> map{smean[i], srstd[i]};
                YOut<YT>::one(y + (r0 + i) * ldy + threadIdx.x,
                              map(XIn<XT>::one(x + (r0 + i) * ldx + threadIdx.x), gj, bj));
            }
        }
        {
            float gw[AFF ? N : 1], bw[AFF ? N : 1];
            if constexpr (AFF) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t j0 = t * kTile + ((int64_t)u * kBlockThreads + threadIdx.x) * E;
                    load_weights<E, VEC>(gh, j0, cb, gw + u * E);
                    load_weights<E, VEC>(bh, j0, cb, bw + u * E);
                }
            }
            if (t < nfull) {
                // whole tiles: row r's tile in A while row r+1's loads fly
                RawTile<XT, VEC, U> A, B;
                A.load(x + r0 * ldx + h + t * kTile);
                for (int i = 0; i < nr; ++i) {
                    const int ip = i + 1 < nr ? i + 1 : i;
                    B.load(x + (r0 + ip) * ldx + h + t * kTile);
                    __builtin_amdgcn_sched_barrier(0);
                    float v[N];
                    A.unpack(v);
                    const LnMap<YT> map{smean[i], srstd[i]};
                    if constexpr (AFF) {
                        map.template chunk<N>(v, gw, bw);
                    } else {
                        float ones[N], zeros[N];
#pragma unroll
                        for (int k = 0; k < N; ++k) {
                            ones[k] = 1.0f;
                            zeros[k] = 0.0f;
                        }
                        map.template chunk<N>(v, ones, zeros);
                    }
                    YT* yt = y + (r0 + i) * ldy + h + t * kTile;
                    if (!VEC || chunk_aligned<YT, E>(yt))
                        store_tile_full<YT, E, VEC, U>(yt, v);
                    else
                        store_tile_full_rt<YT, E, U>(yt, v, false);
                    A = B;
                }
            } else {
                for (int i = 0; i < nr; ++i) {
                    float v[N];
                    load_tile_padded<XT, E, VEC, U>(x + (r0 + i) * ldx + h, t * kTile, cb, v, 0.0f);
                    const LnMap<YT> map{smean[i], srstd[i]};
                    if constexpr (AFF) {
                        map.template chunk<N>(v, gw, bw);
                    } else {
                        float ones[N], zeros[N];
#pragma unroll
                        for (int k = 0; k < N; ++k) {
                            ones[k] = 1.0f;
                            zeros[k] = 0.0f;
                        }
                        map.template chunk<N>(v, ones, zeros);
                    }
                    YT* yb = y + (r0 + i) * ldy + h;
                    store_tile_masked_rt<YT, E, U>(yb, t * kTile, cb, v,
                                                   VEC && chunk_aligned<YT, E>(yb));
                }
            }
        }
    }
}

// ---------------------------------------------------------------- launch
// Persistent grid: the plan's, lowered to the workgroups that can be resident
// at once (the kernel's occupancy times the CUs), so that no workgroup of a
// persistent grid waits for another to finish before it starts.
template <class K>
static rr_status persistent_grid(K kernel, int nt, const rr_plan& p, const LayernormLaunch& a,
                                 dim3* grid)
{
    int per_cu = 0;
    if (blocks_per_cu(kernel, nt, &per_cu) != RR_OK)
        return RR_ERR_HIP;
    const int64_t cap = (int64_t)per_cu * a.cu;
    *grid = dim3((unsigned)(p.grid < cap ? p.grid : cap));
    return RR_OK;
}

template <class XT, class YT, int NCH, int NT, bool AFF>
static rr_status launch_pf_aff(const XT* x, YT* y, const Weights& g, const Weights& b,
                               const rr_plan& p, const LayernormLaunch& a)
{
    constexpr int64_t kExactCols = (int64_t)NT * NCH * XIn<XT>::kChunk;
    const bool exact = a.cols == kExactCols;
    auto kernel = exact ? k_layernorm_rows_pf<XT, YT, NCH, NT, true, AFF>
                        : k_layernorm_rows_pf<XT, YT, NCH, NT, false, AFF>;
    dim3 grid;
    const rr_status st = persistent_grid(kernel, NT, p, a, &grid);
    if (st != RR_OK)
        return st;
    return launch_kernel(kernel, grid, dim3(NT), 0, a.stream, x, y, g, b, a.mean_out, a.rstd_out,
                         a.rows, a.cols, a.ld_x, a.ld_y, a.eps);
}

template <class XT, class YT, int NCH, int NT>
static rr_status launch_pf(const XT* x, YT* y, const Weights& g, const Weights& b,
                           const rr_plan& p, const LayernormLaunch& a)
{
    if (!(a.rows16 && a.cols % XIn<XT>::kChunk == 0)) {
        // gamma and beta (when given) through LDS when both fit: a (gamma,
        // beta) pair per column plus one pad pair per chunk, rounded up to
        // 1 KiB (the occupancy query takes the same size as the launch)
        const int64_t wbytes =
            2 * (a.cols + a.cols / XIn<XT>::kChunk + 1) * (int64_t)sizeof(float);
        const bool ldsw = (g.p || b.p) && wbytes <= kLnLdsWeightBytes;
        auto kernel = ldsw ? k_layernorm_rows_peel<XT, YT, NCH, NT, true, true>
                      : (g.p || b.p) ? k_layernorm_rows_peel<XT, YT, NCH, NT, false, true>
                                     : k_layernorm_rows_peel<XT, YT, NCH, NT, false, false>;
        const size_t lds = ldsw ? (size_t)((wbytes + 1023) / 1024 * 1024) : 0;
        int per_cu = 0;
        if (blocks_per_cu(kernel, NT, &per_cu, lds) != RR_OK)
            return RR_ERR_HIP;
        const int64_t cap = (int64_t)per_cu * a.cu;
        const dim3 grid((unsigned)(p.grid < cap ? p.grid : cap));
        return launch_kernel(kernel, grid, dim3(NT), lds, a.stream, x, y, g, b, a.mean_out,
                             a.rstd_out, a.rows, a.cols, a.ld_x, a.ld_y, a.eps);
    }
    if (g.p || b.p)
        return launch_pf_aff<XT, YT, NCH, NT, true>(x, y, g, b, p, a);
    return launch_pf_aff<XT, YT, NCH, NT, false>(x, y, g, b, p, a);
}

#define RR_LN_ARGS x, y, g, b, a.mean_out, a.rstd_out, a.rows, a.cols, a.ld_x, a.ld_y, a.eps

template <class XT, class YT, bool VEC>
static rr_status launch_block(const rr_plan& p, const XT* x, YT* y, const Weights& g,
                              const Weights& b, const LayernormLaunch& a)
{
    constexpr int NT = kBlockThreads;
    constexpr int E = VEC ? XIn<XT>::kChunk : 1;
    const dim3 grid((unsigned)p.grid), block(NT);
    const hipStream_t s = a.stream;
    const int64_t nch = ceil_div(ceil_div(a.cols, E), NT);
    if constexpr (VEC) {
        {
            // persistent rows (any alignment); the plan chose the shape and
            // sized the grid
            const RowPfShape sh = row_pf_shape(ceil_div(a.cols, E));
            if (sh.nt > 0 && sh.nt != p.block)
                return RR_ERR_TIER;  // plan and launch disagree: refuse, launch nothing
            switch (sh.nt * 16 + sh.nch) {
            case 64 * 16 + 1: return launch_pf<XT, YT, 1, 64>(x, y, g, b, p, a);
            case 64 * 16 + 2: return launch_pf<XT, YT, 2, 64>(x, y, g, b, p, a);
            case 64 * 16 + 4: return launch_pf<XT, YT, 4, 64>(x, y, g, b, p, a);
            case 128 * 16 + 4: return launch_pf<XT, YT, 4, 128>(x, y, g, b, p, a);
            case 256 * 16 + 4: return launch_pf<XT, YT, 4, 256>(x, y, g, b, p, a);
            case 512 * 16 + 4: return launch_pf<XT, YT, 4, 512>(x, y, g, b, p, a);
            default: break;  // too long for registers: stream below
            }
        }
    }
    if (nch <= 1)
        return launch_kernel(k_layernorm_block<XT, YT, 1, VEC, NT>, grid, block, 0, s, RR_LN_ARGS);
    if (nch <= 2)
        return launch_kernel(k_layernorm_block<XT, YT, 2, VEC, NT>, grid, block, 0, s, RR_LN_ARGS);
    if (nch <= 4)
        return launch_kernel(k_layernorm_block<XT, YT, 4, VEC, NT>, grid, block, 0, s, RR_LN_ARGS);
    if (nch <= kLnMaxChunks)
        return launch_kernel(k_layernorm_block<XT, YT, kLnMaxChunks, VEC, NT>, grid, block, 0, s,
                             RR_LN_ARGS);
    return launch_kernel(k_layernorm_stream<XT, YT, VEC, NT>, grid, block, 0, s, RR_LN_ARGS);
}

template <class XT, class YT, bool VEC>
static rr_status launch_wave(const rr_plan& p, const XT* x, YT* y, const Weights& g,
                             const Weights& b, const LayernormLaunch& a);
template <class XT, class YT, bool VEC>
static rr_status launch_splitk(const rr_plan& p, const XT* x, YT* y, const Weights& g,
                               const Weights& b, const LayernormLaunch& a);

// VEC (x, y, gamma and beta aligned to their element sizes): the block tier
// takes each row's body from its first 16-byte boundary in chunks (persistent
// rows only when every row starts aligned and ends on a chunk, rows16); the
// wave tier needs rows16 too, split-K rows at one offset (same_phase).
template <class XT, class YT, bool VEC>
static rr_status launch_typed(const rr_plan& p, const LayernormLaunch& a)
{
    const XT* x = static_cast<const XT*>(a.x);
    YT* y = static_cast<YT*>(a.y);
    const Weights g{a.gamma, a.w_dtype == RR_BF16, 1.0f};
    const Weights b{a.beta, a.w_dtype == RR_BF16, 0.0f};
    const dim3 grid((unsigned)(p.grid > kMaxGrid ? kMaxGrid : p.grid)), block(kBlockThreads);
    const hipStream_t s = a.stream;
    switch (p.tier) {
    case RR_TIER_BLOCK:
        return launch_block<XT, YT, VEC>(p, x, y, g, b, a);
    case RR_TIER_WAVE:
        return VEC && a.rows16 ? launch_wave<XT, YT, true>(p, x, y, g, b, a)
                               : launch_wave<XT, YT, false>(p, x, y, g, b, a);
    case RR_TIER_TILED:
        return launch_kernel(k_layernorm_tiled<XT, YT, kTiledRows>, grid, block, 0, s, RR_LN_ARGS);
    case RR_TIER_SERIAL:
        return launch_kernel(k_layernorm_tiled<XT, YT, 1>, grid, block, 0, s, RR_LN_ARGS);
    case RR_TIER_SPLITK:
        return VEC && a.same_phase ? launch_splitk<XT, YT, true>(p, x, y, g, b, a)
                                   : launch_splitk<XT, YT, false>(p, x, y, g, b, a);
    default:
        return RR_ERR_TIER;
    }
}

template <class XT, class YT, bool VEC>
static rr_status launch_wave(const rr_plan& p, const XT* x, YT* y, const Weights& g,
                             const Weights& b, const LayernormLaunch& a)
{
    const dim3 grid((unsigned)(p.grid > kMaxGrid ? kMaxGrid : p.grid)), block(kBlockThreads);
    const hipStream_t s = a.stream;
    switch (p.lanes_per_row) {
    case 4: return launch_kernel(k_layernorm_wave<XT, YT, VEC, 4>, grid, block, 0, s, RR_LN_ARGS);
    case 16: return launch_kernel(k_layernorm_wave<XT, YT, VEC, 16>, grid, block, 0, s, RR_LN_ARGS);
    case 64: return launch_kernel(k_layernorm_wave<XT, YT, VEC, 64>, grid, block, 0, s, RR_LN_ARGS);
    default: return RR_ERR_TIER;
    }
}

// Split-K: VEC needs every row of x at the same offset from a 16-byte
// boundary (the map pass shares one tile of gamma / beta between rows).
template <class XT, class YT, bool VEC>
static rr_status launch_splitk(const rr_plan& p, const XT* x, YT* y, const Weights& g,
                               const Weights& b, const LayernormLaunch& a)
{
    const dim3 grid((unsigned)(p.grid > kMaxGrid ? kMaxGrid : p.grid)), block(kBlockThreads);
    const hipStream_t s = a.stream;
    {
        double* part = static_cast<double*>(a.workspace);
        rr_status st = launch_kernel(k_layernorm_splitk_stats<XT, VEC>, grid, block, 0, s, x,
                                     a.rows, a.cols, a.ld_x, p.slices, part);
        if (st != RR_OK)
            return st;
        // map: work items of one column tile x a chunk of rows; chunks of at
        // least kLnMapMinRows rows (gamma / beta reuse), enough of them to give
        // 2 work items per CU, at most kSplitKHeavyBlocksPerCU workgroups per CU
        constexpr int E = VEC ? XIn<XT>::kChunk : 1;
        const int64_t ntiles = ceil_div(a.cols, (int64_t)kLnSplitKUnroll * kBlockThreads * E);
        int64_t nchunk = ceil_div((int64_t)2 * a.cu, ntiles);
        const int64_t max_chunks = ceil_div(a.rows, (int64_t)kLnMapMinRows);
        if (nchunk > max_chunks) nchunk = max_chunks;
        if (nchunk < 1) nchunk = 1;
        int64_t rc = ceil_div(a.rows, nchunk);
        if (rc > kBlockThreads) rc = kBlockThreads;
        const int64_t items = ntiles * ceil_div(a.rows, rc);
        const int64_t cap = (int64_t)kSplitKHeavyBlocksPerCU * a.cu;
        const dim3 mgrid((unsigned)(items < cap ? items : cap));
        if (g.p || b.p)
            return launch_kernel(k_layernorm_splitk_map<XT, YT, VEC, true>, mgrid, block, 0, s,
                                 RR_LN_ARGS, p.slices, (const double*)part, (int32_t)rc);
        return launch_kernel(k_layernorm_splitk_map<XT, YT, VEC, false>, mgrid, block, 0, s,
                             RR_LN_ARGS, p.slices, (const double*)part, (int32_t)rc);
    }
}

#undef RR_LN_ARGS

template <class XT, class YT>
static rr_status launch_xy(const rr_plan& p, const LayernormLaunch& a)
{
    return a.vec ? launch_typed<XT, YT, true>(p, a) : launch_typed<XT, YT, false>(p, a);
}

rr_status launch_layernorm(const rr_plan& p, const LayernormLaunch& a)
{
    const bool xb = a.x_dtype == RR_BF16, yb = a.y_dtype == RR_BF16;
    if (xb && yb) return launch_xy<uint16_t, uint16_t>(p, a);
    if (xb) return launch_xy<uint16_t, float>(p, a);
    if (yb) return launch_xy<float, uint16_t>(p, a);
    return launch_xy<float, float>(p, a);
}

}  // namespace rr
