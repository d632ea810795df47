// rr_attention.hip -- split-K attention partials on MFMA, gfx950.
//
// The producer side of the LSE merge ("fa4_splitk_reduce_scatter_write",
// per-band steps: the partial output of each partition carries its row max
// and row sum).  The keys of a head are cut into P contiguous partitions
// (partition p holds keys p*n/P .. (p+1)*n/P - 1); for every query row and
// partition the kernel writes
//   m_p = max_j s_j,  l_p = sum_j exp(s_j - m_p),
//   O_p = sum_j exp(s_j - m_p) v_j / l_p,       s_j = scale * q . k_j,
// in the merge's layout: O [P][rows][depth], m and l [P][rows] (float),
// rows = batch * heads * q_rows.  A partition with no key gets (-inf, 0, 0).
//
// This is a dense contraction, so it runs on the matrix cores
// (v_mfma_f32_32x32x16_bf16).  A workgroup of four wavefronts takes 128
// query rows (32 per wavefront) of one head and one partition and walks the
// partition's keys in stages of kAttnStageKeys, kAttnStages of them in
// flight: each stage's K and V tiles go from HBM straight into LDS (buffer
// loads with the lds modifier, non-temporal), so no registers hold data in
// transit.  Per stage a wavefront forms S^T = K Q^T (keys x its 32 queries)
// and, after the online max / sum update, O^T += V^T P^T; in both products a
// lane owns one query column of the accumulator, so the rescale of O and the
// row statistics stay inside the lane.  Q stays in registers as the B
// operand for the whole walk.  At the end O goes out through LDS as whole
// 128-byte lines.  Depth 128 runs 3 stages in flight at 3 workgroups per CU
// (the LDS read addresses are formed in every stage rather than held in
// registers, which keeps the kernel under the 168 registers that allows);
// depth 64 runs 4 stages.
//
// The one-launch variant (FUSED) adds the merge: the last of a query tile's
// P workgroups to take the tile's ticket folds the P partials, which the
// workgroups wrote to a workspace through the device-coherent level, with
// the merge's own per-row functions.
//
// Precision: q.k and P V accumulate in float32 inside the MFMA; P is rounded
// to bf16 as the MFMA operand (the usual flash-attention practice); the
// running max and sum are float32.  Everything is in a fixed order, so the
// bits do not change from run to run.
#include <hip/hip_runtime.h>

#include "rr_config.hpp"
#include "rr_device.hpp"
#include "rr_launch.hpp"
#include "rr_launch_util.hpp"
#include "rr_merge_math.hpp"
#include "rr_rowio.hpp"

namespace rr {

typedef __bf16 rr_bf16x8 __attribute__((ext_vector_type(8)));
typedef float rr_f32x16 __attribute__((ext_vector_type(16)));

// Accumulator layout of the 32x32 MFMA (checked on MI355X against a host
// product): register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4 and
// column l%32; an A operand lane holds row l%32, a B operand lane column
// l%32, both at k = 8*(l/32) + 0..7 of the 16-deep step.

__device__ __forceinline__ rr_bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(rr_bf16x8, u); }

// Pack eight floats to bf16 (round to nearest even).
__device__ __forceinline__ rr_bf16x8 pack8(const float* f)
{
    uint4 u;
    u.x = pack_bf16x2(f[0], f[1]);
    u.y = pack_bf16x2(f[2], f[3]);
    u.z = pack_bf16x2(f[4], f[5]);
    u.w = pack_bf16x2(f[6], f[7]);
    return as_bf16x8(u);
}

// ------------------------------------------------ staged through LDS by DMA
// Keys stream in stages of kAttnStageKeys; each stage's K and V tiles go from
// HBM straight into LDS (buffer loads with the lds modifier: no registers),
// NS stages in flight.  Tiles are unpadded and XOR-swizzled by 16-byte chunk
// (each lane picks the global chunk that belongs at its LDS slot):
//   K: chunk c of row r at slot c ^ (r mod chunks-per-row): the S operand
//      reads (16 lanes = 16 rows, one chunk) hit 16 distinct bank groups;
//   V: chunk c of row r at slot c ^ v_swz(r): the transposed reads below
//      (4 rows x 4 half-chunks per 16 lanes, two such groups per 32 lanes)
//      hit 32 distinct 8-byte bank pairs.  The LDS serves 256 bytes per
//      cycle (64 banks; an 8-byte read takes 32 lanes at once, measured on
//      MI355X), so with 256-byte rows (depth 128) the row does not change
//      the bank and the XOR must separate all 32 lanes: 4 (r mod 4) moves
//      the two high chunk bits.  With 128-byte rows the row's parity picks
//      the bank half, and 2 (r mod 4) suffices.
// V stays row-major (keys x depth); the A operand of O^T += V^T P^T comes from
// ds_read_b64_tr_b16, which hands lane i of a 16-lane group element i%4 of
// the 8 bytes addressed by lane 4j + i/4, j = 0..3 (checked on MI355X): with
// lane 4j + q pointing at V[k0 + j][d0 + 4q], lane i receives
// V[k0 .. k0+3][d0 + i] -- four consecutive keys at one depth.
template <int D, int KB>
struct AttnStage {
    uint16_t k[KB * D];
    uint16_t v[KB * D];
};

template <int D>
__device__ __forceinline__ int v_swz(int row)
{
    return D == 128 ? (row & 3) << 2 : (row & 3) << 1;
}

// s_waitcnt on the vector-memory counter only (N < 16): expcnt and lgkmcnt
// fields at their maxima.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 16, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(N | 0x70 | 0xF00);
}

// Wait until at most `after` stages of OPS DMA operations each are still
// outstanding (every stage issued before them has landed); at most NS - 2
// stages are ever outstanding after the one about to be read.
template <int OPS, int NS>
__device__ __forceinline__ void wait_stages(int64_t after)
{
    if constexpr (NS - 2 >= 3) {
        if (after >= 3) { wait_vmcnt<OPS * 3>(); return; }
    }
    if constexpr (NS - 2 >= 2) {
        if (after >= 2) { wait_vmcnt<OPS * 2>(); return; }
    }
    if constexpr (NS - 2 >= 1) {
        if (after >= 1) { wait_vmcnt<OPS>(); return; }
    }
    wait_vmcnt<0>();
}

// A thread's share of one stage's DMA: OPS 16-byte chunks of K and of V.
// Slot i * kBlockThreads + threadIdx.x of a stage holds chunk `pos` of key
// row `row`; the byte offsets into the stage's keys (with the K and V
// swizzles) do not depend on the stage, so they are formed once.
// row_bytes: bytes between consecutive keys of one head in K and V (D * 2
// for the dense layout, kv_heads * D * 2 for tokens packed with their heads).
template <int D, int KB>
struct AttnDmaLane {
    static constexpr int CH = D / 8;                       // 16-byte chunks per row
    static constexpr int OPS = KB * CH / kBlockThreads;    // per tensor per thread
    int koff[OPS], voff[OPS];
    __device__ explicit AttnDmaLane(int row_bytes)
    {
#pragma unroll
        for (int i = 0; i < OPS; ++i) {
            const int slot = i * kBlockThreads + (int)threadIdx.x;
            const int row = slot / CH, pos = slot % CH;
            koff[i] = row * row_bytes + 16 * (pos ^ (row & (CH - 1)));
            voff[i] = row * row_bytes + 16 * (pos ^ v_swz<D>(row));
        }
    }
};

// DMA of one stage: keys [js, js + nvalid) of a head into stage buffer st;
// key j of the head starts kstride elements after key j - 1.  In a partial
// stage (nvalid < KB) rows past nvalid repeat row nvalid - 1 (finite values;
// their scores are masked), so every load stays inside the head's keys.
template <int D, int KB>
__device__ __forceinline__ void attn_dma_stage(const uint16_t* kh, const uint16_t* vh, int64_t js,
                                               int nvalid, AttnStage<D, KB>* st,
                                               const AttnDmaLane<D, KB>& dl, int kstride)
{
    using L = AttnDmaLane<D, KB>;
    const int span = (nvalid - 1) * kstride * 2 + D * 2;  // bytes from the first key to the end of the last
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(kh + js * kstride), 0, span, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(vh + js * kstride), 0, span, kBufferWord3);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
#pragma unroll
    for (int i = 0; i < L::OPS; ++i) {
        const int base = i * kBlockThreads + wave * kWave;   // first slot of this wave's op
        int ko = dl.koff[i], vo = dl.voff[i];
        if (nvalid < KB) {                                   // uniform: the partial stage only
            const int row = (base + lane_id()) / L::CH;
            const int shift = ((row < nvalid ? row : nvalid - 1) - row) * kstride * 2;
            ko += shift;
            vo += shift;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rk, (__attribute__((address_space(3))) void*)((char*)st->k + 16 * base), 16, ko, 0, 0,
            kBufferNonTemporal);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rv, (__attribute__((address_space(3))) void*)((char*)st->v + 16 * base), 16, vo, 0, 0,
            kBufferNonTemporal);
    }
}

typedef short rr_i16x4 __attribute__((ext_vector_type(4)));

// The larger of a lane's value and that of lane i ^ 32 (the other half of
// the wavefront), in every lane: v_permlane32_swap hands each half the
// other half's values without going through LDS.
__device__ __forceinline__ float max_halves(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Workgroup barrier between stages.  __syncthreads() carries a workgroup
// release fence, which on this target waits for every outstanding LDS DMA
// (vmcnt(0)) and would drain the stages in flight.  Here each wave has
// already waited for its own DMA of the stage it is about to read
// (wait_vmcnt), so a bare s_barrier suffices; before it, lgkmcnt(0) retires
// the wave's LDS reads of the previous stage, whose buffer the next DMA
// overwrites.  The signal fences keep the compiler from moving LDS accesses
// across the barrier.
__device__ __forceinline__ void stage_barrier()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maxima
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// The fold of a fused group's O partials: out_rows[r][d] = sum over p of
// cell[r][p] * O_p[r][d] in ascending p (merge_accumulate), for r < nr.  A
// thread owns 4 columns of rows r0, r0 + RPP, ...; it issues the loads of RB
// whole rows (RB * PC cells, PC >= P a compile-time bound) before folding any
// of them, so that a round trip to the device-coherent level is paid once
// per RB rows.  Loads of cells p >= P are not issued.
template <int D, int PC, class YT>
__device__ __forceinline__ void fold_group_rows(const __amdgpu_buffer_rsrc_t rg,
                                                const double* cell, YT* out_rows, int32_t P,
                                                int nr)
{
    constexpr int LPR = D / 4;                          // lanes per row, 4 columns each
    constexpr int RPP = kBlockThreads / LPR;            // rows per pass
    constexpr int kCells = 16;                          // 16-byte loads in flight per thread
    constexpr int RB = kCells / PC < kAttnRows / RPP ? kCells / PC : kAttnRows / RPP;
    const int li = threadIdx.x % LPR;
    const int r0 = threadIdx.x / LPR;
    const int lane_off = (r0 * D + 4 * li) * 4;
    for (int kb = 0; r0 + kb * RPP < nr; kb += RB) {
        rr_u32x4 u[RB][PC];
#pragma unroll
        for (int kk = 0; kk < RB; ++kk)
#pragma unroll
            for (int pp = 0; pp < PC; ++pp) {
                u[kk][pp] = rr_u32x4{0u, 0u, 0u, 0u};   // one register per value on both paths
                if (pp < P && r0 + (kb + kk) * RPP < nr)
                    u[kk][pp] = __builtin_amdgcn_raw_buffer_load_b128(
                        rg, lane_off, ((pp * kAttnRows + (kb + kk) * RPP) * D) * 4,
                        kBufferDeviceScope);
            }
#pragma unroll
        for (int kk = 0; kk < RB; ++kk) {
            const int r = r0 + (kb + kk) * RPP;
            if (r < nr) {
                double a4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
                for (int pp = 0; pp < PC; ++pp)
                    if (pp < P) {
                        const float vf[4] = {__uint_as_float(u[kk][pp].x), __uint_as_float(u[kk][pp].y),
                                             __uint_as_float(u[kk][pp].z), __uint_as_float(u[kk][pp].w)};
                        merge_accumulate<4>(a4, cell[r * P + pp], vf);
                    }
                MergeOut<YT>::four(out_rows + r * D + 4 * li, a4);
            }
        }
    }
}

// FUSED: the partitions of a (head, query tile) combine themselves.  Each
// workgroup publishes its partial (O_p, m_p, l_p) with device-scope
// write-through stores, waits for their acknowledgement and takes the
// group's ticket; the workgroup that draws ticket P - 1 arrives last and
// folds the P partials in ascending partition order with the arithmetic of
// rr_splitk_lse_merge (rr_merge_math.hpp) into `out`, then resets the ticket
// ("cluster_allreduce", description: the fold visits ranks in order whatever
// the arrival order).  Without FUSED the partials are the output.
template <int D, bool FUSED>
constexpr int attn_stages()
{
    return D == 128 ? kAttnStages : kAttnStagesOther;
}
template <int D, bool FUSED>
constexpr int attn_workgroups_per_cu()
{
    return D == 128 ? kAttnWorkgroupsPerCU : kAttnWorkgroupsPerCUOther;
}

// RAGGED: packed variable-length sequences ("fa4_splitk_reduce_scatter_write",
// signature: the output tile is placed by a head index and a row index into
// a ragged [tokens][heads][depth] tensor, its row count cut to the
// sequence).  q is [total_q][heads][D] and k, v [total_k][kv_heads][D];
// sequence b has tokens cu_q[b] .. cu_q[b+1] - 1 and keys cu_k[b] ..
// cu_k[b+1] - 1 (offsets clamped into the tensors); q_rows is the longest
// sequence's query count (q_tiles tiles of it), kv_len the total key count;
// the partial of (token t, head h) is row t * heads + h of the rows
// (= total_q * heads) of each partition.  Tiles past a sequence's end exit;
// a sequence's query rows past q_rows are left unwritten.
// The sequence of rank pos when a batch's sequences are ordered by key count,
// most first, ties by index: thread t < batch counts the sequences ahead of
// sequence t, and the one with pos ahead of it is the answer (the order is
// total, so exactly one thread finds it).  Key counts as the work items take
// them, from cu_k clamped into [0, kv_len].  Every thread of the workgroup
// calls it (one barrier).
__device__ int64_t attn_sequence_of_rank(int64_t pos, const int32_t* __restrict__ cu_k,
                                         int64_t batch, int64_t kv_len, int32_t* slot)
{
    auto keys = [&](int64_t s) {
        const int64_t c0 = min(max((int64_t)cu_k[s], (int64_t)0), kv_len);
        return min(max((int64_t)cu_k[s + 1], c0), kv_len) - c0;
    };
    if ((int64_t)threadIdx.x < batch) {
        const int64_t t = threadIdx.x, kt = keys(t);
        int64_t ahead = 0;
        for (int64_t u = 0; u < batch; ++u) {
            const int64_t ku = keys(u);
            ahead += (ku > kt || (ku == kt && u < t)) ? 1 : 0;
        }
        if (ahead == pos)
            *slot = (int32_t)t;
    }
    __syncthreads();
    const int64_t s = *slot;
    return s < 0 ? 0 : s >= batch ? batch - 1 : s;
}

template <int D, int KB, int NS, bool FUSED, class YT, bool RAGGED = false>
__global__ __launch_bounds__(kBlockThreads, (attn_workgroups_per_cu<D, FUSED>())) void k_attn_staged(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    float* __restrict__ o, float* __restrict__ m_out, float* __restrict__ l_out, int64_t heads,
    int64_t kv_heads, int64_t q_rows, int64_t kv_len, int32_t P, float scale, int32_t q_tiles,
    int64_t rows, YT* __restrict__ out, uint32_t* __restrict__ tickets, int32_t skew,
    const int32_t* __restrict__ cu_q = nullptr, const int32_t* __restrict__ cu_k = nullptr,
    int64_t total_q = 0)
{
    static_assert(!(RAGGED && FUSED), "the one-launch fold takes dense query tiles");
    constexpr int NC = D / 16;
    constexpr int NT = D / 32;
    constexpr int CH = D / 8;
    constexpr int OPS = 2 * (KB * CH / kBlockThreads);  // DMA ops per stage per thread
    constexpr int NST = KB / 32;                         // 32-key tiles per stage
    static_assert(OPS * (NS - 2) < 16, "vmcnt immediate");
    static_assert(NS >= 2 && NS <= 5, "stage count");
    static_assert(KB % 32 == 0 && (KB * CH) % kBlockThreads == 0, "stage shape");
    // One LDS object per stage: the compiler's wait insertion then knows that
    // a DMA into one stage cannot alias reads of another, and does not drain
    // the DMA queue before every read.  The stage loop below is unrolled by
    // NS, so every stage reference is to a named object.
    __shared__ AttnStage<D, KB> S0;
    __shared__ AttnStage<D, KB> S1;
    __shared__ AttnStage<D, KB> S2;
    __shared__ AttnStage<D, KB> S3;
    __shared__ AttnStage<D, KB> S4;
#define RR_ATTN_STAGE(u) ((u) == 0 ? &S0 : (u) == 1 ? &S1 : (u) == 2 ? &S2 : (u) == 3 ? &S3 : &S4)

    const int64_t nb = gridDim.x;
    const int64_t per = nb / kXcds, rem = nb % kXcds;
    const int64_t xcd = blockIdx.x % kXcds, idx = blockIdx.x / kXcds;
    int64_t w = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    const int64_t group = heads / kv_heads;
    int32_t qt, p;
    int64_t g, kvl, b;
    if constexpr (RAGGED) {
        // Sequences of different lengths.  A unit of work is (sequence, kv
        // head, partition), numbered partition fastest; its q_tiles * group
        // items share the unit's keys and run one after another on one XCD.
        // When a sequence's units divide evenly over the XCDs (and the batch
        // fits the workgroup), XCD x takes the x-th eighth of every
        // sequence's units (whole kv heads where they divide, so a query
        // tile's partitions meet its q in that XCD's L2), the sequences in
        // order of key count, most first (longest-processing-time order);
        // else the sequence index varies fastest, so that every XCD's range
        // of work still takes its share of each sequence.
        __shared__ int32_t seq_slot;
        const int64_t inner = (int64_t)q_tiles * group;
        const int64_t per_seq = (int64_t)P * kv_heads;
        const int64_t batch = nb / (inner * per_seq);
        int64_t i, unit;
        if (per_seq % kXcds == 0 && batch <= kBlockThreads) {
            const int64_t span = per_seq / kXcds * inner;  // a sequence's items on one XCD
            i = idx % inner;
            unit = xcd * (per_seq / kXcds) + (idx % span) / inner;
            b = attn_sequence_of_rank(idx / span, cu_k, batch, kv_len, &seq_slot);
        } else {
            i = w % inner;
            w /= inner;
            b = w % batch;
            unit = w / batch;
        }
        qt = (int32_t)(i % q_tiles);
        g = i / q_tiles;
        p = (int32_t)(unit % P);
        kvl = unit / P;
    } else {
        qt = (int32_t)(w % q_tiles);
        w /= q_tiles;
        g = w % group;
        w /= group;
        p = (int32_t)(w % P);
        w /= P;
        kvl = w % kv_heads;
        b = w / kv_heads;
    }
    const int64_t bh = b * heads + kvl * group + g;
    const int64_t kvh = b * kv_heads + kvl;

    // The head's query rows: nq of them, row i at partial row prow0 + i * rs
    // (also its row of q), consecutive rows qs elements apart in q; its keys:
    // nk of them from kh / vh, kstride elements apart.
    int64_t nq = q_rows, nk = kv_len, prow0 = bh * q_rows, rs = 1;
    int qs = D, kstride = D;
    const uint16_t* kh = k + kvh * kv_len * D;
    const uint16_t* vh = v + kvh * kv_len * D;
    if constexpr (RAGGED) {
        const int64_t hq = kvl * group + g;            // query head within the token
        const int64_t a0 = min(max((int64_t)cu_q[b], (int64_t)0), total_q);
        const int64_t a1 = min(max((int64_t)cu_q[b + 1], a0), total_q);
        const int64_t c0 = min(max((int64_t)cu_k[b], (int64_t)0), kv_len);
        const int64_t c1 = min(max((int64_t)cu_k[b + 1], c0), kv_len);
        nq = min(a1 - a0, (int64_t)q_rows);            // rows past q_rows are not computed
        nk = c1 - c0;
        prow0 = a0 * heads + hq;
        rs = heads;
        qs = (int)(heads * D);
        kstride = (int)(kv_heads * D);
        kh = k + (c0 * kv_heads + kvl) * D;
        vh = v + (c0 * kv_heads + kvl) * D;
        if ((int64_t)qt * kAttnRows >= nq)
            return;                                    // the tile is past the sequence's end
    }
    const int lane = lane_id();
    const int hf = lane / 32;
    // wave-uniform by construction; said so, so that the per-wavefront O
    // descriptor below is a scalar one (no loop over lanes' descriptors)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t qrow = (int64_t)qt * kAttnRows + wave * 32 + lane % 32;
    const bool row_ok = qrow < nq;
    const int64_t row = prow0 + qrow * rs;
    const int64_t j0 = (int64_t)p * nk / P, j1 = ((int64_t)p + 1) * nk / P;
    float* orow = o + ((int64_t)p * rows + row) * D;

    const bool empty = j1 <= j0;   // a partition with no key: (O, m, l) = (0, -inf, 0)
    if (!FUSED && empty) {
        if (row_ok) {
#pragma unroll
            for (int d = 0; d < D / 2; d += 4)
                *reinterpret_cast<float4*>(orow + hf * (D / 2) + d) = make_float4(0.f, 0.f, 0.f, 0.f);
            if (hf == 0) {
                m_out[(int64_t)p * rows + row] = -__builtin_inff();
                l_out[(int64_t)p * rows + row] = 0.0f;
            }
        }
        return;
    }

    rr_bf16x8 qb[NC];
    if constexpr (!RAGGED) {
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(q + bh * q_rows * D), 0, (int)(q_rows * D * 2), kBufferWord3);
        const int qoff = (int)(qrow < q_rows ? qrow : q_rows) * D * 2;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const rr_u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff + (16 * c + 8 * hf) * 2, 0, 0);
            qb[c] = as_bf16x8(make_uint4(u.x, u.y, u.z, u.w));
        }
    } else {
        // the tile's rows from its first one, qs elements apart; rows past
        // the sequence read as zero (their results are not stored)
        const int64_t tr = nq - (int64_t)qt * kAttnRows;     // rows of the tile in the sequence
        const int tv = (int)(tr < kAttnRows ? tr : kAttnRows);
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(q + (prow0 + (int64_t)qt * kAttnRows * rs) * D), 0,
            (tv - 1) * qs * 2 + D * 2, kBufferWord3);
        const int ri = wave * 32 + lane % 32;
        const int qoff = (ri < tv ? ri : tv) * qs * 2;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const rr_u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff + (16 * c + 8 * hf) * 2, 0, 0);
            qb[c] = as_bf16x8(make_uint4(u.x, u.y, u.z, u.w));
        }
    }

    const int64_t nstg = ceil_div(j1 - j0, KB);
    const AttnDmaLane<D, KB> dl(kstride * 2);
    auto nvalid_of = [&](int64_t s_) {
        const int64_t left = j1 - j0 - s_ * KB;
        return (int)(left < KB ? left : KB);
    };
#pragma unroll
    for (int s_ = 0; s_ < NS - 1; ++s_)
        if (s_ < nstg)
            attn_dma_stage<D, KB>(kh, vh, j0 + (int64_t)s_ * KB, nvalid_of(s_), RR_ATTN_STAGE(s_), dl,
                                  kstride);

    rr_f32x16 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[t][r] = 0.0f;
    // Scores stay raw (q . k, float32 out of the MFMA); with c2 = |scale| *
    // log2(e) the probability is exp2(raw * c2 - m_ref * c2), one FMA per
    // score.  A negative scale is carried by negating q (exact in bf16), and
    // because rounding is monotonic, |scale| * max(raw) is the largest of the
    // rounded scaled scores, which is the m written out.
    // Online (max, sum) with a lazy reference: the exponentials are taken
    // relative to m_ref, which moves (rescaling O and l) only when a block's
    // maximum exceeds it by more than 2^kAttnLazyLog2 in the exponential, so
    // after the first stage the rescale is skipped; m_true is the exact
    // running maximum, and l is brought to it at the end.  O / l does not
    // depend on the reference.
    if (scale < 0.0f) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            uint4 u = __builtin_bit_cast(uint4, qb[c]);
            u.x ^= 0x80008000u; u.y ^= 0x80008000u; u.z ^= 0x80008000u; u.w ^= 0x80008000u;
            qb[c] = as_bf16x8(u);
        }
    }
    const float ascale = fabsf(scale);
    const float c2 = ascale * kLog2e;
    float m_ref = -__builtin_inff();
    float m_true = -__builtin_inff();
    float l_run = 0.0f;
    const int G = (lane / 16) & 1, a16 = lane % 16, jj = a16 / 4, qq = a16 % 4;

    auto stage = [&](int64_t st, AttnStage<D, KB>* T, AttnStage<D, KB>* F) {
        const int64_t issued = nstg < st + NS - 1 ? nstg : st + NS - 1;
        const int64_t after = issued - st - 1;
        wait_stages<OPS, NS>(after);
        stage_barrier();
        if (st + NS - 1 < nstg)
            attn_dma_stage<D, KB>(kh, vh, j0 + (st + NS - 1) * KB, nvalid_of(st + NS - 1), F, dl,
                                  kstride);
        const int nvalid = nvalid_of(st);
        const char* kb = reinterpret_cast<const char*>(T->k);
        const char* vb = reinterpret_cast<const char*>(T->v);
        // LDS read addresses, formed again in every stage from the lane's
        // coordinates (the empty asm hides them from loop-invariant code
        // motion): holding the 16 per-lane addresses across the loop would
        // cost 16 registers, forming them costs a dozen instructions that
        // issue while the matrix cores work.
        int lrow = lane % 32, lhf = hf, ljj = jj, lg = G, lqq = qq;
        asm volatile("" : "+v"(lrow), "+v"(lhf), "+v"(ljj), "+v"(lg), "+v"(lqq));
        // K: chunk 2c + hf of row lrow at slot (2c + hf) ^ (lrow mod D/8),
        // i.e. byte kbase + ((32 c) ^ kx)
        const int kbase = lrow * D * 2 + 16 * ((lhf ^ lrow) & 1);
        const int kx = 16 * (lrow & (D / 8 - 2));
        // V: rows 32 t + 16 c + 4 hf + jj (+ 8), chunk 4 dt + 2 G + (qq >> 1),
        // swizzled by v_swz(jj): byte vbase + ((64 dt + 32 G) ^ vx) + rows
        const int vbase = (4 * lhf + ljj) * D * 2 + 16 * (lqq >> 1) + 8 * (lqq & 1);
        const int vx = 16 * v_swz<D>(ljj);

        rr_f32x16 s[NST];
#pragma unroll
        for (int t = 0; t < NST; ++t) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[t][r] = 0.0f;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const uint4 a = *reinterpret_cast<const uint4*>(
                    kb + 32 * t * D * 2 + kbase + ((32 * c) ^ kx));
                s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qb[c], s[t], 0, 0, 0);
            }
        }
        // Score (t, r) of a lane is key 32 t + 8 (r / 4) + 4 hf + r % 4 of the
        // stage; only the partition's last stage can be partial, and there
        // key (t, r) is in when its offset 32 t + 8 (r / 4) + r % 4 is below
        // lim = nvalid - 4 hf (one register, compared against constants).
        const bool full = nvalid == KB;                 // all keys of the stage are in the partition
        const int lim = nvalid - 4 * hf;
        float bm = -__builtin_inff();
        if (full) {
#pragma unroll
            for (int t = 0; t < NST; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    bm = fmaxf(bm, s[t][r]);
        } else {
#pragma unroll
            for (int t = 0; t < NST; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 * t + 8 * (r / 4) + (r % 4) < lim)
                        bm = fmaxf(bm, s[t][r]);
        }
        bm = max_halves(bm);                            // finite: every stage has a key
        m_true = fmaxf(m_true, bm);
        const bool move = st == 0 || (bm - m_ref) * c2 > kAttnLazyLog2;
        if (__any(move)) {                              // wavefront-uniform branch
            const float m_new = move ? fmaxf(m_ref, bm) : m_ref;
            const float alpha = m_ref == -__builtin_inff() ? 0.0f : exp2_hw((m_ref - m_new) * c2);
            m_ref = m_new;
            l_run *= alpha;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[t][r] *= alpha;
        }
        const float mb = -m_ref * c2;
        float ls = 0.0f;
        if (full) {
#pragma unroll
            for (int t = 0; t < NST; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float pv = exp2_hw(__builtin_fmaf(s[t][r], c2, mb));
                    s[t][r] = pv;
                    ls += pv;
                }
        } else {
#pragma unroll
            for (int t = 0; t < NST; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float pv = 32 * t + 8 * (r / 4) + (r % 4) < lim
                                         ? exp2_hw(__builtin_fmaf(s[t][r], c2, mb)) : 0.0f;
                    s[t][r] = pv;
                    ls += pv;
                }
        }
        l_run += ls;
        rr_bf16x8 pb[NST][2];
#pragma unroll
        for (int t = 0; t < NST; ++t)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                float f[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    f[j] = s[t][8 * c + j];
                pb[t][c] = pack8(f);
            }
#pragma unroll
        for (int dt = 0; dt < NT; ++dt)
#pragma unroll
            for (int t = 0; t < NST; ++t)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int va = vbase + ((64 * dt + 32 * lg) ^ vx) + (32 * t + 16 * c) * D * 2;
                    const rr_i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (rr_i16x4 __attribute__((address_space(3)))*)(vb + va));
                    const rr_i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (rr_i16x4 __attribute__((address_space(3)))*)(vb + va + 8 * D * 2));
                    const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
                    acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        as_bf16x8(make_uint4(l2.x, l2.y, h2.x, h2.y)), pb[t][c], acc[dt], 0, 0, 0);
                }
    };
    for (int64_t st0 = 0; st0 < nstg; st0 += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            if (st0 + u >= nstg)
                break;
            stage(st0 + u, RR_ATTN_STAGE(u), RR_ATTN_STAGE((u + NS - 1) % NS));
        }
    }
#undef RR_ATTN_STAGE

    // Where the partial of (partition p, row) lives.  Unfused: [P][rows]
    // (the layout rr_splitk_lse_merge reads).  Fused: group-major,
    // [group][P][kAttnRows] with group = (head, query tile), so that the
    // fold finds a group's P partials in one range of at most 1 MiB.
    const int64_t grp = bh * q_tiles + qt;
    const int64_t slot0 = FUSED ? (grp * P + p) * kAttnRows
                                : (int64_t)p * rows + prow0 + (int64_t)qt * kAttnRows * rs;
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = empty ? 0.0f : 1.0f / l_tot;
    if (row_ok && hf == 0) {
        const float mv = empty ? -__builtin_inff() : ascale * m_true;
        const float lv = empty ? 0.0f : l_tot * exp2_hw((m_ref - m_true) * c2);
        float* mp = m_out + slot0 + (qrow - (int64_t)qt * kAttnRows) * rs;
        float* lp = l_out + slot0 + (qrow - (int64_t)qt * kAttnRows) * rs;
        if constexpr (FUSED) {
            __hip_atomic_store(mp, mv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(lp, lv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            *mp = mv;
            *lp = lv;
        }
    }
    // O through LDS, one 32-column depth tile at a time: a lane holds one
    // query column of the tile, so stores straight from the accumulator put
    // 32 bytes in each of 32 rows per instruction.  Each wavefront writes its
    // 32 x 32 floats row-major into a region of a stage buffer (rows padded
    // to 36 floats: 16-byte aligned, the b128 writes of 16 lanes on distinct
    // banks), then stores whole 128-byte lines, 8 rows per instruction.
    stage_barrier();                                   // every wavefront is done with the stages
    constexpr int kOStride = 36;                       // floats per staged row
    constexpr int kOWaveBytes = 32 * kOStride * 4;
    constexpr int kWavesPerStage = (kWavesPerBlock + NS - 1) / NS;
    static_assert(kWavesPerStage * kOWaveBytes <= (int)sizeof(AttnStage<D, KB>), "O staging fits");
    const int wst = wave / kWavesPerStage;
    char* sb = reinterpret_cast<char*>(&S0);
    if (NS > 1 && wst == 1) sb = reinterpret_cast<char*>(&S1);
    if (NS > 2 && wst == 2) sb = reinterpret_cast<char*>(&S2);
    if (NS > 3 && wst == 3) sb = reinterpret_cast<char*>(&S3);
    char* obase = sb + (wave % kWavesPerStage) * kOWaveBytes;
    float* ow = reinterpret_cast<float*>(obase);
    const int64_t qrow0 = (int64_t)qt * kAttnRows + wave * 32;
    // the wavefront's 32 rows of O_p, rs * D floats apart; rows past the
    // head's query rows fall outside the range and are not written
    const int64_t wrows = nq - qrow0 < 32 ? (nq - qrow0 > 0 ? nq - qrow0 : 0) : 32;
    const int orow_bytes = (int)(rs * D * 4);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        o + (slot0 + wave * 32 * rs) * D, 0,
        wrows > 0 ? (int)((wrows - 1) * orow_bytes + D * 4) : 0, kBufferWord3);
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
            *reinterpret_cast<float4*>(ow + (lane % 32) * kOStride + 8 * g4 + 4 * hf) =
                make_float4(acc[dt][4 * g4] * inv, acc[dt][4 * g4 + 1] * inv,
                            acc[dt][4 * g4 + 2] * inv, acc[dt][4 * g4 + 3] * inv);
        __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0): the wavefront's writes are in
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = lane / 8 + 8 * i;
            const float4 val = *reinterpret_cast<const float4*>(ow + r * kOStride + 4 * (lane % 8));
            const rr_u32x4 u = {__float_as_uint(val.x), __float_as_uint(val.y),
                                __float_as_uint(val.z), __float_as_uint(val.w)};
            // FUSED: device-scope write-through (another workgroup reads it);
            // otherwise a streaming store
            __builtin_amdgcn_raw_buffer_store_b128(u, ro, r * orow_bytes + (32 * dt + 4 * (lane % 8)) * 4,
                                                   0, FUSED ? kBufferDeviceScope : kBufferNonTemporal);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);            // reads done before the next tile overwrites
        __builtin_amdgcn_wave_barrier();
    }
    if constexpr (FUSED) {
        static_assert(NS >= 3 && kAttnRows * (D / 8) * 8 <= (int)sizeof(AttnStage<D, KB>),
                      "three stage buffers hold the fold's (row, partition) cells for P <= D / 8");
        // the ticket's verdict, in the last stage buffer: free once every
        // wavefront's O has left the staging, and not used by the fold below
        uint32_t* last = reinterpret_cast<uint32_t*>(NS == 5 ? (void*)&S4 : NS == 4 ? (void*)&S3
                                                                                   : (void*)&S2);
        // the agent-scope release of publish_partial (rr_device.hpp): the
        // stores above went through to the device-coherent level, and the
        // wait holds each wavefront until they are acknowledged
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        stage_barrier();                               // every wavefront's partial is in
        if (threadIdx.x == 0) {
            // test hook (normally 0): partition p waits about (P - 1 - p) *
            // skew sleep periods, so the partitions tend to arrive in
            // descending order; the fold below does not depend on it
            for (int i = 0; i < (P - 1 - p) * skew; ++i)
                __builtin_amdgcn_s_sleep(8);
            const uint32_t t = __hip_atomic_fetch_add(&tickets[grp], 1u, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
            *last = t == (uint32_t)P - 1;
        }
        __syncthreads();
        if (!*last)
            return;
        // The last arriver: the fold of rr_splitk_lse_merge over the group's
        // rows, the partials read with device-scope loads.  LDS: the (m, l)
        // pairs, the weights and the coefficients of nr x P (row, partition)
        // cells in three stage buffers (P <= D / 8 keeps each within one).
        const int64_t row_base = bh * q_rows + (int64_t)qt * kAttnRows;
        const int nr = (int)(q_rows - (int64_t)qt * kAttnRows < kAttnRows
                                 ? q_rows - (int64_t)qt * kAttnRows : kAttnRows);
        const int npairs = nr * P;
        constexpr int kMaxP = D / 8;                   // the largest P of the fused call
        constexpr int kCellPasses = kAttnRows * kMaxP / kBlockThreads;
        float2* stat = reinterpret_cast<float2*>(&S0);
        double* wd = reinterpret_cast<double*>(&S1);
        double* cell = reinterpret_cast<double*>(&S2);
        // every load of a phase is issued before the first is used: they are
        // device-scope, served beyond the XCD's L2, and a wait per load would
        // leave the fold latency-bound
        {
            float2 st[kCellPasses];
#pragma unroll
            for (int u = 0; u < kCellPasses; ++u) {
                const int i = threadIdx.x + u * kBlockThreads;
                if (i < npairs) {
                    const int r = i / P, pp = i - r * P;
                    const int64_t at = (grp * P + pp) * kAttnRows + r;
                    st[u] = make_float2(
                        __hip_atomic_load(m_out + at, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                        __hip_atomic_load(l_out + at, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                }
            }
#pragma unroll
            for (int u = 0; u < kCellPasses; ++u)
                if (threadIdx.x + u * kBlockThreads < npairs)
                    stat[threadIdx.x + u * kBlockThreads] = st[u];
        }
        __syncthreads();
        for (int i = threadIdx.x; i < npairs; i += kBlockThreads)
            wd[i] = merge_weight(stat[i], merge_row_max(stat + (i / P) * P, P), 1.0f);
        __syncthreads();
        for (int i = threadIdx.x; i < npairs; i += kBlockThreads)
            cell[i] = merge_coef(stat[i], wd[i], merge_total(wd + (i / P) * P, P));
        __syncthreads();
        // the group's P partials, [P][kAttnRows][D] floats; every partition,
        // empty ones included, wrote its rows
        const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
            o + grp * P * kAttnRows * D, 0, P * kAttnRows * D * 4, kBufferWord3);
        YT* out_rows = out + row_base * D;
        if (P <= 2)
            fold_group_rows<D, 2>(rg, cell, out_rows, P, nr);
        else if (P <= 4)
            fold_group_rows<D, 4>(rg, cell, out_rows, P, nr);
        else if (P <= 8 || kMaxP < 16)
            fold_group_rows<D, (kMaxP < 8 ? kMaxP : 8)>(rg, cell, out_rows, P, nr);
        else
            fold_group_rows<D, (kMaxP < 16 ? kMaxP : 16)>(rg, cell, out_rows, P, nr);
        if (threadIdx.x == 0)
            __hip_atomic_store(&tickets[grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Packed variable-length sequences: q_tiles tiles of the longest sequence
// for every (sequence, head, partition); a.kv_len is the total key count.
static rr_status launch_attn_varlen(const AttentionLaunch& a)
{
    const int32_t q_tiles = (int32_t)ceil_div(a.q_rows, kAttnRows);
    const int64_t nwork = (int64_t)q_tiles * a.P * a.batch * a.heads;
    const int64_t rows = a.total_q * a.heads;
    const dim3 grid((unsigned)nwork), block(kBlockThreads);
    float* none = nullptr;
    if (a.depth == 128)
        return launch_kernel(
            k_attn_staged<128, kAttnStageKeys, attn_stages<128, false>(), false, float, true>, grid,
            block, 0, a.stream, a.q, a.k, a.v, a.o, a.m, a.l, a.heads, a.kv_heads, a.q_rows,
            a.kv_len, a.P, a.scale, q_tiles, rows, none, a.tickets, 0, a.cu_q, a.cu_k, a.total_q);
    return launch_kernel(
        k_attn_staged<64, kAttnStageKeys, attn_stages<64, false>(), false, float, true>, grid,
        block, 0, a.stream, a.q, a.k, a.v, a.o, a.m, a.l, a.heads, a.kv_heads, a.q_rows, a.kv_len,
        a.P, a.scale, q_tiles, rows, none, a.tickets, 0, a.cu_q, a.cu_k, a.total_q);
}

template <bool FUSED, class YT>
static rr_status launch_attn(const AttentionLaunch& a, YT* out)
{
    const int32_t q_tiles = (int32_t)ceil_div(a.q_rows, kAttnRows);
    const int64_t nwork = (int64_t)q_tiles * a.P * a.batch * a.heads;
    const int64_t rows = a.batch * a.heads * a.q_rows;
    const dim3 grid((unsigned)nwork), block(kBlockThreads);
    if (a.depth == 128)
        return launch_kernel(
            k_attn_staged<128, kAttnStageKeys, attn_stages<128, FUSED>(), FUSED, YT>, grid, block, 0,
            a.stream, a.q, a.k, a.v, a.o, a.m, a.l, a.heads, a.kv_heads, a.q_rows, a.kv_len, a.P,
            a.scale, q_tiles, rows, out, a.tickets, a.skew, nullptr, nullptr, 0);
    return launch_kernel(k_attn_staged<64, kAttnStageKeys, attn_stages<64, FUSED>(), FUSED, YT>,
                         grid, block, 0, a.stream, a.q, a.k, a.v, a.o, a.m, a.l, a.heads,
                         a.kv_heads, a.q_rows, a.kv_len, a.P, a.scale, q_tiles, rows, out,
                         a.tickets, a.skew, nullptr, nullptr, 0);
}

rr_status launch_attention(const AttentionLaunch& a)
{
    if (a.cu_q)
        return launch_attn_varlen(a);
    if (!a.out)
        return launch_attn<false, float>(a, nullptr);
    if (a.out_dtype == RR_BF16)
        return launch_attn<true, uint16_t>(a, static_cast<uint16_t*>(a.out));
    return launch_attn<true, float>(a, static_cast<float*>(a.out));
}

}  // namespace rr
