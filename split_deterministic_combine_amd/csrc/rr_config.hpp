// rr_config.hpp -- launch constants shared by the host planner and the
// kernels.  Plain C++ (no HIP), so the planner builds and runs on any host.
#pragma once

#include <stdint.h>

namespace rr {

// Threads per workgroup for the block, split-K and softmax block tiers, and
// for the wave / tiled / serial tiers (which pack rows into a workgroup).
constexpr int kBlockThreads = 256;
constexpr int kWavesPerBlock = kBlockThreads / 64;

// Wave tier: row groups handled by one wavefront per launch (independent
// loads in flight per lane).
constexpr int kWaveRowGroups = 4;

// Tiled tier: rows owned by one thread (the page's emit_tile_width).
constexpr int kTiledRows = 4;

// Split-K trigger and workgroups per row: at least kSplitKMinColsPerGroup
// columns per workgroup.
constexpr int64_t kSplitKMinCols = 65536;
constexpr int64_t kSplitKMinColsPerGroup = 16384;
constexpr int kSplitKMaxSlices = 256;
// G aims at this many workgroups per CU in total: the row reduction streams
// best at 2 (4 or 8 measured slower: more concurrent streams per CU contend);
// the softmax and layernorm split-K passes and the axis split-K, which do
// more work per element, keep 4.
constexpr int kSplitKBlocksPerCU = 2;
constexpr int kSplitKHeavyBlocksPerCU = 4;

// Block-tier loads in flight per thread (128-bit each).
constexpr int kBlockUnroll = 4;
constexpr int kSplitKUnroll = 8;

// Softmax block tier.  Whole-chunk, 16-byte aligned rows run the persistent
// kernel (row_pf_shape below).  Other rows keep up to kSoftmaxMaxChunks
// 16-byte chunks per thread in registers, one row per workgroup; rows too
// long for kBlockThreads threads (more than kSoftmaxWideMinChunks chunks) run
// on workgroups of kSoftmaxWideThreads, and beyond that the streaming variant
// reads x twice.
constexpr int kSoftmaxMaxChunks = 8;
constexpr int kSoftmaxWideThreads = 512;
constexpr int64_t kSoftmaxWideMinChunks = (int64_t)kBlockThreads * kSoftmaxMaxChunks;

// Split-K softmax: 16-byte chunks per thread per tile (a tile is one load
// round of the workgroup).
constexpr int kSoftmaxSplitKUnroll = 4;
// Reduction over a non-last axis: 16-byte loads in flight per thread (one
// per axis step; kAxisSplitKUnroll in the split-K partial pass), split-K when
// there are fewer than kAxisSplitKMaxBlocksPerCU workgroups of outputs per CU
// and the axis has at least kAxisSplitKMinAxis steps, with slices of at least
// kAxisMinStepsPerLane steps per axis lane.  The split-K pass aims at
// kAxisSplitKBlocksPerCU workgroups per CU (swept on [16384, 16384],
// [4096, 65536] and [65536, 1024] f32: 2 beat 3, 4 and 8; unroll 4 beat 8
// and 16; tiles of 64 groups beat 32, 128 and 256).
constexpr int kAxisUnroll = 8;
constexpr int kAxisSplitKUnroll = 4;
constexpr int kAxisSplitKBlocksPerCU = 2;
constexpr int kAxisSplitKMaxBlocksPerCU = 1;
constexpr int64_t kAxisSplitKMinAxis = 512;
constexpr int64_t kAxisNarrowGroups = 64;   // fewer output groups per outer: split-K tiles
constexpr int64_t kAxisMinStepsPerLane = 32;
constexpr int64_t kAxisMaxSlices = 1024;  // the fold pass reads G partials per output

// Axis fold pass: log2 of the slice lanes per output, the largest power of
// two that leaves every lane at least 4 partials (at most 256).
constexpr int axis_fold_lanes_log2(int64_t slices)
{
    int l = 0;
    while (l < 8 && ((int64_t)4 << (l + 1)) <= slices)
        ++l;
    return l;
}

// Split-K axis tile: log2 of the output groups per workgroup (the rest of the
// 256 threads are axis lanes): the groups of one outer index rounded up to a
// power of two, at most 64 (so at least 4 axis lanes).
constexpr int axis_tile_log2(int64_t groups_per_outer)
{
    int l = 0;
    while (l < 6 && ((int64_t)1 << l) < groups_per_outer)
        ++l;
    return l;
}

// Persistent rows (softmax and layernorm block tiers).  Rows of whole
// aligned 16-byte chunks, up to kPfMaxChunks of them, stay in registers on
// persistent workgroups whose size follows the row (row_pf_shape).  A CU gets
// kPfLoadsPerCU / (wavefronts per workgroup * chunks per thread) of them (at
// least one): that many 16-byte loads per lane in flight per CU, the measured
// optimum (fewer starve HBM, more contend).  The launch lowers the grid to
// what the kernel's occupancy allows, so a persistent grid never queues.
constexpr int64_t kPfMaxChunks = 2048;
constexpr int kPfLoadsPerCU = 32;

// Threads per row (nt) and chunks per thread (nch) of a persistent row of
// `chunks` chunks; nt == 0 when the row is too long for registers.
struct RowPfShape {
    int nt;
    int nch;
};
constexpr RowPfShape row_pf_shape(int64_t chunks)
{
    return chunks <= 64     ? RowPfShape{64, 1}
           : chunks <= 128  ? RowPfShape{64, 2}
           : chunks <= 256  ? RowPfShape{64, 4}
           : chunks <= 512  ? RowPfShape{128, 4}
           : chunks <= 1024 ? RowPfShape{256, 4}
           : chunks <= kPfMaxChunks ? RowPfShape{512, 4}
                                    : RowPfShape{0, 0};
}
// Block-tier row reductions take persistent rows (row_pf_shape) when a call
// has at least kReducePfMinRowsPerCU rows per CU, so that every workgroup
// walks several, with kReducePfLoadsPerCU 16-byte loads per lane in flight
// per CU (a pure read stream: [65536, 1000] f32 sums took 45.4, 44.7, 43.9
// and 43.5 us at 32, 24, 48 and 64).
constexpr int64_t kReducePfMinRowsPerCU = 4;
constexpr int kReducePfLoadsPerCU = 64;

constexpr int row_pf_blocks_per_cu(RowPfShape sh, int loads_per_cu = kPfLoadsPerCU)
{
    return loads_per_cu / (sh.nt / 64 * sh.nch) > 0 ? loads_per_cu / (sh.nt / 64 * sh.nch) : 1;
}

// Layernorm: rows that are not persistent-eligible but have up to
// kLnMaxChunks chunks per thread of 256 stay in registers one row per
// workgroup; longer rows stream twice.  Split-K tiles are kLnSplitKUnroll
// chunks per thread.
constexpr int kLnMaxChunks = 8;
constexpr int kLnSplitKUnroll = 4;
constexpr int kLnMapMinRows = 4;  // split-K map: rows sharing one load of a tile's gamma / beta
// Persistent layernorm rows at any alignment: gamma and beta as float in LDS
// (the row's phase moves its columns across the threads, so every row reads
// them at new offsets) when both, padded one word per chunk, fit in
// kLnLdsWeightBytes (bf16 rows up to 4096 columns).
constexpr int64_t kLnLdsWeightBytes = 36880;

// LSE merge: partitions staged per batch of loads, and workgroup size.
constexpr int kMergeBatch = 8;
constexpr int kMergeMaxP = 256;
// Partition-outer merge (one 128-bit chunk per lane): rows per lane and the
// largest partition count it takes (its LDS holds 16 B per row and partition).
constexpr int kMergePOuterRowsPerLane = 4;
constexpr int kMergePOuterMaxP = 32;

// Split-K attention partials: query rows per workgroup (4 wavefronts of 32)
// and keys per LDS stage.  Depth 128: 3 stages in flight at 3 workgroups per
// CU (48 KiB of LDS and at most 168 registers each) measured fastest on
// [8, 32, 128, 128] over 8192 keys, beside 4 and 5 stages at 2 per CU; depth
// 64 keeps 4 stages at (at least) 2 per CU -- 3 stages are too small for its
// O staging.
constexpr int kAttnRows = 128;
constexpr int kAttnStageKeys = 32;
constexpr int kAttnStages = 3;            // depth 128
constexpr int kAttnWorkgroupsPerCU = 3;   // depth 128
constexpr int kAttnStagesOther = 4;
constexpr int kAttnWorkgroupsPerCUOther = 2;
constexpr int kAttnMaxP = 256;
constexpr float kAttnLazyLog2 = 8.0f; // lazy rescale: the reference max moves past 2^8

// XCDs of MI355X: consecutive workgroups are dealt to them in turn.
constexpr int kXcds = 8;

// Largest grid.x the launchers use; kernels loop over the remainder.
constexpr int64_t kMaxGrid = 1 << 30;

// Workspace layout for split-K: per-row tickets (uint32), padded to 256 B,
// then per-(row, workgroup) partials of 8 bytes.
constexpr int64_t kWorkspaceAlign = 256;

constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
constexpr int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Lanes sharing one row in the wave tier, from the number of 128-bit (or
// scalar) chunks a row spans.
constexpr int wave_lanes_for_chunks(int64_t chunks)
{
    if (chunks <= 4) return 4;
    if (chunks <= 16) return 16;
    return 64;
}

}  // namespace rr
