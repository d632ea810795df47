// rr_plan.cpp -- tier selection and launch geometry (host only, no HIP).
//
// "reduce" (algorithm.gpu.rowwise), tier semantics, describes what each tier
// does -- a wavefront per short row, a workgroup striding along a row, a
// thread owning several adjacent rows, one thread per row, and several
// workgroups per row when there are fewer rows than compute units -- but
// gives no thresholds.  The thresholds below are this library's.
#include "rr_plan.hpp"

#include <string.h>

#include "rr_config.hpp"

namespace rr {

uint64_t splitk_workspace_bytes(int64_t rows, int32_t slices, int partial_bytes)
{
    return (uint64_t)(round_up(rows * 4, kWorkspaceAlign) + rows * (int64_t)slices * partial_bytes);
}

uint64_t softmax_splitk_workspace_bytes(int64_t rows, int32_t slices)
{
    // one (m, s) pair per (row, workgroup); no counters
    return (uint64_t)(rows * (int64_t)slices * 8);
}

// Split-K geometry shared by the reduce, softmax and layernorm tiers: G
// workgroups per row; the row is cut into tiles of one load round of a
// workgroup (the kernels give each workgroup its own tiles: a contiguous run
// in the row reduction, every G-th tile in softmax and layernorm).
static void fill_splitk_geometry(int64_t rows, int64_t cols, int64_t tile, int32_t cu_count,
                                 int blocks_per_cu, rr_plan* out)
{
    const int64_t ntiles = ceil_div(cols > 0 ? cols : 1, tile);
    int64_t g = ceil_div((int64_t)blocks_per_cu * cu_count, rows > 0 ? rows : 1);
    int64_t g_cap = ceil_div(cols, kSplitKMinColsPerGroup);
    if (g_cap > kSplitKMaxSlices) g_cap = kSplitKMaxSlices;
    if (g_cap > ntiles) g_cap = ntiles;  // every workgroup gets at least one tile
    if (g > g_cap) g = g_cap;
    if (g < 1) g = 1;
    out->tier = RR_TIER_SPLITK;
    out->block = kBlockThreads;
    out->lanes_per_row = 0;
    out->slices = (int32_t)g;
    out->tile_cols = tile;
    out->grid = rows * g;
}

static rr_tier auto_tier_reduce(int64_t rows, int64_t cols, int32_t cu)
{
    if (rows < cu && cols >= kSplitKMinCols) return RR_TIER_SPLITK;
    if (cols <= 8) return RR_TIER_TILED;
    if (cols <= 64) return RR_TIER_WAVE;
    return RR_TIER_BLOCK;
}

static void fill_rowwise_geometry(rr_tier tier, int64_t rows, int64_t cols, int vec_elems,
                                  rr_plan* p)
{
    p->tier = tier;
    p->block = kBlockThreads;
    p->lanes_per_row = 0;
    p->slices = 1;
    p->tile_cols = 0;
    p->workspace_bytes = 0;
    switch (tier) {
    case RR_TIER_WAVE: {
        int s = wave_lanes_for_chunks(ceil_div(cols, vec_elems));
        p->lanes_per_row = s;
        int64_t rows_per_block = (int64_t)kWavesPerBlock * (64 / s) * kWaveRowGroups;
        p->grid = ceil_div(rows, rows_per_block);
        break;
    }
    case RR_TIER_TILED:
        p->grid = ceil_div(rows, (int64_t)kBlockThreads * kTiledRows);
        break;
    case RR_TIER_SERIAL:
        p->grid = ceil_div(rows, (int64_t)kBlockThreads);
        break;
    default:  // BLOCK: one workgroup per row (persistent rows set their own grid)
        p->grid = rows;
        break;
    }
    if (p->grid > kMaxGrid) p->grid = kMaxGrid;
}

RowPfShape reduce_pf_shape(int64_t rows, int64_t cols, rr_op op, int32_t cu_count, bool vec)
{
    (void)op;  // every statistic, the three-statistic tuple too
    if (!vec || cols < 1 || rows < kReducePfMinRowsPerCU * cu_count)
        return RowPfShape{0, 0};
    const int64_t chunks = ceil_div(cols, 4);
    // up to 128 chunks: a wavefront of 4 chunks per lane over 2 or 4 rows
    return chunks <= 128 ? RowPfShape{64, 4} : row_pf_shape(chunks);
}

int reduce_pf_lanes(int64_t cols, int64_t ld)
{
    const int64_t chunks = ceil_div(cols, 4);
    const int lanes = chunks <= 64 ? 16 : chunks <= 128 ? 32 : 0;
    // a step's rows share one buffer descriptor: its bytes must stay below 2^31
    if (lanes && ((int64_t)(64 / lanes - 1) * ld + cols) * 4 + 64 > (int64_t)INT32_MAX)
        return 0;
    return lanes;
}

rr_status plan_reduce(int64_t rows, int64_t cols, int64_t ld, rr_dtype dtype, rr_op op,
                      rr_tier tier, int32_t cu_count, bool vec, rr_plan* out)
{
    if (!out) return RR_ERR_NULL;
    if (rows < 0 || cols < 0 || ld < cols) return RR_ERR_SHAPE;
    if (dtype != RR_F32 && dtype != RR_I32) return RR_ERR_DTYPE;
    if (op != RR_SUM && op != RR_MAX && op != RR_MIN && op != RR_SUM_MAX_MIN) return RR_ERR_OP;
    if (cu_count < 1) return RR_ERR_SHAPE;
    if ((int)tier < RR_TIER_AUTO || (int)tier > RR_TIER_SPLITK) return RR_ERR_TIER;

    rr_tier t = tier == RR_TIER_AUTO ? auto_tier_reduce(rows, cols, cu_count) : tier;
    if (t == RR_TIER_WAVE && cols > 64) return RR_ERR_TIER;

    memset(out, 0, sizeof *out);
    const int vec_elems = vec ? 4 : 1;
    if (t != RR_TIER_SPLITK) {
        // the wave tier takes 128-bit chunks for rows of at least 7 elements
        // (every row then has a whole chunk after its head)
        fill_rowwise_geometry(t, rows, cols, t == RR_TIER_WAVE && cols < 7 ? 1 : vec_elems, out);
        const RowPfShape sh = reduce_pf_shape(rows, cols, op, cu_count, vec);
        if (t == RR_TIER_BLOCK && sh.nt > 0) {
            // persistent rows: workgroups sized to the row (or a wavefront
            // over 2 or 4 short rows), grid sized to the CUs
            const int lanes = reduce_pf_lanes(cols, ld);
            const int64_t steps = lanes ? ceil_div(rows, (int64_t)(sh.nt / lanes)) : rows;
            out->block = sh.nt;
            out->lanes_per_row = lanes;
            const int64_t g = (int64_t)cu_count * row_pf_blocks_per_cu(sh, kReducePfLoadsPerCU);
            out->grid = steps < g ? steps : g;
        }
        return RR_OK;
    }
    fill_splitk_geometry(rows, cols, (int64_t)kSplitKUnroll * kBlockThreads * vec_elems, cu_count,
                         kSplitKBlocksPerCU, out);
    out->workspace_bytes = splitk_workspace_bytes(rows, out->slices, op == RR_SUM_MAX_MIN ? 16 : 8);
    return RR_OK;
}

// The workspace must not depend on row alignment (the binding sizes it before
// it knows the pointers): a tile never exceeds the columns that justify one
// more workgroup, so the tile count never caps G below that bound.
static_assert((int64_t)kSoftmaxSplitKUnroll * kBlockThreads * 8 <= kSplitKMinColsPerGroup,
              "softmax split-K tile larger than the per-workgroup column minimum");
static_assert((int64_t)kSplitKUnroll * kBlockThreads * 4 <= kSplitKMinColsPerGroup,
              "reduce split-K tile larger than the per-workgroup column minimum");
static_assert((int64_t)kLnSplitKUnroll * kBlockThreads * 8 <= kSplitKMinColsPerGroup,
              "layernorm split-K tile larger than the per-workgroup column minimum");

// AUTO tier of the two-pass row operations (softmax, layernorm): split-K when
// there are fewer rows than CUs and the row is long, or when the row is too
// long to stay in registers (more than kPfMaxChunks 16-byte chunks) at any
// row count -- the split-K passes stream such rows better than one workgroup
// per row (measured: [4096, 32768] bf16 softmax 143 -> 127 us, layernorm
// 189 -> 137 us; [256, 65536] 35 -> 18 us and 64 -> 24 us); else the
// reduce's rule by row length.
rr_tier auto_two_pass_tier(int64_t rows, int64_t cols, rr_dtype x_dtype, int32_t cu_count)
{
    const int64_t chunks = ceil_div(cols, x_dtype == RR_BF16 ? 8 : 4);
    if ((rows < cu_count && cols >= kSplitKMinCols) || chunks > kPfMaxChunks)
        return RR_TIER_SPLITK;
    return cols <= 8 ? RR_TIER_TILED : cols <= 64 ? RR_TIER_WAVE : RR_TIER_BLOCK;
}

rr_status plan_softmax(int64_t rows, int64_t cols, rr_dtype x_dtype, rr_dtype y_dtype,
                       rr_tier tier, int32_t cu_count, bool vec, bool rows16, rr_plan* out)
{
    if (!out) return RR_ERR_NULL;
    if (rows < 0 || cols < 0) return RR_ERR_SHAPE;
    if ((x_dtype != RR_F32 && x_dtype != RR_BF16) || (y_dtype != RR_F32 && y_dtype != RR_BF16))
        return RR_ERR_DTYPE;
    if (cu_count < 1) return RR_ERR_SHAPE;
    if ((int)tier < RR_TIER_AUTO || (int)tier > RR_TIER_SPLITK) return RR_ERR_TIER;
    rr_tier t = tier;
    if (t == RR_TIER_AUTO)
        t = auto_two_pass_tier(rows, cols, x_dtype, cu_count);
    if (t == RR_TIER_WAVE && cols > 64) return RR_ERR_TIER;
    memset(out, 0, sizeof *out);
    const int chunk = x_dtype == RR_BF16 ? 8 : 4;
    const int vec_elems = vec ? chunk : 1;
    if (t == RR_TIER_SPLITK) {
        fill_splitk_geometry(rows, cols, (int64_t)kSoftmaxSplitKUnroll * kBlockThreads * vec_elems,
                             cu_count, kSplitKHeavyBlocksPerCU, out);
        out->workspace_bytes = softmax_splitk_workspace_bytes(rows, out->slices);
        return RR_OK;
    }
    fill_rowwise_geometry(t, rows, cols, t == RR_TIER_WAVE ? (rows16 ? chunk : 1) : vec_elems, out);
    if (t == RR_TIER_BLOCK) {
        const int64_t chunks = ceil_div(cols, vec_elems);
        const RowPfShape sh = row_pf_shape(chunks);
        if (vec && sh.nt > 0) {
            // rows that stay in registers: persistent workgroups sized to the
            // row, with a one-row prefetch (each row's body of whole chunks
            // from its first 16-byte boundary, the rest element by element)
            out->block = sh.nt;
            const int64_t g = (int64_t)cu_count * row_pf_blocks_per_cu(sh);
            out->grid = rows < g ? rows : g;
        } else if (chunks > kSoftmaxWideMinChunks) {
            out->block = kSoftmaxWideThreads;
        }
    }
    return RR_OK;
}

// Layernorm: the softmax's tier rule.  The block tier keeps rows of whole
// aligned chunks in registers on persistent workgroups sized by row_pf_shape,
// row_pf_blocks_per_cu of them per CU (the launch lowers that to what the
// kernel's occupancy allows, so a persistent grid never queues).
rr_status plan_layernorm(int64_t rows, int64_t cols, rr_dtype x_dtype, rr_dtype y_dtype,
                         rr_dtype w_dtype, rr_tier tier, int32_t cu_count, bool vec,
                         bool rows16, rr_plan* out)
{
    if (!out) return RR_ERR_NULL;
    if (rows < 0 || cols < 0) return RR_ERR_SHAPE;
    if ((x_dtype != RR_F32 && x_dtype != RR_BF16) || (y_dtype != RR_F32 && y_dtype != RR_BF16) ||
        (w_dtype != RR_F32 && w_dtype != RR_BF16))
        return RR_ERR_DTYPE;
    if (cu_count < 1) return RR_ERR_SHAPE;
    if ((int)tier < RR_TIER_AUTO || (int)tier > RR_TIER_SPLITK) return RR_ERR_TIER;
    rr_tier t = tier;
    if (t == RR_TIER_AUTO)
        t = auto_two_pass_tier(rows, cols, x_dtype, cu_count);
    if (t == RR_TIER_WAVE && cols > 64) return RR_ERR_TIER;
    memset(out, 0, sizeof *out);
    const int chunk = x_dtype == RR_BF16 ? 8 : 4;
    const int vec_elems = vec ? chunk : 1;
    if (t == RR_TIER_SPLITK) {
        fill_splitk_geometry(rows, cols, (int64_t)kLnSplitKUnroll * kBlockThreads * vec_elems,
                             cu_count, kSplitKHeavyBlocksPerCU, out);
        out->workspace_bytes = (uint64_t)(rows * (int64_t)out->slices * 16);
        return RR_OK;
    }
    fill_rowwise_geometry(t, rows, cols, t == RR_TIER_WAVE ? (rows16 ? chunk : 1) : vec_elems, out);
    // persistent rows: rows that all start 16-byte aligned and are whole
    // chunks keep each thread's gamma / beta in registers; the others read
    // them per row (k_layernorm_rows_peel)
    (void)rows16;
    if (t == RR_TIER_BLOCK && vec && cols > 0) {
        const RowPfShape sh = row_pf_shape(ceil_div(cols, (int64_t)chunk));
        if (sh.nt > 0) {
            out->block = sh.nt;
            const int64_t g = (int64_t)cu_count * row_pf_blocks_per_cu(sh);
            out->grid = rows < g ? rows : g;
        }
    }
    return RR_OK;
}

// Reduction over the middle axis of [outer][axis][inner].  TILED: a thread
// per 4 adjacent outputs (1 on the scalar path); SERIAL: a thread per output;
// SPLITK: workgroup tiles of output groups x axis lanes over G axis slices
// (partials, then a fold).  Block and wave have no meaning here.
rr_status plan_axis(int64_t outer, int64_t axis, int64_t inner, rr_dtype dtype, rr_op op,
                    rr_tier tier, int32_t cu_count, bool vec, rr_plan* out)
{
    if (!out) return RR_ERR_NULL;
    if (outer < 0 || axis < 0 || inner < 0) return RR_ERR_SHAPE;
    int64_t n = 0;
    if (__builtin_mul_overflow(outer, inner, &n) || __builtin_mul_overflow(n, axis, &n))
        return RR_ERR_SHAPE;
    if (dtype != RR_F32 && dtype != RR_I32) return RR_ERR_DTYPE;
    if (op != RR_SUM && op != RR_MAX && op != RR_MIN) return RR_ERR_OP;
    if (cu_count < 1) return RR_ERR_SHAPE;
    if (tier != RR_TIER_AUTO && tier != RR_TIER_TILED && tier != RR_TIER_SERIAL &&
        tier != RR_TIER_SPLITK)
        return RR_ERR_TIER;
    memset(out, 0, sizeof *out);
    const int64_t v = (vec && inner % 4 == 0 && tier != RR_TIER_SERIAL) ? 4 : 1;
    const int64_t gpo = inner / v;  // output groups per outer index
    const int64_t nblk = ceil_div(outer * gpo, (int64_t)kBlockThreads);
    rr_tier t = tier;
    if (t == RR_TIER_AUTO)
        t = axis >= kAxisSplitKMinAxis &&
                    (nblk < (int64_t)kAxisSplitKMaxBlocksPerCU * cu_count || gpo < kAxisNarrowGroups)
                ? RR_TIER_SPLITK
                : RR_TIER_TILED;
    out->tier = t;
    out->block = kBlockThreads;
    out->lanes_per_row = (int32_t)v;
    out->slices = 1;
    out->grid = nblk;
    if (t == RR_TIER_SPLITK) {
        // workgroup tiles of GW output groups x AL axis lanes, per outer index
        const int gwl = axis_tile_log2(gpo);
        const int64_t lanes = kBlockThreads >> gwl;
        const int64_t tiles = outer * ceil_div(gpo, (int64_t)1 << gwl);
        int64_t g = ceil_div((int64_t)kAxisSplitKBlocksPerCU * cu_count, tiles > 0 ? tiles : 1);
        int64_t cap = ceil_div(axis, lanes * kAxisMinStepsPerLane);
        if (cap > kAxisMaxSlices) cap = kAxisMaxSlices;
        if (g > cap) g = cap;
        if (g < 1) g = 1;
        out->slices = (int32_t)g;
        out->tile_cols = ceil_div(axis > 0 ? axis : 1, g);
        out->grid = tiles * g;
        out->workspace_bytes = (uint64_t)(g * outer * inner * 8);
    }
    if (out->grid > kMaxGrid) out->grid = kMaxGrid;
    return RR_OK;
}

}  // namespace rr

extern "C" rr_status rr_plan_axis(int64_t outer, int64_t axis, int64_t inner, rr_dtype dtype,
                                  rr_op op, rr_tier tier, int32_t cu_count, rr_plan* plan_out)
{
    return rr::plan_axis(outer, axis, inner, dtype, op, tier, cu_count, true, plan_out);
}

extern "C" rr_status rr_plan_layernorm(int64_t rows, int64_t cols, rr_dtype x_dtype,
                                       rr_dtype y_dtype, rr_dtype w_dtype, rr_tier tier,
                                       int32_t cu_count, rr_plan* plan_out)
{
    return rr::plan_layernorm(rows, cols, x_dtype, y_dtype, w_dtype, tier, cu_count, true, true,
                              plan_out);
}

extern "C" rr_status rr_plan_reduce(int64_t rows, int64_t cols, int64_t ld, rr_dtype dtype,
                                    rr_op op, rr_tier tier, int32_t cu_count, rr_plan* plan_out)
{
    return rr::plan_reduce(rows, cols, ld, dtype, op, tier, cu_count, true, plan_out);
}

extern "C" rr_status rr_plan_softmax(int64_t rows, int64_t cols, rr_dtype x_dtype,
                                     rr_dtype y_dtype, rr_tier tier, int32_t cu_count,
                                     rr_plan* plan_out)
{
    return rr::plan_softmax(rows, cols, x_dtype, y_dtype, tier, cu_count, true, true, plan_out);
}

extern "C" const char* rr_status_string(rr_status s)
{
    switch (s) {
    case RR_OK: return "ok";
    case RR_ERR_NULL: return "a required pointer is NULL";
    case RR_ERR_SHAPE: return "invalid shape or value (negative size, ld < cols, P/depth out of range, or eps negative or not finite)";
    case RR_ERR_DTYPE: return "unsupported dtype or dtype combination";
    case RR_ERR_TIER: return "forced tier is not legal for this shape or operation";
    case RR_ERR_WORKSPACE: return "split-K workspace missing or too small";
    case RR_ERR_HIP: return "HIP runtime error";
    case RR_ERR_OP: return "unknown reduction op";
    case RR_ERR_SCRATCH: return "the shape needs more split-K workspace than the library's "
                                "scratch array holds (RR_NOALLOC_SCRATCH_BYTES); pass a "
                                "workspace to rr_reduce_rows instead";
    }
    return "unknown status";
}

extern "C" int rr_version(void) { return RR_VERSION; }
