/*
 * rr.h -- deterministic row reductions on AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Eight operations:
 *
 *   rr_reduce_rows       sum / max / min of every row over its last axis, on
 *                        float32 or int32 values, through one of five tiers
 *                        (wave, block, tiled, serial, split-K).
 *   rr_reduce_rows_multi sum, max and min of every row over one read.
 *   rr_reduce_axis       sum / max / min over the middle axis of
 *                        [outer][axis][inner] (a non-last axis).
 *   rr_softmax_rows      two-pass softmax of every row (pass 1: the online
 *                        (max, sum) monoid; pass 2: a map that writes y).
 *   rr_layernorm_rows    two-pass layer normalisation of every row (pass 1:
 *                        mean and variance; pass 2: a map that writes y).
 *   rr_splitk_lse_merge  combine P split-K partial attention outputs by their
 *                        per-row (max, sum) statistics into bf16 or f32 rows.
 *   rr_splitk_attention_partials
 *                        the producer of those partials: attention of every
 *                        query row over each of P partitions of the keys, with
 *                        the partition's row max and row sum (matrix cores).
 *   rr_splitk_attention  both in one launch: the last workgroup of each
 *                        query tile to finish folds its P partials in
 *                        partition order into the output rows.
 *
 * Sources (Modular API pages, cited by title and section):
 *   "reduce" (algorithm.gpu.rowwise): the tier semantics list and the
 *       state-carrying overload -- a monoid state folded along the reduce
 *       axis, and the two-pass softmax whose second pass is a pure map.
 *   "cluster_allreduce": description and Parameters -- a combine_fn that is an
 *       associative add/max/min over 32-bit elements, and a cross-group fold
 *       that visits peers in rank order so every run gives the same bits.
 *   "fa4_splitk_reduce_scatter_write": the per-band steps -- each partition's
 *       output is scaled by its weight, the partitions are accumulated, and
 *       the result is packed to bf16; every partition, empty or not, joins.
 *
 * Conventions for every call below
 *   - Pointers named x, y, gamma, beta, mean_out, rstd_out, o_part, m_part,
 *     l_part, out and workspace are
 *     DEVICE pointers on the current HIP device.  The caller owns them.  The
 *     library never allocates or frees device memory and never synchronises.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every launch is asynchronous on that stream.
 *   - Arguments are validated before any launch: on any error status nothing
 *     has been launched and no output byte has been written.  After a launch
 *     the HIP launch status is checked and reported as RR_ERR_HIP.
 *   - Rows are laid out with a stride `ld` (in elements) between row starts;
 *     the last axis is contiguous (stride 1).  Rows may start at any element
 *     offset: the block, wave and split-K tiers load each row's body from its
 *     first 16-byte boundary with 128-bit loads and its head and tail (the
 *     elements before that boundary and after the last whole 16 bytes) one
 *     element at a time ("reduce", algorithm.gpu.rowwise, tier semantics:
 *     the full-width tile function on aligned chunks, the one-element one on
 *     the rest); outputs are stored 128 bits at a time where they are aligned
 *     for it.  Only bytes of the rows' elements are read or written.  The
 *     tiled and serial tiers, the softmax and layernorm wave tiers and the
 *     layernorm's persistent rows take 128-bit loads only when every row is
 *     16-byte aligned; pointers not aligned to their element size run every
 *     tier element by element.
 *   - Results are bit-identical from run to run for the same device, shape,
 *     strides, alignment, tier and library build.
 *   - No C++ exception crosses this interface.
 *   - The library prints nothing, unless the environment variable RR_LOG is
 *     "1" when a call is made: then every call that launches writes one line
 *     to stderr with its dimensions, vector path and plan (tier, workgroup
 *     size, grid, lanes per row, slices, tile columns, workspace bytes).
 */
#ifndef RR_H
#define RR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RR_VERSION 1

typedef enum {
    RR_OK = 0,
    RR_ERR_NULL = 1,      /* a required pointer is NULL */
    RR_ERR_SHAPE = 2,     /* negative size, ld < cols, P out of range, ... */
    RR_ERR_DTYPE = 3,     /* unsupported dtype or dtype combination */
    RR_ERR_TIER = 4,      /* forced tier is not legal for this shape / kind */
    RR_ERR_WORKSPACE = 5, /* split-K workspace missing or too small */
    RR_ERR_HIP = 6,       /* a HIP runtime call or launch failed */
    RR_ERR_OP = 7,        /* unknown reduction op */
    RR_ERR_SCRATCH = 8    /* rr_reduce_rows_noalloc: the plan's split-K workspace is
                             larger than RR_NOALLOC_SCRATCH_BYTES */
} rr_status;

typedef enum { RR_F32 = 0, RR_I32 = 1, RR_BF16 = 2 } rr_dtype;

/* RR_SUM_MAX_MIN names the three statistics of rr_reduce_rows_multi in the
 * planner queries (rr_plan_reduce, rr_workspace_bytes); rr_reduce_rows rejects
 * it with RR_ERR_OP. */
typedef enum { RR_SUM = 0, RR_MAX = 1, RR_MIN = 2, RR_SUM_MAX_MIN = 3 } rr_op;

/* Tiers of "reduce" (algorithm.gpu.rowwise), tier semantics. */
typedef enum {
    RR_TIER_AUTO = 0,   /* pick by the rule documented at rr_plan_reduce */
    RR_TIER_WAVE = 1,   /* a group of lanes of one 64-wide wavefront per row (cols <= 64) */
    RR_TIER_BLOCK = 2,  /* a workgroup per row at a time, strided 128-bit loads */
    RR_TIER_TILED = 3,  /* one thread owns RR_TILED_ROWS adjacent rows, no cross-thread combine */
    RR_TIER_SERIAL = 4, /* one thread per row, element by element */
    RR_TIER_SPLITK = 5  /* several workgroups per row, rank-order fold of partials */
} rr_tier;

typedef enum { RR_KIND_REDUCE = 0, RR_KIND_SOFTMAX = 1, RR_KIND_LAYERNORM = 2 } rr_kind;

/* Rows owned by one thread in the tiled tier (the page's emit_tile_width). */
#define RR_TILED_ROWS 4
/* Bytes of device memory per GPU that rr_reduce_rows_noalloc uses as its
 * split-K workspace (a scratch array inside the library). */
#define RR_NOALLOC_SCRATCH_BYTES (1 << 20)
/* Largest partition count accepted by rr_splitk_lse_merge. */
#define RR_MERGE_MAX_P 256

/*
 * Launch plan: what the library will run for a shape.  Host-only, no device
 * work; filled by rr_plan_reduce / rr_plan_softmax.
 */
typedef struct {
    int32_t tier;            /* rr_tier actually used (never RR_TIER_AUTO) */
    int32_t block;           /* threads per workgroup */
    int64_t grid;            /* workgroups launched */
    int32_t lanes_per_row;   /* wave tier: lanes that share one row; else 0 */
    int32_t slices;          /* split-K: workgroups per row (G); else 1 */
    int64_t tile_cols;       /* split-K: columns per tile (the last tile of a row may be
                                shorter); of a row's T tiles, workgroup g folds the
                                contiguous run [g*T/G, (g+1)*T/G) in the row reduction,
                                and tiles g, g+G, g+2G, ... in softmax and layernorm;
                                else 0 */
    uint64_t workspace_bytes;/* bytes of workspace the call needs (0 if none) */
} rr_plan;

/*
 * rr_plan_reduce -- tier selection and launch geometry for rr_reduce_rows.
 * Pure host computation (no HIP call), deterministic in its arguments.
 * cu_count is the device's compute-unit count (256 on MI355X).
 *
 * "reduce" (algorithm.gpu.rowwise), tier semantics, gives each tier's shape
 * of work but no thresholds; this library picks, first match wins:
 *   forced tier (if legal for the shape)
 *   SPLITK  if rows < cu_count and cols >= 65536
 *   TILED   if cols <= 8
 *   WAVE    if cols <= 64
 *   BLOCK   otherwise
 * SERIAL is used only when forced.  WAVE is legal for cols <= 64 only.
 * BLOCK with at least 4 * cu_count rows of c <= 2048 16-byte chunks (also
 * for RR_SUM_MAX_MIN): persistent workgroups sized to the row, n = 4 chunks
 * per thread -- a wavefront over 4 rows of 16 lanes (lanes_per_row = 16) for
 * c <= 64 or over 2 rows of 32 lanes for c <= 128 (when 3 or 1 row strides
 * plus the row stay below 2^31 bytes; else one row of 64 lanes), 64 threads
 * for c <= 256, then 128, 256 and 512 threads for c <= 512, 1024 and 2048 --
 * and grid = min(steps, cu_count * max(1, 64 / (block / 64 * n))), steps =
 * rows divided by the rows per step, rounded up; otherwise one workgroup of
 * 256 threads per row.
 * SPLITK: G = clamp(ceil(2*cu_count/rows), 1, min(256, ceil(cols/16384), tiles))
 * with tiles = ceil(cols / tile_cols), tile_cols = 8192 (2048 on the scalar path).
 * Workspace: rows * 4 ticket bytes padded to 256, then rows * G partials of 8
 * bytes (16 for RR_SUM_MAX_MIN).
 * Returns RR_ERR_SHAPE for negative sizes or ld < cols, RR_ERR_DTYPE/OP for
 * unsupported dtype/op, RR_ERR_TIER for an illegal forced tier.
 */
rr_status rr_plan_reduce(int64_t rows, int64_t cols, int64_t ld, rr_dtype dtype, rr_op op,
                         rr_tier tier, int32_t cu_count, rr_plan* plan_out);

/*
 * rr_plan_softmax -- tier selection for rr_softmax_rows: SPLITK when
 * rows < cu_count and cols >= 65536, or when a row spans more than 2048
 * 16-byte chunks (cols > 16384 for bf16 input, > 8192 for float32) at any
 * row count -- too long to stay in registers; else TILED (cols <= 8), WAVE
 * (cols <= 64), BLOCK.  BLOCK: rows of whole 16-byte chunks (c chunks, c <= 2048, aligned)
 * run persistent workgroups sized to the row -- (threads, chunks per thread)
 * = (64, 1) for c <= 64, (64, 2) <= 128, (64, 4) <= 256, (128, 4) <= 512,
 * (256, 4) <= 1024, (512, 4) <= 2048 -- with 32 / (wavefronts x chunks per
 * thread) workgroups per CU (at least 1), lowered at launch to what the
 * kernel's occupancy allows; other rows take one workgroup of 256 threads
 * per row (512 beyond 2048 chunks, reached when BLOCK is forced), reading x
 * twice beyond 8 chunks per thread.  SPLITK uses tiles of 4 * 256 * 16-byte chunks (4 * 256 elements
 * on the scalar path), G as for rr_plan_reduce with that tile but
 * 4 * cu_count workgroups in all, and needs the workspace reported in
 * workspace_bytes (rows * G * 8).
 */
rr_status rr_plan_softmax(int64_t rows, int64_t cols, rr_dtype x_dtype, rr_dtype y_dtype,
                          rr_tier tier, int32_t cu_count, rr_plan* plan_out);

/*
 * rr_plan_layernorm -- tier selection for rr_layernorm_rows: the softmax rule,
 * with the same persistent BLOCK shapes; unaligned or ragged rows of up to 8
 * chunks per thread of 256 stay in registers one row per workgroup, longer
 * rows are read twice.  SPLITK tiles are 4 * 256 16-byte chunks, G as for the
 * softmax; its workspace is rows * G * 16 bytes (workspace_bytes).
 */
rr_status rr_plan_layernorm(int64_t rows, int64_t cols, rr_dtype x_dtype, rr_dtype y_dtype,
                            rr_dtype w_dtype, rr_tier tier, int32_t cu_count, rr_plan* plan_out);

/*
 * rr_reduce_rows -- y[r] = fold of x[r*ld + 0 .. r*ld + cols-1].
 * "reduce" (algorithm.gpu.rowwise), state-carrying overload and tier
 * semantics; "cluster_allreduce", description (rank-order fold).
 *
 *   x      device, [rows][ld] of dtype (cols elements of each row are read)
 *   y      device, [rows] of dtype (written)
 *   dtype  RR_F32 or RR_I32 (same type in and out)
 *   op     RR_SUM, RR_MAX or RR_MIN
 *   tier   RR_TIER_AUTO or a forced tier
 *   workspace, workspace_bytes
 *          device scratch for RR_TIER_SPLITK (ignored otherwise; may be NULL
 *          when the plan needs 0 bytes).  Size: rr_workspace_bytes.  It must
 *          be all zero before its first use (rr_workspace_reset); every
 *          completed call leaves every byte it used zero again (the last
 *          workgroup of a row resets the row's ticket and clears the partial
 *          slots it read), so calls of any shape may share one workspace.
 *          One workspace must not serve two calls in flight.
 *
 * Arithmetic: float SUM accumulates in double and rounds once to float
 * (nearest even); int32 SUM wraps modulo 2^32; MAX/MIN on float use the
 * IEEE 754 totalOrder (-0 < +0, NaNs ordered by sign and payload); cols == 0
 * writes the identity (0, -inf / INT32_MIN for MAX, +inf / INT32_MAX for MIN).
 * The split-K tier writes one partial per (row, workgroup) into the workspace
 * and the last workgroup of a row to arrive folds the partials in ascending
 * workgroup order, so the result does not depend on arrival order.
 * rows == 0 is a no-op.
 */
rr_status rr_reduce_rows(const void* x, void* y, int64_t rows, int64_t cols, int64_t ld,
                         rr_dtype dtype, rr_op op, rr_tier tier, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * rr_reduce_rows_noalloc -- rr_reduce_rows for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  Arguments, results and errors as
 * rr_reduce_rows, without the workspace: the split-K tier uses a scratch
 * array inside the library instead, RR_NOALLOC_SCRATCH_BYTES (1 MiB) of
 * device memory per GPU, which each GPU the call runs on holds from the
 * first call there until the process ends.  The call allocates nothing
 * (no hipMalloc, no allocating library routine).  The same plan and kernels
 * as rr_reduce_rows run, so the results are bit-identical to it.
 *
 *   x, y, rows, cols, ld, dtype, op, tier, stream   as rr_reduce_rows
 *
 * Split-K: the first call on a device looks up the device address of that
 * GPU's copy of the array (RR_ERR_HIP if that fails); every split-K call
 * then clears the bytes it uses with a fill kernel on `stream` (tickets must
 * start at zero; the array keeps what the previous call left) before its
 * reduction launch.  Every call on one GPU shares that GPU's array: calls
 * that overlap in time on one GPU (two streams, or two host threads) race
 * and give wrong results.  Returns RR_ERR_SCRATCH, launching nothing, when
 * the plan's workspace (rr_workspace_bytes) exceeds RR_NOALLOC_SCRATCH_BYTES
 * (a forced split-K over very many rows; an automatic split-K plan has
 * rows < CU count and needs at most a few KiB).  Tiers other than split-K
 * use no workspace and behave exactly as rr_reduce_rows.
 */
rr_status rr_reduce_rows_noalloc(const void* x, void* y, int64_t rows, int64_t cols, int64_t ld,
                                 rr_dtype dtype, rr_op op, rr_tier tier, void* stream);

/*
 * rr_reduce_rows_multi -- the sum, the maximum and the minimum of every row
 * over one read of x.  "reduce" (algorithm.gpu.rowwise), description: the
 * body combines each state that needs a cross-thread combine on its own;
 * here the three states travel together through every fold, each combined
 * by its own operation with the arithmetic of rr_reduce_rows (so each output
 * equals, bit for bit, what rr_reduce_rows gives for that op on the same
 * tier).
 *
 *   x                   device, [rows][ld] of dtype (RR_F32 or RR_I32)
 *   y_sum, y_max, y_min device, [rows] of dtype, or NULL (not computed into
 *                       memory); at least one must be non-NULL (RR_ERR_NULL)
 *   tier, workspace, workspace_bytes
 *                       as rr_reduce_rows; the split-K workspace holds
 *                       16-byte partials (rr_workspace_bytes with op
 *                       RR_SUM_MAX_MIN), tickets zero before first use and
 *                       left zero by every completed call.
 * rows == 0 is a no-op; cols == 0 writes each identity.
 */
rr_status rr_reduce_rows_multi(const void* x, void* y_sum, void* y_max, void* y_min,
                               int64_t rows, int64_t cols, int64_t ld, rr_dtype dtype,
                               rr_tier tier, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * rr_plan_axis -- tier selection and geometry for rr_reduce_axis (host only).
 * Legal tiers: AUTO, TILED, SERIAL, SPLITK (others: RR_ERR_TIER).  With g the
 * output groups (outer * inner / 4 when inner % 4 == 0, else outer * inner),
 * per outer index gpo = g / outer and B = ceil(g / 256): AUTO picks SPLITK
 * when axis >= 512 and (B < cu_count or gpo < 64), else TILED.  SPLITK
 * workgroups are tiles of GW = min(64, gpo rounded up to a power of two)
 * output groups by AL = 256 / GW axis lanes; with T tiles, G =
 * clamp(ceil(2 * cu_count / T), 1, min(1024, ceil(axis / (32 * AL)))) slices
 * of ceil(axis / G) steps (tile_cols); workspace G * outer * inner * 8
 * bytes.  lanes_per_row holds the outputs per thread (4 or 1).  The planner
 * assumes 16-byte aligned pointers.
 */
rr_status rr_plan_axis(int64_t outer, int64_t axis, int64_t inner, rr_dtype dtype, rr_op op,
                       rr_tier tier, int32_t cu_count, rr_plan* plan_out);

/*
 * rr_reduce_axis -- y[o][i] = fold over a of x[o][a][i]: a reduction over a
 * non-last axis.  "reduce" (algorithm.gpu.rowwise), Args (ctx.axis is the
 * reduce axis, the other dims pinned) and tier semantics (the tiled tier's
 * thread owns emit_tile_width adjacent output rows and sends each lane of a
 * tile to its own state).  Same arithmetic as rr_reduce_rows.
 *
 *   x       device, [outer][axis][inner] of dtype, contiguous
 *   y       device, [outer][inner] of dtype (written)
 *   dtype   RR_F32 or RR_I32;  op  RR_SUM, RR_MAX or RR_MIN
 *   tier    AUTO, TILED (a thread owns 4 adjacent outputs -- 1 when inner is
 *           not a multiple of 4 or a pointer is not 16-byte aligned -- and
 *           walks the whole axis in order), SERIAL (a thread per output), or
 *           SPLITK (G axis slices, AL axis lanes per output group in each:
 *           partials folded in lane order, then a fold in ascending slice
 *           order, two launches)
 *   workspace, workspace_bytes
 *           device scratch for SPLITK, 8-byte aligned, size from
 *           rr_plan_axis; no initial contents needed.  Ignored otherwise.
 * TILED and SERIAL fold each output in the index order of the axis, so a
 * float sum equals the double sum in that order rounded once.  outer or
 * inner == 0 is a no-op; axis == 0 writes the identity.  inner == 1 is a
 * row reduction, which rr_reduce_rows does faster.
 */
rr_status rr_reduce_axis(const void* x, void* y, int64_t outer, int64_t axis, int64_t inner,
                         rr_dtype dtype, rr_op op, rr_tier tier, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * rr_softmax_rows -- y[r][j] = exp(x[r][j] - m_r) / s_r with
 * m_r = max_j x[r][j] and s_r = sum_j exp(x[r][j] - m_r).
 * "reduce" (algorithm.gpu.rowwise), description: pass 1 folds the online
 * (max, sum) monoid, pass 2 is a pure map that writes y.
 *
 *   x        device, [rows][ld_x] of x_dtype (RR_BF16 or RR_F32)
 *   y        device, [rows][ld_y] of y_dtype (RR_BF16 or RR_F32)
 *   tier     RR_TIER_AUTO, WAVE, BLOCK, TILED, SERIAL or SPLITK
 *   workspace, workspace_bytes
 *            device scratch for RR_TIER_SPLITK: rows * G * 8 bytes, 8-byte
 *            aligned (size: rr_workspace_bytes with RR_KIND_SOFTMAX).  No
 *            initial contents are needed; every call writes before it reads.
 *            Ignored by the other tiers (may be NULL).  One workspace must
 *            not serve two calls in flight, and a buffer used here must be
 *            zeroed (rr_workspace_reset) before it serves rr_reduce_rows,
 *            whose tickets live where this call writes its pairs.
 * Split-K ("reduce", tier semantics: several blocks per row; and
 * "cluster_allreduce", description: the all-gather variant, where every
 * group needs the folded value) runs two launches on the stream: G
 * workgroups per row fold (max, sum) over their tiles and store the pair;
 * then every workgroup of the map pass folds its row's G pairs in rank order
 * (M = max of the m_g, S = sum of s_g * exp(m_g - M) over a fixed tree with
 * the ranks as leaves, in double) and writes y over its tiles.  All
 * workgroups of a row fold the same pairs the same way, so they use the same
 * (M, S), and the result does not depend on scheduling.
 * Arithmetic in float32; bf16 results are rounded to nearest even.  y may
 * alias x only when ld_y == ld_x and the dtypes match.  cols == 0 or
 * rows == 0 is a no-op.
 */
rr_status rr_softmax_rows(const void* x, void* y, int64_t rows, int64_t cols, int64_t ld_x,
                          int64_t ld_y, rr_dtype x_dtype, rr_dtype y_dtype, rr_tier tier,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * rr_layernorm_rows -- layer normalisation of every row over its last axis.
 * "reduce" (algorithm.gpu.rowwise), description: layernorm is a two-pass
 * algorithm -- pass 1 reduces the row's statistics, each state combined
 * across threads on its own, pass 2 is a pure map.  The page gives no
 * formula; the standard one is used:
 *   mean_r = sum_j x[r][j] / cols
 *   var_r  = sum_j (x[r][j] - mean_r)^2 / cols        (population variance)
 *   rstd_r = 1 / sqrt(var_r + eps)
 *   y[r][j] = (x[r][j] - mean_r) * rstd_r * gamma[j] + beta[j]
 *
 *   x        device, [rows][ld_x] of x_dtype (RR_BF16 or RR_F32)
 *   y        device, [rows][ld_y] of y_dtype (RR_BF16 or RR_F32); may alias x
 *            only when ld_y == ld_x and the dtypes match
 *   gamma, beta  device, [cols] of w_dtype (RR_F32 or RR_BF16), or NULL
 *            (gamma 1, beta 0)
 *   mean_out, rstd_out  device, float [rows] (written), or NULL; must not
 *            overlap x or y
 *   eps      finite and >= 0 (else RR_ERR_SHAPE)
 *   tier     RR_TIER_AUTO, WAVE, BLOCK, TILED, SERIAL or SPLITK
 *   workspace, workspace_bytes
 *            device scratch for RR_TIER_SPLITK: rows * G * 16 bytes, 8-byte
 *            aligned (rr_workspace_bytes with RR_KIND_LAYERNORM); no initial
 *            contents needed.  Ignored by the other tiers (may be NULL).  As
 *            for rr_softmax_rows, a buffer used here must be zeroed before it
 *            serves rr_reduce_rows.
 * Statistics are formed in double (rows held in registers: the sum of x,
 * then the sum of squared deviations from the mean; streamed rows: sums of
 * x - x[r][0] and its square, whose cancellation Samuelson's inequality
 * bounds by log2(cols) bits), each combined over a fixed-shape tree so the
 * result does not change from run to run.  The map runs in float; bf16
 * results are rounded to nearest even.  Split-K (rows < CU and long rows, or
 * rows too long for registers):
 * G workgroups per row store their two sums, then every workgroup of the map
 * pass sums its row's G pairs over a fixed tree ("cluster_allreduce",
 * description: the all-gather variant) and maps its tiles.  rows == 0 or
 * cols == 0 is a no-op (nothing is written).
 */
rr_status rr_layernorm_rows(const void* x, void* y, const void* gamma, const void* beta,
                            float* mean_out, float* rstd_out, int64_t rows, int64_t cols,
                            int64_t ld_x, int64_t ld_y, rr_dtype x_dtype, rr_dtype y_dtype,
                            rr_dtype w_dtype, float eps, rr_tier tier, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * rr_splitk_lse_merge -- combine P split-K partitions of an attention output.
 * "fa4_splitk_reduce_scatter_write", the per-band steps: each partition's
 * output is scaled by its weight w[b], the partitions are accumulated, and
 * the result is packed to bf16; every partition joins, empty or not.
 *
 *   o_part  device, float32 [P][rows][depth]: partition p's NORMALISED output
 *           O_p (already divided by its own l_p)
 *   m_part  device, float32 [P][rows]: row max m_p of partition p's scores
 *   l_part  device, float32 [P][rows]: row sum l_p = sum exp(score - m_p)
 *   out     device, [rows][depth] of out_dtype (RR_BF16 or RR_F32)
 *   P       1 .. RR_MERGE_MAX_P;  rows >= 0;  depth >= 1
 *   scale   multiplies (m_p - M) inside the exponent (1.0 when m_p are
 *           already in natural-log units)
 * Per row: partition p is empty when l_p <= 0 or m_p == -inf; M = max m_p
 * over the non-empty ones; w_p = exp(scale*(m_p - M)) * l_p; W = sum w_p;
 * out = sum over non-empty p, in ascending p, of (w_p / W) * O_p, with
 * weights and accumulation in double and one rounding to out_dtype.  Empty
 * partitions are skipped (their O_p never enters the sum); a row with no
 * non-empty partition is written as zeros.  P == 1 reproduces O_1 exactly
 * (rounded once to out_dtype).
 */
rr_status rr_splitk_lse_merge(const float* o_part, const float* m_part, const float* l_part,
                              void* out, int32_t P, int64_t rows, int32_t depth, float scale,
                              rr_dtype out_dtype, void* stream);

/*
 * rr_splitk_attention_partials -- split-K attention partials, the inputs of
 * rr_splitk_lse_merge.  "fa4_splitk_reduce_scatter_write", per-band steps:
 * each partition's partial output carries its own row max and row sum, which
 * the merge uses to reweight it.
 *
 *   q       device, bf16 [batch][heads][q_rows][depth]
 *   k, v    device, bf16 [batch][kv_heads][kv_len][depth]; query head h of a
 *           batch reads key/value head h / (heads / kv_heads) (grouped heads;
 *           kv_heads == heads is plain multi-head attention)
 *   o_part  device, float32 [P][batch*heads*q_rows][depth] (written)
 *   m_part, l_part  device, float32 [P][batch*heads*q_rows] (written)
 *   depth   64 or 128;  P 1 .. RR_MERGE_MAX_P;  heads % kv_heads == 0;
 *           batch, q_rows, kv_len >= 0;  q_rows * depth * 2 < 2^31
 *   scale   finite; multiplies q . k (1/sqrt(depth) for standard attention)
 * The keys are cut into P contiguous partitions: partition p holds keys
 * p*kv_len/P .. (p+1)*kv_len/P - 1 (integer division).  For query row i and
 * partition p, with s_j = scale * q_i . k_j over the partition's keys:
 *   m_part[p][i] = max_j s_j,   l_part[p][i] = sum_j exp(s_j - m_part[p][i]),
 *   o_part[p][i][d] = sum_j exp(s_j - m_part[p][i]) * v_j[d] / l_part[p][i]
 * (normalised partials in natural-log units, so rr_splitk_lse_merge takes
 * them with scale 1.0).  A partition with no key is written as m = -inf,
 * l = 0, O = 0, which the merge skips.  Rows are ordered (batch, head, query
 * row).  q . k and P v accumulate in float32 on the matrix cores with the
 * probabilities rounded to bf16 as the second product's operand; the row
 * statistics are float32.  q, k, v and o_part must be 16-byte aligned.
 * Errors (nothing launched): RR_ERR_SHAPE (sizes, depth, P, alignment,
 * scale), RR_ERR_NULL; batch*heads*q_rows == 0 is a no-op.
 */
rr_status rr_splitk_attention_partials(const void* q, const void* k, const void* v, float* o_part,
                                       float* m_part, float* l_part, int64_t batch, int64_t heads,
                                       int64_t kv_heads, int64_t q_rows, int64_t kv_len,
                                       int32_t depth, int32_t P, float scale, void* stream);

/*
 * rr_splitk_attention_partials_varlen -- the partials of
 * rr_splitk_attention_partials for a batch of sequences of different lengths
 * packed token after token, each attending only to its own keys.
 * "fa4_splitk_reduce_scatter_write", signature and semantics: each output
 * tile is placed by a head index and a row index into a ragged [tokens]
 * [heads][depth] tensor, its row count cut to the sequence's length.
 *
 *   q             device, bf16 [total_q][heads][depth]
 *   k, v          device, bf16 [total_k][kv_heads][depth] (grouped heads as
 *                 rr_splitk_attention_partials)
 *   cu_seqlens_q  device, int32 [batch + 1], non-decreasing: sequence b owns
 *                 query tokens cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1
 *   cu_seqlens_k  device, int32 [batch + 1]: its keys cu_seqlens_k[b] ..
 *                 cu_seqlens_k[b+1] - 1.  Offsets are clamped into
 *                 [0, total_q] and [0, total_k] (a decreasing pair gives an
 *                 empty sequence); a sequence may have no query or no key.
 *   o_part        device, float32 [P][total_q][heads][depth] (written)
 *   m_part, l_part  device, float32 [P][total_q][heads] (written)
 *   max_q_rows    the query rows computed per sequence, normally the
 *                 longest sequence's count: a sequence's query rows past
 *                 it are not computed (left unwritten)
 *   depth, P, scale  as rr_splitk_attention_partials;
 *                 heads * depth * 512 < 2^31;  total_q, total_k < 2^31
 * For sequence b its keys are cut into P contiguous partitions as
 * rr_splitk_attention_partials cuts kv_len keys (partition p holds keys
 * p*n_b/P .. (p+1)*n_b/P - 1 of the sequence's n_b keys), and every
 * (token, head, partition) of the sequence gets m, l and O as there; a
 * partition with no key is written as m = -inf, l = 0, O = 0.  Tokens that
 * belong to no sequence are not written.  The rows of o_part, m_part and
 * l_part, (token, head) in token order, are the rows of rr_splitk_lse_merge
 * with rows = total_q * heads, which then writes the output as [total_q]
 * [heads][depth].  The cu_seqlens arrays are read on the device only.
 * q, k, v and o_part must be 16-byte aligned.
 * Errors (nothing launched): RR_ERR_SHAPE, RR_ERR_NULL; batch, total_q or
 * max_q_rows == 0 is a no-op.
 */
rr_status rr_splitk_attention_partials_varlen(const void* q, const void* k, const void* v,
                                              const int32_t* cu_seqlens_q,
                                              const int32_t* cu_seqlens_k, float* o_part,
                                              float* m_part, float* l_part, int64_t batch,
                                              int64_t heads, int64_t kv_heads, int64_t total_q,
                                              int64_t total_k, int64_t max_q_rows, int32_t depth,
                                              int32_t P, float scale, void* stream);

/*
 * rr_splitk_attention -- the whole split-K attention in one launch: the
 * partials of rr_splitk_attention_partials, combined as rr_splitk_lse_merge
 * combines them (scale 1.0), into one output row per query row.
 * "fa4_splitk_reduce_scatter_write" (the partials and their LSE weights) with
 * the rank-ordered fold of "cluster_allreduce": every (head, 128 query rows,
 * partition) workgroup writes its partial into the workspace and takes a
 * ticket for its (head, query rows) group; the workgroup that draws the last
 * ticket folds the group's P partials in ascending partition order.  The
 * result is bit-identical to rr_splitk_attention_partials followed by
 * rr_splitk_lse_merge(..., scale 1.0, out_dtype) on the same inputs, whatever
 * order the workgroups run in.
 *
 *   q, k, v     as rr_splitk_attention_partials
 *   out         device, out_dtype [batch][heads][q_rows][depth] (written),
 *               16-byte aligned
 *   out_dtype   RR_BF16 (rounded to nearest even) or RR_F32
 *   P           1 .. depth / 8 (the fold keeps P (m, l, weight) cells per row
 *               in LDS)
 *   workspace, workspace_bytes
 *               device, 16-byte aligned, at least the bytes_out of
 *               rr_splitk_attention_workspace_bytes; owned by the caller.
 *               Its first ticket_bytes_out bytes (same query) are the
 *               tickets and must be zero when the call starts; a completed
 *               call leaves them zero and overwrites the bytes after them
 *               with partials.  So a workspace that served a call with a
 *               smaller ticket region must have the bytes between the two
 *               ticket sizes cleared (rr_workspace_reset) before a call with
 *               a larger one, and one that then serves rr_reduce_rows must be
 *               reset first.  One workspace must not serve two calls in
 *               flight.
 * Errors (nothing launched): RR_ERR_SHAPE (as rr_splitk_attention_partials,
 * and P > depth / 8), RR_ERR_DTYPE, RR_ERR_NULL, RR_ERR_WORKSPACE;
 * batch*heads*q_rows == 0 is a no-op.
 */
rr_status rr_splitk_attention(const void* q, const void* k, const void* v, void* out,
                              rr_dtype out_dtype, int64_t batch, int64_t heads, int64_t kv_heads,
                              int64_t q_rows, int64_t kv_len, int32_t depth, int32_t P,
                              float scale, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace rr_splitk_attention needs for this shape (bytes_out)
 * and how many of its first bytes are tickets that must be zero when a call
 * starts (ticket_bytes_out, may be NULL): 4 per (head, 128 query rows),
 * rounded up to 256.  0 and 0 for a no-op shape; the same shape errors as
 * rr_splitk_attention.  Host only. */
rr_status rr_splitk_attention_workspace_bytes(int64_t batch, int64_t heads, int64_t kv_heads,
                                              int64_t q_rows, int64_t kv_len, int32_t depth,
                                              int32_t P, size_t* bytes_out,
                                              size_t* ticket_bytes_out);

/* Bytes of workspace rr_reduce_rows (RR_KIND_REDUCE), rr_softmax_rows
 * (RR_KIND_SOFTMAX, dtype = x_dtype) or rr_layernorm_rows (RR_KIND_LAYERNORM,
 * dtype = x_dtype) needs for this shape on the current
 * device (0 unless the plan is split-K). */
rr_status rr_workspace_bytes(rr_kind kind, int64_t rows, int64_t cols, rr_dtype dtype,
                             rr_op op, rr_tier tier, size_t* bytes_out);

/* Tier AUTO would pick for this shape on the current device. */
rr_status rr_select_tier(rr_kind kind, int64_t rows, int64_t cols, rr_dtype dtype, rr_op op,
                         rr_tier* tier_out);

/* Zero `bytes` of a workspace on `stream` with a fill kernel (no memset
 * node, so the call may be captured into a HIP graph).  Use it to recover a
 * workspace after an aborted call. */
rr_status rr_workspace_reset(void* workspace, size_t bytes, void* stream);

/* Compute units of the current device, as the library sees them. */
rr_status rr_device_cu_count(int32_t* cu_out);

/* Static text for a status code; never NULL. */
const char* rr_status_string(rr_status s);

/* RR_VERSION of the built library. */
int rr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RR_H */
