// rr_api.cpp -- the C ABI entry points of librr (see include/rr.h).
//
// Every entry point validates its arguments completely before it launches
// anything, then launches on the caller's stream and returns without
// synchronising.  No C++ exception leaves this file.
#include <hip/hip_runtime.h>

#include <atomic>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/rr.h"
#include "../../include/rr_test.h"
#include "rr_config.hpp"
#include "rr_launch.hpp"
#include "rr_plan.hpp"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int32_t> g_cu_count[kMaxDevices];
std::atomic<int32_t> g_splitk_skew{0};

rr_status current_cu(int32_t* cu)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return RR_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices) {
        int32_t c = g_cu_count[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *cu = c;
            return RR_OK;
        }
    }
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1)
        return RR_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(v, std::memory_order_relaxed);
    *cu = v;
    return RR_OK;
}

// RR_LOG=1 in the environment (read at every call): every call that
// launches prints its plan to stderr, one line.  Otherwise nothing is printed.
bool log_enabled()
{
    const char* e = getenv("RR_LOG");
    return e && e[0] == '1' && e[1] == '\0';
}

const char* tier_name(int32_t t)
{
    switch (t) {
    case RR_TIER_WAVE: return "wave";
    case RR_TIER_BLOCK: return "block";
    case RR_TIER_TILED: return "tiled";
    case RR_TIER_SERIAL: return "serial";
    case RR_TIER_SPLITK: return "splitk";
    default: return "auto";
    }
}

// dims: "rows=R cols=C", or "outer=O axis=A inner=I" for rr_reduce_axis.
void log_plan(const char* call, const char* d0, int64_t v0, const char* d1, int64_t v1,
              const char* d2, int64_t v2, bool vec, const rr_plan& p)
{
    if (!log_enabled())
        return;
    char extra[48] = "";
    if (d2)
        snprintf(extra, sizeof extra, " %s=%lld", d2, (long long)v2);
    fprintf(stderr,
            "rr: %s %s=%lld %s=%lld%s vec=%d tier=%s block=%d grid=%lld lanes_per_row=%d "
            "slices=%d tile_cols=%lld workspace=%llu\n",
            call, d0, (long long)v0, d1, (long long)v1, extra, (int)vec, tier_name(p.tier),
            p.block, (long long)p.grid, p.lanes_per_row, p.slices, (long long)p.tile_cols,
            (unsigned long long)p.workspace_bytes);
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Rows of `elem` bytes at stride `ld` elements start 16-byte aligned when the
// base is and the stride is a multiple of 16 bytes (or there is one row).
bool rows_aligned16(const void* p, int64_t ld, int64_t rows, int elem)
{
    return aligned(p, 16) && (rows <= 1 || ((ld * elem) % 16) == 0);
}

int elem_size(rr_dtype d) { return d == RR_BF16 ? 2 : 4; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" rr_status rr_device_cu_count(int32_t* cu_out)
{
    if (!cu_out) return RR_ERR_NULL;
    return current_cu(cu_out);
}

// rr_reduce_rows and rr_reduce_rows_noalloc: the same plan and kernels; the
// split-K workspace is the caller's (noalloc false) or the library's own
// per-device scratch array (noalloc true).
static rr_status reduce_rows_common(const void* x, void* y, int64_t rows, int64_t cols,
                                    int64_t ld, rr_dtype dtype, rr_op op, rr_tier tier,
                                    bool noalloc, void* workspace, size_t workspace_bytes,
                                    void* stream)
{
    if (op == RR_SUM_MAX_MIN) return RR_ERR_OP;  // that is rr_reduce_rows_multi
    // Shape / type / tier checks that need no device.
    rr_plan p;
    rr_status st = rr::plan_reduce(rows, cols, ld, dtype, op, tier, 1, true, &p);
    if (st != RR_OK) return st;
    if (rows == 0) return RR_OK;
    if (!y || (!x && cols > 0)) return RR_ERR_NULL;
    int32_t cu = 0;
    if ((st = current_cu(&cu)) != RR_OK) return st;
    const bool vec = aligned(x, 4);
    if ((st = rr::plan_reduce(rows, cols, ld, dtype, op, tier, cu, vec, &p)) != RR_OK) return st;

    rr::ReduceLaunch a{x, y, rows, cols, ld, dtype, op, false, {nullptr, nullptr, nullptr}, vec,
                       rows_aligned16(x, ld, rows, 4), workspace,
                       g_splitk_skew.load(std::memory_order_relaxed), as_stream(stream), cu};
    if (cols == 0) return rr::launch_reduce_identity(a);
    if (p.tier == RR_TIER_SPLITK) {
        if (noalloc) {
            if (p.workspace_bytes > RR_NOALLOC_SCRATCH_BYTES) return RR_ERR_SCRATCH;
            void* ws = nullptr;
            if ((st = rr::noalloc_scratch(&ws)) != RR_OK) return st;
            // The array keeps what the last call on this GPU left there; the
            // tickets must start at zero, so the bytes this call uses are
            // cleared first (a fill kernel: no memset node, no allocation).
            if ((st = rr::launch_fill_zero(ws, (size_t)p.workspace_bytes, a.stream)) != RR_OK)
                return st;
            a.workspace = ws;
        } else if (!workspace || workspace_bytes < p.workspace_bytes || !aligned(workspace, 8)) {
            return RR_ERR_WORKSPACE;
        }
    }
    log_plan(noalloc ? "rr_reduce_rows_noalloc" : "rr_reduce_rows", "rows", rows, "cols", cols,
             nullptr, 0, vec, p);
    return rr::launch_reduce(p, a);
}

extern "C" rr_status rr_reduce_rows(const void* x, void* y, int64_t rows, int64_t cols,
                                    int64_t ld, rr_dtype dtype, rr_op op, rr_tier tier,
                                    void* workspace, size_t workspace_bytes, void* stream)
{
    return reduce_rows_common(x, y, rows, cols, ld, dtype, op, tier, false, workspace,
                              workspace_bytes, stream);
}

extern "C" rr_status rr_reduce_rows_noalloc(const void* x, void* y, int64_t rows, int64_t cols,
                                            int64_t ld, rr_dtype dtype, rr_op op, rr_tier tier,
                                            void* stream)
{
    return reduce_rows_common(x, y, rows, cols, ld, dtype, op, tier, true, nullptr, 0, stream);
}

extern "C" rr_status rr_reduce_rows_multi(const void* x, void* y_sum, void* y_max, void* y_min,
                                          int64_t rows, int64_t cols, int64_t ld, rr_dtype dtype,
                                          rr_tier tier, void* workspace, size_t workspace_bytes,
                                          void* stream)
{
    rr_plan p;
    rr_status st = rr::plan_reduce(rows, cols, ld, dtype, RR_SUM_MAX_MIN, tier, 1, true, &p);
    if (st != RR_OK) return st;
    if (rows == 0) return RR_OK;
    if (!y_sum && !y_max && !y_min) return RR_ERR_NULL;
    if (!x && cols > 0) return RR_ERR_NULL;
    int32_t cu = 0;
    if ((st = current_cu(&cu)) != RR_OK) return st;
    const bool vec = aligned(x, 4);
    if ((st = rr::plan_reduce(rows, cols, ld, dtype, RR_SUM_MAX_MIN, tier, cu, vec, &p)) != RR_OK)
        return st;
    rr::ReduceLaunch a{x, nullptr, rows, cols, ld, dtype, RR_SUM, true, {y_sum, y_max, y_min},
                       vec, rows_aligned16(x, ld, rows, 4), workspace,
                       g_splitk_skew.load(std::memory_order_relaxed), as_stream(stream), cu};
    if (cols == 0) return rr::launch_reduce_identity(a);
    if (p.tier == RR_TIER_SPLITK) {
        if (!workspace || workspace_bytes < p.workspace_bytes || !aligned(workspace, 8))
            return RR_ERR_WORKSPACE;
    }
    log_plan("rr_reduce_rows_multi", "rows", rows, "cols", cols, nullptr, 0, vec, p);
    return rr::launch_reduce(p, a);
}

extern "C" rr_status rr_reduce_axis(const void* x, void* y, int64_t outer, int64_t axis,
                                    int64_t inner, rr_dtype dtype, rr_op op, rr_tier tier,
                                    void* workspace, size_t workspace_bytes, void* stream)
{
    rr_plan p;
    rr_status st = rr::plan_axis(outer, axis, inner, dtype, op, tier, 1, true, &p);
    if (st != RR_OK) return st;
    if (outer == 0 || inner == 0) return RR_OK;
    if (!y || (!x && axis > 0)) return RR_ERR_NULL;
    if (axis == 0) {  // every output is the identity
        rr::ReduceLaunch a{x, y, outer * inner, 0, 0, dtype, op, false,
                           {nullptr, nullptr, nullptr}, false, false, nullptr, 0,
                           as_stream(stream)};
        return rr::launch_reduce_identity(a);
    }
    int32_t cu = 0;
    if ((st = current_cu(&cu)) != RR_OK) return st;
    const bool vec = aligned(x, 16) && aligned(y, 16) && inner % 4 == 0;
    if ((st = rr::plan_axis(outer, axis, inner, dtype, op, tier, cu, vec, &p)) != RR_OK)
        return st;
    if (p.tier == RR_TIER_SPLITK) {
        if (!workspace || workspace_bytes < p.workspace_bytes || !aligned(workspace, 8))
            return RR_ERR_WORKSPACE;
    }
    rr::AxisLaunch a{x, y, outer, axis, inner, dtype, op, p.lanes_per_row == 4, workspace,
                     as_stream(stream)};
    log_plan("rr_reduce_axis", "outer", outer, "axis", axis, "inner", inner, vec, p);
    return rr::launch_reduce_axis(p, a);
}

extern "C" rr_status rr_softmax_rows(const void* x, void* y, int64_t rows, int64_t cols,
                                     int64_t ld_x, int64_t ld_y, rr_dtype x_dtype,
                                     rr_dtype y_dtype, rr_tier tier, void* workspace,
                                     size_t workspace_bytes, void* stream)
{
    rr_plan p;
    rr_status st = rr::plan_softmax(rows, cols, x_dtype, y_dtype, tier, 1, true, true, &p);
    if (st != RR_OK) return st;
    if (ld_x < cols || ld_y < cols) return RR_ERR_SHAPE;
    if (rows == 0 || cols == 0) return RR_OK;
    if (!x || !y) return RR_ERR_NULL;
    if (x == y && (ld_x != ld_y || x_dtype != y_dtype)) return RR_ERR_SHAPE;
    int32_t cu = 0;
    if ((st = current_cu(&cu)) != RR_OK) return st;
    // element-aligned rows take 128-bit chunks from each row's first 16-byte
    // boundary (block and split-K tiers); the wave tier needs aligned rows
    const bool vec = aligned(x, elem_size(x_dtype)) && aligned(y, elem_size(y_dtype));
    const bool rows16 = rows_aligned16(x, ld_x, rows, elem_size(x_dtype)) &&
                        rows_aligned16(y, ld_y, rows, elem_size(y_dtype));
    if ((st = rr::plan_softmax(rows, cols, x_dtype, y_dtype, tier, cu, vec, rows16, &p)) != RR_OK)
        return st;
    if (p.tier == RR_TIER_SPLITK) {
        if (!workspace || workspace_bytes < p.workspace_bytes || !aligned(workspace, 8))
            return RR_ERR_WORKSPACE;
    }
    rr::SoftmaxLaunch a{x, y, rows, cols, ld_x, ld_y, x_dtype, y_dtype, vec, rows16, workspace, cu,
                        as_stream(stream)};
    log_plan("rr_softmax_rows", "rows", rows, "cols", cols, nullptr, 0, vec, p);
    return rr::launch_softmax(p, a);
}

extern "C" rr_status rr_layernorm_rows(const void* x, void* y, const void* gamma,
                                       const void* beta, float* mean_out, float* rstd_out,
                                       int64_t rows, int64_t cols, int64_t ld_x, int64_t ld_y,
                                       rr_dtype x_dtype, rr_dtype y_dtype, rr_dtype w_dtype,
                                       float eps, rr_tier tier, void* workspace,
                                       size_t workspace_bytes, void* stream)
{
    rr_plan p;
    rr_status st = rr::plan_layernorm(rows, cols, x_dtype, y_dtype, w_dtype, tier, 1, true, true, &p);
    if (st != RR_OK) return st;
    if (ld_x < cols || ld_y < cols) return RR_ERR_SHAPE;
    if (!(eps >= 0.0f) || isinf(eps)) return RR_ERR_SHAPE;
    if (rows == 0 || cols == 0) return RR_OK;
    if (!x || !y) return RR_ERR_NULL;
    if (x == y && (ld_x != ld_y || x_dtype != y_dtype)) return RR_ERR_SHAPE;
    int32_t cu = 0;
    if ((st = current_cu(&cu)) != RR_OK) return st;
    const int ew = elem_size(w_dtype);
    const bool vec = aligned(x, elem_size(x_dtype)) && aligned(y, elem_size(y_dtype)) &&
                     (!gamma || aligned(gamma, ew)) && (!beta || aligned(beta, ew));
    const bool rows16 = rows_aligned16(x, ld_x, rows, elem_size(x_dtype)) &&
                        rows_aligned16(y, ld_y, rows, elem_size(y_dtype)) &&
                        (!gamma || aligned(gamma, 16)) && (!beta || aligned(beta, 16));
    const bool same_phase = rows <= 1 || (ld_x * elem_size(x_dtype)) % 16 == 0;
    if ((st = rr::plan_layernorm(rows, cols, x_dtype, y_dtype, w_dtype, tier, cu, vec, rows16,
                                 &p)) != RR_OK)
        return st;
    if (p.tier == RR_TIER_SPLITK) {
        if (!workspace || workspace_bytes < p.workspace_bytes || !aligned(workspace, 8))
            return RR_ERR_WORKSPACE;
    }
    rr::LayernormLaunch a{x, y, gamma, beta, mean_out, rstd_out, rows, cols, ld_x, ld_y,
                          x_dtype, y_dtype, w_dtype, eps, vec, rows16, same_phase, workspace, cu,
                          as_stream(stream)};
    log_plan("rr_layernorm_rows", "rows", rows, "cols", cols, nullptr, 0, vec, p);
    return rr::launch_layernorm(p, a);
}

extern "C" rr_status rr_splitk_lse_merge(const float* o_part, const float* m_part,
                                         const float* l_part, void* out, int32_t P, int64_t rows,
                                         int32_t depth, float scale, rr_dtype out_dtype,
                                         void* stream)
{
    if (P < 1 || P > RR_MERGE_MAX_P || rows < 0 || depth < 1) return RR_ERR_SHAPE;
    if (out_dtype != RR_BF16 && out_dtype != RR_F32) return RR_ERR_DTYPE;
    if (rows == 0) return RR_OK;
    if (!o_part || !m_part || !l_part || !out) return RR_ERR_NULL;
    const bool vec = (depth % 4) == 0 && aligned(o_part, 16) &&
                     aligned(out, out_dtype == RR_F32 ? 16 : 8);
    rr::MergeLaunch a{o_part, m_part, l_part, out, P, rows, depth, scale, out_dtype, vec,
                      as_stream(stream)};
    if (log_enabled())
        fprintf(stderr, "rr: rr_splitk_lse_merge P=%d rows=%lld depth=%d vec=%d\n", P,
                (long long)rows, depth, (int)vec);
    return rr::launch_merge(a);
}

// Shape checks common to the attention calls; *work_out is the grid size
// (one workgroup per 128 query rows, partition and head), 0 for a no-op.
static rr_status check_attention(int64_t batch, int64_t heads, int64_t kv_heads, int64_t q_rows,
                                 int64_t kv_len, int32_t depth, int32_t P, float scale,
                                 int64_t* work_out)
{
    *work_out = 0;
    if (batch < 0 || heads < 1 || kv_heads < 1 || heads % kv_heads != 0 || q_rows < 0 ||
        kv_len < 0 || P < 1 || P > RR_MERGE_MAX_P || (depth != 64 && depth != 128) ||
        !isfinite(scale))
        return RR_ERR_SHAPE;
    if (q_rows > (int64_t)INT32_MAX / (2 * depth)) return RR_ERR_SHAPE;  // q_rows*depth*2 < 2^31
    // the grid must fit in 31 bits; checked factor by factor so no product
    // can overflow
    const int64_t q_tiles = (q_rows + rr::kAttnRows - 1) / rr::kAttnRows;
    if (q_rows == 0 || batch == 0) return RR_OK;
    int64_t work = q_tiles * P;                      // <= 2^24 * 256
    if (batch > (int64_t)INT32_MAX / work) return RR_ERR_SHAPE;
    work *= batch;
    if (heads > (int64_t)INT32_MAX / work) return RR_ERR_SHAPE;
    *work_out = work * heads;
    return RR_OK;
}

extern "C" rr_status rr_splitk_attention_partials(const void* q, const void* k, const void* v,
                                                  float* o_part, float* m_part, float* l_part,
                                                  int64_t batch, int64_t heads, int64_t kv_heads,
                                                  int64_t q_rows, int64_t kv_len, int32_t depth,
                                                  int32_t P, float scale, void* stream)
{
    int64_t work = 0;
    rr_status st = check_attention(batch, heads, kv_heads, q_rows, kv_len, depth, P, scale, &work);
    if (st != RR_OK || work == 0) return st;
    if (!q || !o_part || !m_part || !l_part || (kv_len > 0 && (!k || !v))) return RR_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o_part, 16))
        return RR_ERR_SHAPE;
    rr::AttentionLaunch a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                          static_cast<const uint16_t*>(v), o_part, m_part, l_part, batch, heads,
                          kv_heads, q_rows, kv_len, depth, P, scale, nullptr, RR_F32, nullptr, 0,
                          as_stream(stream)};
    if (log_enabled())
        fprintf(stderr,
                "rr: rr_splitk_attention_partials batch=%lld heads=%lld kv_heads=%lld "
                "q_rows=%lld kv_len=%lld depth=%d P=%d workgroups=%lld\n",
                (long long)batch, (long long)heads, (long long)kv_heads, (long long)q_rows,
                (long long)kv_len, depth, P, (long long)work);
    return rr::launch_attention(a);
}

extern "C" rr_status rr_splitk_attention_partials_varlen(
    const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
    const int32_t* cu_seqlens_k, float* o_part, float* m_part, float* l_part, int64_t batch,
    int64_t heads, int64_t kv_heads, int64_t total_q, int64_t total_k, int64_t max_q_rows,
    int32_t depth, int32_t P, float scale, void* stream)
{
    int64_t work = 0;
    if (total_q < 0 || total_k < 0 || total_q > INT32_MAX || total_k > INT32_MAX)
        return RR_ERR_SHAPE;
    rr_status st = check_attention(batch, heads, kv_heads, max_q_rows, total_k, depth, P, scale,
                                   &work);
    if (st != RR_OK) return st;
    // byte ranges of one tile's rows inside the kernel stay below 2^31: the
    // 128 query rows (heads * depth * 2 bytes apart) and the 32 output rows
    // of a wavefront (heads * depth * 4 bytes apart)
    if (heads > (int64_t)INT32_MAX / ((int64_t)depth * 4 * rr::kAttnRows)) return RR_ERR_SHAPE;
    if (work == 0 || total_q == 0) return RR_OK;
    if (!q || !o_part || !m_part || !l_part || !cu_seqlens_q || !cu_seqlens_k ||
        (total_k > 0 && (!k || !v)))
        return RR_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o_part, 16))
        return RR_ERR_SHAPE;
    rr::AttentionLaunch a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                          static_cast<const uint16_t*>(v), o_part, m_part, l_part, batch, heads,
                          kv_heads, max_q_rows, total_k, depth, P, scale, nullptr, RR_F32, nullptr,
                          0, as_stream(stream), cu_seqlens_q, cu_seqlens_k, total_q};
    if (log_enabled())
        fprintf(stderr,
                "rr: rr_splitk_attention_partials_varlen batch=%lld heads=%lld kv_heads=%lld "
                "total_q=%lld total_k=%lld max_q_rows=%lld depth=%d P=%d workgroups=%lld\n",
                (long long)batch, (long long)heads, (long long)kv_heads, (long long)total_q,
                (long long)total_k, (long long)max_q_rows, depth, P, (long long)work);
    return rr::launch_attention(a);
}

// Workspace of the fused call: the tickets (one per group = head and 128
// query rows), padded to 256 bytes, then O_p, m_p and l_p group-major,
// [group][P][128 rows] (the kernel's fold reads a group's partials from one
// range).
namespace {
struct AttnWorkspace {
    uint64_t tickets, o, m, l, total;
};
AttnWorkspace attn_workspace(int64_t batch, int64_t heads, int64_t q_rows, int32_t depth, int32_t P)
{
    const uint64_t groups = (uint64_t)batch * (uint64_t)heads *
                            (uint64_t)((q_rows + rr::kAttnRows - 1) / rr::kAttnRows);
    const uint64_t cells = groups * (uint64_t)P * rr::kAttnRows;
    AttnWorkspace w;
    w.tickets = 0;
    w.o = (groups * 4 + 255) / 256 * 256;
    w.m = w.o + cells * (uint64_t)depth * 4;
    w.l = w.m + cells * 4;
    w.total = w.l + cells * 4;
    return w;
}
}  // namespace

extern "C" rr_status rr_splitk_attention_workspace_bytes(int64_t batch, int64_t heads,
                                                         int64_t kv_heads, int64_t q_rows,
                                                         int64_t kv_len, int32_t depth, int32_t P,
                                                         size_t* bytes_out,
                                                         size_t* ticket_bytes_out)
{
    if (!bytes_out) return RR_ERR_NULL;
    int64_t work = 0;
    rr_status st = check_attention(batch, heads, kv_heads, q_rows, kv_len, depth, P, 1.0f, &work);
    if (st != RR_OK) return st;
    if (P > depth / 8) return RR_ERR_SHAPE;
    const AttnWorkspace w = attn_workspace(batch, heads, q_rows, depth, P);
    *bytes_out = work == 0 ? 0 : (size_t)w.total;
    if (ticket_bytes_out) *ticket_bytes_out = work == 0 ? 0 : (size_t)w.o;
    return RR_OK;
}

extern "C" rr_status rr_splitk_attention(const void* q, const void* k, const void* v, void* out,
                                         rr_dtype out_dtype, int64_t batch, int64_t heads,
                                         int64_t kv_heads, int64_t q_rows, int64_t kv_len,
                                         int32_t depth, int32_t P, float scale, void* workspace,
                                         size_t workspace_bytes, void* stream)
{
    int64_t work = 0;
    rr_status st = check_attention(batch, heads, kv_heads, q_rows, kv_len, depth, P, scale, &work);
    if (st != RR_OK) return st;
    if (P > depth / 8) return RR_ERR_SHAPE;          // the fold's (row, partition) cells fit in LDS
    if (out_dtype != RR_BF16 && out_dtype != RR_F32) return RR_ERR_DTYPE;
    if (work == 0) return RR_OK;
    if (!q || !out || (kv_len > 0 && (!k || !v))) return RR_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return RR_ERR_SHAPE;
    const AttnWorkspace w = attn_workspace(batch, heads, q_rows, depth, P);
    if (!workspace || workspace_bytes < w.total || !aligned(workspace, 16))
        return RR_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    rr::AttentionLaunch a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                          static_cast<const uint16_t*>(v), reinterpret_cast<float*>(ws + w.o),
                          reinterpret_cast<float*>(ws + w.m), reinterpret_cast<float*>(ws + w.l),
                          batch, heads, kv_heads, q_rows, kv_len, depth, P, scale, out, out_dtype,
                          reinterpret_cast<uint32_t*>(ws + w.tickets),
                          g_splitk_skew.load(std::memory_order_relaxed), as_stream(stream)};
    if (log_enabled())
        fprintf(stderr,
                "rr: rr_splitk_attention batch=%lld heads=%lld kv_heads=%lld q_rows=%lld "
                "kv_len=%lld depth=%d P=%d out=%s workgroups=%lld\n",
                (long long)batch, (long long)heads, (long long)kv_heads, (long long)q_rows,
                (long long)kv_len, depth, P, out_dtype == RR_BF16 ? "bf16" : "f32",
                (long long)work);
    return rr::launch_attention(a);
}

extern "C" rr_status rr_workspace_bytes(rr_kind kind, int64_t rows, int64_t cols, rr_dtype dtype,
                                        rr_op op, rr_tier tier, size_t* bytes_out)
{
    if (!bytes_out) return RR_ERR_NULL;
    if (kind != RR_KIND_REDUCE && kind != RR_KIND_SOFTMAX && kind != RR_KIND_LAYERNORM)
        return RR_ERR_TIER;
    int32_t cu = 0;
    rr_status st = current_cu(&cu);
    if (st != RR_OK) return st;
    rr_plan p;
    if (kind == RR_KIND_REDUCE)
        st = rr::plan_reduce(rows, cols, cols, dtype, op, tier, cu, true, &p);
    else if (kind == RR_KIND_SOFTMAX)
        st = rr::plan_softmax(rows, cols, dtype, dtype, tier, cu, true, true, &p);
    else
        st = rr::plan_layernorm(rows, cols, dtype, dtype, RR_F32, tier, cu, true, true, &p);
    if (st != RR_OK) return st;
    *bytes_out = (size_t)p.workspace_bytes;
    return RR_OK;
}

extern "C" rr_status rr_select_tier(rr_kind kind, int64_t rows, int64_t cols, rr_dtype dtype,
                                    rr_op op, rr_tier* tier_out)
{
    if (!tier_out) return RR_ERR_NULL;
    int32_t cu = 0;
    rr_status st = current_cu(&cu);
    if (st != RR_OK) return st;
    rr_plan p;
    if (kind == RR_KIND_REDUCE)
        st = rr::plan_reduce(rows, cols, cols, dtype, op, RR_TIER_AUTO, cu, true, &p);
    else if (kind == RR_KIND_SOFTMAX)
        st = rr::plan_softmax(rows, cols, dtype, dtype, RR_TIER_AUTO, cu, true, true, &p);
    else if (kind == RR_KIND_LAYERNORM)
        st = rr::plan_layernorm(rows, cols, dtype, dtype, RR_F32, RR_TIER_AUTO, cu, true, true, &p);
    else
        return RR_ERR_TIER;
    if (st != RR_OK) return st;
    *tier_out = (rr_tier)p.tier;
    return RR_OK;
}

extern "C" rr_status rr_workspace_reset(void* workspace, size_t bytes, void* stream)
{
    if (bytes == 0) return RR_OK;
    if (!workspace) return RR_ERR_NULL;
    return rr::launch_fill_zero(workspace, bytes, as_stream(stream));
}

extern "C" void rr_test_set_splitk_skew(int32_t sleeps_per_rank)
{
    g_splitk_skew.store(sleeps_per_rank < 0 ? 0 : sleeps_per_rank, std::memory_order_relaxed);
}
