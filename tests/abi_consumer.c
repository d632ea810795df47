/*
 * A plain C (C11) consumer of the librr C ABI: includes rr.h, links against
 * librr.so, and calls the host-only entry points (no GPU needed).  Built and
 * run by tests/test_abi_cpu.py; it proves the header is C, not C++, and that
 * the boundary carries plain pointers and sizes only.
 */
#include <stdio.h>
#include <string.h>

#include "rr.h"

int main(void)
{
    rr_plan p;
    memset(&p, 0, sizeof p);
    if (rr_plan_reduce(16, 1 << 24, 1 << 24, RR_F32, RR_SUM, RR_TIER_AUTO, 256, &p) != RR_OK)
        return 1;
    printf("reduce tier=%d slices=%d grid=%lld ws=%llu\n", p.tier, p.slices, (long long)p.grid,
           (unsigned long long)p.workspace_bytes);
    if (rr_plan_softmax(8192, 8192, RR_BF16, RR_BF16, RR_TIER_AUTO, 256, &p) != RR_OK)
        return 1;
    printf("softmax tier=%d block=%d grid=%lld\n", p.tier, p.block, (long long)p.grid);
    if (rr_plan_layernorm(16384, 4096, RR_BF16, RR_BF16, RR_F32, RR_TIER_AUTO, 256, &p) != RR_OK)
        return 1;
    printf("layernorm tier=%d block=%d grid=%lld\n", p.tier, p.block, (long long)p.grid);
    if (rr_plan_axis(1, 4096, 65536, RR_F32, RR_SUM, RR_TIER_AUTO, 256, &p) != RR_OK)
        return 1;
    printf("axis tier=%d slices=%d\n", p.tier, p.slices);
    /* argument errors come back before any device work */
    rr_status s = rr_reduce_rows(NULL, NULL, 4, 8, 4, RR_F32, RR_SUM, RR_TIER_AUTO, NULL, 0, NULL);
    printf("bad ld -> %d (%s)\n", (int)s, rr_status_string(s));
    s = rr_softmax_rows(NULL, NULL, 0, 8, 8, 8, RR_BF16, RR_BF16, RR_TIER_AUTO, NULL, 0, NULL);
    printf("empty softmax -> %d\n", (int)s);
    s = rr_splitk_lse_merge(NULL, NULL, NULL, NULL, 0, 4, 8, 1.0f, RR_BF16, NULL);
    printf("P=0 merge -> %d\n", (int)s);
    s = rr_reduce_rows_noalloc(NULL, NULL, 4, 8, 4, RR_F32, RR_SUM, RR_TIER_AUTO, NULL);
    printf("noalloc bad ld -> %d\n", (int)s);
    s = rr_splitk_attention_partials_varlen(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 2, 4, 2,
                                            10, 10, 8, 64, 4, 0.125f, NULL);
    printf("varlen without buffers -> %d\n", (int)s);
    s = rr_splitk_attention_partials_varlen(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 2, 4, 3,
                                            10, 10, 8, 64, 4, 0.125f, NULL);
    printf("varlen heads not a multiple of kv heads -> %d\n", (int)s);
    size_t ws = 0, tickets = 0;
    s = rr_splitk_attention_workspace_bytes(8, 32, 32, 128, 8192, 128, 8, &ws, &tickets);
    printf("attention workspace %d %llu %llu\n", (int)s, (unsigned long long)ws,
           (unsigned long long)tickets);
    printf("version %d\n", rr_version());
    return 0;
}
