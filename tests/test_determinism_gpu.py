"""Run-to-run bit identity ("cluster_allreduce", description: every group
folds the others' values in rank order, so every run gives the same bits).

* The small-row, short-row and LSE-merge workloads at their full sizes, ten
  runs each, compared bit for bit (the long-row and softmax workloads have
  their ten-run checks beside their parity tests).
* A soak of the cross-workgroup publish: thousands of split-K calls -- row
  reductions, the fused sum/max/min and the split-K softmax -- over several
  shapes, with the arrival-order skew hook cycling through 0, 1, 4, 16 and 32
  sleep periods per rank, every result compared with the first run's bits.
  It stops at the first mismatch.
"""
import numpy as np
import pytest
import torch

import split_deterministic_combine_amd as rr
from split_deterministic_combine_amd import synth
from tests.gpu_util import to_gpu

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _assert_ten_runs(fn, what):
    first = [_bits(t).clone() for t in fn()]
    for run in range(1, 10):
        again = fn()
        for k, (a, b) in enumerate(zip(again, first)):
            assert torch.equal(_bits(a), b), "%s: output %d differs on run %d" % (what, k, run)


def test_small_rows_config_ten_runs_bit_identical():
    xf, xi = synth.small_rows()
    gf, gi = to_gpu(xf), to_gpu(xi)
    assert rr.plan_reduce(64, 1024, cu_count=rr.device_cu_count())["tier"] == "block"
    _assert_ten_runs(lambda: (rr.reduce_rows(gf, "sum"), rr.reduce_rows(gf, "max"),
                              rr.reduce_rows(gi, "sum")), "small rows [64, 1024]")


def test_short_rows_config_ten_runs_bit_identical():
    g = to_gpu(synth.short_rows())
    assert rr.plan_reduce(1048576, 48, cu_count=rr.device_cu_count())["tier"] == "wave"
    _assert_ten_runs(lambda: (rr.reduce_rows(g, "sum"), rr.reduce_rows(g, "max")),
                     "short rows [1048576, 48]")


def test_merge_config_ten_runs_bit_identical():
    o, m, l = synth.lse_merge()
    go, gm, gl = to_gpu(o), to_gpu(m), to_gpu(l)
    _assert_ten_runs(lambda: (rr.splitk_lse_merge(go, gm, gl, 1.0, torch.bfloat16),),
                     "LSE merge P=8 [8, 32, 128, 128]")


SKEWS = (0, 1, 4, 16, 32)
SOAK_CALLS = 2000


def _soak_cases():
    """(name, callable) pairs, each a split-K plan with several slices per row."""
    cu = rr.device_cu_count()
    f1 = to_gpu(synth.uniform_f32(81, (16, 1 << 20)))
    i1 = to_gpu(synth.ints_i32(82, (3, 70001), -(2 ** 30), 2 ** 30))
    f2 = to_gpu(synth.normal_f32(83, (37, 131077 + 3)))[:, 1:131078]   # misaligned rows
    i2 = to_gpu(synth.ints_i32(84, (255, 65536), -(2 ** 31), 2 ** 31 - 1))
    f3 = to_gpu(synth.normal_f32(85, (1, 1 << 18)))
    i3 = to_gpu(synth.ints_i32(86, (7, 100003), -1000, 1000))
    s1 = to_gpu(synth.normal_bf16(87, (5, 131071)))
    s2 = to_gpu(synth.normal_f32(88, (16, 1 << 18), 3.0))
    for t in (f1, i1, f2, i2, f3, i3):
        assert rr.plan_reduce(t.shape[0], t.shape[1], t.dtype, "sum", cu_count=cu)["slices"] > 1
    for t in (s1, s2):
        assert rr.plan_softmax(t.shape[0], t.shape[1], t.dtype, t.dtype, cu_count=cu)["slices"] > 1

    def multi(t):
        d = rr.reduce_rows_multi(t)
        return (d["sum"], d["max"], d["min"])

    return [
        ("f32 sum [16, 2^20]", lambda: (rr.reduce_rows(f1, "sum"),)),
        ("i32 max [3, 70001]", lambda: (rr.reduce_rows(i1, "max"),)),
        ("f32 sum [37, 131077] misaligned", lambda: (rr.reduce_rows(f2, "sum"),)),
        ("i32 sum [255, 65536]", lambda: (rr.reduce_rows(i2, "sum"),)),
        ("f32 max [1, 2^18]", lambda: (rr.reduce_rows(f3, "max"),)),
        ("f32 min [16, 2^20]", lambda: (rr.reduce_rows(f1, "min"),)),
        ("f32 sum/max/min [16, 2^20]", lambda: multi(f1)),
        ("i32 sum/max/min [7, 100003]", lambda: multi(i3)),
        ("f32 sum/max/min [37, 131077] misaligned", lambda: multi(f2)),
        ("bf16 softmax [5, 131071]", lambda: (rr.softmax_rows(s1),)),
        ("f32 softmax [16, 2^18]", lambda: (rr.softmax_rows(s2, torch.float32),)),
    ]


def test_splitk_publish_soak_under_arrival_skew():
    cases = _soak_cases()
    first = [[_bits(t).clone() for t in fn()] for _, fn in cases]
    torch.cuda.synchronize()
    calls = 0
    seen_skews = set()
    try:
        while calls < SOAK_CALLS:
            for skew in SKEWS:
                rr._set_splitk_skew(skew)
                seen_skews.add(skew)
                for (name, fn), want in zip(cases, first):
                    got = fn()
                    calls += 1
                    for k, (a, b) in enumerate(zip(got, want)):
                        if not torch.equal(_bits(a), b):
                            pytest.fail("%s, output %d: bits differ from the first run at call %d "
                                        "(skew %d)" % (name, k, calls, skew))
    finally:
        rr._set_splitk_skew(0)
    torch.cuda.synchronize()
    assert calls >= SOAK_CALLS and seen_skews == set(SKEWS)
    # the soaked results are the oracle-checked kernels' results: the first
    # run of the plain reductions equals the single-statistic calls
    np.testing.assert_array_equal(first[6][0].cpu().numpy(), first[0][0].cpu().numpy())
