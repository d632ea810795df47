"""GPU parity for rr_reduce_rows_multi (sum, max and min over one read).

Each requested output must equal, bit for bit, rr_reduce_rows of that op on
the same tier (the three states fold and combine exactly as the single-op
kernels do), and match the oracle to the reduce bars: float sums within
rel 1e-5 / abs 1e-6, everything else bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import split_deterministic_combine_amd as rr
from split_deterministic_combine_amd import synth
from tests.gpu_util import assert_close_f32, assert_exact, to_gpu, to_host

pytestmark = pytest.mark.gpu

COLS = [0, 1, 3, 4, 7, 8, 9, 48, 63, 64, 65, 1000, 1023, 1024, 4097, 70001]


def _input(dt, rows, cols, seed):
    if dt == "i32":
        return synth.ints_i32(seed, (rows, cols), -(2 ** 31), 2 ** 31 - 1)
    return synth.normal_f32(seed, (rows, cols))


def _tiers(cols):
    t = ["auto", "block", "tiled", "serial", "splitk"]
    if cols <= 64:
        t.append("wave")
    return t


def _check(name, dt, got, x_host, what):
    ref = oracle.reduce_rows(x_host, name)
    if dt == "f32" and name == "sum":
        assert_close_f32(got, ref, what)
    else:
        assert_exact(got, ref, what)


@pytest.mark.parametrize("cols", COLS)
@pytest.mark.parametrize("dt", ["f32", "i32"])
def test_multi_matches_single_ops_and_oracle(cols, dt):
    rows = 37
    x = _input(dt, rows, cols, 1300 + cols)
    g = to_gpu(x)
    for tier in _tiers(cols):
        if tier == "serial" and cols > 5000:
            continue
        got = rr.reduce_rows_multi(g, tier=tier)
        for name in ("sum", "max", "min"):
            single = rr.reduce_rows(g, name, tier)
            what = "%s %s cols %d %s" % (dt, name, cols, tier)
            assert torch.equal(got[name].view(torch.int32), single.view(torch.int32)), what
            _check(name, dt, to_host(got[name]), x, what)


def test_multi_subsets_write_only_what_is_asked():
    x = synth.normal_f32(1400, (19, 3000))
    g = to_gpu(x)
    for stats in (("max",), ("sum", "min"), ("min", "max")):
        sentinel = {k: torch.full((19,), 12345.0, device="cuda") for k in ("sum", "max", "min")}
        got = rr.reduce_rows_multi(g, stats, out=dict(sentinel))
        assert set(got) == set(stats)
        for k in ("sum", "max", "min"):
            if k in stats:
                _check(k, "f32", to_host(got[k]), x, "subset %s %s" % (stats, k))
            else:
                assert torch.all(sentinel[k] == 12345.0), "unrequested %s written" % k


@pytest.mark.parametrize("pad,offset", [(4, 0), (0, 1), (3, 2)])
def test_multi_strided_and_misaligned_rows(pad, offset):
    rows, cols = 21, 777
    x = synth.normal_f32(1500, (rows, cols))
    big = np.zeros((rows, cols + pad + offset), dtype=np.float32)
    big[:, offset:offset + cols] = x
    g = to_gpu(big)[:, offset:offset + cols]
    for tier in ("auto", "block", "tiled", "splitk"):
        got = rr.reduce_rows_multi(g, tier=tier)
        for name in ("sum", "max", "min"):
            _check(name, "f32", to_host(got[name]), x, "strided %s %s" % (name, tier))


@pytest.mark.parametrize("rows,cols,pad,offset", [(5000, 1000, 0, 0), (5000, 1001, 0, 0),
                                                   (3000, 2048, 4, 1), (20000, 65, 0, 3)])
@pytest.mark.parametrize("dt", ["f32", "i32"])
def test_multi_block_tier_persistent_rows(rows, cols, pad, offset, dt):
    # at least 4 rows per CU: persistent workgroups walk several rows; each
    # output equals the single-op kernel's bits, unrequested ones stay as
    # they were
    cu = rr.device_cu_count()
    plan = rr.plan_reduce(rows, cols, torch.float32 if dt == "f32" else torch.int32,
                          "sum_max_min", "block", cu_count=cu)
    assert plan["grid"] < rows, plan
    x = _input(dt, rows, cols, 1450 + cols + offset)
    big = np.zeros((rows, cols + pad + offset), dtype=x.dtype)
    big[:, offset:offset + cols] = x
    g = to_gpu(big)[:, offset:offset + cols]
    got = rr.reduce_rows_multi(g, tier="block")
    for name in ("sum", "max", "min"):
        single = rr.reduce_rows(g, name, "block")
        what = "%s %s %dx%d pad %d off %d" % (dt, name, rows, cols, pad, offset)
        assert torch.equal(got[name].view(torch.int32), single.view(torch.int32)), what
        _check(name, dt, to_host(got[name]), x, what)
    fill = 12345 if dt == "i32" else 12345.0
    sentinel = {k: torch.full((rows,), fill, dtype=got["sum"].dtype, device="cuda")
                for k in ("sum", "max", "min")}
    part = rr.reduce_rows_multi(g, ("min",), tier="block", out=dict(sentinel))
    assert torch.equal(part["min"].view(torch.int32), got["min"].view(torch.int32))
    assert torch.all(sentinel["sum"] == fill) and torch.all(sentinel["max"] == fill)


def test_multi_special_values_total_order():
    x = np.array([[-0.0, 0.0, -0.0, 1.0, -1.0] * 12,
                  [np.nan, 1.0, -np.inf, np.inf, 2.0] * 12,
                  [-np.nan, 1.0, -2.0, 3.0, 0.0] * 12], dtype=np.float32)
    g = to_gpu(x)
    for tier in ("block", "wave", "tiled", "serial", "splitk"):
        got = rr.reduce_rows_multi(g, tier=tier)
        for name in ("max", "min"):
            assert_exact(to_host(got[name]), oracle.reduce_rows(x, name), "special %s %s" % (name, tier))


def test_multi_splitk_long_rows_deterministic_under_skew():
    x = synth.uniform_f32(1600, (16, 1 << 20))
    xi = synth.ints_i32(1601, (16, 1 << 20), -(2 ** 30), 2 ** 30)
    g, gi = to_gpu(x), to_gpu(xi)
    assert rr.plan_reduce(16, 1 << 20, op="sum_max_min", cu_count=rr.device_cu_count())["tier"] == "splitk"
    first = {k: v.clone() for k, v in rr.reduce_rows_multi(g).items()}
    first_i = {k: v.clone() for k, v in rr.reduce_rows_multi(gi).items()}
    try:
        rr._set_splitk_skew(16)
        skew = rr.reduce_rows_multi(g)
        skew_i = rr.reduce_rows_multi(gi)
        torch.cuda.synchronize()
    finally:
        rr._set_splitk_skew(0)
    for k in ("sum", "max", "min"):
        assert torch.equal(skew[k].view(torch.int32), first[k].view(torch.int32)), k
        assert torch.equal(skew_i[k], first_i[k]), k
        _check(k, "f32", to_host(first[k]), x, "long f32 " + k)
        _check(k, "i32", to_host(first_i[k]), xi, "long i32 " + k)
    # the whole workspace is left zero for the next call
    for key, ws in rr._workspaces.items():
        if key[0] == "reduce":
            assert int(ws.count_nonzero()) == 0
