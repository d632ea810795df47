"""GPU parity for rr_reduce_axis (reduction over a non-last axis).

x is [outer, axis, inner]; y[o, i] folds x[o, :, i].  Bars: int32 results
and float max/min bit-exact; float sums bit-exact on the tiled and serial
tiers (they add in axis order in double, as the oracle does) and within
rel 1e-5 / abs 1e-6 on split-K (slices are added to each other).
"""
import numpy as np
import pytest
import torch

import oracle
import split_deterministic_combine_amd as rr
from split_deterministic_combine_amd import synth
from tests.gpu_util import assert_close_f32, assert_exact, to_gpu, to_host

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1, 1), (3, 5, 7), (2, 100, 4), (2, 100, 8), (1, 1000, 64), (1, 70001, 12),
          (4, 3000, 1), (5, 17, 1023), (1, 2049, 3), (2, 513, 256), (7, 9, 4100)]


def _input(dt, shape, seed):
    if dt == "i32":
        return synth.ints_i32(seed, shape, -(2 ** 31), 2 ** 31 - 1)
    return synth.normal_f32(seed, shape)


def _run(xg, op, tier):
    o, a, i = xg.shape
    y = torch.empty((o, i), dtype=xg.dtype, device="cuda")
    rr.reduce_axis(xg, 1, op, tier, out=y)
    torch.cuda.synchronize()
    return to_host(y)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dt", ["f32", "i32"])
def test_axis_all_tiers_match_oracle(shape, dt):
    x = _input(dt, shape, 2100 + sum(shape))
    xg = to_gpu(x)
    for op in ("sum", "max", "min"):
        ref = oracle.reduce_axis(x, op)
        for tier in ("auto", "tiled", "serial", "splitk"):
            got = _run(xg, op, tier)
            what = "%s %s %s %s" % (dt, op, shape, tier)
            if dt == "f32" and op == "sum" and rr.plan_axis(*shape, tier=tier)["tier"] == "splitk":
                assert_close_f32(got, ref, what)
            else:
                assert_exact(got, ref, what)


def test_axis_any_dim_of_a_4d_tensor_matches_torch():
    x = synth.normal_f32(2200, (6, 33, 20, 12))
    xg = to_gpu(x)
    for dim in (0, 1, 2, 3, -1):
        for op, tref in (("sum", None), ("max", torch.amax), ("min", torch.amin)):
            got = rr.reduce_axis(xg, dim, op)
            xd = torch.from_numpy(x)
            if op == "sum":
                want = xd.double().sum(dim=dim).float()
                assert torch.allclose(got.cpu(), want, rtol=1e-5, atol=1e-6), (dim, op)
            else:
                assert torch.equal(got.cpu(), tref(xd, dim=dim)), (dim, op)


def test_axis_misaligned_base_takes_the_scalar_path():
    x = synth.normal_f32(2300, (2, 600, 16))
    flat = torch.zeros(x.size + 1, dtype=torch.float32, device="cuda")
    flat[1:] = to_gpu(x).reshape(-1)
    xg = flat[1:].view(2, 600, 16)             # 4-byte aligned, not 16
    for tier in ("auto", "tiled", "splitk"):
        got = to_host(rr.reduce_axis(xg, 1, "max", tier))
        assert_exact(got, oracle.reduce_axis(x, "max"), "misaligned " + tier)


def test_axis_empty_axis_writes_identities_and_empty_outputs_are_noops():
    xg = torch.zeros((3, 0, 5), dtype=torch.float32, device="cuda")
    assert torch.all(rr.reduce_axis(xg, 1, "max") == -float("inf"))
    assert torch.all(rr.reduce_axis(xg, 1, "sum") == 0)
    xi = torch.zeros((3, 0, 5), dtype=torch.int32, device="cuda")
    assert torch.all(rr.reduce_axis(xi, 1, "min") == 2 ** 31 - 1)
    assert rr.reduce_axis(torch.zeros((0, 4, 5), device="cuda"), 1).shape == (0, 5)


def test_axis_splitk_bit_identical_across_runs():
    xg = to_gpu(synth.normal_f32(2400, (1, 1 << 18, 64)))
    assert rr.plan_axis(1, 1 << 18, 64, cu_count=rr.device_cu_count())["tier"] == "splitk"
    first = rr.reduce_axis(xg, 1, "sum").clone()
    for _ in range(4):
        assert torch.equal(rr.reduce_axis(xg, 1, "sum").view(torch.int32), first.view(torch.int32))
    ref = oracle.reduce_axis(to_host(xg), "sum")
    assert_close_f32(to_host(first), ref, "splitk [1, 2^18, 64]")
