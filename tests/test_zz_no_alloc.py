"""rr_reduce_rows_noalloc against rr_reduce_rows, through the C ABI.

The entry point for callers that cannot allocate uses the library's own
per-GPU scratch array as its split-K workspace; it runs the same plan and
kernels as rr_reduce_rows, so its outputs must equal rr_reduce_rows's bit for
bit.  Two calls in a row (the second on a smaller input) check that what the
first call leaves in the shared array does not change the second's result.
"""
import ctypes

import numpy as np
import pytest
import torch

import split_deterministic_combine_amd as rr
from split_deterministic_combine_amd import synth
from tests.gpu_util import assert_exact, to_gpu, to_host

pytestmark = pytest.mark.gpu


def _pair(x, op, tier):
    """(rr_reduce_rows result, rr_reduce_rows_noalloc result) for x."""
    want = rr.reduce_rows(x, op, tier)
    out = torch.full(x.shape[:-1], -7, dtype=x.dtype, device=x.device)
    got = rr.reduce_rows_noalloc(x, out, op, tier)
    torch.cuda.synchronize()
    return to_host(want), to_host(got)


@pytest.mark.parametrize("dtype,op", [(np.float32, "sum"), (np.int32, "max"), (np.float32, "min")])
def test_noalloc_equals_reduce_rows_on_two_calls_in_a_row(dtype, op):
    shapes = [(37, 300007), (5, 70001)]  # split-K; the second call smaller
    for i, (rows, cols) in enumerate(shapes):
        if dtype == np.int32:
            x = synth.ints_i32(60 + i, (rows, cols), -(2 ** 31), 2 ** 31 - 1)
        else:
            x = synth.normal_f32(60 + i, (rows, cols))
        g = to_gpu(x)
        assert rr.plan_reduce(rows, cols, g.dtype, op, cu_count=rr.device_cu_count())["tier"] == "splitk"
        want, got = _pair(g, op, "auto")
        assert_exact(got, want, "noalloc %s %s call %d" % (op, x.dtype, i))


def test_noalloc_other_tiers_and_strided_rows():
    x = synth.normal_f32(70, (64, 1024))
    g = to_gpu(x)
    for tier in ("auto", "block", "tiled", "serial", "splitk"):
        want, got = _pair(g, "sum", tier)
        assert_exact(got, want, "noalloc tier " + tier)
    # misaligned rows (scalar path) and a split-K plan with one slice per row
    big = to_gpu(synth.normal_f32(71, (9, 100003)))[:, 1:100002]
    want, got = _pair(big, "max", "splitk")
    assert_exact(got, want, "noalloc misaligned split-K")


def test_noalloc_refuses_a_plan_larger_than_its_scratch():
    rows, cols = 200000, 64
    plan = rr.plan_reduce(rows, cols, torch.float32, "sum", "splitk", rr.device_cu_count())
    assert plan["workspace_bytes"] > rr.NOALLOC_SCRATCH_BYTES
    x = torch.ones(rows, cols, device="cuda")
    out = torch.full((rows,), -1.0, device="cuda")
    with pytest.raises(rr.RRError) as e:
        rr.reduce_rows_noalloc(x, out, "sum", "splitk")
    assert e.value.status == 8
    torch.cuda.synchronize()
    assert bool((out == -1.0).all())  # nothing was launched
    # the same shape on the automatic tier needs no workspace
    rr.reduce_rows_noalloc(x, out, "sum")
    torch.cuda.synchronize()
    assert bool((out == 64.0).all())


def test_noalloc_repeated_calls_are_bit_identical():
    g = to_gpu(synth.uniform_f32(72, (16, 1 << 20)))
    out = torch.empty(16, device="cuda")
    first = rr.reduce_rows_noalloc(g, out, "sum").clone()
    for _ in range(9):
        again = rr.reduce_rows_noalloc(g, torch.empty(16, device="cuda"), "sum")
        assert torch.equal(again.view(torch.int32), first.view(torch.int32))
    assert torch.equal(rr.reduce_rows(g, "sum").view(torch.int32), first.view(torch.int32))
