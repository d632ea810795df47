"""Seeded random sweep: shapes, strides, offsets, dtypes, ops and tiers drawn
at random (fixed seed), every case checked against the oracle at the bars of
the other parity tests.  Complements the hand-picked edge cases."""
import numpy as np
import pytest
import torch

import oracle
import split_deterministic_combine_amd as rr
from split_deterministic_combine_amd import synth
from tests.gpu_util import (assert_bf16_within_1ulp,
                            assert_close_f32, assert_exact, to_gpu, to_host)

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(20261202)


def _cols(rng):
    # mostly small, sometimes around tier boundaries, sometimes long
    kind = rng.integers(0, 4)
    if kind == 0:
        return int(rng.integers(1, 70))
    if kind == 1:
        return int(rng.choice([63, 64, 65, 127, 128, 129, 1023, 1024, 1025, 2048, 4096, 8192]))
    if kind == 2:
        return int(rng.integers(70, 9000))
    return int(rng.integers(65536, 200000))


def _strided(x_host, pad, offset):
    rows, cols = x_host.shape
    big = np.zeros((rows, cols + pad + offset), dtype=x_host.dtype)
    big[:, offset:offset + cols] = x_host
    return to_gpu(big)[:, offset:offset + cols]


REDUCE_CASES = []
for i in range(40):
    cols = _cols(RNG)
    rows = int(RNG.integers(1, 40)) if cols > 60000 else int(RNG.integers(1, 600))
    REDUCE_CASES.append((i, rows, cols, int(RNG.integers(0, 5)), int(RNG.integers(0, 3)),
                         str(RNG.choice(["f32", "i32"])), str(RNG.choice(["sum", "max", "min"]))))


@pytest.mark.parametrize("case", REDUCE_CASES, ids=lambda c: "r%d_%dx%d" % (c[0], c[1], c[2]))
def test_random_reduce(case):
    i, rows, cols, pad, offset, dt, op = case
    x = (synth.ints_i32(4000 + i, (rows, cols), -(2 ** 31), 2 ** 31 - 1) if dt == "i32"
         else synth.normal_f32(4000 + i, (rows, cols)))
    g = _strided(x, pad, offset)
    ref = oracle.reduce_rows(x, op)
    tiers = ["auto", "block", "tiled", "splitk"] + (["wave"] if cols <= 64 else [])
    if cols <= 4096:
        tiers.append("serial")
    for tier in tiers:
        got = to_host(rr.reduce_rows(g, op, tier))
        what = "%s %s %dx%d pad %d off %d %s" % (dt, op, rows, cols, pad, offset, tier)
        if dt == "f32" and op == "sum":
            assert_close_f32(got, ref, what)
        else:
            assert_exact(got, ref, what)


SOFTMAX_CASES = []
for i in range(30):
    cols = _cols(RNG)
    rows = int(RNG.integers(1, 20)) if cols > 60000 else int(RNG.integers(1, 400))
    SOFTMAX_CASES.append((i, rows, cols, int(RNG.integers(0, 5)), int(RNG.integers(0, 3)),
                          str(RNG.choice(["bf16", "f32"])), str(RNG.choice(["bf16", "f32"]))))


@pytest.mark.parametrize("case", SOFTMAX_CASES, ids=lambda c: "s%d_%dx%d" % (c[0], c[1], c[2]))
def test_random_softmax_and_layernorm(case):
    i, rows, cols, pad, offset, xt, yt = case
    x = (synth.normal_bf16(5000 + i, (rows, cols)) if xt == "bf16"
         else synth.normal_f32(5000 + i, (rows, cols), 3.0))
    g = _strided(x, pad, offset)
    ydt = torch.bfloat16 if yt == "bf16" else torch.float32
    tiers = ["auto", "block", "tiled", "splitk"] + (["wave"] if cols <= 64 else [])
    ref = oracle.softmax_rows(x, yt)
    for tier in tiers:
        got = to_host(rr.softmax_rows(g, ydt, tier))
        what = "softmax %s->%s %dx%d pad %d off %d %s" % (xt, yt, rows, cols, pad, offset, tier)
        if yt == "bf16":
            assert_bf16_within_1ulp(got, ref, what)
        else:
            assert_close_f32(got, ref, what)
    ref, _, _ = oracle.layernorm_rows(x, None, None, 1e-5, yt)
    for tier in tiers:
        got = to_host(rr.layernorm_rows(g, eps=1e-5, out_dtype=ydt, tier=tier))
        what = "layernorm %s->%s %dx%d pad %d off %d %s" % (xt, yt, rows, cols, pad, offset, tier)
        if yt == "bf16":
            assert_bf16_within_1ulp(got, ref, what)
        else:
            assert_close_f32(got, ref, what)


AXIS_CASES = []
for i in range(20):
    AXIS_CASES.append((i, int(RNG.integers(1, 6)), int(RNG.integers(1, 3000)),
                       int(RNG.integers(1, 600)), str(RNG.choice(["f32", "i32"])),
                       str(RNG.choice(["sum", "max", "min"]))))


@pytest.mark.parametrize("case", AXIS_CASES, ids=lambda c: "a%d_%dx%dx%d" % c[:4])
def test_random_axis(case):
    i, outer, axis, inner, dt, op = case
    shape = (outer, axis, inner)
    x = (synth.ints_i32(6000 + i, shape, -(2 ** 31), 2 ** 31 - 1) if dt == "i32"
         else synth.normal_f32(6000 + i, shape))
    ref = oracle.reduce_axis(x, op)
    xg = to_gpu(x)
    for tier in ("auto", "tiled", "serial", "splitk"):
        got = to_host(rr.reduce_axis(xg, 1, op, tier))
        what = "axis %s %s %s %s" % (dt, op, shape, tier)
        if dt == "f32" and op == "sum":
            assert_close_f32(got, ref, what)
        else:
            assert_exact(got, ref, what)


# Layernorm with per-column weights (float32 or bf16 gamma / beta) and its
# mean / rstd outputs; drawn after the cases above, which stay as they were.
LN_AFFINE_CASES = []
for i in range(15):
    cols = _cols(RNG)
    rows = int(RNG.integers(1, 20)) if cols > 60000 else int(RNG.integers(1, 400))
    LN_AFFINE_CASES.append((i, rows, cols, int(RNG.integers(0, 5)), int(RNG.integers(0, 3)),
                            str(RNG.choice(["bf16", "f32"])), str(RNG.choice(["bf16", "f32"])),
                            str(RNG.choice(["bf16", "f32"]))))


@pytest.mark.parametrize("case", LN_AFFINE_CASES, ids=lambda c: "n%d_%dx%d" % (c[0], c[1], c[2]))
def test_random_layernorm_with_weights(case):
    i, rows, cols, pad, offset, xt, yt, wt = case
    x = (synth.normal_bf16(7000 + i, (rows, cols)) if xt == "bf16"
         else synth.normal_f32(7000 + i, (rows, cols), 3.0))
    g = _strided(x, pad, offset)
    if wt == "bf16":
        gamma, beta = synth.normal_bf16(7100 + i, (cols,), 2.0), synth.normal_bf16(7200 + i, (cols,), 1.0)
    else:
        gamma, beta = synth.normal_f32(7100 + i, (cols,), 2.0), synth.normal_f32(7200 + i, (cols,))
    ydt = torch.bfloat16 if yt == "bf16" else torch.float32
    ref, ref_mean, ref_rstd = oracle.layernorm_rows(x, gamma, beta, 1e-5, yt)
    for tier in ["auto", "block", "tiled", "splitk"] + (["wave"] if cols <= 64 else []):
        mean = torch.empty(rows, device="cuda")
        rstd = torch.empty(rows, device="cuda")
        got = to_host(rr.layernorm_rows(g, to_gpu(gamma), to_gpu(beta), 1e-5, ydt, tier,
                                        mean_out=mean, rstd_out=rstd))
        what = "layernorm %s->%s, %s weights, %dx%d pad %d off %d %s" % (
            xt, yt, wt, rows, cols, pad, offset, tier)
        if yt == "bf16":
            assert_bf16_within_1ulp(got, ref, what)
        else:
            assert_close_f32(got, ref, what)
        assert_close_f32(to_host(mean), ref_mean, what + " mean")
        assert_close_f32(to_host(rstd), ref_rstd, what + " rstd")


# Sum, max and min from one read: each against the oracle, and each with the
# bits of the single-statistic call on the same tier.
MULTI_CASES = []
for i in range(15):
    cols = _cols(RNG)
    rows = int(RNG.integers(1, 40)) if cols > 60000 else int(RNG.integers(1, 600))
    MULTI_CASES.append((i, rows, cols, int(RNG.integers(0, 5)), int(RNG.integers(0, 3)),
                        str(RNG.choice(["f32", "i32"]))))


@pytest.mark.parametrize("case", MULTI_CASES, ids=lambda c: "m%d_%dx%d" % (c[0], c[1], c[2]))
def test_random_sum_max_min_one_read(case):
    i, rows, cols, pad, offset, dt = case
    x = (synth.ints_i32(7300 + i, (rows, cols), -(2 ** 31), 2 ** 31 - 1) if dt == "i32"
         else synth.normal_f32(7300 + i, (rows, cols)))
    g = _strided(x, pad, offset)
    refs = {k: oracle.reduce_rows(x, k) for k in ("sum", "max", "min")}
    for tier in ["auto", "block", "tiled", "splitk"] + (["wave"] if cols <= 64 else []):
        got = rr.reduce_rows_multi(g, tier=tier)
        for k in ("sum", "max", "min"):
            what = "%s %s of three %dx%d pad %d off %d %s" % (dt, k, rows, cols, pad, offset, tier)
            mine = to_host(got[k])
            if dt == "f32" and k == "sum":
                assert_close_f32(mine, refs[k], what)
            else:
                assert_exact(mine, refs[k], what)
            single = to_host(rr.reduce_rows(g, k, tier))
            assert_exact(mine.view(np.int32), single.view(np.int32), what + " vs single call")
