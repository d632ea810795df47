"""GPU parity for the two-pass layernorm: the HIP path (through the C ABI)
against the CPU oracle, element by element, on seeded inputs.

Bars: float32 outputs (y, mean, rstd) within rel 1e-5 / abs 1e-6 of the
oracle; bf16 outputs within 1 bf16 ulp, or within the float32 bar's absolute
1e-6 where gamma * d * rstd + beta cancels to near zero (float arithmetic's
error there is absolute).
"""
import numpy as np
import pytest
import torch

import oracle
import split_deterministic_combine_amd as rr
from split_deterministic_combine_amd import synth
from tests.gpu_util import (assert_bf16_within_1ulp, assert_close_f32, to_gpu,
                            to_host)

pytestmark = pytest.mark.gpu

LN_COLS = [1, 2, 3, 5, 8, 9, 16, 31, 33, 64, 65, 100, 1000, 2047, 2048, 2049, 4096, 8191, 8192,
           8200, 16384, 16385, 20000]
LN_TYPES = [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32"), ("f32", "bf16")]
TORCH = {"bf16": torch.bfloat16, "f32": torch.float32}


def _x(xt, rows, cols, seed, std=2.0, mean=0.5):
    x = synth.normal_f32(seed, (rows, cols), std) + np.float32(mean)
    return synth._bf16_bits(x) if xt == "bf16" else x


def _weights(mode, cols, seed):
    if mode == "none":
        return None, None
    g = synth.uniform_f32(seed, (cols,), 0.5, 1.5)
    b = synth.uniform_f32(seed + 1, (cols,), -0.5, 0.5)
    if mode == "bf16":
        return synth._bf16_bits(g), synth._bf16_bits(b)
    return g, b


def _check_y(gpu, ref, yt, what):
    if yt == "bf16":
        assert_bf16_within_1ulp(gpu, ref, what)
    else:
        assert_close_f32(gpu, ref, what)


def _run(xh, yt, tier, g=None, b=None, eps=1e-5, x_dev=None, out=None):
    """Run the GPU layernorm; returns host (y, mean, rstd)."""
    xg = to_gpu(xh) if x_dev is None else x_dev
    rows = xg.shape[0]
    mean = torch.full((rows,), float("nan"), device="cuda")
    rstd = torch.full((rows,), float("nan"), device="cuda")
    gg = None if g is None else to_gpu(g)
    bb = None if b is None else to_gpu(b)
    y = rr.layernorm_rows(xg, gg, bb, eps, TORCH[yt], tier, out=out, mean_out=mean, rstd_out=rstd)
    torch.cuda.synchronize()
    return to_host(y), to_host(mean), to_host(rstd)


def _tiers(cols):
    tiers = ["auto", "block", "tiled", "splitk"]
    if cols <= 5000:
        tiers.append("serial")
    if cols <= 64:
        tiers.append("wave")
    return tiers


@pytest.mark.parametrize("tier,rows,cols", [("auto", 512, 4096), ("block", 64, 5000),
                                             ("wave", 600, 40), ("tiled", 300, 33),
                                             ("splitk", 4, 70000), ("block", 16, 100000)])
def test_layernorm_rounds_once_from_double(tier, rows, cols):
    # every tier forms y = (x - mean) * rstd * gamma + beta in double and
    # rounds it once, as the oracle does: all but a tiny fraction of the bf16
    # outputs (those whose double value lies within a few double ulps of a
    # rounding boundary, where the two summation orders may fall either
    # side) carry the oracle's bits; the rest are 1 ulp away.  With gamma and
    # beta spread so that gamma * d and beta cancel often.
    x = synth.normal_f32(1700 + cols, (rows, cols), 2.0) + np.float32(0.5)
    x = synth._bf16_bits(x)
    g = synth.uniform_f32(1701 + cols, (cols,), -2.0, 2.0)
    b = synth.uniform_f32(1702 + cols, (cols,), -2.0, 2.0)
    ref, _, _ = oracle.layernorm_rows(x, g, b, 1e-5, "bf16")
    y, _, _ = _run(x, "bf16", tier, g, b)
    off = assert_bf16_within_1ulp(y, ref, "layernorm %s %dx%d" % (tier, rows, cols))
    assert off <= max(2, y.size // 100000), (tier, off, y.size)


@pytest.mark.parametrize("cols", LN_COLS)
@pytest.mark.parametrize("xt,yt", LN_TYPES)
def test_layernorm_edge_widths_all_tiers(cols, xt, yt):
    rows = 13
    x = _x(xt, rows, cols, 700 + cols)
    for wmode in ("none", "f32", "bf16"):
        g, b = _weights(wmode, cols, 800 + cols)
        ref, rmean, rrstd = oracle.layernorm_rows(x, g, b, 1e-5, yt)
        for tier in _tiers(cols):
            y, mean, rstd = _run(x, yt, tier, g, b)
            what = "cols %d %s->%s w %s %s" % (cols, xt, yt, wmode, tier)
            _check_y(y, ref, yt, what)
            assert_close_f32(mean, rmean, what + " mean")
            assert_close_f32(rstd, rrstd, what + " rstd")


@pytest.mark.parametrize("pad,offset", [(8, 0), (0, 1), (3, 5)])
@pytest.mark.parametrize("cols", [7, 40, 1000, 4096])
def test_layernorm_strided_and_misaligned_rows(pad, offset, cols):
    rows = 11
    x = _x("bf16", rows, cols, 900 + cols)
    g, b = _weights("f32", cols, 950)
    ref, _, _ = oracle.layernorm_rows(x, g, b, 1e-5, "bf16")
    big = np.zeros((rows, cols + pad + offset), dtype=np.uint16)
    big[:, offset:offset + cols] = x
    xg = to_gpu(big)[:, offset:offset + cols]
    for tier in _tiers(cols):
        out = torch.empty((rows, cols + pad + offset), dtype=torch.bfloat16, device="cuda")
        yv = out[:, offset:offset + cols]
        rr.layernorm_rows(xg, to_gpu(g), to_gpu(b), 1e-5, torch.bfloat16, tier, out=yv)
        _check_y(to_host(yv), ref, "bf16", "cols %d pad %d off %d %s" % (cols, pad, offset, tier))


def test_layernorm_misaligned_weights():
    cols = 1000
    x = _x("f32", 5, cols, 31)
    g, b = _weights("f32", cols + 1, 32)
    ref, _, _ = oracle.layernorm_rows(x, g[1:].copy(), b[1:].copy(), 1e-5, "f32")
    gg, bb = to_gpu(g)[1:], to_gpu(b)[1:]
    for tier in ("block", "splitk", "tiled"):
        y = rr.layernorm_rows(to_gpu(x), gg, bb, 1e-5, torch.float32, tier)
        assert_close_f32(to_host(y), ref, "misaligned weights " + tier)


@pytest.mark.parametrize("shape", [(9, 3000), (3, 100003), (40, 48)])
def test_layernorm_large_mean_offset(shape):
    # |mean| / sd = 1000: the statistics must not lose the deviations
    x = synth.normal_f32(33, shape) + np.float32(1000.0)
    ref, rmean, rrstd = oracle.layernorm_rows(x, None, None, 1e-5, "f32")
    for tier in _tiers(shape[1]):
        y, mean, rstd = _run(x, "f32", tier)
        assert_close_f32(y, ref, "offset %s %s" % (shape, tier))
        assert_close_f32(mean, rmean, "offset mean %s" % tier)
        assert_close_f32(rstd, rrstd, "offset rstd %s" % tier)


def test_layernorm_constant_rows():
    cols = 3000
    x = np.full((4, cols), 2.5, dtype=np.float32)
    g, b = _weights("f32", cols, 40)
    for tier in _tiers(cols):
        y, mean, rstd = _run(x, "f32", tier, g, b, eps=0.25)
        assert np.array_equal(y, np.broadcast_to(b, y.shape)), tier   # x - mean = 0 exactly
        assert np.all(mean == 2.5) and np.all(rstd == 2.0), tier
        y, _, rstd = _run(x, "f32", tier, eps=0.0)
        assert np.isnan(y).all() and np.isinf(rstd).all(), tier       # 0 * inf, as defined


def test_layernorm_in_place():
    x = _x("bf16", 9, 3000, 41)
    ref, _, _ = oracle.layernorm_rows(x, None, None, 1e-5, "bf16")
    for tier in ("block", "splitk", "tiled"):
        g = to_gpu(x)
        rr.layernorm_rows(g, eps=1e-5, tier=tier, out=g)
        assert_bf16_within_1ulp(to_host(g), ref, "in place " + tier)


SPLITK_LN_SHAPES = [(1, 65536), (3, 70001), (7, 100003), (2, 262144 + 8), (5, 131072 - 1)]


@pytest.mark.parametrize("rows,cols", SPLITK_LN_SHAPES)
@pytest.mark.parametrize("xt,yt", LN_TYPES)
def test_layernorm_splitk_parity(rows, cols, xt, yt):
    x = _x(xt, rows, cols, 1900 + cols + rows)
    g, b = _weights("f32", cols, 1950)
    ref, rmean, rrstd = oracle.layernorm_rows(x, g, b, 1e-5, yt)
    xtd = TORCH[xt]
    assert rr.plan_layernorm(rows, cols, xtd, TORCH[yt], cu_count=rr.device_cu_count())["slices"] > 1
    assert rr.select_tier("layernorm", rows, cols, xtd) == "splitk"
    for tier in ("auto", "splitk"):
        y, mean, rstd = _run(x, yt, tier, g, b)
        what = "splitk %dx%d %s->%s %s" % (rows, cols, xt, yt, tier)
        _check_y(y, ref, yt, what)
        assert_close_f32(mean, rmean, what + " mean")
        assert_close_f32(rstd, rrstd, what + " rstd")


def test_layernorm_splitk_bit_identical_and_workspace_contents_unused():
    xg = to_gpu(synth.normal_bf16(51, (16, 1 << 20)))
    first = rr.layernorm_rows(xg).clone()
    for _ in range(3):
        assert torch.equal(rr.layernorm_rows(xg).view(torch.int16), first.view(torch.int16))
    for key, ws in rr._workspaces.items():
        if key[0] == "layernorm":
            ws.fill_(0x5A)
    assert torch.equal(rr.layernorm_rows(xg).view(torch.int16), first.view(torch.int16))
    sample = np.array([0, 9])
    ref, _, _ = oracle.layernorm_rows(np.ascontiguousarray(to_host(xg)[sample]), None, None,
                                      1e-5, "bf16")
    assert_bf16_within_1ulp(to_host(first)[sample], ref, "splitk 16 x 2^20 sample rows")


def test_layernorm_rows_config_full_size():
    x, g, b = synth.layernorm_rows()
    xg = to_gpu(x)
    mean = torch.empty(x.shape[0], device="cuda")
    rstd = torch.empty(x.shape[0], device="cuda")
    y = rr.layernorm_rows(xg, to_gpu(g), to_gpu(b), 1e-5, mean_out=mean, rstd_out=rstd)
    again = rr.layernorm_rows(xg, to_gpu(g), to_gpu(b), 1e-5)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), again.view(torch.int16))
    sample = np.linspace(0, x.shape[0] - 1, 61).astype(np.int64)
    ref, rmean, rrstd = oracle.layernorm_rows(np.ascontiguousarray(x[sample]), g, b, 1e-5, "bf16")
    assert_bf16_within_1ulp(to_host(y)[sample], ref, "layernorm_rows sample")
    assert_close_f32(to_host(mean)[sample], rmean, "layernorm_rows mean")
    assert_close_f32(to_host(rstd)[sample], rrstd, "layernorm_rows rstd")


PERSISTENT_SHAPES = [(40000, 512), (20000, 1000), (20000, 1024), (6000, 2048), (4000, 4096),
                     (2000, 8192), (700, 16384), (3000, 4000)]


@pytest.mark.parametrize("rows,cols", PERSISTENT_SHAPES)
def test_layernorm_persistent_rows_walk_several_rows(rows, cols):
    # every persistent (threads, chunks) shape with several rows per workgroup
    x = _x("bf16", rows, cols, 3200 + cols)
    g, b = _weights("f32", cols, 3300 + cols)
    plan = rr.plan_layernorm(rows, cols, cu_count=rr.device_cu_count())
    assert plan["tier"] == "block" and plan["grid"] < rows
    mean = torch.empty(rows, device="cuda")
    rstd = torch.empty(rows, device="cuda")
    y = rr.layernorm_rows(to_gpu(x), to_gpu(g), to_gpu(b), 1e-5, mean_out=mean, rstd_out=rstd)
    torch.cuda.synchronize()
    sample = np.unique(np.concatenate([np.linspace(0, rows - 1, 40).astype(np.int64),
                                       np.arange(rows - 5, rows)]))
    ref, rm, rs = oracle.layernorm_rows(np.ascontiguousarray(x[sample]), g, b, 1e-5, "bf16")
    what = "persistent %dx%d" % (rows, cols)
    assert_bf16_within_1ulp(to_host(y)[sample], ref, what)
    assert_close_f32(to_host(mean)[sample], rm, what + " mean")
    assert_close_f32(to_host(rstd)[sample], rs, what + " rstd")


def test_layernorm_block_tier_bit_identical_across_runs():
    g = to_gpu(synth.normal_bf16(52, (2048, 8192)))
    first = rr.layernorm_rows(g).clone()
    for _ in range(3):
        assert torch.equal(rr.layernorm_rows(g).view(torch.int16), first.view(torch.int16))
