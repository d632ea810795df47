"""Rows at any element offset and stride: each row's body from its first
16-byte boundary goes in 128-bit chunks, its head and tail element by element
("reduce", algorithm.gpu.rowwise, tier semantics: the full-width tile
function on the aligned chunks, the one-element one on the rest).

Odd row strides put every row at a different offset from a 16-byte boundary;
outputs at another offset than the input exercise the element-wise store
path.  Every case is checked against the oracle at the bars of the other
parity tests."""
import numpy as np
import pytest
import torch

import oracle
import split_deterministic_combine_amd as rr
from split_deterministic_combine_amd import synth
from tests.gpu_util import (assert_bf16_within_1ulp,
                            assert_close_f32, assert_exact, to_gpu, to_host)

pytestmark = pytest.mark.gpu

TORCH = {"bf16": torch.bfloat16, "f32": torch.float32}


def _placed(x_host, offset, pad):
    """x_host's rows at stride cols + pad + offset, each `offset` elements in."""
    rows, cols = x_host.shape
    big = np.zeros((rows, cols + pad + offset), dtype=x_host.dtype)
    big[:, offset:offset + cols] = x_host
    return to_gpu(big)[:, offset:offset + cols]


def _out(rows, cols, dtype, offset, pad):
    big = torch.full((rows, cols + pad + offset), float("nan"), dtype=dtype, device="cuda")
    return big[:, offset:offset + cols]


# --------------------------------------------------------------- reductions

@pytest.mark.parametrize("rows,cols,tiers", [
    (1000, 47, ("auto", "wave", "block", "splitk")),
    (999, 61, ("wave", "block")),
    (777, 5, ("wave", "block", "tiled")),
    (300, 3, ("wave",)),
    (500, 9, ("wave",)),               # 4 lanes per row, head and tail as quads
    (400, 11, ("wave",)),
    (333, 14, ("wave",)),              # 4 lanes: no two lanes past the body
    (300, 55, ("wave",)),              # 16 lanes per row, quads
    (200, 59, ("wave",)),
    (200, 60, ("wave",)),              # 16 lanes: element by element when misaligned
    (64, 1001, ("auto", "block", "splitk")),
    (33, 4099, ("block", "splitk")),
    (5, 70001, ("auto", "block")),
    (3, 131075, ("auto", "splitk")),
])
@pytest.mark.parametrize("offset,pad", [(0, 0), (1, 0), (2, 1), (3, 3)])
def test_reduce_rows_at_any_offset(rows, cols, tiers, offset, pad):
    xf = synth.normal_f32(rows + cols + offset, (rows, cols))
    xi = synth.ints_i32(rows + cols + offset + 1, (rows, cols), -(2 ** 31), 2 ** 31 - 1)
    gf, gi = _placed(xf, offset, pad), _placed(xi, offset, pad)
    for tier in tiers:
        what = "%dx%d off %d pad %d %s" % (rows, cols, offset, pad, tier)
        assert_close_f32(to_host(rr.reduce_rows(gf, "sum", tier)), oracle.reduce_rows(xf, "sum"),
                         "f32 sum " + what)
        assert_exact(to_host(rr.reduce_rows(gf, "max", tier)), oracle.reduce_rows(xf, "max"),
                     "f32 max " + what)
        assert_exact(to_host(rr.reduce_rows(gi, "sum", tier)), oracle.reduce_rows(xi, "sum"),
                     "i32 sum " + what)
        multi = rr.reduce_rows_multi(gi, tier=tier)
        assert_exact(to_host(multi["min"]), oracle.reduce_rows(xi, "min"), "i32 multi min " + what)


def test_reduce_misaligned_rows_are_bit_identical_to_repeats():
    g = _placed(synth.normal_f32(91, (16, 1 << 20)), 1, 0)
    first = rr.reduce_rows(g, "sum").clone()
    for _ in range(9):
        assert torch.equal(rr.reduce_rows(g, "sum").view(torch.int32), first.view(torch.int32))


# ------------------------------------------------------------------ softmax

SOFTMAX_SHAPES = [
    (300, 8191, ("auto",)),            # persistent rows, 1024 chunks, odd stride
    (500, 1001, ("auto", "block")),    # persistent rows, ragged
    (64, 20001, ("block",)),           # long rows, 512 threads in registers
    (9, 40001, ("block",)),            # longer: streamed twice
    (5, 70001, ("auto", "splitk")),    # split-K
    (40, 61, ("block",)),
]


@pytest.mark.parametrize("rows,cols,tiers", SOFTMAX_SHAPES)
@pytest.mark.parametrize("xt,yt", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32"),
                                   ("f32", "bf16")])
@pytest.mark.parametrize("xo,yo,pad", [(0, 0, 1), (1, 1, 0), (3, 0, 2), (5, 2, 0)])
def test_softmax_rows_at_any_offset(rows, cols, tiers, xt, yt, xo, yo, pad):
    x = (synth.normal_bf16(rows + cols + xo, (rows, cols)) if xt == "bf16"
         else synth.normal_f32(rows + cols + xo, (rows, cols), 3.0))
    g = _placed(x, xo, pad)
    ref = oracle.softmax_rows(x, yt)
    for tier in tiers:
        y = _out(rows, cols, TORCH[yt], yo, pad)
        rr.softmax_rows(g, TORCH[yt], tier, out=y)
        what = "%s->%s %dx%d x off %d y off %d pad %d %s" % (xt, yt, rows, cols, xo, yo, pad, tier)
        if yt == "bf16":
            assert_bf16_within_1ulp(to_host(y), ref, what)
        else:
            assert_close_f32(to_host(y), ref, what)


@pytest.mark.parametrize("rows,cols,ld,xt", [
    (300, 8192, 8200, "bf16"),   # whole rows of 1024 chunks, row phase steps by 16 bytes
    (300, 8184, 8184, "bf16"),   # 1023 chunks a row
    (257, 2048, 2056, "bf16"),   # 64 threads x 4 chunks
    (200, 4096, 4100, "f32"),    # f32 chunks of 4
    (150, 1000, 1000, "f32"),
])
@pytest.mark.parametrize("yt", ["bf16", "f32"])
def test_softmax_whole_chunk_rows_off_line(rows, cols, ld, xt, yt):
    # rows that start 16-byte aligned but not on a 128-byte line: the
    # persistent kernel rotates its chunk slots to the lines
    x = (synth.normal_bf16(rows + ld, (rows, cols)) if xt == "bf16"
         else synth.normal_f32(rows + ld, (rows, cols), 3.0))
    g = _placed(x, 0, ld - cols)
    y = _out(rows, cols, TORCH[yt], 0, ld - cols)
    rr.softmax_rows(g, TORCH[yt], out=y)
    ref = oracle.softmax_rows(x, yt)
    what = "%s->%s %dx%d ld %d" % (xt, yt, rows, cols, ld)
    if yt == "bf16":
        assert_bf16_within_1ulp(to_host(y), ref, what)
    else:
        assert_close_f32(to_host(y), ref, what)
    # the padding between rows is never written
    big = y.as_strided((rows, ld - cols), (ld, 1), cols)
    assert torch.all(torch.isnan(big.float())), what


def test_softmax_odd_stride_rows_persistent_plan_and_repeats():
    x = synth.normal_bf16(92, (2000, 8191))
    g = to_gpu(x)
    plan = rr.plan_softmax(2000, 8191, cu_count=rr.device_cu_count())
    assert plan["tier"] == "block" and plan["grid"] < 2000  # persistent rows
    first = rr.softmax_rows(g).clone()
    for _ in range(4):
        assert torch.equal(rr.softmax_rows(g).view(torch.int16), first.view(torch.int16))
    sample = np.array([0, 1, 2, 3, 999, 1998, 1999])
    ref = oracle.softmax_rows(np.ascontiguousarray(x[sample]), "bf16")
    assert_bf16_within_1ulp(to_host(first)[sample], ref, "odd stride sample rows")


# ---------------------------------------------------------------- layernorm

LN_SHAPES = [
    (300, 4095, ("auto", "block")),    # one row per workgroup, odd stride
    (70, 1001, ("auto", "block")),
    (9, 40001, ("block",)),            # streamed
    (3, 70001, ("auto", "splitk")),    # split-K: one phase for every row, or element-wise
    (50, 33, ("block",)),
]


@pytest.mark.parametrize("rows,cols,tiers", LN_SHAPES)
@pytest.mark.parametrize("xt,yt", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32")])
@pytest.mark.parametrize("xo,yo,pad", [(1, 1, 0), (3, 0, 2), (4, 4, 4), (3, 3, 4)])
def test_layernorm_rows_at_any_offset(rows, cols, tiers, xt, yt, xo, yo, pad):
    x = synth.normal_f32(rows + cols + xo, (rows, cols), 2.0) + np.float32(0.5)
    if xt == "bf16":
        x = synth._bf16_bits(x)
    g = _placed(x, xo, pad)
    for wmode in ("f32", "bf16"):
        gw = synth.uniform_f32(cols + 7, (cols,), 0.5, 1.5)
        bw = synth.uniform_f32(cols + 8, (cols,), -0.5, 0.5)
        if wmode == "bf16":
            gw, bw = synth._bf16_bits(gw), synth._bf16_bits(bw)
        ref, rmean, rrstd = oracle.layernorm_rows(x, gw, bw, 1e-5, yt)
        for tier in tiers:
            y = _out(rows, cols, TORCH[yt], yo, pad)
            mean = torch.full((rows,), float("nan"), device="cuda")
            rstd = torch.full((rows,), float("nan"), device="cuda")
            rr.layernorm_rows(g, to_gpu(gw), to_gpu(bw), 1e-5, TORCH[yt], tier, out=y,
                              mean_out=mean, rstd_out=rstd)
            what = "%s->%s %dx%d x off %d y off %d pad %d w %s %s" % (
                xt, yt, rows, cols, xo, yo, pad, wmode, tier)
            if yt == "bf16":
                assert_bf16_within_1ulp(to_host(y), ref, what)
            else:
                assert_close_f32(to_host(y), ref, what)
            assert_close_f32(to_host(mean), rmean, what + " mean")
            assert_close_f32(to_host(rstd), rrstd, what + " rstd")
