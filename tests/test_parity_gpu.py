"""GPU parity: the HIP path (through the C ABI) against the CPU oracle,
element by element, on seeded inputs from the shared generators.

Bars: int32 results and float max/min bit-exact; float32 results within
rel 1e-5 / abs 1e-6 of the oracle; bf16 results within 1 bf16 ulp.
"""
import numpy as np
import pytest
import torch

import oracle
import split_deterministic_combine_amd as rr
from split_deterministic_combine_amd import synth
from tests.gpu_util import (assert_bf16_within_1ulp, assert_close_f32, assert_exact, to_gpu,
                            to_host)

pytestmark = pytest.mark.gpu

REDUCE_OPS = [(np.float32, "sum"), (np.float32, "max"), (np.float32, "min"),
              (np.int32, "sum"), (np.int32, "max"), (np.int32, "min")]


def _legal_tiers(cols):
    tiers = ["auto", "block", "tiled", "serial", "splitk"]
    if cols <= 64:
        tiers.append("wave")
    return tiers


def _make_reduce_input(dtype, rows, cols, seed):
    if dtype == np.int32:
        return synth.ints_i32(seed, (rows, cols), -(2 ** 31), 2 ** 31 - 1)
    return synth.normal_f32(seed, (rows, cols))


def _check_reduce(gpu, ref, dtype, op, what):
    if dtype == np.float32 and op == "sum":
        assert_close_f32(gpu, ref, what)
    else:
        assert_exact(gpu, ref, what)


def _run_reduce(x_host, op, tier, pad=0, offset=0):
    """Run rr.reduce_rows on a copy of x_host whose rows sit at stride
    cols + pad + offset, starting `offset` elements into each row."""
    rows, cols = x_host.shape
    if pad or offset:
        big = np.zeros((rows, cols + pad + offset), dtype=x_host.dtype)
        big[:, offset:offset + cols] = x_host
        g = to_gpu(big)[:, offset:offset + cols]
    else:
        g = to_gpu(x_host)
    y = rr.reduce_rows(g, op, tier)
    torch.cuda.synchronize()
    return to_host(y)


# ------------------------------------------------------------------ reduce

@pytest.mark.parametrize("tier", ["auto", "block", "tiled", "serial", "splitk"])
def test_reduce_small_rows_config(tier):
    xf, xi = synth.small_rows()
    for x in (xf, xi):
        for op in ("sum", "max", "min"):
            _check_reduce(_run_reduce(x, op, tier), oracle.reduce_rows(x, op), x.dtype.type, op,
                          "small_rows %s %s %s" % (x.dtype, op, tier))


EDGE_COLS = [0, 1, 2, 3, 4, 5, 7, 8, 15, 16, 17, 47, 48, 63, 64, 65, 127, 128, 1000, 1024, 4097]


@pytest.mark.parametrize("cols", EDGE_COLS)
@pytest.mark.parametrize("dtype,op", REDUCE_OPS)
def test_reduce_edge_widths_all_tiers(cols, dtype, op):
    x = _make_reduce_input(dtype, 37, cols, 1000 + cols)
    ref = oracle.reduce_rows(x, op)
    for tier in _legal_tiers(cols):
        _check_reduce(_run_reduce(x, op, tier), ref, dtype, op, "cols %d %s" % (cols, tier))


@pytest.mark.parametrize("pad,offset", [(3, 0), (0, 1), (5, 2), (4, 0)])
@pytest.mark.parametrize("cols", [5, 48, 61, 1000, 70001])
def test_reduce_strided_and_misaligned_rows(pad, offset, cols):
    rows = 6 if cols > 10000 else 29
    for dtype, op in REDUCE_OPS:
        x = _make_reduce_input(dtype, rows, cols, 77 + cols + pad)
        ref = oracle.reduce_rows(x, op)
        for tier in _legal_tiers(cols):
            if tier == "serial" and cols > 10000:
                continue
            got = _run_reduce(x, op, tier, pad, offset)
            _check_reduce(got, ref, dtype, op, "cols %d pad %d off %d %s" % (cols, pad, offset, tier))


def test_reduce_short_rows_config_full_size():
    x = synth.short_rows()
    g = to_gpu(x)
    for op in ("sum", "max"):
        y = to_host(rr.reduce_rows(g, op))
        _check_reduce(y, oracle.reduce_rows(x, op), np.float32, op, "short_rows " + op)


@pytest.mark.parametrize("rows,cols", [(1, 65536), (3, 70001), (7, 100003), (5, 1 << 20), (255, 65536)])
def test_reduce_splitk_shapes(rows, cols):
    for dtype, op in REDUCE_OPS:
        x = _make_reduce_input(dtype, rows, cols, rows * 7 + cols)
        ref = oracle.reduce_rows(x, op)
        for tier in ("auto", "splitk", "block"):
            _check_reduce(_run_reduce(x, op, tier), ref, dtype, op, "%dx%d %s" % (rows, cols, tier))


# Block tier on persistent rows: calls with at least 4 rows per CU whose rows
# fit a workgroup's registers (up to 2048 16-byte chunks) walk several rows
# per workgroup with the next row's loads in flight; every row shape, aligned,
# strided and starting at every element offset.
PF_REDUCE_SHAPES = [  # rows, cols, pad, offset
    (20000, 65, 0, 0), (20000, 100, 0, 1), (20000, 256, 0, 0), (20000, 257, 2, 3),
    (5000, 1000, 0, 0), (5000, 1001, 0, 0), (3000, 2048, 4, 0), (1100, 4095, 0, 2),
    (1030, 8192, 0, 0), (1030, 8191, 1, 1),
    # rows shorter than a chunk (head and tail elements only), forced to the block tier
    (20000, 1, 0, 1), (20000, 3, 1, 2), (20000, 5, 0, 3), (20000, 7, 2, 1),
    # 2 and 4 rows per wavefront, with a last step that has fewer rows
    (20001, 300, 0, 1), (20003, 120, 0, 0), (20002, 96, 3, 2), (20001, 512, 0, 0)]


def _pf_threads(cols):
    chunks = -(-cols // 4)
    return 64 if chunks <= 256 else 128 if chunks <= 512 else 256 if chunks <= 1024 else 512


@pytest.mark.parametrize("rows,cols,pad,offset", PF_REDUCE_SHAPES)
def test_reduce_block_tier_persistent_rows(rows, cols, pad, offset):
    cu = rr.device_cu_count()
    plan = rr.plan_reduce(rows, cols, cu_count=cu, tier="block")
    assert rows >= 4 * cu and plan["block"] == _pf_threads(cols), plan
    assert plan["grid"] < rows, plan                      # every workgroup walks several rows
    for dtype, op in REDUCE_OPS:
        x = _make_reduce_input(dtype, rows, cols, rows + 3 * cols + offset)
        ref = oracle.reduce_rows(x, op)
        first = _run_reduce(x, op, "block", pad, offset)
        _check_reduce(first, ref, dtype, op, "%dx%d pad %d off %d %s" % (rows, cols, pad, offset, op))
        again = _run_reduce(x, op, "auto" if cols > 64 else "block", pad, offset)
        if rr.plan_reduce(rows, cols, cu_count=cu)["tier"] == "block":
            assert np.array_equal(first.view(np.int32), again.view(np.int32)), (rows, cols, op)


def test_splitk_with_one_slice_equals_block_tier_bitwise():
    for cols in (100, 1000, 4097, 16384):
        x = synth.uniform_f32(cols, (40, cols))
        assert rr.plan_reduce(40, cols, tier="splitk")["slices"] == 1
        for op in ("sum", "max"):
            assert_exact(_run_reduce(x, op, "splitk"), _run_reduce(x, op, "block"), "G=1 %d" % cols)


def test_int_results_identical_across_tiers():
    x = synth.ints_i32(5, (50, 64), -(2 ** 31), 2 ** 31 - 1)
    for op in ("sum", "max", "min"):
        outs = [_run_reduce(x, op, t) for t in ("wave", "block", "tiled", "serial", "splitk")]
        for o in outs[1:]:
            assert_exact(o, outs[0], op)


@pytest.mark.parametrize("rows,cols", [(37, 4097), (3, 70001), (600, 48)])
def test_int_results_invariant_under_column_permutation(rows, cols):
    """The combine is associative and commutative for int32 sum (wrapping),
    max and min ("cluster_allreduce", description of combine_fn), so a row
    and its columns in any order give the same bits, on every tier."""
    x = synth.ints_i32(31 + cols, (rows, cols), -(2 ** 31), 2 ** 31 - 1)
    xp = np.ascontiguousarray(x[:, np.random.default_rng(cols).permutation(cols)])
    tiers = ["auto", "block", "tiled", "splitk"] + (["wave"] if cols <= 64 else [])
    if cols <= 4096:
        tiers.append("serial")
    for op in ("sum", "max", "min"):
        ref = oracle.reduce_rows(x, op)
        for t in tiers:
            a, b = _run_reduce(x, op, t), _run_reduce(xp, op, t)
            assert_exact(a, ref, "%s %s" % (op, t))
            assert_exact(b, a, "%s %s permuted" % (op, t))


def test_reduce_rows_zero_is_noop_and_empty_rows_get_identity():
    g = torch.zeros((0, 16), device="cuda")
    assert rr.reduce_rows(g).shape == (0,)
    e = torch.zeros((5, 0), device="cuda")
    assert torch.all(rr.reduce_rows(e, "max") == -float("inf"))
    assert torch.all(rr.reduce_rows(e, "min") == float("inf"))
    assert torch.all(rr.reduce_rows(e, "sum") == 0)
    ei = torch.zeros((5, 0), dtype=torch.int32, device="cuda")
    assert torch.all(rr.reduce_rows(ei, "max") == -(2 ** 31))


def test_reduce_float_max_min_total_order_cases():
    rows = np.array([[-0.0, 0.0, -0.0], [0.0, -0.0, 0.0], [1.0, np.nan, -2.0], [-np.inf, -1.0, -5.0]],
                    dtype=np.float32)
    neg_nan = np.array([0xFFC00000], dtype=np.uint32).view(np.float32)[0]
    rows = np.concatenate([rows, np.array([[3.0, neg_nan, 1.0]], dtype=np.float32)])
    for op in ("max", "min"):
        ref = oracle.reduce_rows(rows, op)
        for tier in ("wave", "block", "tiled", "serial", "splitk"):
            assert_exact(_run_reduce(rows, op, tier), ref, "%s %s" % (op, tier))


# ----------------------------------------------------- long rows (split-K)

@pytest.fixture(scope="module")
def long_rows_data():
    xf, xi = synth.long_rows()
    return xf, xi, to_gpu(xf), to_gpu(xi)


def test_long_rows_config_matches_oracle(long_rows_data):
    xf, xi, gf, gi = long_rows_data
    assert rr.plan_reduce(16, 1 << 24)["tier"] == "splitk"
    assert_close_f32(to_host(rr.reduce_rows(gf, "sum")), oracle.reduce_rows(xf, "sum"), "f32 sum")
    assert_exact(to_host(rr.reduce_rows(gi, "max")), oracle.reduce_rows(xi, "max"), "i32 max")


def test_long_rows_bit_identical_across_ten_runs(long_rows_data):
    _, _, gf, gi = long_rows_data
    first_f = rr.reduce_rows(gf, "sum").clone()
    first_i = rr.reduce_rows(gi, "max").clone()
    for _ in range(9):
        assert torch.equal(rr.reduce_rows(gf, "sum").view(torch.int32), first_f.view(torch.int32))
        assert torch.equal(rr.reduce_rows(gi, "max"), first_i)


def test_long_rows_bits_do_not_depend_on_arrival_order(long_rows_data):
    # Slices publish in (roughly) descending rank order under the skew hook;
    # the last-arriver fold still visits ranks in ascending order.
    _, _, gf, gi = long_rows_data
    plain_f = rr.reduce_rows(gf, "sum").clone()
    plain_i = rr.reduce_rows(gi, "max").clone()
    try:
        rr._set_splitk_skew(16)
        skew_f = rr.reduce_rows(gf, "sum").clone()
        skew_i = rr.reduce_rows(gi, "max").clone()
        torch.cuda.synchronize()
    finally:
        rr._set_splitk_skew(0)
    assert torch.equal(skew_f.view(torch.int32), plain_f.view(torch.int32))
    assert torch.equal(skew_i, plain_i)


def test_splitk_workspace_is_left_zero_for_any_next_shape():
    # The last workgroup of each row resets its ticket and clears the partial
    # slots it read, so the whole workspace is zero after every call and a
    # call with more rows (tickets where the last call kept partials) works.
    x = synth.uniform_f32(9, (3, 200000))
    rr.reduce_rows(to_gpu(x), "sum", "splitk")
    torch.cuda.synchronize()
    for key, ws in rr._workspaces.items():
        if key[0] == "reduce":
            assert int(ws.count_nonzero()) == 0
    xb = synth.uniform_f32(10, (255, 65536))
    y = rr.reduce_rows(to_gpu(xb), "sum", "splitk")
    assert_close_f32(to_host(y), oracle.reduce_rows(xb, "sum"), "more rows after fewer")
    torch.cuda.synchronize()
    reduce_ws = [ws for key, ws in rr._workspaces.items() if key[0] == "reduce"]
    assert reduce_ws
    for ws in reduce_ws:
        assert int(ws[:256].count_nonzero()) == 0


# ----------------------------------------------------------------- softmax

SOFTMAX_COLS = [1, 2, 3, 5, 8, 9, 16, 31, 33, 64, 65, 100, 1000, 2047, 2048, 2049, 4096, 8191,
                8192, 8200, 16384, 16385, 20000]
SOFTMAX_TYPES = [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32"), ("f32", "bf16")]


def _softmax_input(xt, rows, cols, seed, std=3.0):
    return synth.normal_bf16(seed, (rows, cols), std) if xt == "bf16" else synth.normal_f32(
        seed, (rows, cols), std)


def _check_softmax(gpu, ref, yt, what):
    if yt == "bf16":
        assert_bf16_within_1ulp(gpu, ref, what)
    else:
        assert_close_f32(gpu, ref, what)


def _softmax_tiers(cols):
    tiers = ["auto", "block", "tiled", "serial", "splitk"]
    if cols <= 64:
        tiers.append("wave")
    return tiers


@pytest.mark.parametrize("cols", SOFTMAX_COLS)
@pytest.mark.parametrize("xt,yt", SOFTMAX_TYPES)
def test_softmax_edge_widths_all_tiers(cols, xt, yt):
    rows = 13
    x = _softmax_input(xt, rows, cols, 500 + cols)
    ref = oracle.softmax_rows(x, yt)
    ydt = torch.bfloat16 if yt == "bf16" else torch.float32
    for tier in _softmax_tiers(cols):
        if tier == "serial" and cols > 5000:
            continue
        y = to_host(rr.softmax_rows(to_gpu(x), ydt, tier))
        _check_softmax(y, ref, yt, "cols %d %s->%s %s" % (cols, xt, yt, tier))


@pytest.mark.parametrize("pad,offset", [(8, 0), (0, 1), (3, 5)])
@pytest.mark.parametrize("cols", [7, 40, 1000, 8192])
def test_softmax_strided_and_misaligned_rows(pad, offset, cols):
    rows = 11
    x = _softmax_input("bf16", rows, cols, 900 + cols)
    ref = oracle.softmax_rows(x, "bf16")
    big = np.zeros((rows, cols + pad + offset), dtype=np.uint16)
    big[:, offset:offset + cols] = x
    g = to_gpu(big)[:, offset:offset + cols]
    for tier in _softmax_tiers(cols):
        out = torch.empty((rows, cols + pad + offset), dtype=torch.bfloat16, device="cuda")
        yv = out[:, offset:offset + cols]
        rr.softmax_rows(g, torch.bfloat16, tier, out=yv)
        _check_softmax(to_host(yv), ref, "bf16", "cols %d pad %d off %d %s" % (cols, pad, offset, tier))


# Persistent block tier: every (threads, chunks) shape, with enough rows that
# each workgroup walks several rows through its prefetch loop.
PERSISTENT_SHAPES = [(40000, 512), (20000, 1000), (20000, 1024), (6000, 2048), (4000, 4096),
                     (2000, 8192), (700, 16384), (3000, 4000)]


@pytest.mark.parametrize("rows,cols", PERSISTENT_SHAPES)
def test_softmax_persistent_rows_walk_several_rows(rows, cols):
    x = synth.normal_bf16(3100 + cols, (rows, cols))
    plan = rr.plan_softmax(rows, cols, cu_count=rr.device_cu_count())
    assert plan["tier"] == "block" and plan["grid"] < rows
    y = rr.softmax_rows(to_gpu(x))
    torch.cuda.synchronize()
    # sampled rows against the oracle, including the last rows of the walk
    sample = np.unique(np.concatenate([np.linspace(0, rows - 1, 40).astype(np.int64),
                                       np.arange(rows - 5, rows)]))
    ref = oracle.softmax_rows(np.ascontiguousarray(x[sample]), "bf16")
    assert_bf16_within_1ulp(to_host(y)[sample], ref, "persistent %dx%d" % (rows, cols))
    s = y.float().sum(dim=1)
    assert float((s - 1).abs().max()) <= 2.0 ** -8


def test_softmax_rows_config_full_size():
    # bf16 [8192, 8192], logits normal(0, 3): every row against the oracle,
    # in the launch the planner picks for this shape, then ten runs bit-identical.
    x = synth.softmax_rows()
    rows, cols = x.shape
    plan = rr.plan_softmax(rows, cols, cu_count=rr.device_cu_count())
    assert plan["tier"] == "block"
    g = to_gpu(x)
    y = rr.softmax_rows(g)
    torch.cuda.synchronize()
    assert_bf16_within_1ulp(to_host(y), oracle.softmax_rows(x, "bf16"), "softmax config")
    first = y.clone()
    for _ in range(9):
        assert torch.equal(rr.softmax_rows(g).view(torch.int16), first.view(torch.int16))


def test_softmax_uniform_row_is_exactly_2_pow_minus_13():
    x = torch.full((4, 8192), 3.0, dtype=torch.bfloat16, device="cuda")
    y = to_host(rr.softmax_rows(x))
    assert np.all(y == 0x3900)


def test_softmax_special_values():
    x = np.array([[0.0, -np.inf, 1.0, 2.0] * 16,
                  [-np.inf] * 64,
                  [-100.0, 0.0, 100.0, -50.0] * 16,
                  [87.0, -87.0, 0.0, 60.0] * 16], dtype=np.float32)
    for xt in ("f32", "bf16"):
        xin = x if xt == "f32" else synth._bf16_bits(x)
        for yt in ("f32", "bf16"):
            ref = oracle.softmax_rows(xin, yt)
            ydt = torch.bfloat16 if yt == "bf16" else torch.float32
            for tier in ("wave", "block", "tiled", "serial", "splitk"):
                y = to_host(rr.softmax_rows(to_gpu(xin), ydt, tier))
                _check_softmax(y, ref, yt, "special %s->%s %s" % (xt, yt, tier))


def test_softmax_wide_logit_range():
    # exp of differences below -87 lands in the float32 subnormal range
    x = synth.uniform_f32(31, (16, 3000), -120.0, 20.0)
    for yt in ("f32", "bf16"):
        ref = oracle.softmax_rows(x, yt)
        ydt = torch.bfloat16 if yt == "bf16" else torch.float32
        y = to_host(rr.softmax_rows(to_gpu(x), ydt))
        _check_softmax(y, ref, yt, "wide range " + yt)


def _spiked_rows(seed, rows, cols, offset, spikes=8):
    """Rows at a large common offset: `spikes` entries spread over the row at
    offset + N(0, 1), the rest 40 below (their exponentials ~1e-17), so the
    outputs that matter are ~1/spikes and the relative 1e-5 term of the f32
    bar decides pass or fail, wherever the tier puts its per-thread maxima."""
    rng = np.random.default_rng(seed)
    x = (offset - 40.0 + rng.standard_normal((rows, cols))).astype(np.float32)
    for r in range(rows):
        at = rng.choice(cols, size=min(spikes, cols), replace=False)
        x[r, at] = (offset + rng.standard_normal(at.size)).astype(np.float32)
    return x


@pytest.mark.parametrize("offset", [-3000.0, -1000.0, 1000.0, 3000.0, 1.0e6])
def test_softmax_large_row_maxima_keep_the_relative_bar(offset):
    # The exponent argument must be formed from x - m: a rounded m*log2(e)
    # would put an error of half an ulp of |m|*1.44 into every exponent (a
    # relative error of 4e-5 at |m| = 1000), different in every thread.
    for cols, tiers in ((10, ("auto", "wave", "block", "tiled", "serial")),
                        (3000, ("auto", "block", "tiled")),
                        (8192, ("auto", "block")),
                        (70001, ("auto", "splitk"))):
        rows = 7 if cols > 5000 else 24
        x = _spiked_rows(int(abs(offset)) + cols, rows, cols, offset)
        ref = oracle.softmax_rows(x, "f32")
        assert ref.max() > 0.05  # the relative term decides
        for tier in tiers:
            y = to_host(rr.softmax_rows(to_gpu(x), torch.float32, tier))
            assert_close_f32(y, ref, "offset %g cols %d %s" % (offset, cols, tier))


def test_softmax_in_place():
    x = _softmax_input("bf16", 9, 3000, 41)
    ref = oracle.softmax_rows(x, "bf16")
    for tier in ("block", "splitk"):
        g = to_gpu(x)
        rr.softmax_rows(g, torch.bfloat16, tier, out=g)
        assert_bf16_within_1ulp(to_host(g), ref, "in place " + tier)


# split-K softmax: rows < CU with long rows, several workgroups per row
SPLITK_SOFTMAX_SHAPES = [(1, 65536), (3, 70001), (7, 100003), (2, 262144 + 8), (5, 131072 - 1)]


@pytest.mark.parametrize("rows,cols", SPLITK_SOFTMAX_SHAPES)
@pytest.mark.parametrize("xt,yt", SOFTMAX_TYPES)
def test_softmax_splitk_parity(rows, cols, xt, yt):
    x = _softmax_input(xt, rows, cols, 1700 + cols + rows)
    ref = oracle.softmax_rows(x, yt)
    ydt = torch.bfloat16 if yt == "bf16" else torch.float32
    xtd = torch.bfloat16 if xt == "bf16" else torch.float32
    plan = rr.plan_softmax(rows, cols, xtd, ydt, "splitk", rr.device_cu_count())
    assert plan["slices"] > 1
    assert rr.select_tier("softmax", rows, cols, xtd) == "splitk"
    for tier in ("auto", "splitk"):
        y = to_host(rr.softmax_rows(to_gpu(x), ydt, tier))
        _check_softmax(y, ref, yt, "splitk %dx%d %s->%s %s" % (rows, cols, xt, yt, tier))


@pytest.mark.parametrize("offset", [1, 3])
def test_softmax_splitk_misaligned_rows(offset):
    rows, cols = 3, 90001
    for xt in ("bf16", "f32"):
        x = _softmax_input(xt, rows, cols, 77 + offset)
        ref = oracle.softmax_rows(x, "f32")
        big = np.zeros((rows, cols + 8 + offset), dtype=x.dtype)
        big[:, offset:offset + cols] = x
        g = to_gpu(big)[:, offset:offset + cols]
        y = to_host(rr.softmax_rows(g, torch.float32, "splitk"))
        assert_close_f32(y, ref, "splitk misaligned %s off %d" % (xt, offset))


def test_softmax_splitk_wide_range_and_special_rows():
    rows, cols = 4, 80000
    x = synth.uniform_f32(33, (rows, cols), -120.0, 20.0)
    x[1, :] = -np.inf                      # whole row -inf: NaN, as in the definition
    x[2, ::7] = -np.inf                    # -inf entries give exact zeros
    x[3, 12345] = 200.0                    # one dominant entry in the middle slice
    for yt in ("f32", "bf16"):
        ref = oracle.softmax_rows(x, yt)
        ydt = torch.bfloat16 if yt == "bf16" else torch.float32
        y = to_host(rr.softmax_rows(to_gpu(x), ydt, "splitk"))
        _check_softmax(y, ref, yt, "splitk special " + yt)


def test_softmax_splitk_long_rows_bit_identical_across_runs():
    g = to_gpu(synth.normal_bf16(12, (16, 1 << 20)))
    assert rr.plan_softmax(16, 1 << 20, cu_count=rr.device_cu_count())["tier"] == "splitk"
    first = rr.softmax_rows(g).clone()
    for _ in range(4):
        assert torch.equal(rr.softmax_rows(g).view(torch.int16), first.view(torch.int16))
    # every row sums to 1 within the bf16 rounding of its outputs
    s = first.float().sum(dim=1)
    assert float((s - 1).abs().max()) <= 2.0 ** -8
    sample = np.array([0, 5, 15])
    ref = oracle.softmax_rows(np.ascontiguousarray(to_host(g)[sample]), "bf16")
    assert_bf16_within_1ulp(to_host(first)[sample], ref, "splitk 16 x 2^20 sample rows")


def test_softmax_and_reduce_splitk_interleaved_on_one_stream():
    xs = synth.normal_f32(14, (5, 100000))
    xr = synth.normal_f32(15, (7, 90000))
    gs, gr = to_gpu(xs), to_gpu(xr)
    for _ in range(3):
        ys = rr.softmax_rows(gs, torch.float32, "splitk")
        yr = rr.reduce_rows(gr, "sum", "splitk")
        assert_close_f32(to_host(ys), oracle.softmax_rows(xs, "f32"), "interleaved softmax")
        assert_close_f32(to_host(yr), oracle.reduce_rows(xr, "sum"), "interleaved reduce")


def test_softmax_splitk_workspace_needs_no_initial_contents():
    # the pairs are written before they are read: garbage in the workspace
    # must not change the result
    x = to_gpu(synth.normal_f32(10, (3, 200000)))
    first = rr.softmax_rows(x, torch.float32, "splitk").clone()
    torch.cuda.synchronize()
    for key, ws in rr._workspaces.items():
        if key[0] == "softmax":
            ws.fill_(0xA5)
    again = rr.softmax_rows(x, torch.float32, "splitk")
    assert torch.equal(again.view(torch.int32), first.view(torch.int32))


# --------------------------------------------------------------- LSE merge

def _merge_case(P, rows, depth, seed):
    o, m, l = synth.lse_merge(seed, P=P, batch=1, heads=1, q_rows=rows, depth=depth)
    return o.reshape(P, rows, depth), m.reshape(P, rows), l.reshape(P, rows)


def _run_merge(o, m, l, scale=1.0, out="bf16"):
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    y = rr.splitk_lse_merge(to_gpu(o), to_gpu(m), to_gpu(l), scale, odt)
    torch.cuda.synchronize()
    return to_host(y)


def _check_merge(o, m, l, scale, what):
    for out in ("bf16", "f32"):
        ref = oracle.splitk_lse_merge(o, m, l, scale, out)
        got = _run_merge(o, m, l, scale, out)
        if out == "bf16":
            assert_bf16_within_1ulp(got, ref, what + " bf16")
        else:
            assert_close_f32(got, ref, what + " f32")


@pytest.mark.parametrize("P", [1, 2, 3, 8, 9, 16, 64, 256])
@pytest.mark.parametrize("depth", [1, 3, 4, 64, 100, 128, 129, 300])
def test_merge_partition_counts_and_depths(P, depth):
    rows = 37
    o, m, l = _merge_case(P, rows, depth, P * 1000 + depth)
    _check_merge(o, m, l, 1.0, "P %d depth %d" % (P, depth))


def test_merge_single_partition_is_bit_exact_identity():
    o, m, l = _merge_case(1, 300, 128, 7)
    assert_exact(_run_merge(o, m, l, 1.0, "f32"), o[0], "P=1 f32")
    want = o[0].astype(np.float32)
    want_bits = torch.from_numpy(want).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert_exact(_run_merge(o, m, l, 1.0, "bf16"), want_bits, "P=1 bf16")


def test_merge_empty_partitions_and_rows():
    P, rows, depth = 8, 64, 128
    o, m, l = _merge_case(P, rows, depth, 11)
    rng = np.random.default_rng(12)
    empty = rng.random((P, rows)) < 0.3
    o[empty] = np.nan                       # poison: must never enter the sum
    l[empty & (rng.random((P, rows)) < 0.5)] = 0.0
    m[empty & (l != 0)] = -np.inf
    m[:, 5], l[:, 5] = -np.inf, 1.0         # row 5: every partition empty
    l[:, 9] = 0.0                           # row 9: every partition empty
    _check_merge(o, m, l, 1.0, "empties")
    got = _run_merge(o, m, l, 1.0, "f32")
    assert np.all(got[5] == 0) and np.all(got[9] == 0)


@pytest.mark.parametrize("scale", [0.0, 0.125, 1.0, 2.5])
def test_merge_scales(scale):
    o, m, l = _merge_case(8, 50, 128, 21)
    _check_merge(o, m, l, scale, "scale %g" % scale)


def test_merge_large_spread_of_maxima():
    o, m, l = _merge_case(4, 40, 64, 23)
    m[1] += 900.0   # exp(scale * (m_p - M)) underflows for every other partition
    _check_merge(o, m, l, 1.0, "spread")


def _bf16_ties(rng, n):
    """Float bit patterns of bf16 ties: a random normal bf16 value plus half a
    bf16 ulp (fraction bit 15 set, bits 0..14 clear), both signs."""
    h = rng.integers(0x3800, 0x4800, size=n).astype(np.uint32)  # |v| in [2^-15, 2^17)
    sign = rng.integers(0, 2, size=n).astype(np.uint32) << 31
    return sign | (h << 16) | 0x8000


def test_merge_bf16_rounds_once_near_ties():
    # P = 2 with equal statistics: c_0 = c_1 = 1/2 exactly, so the double sum
    # is (O_0 + O_1) / 2 with no error.  O_0 is a bf16 tie and O_1 the float
    # one step above or below it, so the sum lies half a float ulp off the
    # tie: rounded to float first it becomes the tie (float's nearest even)
    # and then rounds to the even bf16, the wrong way in half of the cases.
    # One rounding of the double, as the oracle does, must give the oracle's
    # bits exactly.
    rng = np.random.default_rng(404)
    rows, depth = 64, 128
    tie = _bf16_ties(rng, rows * depth)
    step = np.where(rng.random(rows * depth) < 0.5, 1, -1).astype(np.int64)
    o = np.empty((2, rows, depth), dtype=np.float32)
    o[0] = tie.view(np.float32).reshape(rows, depth)
    o[1] = (tie.astype(np.int64) + step).astype(np.uint32).view(np.float32).reshape(rows, depth)
    m = np.full((2, rows), 0.75, dtype=np.float32)
    l = np.full((2, rows), 3.0, dtype=np.float32)
    ref = oracle.splitk_lse_merge(o, m, l, 1.0, "bf16")
    # the case is live: rounding the exact mean to float first, then to bf16,
    # differs from the oracle's one rounding on many elements
    mean_f = ((o[0].astype(np.float64) + o[1]) / 2).astype(np.float32)
    twice = torch.from_numpy(mean_f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (twice != ref).sum() > rows * depth // 8
    assert_exact(_run_merge(o, m, l, 1.0, "bf16"), ref, "bf16 near ties")
    assert_exact(_run_merge(o, m, l, 1.0, "f32"), oracle.splitk_lse_merge(o, m, l, 1.0, "f32"),
                 "f32 near ties")
    # the same rows through the row-outer kernel (depth not one 128-bit chunk per lane)
    o3 = np.ascontiguousarray(o[:, :, :100])
    assert_exact(_run_merge(o3, m, l, 1.0, "bf16"), oracle.splitk_lse_merge(o3, m, l, 1.0, "bf16"),
                 "bf16 near ties, depth 100")


def test_merge_config_full_size():
    o, m, l = synth.lse_merge()
    P, depth = o.shape[0], o.shape[-1]
    g = rr.splitk_lse_merge(to_gpu(o), to_gpu(m), to_gpu(l), 1.0, torch.bfloat16)
    torch.cuda.synchronize()
    assert tuple(g.shape) == (8, 32, 128, 128)
    ref = oracle.splitk_lse_merge(o.reshape(P, -1, depth), m.reshape(P, -1), l.reshape(P, -1), 1.0,
                                  "bf16")
    assert_bf16_within_1ulp(to_host(g).reshape(-1, depth), ref, "lse_merge config")


def test_merge_bit_identical_across_runs():
    o, m, l = synth.lse_merge(P=8, batch=2, heads=8, q_rows=128, depth=128)
    go, gm, gl = to_gpu(o), to_gpu(m), to_gpu(l)
    first = rr.splitk_lse_merge(go, gm, gl).clone()
    for _ in range(4):
        assert torch.equal(rr.splitk_lse_merge(go, gm, gl).view(torch.int16), first.view(torch.int16))


# ------------------------------------------------------------- large sizes

def test_reduce_beyond_32bit_element_offsets():
    # The second row starts 2^30 + 3 elements (> 4 GiB) into the buffer, so any
    # 32-bit element or byte offset in a kernel would read the wrong data.
    rows, cols = 2, (1 << 30) + 3
    x = synth.ints_i32(77, (rows, cols), -1000, 1000)
    g = to_gpu(x)
    for op in ("sum", "max"):
        ref = oracle.reduce_rows(x, op)
        for tier in ("auto", "block"):
            assert_exact(to_host(rr.reduce_rows(g, op, tier)), ref, "large %s %s" % (op, tier))
    del g
    torch.cuda.empty_cache()


@pytest.mark.gpu
def test_rr_log_prints_plan(capfd, monkeypatch):
    """RR_LOG=1: each launching call writes its plan to stderr; unset, nothing."""
    x = torch.randn(64, 1024, device="cuda")
    monkeypatch.delenv("RR_LOG", raising=False)
    rr.reduce_rows(x, "sum")
    torch.cuda.synchronize()
    assert "rr:" not in capfd.readouterr().err
    monkeypatch.setenv("RR_LOG", "1")
    rr.reduce_rows(x, "sum")
    rr.softmax_rows(x.bfloat16())
    rr.reduce_axis(x.view(64, 8, 128), 1, "max")
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    plan = rr.plan_reduce(64, 1024, torch.float32, "sum", cu_count=rr.device_cu_count())
    assert ("rr: rr_reduce_rows rows=64 cols=1024 vec=1 tier=block block=%d grid=%d"
            % (plan["block"], plan["grid"])) in err, err
    assert "rr: rr_softmax_rows rows=64 cols=1024" in err, err
    assert "rr: rr_reduce_axis outer=64 axis=8 inner=128" in err, err


def test_host_outputs_are_refused_before_any_launch():
    x = torch.randn(64, 256, device="cuda")
    with pytest.raises(ValueError):
        rr.reduce_rows(x, "sum", out=torch.empty(64))
    with pytest.raises(ValueError):
        rr.reduce_rows_multi(x, out={"sum": torch.empty(64)})
    with pytest.raises(ValueError):
        rr.reduce_axis(x, 0, "sum", out=torch.empty(256))
    with pytest.raises(ValueError):
        rr.softmax_rows(x, out=torch.empty(64, 256))
    with pytest.raises(ValueError):
        rr.layernorm_rows(x, out=torch.empty(64, 256))
    with pytest.raises(ValueError):
        rr.layernorm_rows(x, torch.ones(256), torch.zeros(256, device="cuda"))
    with pytest.raises(ValueError):
        rr.layernorm_rows(x, mean_out=torch.empty(64))
    torch.cuda.synchronize()
