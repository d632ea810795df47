"""Element offsets beyond 2^31 (byte offsets beyond 4 GiB) on every path
other than the row reduction (covered in test_parity_gpu.py).

Inputs are drawn on the device from a seeded generator (the data is too
large to draw on the host quickly); the oracle checks sampled rows copied
back to the host, so both sides see the same bytes.  Any 32-bit element or
byte offset in a kernel would read or write the wrong place for the rows
past the 2^31st element.
"""
import numpy as np
import pytest
import torch

import oracle
import split_deterministic_combine_amd as rr
from tests.gpu_util import (assert_bf16_within_1ulp,
                            assert_close_f32, to_host)

pytestmark = pytest.mark.gpu


def _randn(shape, seed, scale=1.0, dtype=torch.float32):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    x = torch.randn(shape, generator=gen, device="cuda")
    if scale != 1.0:
        x.mul_(scale)
    return x.to(dtype)


ROWS, COLS = 2100, 1 << 20   # rows past 2048 start beyond element 2^31
SAMPLE = np.array([0, 1, 2047, 2048, 2049, 2099])


def test_softmax_and_layernorm_rows_beyond_2_pow_31_elements():
    x = _randn((ROWS, COLS), 90, 3.0, torch.bfloat16)
    xs = to_host(x[SAMPLE])
    y = rr.softmax_rows(x)
    torch.cuda.synchronize()
    assert_bf16_within_1ulp(to_host(y[SAMPLE]), oracle.softmax_rows(xs, "bf16"), "large softmax")
    del y
    y = rr.layernorm_rows(x, eps=1e-5)
    torch.cuda.synchronize()
    ref, _, _ = oracle.layernorm_rows(xs, None, None, 1e-5, "bf16")
    assert_bf16_within_1ulp(to_host(y[SAMPLE]), ref, "large layernorm")
    del x, y
    torch.cuda.empty_cache()


def test_merge_beyond_2_pow_31_elements():
    P, rows, depth = 8, 1 << 22, 128          # partition 7 starts at element 7 * 2^29
    o = _randn((P, rows, depth), 91)
    m = _randn((P, rows), 92, 4.0)
    l = _randn((P, rows), 93).abs_().mul_(1000).add_(1)
    out = rr.splitk_lse_merge(o, m, l, 1.0, torch.bfloat16)
    torch.cuda.synchronize()
    pick = np.array([0, 1, rows // 2, rows - 2, rows - 1])
    idx = torch.from_numpy(pick).cuda()
    oh = np.ascontiguousarray(to_host(o[:, idx, :]))
    mh = np.ascontiguousarray(to_host(m[:, idx]))
    lh = np.ascontiguousarray(to_host(l[:, idx]))
    ref = oracle.splitk_lse_merge(oh, mh, lh, 1.0, "bf16")
    assert_bf16_within_1ulp(to_host(out.reshape(rows, depth)[idx]), ref, "large merge")
    del o, m, l, out
    torch.cuda.empty_cache()


def test_axis_reduction_beyond_2_pow_31_elements():
    outer, axis, inner = 2, (1 << 15) + 1, 1 << 15   # outer index 1 starts past 2^30 elements
    x = _randn((outer, axis, inner), 94)             # 2^31 + 2^16 elements in all
    cols = np.array([0, 1, 777, inner - 1])
    xs = np.ascontiguousarray(to_host(x[:, :, torch.from_numpy(cols).cuda()]))
    ref = oracle.reduce_axis(xs, "sum")
    for tier in ("auto", "tiled", "splitk"):
        y = rr.reduce_axis(x, 1, "sum", tier)
        torch.cuda.synchronize()
        assert_close_f32(to_host(y)[:, cols], ref, "large axis " + tier)
    del x
    torch.cuda.empty_cache()
