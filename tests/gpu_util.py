"""Comparison helpers for the GPU parity tests (HIP path vs the CPU oracle)."""
import numpy as np
import torch

from tests.exact import bf16_ulp_diff

# float32 results: |gpu - oracle| <= ABS + REL * |oracle|
REL, ABS = 1e-5, 1e-6


def to_gpu(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def assert_exact(gpu, ref, what=""):
    g, r = np.asarray(gpu), np.asarray(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    bad = g.view(np.uint32 if g.itemsize == 4 else np.uint16) != r.view(
        np.uint32 if r.itemsize == 4 else np.uint16)
    if bad.any():
        i = np.flatnonzero(bad.ravel())[:5]
        raise AssertionError("%s: %d of %d differ bitwise; first at %s: gpu %s oracle %s" % (
            what, bad.sum(), bad.size, i, g.ravel()[i], r.ravel()[i]))


def assert_close_f32(gpu, ref, what="", rel=REL, abs_=ABS):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    both_nan = np.isnan(g) & np.isnan(r)
    same_inf = np.isinf(g) & (g == r)
    err = np.abs(g - r)
    ok = (err <= abs_ + rel * np.abs(r)) | both_nan | same_inf
    if not ok.all():
        i = np.flatnonzero(~ok.ravel())[:5]
        raise AssertionError("%s: %d of %d outside rel %g / abs %g; first at %s: gpu %s oracle %s" % (
            what, (~ok).sum(), ok.size, rel, abs_, i, g.ravel()[i], r.ravel()[i]))


def _bf16_nan(b):
    b = np.asarray(b, dtype=np.uint16)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


def assert_bf16_within_1ulp(gpu, ref, what=""):
    g, r = np.asarray(gpu, dtype=np.uint16), np.asarray(ref, dtype=np.uint16)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    gn, rn = _bf16_nan(g), _bf16_nan(r)
    d = bf16_ulp_diff(g, r)
    ok = (d <= 1) & ~gn & ~rn | (gn & rn)
    if not ok.all():
        i = np.flatnonzero(~ok.ravel())[:5]
        raise AssertionError("%s: %d of %d more than 1 bf16 ulp apart; first at %s: gpu %s oracle %s" % (
            what, (~ok).sum(), ok.size, i, [hex(v) for v in g.ravel()[i]],
            [hex(v) for v in r.ravel()[i]]))
    return int((d > 0).sum())


def assert_bf16_within_1ulp_or_abs(gpu, ref, what="", abs_=ABS):
    """bf16 results within 1 ulp of the oracle, or within `abs_` of it in value.

    For outputs formed by cancellation in float arithmetic (a layernorm's
    gamma * d * rstd + beta near zero), float's error is absolute, about
    1e-7 of the terms, and can be several bf16 ulps of a tiny result; the
    absolute floor is the float32 bar's.
    """
    g, r = np.asarray(gpu, dtype=np.uint16), np.asarray(ref, dtype=np.uint16)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    gn, rn = _bf16_nan(g), _bf16_nan(r)
    d = bf16_ulp_diff(g, r)
    gv = (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rv = (r.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    with np.errstate(invalid="ignore"):
        near = np.abs(gv - rv) <= abs_
    ok = ((d <= 1) | near) & ~gn & ~rn | (gn & rn)
    if not ok.all():
        i = np.flatnonzero(~ok.ravel())[:5]
        raise AssertionError("%s: %d of %d beyond 1 bf16 ulp and abs %g; first at %s: gpu %s oracle %s" % (
            what, (~ok).sum(), ok.size, abs_, i, [hex(v) for v in g.ravel()[i]],
            [hex(v) for v in r.ravel()[i]]))
