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

