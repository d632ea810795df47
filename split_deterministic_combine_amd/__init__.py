"""Deterministic row reductions on AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``librr.so`` (the C ABI in ``include/rr.h``).  This
module only marshals arguments -- shapes, strides, dtypes, device pointers and
the current stream -- and every step of the computation runs in the HIP
kernels of the library.  There is no CPU fallback: if the library is not built
the first call raises.

Operations (names as in the C ABI):
  reduce_rows        sum / max / min over the last axis (float32, int32)
  reduce_rows_noalloc
                     the same with the library's own split-K scratch (for
                     callers that cannot allocate; the output is passed in)
  reduce_rows_multi  sum, max and min over the last axis from one read
  reduce_axis        sum / max / min over a non-last axis
  softmax_rows       two-pass softmax over the last axis (bf16 / float32)
  layernorm_rows     two-pass layer normalisation over the last axis
  splitk_lse_merge   merge of P split-K partial attention outputs by their
                     per-row (max, sum) statistics
  splitk_attention_partials
                     the producer of those partials (attention over each of P
                     partitions of the keys, on the matrix cores)
  splitk_attention_partials_varlen
                     the same for sequences of different lengths packed token
                     after token, partials placed by (token, head)
  splitk_attention   both in one launch, the partials folded in partition
                     order by the last workgroup of each query tile
"""
import ctypes
import math
import os
import threading

import torch

__all__ = [
    "RRError", "reduce_rows", "reduce_rows_noalloc", "reduce_rows_multi", "reduce_axis", "plan_axis", "softmax_rows", "layernorm_rows", "splitk_lse_merge",
    "splitk_attention_partials", "splitk_attention_partials_varlen", "splitk_attention",
    "splitk_attention_workspace_bytes",
    "plan_reduce", "plan_softmax", "plan_layernorm", "select_tier", "workspace_bytes", "workspace_reset", "device_cu_count",
    "version", "lib_path", "TIERS", "OPS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librr.so")

RR_OK = 0
_DTYPES = {torch.float32: 0, torch.int32: 1, torch.bfloat16: 2}
OPS = {"sum": 0, "max": 1, "min": 2}
OP_SUM_MAX_MIN = 3  # the three statistics of reduce_rows_multi (planner queries)
TIERS = {"auto": 0, "wave": 1, "block": 2, "tiled": 3, "serial": 4, "splitk": 5}
TIER_NAMES = {v: k for k, v in TIERS.items()}
KIND_REDUCE, KIND_SOFTMAX, KIND_LAYERNORM = 0, 1, 2


class RRError(RuntimeError):
    """A librr call returned an error status."""

    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


class _Plan(ctypes.Structure):
    _fields_ = [
        ("tier", ctypes.c_int32), ("block", ctypes.c_int32), ("grid", ctypes.c_int64),
        ("lanes_per_row", ctypes.c_int32), ("slices", ctypes.c_int32),
        ("tile_cols", ctypes.c_int64), ("workspace_bytes", ctypes.c_uint64),
    ]


_lib = None
_lib_lock = threading.Lock()


def lib_path():
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                "librr.so is not built (%s); build it with "
                "`python -m split_deterministic_combine_amd.build`" % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i64, i32, st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
        lib.rr_reduce_rows.argtypes = [vp, vp, i64, i64, i64, st, st, st, vp, ctypes.c_size_t, vp]
        lib.rr_reduce_rows_noalloc.argtypes = [vp, vp, i64, i64, i64, st, st, st, vp]
        lib.rr_reduce_rows_multi.argtypes = [vp, vp, vp, vp, i64, i64, i64, st, st, vp,
                                             ctypes.c_size_t, vp]
        lib.rr_softmax_rows.argtypes = [vp, vp, i64, i64, i64, i64, st, st, st, vp,
                                        ctypes.c_size_t, vp]
        lib.rr_splitk_lse_merge.argtypes = [vp, vp, vp, vp, i32, i64, i32, ctypes.c_float, st, vp]
        lib.rr_splitk_attention_partials.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                                     i64, i32, i32, ctypes.c_float, vp]
        lib.rr_splitk_attention_partials_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64,
                                                            i64, i64, i64, i64, i64, i32, i32,
                                                            ctypes.c_float, vp]
        lib.rr_splitk_attention.argtypes = [vp, vp, vp, vp, st, i64, i64, i64, i64, i64, i32, i32,
                                            ctypes.c_float, vp, ctypes.c_size_t, vp]
        lib.rr_splitk_attention_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32, i32,
                                                            ctypes.POINTER(ctypes.c_size_t),
                                                            ctypes.POINTER(ctypes.c_size_t)]
        lib.rr_reduce_axis.argtypes = [vp, vp, i64, i64, i64, st, st, st, vp, ctypes.c_size_t, vp]
        lib.rr_plan_axis.argtypes = [i64, i64, i64, st, st, st, i32, ctypes.POINTER(_Plan)]
        lib.rr_layernorm_rows.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, st, st, st,
                                          ctypes.c_float, st, vp, ctypes.c_size_t, vp]
        lib.rr_plan_layernorm.argtypes = [i64, i64, st, st, st, st, i32, ctypes.POINTER(_Plan)]
        lib.rr_plan_reduce.argtypes = [i64, i64, i64, st, st, st, i32, ctypes.POINTER(_Plan)]
        lib.rr_plan_softmax.argtypes = [i64, i64, st, st, st, i32, ctypes.POINTER(_Plan)]
        lib.rr_workspace_bytes.argtypes = [st, i64, i64, st, st, st, ctypes.POINTER(ctypes.c_size_t)]
        lib.rr_select_tier.argtypes = [st, i64, i64, st, st, ctypes.POINTER(ctypes.c_int)]
        lib.rr_workspace_reset.argtypes = [vp, ctypes.c_size_t, vp]
        lib.rr_device_cu_count.argtypes = [ctypes.POINTER(ctypes.c_int32)]
        lib.rr_status_string.argtypes = [st]
        lib.rr_status_string.restype = ctypes.c_char_p
        lib.rr_version.restype = ctypes.c_int
        lib.rr_test_set_splitk_skew.argtypes = [i32]
        lib.rr_test_set_splitk_skew.restype = None
        lib.rr_test_stream.argtypes = [i32, vp, vp, ctypes.c_size_t, i32, vp]
        for name in ("rr_reduce_rows", "rr_reduce_rows_noalloc", "rr_reduce_rows_multi", "rr_reduce_axis", "rr_plan_axis",
                     "rr_softmax_rows", "rr_splitk_lse_merge", "rr_plan_reduce",
                     "rr_plan_softmax", "rr_layernorm_rows", "rr_plan_layernorm",
                     "rr_workspace_bytes", "rr_select_tier",
                     "rr_workspace_reset", "rr_device_cu_count", "rr_test_stream",
                     "rr_splitk_attention_partials", "rr_splitk_attention_partials_varlen",
                     "rr_splitk_attention",
                     "rr_splitk_attention_workspace_bytes"):
            getattr(lib, name).restype = st
        _lib = lib
    return _lib


def _check(status):
    if status != RR_OK:
        lib = _load()
        raise RRError(status, lib.rr_status_string(status).decode())


def version():
    return _load().rr_version()


def _stream_ptr(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class _OnDevice:
    """Make ``device`` current only when it is not already (the common case)."""

    __slots__ = ("dev", "prev")

    def __init__(self, device):
        self.dev = device.index
        self.prev = None

    def __enter__(self):
        cur = torch.cuda.current_device()
        if cur != self.dev:
            self.prev = cur
            torch.cuda.set_device(self.dev)

    def __exit__(self, *exc):
        if self.prev is not None:
            torch.cuda.set_device(self.prev)


def _as_rows(x, name="x"):
    """View ``x`` as [rows, cols] with a row stride; the last axis must be contiguous."""
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if x.dim() == 0:
        raise ValueError("%s must have at least one dimension" % name)
    cols = x.shape[-1]
    if x.dim() == 1:
        x2 = x.reshape(1, cols)
    else:
        x2 = x.reshape(-1, cols) if not (x.dim() == 2) else x
    if cols > 1 and x2.stride(1) != 1:
        raise ValueError("%s: the last axis must be contiguous" % name)
    rows = x2.shape[0]
    ld = x2.stride(0) if rows > 1 else cols
    return x2, rows, cols, max(ld, cols)


def _same_gpu(t, device, name):
    """Refuse a tensor the kernels cannot address: not on the GPU, or on
    another GPU than the call's inputs."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != device:
        raise ValueError("%s must be a GPU tensor on %s" % (name, device))


def _dtype_code(t):
    try:
        return _DTYPES[t]
    except KeyError:
        raise TypeError("unsupported dtype %s" % t) from None


_cu_counts = {}


def _cu_count(device):
    n = _cu_counts.get(device.index)
    if n is None:
        with _OnDevice(device):
            n = device_cu_count()
        _cu_counts[device.index] = n
    return n


_ws_need = {}


def _workspace_need(rows, cols, ld, dt, op, tier, cu):
    """Split-K workspace bytes of a reduction (host-only plan, cached)."""
    key = ("reduce", rows, cols, ld, dt, op, tier, cu)
    n = _ws_need.get(key)
    if n is None:
        plan = _Plan()
        _check(_load().rr_plan_reduce(rows, cols, ld, dt, op, tier, cu, ctypes.byref(plan)))
        n = _ws_need[key] = plan.workspace_bytes
    return n


def _softmax_workspace_need(rows, cols, xdt, ydt, tier, cu):
    """Split-K workspace bytes of a softmax (host-only plan, cached)."""
    key = ("softmax", rows, cols, xdt, ydt, tier, cu)
    n = _ws_need.get(key)
    if n is None:
        plan = _Plan()
        _check(_load().rr_plan_softmax(rows, cols, xdt, ydt, tier, cu, ctypes.byref(plan)))
        n = _ws_need[key] = plan.workspace_bytes
    return n


# split-K workspaces, one per (kind, device, stream).  A reduction's tickets
# reset themselves, so its workspace stays zero between calls on its stream;
# the softmax workspace holds only pairs that each call writes before reading;
# the fused attention's tickets reset themselves and its partials are
# rewritten by every call.
_workspaces = {}


def _workspace(kind, device, stream_id, nbytes):
    key = (kind, device.index, stream_id)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 4096), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def reduce_rows(x, op="sum", tier="auto", out=None):
    """Reduce every row of ``x`` over its last axis; returns shape ``x.shape[:-1]``.

    ``op`` is "sum", "max" or "min"; ``x`` is float32 or int32 on the GPU.
    ``tier`` is "auto" or one of "wave", "block", "tiled", "serial", "splitk".
    """
    lib = _lib or _load()
    x2, rows, cols, ld = _as_rows(x)
    dt = _dtype_code(x.dtype)
    if out is None:
        out = torch.empty(x.shape[:-1], dtype=x.dtype, device=x.device)
    _same_gpu(out, x.device, "out")
    if out.dtype != x.dtype or out.numel() != rows or not out.is_contiguous():
        raise ValueError("out must be a contiguous %s tensor of %d elements" % (x.dtype, rows))
    o, t = OPS[op], TIERS[tier]
    with _OnDevice(x.device):
        stream = _stream_ptr(x.device)
        need = _workspace_need(rows, cols, ld, dt, o, t, _cu_count(x.device))
        ws_ptr, ws_len = None, 0
        if need:
            ws = _workspace("reduce", x.device, stream.value, need)
            ws_ptr, ws_len = ctypes.c_void_p(ws.data_ptr()), ws.numel()
        _check(lib.rr_reduce_rows(ctypes.c_void_p(x2.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                  rows, cols, ld, dt, o, t, ws_ptr, ws_len, stream))
    return out


NOALLOC_SCRATCH_BYTES = 1 << 20  # RR_NOALLOC_SCRATCH_BYTES


def reduce_rows_noalloc(x, out, op="sum", tier="auto"):
    """``reduce_rows`` through ``rr_reduce_rows_noalloc``: no workspace and no
    allocation -- ``out`` (contiguous, ``rows`` elements of x's dtype, on x's
    GPU) must be passed in; the split-K tier uses the library's scratch array
    (RR_NOALLOC_SCRATCH_BYTES per GPU).  Calls that overlap in time on one GPU
    share that array and must not be made."""
    lib = _lib or _load()
    x2, rows, cols, ld = _as_rows(x)
    dt = _dtype_code(x.dtype)
    _same_gpu(out, x.device, "out")
    if out.dtype != x.dtype or out.numel() != rows or not out.is_contiguous():
        raise ValueError("out must be a contiguous %s tensor of %d elements" % (x.dtype, rows))
    with _OnDevice(x.device):
        _check(lib.rr_reduce_rows_noalloc(ctypes.c_void_p(x2.data_ptr()),
                                          ctypes.c_void_p(out.data_ptr()), rows, cols, ld, dt,
                                          OPS[op], TIERS[tier], _stream_ptr(x.device)))
    return out


def reduce_rows_multi(x, stats=("sum", "max", "min"), tier="auto", out=None):
    """Several row statistics of ``x`` over its last axis from one read.

    ``stats`` is any non-empty subset of ("sum", "max", "min"); returns a dict
    from each requested name to a tensor of shape ``x.shape[:-1]`` (``out``, a
    dict of such tensors, may supply them).  Each result equals, bit for bit,
    ``reduce_rows`` of that op on the same tier.
    """
    lib = _load()
    stats = tuple(stats)
    if not stats or any(k not in OPS for k in stats):
        raise ValueError("stats must be a non-empty subset of %s" % (tuple(OPS),))
    x2, rows, cols, ld = _as_rows(x)
    dt = _dtype_code(x.dtype)
    out = dict(out or {})
    ptrs = []
    for k in ("sum", "max", "min"):
        if k not in stats:
            ptrs.append(None)
            continue
        t = out.get(k)
        if t is None:
            t = out[k] = torch.empty(x.shape[:-1], dtype=x.dtype, device=x.device)
        _same_gpu(t, x.device, "out[%r]" % k)
        if t.dtype != x.dtype or t.numel() != rows or not t.is_contiguous():
            raise ValueError("out[%r] must be a contiguous %s tensor of %d elements" % (
                k, x.dtype, rows))
        ptrs.append(ctypes.c_void_p(t.data_ptr()))
    t = TIERS[tier]
    with _OnDevice(x.device):
        stream = _stream_ptr(x.device)
        need = _workspace_need(rows, cols, ld, dt, OP_SUM_MAX_MIN, t, _cu_count(x.device))
        ws_ptr, ws_len = None, 0
        if need:
            ws = _workspace("reduce", x.device, stream.value, need)
            ws_ptr, ws_len = ctypes.c_void_p(ws.data_ptr()), ws.numel()
        _check(lib.rr_reduce_rows_multi(ctypes.c_void_p(x2.data_ptr()), *ptrs, rows, cols, ld, dt,
                                        t, ws_ptr, ws_len, stream))
    return {k: out[k] for k in stats}


def reduce_axis(x, dim, op="sum", tier="auto", out=None):
    """Reduce a contiguous tensor ``x`` over dimension ``dim`` (any axis).

    The tensor is viewed as [outer, axis, inner] around ``dim``; the result
    has ``x``'s shape without ``dim``.  ``op`` is "sum", "max" or "min";
    ``tier`` is "auto", "tiled", "serial" or "splitk".
    """
    lib = _load()
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise ValueError("x must be a GPU tensor")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    dim = dim % x.dim()
    shape = tuple(x.shape)
    outer = 1
    for d in shape[:dim]:
        outer *= d
    inner = 1
    for d in shape[dim + 1:]:
        inner *= d
    axis = shape[dim]
    oshape = shape[:dim] + shape[dim + 1:]
    dt = _dtype_code(x.dtype)
    if out is None:
        out = torch.empty(oshape, dtype=x.dtype, device=x.device)
    _same_gpu(out, x.device, "out")
    if out.dtype != x.dtype or tuple(out.shape) != oshape or not out.is_contiguous():
        raise ValueError("out must be a contiguous %s tensor of shape %s" % (x.dtype, oshape))
    o, t = OPS[op], TIERS[tier]
    with _OnDevice(x.device):
        stream = _stream_ptr(x.device)
        key = ("axis", outer, axis, inner, dt, o, t, _cu_count(x.device))
        need = _ws_need.get(key)
        if need is None:
            plan = _Plan()
            _check(lib.rr_plan_axis(outer, axis, inner, dt, o, t, key[-1], ctypes.byref(plan)))
            need = _ws_need[key] = plan.workspace_bytes
        ws_ptr, ws_len = None, 0
        if need:
            ws = _workspace("axis", x.device, stream.value, need)
            ws_ptr, ws_len = ctypes.c_void_p(ws.data_ptr()), ws.numel()
        _check(lib.rr_reduce_axis(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                  outer, axis, inner, dt, o, t, ws_ptr, ws_len, stream))
    return out


def softmax_rows(x, out_dtype=None, tier="auto", out=None):
    """Softmax of every row of ``x`` over its last axis (x: bfloat16 or float32)."""
    lib = _lib or _load()
    x2, rows, cols, ld_x = _as_rows(x)
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype, device=x.device)
    _same_gpu(out, x.device, "out")
    if out.dtype != out_dtype or out.shape != x.shape:
        raise ValueError("out must be a %s tensor of shape %s" % (out_dtype, tuple(x.shape)))
    y2, _, _, ld_y = _as_rows(out, "out")
    xdt, ydt, t = _dtype_code(x.dtype), _dtype_code(out_dtype), TIERS[tier]
    with _OnDevice(x.device):
        stream = _stream_ptr(x.device)
        need = _softmax_workspace_need(rows, cols, xdt, ydt, t, _cu_count(x.device))
        ws_ptr, ws_len = None, 0
        if need:
            ws = _workspace("softmax", x.device, stream.value, need)
            ws_ptr, ws_len = ctypes.c_void_p(ws.data_ptr()), ws.numel()
        _check(lib.rr_softmax_rows(ctypes.c_void_p(x2.data_ptr()), ctypes.c_void_p(y2.data_ptr()),
                                   rows, cols, ld_x, ld_y, xdt, ydt, t, ws_ptr, ws_len, stream))
    return out


def _layernorm_workspace_need(rows, cols, xdt, ydt, wdt, tier, cu):
    """Split-K workspace bytes of a layernorm (host-only plan, cached)."""
    key = ("layernorm", rows, cols, xdt, ydt, wdt, tier, cu)
    n = _ws_need.get(key)
    if n is None:
        plan = _Plan()
        _check(_load().rr_plan_layernorm(rows, cols, xdt, ydt, wdt, tier, cu, ctypes.byref(plan)))
        n = _ws_need[key] = plan.workspace_bytes
    return n


def _vector_arg(t, n, dtypes, name, device):
    """Device pointer of an optional contiguous [n] tensor (None -> NULL)."""
    if t is None:
        return None
    _same_gpu(t, device, name)
    if t.dtype not in dtypes or t.numel() != n or not t.is_contiguous():
        raise ValueError("%s must be a contiguous tensor of %d elements of %s" % (
            name, n, " or ".join(str(d) for d in dtypes)))
    return ctypes.c_void_p(t.data_ptr())


def layernorm_rows(x, gamma=None, beta=None, eps=1e-5, out_dtype=None, tier="auto", out=None,
                   mean_out=None, rstd_out=None):
    """Layer normalisation of every row of ``x`` over its last axis.

    y = (x - mean) / sqrt(var + eps) * gamma + beta with the population
    variance; ``x`` is bfloat16 or float32, ``gamma`` / ``beta`` are [cols]
    (one dtype, float32 or bfloat16) or None.  ``mean_out`` / ``rstd_out``:
    optional float32 tensors of ``x.shape[:-1]`` elements that receive the
    row statistics.  Returns ``out``.
    """
    lib = _load()
    x2, rows, cols, ld_x = _as_rows(x)
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype, device=x.device)
    _same_gpu(out, x.device, "out")
    if out.dtype != out_dtype or out.shape != x.shape:
        raise ValueError("out must be a %s tensor of shape %s" % (out_dtype, tuple(x.shape)))
    y2, _, _, ld_y = _as_rows(out, "out")
    wts = [w for w in (gamma, beta) if w is not None]
    w_dtype = wts[0].dtype if wts else torch.float32
    if any(w.dtype != w_dtype for w in wts):
        raise ValueError("gamma and beta must have the same dtype")
    wdt = _dtype_code(w_dtype)
    g_ptr = _vector_arg(gamma, cols, (torch.float32, torch.bfloat16), "gamma", x.device)
    b_ptr = _vector_arg(beta, cols, (torch.float32, torch.bfloat16), "beta", x.device)
    m_ptr = _vector_arg(mean_out, rows, (torch.float32,), "mean_out", x.device)
    r_ptr = _vector_arg(rstd_out, rows, (torch.float32,), "rstd_out", x.device)
    xdt, ydt, t = _dtype_code(x.dtype), _dtype_code(out_dtype), TIERS[tier]
    with _OnDevice(x.device):
        stream = _stream_ptr(x.device)
        need = _layernorm_workspace_need(rows, cols, xdt, ydt, wdt, t, _cu_count(x.device))
        ws_ptr, ws_len = None, 0
        if need:
            ws = _workspace("layernorm", x.device, stream.value, need)
            ws_ptr, ws_len = ctypes.c_void_p(ws.data_ptr()), ws.numel()
        _check(lib.rr_layernorm_rows(ctypes.c_void_p(x2.data_ptr()), ctypes.c_void_p(y2.data_ptr()),
                                     g_ptr, b_ptr, m_ptr, r_ptr, rows, cols, ld_x, ld_y, xdt, ydt,
                                     wdt, float(eps), t, ws_ptr, ws_len, stream))
    return out


def splitk_lse_merge(o_part, m_part, l_part, scale=1.0, out_dtype=torch.bfloat16, out=None):
    """Merge P split-K partitions: o_part [P, *rows, depth], m_part / l_part [P, *rows].

    Returns [*rows, depth] in ``out_dtype`` (bfloat16 or float32).
    """
    lib = _load()
    for t, n in ((o_part, "o_part"), (m_part, "m_part"), (l_part, "l_part")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float32:
            raise ValueError("%s must be a float32 GPU tensor" % n)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % n)
    P, depth = o_part.shape[0], o_part.shape[-1]
    rows_shape = o_part.shape[1:-1]
    rows = 1
    for s in rows_shape:
        rows *= s
    if tuple(m_part.shape) != (P, *rows_shape) or tuple(l_part.shape) != (P, *rows_shape):
        raise ValueError("m_part and l_part must have shape %s" % ((P, *rows_shape),))
    for t, n in ((m_part, "m_part"), (l_part, "l_part")):
        _same_gpu(t, o_part.device, n)
    if out is None:
        out = torch.empty((*rows_shape, depth), dtype=out_dtype, device=o_part.device)
    _same_gpu(out, o_part.device, "out")
    if out.dtype != out_dtype or not out.is_contiguous() or out.numel() != rows * depth:
        raise ValueError("out must be a contiguous %s tensor of %d elements" % (out_dtype, rows * depth))
    with _OnDevice(o_part.device):
        _check(lib.rr_splitk_lse_merge(ctypes.c_void_p(o_part.data_ptr()),
                                       ctypes.c_void_p(m_part.data_ptr()),
                                       ctypes.c_void_p(l_part.data_ptr()),
                                       ctypes.c_void_p(out.data_ptr()), P, rows, depth,
                                       float(scale), _dtype_code(out_dtype),
                                       _stream_ptr(o_part.device)))
    return out


def splitk_attention_partials(q, k, v, P, scale=None, out=None):
    """Split-K attention partials: q bf16 [batch, heads, q_rows, depth], k and v
    bf16 [batch, kv_heads, kv_len, depth] (depth 64 or 128).

    Returns (o_part [P, batch*heads*q_rows, depth], m_part [P, rows],
    l_part [P, rows]) in float32 -- the inputs of splitk_lse_merge (scale 1.0).
    ``scale`` defaults to 1/sqrt(depth); ``out`` may give the three tensors.
    """
    lib = _load()
    batch, heads, kv_heads, q_rows, kv_len, depth = _attention_shapes(q, k, v)
    rows = batch * heads * q_rows
    if scale is None:
        scale = 1.0 / math.sqrt(depth)
    if out is None:
        out = (torch.empty((P, rows, depth), dtype=torch.float32, device=q.device),
               torch.empty((P, rows), dtype=torch.float32, device=q.device),
               torch.empty((P, rows), dtype=torch.float32, device=q.device))
    o, m, l = out
    for t, shape in ((o, (P, rows, depth)), (m, (P, rows)), (l, (P, rows))):
        _same_gpu(t, q.device, "out")
        if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != shape:
            raise ValueError("outputs must be contiguous float32 %s, %s, %s"
                             % ((P, rows, depth), (P, rows), (P, rows)))
    with _OnDevice(q.device):
        _check(lib.rr_splitk_attention_partials(
            ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
            ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(o.data_ptr()),
            ctypes.c_void_p(m.data_ptr()), ctypes.c_void_p(l.data_ptr()), batch, heads, kv_heads,
            q_rows, kv_len, depth, int(P), float(scale), _stream_ptr(q.device)))
    return o, m, l


def splitk_attention_partials_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_q_rows, P,
                                     scale=None, out=None):
    """Split-K attention partials of sequences packed token after token: q bf16
    [total_q, heads, depth], k and v bf16 [total_k, kv_heads, depth], and int32
    GPU offsets cu_seqlens_q, cu_seqlens_k [batch + 1] (sequence b owns tokens
    cu[b] .. cu[b+1] - 1 of each).  ``max_q_rows``: the query rows computed
    per sequence, normally the longest sequence's count (a sequence's rows
    past it are left unwritten; read by the host as given, the offsets stay
    on the device).

    Returns (o_part [P, total_q, heads, depth], m_part [P, total_q, heads],
    l_part [P, total_q, heads]) in float32; tokens outside every sequence are
    not written.  splitk_lse_merge takes them as rows = total_q * heads.
    """
    lib = _load()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.bfloat16:
            raise ValueError("%s must be a bfloat16 GPU tensor" % n)
        if not t.is_contiguous() or t.dim() != 3:
            raise ValueError("%s must be a contiguous 3-d tensor" % n)
    for t, n in ((k, "k"), (v, "v"), (cu_seqlens_q, "cu_seqlens_q"),
                 (cu_seqlens_k, "cu_seqlens_k")):
        _same_gpu(t, q.device, n)
    total_q, heads, depth = q.shape
    total_k, kv_heads, kd = k.shape
    if kd != depth or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [total_k, kv_heads, depth] matching q")
    for t, n in ((cu_seqlens_q, "cu_seqlens_q"), (cu_seqlens_k, "cu_seqlens_k")):
        if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous() or t.numel() < 1:
            raise ValueError("%s must be a contiguous 1-d int32 tensor of batch + 1 offsets" % n)
    batch = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != batch + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    if scale is None:
        scale = 1.0 / math.sqrt(depth)
    shapes = ((P, total_q, heads, depth), (P, total_q, heads), (P, total_q, heads))
    if out is None:
        out = tuple(torch.empty(sh, dtype=torch.float32, device=q.device) for sh in shapes)
    for t, shape in zip(out, shapes):
        _same_gpu(t, q.device, "out")
        if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != shape:
            raise ValueError("outputs must be contiguous float32 %s, %s, %s" % shapes)
    o, m, l = out
    with _OnDevice(q.device):
        _check(lib.rr_splitk_attention_partials_varlen(
            ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
            ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(cu_seqlens_q.data_ptr()),
            ctypes.c_void_p(cu_seqlens_k.data_ptr()), ctypes.c_void_p(o.data_ptr()),
            ctypes.c_void_p(m.data_ptr()), ctypes.c_void_p(l.data_ptr()), batch, heads, kv_heads,
            total_q, total_k, int(max_q_rows), depth, int(P), float(scale),
            _stream_ptr(q.device)))
    return o, m, l


def _attention_shapes(q, k, v):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.bfloat16:
            raise ValueError("%s must be a bfloat16 GPU tensor" % n)
        if not t.is_contiguous() or t.dim() != 4:
            raise ValueError("%s must be a contiguous 4-d tensor" % n)
    for t, n in ((k, "k"), (v, "v")):
        _same_gpu(t, q.device, n)
    batch, heads, q_rows, depth = q.shape
    kb, kv_heads, kv_len, kd = k.shape
    if kb != batch or kd != depth or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [batch, kv_heads, kv_len, depth] matching q")
    return batch, heads, kv_heads, q_rows, kv_len, depth


def splitk_attention_workspace_bytes(batch, heads, kv_heads, q_rows, kv_len, depth, P,
                                     with_tickets=False):
    """Bytes of workspace splitk_attention needs (host only); with
    ``with_tickets``, also how many of its first bytes must be zero when a
    call starts (the tickets)."""
    n, t = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(_load().rr_splitk_attention_workspace_bytes(batch, heads, kv_heads, q_rows, kv_len,
                                                       depth, int(P), ctypes.byref(n),
                                                       ctypes.byref(t)))
    return (n.value, t.value) if with_tickets else n.value


# The cached one-launch attention workspaces, per (device, stream): the
# tensor and how many of its first bytes are known to be zero.  A completed
# call leaves its ticket bytes zero and its partials after them, so before a
# call whose ticket region is larger, the bytes in between are cleared.
_attn_ws = {}


def _attention_workspace(device, stream, need, tickets):
    key = (device.index, stream.value)
    ent = _attn_ws.get(key)
    if ent is None or ent[0].numel() < need:
        ws = torch.zeros(max(need, 4096), dtype=torch.uint8, device=device)
        ent = _attn_ws[key] = [ws, ws.numel()]
    ws, zero = ent
    if tickets > zero:
        _check(_load().rr_workspace_reset(ctypes.c_void_p(ws.data_ptr() + zero), tickets - zero,
                                          stream))
    ent[1] = tickets        # after this call: tickets zero, partials after them
    return ws


def splitk_attention(q, k, v, P, scale=None, out_dtype=torch.bfloat16, out=None, workspace=None):
    """Split-K attention in one launch: softmax(scale q k^T) v computed over P
    partitions of the keys and combined in partition order (1 <= P <= depth/8).

    Shapes as splitk_attention_partials; returns [batch, heads, q_rows, depth]
    in ``out_dtype`` (bfloat16 or float32), bit-identical to
    ``splitk_lse_merge(*splitk_attention_partials(q, k, v, P, scale), 1.0,
    out_dtype)``.  ``workspace`` (uint8) defaults to one cached per device and
    stream; a caller's own must hold zeros in its first ticket bytes
    (``splitk_attention_workspace_bytes(..., with_tickets=True)``) when the
    call starts, which every completed call leaves so.
    """
    lib = _load()
    batch, heads, kv_heads, q_rows, kv_len, depth = _attention_shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(depth)
    if out is None:
        out = torch.empty((batch, heads, q_rows, depth), dtype=out_dtype, device=q.device)
    _same_gpu(out, q.device, "out")
    if out.dtype != out_dtype or not out.is_contiguous() or out.numel() != batch * heads * q_rows * depth:
        raise ValueError("out must be a contiguous %s tensor of %d elements"
                         % (out_dtype, batch * heads * q_rows * depth))
    need, tickets = splitk_attention_workspace_bytes(batch, heads, kv_heads, q_rows, kv_len,
                                                     depth, P, with_tickets=True)
    with _OnDevice(q.device):
        stream = _stream_ptr(q.device)
        if workspace is None:
            ws = _attention_workspace(q.device, stream, need, tickets) if need else None
        else:
            _same_gpu(workspace, q.device, "workspace")
            if not workspace.is_contiguous():
                raise ValueError("workspace must be contiguous")
            ws = workspace
        ws_ptr = ctypes.c_void_p(ws.data_ptr()) if ws is not None else None
        ws_len = ws.numel() * ws.element_size() if ws is not None else 0
        _check(lib.rr_splitk_attention(
            ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
            ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(out.data_ptr()),
            _dtype_code(out_dtype), batch, heads, kv_heads, q_rows, kv_len, depth, int(P),
            float(scale), ws_ptr, ws_len, stream))
    return out


def _plan_dict(plan):
    return {"tier": TIER_NAMES[plan.tier], "block": plan.block, "grid": plan.grid,
            "lanes_per_row": plan.lanes_per_row, "slices": plan.slices,
            "tile_cols": plan.tile_cols, "workspace_bytes": plan.workspace_bytes}


def plan_reduce(rows, cols, dtype=torch.float32, op="sum", tier="auto", cu_count=256, ld=None):
    """Host-only launch plan of rr_reduce_rows (op "sum_max_min": of
    rr_reduce_rows_multi); needs no GPU."""
    lib = _load()
    plan = _Plan()
    code = OP_SUM_MAX_MIN if op == "sum_max_min" else OPS[op]
    _check(lib.rr_plan_reduce(rows, cols, cols if ld is None else ld, _dtype_code(dtype), code,
                              TIERS[tier], cu_count, ctypes.byref(plan)))
    return _plan_dict(plan)


def plan_softmax(rows, cols, x_dtype=torch.bfloat16, y_dtype=None, tier="auto", cu_count=256):
    """Host-only launch plan of rr_softmax_rows (needs no GPU)."""
    lib = _load()
    plan = _Plan()
    y_dtype = x_dtype if y_dtype is None else y_dtype
    _check(lib.rr_plan_softmax(rows, cols, _dtype_code(x_dtype), _dtype_code(y_dtype),
                               TIERS[tier], cu_count, ctypes.byref(plan)))
    return _plan_dict(plan)


def plan_axis(outer, axis, inner, dtype=torch.float32, op="sum", tier="auto", cu_count=256):
    """Host-only launch plan of rr_reduce_axis (needs no GPU)."""
    lib = _load()
    plan = _Plan()
    _check(lib.rr_plan_axis(outer, axis, inner, _dtype_code(dtype), OPS[op], TIERS[tier],
                            cu_count, ctypes.byref(plan)))
    return _plan_dict(plan)


def plan_layernorm(rows, cols, x_dtype=torch.bfloat16, y_dtype=None, w_dtype=torch.float32,
                   tier="auto", cu_count=256):
    """Host-only launch plan of rr_layernorm_rows (needs no GPU)."""
    lib = _load()
    plan = _Plan()
    y_dtype = x_dtype if y_dtype is None else y_dtype
    _check(lib.rr_plan_layernorm(rows, cols, _dtype_code(x_dtype), _dtype_code(y_dtype),
                                 _dtype_code(w_dtype), TIERS[tier], cu_count, ctypes.byref(plan)))
    return _plan_dict(plan)


def select_tier(kind, rows, cols, dtype=torch.float32, op="sum"):
    """Tier AUTO picks on the current device; kind is "reduce" or "softmax"."""
    lib = _load()
    t = ctypes.c_int(0)
    k = {"reduce": KIND_REDUCE, "softmax": KIND_SOFTMAX, "layernorm": KIND_LAYERNORM}[kind]
    _check(lib.rr_select_tier(k, rows, cols, _dtype_code(dtype), OPS[op], ctypes.byref(t)))
    return TIER_NAMES[t.value]


def workspace_bytes(rows, cols, dtype=torch.float32, op="sum", tier="auto"):
    lib = _load()
    n = ctypes.c_size_t(0)
    _check(lib.rr_workspace_bytes(KIND_REDUCE, rows, cols, _dtype_code(dtype), OPS[op],
                                  TIERS[tier], ctypes.byref(n)))
    return n.value


def workspace_reset(ws):
    """Zero a workspace tensor on the current stream (fill kernel, no memset)."""
    lib = _load()
    with _OnDevice(ws.device):
        _check(lib.rr_workspace_reset(ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(),
                                      _stream_ptr(ws.device)))


def device_cu_count():
    lib = _load()
    cu = ctypes.c_int32(0)
    _check(lib.rr_device_cu_count(ctypes.byref(cu)))
    return cu.value


def _set_splitk_skew(sleeps_per_rank):
    """Test hook: arrival-order skew for the split-K tier (0 turns it off)."""
    _load().rr_test_set_splitk_skew(int(sleeps_per_rank))


_STREAM_MODES = {"read": 0, "write": 1, "copy": 2}


def _test_stream(mode, x=None, y=None, blocks_per_cu=0):
    """Test hook: a reference stream of known size ("read" x, "write" y, or
    "copy" x to y), the achievable-bandwidth reference for the rooflines.
    Asynchronous on the current stream."""
    t = x if x is not None else y
    if t is None or not t.is_cuda:
        raise RuntimeError("rr._test_stream needs CUDA tensors")
    for a in (x, y):
        if a is not None and not a.is_contiguous():
            raise RuntimeError("rr._test_stream needs contiguous tensors")
    nbytes = (x if mode != "write" else y).numel() * (x if mode != "write" else y).element_size()
    if mode == "copy" and y.numel() * y.element_size() < nbytes:
        raise RuntimeError("rr._test_stream: y is smaller than x")
    _check(_load().rr_test_stream(_STREAM_MODES[mode], None if x is None else x.data_ptr(),
                                  None if y is None else y.data_ptr(), nbytes, int(blocks_per_cu),
                                  _stream_ptr(t.device)))
