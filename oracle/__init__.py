"""CPU oracle for the deterministic row-reduce path -- TEST INFRASTRUCTURE.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this module.  The GPU library never does, and this module imports
nothing from it: the two share no code.

The arithmetic lives in ``rro.c`` (plain C, double precision, single thread);
this file only marshals numpy arrays through ctypes.  bf16 arrays are carried
as ``numpy.uint16`` bit patterns.

Sources: the Modular API pages "cluster_allreduce" (associative add/max/min
over 32-bit values, folded in ascending rank order), "reduce" from
algorithm.gpu.rowwise (the monoid fold along the last axis and the two-pass
softmax and layernorm) and "fa4_splitk_reduce_scatter_write" (the split-K (max, sum)
reweighting of partial outputs into bf16 rows, and the per-partition partial
outputs with their row max and row sum that it takes).  See rro.c for the
readings.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build_oracle

F32, I32, BF16 = 0, 1, 2
SUM, MAX, MIN = 0, 1, 2
_OPS = {"sum": SUM, "max": MAX, "min": MIN}
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build_oracle()
        lib = ctypes.CDLL(LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        lib.rro_reduce_rows.argtypes = [vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int]
        lib.rro_reduce_rows.restype = ctypes.c_int
        lib.rro_softmax_rows.argtypes = [vp, vp, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
        lib.rro_softmax_rows.restype = ctypes.c_int
        lib.rro_splitk_lse_merge.argtypes = [vp, vp, vp, vp, i32, i64, i32, ctypes.c_float,
                                             ctypes.c_int]
        lib.rro_splitk_lse_merge.restype = ctypes.c_int
        lib.rro_reduce_axis.argtypes = [vp, vp, i64, i64, i64, ctypes.c_int, ctypes.c_int]
        lib.rro_reduce_axis.restype = ctypes.c_int
        lib.rro_layernorm_rows.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_double]
        lib.rro_layernorm_rows.restype = ctypes.c_int
        lib.rro_attention_partials.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                               i32, i32, ctypes.c_float]
        lib.rro_attention_partials_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64,
                                                      i64, i64, i64, i32, i32, ctypes.c_float]
        lib.rro_attention_partials_varlen.restype = ctypes.c_int
        lib.rro_bf16_from_double.argtypes = [ctypes.c_double]
        lib.rro_bf16_from_double.restype = ctypes.c_uint16
        lib.rro_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.rro_bf16_to_double.restype = ctypes.c_double
        _lib = lib
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def _rows_view(x):
    """(rows, cols, ld) of a 2-D array whose last axis is contiguous."""
    if x.ndim != 2:
        raise ValueError("expected a 2-D array")
    rows, cols = x.shape
    es = x.itemsize
    if rows > 0 and cols > 1 and x.strides[1] != es:
        raise ValueError("last axis must be contiguous")
    ld = x.strides[0] // es if rows > 1 else cols
    if rows > 1 and x.strides[0] % es:
        raise ValueError("row stride must be a whole number of elements")
    return rows, cols, max(ld, cols)


def reduce_rows(x, op):
    """Row-wise sum/max/min over the last axis of a 2-D float32 or int32 array."""
    lib = _load()
    if x.dtype == np.float32:
        dt = F32
    elif x.dtype == np.int32:
        dt = I32
    else:
        raise TypeError("reduce_rows takes float32 or int32")
    rows, cols, ld = _rows_view(x)
    y = np.empty(rows, dtype=x.dtype)
    rc = lib.rro_reduce_rows(_ptr(x), _ptr(y), rows, cols, ld, dt, _OPS[op])
    if rc:
        raise ValueError("rro_reduce_rows rejected its arguments")
    return y


def reduce_axis(x, op):
    """Sum/max/min over the middle axis of a contiguous [outer, axis, inner]
    float32 or int32 array; returns [outer, inner]."""
    lib = _load()
    if x.dtype == np.float32:
        dt = F32
    elif x.dtype == np.int32:
        dt = I32
    else:
        raise TypeError("reduce_axis takes float32 or int32")
    if x.ndim != 3:
        raise ValueError("expected [outer, axis, inner]")
    x = np.ascontiguousarray(x)
    outer, axis, inner = x.shape
    y = np.empty((outer, inner), dtype=x.dtype)
    rc = lib.rro_reduce_axis(_ptr(x), _ptr(y), outer, axis, inner, dt, _OPS[op])
    if rc:
        raise ValueError("rro_reduce_axis rejected its arguments")
    return y


def softmax_rows(x, out_dtype="bf16", x_is_bf16=None):
    """Softmax over the last axis.  ``x``: float32, or uint16 bf16 bit patterns.

    Returns float32, or uint16 bf16 bit patterns when ``out_dtype == 'bf16'``.
    """
    lib = _load()
    if x.dtype == np.uint16:
        xd = BF16
    elif x.dtype == np.float32:
        xd = F32
    else:
        raise TypeError("softmax_rows takes float32 or bf16 (uint16 bits)")
    rows, cols, ld = _rows_view(x)
    if out_dtype == "bf16":
        y = np.empty((rows, cols), dtype=np.uint16)
        yd = BF16
    else:
        y = np.empty((rows, cols), dtype=np.float32)
        yd = F32
    rc = lib.rro_softmax_rows(_ptr(x), _ptr(y), rows, cols, ld, cols, xd, yd)
    if rc:
        raise ValueError("rro_softmax_rows rejected its arguments")
    return y


def _real_code(a, what):
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError("%s must be float32 or bf16 (uint16 bits)" % what)


def layernorm_rows(x, gamma=None, beta=None, eps=1e-5, out_dtype="bf16"):
    """Layer normalisation over the last axis (population variance).

    ``x``: float32 or uint16 bf16 bits, 2-D.  ``gamma`` / ``beta``: [cols] of
    one type (float32 or bf16 bits), or None for 1 / 0.  ``eps`` is taken as
    the float32 value the GPU path receives.  Returns (y, mean, rstd): y as
    float32 or uint16 bf16 bits, mean and rstd float32 [rows].
    """
    lib = _load()
    xd = _real_code(x, "x")
    rows, cols, ld = _rows_view(x)
    wd = F32
    ws = [w for w in (gamma, beta) if w is not None]
    if ws:
        wd = _real_code(ws[0], "gamma/beta")
        for w in ws:
            if _real_code(w, "gamma/beta") != wd or w.shape != (cols,):
                raise ValueError("gamma and beta must share one type and have shape [cols]")
    gamma = None if gamma is None else np.ascontiguousarray(gamma)
    beta = None if beta is None else np.ascontiguousarray(beta)
    if out_dtype == "bf16":
        y = np.empty((rows, cols), dtype=np.uint16)
        yd = BF16
    else:
        y = np.empty((rows, cols), dtype=np.float32)
        yd = F32
    mean = np.full(rows, np.nan, dtype=np.float32)
    rstd = np.full(rows, np.nan, dtype=np.float32)
    rc = lib.rro_layernorm_rows(_ptr(x), _ptr(y), None if gamma is None else _ptr(gamma),
                                None if beta is None else _ptr(beta), _ptr(mean), _ptr(rstd),
                                rows, cols, ld, cols, xd, yd, wd, float(np.float32(eps)))
    if rc:
        raise ValueError("rro_layernorm_rows rejected its arguments")
    return y, mean, rstd


def splitk_lse_merge(o, m, l, scale=1.0, out_dtype="bf16"):
    """LSE merge of P partitions.

    o: float32 [P, rows, depth]; m, l: float32 [P, rows].
    Returns [rows, depth] as float32, or uint16 bf16 bits for ``'bf16'``.
    """
    lib = _load()
    o = np.ascontiguousarray(o, dtype=np.float32)
    m = np.ascontiguousarray(m, dtype=np.float32)
    l = np.ascontiguousarray(l, dtype=np.float32)
    P, rows, depth = o.shape
    if m.shape != (P, rows) or l.shape != (P, rows):
        raise ValueError("m and l must be [P, rows]")
    if out_dtype == "bf16":
        out = np.empty((rows, depth), dtype=np.uint16)
        od = BF16
    else:
        out = np.empty((rows, depth), dtype=np.float32)
        od = F32
    rc = lib.rro_splitk_lse_merge(_ptr(o), _ptr(m), _ptr(l), _ptr(out), P, rows, depth,
                                  float(scale), od)
    if rc:
        raise ValueError("rro_splitk_lse_merge rejected its arguments")
    return out


def attention_partials(q, k, v, P, scale, kv_heads=None):
    """Split-K attention partials (m_p, l_p, normalised O_p) of every query row.

    q: bf16 bits (uint16) [batch, heads, q_rows, depth]; k, v: bf16 bits
    [batch, kv_heads, kv_len, depth].  Returns (o [P, batch*heads*q_rows, depth],
    m [P, rows], l [P, rows]) as float32 -- the layout the LSE merge takes.
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    batch, heads, q_rows, depth = q.shape
    kb, kvh, kv_len, kd = k.shape
    if kb != batch or kd != depth or v.shape != k.shape:
        raise ValueError("k and v must be [batch, kv_heads, kv_len, depth]")
    if kv_heads is not None and kv_heads != kvh:
        raise ValueError("kv_heads does not match k")
    rows = batch * heads * q_rows
    o = np.empty((P, rows, depth), dtype=np.float32)
    m = np.empty((P, rows), dtype=np.float32)
    l = np.empty((P, rows), dtype=np.float32)
    rc = lib.rro_attention_partials(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(m), _ptr(l), batch,
                                    heads, kvh, q_rows, kv_len, depth, P, float(scale))
    if rc:
        raise ValueError("rro_attention_partials rejected its arguments")
    return o, m, l


def attention_partials_varlen(q, k, v, cu_q, cu_k, P, scale):
    """Split-K attention partials of packed variable-length sequences.

    q: bf16 bits [total_q, heads, depth]; k, v: bf16 bits [total_k, kv_heads,
    depth]; cu_q, cu_k: int32 [batch + 1] token offsets of each sequence.
    Returns (o [P, total_q * heads, depth], m [P, total_q * heads],
    l [P, total_q * heads]) float32, partial row t * heads + h for token t and
    head h; rows of tokens that belong to no sequence are NaN (not written).
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    cu_q = np.ascontiguousarray(cu_q, dtype=np.int32)
    cu_k = np.ascontiguousarray(cu_k, dtype=np.int32)
    total_q, heads, depth = q.shape
    total_k, kvh, kd = k.shape
    if kd != depth or v.shape != k.shape or cu_q.shape != cu_k.shape or cu_q.ndim != 1:
        raise ValueError("q [total_q, heads, depth], k and v [total_k, kv_heads, depth], "
                         "cu_q and cu_k [batch + 1]")
    batch = cu_q.size - 1
    rows = total_q * heads
    o = np.full((P, rows, depth), np.nan, dtype=np.float32)
    m = np.full((P, rows), np.nan, dtype=np.float32)
    l = np.full((P, rows), np.nan, dtype=np.float32)
    rc = lib.rro_attention_partials_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_q), _ptr(cu_k),
                                           _ptr(o), _ptr(m), _ptr(l), batch, heads, kvh, total_q,
                                           total_k, depth, P, float(scale))
    if rc:
        raise ValueError("rro_attention_partials_varlen rejected its arguments")
    return o, m, l


def bf16_from_double(values):
    """Round each double to bf16 (nearest, ties to even); returns uint16 bits."""
    lib = _load()
    flat = np.asarray(values, dtype=np.float64).ravel()
    out = np.fromiter((lib.rro_bf16_from_double(float(v)) for v in flat), dtype=np.uint16,
                      count=flat.size)
    return out.reshape(np.shape(values))


def bf16_to_double(bits):
    """Value of each bf16 bit pattern as a double."""
    lib = _load()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    out = np.fromiter((lib.rro_bf16_to_double(int(b)) for b in flat), dtype=np.float64,
                      count=flat.size)
    return out.reshape(np.shape(bits))
