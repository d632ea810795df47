"""Seeded synthetic inputs for the row-reduce workloads.

This module only draws random numbers; it holds none of the arithmetic of
the reductions, the softmax or the merge, and imports nothing else from this
package.  The tests, the benchmark and the oracle checks all take their
inputs from here, so the GPU path and the CPU oracle see identical bytes.

Every generator uses ``numpy.random.default_rng(seed)`` and draws in the
order written.  bf16 inputs are returned as ``numpy.uint16`` bit patterns,
made by torch's float32 -> bfloat16 cast (round to nearest even).

Workloads (sizes are the defaults; smaller sizes keep the distributions):
  small_rows   f32 uniform(-1, 1) and int32 uniform in [-1000, 1000], [64, 1024]
  short_rows   f32 standard normal, [1048576, 48]
  softmax_rows bf16 of 3 * standard normal, [8192, 8192]
  long_rows    f32 uniform(-1, 1) and int32 uniform in [-2^30, 2^30], [16, 2^24]
  lse_merge    P = 8 partitions of O [8, 32, 128, 128] standard normal,
               m = 4 * standard normal, l = uniform(1, 4096), scale 1.0
  softmax_long_rows  bf16 of 3 * standard normal, [16, 2^22] (split-K softmax)
  layernorm_rows     bf16 of 0.5 + 2 * standard normal, [16384, 4096], with
                     float32 gamma = 1 + 0.1 * standard normal and
                     beta = 0.1 * standard normal over the columns
  attention    bf16 of standard normal q [8, 32, 128, 128], k and v
               [8, 32, 8192, 128] (the producer of the LSE merge's partials)
"""
import numpy as np

SEED_SMALL_ROWS = 1
SEED_SHORT_ROWS = 2
SEED_SOFTMAX_ROWS = 3
SEED_LONG_ROWS = 4
SEED_LSE_MERGE = 5
SEED_SOFTMAX_LONG_ROWS = 6
SEED_LAYERNORM_ROWS = 7
SEED_ATTENTION = 8


def _bf16_bits(x_f32):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def small_rows(seed=SEED_SMALL_ROWS, rows=64, cols=1024):
    """f32 uniform(-1, 1) [rows, cols], then int32 uniform in [-1000, 1000]."""
    rng = np.random.default_rng(seed)
    xf = rng.uniform(-1.0, 1.0, (rows, cols)).astype(np.float32)
    xi = rng.integers(-1000, 1000, (rows, cols), endpoint=True, dtype=np.int32)
    return xf, xi


def short_rows(seed=SEED_SHORT_ROWS, rows=1048576, cols=48):
    """f32 standard normal [rows, cols]."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((rows, cols), dtype=np.float32)


def softmax_rows(seed=SEED_SOFTMAX_ROWS, rows=8192, cols=8192, std=3.0):
    """bf16 bits of std * standard normal [rows, cols]."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    x *= np.float32(std)
    return _bf16_bits(x)


def long_rows(seed=SEED_LONG_ROWS, rows=16, cols=1 << 24):
    """f32 uniform(-1, 1) [rows, cols], then int32 uniform in [-2^30, 2^30]."""
    rng = np.random.default_rng(seed)
    xf = rng.random((rows, cols), dtype=np.float32)
    xf *= np.float32(2.0)
    xf -= np.float32(1.0)
    xi = rng.integers(-(2 ** 30), 2 ** 30, (rows, cols), endpoint=True, dtype=np.int32)
    return xf, xi


def softmax_long_rows(seed=SEED_SOFTMAX_LONG_ROWS, rows=16, cols=1 << 22, std=3.0):
    """Few very long softmax rows (fewer rows than compute units)."""
    return normal_bf16(seed, (rows, cols), std)


def layernorm_rows(seed=SEED_LAYERNORM_ROWS, rows=16384, cols=4096):
    """(x bf16 bits [rows, cols], gamma f32 [cols], beta f32 [cols])."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    x *= np.float32(2.0)
    x += np.float32(0.5)
    gamma = np.float32(1.0) + np.float32(0.1) * rng.standard_normal(cols, dtype=np.float32)
    beta = np.float32(0.1) * rng.standard_normal(cols, dtype=np.float32)
    return _bf16_bits(x), gamma.astype(np.float32), beta.astype(np.float32)


def lse_merge(seed=SEED_LSE_MERGE, P=8, batch=8, heads=32, q_rows=128, depth=128):
    """Partial outputs O [P, batch, heads, q_rows, depth], m and l [P, batch, heads, q_rows].

    O ~ standard normal, m ~ 4 * standard normal, l ~ uniform(1, 4096).
    """
    rng = np.random.default_rng(seed)
    o = rng.standard_normal((P, batch, heads, q_rows, depth), dtype=np.float32)
    m = rng.standard_normal((P, batch, heads, q_rows), dtype=np.float32)
    m *= np.float32(4.0)
    l = rng.uniform(1.0, 4096.0, (P, batch, heads, q_rows)).astype(np.float32)
    return o, m, l


def uniform_f32(seed, shape, lo=-1.0, hi=1.0):
    rng = np.random.default_rng(seed)
    return rng.uniform(lo, hi, shape).astype(np.float32)


def normal_f32(seed, shape, std=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    x *= np.float32(std)
    return x


def ints_i32(seed, shape, lo, hi):
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi, shape, endpoint=True, dtype=np.int32)


def normal_bf16(seed, shape, std=3.0):
    return _bf16_bits(normal_f32(seed, shape, std))


def attention(seed=SEED_ATTENTION, batch=8, heads=32, kv_heads=32, q_rows=128, kv_len=8192,
              depth=128):
    """bf16 bits of standard normal q [batch, heads, q_rows, depth], then k and
    v [batch, kv_heads, kv_len, depth]."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((batch, heads, q_rows, depth), dtype=np.float32)
    k = rng.standard_normal((batch, kv_heads, kv_len, depth), dtype=np.float32)
    v = rng.standard_normal((batch, kv_heads, kv_len, depth), dtype=np.float32)
    return _bf16_bits(q), _bf16_bits(k), _bf16_bits(v)


def attention_varlen(seed, q_lens, k_lens, heads, kv_heads, depth, q_lead=0, k_lead=0):
    """Packed variable-length sequences: bf16 bits of standard normal
    q [total_q, heads, depth], then k and v [total_k, kv_heads, depth], and the
    int32 token offsets cu_q, cu_k [batch + 1] of sequences of q_lens[b]
    queries and k_lens[b] keys, laid out one after another from token q_lead
    (k_lead) on; the lead tokens belong to no sequence."""
    q_lens = np.asarray(q_lens, dtype=np.int64)
    k_lens = np.asarray(k_lens, dtype=np.int64)
    cu_q = (q_lead + np.concatenate([[0], np.cumsum(q_lens)])).astype(np.int32)
    cu_k = (k_lead + np.concatenate([[0], np.cumsum(k_lens)])).astype(np.int32)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((int(cu_q[-1]), heads, depth), dtype=np.float32)
    k = rng.standard_normal((int(cu_k[-1]), kv_heads, depth), dtype=np.float32)
    v = rng.standard_normal((int(cu_k[-1]), kv_heads, depth), dtype=np.float32)
    return _bf16_bits(q), _bf16_bits(k), _bf16_bits(v), cu_q, cu_k
