"""GPU parity of the split-K attention partials (rr_splitk_attention_partials)
against the CPU oracle, and of the whole split-K attention (partials, then the
LSE merge) against softmax attention.

Tolerance, from the arithmetic of the kernel (the oracle is exact in double):
  * scores: q . k of bf16 values accumulates in float32 over `depth` products,
    so |ds_j| <= B_s = scale * depth * 2^-24 * max_j sum_d |q_d k_jd| + 2^-24 |m|;
    the row max moves by at most B_s;
  * l = sum exp(s_j - m): each term moves by a relative 2 B_s, the float32
    sum over the partition's n keys adds n 2^-24, the exponential 2^-22;
  * O = sum_j w_j v_j with w_j = exp(s_j - m) / l: the probabilities enter
    the second product rounded to bf16 (relative 2^-8), plus 2 B_s from the
    scores and 2^-13 for the float32 accumulation and the rescaling, so
    |dO_d| <= (2^-8 + 2^-13 + 2 B_s) * sum_j w_j |v_jd| + 1e-6, where the
    weighted sum of |v| is the oracle's own output for |v|.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import split_deterministic_combine_amd as rr
from split_deterministic_combine_amd import synth
from tests.gpu_util import assert_bf16_within_1ulp, to_host

pytestmark = pytest.mark.gpu


def _bf16_tensor(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _bf16_double(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _score_bound(q, k, scale):
    """B_s per query row: scale * depth * 2^-24 * max_j sum_d |q_d k_jd|."""
    qd, kd = np.abs(_bf16_double(q)), np.abs(_bf16_double(k))
    group = qd.shape[1] // kd.shape[1]
    kd = np.repeat(kd, group, axis=1)
    worst = np.matmul(qd, np.swapaxes(kd, -1, -2)).max(-1) if kd.shape[2] else np.zeros(qd.shape[:3])
    return (abs(scale) * qd.shape[-1] * 2.0 ** -24 * worst).reshape(-1)


def _check_partials(q, k, v, P, scale, what):
    o_g, m_g, l_g = rr.splitk_attention_partials(_bf16_tensor(q), _bf16_tensor(k), _bf16_tensor(v),
                                                 P, scale)
    torch.cuda.synchronize()
    o_g, m_g, l_g = to_host(o_g), to_host(m_g), to_host(l_g)
    o_r, m_r, l_r = oracle.attention_partials(q, k, v, P, scale)
    o_abs, _, _ = oracle.attention_partials(q, k, v & np.uint16(0x7FFF), P, scale)
    kv_len = k.shape[2]
    bs = _score_bound(q, k, scale)[None, :] + 2.0 ** -24 * np.abs(np.where(np.isfinite(m_r), m_r, 0))
    empty = ~np.isfinite(m_r)
    # empty partitions: exactly (-inf, 0, 0)
    assert np.all(m_g[empty] == -np.inf) and np.all(l_g[empty] == 0), what
    assert np.all(o_g[empty] == 0), what
    live = ~empty
    dm = np.abs(m_g[live] - m_r[live])
    assert np.all(dm <= bs[live]), (what, "m", np.max(dm))
    n_keys = -(-kv_len // P)
    tol_l = 2 * bs + n_keys * 2.0 ** -24 + 2.0 ** -22
    rel_l = np.abs(l_g - l_r) / np.where(live, l_r, 1)
    assert np.all(rel_l[live] <= tol_l[live]), (what, "l", np.max(rel_l[live]))
    tol_o = (2.0 ** -8 + 2.0 ** -13 + 2 * bs)[:, :, None] * o_abs + 1e-6
    err = np.abs(o_g - o_r)
    assert np.all(err[live] <= tol_o[live]), (what, "O", np.max(err[live] / tol_o[live]))
    return o_g, m_g, l_g


@pytest.mark.parametrize("depth", [64, 128])
@pytest.mark.parametrize("q_rows,kv_len,P", [(130, 300, 3), (32, 64, 1), (7, 1000, 8), (128, 129, 2)])
def test_partials_match_oracle(depth, q_rows, kv_len, P):
    q, k, v = synth.attention(900 + q_rows + kv_len, batch=1, heads=2, kv_heads=2, q_rows=q_rows,
                              kv_len=kv_len, depth=depth)
    _check_partials(q, k, v, P, 1.0 / math.sqrt(depth), "%d rows %d keys P=%d d=%d"
                    % (q_rows, kv_len, P, depth))


def test_partials_grouped_heads():
    q, k, v = synth.attention(951, batch=2, heads=8, kv_heads=2, q_rows=40, kv_len=700, depth=128)
    _check_partials(q, k, v, 8, 0.0883883, "grouped heads")


def test_partials_empty_partitions_and_no_keys():
    q, k, v = synth.attention(952, batch=1, heads=2, kv_heads=1, q_rows=9, kv_len=5, depth=64)
    _check_partials(q, k, v, 8, 0.125, "more partitions than keys")
    q, k, v = synth.attention(953, batch=1, heads=1, kv_heads=1, q_rows=3, kv_len=0, depth=128)
    o, m, l = rr.splitk_attention_partials(_bf16_tensor(q), _bf16_tensor(k), _bf16_tensor(v), 4)
    torch.cuda.synchronize()
    assert torch.all(m == -math.inf) and torch.all(l == 0) and torch.all(o == 0)


def test_partials_scales_and_wide_scores():
    q, k, v = synth.attention(954, batch=1, heads=1, kv_heads=1, q_rows=33, kv_len=200, depth=128)
    for scale in (-0.3, 1.0, 4.0):   # a negative scale flips which key is the max
        _check_partials(q, k, v, 2, scale, "scale %g" % scale)


def test_partials_bit_identical_across_runs():
    q, k, v = synth.attention(955, batch=2, heads=4, kv_heads=4, q_rows=128, kv_len=1024, depth=128)
    tq, tk, tv = _bf16_tensor(q), _bf16_tensor(k), _bf16_tensor(v)
    first = [t.clone() for t in rr.splitk_attention_partials(tq, tk, tv, 8)]
    for _ in range(4):
        again = rr.splitk_attention_partials(tq, tk, tv, 8)
        for a, b in zip(first, again):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_partials_then_merge_is_attention():
    # the whole split-K attention: partials on the matrix cores, then the LSE
    # merge, against softmax(scale q k^T) v in double
    q, k, v = synth.attention(956, batch=1, heads=4, kv_heads=2, q_rows=64, kv_len=1500, depth=128)
    scale = 1.0 / math.sqrt(128)
    o, m, l = rr.splitk_attention_partials(_bf16_tensor(q), _bf16_tensor(k), _bf16_tensor(v), 8,
                                           scale)
    got = to_host(rr.splitk_lse_merge(o, m, l, 1.0, torch.float32))
    ref_o, ref_m, ref_l = oracle.attention_partials(q, k, v, 1, scale)
    abs_o, _, _ = oracle.attention_partials(q, k, v & np.uint16(0x7FFF), 1, scale)
    bs = _score_bound(q, k, scale)
    tol = (2.0 ** -8 + 2.0 ** -13 + 4 * bs)[:, None] * abs_o[0] + 1e-6
    assert np.all(np.abs(got - ref_o[0]) <= tol)
    # and the bf16 merge of the same partials rounds the f32 merge to within 1 ulp
    got_b = to_host(rr.splitk_lse_merge(o, m, l, 1.0, torch.bfloat16))
    assert_bf16_within_1ulp(got_b, oracle.bf16_from_double(got.astype(np.float64)), "bf16 merge")


def test_partials_config_full_size_sampled_heads():
    # [8, 32, 128, 128] queries over 8192 keys in 8 partitions, inputs drawn on
    # the device; three heads copied back and checked against the oracle
    B, H, S, D, N, P = 8, 32, 128, 128, 8192, 8
    gen = torch.Generator(device="cuda")
    gen.manual_seed(957)
    q = torch.randn((B, H, S, D), generator=gen, device="cuda").to(torch.bfloat16)
    k = torch.randn((B, H, N, D), generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, H, N, D), generator=gen, device="cuda").to(torch.bfloat16)
    o, m, l = rr.splitk_attention_partials(q, k, v, P)
    torch.cuda.synchronize()
    for (b, h) in ((0, 0), (3, 17), (7, 31)):
        bits = [t[b:b + 1, h:h + 1].contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
                for t in (q, k, v)]
        o_r, m_r, l_r = oracle.attention_partials(*bits, P, 1.0 / math.sqrt(D))
        o_a, _, _ = oracle.attention_partials(bits[0], bits[1], bits[2] & np.uint16(0x7FFF), P,
                                              1.0 / math.sqrt(D))
        rows = slice((b * H + h) * S, (b * H + h + 1) * S)
        og, mg, lg = to_host(o[:, rows]), to_host(m[:, rows]), to_host(l[:, rows])
        bs = _score_bound(*bits[:2], 1.0 / math.sqrt(D))[None, :] + 2.0 ** -24 * np.abs(m_r)
        assert np.all(np.abs(mg - m_r) <= bs), (b, h)
        assert np.all(np.abs(lg - l_r) / l_r <= 2 * bs + 1024 * 2.0 ** -24 + 2.0 ** -22), (b, h)
        tol = (2.0 ** -8 + 2.0 ** -13 + 2 * bs)[:, :, None] * o_a + 1e-6
        assert np.all(np.abs(og - o_r) <= tol), (b, h)


def _random_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        kv_heads = int(rng.choice([1, 2]))
        heads = kv_heads * int(rng.choice([1, 2, 3]))
        cases.append((i, int(rng.integers(1, 3)), heads, kv_heads, int(rng.integers(1, 300)),
                      int(rng.integers(0, 2000)), int(rng.choice([64, 128])),
                      int(rng.integers(1, 13)), float(rng.uniform(-0.3, 0.3))))
    return cases


@pytest.mark.parametrize("case", _random_cases(12, 958),
                         ids=lambda c: "t%d_b%dh%dk%dq%dn%dd%dP%d" % c[:8])
def test_partials_random_shapes(case):
    i, batch, heads, kv_heads, q_rows, kv_len, depth, P, scale = case
    q, k, v = synth.attention(960 + i, batch=batch, heads=heads, kv_heads=kv_heads, q_rows=q_rows,
                              kv_len=kv_len, depth=depth)
    if kv_len == 0:
        o, m, l = rr.splitk_attention_partials(_bf16_tensor(q), _bf16_tensor(k), _bf16_tensor(v), P,
                                               scale)
        torch.cuda.synchronize()
        assert torch.all(m == -math.inf) and torch.all(l == 0) and torch.all(o == 0)
        return
    _check_partials(q, k, v, P, scale, "random %r" % (case,))


# ------------------------------------------------ fused split-K attention
def _fused_vs_two_launch(q, k, v, P, scale, out_dtype, what, workspace=None):
    """rr_splitk_attention against rr_splitk_attention_partials followed by
    rr_splitk_lse_merge: the same bits, and the tickets left zero."""
    tq, tk, tv = _bf16_tensor(q), _bf16_tensor(k), _bf16_tensor(v)
    ref = rr.splitk_lse_merge(*rr.splitk_attention_partials(tq, tk, tv, P, scale), 1.0, out_dtype)
    got = rr.splitk_attention(tq, tk, tv, P, scale, out_dtype, workspace=workspace)
    torch.cuda.synchronize()
    a = got.reshape(-1).view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32)
    b = ref.reshape(-1).view(a.dtype)
    bad = torch.nonzero(a != b)
    assert bad.numel() == 0, (what, "first differing element", int(bad[0]), bad.numel())
    return got


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("depth", [64, 128])
@pytest.mark.parametrize("q_rows,kv_len,P", [(130, 300, 3), (32, 64, 1), (7, 1000, 8),
                                             (256, 129, 2), (9, 5, 8)])
def test_fused_equals_partials_then_merge(out_dtype, depth, q_rows, kv_len, P):
    q, k, v = synth.attention(1000 + q_rows + kv_len, batch=2, heads=4, kv_heads=2, q_rows=q_rows,
                              kv_len=kv_len, depth=depth)
    _fused_vs_two_launch(q, k, v, P, 1.0 / math.sqrt(depth), out_dtype,
                         "%d rows %d keys P=%d d=%d" % (q_rows, kv_len, P, depth))


def test_fused_largest_p_negative_scale_and_no_keys():
    q, k, v = synth.attention(1010, batch=1, heads=2, kv_heads=1, q_rows=77, kv_len=2000, depth=128)
    _fused_vs_two_launch(q, k, v, 16, -0.2, torch.float32, "P=16, negative scale")
    q, k, v = synth.attention(1011, batch=1, heads=2, kv_heads=2, q_rows=3, kv_len=0, depth=64)
    got = _fused_vs_two_launch(q, k, v, 8, 0.125, torch.bfloat16, "no keys")
    assert torch.all(got.float() == 0)


def test_fused_is_attention_and_leaves_tickets_zero():
    q, k, v = synth.attention(1012, batch=1, heads=4, kv_heads=2, q_rows=64, kv_len=1500, depth=128)
    scale = 1.0 / math.sqrt(128)
    need = rr.splitk_attention_workspace_bytes(1, 4, 2, 64, 1500, 128, 8)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for _ in range(3):                             # the tickets must be reusable
        got = to_host(_fused_vs_two_launch(q, k, v, 8, scale, torch.float32, "fused", ws))
        assert torch.all(ws[:256] == 0)
    ref_o, _, _ = oracle.attention_partials(q, k, v, 1, scale)
    abs_o, _, _ = oracle.attention_partials(q, k, v & np.uint16(0x7FFF), 1, scale)
    bs = _score_bound(q, k, scale)
    tol = (2.0 ** -8 + 2.0 ** -13 + 4 * bs)[:, None] * abs_o[0] + 1e-6
    assert np.all(np.abs(got.reshape(ref_o[0].shape) - ref_o[0]) <= tol)


def test_fused_bit_identical_across_runs_and_shapes_sharing_a_workspace():
    q, k, v = synth.attention(1013, batch=2, heads=4, kv_heads=4, q_rows=128, kv_len=1024, depth=128)
    tq, tk, tv = _bf16_tensor(q), _bf16_tensor(k), _bf16_tensor(v)
    first = rr.splitk_attention(tq, tk, tv, 8).clone()
    q2, k2, v2 = synth.attention(1014, batch=1, heads=2, kv_heads=1, q_rows=300, kv_len=99, depth=64)
    for _ in range(4):
        again = rr.splitk_attention(tq, tk, tv, 8)
        assert torch.equal(again.view(torch.int16), first.view(torch.int16))
        # another shape on the same cached workspace between the runs
        _fused_vs_two_launch(q2, k2, v2, 5, 0.125, torch.bfloat16, "interleaved shape")


def test_fused_config_full_size_matches_two_launch():
    # [8, 32, 128, 128] queries over 8192 keys in 8 partitions, as the
    # benchmark runs it: the fused launch against partials + merge, every element
    B, H, S, D, N, P = 8, 32, 128, 128, 8192, 8
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1015)
    q = torch.randn((B, H, S, D), generator=gen, device="cuda").to(torch.bfloat16)
    k = torch.randn((B, H, N, D), generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, H, N, D), generator=gen, device="cuda").to(torch.bfloat16)
    ref = rr.splitk_lse_merge(*rr.splitk_attention_partials(q, k, v, P), 1.0, torch.bfloat16)
    for _ in range(2):
        got = rr.splitk_attention(q, k, v, P)
        assert torch.equal(got.reshape(-1).view(torch.int16), ref.reshape(-1).view(torch.int16))


def _fused_random_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        kv_heads = int(rng.choice([1, 2]))
        depth = int(rng.choice([64, 128]))
        cases.append((i, int(rng.integers(1, 3)), kv_heads * int(rng.choice([1, 2, 3])), kv_heads,
                      int(rng.integers(1, 300)), int(rng.integers(0, 2000)), depth,
                      int(rng.integers(1, depth // 8 + 1)), float(rng.uniform(-0.3, 0.3)),
                      bool(rng.integers(0, 2))))
    return cases


@pytest.mark.parametrize("case", _fused_random_cases(12, 1016),
                         ids=lambda c: "t%d_b%dh%dk%dq%dn%dd%dP%d" % c[:8])
def test_fused_random_shapes(case):
    i, batch, heads, kv_heads, q_rows, kv_len, depth, P, scale, bf16 = case
    q, k, v = synth.attention(1020 + i, batch=batch, heads=heads, kv_heads=kv_heads, q_rows=q_rows,
                              kv_len=kv_len, depth=depth)
    _fused_vs_two_launch(q, k, v, P, scale, torch.bfloat16 if bf16 else torch.float32,
                         "random %r" % (case,))


def test_host_tensors_are_refused_before_any_launch():
    q, k, v = synth.attention(1030, batch=1, heads=2, kv_heads=2, q_rows=16, kv_len=64, depth=64)
    tq, tk, tv = _bf16_tensor(q), _bf16_tensor(k), _bf16_tensor(v)
    with pytest.raises(ValueError):
        rr.splitk_attention(tq, tk, tv, 2, out=torch.empty((1, 2, 16, 64), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        rr.splitk_attention(tq, tk, tv, 2, workspace=torch.zeros(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError):
        rr.splitk_attention(tq, tk.cpu(), tv, 2)
    with pytest.raises(ValueError):
        rr.splitk_attention_partials(tq, tk, tv, 2, out=(torch.empty((2, 32, 64)),
                                                         torch.empty((2, 32)), torch.empty((2, 32))))
    o, m, l = rr.splitk_attention_partials(tq, tk, tv, 2)
    with pytest.raises(ValueError):
        rr.splitk_lse_merge(o, m.cpu(), l, 1.0)
    with pytest.raises(ValueError):
        rr.splitk_lse_merge(o, m, l, 1.0, torch.bfloat16, out=torch.empty((32, 64), dtype=torch.bfloat16))


def test_fused_bits_do_not_depend_on_arrival_order():
    # Under the skew hook the partitions of a query tile take their ticket in
    # (roughly) descending order, so another workgroup does the fold; it
    # still visits the partitions in ascending order.
    q, k, v = synth.attention(1040, batch=2, heads=4, kv_heads=2, q_rows=200, kv_len=3000, depth=128)
    tq, tk, tv = _bf16_tensor(q), _bf16_tensor(k), _bf16_tensor(v)
    plain = rr.splitk_attention(tq, tk, tv, 8, None, torch.float32).clone()
    try:
        rr._set_splitk_skew(16)
        skewed = rr.splitk_attention(tq, tk, tv, 8, None, torch.float32).clone()
        torch.cuda.synchronize()
    finally:
        rr._set_splitk_skew(0)
    assert torch.equal(skewed.view(torch.int32), plain.view(torch.int32))
    _fused_vs_two_launch(q, k, v, 8, 1.0 / math.sqrt(128), torch.float32, "after the skewed run")


def test_fused_cached_workspace_grows_its_ticket_region():
    # A call with few query tiles but large partials, then one with more
    # tiles (a ticket region past the first 256 bytes) and smaller partials:
    # the cached workspace is reused, and the second call's tickets lie where
    # the first call left partials, so the binding clears them first.
    qa, ka, va = synth.attention(1050, batch=1, heads=1, kv_heads=1, q_rows=1024, kv_len=64,
                                 depth=128)
    _fused_vs_two_launch(qa, ka, va, 16, 0.1, torch.float32, "few tiles, large partials")
    qb, kb, vb = synth.attention(1051, batch=4, heads=32, kv_heads=32, q_rows=16, kv_len=50,
                                 depth=64)
    need_a = rr.splitk_attention_workspace_bytes(1, 1, 1, 1024, 64, 128, 16)
    need_b, tick_b = rr.splitk_attention_workspace_bytes(4, 32, 32, 16, 50, 64, 1,
                                                         with_tickets=True)
    assert need_b < need_a and tick_b > 256
    for _ in range(2):
        _fused_vs_two_launch(qb, kb, vb, 1, 0.125, torch.bfloat16, "more tiles, reused workspace")
