"""GPU parity of the split-K attention partials of packed variable-length
sequences (rr_splitk_attention_partials_varlen) against the CPU oracle, and of
their LSE merge into the ragged [tokens][heads][depth] output.

The bar is the one of the dense partials (the arithmetic per query row is the
same): with B_s the score bound of a row over its own sequence's keys,
|dm| <= B_s, |dl| / l <= 2 B_s + n 2^-24 + 2^-22 and
|dO| <= (2^-8 + 2^-13 + 2 B_s) * (the oracle's output for |v|) + 1e-6.
Tokens that belong to no sequence keep what the output held (NaN here).
A sequence in the packed layout gives the same bits as the dense call on it.
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


def _score_bound(q, k, cu_q, cu_k, scale):
    """B_s per partial row (token, head): scale * depth * 2^-24 * the largest
    sum_d |q_d k_jd| over the keys j of the token's sequence (0 off sequences)."""
    total_q, heads, depth = q.shape
    group = heads // k.shape[1]
    qd, kd = np.abs(_bf16_double(q)), np.abs(_bf16_double(k))
    bs = np.zeros((total_q, heads))
    for b in range(cu_q.size - 1):
        a0, a1, c0, c1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if a1 <= a0 or c1 <= c0:
            continue
        for h in range(heads):
            worst = (qd[a0:a1, h] @ kd[c0:c1, h // group].T).max(-1)
            bs[a0:a1, h] = abs(scale) * depth * 2.0 ** -24 * worst
    return bs.reshape(-1)


def _varlen(q, k, v, cu_q, cu_k, P, scale, max_q=None):
    """The GPU partials, written into NaN-filled outputs (max_q: the longest
    sequence unless given)."""
    total_q, heads, depth = q.shape
    out = (torch.full((P, total_q, heads, depth), float("nan"), device="cuda"),
           torch.full((P, total_q, heads), float("nan"), device="cuda"),
           torch.full((P, total_q, heads), float("nan"), device="cuda"))
    if max_q is None:
        max_q = int(np.max(np.diff(cu_q))) if cu_q.size > 1 else 0
    rr.splitk_attention_partials_varlen(
        _bf16_tensor(q), _bf16_tensor(k), _bf16_tensor(v),
        torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda(), max_q, P, scale, out=out)
    torch.cuda.synchronize()
    return out


def _check(q, k, v, cu_q, cu_k, P, scale, what):
    total_q, heads, depth = q.shape
    rows = total_q * heads
    o_t, m_t, l_t = _varlen(q, k, v, cu_q, cu_k, P, scale)
    o_g = to_host(o_t).reshape(P, rows, depth)
    m_g, l_g = to_host(m_t).reshape(P, rows), to_host(l_t).reshape(P, rows)
    o_r, m_r, l_r = oracle.attention_partials_varlen(q, k, v, cu_q, cu_k, P, scale)
    o_abs, _, _ = oracle.attention_partials_varlen(q, k, v & np.uint16(0x7FFF), cu_q, cu_k, P,
                                                   scale)
    # tokens outside every sequence: not written by either side
    off = np.isnan(m_r)
    assert np.array_equal(np.isnan(m_g), off) and np.array_equal(np.isnan(l_g), off), what
    assert np.all(np.isnan(o_g[off])), what
    assert not np.any(np.isnan(o_g[~off])), what
    on = ~off
    empty = on & (m_r == -np.inf)
    assert np.all(m_g[empty] == -np.inf) and np.all(l_g[empty] == 0), what
    assert np.all(o_g[empty] == 0), what
    live = on & ~empty
    bs = _score_bound(q, k, cu_q, cu_k, scale)[None, :] + \
        2.0 ** -24 * np.abs(np.where(live, m_r, 0))
    dm = np.abs(m_g[live] - m_r[live])
    assert np.all(dm <= bs[live]), (what, "m", np.max(dm, initial=0))
    n_keys = -(-int(np.max(np.diff(cu_k), initial=0)) // P)
    tol_l = 2 * bs + n_keys * 2.0 ** -24 + 2.0 ** -22
    rel_l = np.abs(l_g - l_r) / np.where(live, l_r, 1)
    assert np.all(rel_l[live] <= tol_l[live]), (what, "l", np.max(rel_l[live], initial=0))
    tol_o = (2.0 ** -8 + 2.0 ** -13 + 2 * bs)[:, :, None] * o_abs + 1e-6
    err = np.abs(o_g - o_r)
    assert np.all(err[live] <= tol_o[live]), (what, "O", np.max(err[live] / tol_o[live], initial=0))
    return o_t, m_t, l_t


CASES = [
    # q_lens, k_lens, heads, kv_heads, depth, P, q_lead, k_lead
    ([130, 0, 7, 257, 1], [300, 50, 0, 129, 1000], 4, 2, 128, 3, 5, 3),
    ([128, 129, 1], [64, 64, 8], 2, 2, 64, 8, 0, 0),
    ([0, 0, 33], [5, 0, 40], 3, 1, 128, 4, 2, 1),
    ([200, 17, 64, 300], [17, 1024, 200, 1], 8, 2, 128, 8, 0, 11),
    # many short sequences: the longest-first order over a batch of 256 (one
    # per thread of the ranking) and, past 256, the sequence-fastest order
    ([(i * 7) % 4 for i in range(256)], [(i * 13) % 21 for i in range(256)], 1, 1, 64, 8, 1, 0),
    ([(i * 5) % 3 for i in range(260)], [(i * 11) % 17 for i in range(260)], 2, 1, 64, 8, 0, 2),
]


@pytest.mark.parametrize("q_lens,k_lens,heads,kv_heads,depth,P,q_lead,k_lead", CASES)
def test_varlen_partials_match_oracle(q_lens, k_lens, heads, kv_heads, depth, P, q_lead, k_lead):
    q, k, v, cu_q, cu_k = synth.attention_varlen(700 + sum(q_lens) + sum(k_lens), q_lens, k_lens,
                                                 heads, kv_heads, depth, q_lead, k_lead)
    _check(q, k, v, cu_q, cu_k, P, 1.0 / math.sqrt(depth),
           "q %s k %s h %d/%d d %d P %d" % (q_lens, k_lens, heads, kv_heads, depth, P))


def test_varlen_no_sequence_has_tokens():
    # every sequence empty: nothing is written; q has only lead tokens
    q, k, v, cu_q, cu_k = synth.attention_varlen(760, [0, 0, 0], [3, 0, 2], 2, 2, 64, 4, 0)
    o, m, l = _varlen(q, k, v, cu_q, cu_k, 2, 0.125)
    assert torch.all(torch.isnan(o)) and torch.all(torch.isnan(m)) and torch.all(torch.isnan(l))


def test_varlen_sequence_equals_dense_call_bitwise():
    # each sequence alone through the dense producer ([1][heads][rows][depth])
    # gives the bits of its rows in the packed call
    q_lens, k_lens, heads, kvh, depth, P = [77, 300, 128], [500, 129, 2000], 4, 2, 128, 8
    q, k, v, cu_q, cu_k = synth.attention_varlen(761, q_lens, k_lens, heads, kvh, depth)
    o, m, l = _varlen(q, k, v, cu_q, cu_k, P, 0.0883883)
    for b in range(len(q_lens)):
        a0, a1, c0, c1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        qd = np.ascontiguousarray(q[a0:a1].transpose(1, 0, 2))[None]
        kd = np.ascontiguousarray(k[c0:c1].transpose(1, 0, 2))[None]
        vd = np.ascontiguousarray(v[c0:c1].transpose(1, 0, 2))[None]
        od, md, ld = rr.splitk_attention_partials(_bf16_tensor(qd), _bf16_tensor(kd),
                                                  _bf16_tensor(vd), P, 0.0883883)
        n = a1 - a0
        od = od.view(P, heads, n, depth).permute(0, 2, 1, 3)
        md, ld = md.view(P, heads, n).permute(0, 2, 1), ld.view(P, heads, n).permute(0, 2, 1)
        assert torch.equal(o[:, a0:a1].view(torch.int32), od.contiguous().view(torch.int32)), b
        assert torch.equal(m[:, a0:a1].view(torch.int32), md.contiguous().view(torch.int32)), b
        assert torch.equal(l[:, a0:a1].view(torch.int32), ld.contiguous().view(torch.int32)), b


def test_varlen_partials_then_merge_is_ragged_attention():
    # partials, then the merge over rows = total_q * heads: the ragged output
    # [total_q][heads][depth] of each sequence's own attention, against the
    # oracle's merge of the same partials (bf16 within 1 ulp) and the
    # oracle's one-partition attention (float32 within the partials' bar)
    q_lens, k_lens, heads, kvh, depth, P = [130, 0, 45, 1], [700, 20, 0, 3000], 4, 2, 128, 8
    q, k, v, cu_q, cu_k = synth.attention_varlen(762, q_lens, k_lens, heads, kvh, depth, 3, 0)
    scale = 1.0 / math.sqrt(depth)
    o, m, l = _check(q, k, v, cu_q, cu_k, P, scale, "merge case")
    total_q = q.shape[0]
    rows = total_q * heads
    o2, m2, l2 = o.view(P, rows, depth), m.view(P, rows), l.view(P, rows)
    got_b = to_host(rr.splitk_lse_merge(o2, m2, l2, 1.0, torch.bfloat16))
    ref_b = oracle.splitk_lse_merge(to_host(o2), to_host(m2), to_host(l2), 1.0, "bf16")
    assert_bf16_within_1ulp(got_b, ref_b, "ragged bf16 merge")
    got = to_host(rr.splitk_lse_merge(o2, m2, l2, 1.0, torch.float32))
    ref_o, ref_m, _ = oracle.attention_partials_varlen(q, k, v, cu_q, cu_k, 1, scale)
    abs_o, _, _ = oracle.attention_partials_varlen(q, k, v & np.uint16(0x7FFF), cu_q, cu_k, 1,
                                                   scale)
    live = np.isfinite(ref_m[0])        # NaN off every sequence, -inf with no key
    bs = _score_bound(q, k, cu_q, cu_k, scale)
    tol = (2.0 ** -8 + 2.0 ** -13 + 4 * bs)[:, None] * abs_o[0] + 1e-6
    assert np.all(np.abs(got[live] - ref_o[0][live]) <= tol[live])
    # rows with no key or of no sequence merge to zeros
    assert np.all(got[~live] == 0)


def test_varlen_rows_past_max_q_rows_are_not_written():
    # max_q_rows below the longest sequence: each sequence's first max_q_rows
    # query rows carry the bits of the call with the full bound, and the rest
    # keep what the outputs held
    q_lens, k_lens, heads, kvh, depth, P, max_q = [130, 40, 97, 0], [300, 17, 90, 5], 2, 1, 64, 4, 64
    q, k, v, cu_q, cu_k = synth.attention_varlen(764, q_lens, k_lens, heads, kvh, depth, 2, 0)
    full = _varlen(q, k, v, cu_q, cu_k, P, 0.125)
    part = _varlen(q, k, v, cu_q, cu_k, P, 0.125, max_q=max_q)
    local = np.full(q.shape[0], -1)
    for b in range(len(q_lens)):
        local[cu_q[b]:cu_q[b + 1]] = np.arange(cu_q[b + 1] - cu_q[b])
    done = torch.from_numpy((local >= 0) & (local < max_q)).cuda()
    assert int(done.sum()) == sum(min(n, max_q) for n in q_lens)
    for f, g in zip(full, part):
        assert torch.equal(f[:, done].view(torch.int32), g[:, done].view(torch.int32))
        assert torch.all(torch.isnan(g[:, ~done]))


def test_varlen_mixed_batch_ten_runs_bit_identical():
    # eight sequences with key counts 512 .. 3584 (the bench row's mix at a
    # quarter of its length): the longest-first work order ranks them on the
    # device; ten calls give the same bits, and sampled sequences match the
    # oracle
    k_lens = [512, 1024, 1536, 2048, 2048, 2560, 3072, 3584]
    q, k, v, cu_q, cu_k = synth.attention_varlen(765, [128] * 8, k_lens, 32, 32, 128)
    args = (_bf16_tensor(q), _bf16_tensor(k), _bf16_tensor(v), torch.from_numpy(cu_q).cuda(),
            torch.from_numpy(cu_k).cuda(), 128, 8)
    first = [t.clone() for t in rr.splitk_attention_partials_varlen(*args)]
    for _ in range(9):
        again = rr.splitk_attention_partials_varlen(*args)
        for f, g in zip(first, again):
            assert torch.equal(f.view(torch.int32), g.view(torch.int32))
    for b in (0, 7):
        a0, a1, c0, c1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        sel = [t[a0:a1, 5:6] for t in (q,)] + [t[c0:c1, 5:6] for t in (k, v)]
        sub_cq, sub_ck = np.array([0, a1 - a0], np.int32), np.array([0, c1 - c0], np.int32)
        o_r, m_r, _ = oracle.attention_partials_varlen(*sel, sub_cq, sub_ck, 8, 1.0 / math.sqrt(128))
        o_a, _, _ = oracle.attention_partials_varlen(sel[0], sel[1], sel[2] & np.uint16(0x7FFF),
                                                     sub_cq, sub_ck, 8, 1.0 / math.sqrt(128))
        og = to_host(first[0][:, a0:a1, 5])
        mg = to_host(first[1][:, a0:a1, 5])
        assert np.all(np.abs(og - o_r) <= (2.0 ** -8 + 2.0 ** -12) * o_a + 1e-6), b
        assert np.all(np.abs(mg - m_r[:, :]) <= 1e-5 * (1 + np.abs(m_r))), b


def test_varlen_rejects_bad_arguments():
    q, k, v, cu_q, cu_k = synth.attention_varlen(763, [4], [4], 2, 2, 64)
    tq, tk, tv = _bf16_tensor(q), _bf16_tensor(k), _bf16_tensor(v)
    cq, ck = torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda()
    with pytest.raises(ValueError):
        rr.splitk_attention_partials_varlen(tq, tk, tv, cq.long(), ck, 4, 2)
    with pytest.raises(ValueError):
        rr.splitk_attention_partials_varlen(tq, tk, tv, cq, ck[:1], 4, 2)
    with pytest.raises(rr.RRError):
        rr.splitk_attention_partials_varlen(tq, tk, tv, cq, ck, 4, 0)
