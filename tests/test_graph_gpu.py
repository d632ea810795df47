"""HIP graph capture and replay of the library's launches.

A caller may capture these calls in a graph (torch.cuda.CUDAGraph).  Nothing
the library launches clears memory with a memset: the split-K reduction's
tickets reset themselves and every other workspace is written before it is
read, so the captured kernels alone reproduce the eager results.  The graph
is replayed several times with the program's own eager work and
synchronisations in between, and every replay is checked bit for bit
against the eager result.
"""
import pytest
import torch

import split_deterministic_combine_amd as rr
from split_deterministic_combine_amd import synth
from tests.gpu_util import to_gpu

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def test_graph_replays_match_eager_bit_for_bit():
    dev = torch.device("cuda")
    x_long = to_gpu(synth.uniform_f32(40, (16, 1 << 20)))             # split-K reduce
    x_short = to_gpu(synth.normal_f32(41, (65536, 48)))               # wave tier
    x_sm = to_gpu(synth.normal_bf16(42, (4, 200000)))                 # split-K softmax
    x_blk = to_gpu(synth.normal_bf16(43, (2048, 4096)))               # persistent softmax
    x_ln = to_gpu(synth.normal_bf16(44, (2048, 4096)))                # persistent layernorm
    g_ln = to_gpu(synth.uniform_f32(45, (4096,), 0.5, 1.5))
    b_ln = to_gpu(synth.uniform_f32(46, (4096,), -0.5, 0.5))
    x_lnk = to_gpu(synth.normal_bf16(47, (8, 300000)))                # split-K layernorm
    x_ax = to_gpu(synth.normal_f32(48, (1, 1 << 16, 64)))             # axis split-K
    o, m, l = synth.lse_merge(49, P=8, batch=1, heads=4, q_rows=64, depth=128)
    o, m, l = to_gpu(o), to_gpu(m), to_gpu(l)
    aq, ak, av = (to_gpu(a) for a in synth.attention(50, batch=1, heads=4, kv_heads=2, q_rows=130,
                                                     kv_len=777, depth=128))
    # packed sequences (longest-first work order: 4 x 2 units per sequence)
    vq, vk, vv, cq, ck = synth.attention_varlen(51, [130, 0, 77], [300, 20, 1000], 4, 2, 128, 1, 0)
    vq, vk, vv, cq, ck = (to_gpu(a) for a in (vq, vk, vv, cq, ck))
    # misaligned layernorm rows (odd stride) with weights staged in LDS
    x_lnm = to_gpu(synth.normal_bf16(52, (1024, 4095)))
    g_lnm = to_gpu(synth.uniform_f32(53, (4095,), 0.5, 1.5))
    b_lnm = to_gpu(synth.uniform_f32(54, (4095,), -0.5, 0.5))

    outs = {
        "long_sum": torch.empty(16, device=dev),
        "long_max": torch.empty(16, device=dev),
        "short_sum": torch.empty(65536, device=dev),
        "multi": {k: torch.empty(16, device=dev) for k in ("sum", "max", "min")},
        "sm_splitk": torch.empty_like(x_sm),
        "sm_block": torch.empty_like(x_blk),
        "ln": torch.empty_like(x_ln),
        "ln_mean": torch.empty(2048, device=dev),
        "ln_splitk": torch.empty_like(x_lnk),
        "axis": torch.empty((1, 64), device=dev),
        "merge": torch.empty((1, 4, 64, 128), dtype=torch.bfloat16, device=dev),
        "attn": {"o": torch.empty((4, 520, 128), device=dev), "m": torch.empty((4, 520), device=dev),
                 "l": torch.empty((4, 520), device=dev)},
        "attn_fused": torch.empty((1, 4, 130, 128), dtype=torch.bfloat16, device=dev),
        "varlen": {"o": torch.empty((4, 208, 4, 128), device=dev),
                   "m": torch.empty((4, 208, 4), device=dev), "l": torch.empty((4, 208, 4), device=dev)},
        "ln_peel": torch.empty_like(x_lnm),
    }
    # tokens of no sequence are never written: every output starts from the
    # bytes each replay's scribble leaves
    for v in outs.values():
        for t in (v.values() if isinstance(v, dict) else (v,)):
            t.view(torch.uint8).fill_(0x7F)

    def run_all():
        rr.reduce_rows(x_long, "sum", out=outs["long_sum"])
        rr.reduce_rows(x_long, "max", out=outs["long_max"])
        rr.reduce_rows(x_short, "sum", out=outs["short_sum"])
        rr.reduce_rows_multi(x_long, out=outs["multi"])
        rr.softmax_rows(x_sm, out=outs["sm_splitk"])
        rr.softmax_rows(x_blk, out=outs["sm_block"])
        rr.layernorm_rows(x_ln, g_ln, b_ln, 1e-5, out=outs["ln"], mean_out=outs["ln_mean"])
        rr.layernorm_rows(x_lnk, eps=1e-5, out=outs["ln_splitk"])
        rr.reduce_axis(x_ax, 1, "sum", out=outs["axis"])
        rr.splitk_lse_merge(o, m, l, 1.0, torch.bfloat16, out=outs["merge"])
        rr.splitk_attention_partials(aq, ak, av, 4, out=(outs["attn"]["o"], outs["attn"]["m"],
                                                         outs["attn"]["l"]))
        rr.splitk_attention(aq, ak, av, 4, out=outs["attn_fused"])
        rr.splitk_attention_partials_varlen(vq, vk, vv, cq, ck, 130, 4,
                                            out=(outs["varlen"]["o"], outs["varlen"]["m"],
                                                 outs["varlen"]["l"]))
        rr.layernorm_rows(x_lnm, g_lnm, b_lnm, 1e-5, out=outs["ln_peel"])

    def snapshot():
        flat = {}
        for k, v in outs.items():
            if isinstance(v, dict):
                for kk, vv in v.items():
                    flat[k + "." + kk] = vv.clone()
            else:
                flat[k] = v.clone()
        return flat

    # eager reference (also creates the workspaces of the capture stream)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_all()
        run_all()
    s.synchronize()
    with torch.cuda.stream(s):
        run_all()
    s.synchronize()
    eager = snapshot()
    assert rr.plan_reduce(16, 1 << 20, cu_count=rr.device_cu_count())["tier"] == "splitk"

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        run_all()
    for replay in range(3):
        for v in outs.values():  # scribble on the outputs so a replay must rewrite them
            for t in (v.values() if isinstance(v, dict) else (v,)):
                t.view(torch.uint8).fill_(0x7F)
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for k in eager:
            assert torch.equal(_bits(got[k]), _bits(eager[k])), "replay %d: %s" % (replay, k)
        # eager work on the default stream between replays
        torch.cuda.current_stream().wait_stream(s)
        junk = rr.softmax_rows(x_blk)
        rr.reduce_rows(x_short, "max")
        torch.cuda.synchronize()
        del junk
