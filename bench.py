"""Benchmark of the row-reduce hot path on one MI355X.

One step runs every operation of the path once on its synthetic workload:
  short_rows  f32 row sum and row max over [1048576, 48]     (wave tier)
  softmax     bf16 softmax over [8192, 8192]                  (block tier)
  long_rows   f32 row sum and int32 row max over [16, 2^24]   (split-K tier)
  lse_merge   P = 8 merge of O [8, 8, 32, 128, 128] -> bf16 [8, 32, 128, 128]

Outside the step (and outside `value`), the operations built after it are
timed on their own workloads and reported under "next_rows":
  softmax_long  bf16 softmax over [16, 2^22]                 (split-K tier)
  layernorm     bf16 layernorm over [16384, 4096], float32 gamma/beta,
                float32 mean/rstd written                      (block tier)
  multi_long    f32 sum, max and min over [16, 2^24] from one read (split-K)
  axis_cols     f32 column sums of [16384, 16384] (non-last axis, split-K)
  attention     split-K attention partials: bf16 q [8, 32, 128, 128] over 8192
                keys in 8 partitions -> float32 O, m, l (matrix cores)
  attention_merged  the same, then the LSE merge of the partials -> bf16
  attention_fused   the same in one launch: the last workgroup of each query
                tile folds the partials in partition order -> bf16 (the
                same bits as attention_merged)

Inputs are resident in HBM before timing.  Buffer sets rotate from one step
to the next so that the data touched by consecutive launches exceeds the
~256 MB Infinity Cache (the long-row inputs are 1 GiB each by themselves).

`value` is whole-step throughput in GB/s: algorithmic bytes of all launches
(each input element read once, each output written once) divided by the
measured step time.  Per-launch durations come from HIP events recorded on
the stream the kernels are launched on; each operation's GB/s is taken from
its median launch, the roofline's from the dominant kernel's mean launch in
the timed region, and each next-row operation also reports its launches run
back to back between one pair of events (the sustained rate).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import gc
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "achieved HBM GB/s and % of peak for rowwise reduce/softmax/split-K merge"
CSRC = os.path.join(ROOT, "split_deterministic_combine_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash():
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


# op name -> substring of the kernel symbol that runs it at the benchmark shapes
KERNEL_OF_OP = {
    "short_sum": "k_reduce_wave<rr::SumF32, 4, 16, 0>",
    "short_max": "k_reduce_wave<rr::MaxF32, 4, 16, 0>",
    "softmax": "k_softmax_rows_pf<unsigned short, unsigned short, 4, 256, true, false, false>",
    "long_sum": "k_reduce_splitk<rr::SumF32, 4>",
    "long_max": "k_reduce_splitk<rr::MaxI32, 4>",
    "merge": "k_lse_merge_po<unsigned short, 32, 4, true>",
    "softmax_long_stats": "k_softmax_splitk_stats<unsigned short, true>",
    "softmax_long_map": "k_softmax_splitk_map<unsigned short, unsigned short, true>",
    "layernorm": "k_layernorm_rows_pf<unsigned short, unsigned short, 4, 128, true, true>",
    "multi_long": "k_reduce_splitk<rr::MultiF32, 4>",
    "axis_cols_partial": "k_reduce_axis_partial<rr::SumF32, 4>",
    "axis_cols_fold": "k_reduce_axis_fold<rr::SumF32>",
    "attention": "k_attn_staged<128, 32, 3, false, float, false>",
    "attention_fused": "k_attn_staged<128, 32, 3, true, unsigned short, false>",
    "attention_varlen": "k_attn_staged<128, 32, 3, false, float, true>",
    # rows at every offset from a 16-byte boundary and their aligned neighbour
    "sum_47": "k_reduce_wave<rr::SumF32, 4, 16, 2>",
    "sum_1001": "k_reduce_rows_pf<rr::SumF32, 4, 64, true, 64>",
    "sum_1000": "k_reduce_rows_pf<rr::SumF32, 4, 64, false, 64>",
    "softmax_8191": "k_softmax_rows_pf<unsigned short, unsigned short, 4, 256, false, true, true>",
    # reference streams of known size (not ops of the step): rr_test_stream;
    # launches of one kernel at two sizes are told apart by their bytes
    "stream_read": "k_stream<0>",
    "stream_read_128MiB": "k_stream<0>",
    "stream_write": "k_stream<1>",
}
LAYERNORM = (16384, 4096)
SOFTMAX_LONG = (16, 1 << 22)
AXIS_COLS = (16384, 16384)
# split-K attention partials: batch, heads, query rows, depth, keys, partitions
ATTN = (8, 32, 128, 128, 8192, 8)
# the same attention over packed sequences of mixed key lengths (ragged
# placement): ATTN's batch of 128-query sequences, key lengths summing to
# batch * keys, so the bytes and flops equal the dense row's
ATTN_VARLEN_K = (2048, 4096, 6144, 8192, 8192, 10240, 12288, 14336)
assert sum(ATTN_VARLEN_K) == ATTN[0] * ATTN[4] and len(ATTN_VARLEN_K) == ATTN[0]
CU_MI355X = 256


def _attn_bytes():
    """q, k, v read once (bf16); O (float32), m and l written once."""
    b, h, sq, d, n, p = ATTN
    return b * h * sq * d * 2 + 2 * b * h * n * d * 2 + p * b * h * sq * d * 4 + 2 * p * b * h * sq * 4


def _attn_fused_bytes():
    """q, k, v read once and the bf16 attention output written once."""
    b, h, sq, d, n, _ = ATTN
    return b * h * sq * d * 2 + 2 * b * h * n * d * 2 + b * h * sq * d * 2


def _attn_flops():
    """q k^T and P v: 2 flops per multiply-add, 4 * batch*heads*q_rows*keys*depth."""
    b, h, sq, d, n, _ = ATTN
    return 4 * b * h * sq * n * d


def _algo_bytes():
    """Algorithmic bytes per launch of each timed kernel.  The split-K
    workspace terms depend on the slice count G, taken from the library's
    host planner for a 256-CU MI355X (the same plan the launches use)."""
    import split_deterministic_combine_amd as rr_host

    g_sm = rr_host.plan_softmax(*SOFTMAX_LONG, cu_count=CU_MI355X)["slices"]
    g_ax = rr_host.plan_axis(1, AXIS_COLS[0], AXIS_COLS[1], cu_count=CU_MI355X)["slices"]
    sr, sc = SOFTMAX_LONG
    ar, ac = AXIS_COLS
    return {
        "short_sum": 1048576 * 48 * 4 + 1048576 * 4,
        "short_max": 1048576 * 48 * 4 + 1048576 * 4,
        "softmax": 8192 * 8192 * 2 * 2,
        "long_sum": 16 * (1 << 24) * 4 + 16 * 4,
        "long_max": 16 * (1 << 24) * 4 + 16 * 4,
        "merge": 8 * 32768 * 128 * 4 + 2 * 8 * 32768 * 4 + 32768 * 128 * 2,
        # split-K softmax, per kernel: the statistics pass reads x and stores
        # rows x G (max, sum) pairs; the map pass reads x and, in each of the
        # G workgroups of a row, the row's G pairs, and writes y
        "softmax_long_stats": sr * sc * 2 + sr * g_sm * 8,
        "softmax_long_map": sr * sc * 2 * 2 + sr * g_sm * g_sm * 8,
        # x read and y written once (bf16), gamma/beta read once, mean/rstd written
        "layernorm": 16384 * 4096 * 2 * 2 + 2 * 4096 * 4 + 2 * 16384 * 4,
        "multi_long": 16 * (1 << 24) * 4 + 3 * 16 * 4,
        # column sums: the partial pass reads x and writes G partials (8 B)
        # per column; the fold pass reads them and writes y
        "axis_cols_partial": ar * ac * 4 + g_ax * ac * 8,
        "axis_cols_fold": g_ax * ac * 8 + ac * 4,
        "attention": _attn_bytes(),
        # one launch: q, k, v read once and the bf16 output written once (the
        # partials pass through the device-coherent level, not counted)
        "attention_fused": _attn_fused_bytes(),
        "attention_varlen": _attn_bytes(),
        "sum_47": 1048576 * 47 * 4 + 1048576 * 4,
        "sum_1001": 65536 * 1001 * 4 + 65536 * 4,
        "sum_1000": 65536 * 1000 * 4 + 65536 * 4,
        "softmax_8191": 8192 * 8191 * 2 * 2,
        "stream_read": 1 << 30,
        "stream_read_128MiB": 128 << 20,
        "stream_write": 1 << 30,
    }


# next-row operations as a whole: x read once and y written once
NEXT_BYTES = {"multi_long": 16 * (1 << 24) * 4 + 3 * 16 * 4,
              "axis_cols": AXIS_COLS[0] * AXIS_COLS[1] * 4 + AXIS_COLS[1] * 4,
              "softmax_long": 16 * (1 << 22) * 2 * 2,
              "layernorm": 16384 * 4096 * 2 * 2 + 2 * 4096 * 4 + 2 * 16384 * 4,
              "attention": _attn_bytes(),
              # q, k, v read and bf16 attention written once (the partials are internal)
              "attention_merged": _attn_fused_bytes(),
              "attention_fused": _attn_fused_bytes(),
              # packed sequences: the dense row's q, k, v and partial bytes
              "attention_varlen": _attn_bytes(),
              # rows that do not all start 16-byte aligned (odd row strides),
              # beside their aligned neighbours: each row's body from its
              # first 16-byte boundary in 128-bit loads, head and tail scalar
              "sum_47": 1048576 * 47 * 4 + 1048576 * 4,
              "sum_1001": 65536 * 1001 * 4 + 65536 * 4,
              "sum_1000": 65536 * 1000 * 4 + 65536 * 4,
              "softmax_8191": 8192 * 8191 * 2 * 2}
# each odd-stride row's aligned neighbour: a step op or another next row
NEIGHBOUR = {"sum_47": "short_sum", "sum_1001": "sum_1000", "softmax_8191": "softmax"}
STEP_OPS = ("short_sum", "short_max", "softmax", "long_sum", "long_max", "merge")
COPY_BYTES = 512 << 20


def _csv_rows(directory, suffix):
    import csv
    import glob

    rows = []
    for f in sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def ingest_counters(trace_dir, fetch_dir, write_dir):
    """Turn rocprofv3 CSVs into profiles/traffic.json and markdown summaries."""
    ALGO_BYTES = _algo_bytes()
    per_counter = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            if r.get("Counter_Name") != name:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        per_counter[name] = vals

    def mean_for(vals, pattern, kib_expected=None):
        # dispatches of the pattern; where one kernel runs at several sizes,
        # only those within a factor of 2.5 of the op's expected KiB
        hits = [v for k, vs in vals.items() if pattern in k for v in vs
                if kib_expected is None or v == 0 or 0.4 * kib_expected <= v <= 2.5 * kib_expected]
        return sum(hits) / len(hits) if hits else None

    copy_pat = "neg"  # torch's elementwise negation kernel run by --calibrate-copy
    copy_fetch = [v for k, vs in per_counter["FETCH_SIZE"].items() if copy_pat in k.lower() for v in vs]
    copy_write = [v for k, vs in per_counter["WRITE_SIZE"].items() if copy_pat in k.lower() for v in vs]
    # counters are in KiB per dispatch; the calibration copy moves COPY_BYTES each way
    fetch_scale = COPY_BYTES / (1024.0 * max(copy_fetch)) if copy_fetch else None
    write_scale = COPY_BYTES / (1024.0 * max(copy_write)) if copy_write else None
    kernels = {}
    for op, pat in KERNEL_OF_OP.items():
        shared = sum(1 for q in KERNEL_OF_OP.values() if q == pat) > 1
        exp_kib = ALGO_BYTES[op] / 1024.0 if shared else None
        f = mean_for(per_counter["FETCH_SIZE"], pat,
                     exp_kib / fetch_scale if exp_kib and fetch_scale else None)
        w = mean_for(per_counter["WRITE_SIZE"], pat)
        if f is None or w is None or fetch_scale is None or write_scale is None:
            continue
        fb, wb = f * 1024.0 * fetch_scale, w * 1024.0 * write_scale
        kernels[op] = {"kernel": pat, "fetch_kib_raw": round(f, 1), "write_kib_raw": round(w, 1),
                       "fetch_bytes": int(fb), "write_bytes": int(wb),
                       "bytes_per_launch": int(fb + wb), "algorithmic_bytes": ALGO_BYTES[op],
                       "traffic_over_algorithmic": round((fb + wb) / ALGO_BYTES[op], 3)}
    out = {"source_hash": kernel_source_hash(),
           "calibration": {"copy_bytes_each_way": COPY_BYTES,
                           "copy_fetch_kib_raw": max(copy_fetch) if copy_fetch else None,
                           "copy_write_kib_raw": max(copy_write) if copy_write else None,
                           "fetch_scale": fetch_scale, "write_scale": write_scale},
           "kernels": kernels}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    # durations per dispatch (the trace), so that launches of one kernel at
    # two sizes are told apart: an op whose kernel also runs another op keeps
    # the dispatches whose algorithmic rate would lie between 2 and 9 TB/s
    durs = {}
    for r in _csv_rows(trace_dir, "kernel_trace.csv"):
        durs.setdefault(r["Kernel_Name"], []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["| kernel (op) | launches | avg us | median us | min us | max us | algorithmic GB/s "
             "| % of 8 TB/s |", "|---|---|---|---|---|---|---|---|"]
    for op, pat in KERNEL_OF_OP.items():
        shared = sum(1 for q in KERNEL_OF_OP.values() if q == pat) > 1
        ds = sorted(d for k, v in durs.items() if pat in k for d in v
                    if d > 0 and (not shared or 2e12 <= ALGO_BYTES[op] / (d * 1e-6) <= 9e12))
        if not ds:
            continue
        avg = sum(ds) / len(ds)
        gbs = ALGO_BYTES[op] / (avg * 1e-6) / 1e9
        lines.append("| `%s` (%s) | %d | %.1f | %.1f | %.1f | %.1f | %.0f | %.1f |" % (
            pat, op, len(ds), avg, ds[len(ds) // 2], ds[0], ds[-1], gbs,
            100 * gbs / PEAK_HBM_GBS))
    table = "\n".join(lines)
    prof = os.path.dirname(TRAFFIC_FILE)
    with open(os.path.join(prof, "kernels_rowwise_suite.md"), "w") as f:
        f.write("# Kernel durations, row-wise suite (one MI355X)\n\n"
                "Command (`R` the repository root, `OUT` an output directory):\n\n"
                "    cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -f csv "
                "-d $OUT/prof_trace -o trace -- python3 $R/bench.py\n\n"
                "summarised by `python bench.py --ingest-counters "
                "$OUT/prof_trace $OUT/prof_fetch $OUT/prof_write`.\n"
                "GB/s = algorithmic bytes per launch / average kernel duration (the "
                "trace's per-dispatch times).\n\n" + table + "\n")
    tl = ["| op | kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (scaled) | algorithmic bytes | ratio |",
          "|---|---|---|---|---|---|---|"]
    for op, k in kernels.items():
        tl.append("| %s | `%s` | %.1f | %.1f | %d | %d | %.3f |" % (
            op, k["kernel"], k["fetch_kib_raw"], k["write_kib_raw"], k["bytes_per_launch"],
            k["algorithmic_bytes"], k["traffic_over_algorithmic"]))
    cal = out["calibration"]
    with open(os.path.join(prof, "traffic_rowwise_suite.md"), "w") as f:
        f.write("# HBM traffic per launch, row-wise suite (one MI355X)\n\n"
                "Two counter passes, one counter each (`R` the repository root, `OUT` an "
                "output directory):\n\n"
                "    cd /tmp && export TMPDIR=/tmp && timeout -s KILL 240 rocprofv3 --pmc FETCH_SIZE "
                "-f csv -d $OUT/prof_fetch -o fetch -- python3 $R/bench.py --steps 2 "
                "--warmup 1 --no-cpu-baseline --no-parity --calibrate-copy\n"
                "    cd /tmp && export TMPDIR=/tmp && timeout -s KILL 240 rocprofv3 --pmc WRITE_SIZE "
                "-f csv -d $OUT/prof_write -o write -- python3 $R/bench.py --steps 2 "
                "--warmup 1 --no-cpu-baseline --no-parity --calibrate-copy\n\n"
                "Counters are KiB per dispatch (mean over dispatches).  `--calibrate-copy` runs a "
                "plain elementwise pass (torch `neg`) that reads and writes %d bytes; its readings "
                "(FETCH %.1f KiB, WRITE %.1f KiB) give the scale factors %.4f (fetch) and %.4f "
                "(write) applied to every kernel.\n\n" % (
                    cal["copy_bytes_each_way"], cal["copy_fetch_kib_raw"] or 0,
                    cal["copy_write_kib_raw"] or 0, cal["fetch_scale"] or 0, cal["write_scale"] or 0)
                + "\n".join(tl) + "\n\nKernel sources hash: `%s` (bench.py reports `traffic` only "
                "while the sources match).\n" % out["source_hash"])
    return out, table


# SQ counter passes behind profiles/counters_<op>.md (at most 8 SQ counters
# per rocprofv3 run)
SQ_PASSES = (
    ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES",
     "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS", "SQ_WAIT_ANY"),
    ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_ADDR_CONFLICT", "SQ_INSTS_LDS",
     "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY"),
)


def sq_summary(op, dirs):
    """profiles/counters_<op>.md: the mean of every SQ counter over the
    dispatches of op's kernel in the rocprofv3 --pmc output directories."""
    pat = KERNEL_OF_OP[op]
    vals = {}
    for d in dirs:
        for r in _csv_rows(d, "counter_collection.csv"):
            if pat in r["Kernel_Name"]:
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    cmds = "\n".join(
        "    cd /tmp && export TMPDIR=/tmp && timeout -s KILL 120 rocprofv3 --pmc %s -f csv "
        "-d $OUT/sq_%s_%d -o sq -- python3 $R/bench.py --only %s --steps 3 --warmup 0 "
        "--no-parity --no-cpu-baseline" % (" ".join(c), op, i, op) for i, c in enumerate(SQ_PASSES))
    rows = ["| counter | mean per dispatch | dispatches |", "|---|---|---|"]
    for k in sorted(vals):
        rows.append("| %s | %.4g | %d |" % (k, sum(vals[k]) / len(vals[k]), len(vals[k])))
    path = os.path.join(os.path.dirname(TRAFFIC_FILE), "counters_%s.md" % op)
    with open(path, "w") as f:
        f.write("# SQ counters, `%s` (%s, one MI355X)\n\nTwo counter passes (`R` the repository "
                "root, `OUT` an output directory):\n\n%s\n\nsummarised by `python bench.py "
                "--sq-summary %s $OUT/sq_%s_0 $OUT/sq_%s_1`. "
                "Values as rocprofv3 reports them per dispatch (accumulated over the chip); "
                "read them as ratios of one another (bank-conflict cycles against LDS-active "
                "cycles, waiting against wave cycles, instructions per dispatch)."
                "\n\n%s\n\nKernel sources hash: `%s`.\n" % (pat, op, cmds, op, op, op,
                                                             "\n".join(rows), kernel_source_hash()))
    return path


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the operations outside the step (next_rows)")
    ap.add_argument("--only", default=None, help="comma list of ops to run (profiling)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the reference streams (plain read / write / copy of known size)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 512 MiB elementwise copy (negation) three times: "
                         "the known-size reference for scaling FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--sq-summary", nargs="+", metavar="OP_OR_DIR",
                    help="host only: OP then the rocprofv3 --pmc output directories of the "
                         "SQ counter passes; writes profiles/counters_OP.md")
    ap.add_argument("--ingest-counters", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="host only: read rocprofv3 CSV output (kernel stats, FETCH_SIZE run, "
                         "WRITE_SIZE run) and write profiles/traffic.json and summaries")
    return ap.parse_args()


def bf16_ulp_diff(a, b):
    """Distance in bf16 units in the last place (sign-magnitude patterns ordered)."""
    def ordered(u):
        u = u.astype(np.int64) & 0xFFFF
        return np.where(u & 0x8000, -(u & 0x7FFF), u & 0x7FFF)
    return np.abs(ordered(a) - ordered(b))


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


def main():
    args = parse()
    if args.sq_summary:
        print(sq_summary(args.sq_summary[0], args.sq_summary[1:]))
        return
    if args.ingest_counters:
        out, table = ingest_counters(*args.ingest_counters)
        print(json.dumps(out, indent=1))
        print(table)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import split_deterministic_combine_amd as rr
    from split_deterministic_combine_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        # a plain elementwise pass of known size: reads and writes COPY_BYTES once
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    def gpu(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ------------------------------------------------------------ inputs
    t0 = time.time()
    log("generating inputs")
    host = {}
    host["short"] = synth.short_rows()
    host["softmax"] = synth.softmax_rows()
    host["long_f"], host["long_i"] = synth.long_rows()
    host["merge"] = synth.lse_merge()
    if not args.no_next:
        host["softmax_long"] = synth.softmax_long_rows()
        host["layernorm"] = synth.layernorm_rows()
    log("inputs generated in %.1f s" % (time.time() - t0))

    sets = {"short": 5, "softmax": 4, "long_f": 1, "long_i": 1, "merge": 8}
    dx = {}
    base = gpu(host["short"])
    dx["short"] = [base] + [base.clone() for _ in range(sets["short"] - 1)]
    base = gpu(host["softmax"])
    dx["softmax"] = [base] + [base.clone() for _ in range(sets["softmax"] - 1)]
    dx["softmax_out"] = [torch.empty_like(base) for _ in range(sets["softmax"])]
    dx["long_f"] = [gpu(host["long_f"])]
    dx["long_i"] = [gpu(host["long_i"])]
    o, m, l = (gpu(a) for a in host["merge"])
    dx["merge"] = [(o, m, l)] + [(o.clone(), m.clone(), l.clone()) for _ in range(sets["merge"] - 1)]
    dx["merge_out"] = [torch.empty((8, 32, 128, 128), dtype=torch.bfloat16, device=dev)
                       for _ in range(sets["merge"])]
    if not args.no_next:
        base = gpu(host["softmax_long"])
        dx["softmax_long"] = [base] + [base.clone() for _ in range(2)]
        dx["softmax_long_out"] = [torch.empty_like(base) for _ in range(3)]
        xl, gl, bl = host["layernorm"]
        base = gpu(xl)
        dx["layernorm"] = [base] + [base.clone() for _ in range(3)]
        dx["layernorm_out"] = [torch.empty_like(base) for _ in range(4)]
        dx["layernorm_w"] = (gpu(gl), gpu(bl))
        dx["layernorm_stats"] = [(torch.empty(LAYERNORM[0], device=dev),
                                  torch.empty(LAYERNORM[0], device=dev)) for _ in range(4)]
    if not args.no_next:
        # attention inputs drawn on the device (1 GiB of keys and values):
        # standard normal from a seeded generator, rounded to bf16
        ab, ah, asq, ad, an, ap = ATTN
        gen = torch.Generator(device=dev)
        gen.manual_seed(synth.SEED_ATTENTION)
        dx["attn_qkv"] = tuple(torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
                               for shape in ((ab, ah, asq, ad), (ab, ah, an, ad), (ab, ah, an, ad)))
        arows = ab * ah * asq
        dx["attn_out"] = (torch.empty((ap, arows, ad), device=dev), torch.empty((ap, arows), device=dev),
                          torch.empty((ap, arows), device=dev))
        dx["attn_merged"] = torch.empty((arows, ad), dtype=torch.bfloat16, device=dev)
        dx["attn_fused"] = torch.empty((ab, ah, asq, ad), dtype=torch.bfloat16, device=dev)
        dx["attn_ws"] = torch.zeros(rr.splitk_attention_workspace_bytes(ab, ah, ah, asq, an, ad, ap),
                                    dtype=torch.uint8, device=dev)
        # packed sequences: q [tokens, heads, depth], k / v [key tokens, heads,
        # depth], standard normal rounded to bf16, int32 token offsets
        gen.manual_seed(synth.SEED_ATTENTION + 1)
        tq, tk = ab * asq, sum(ATTN_VARLEN_K)
        dx["varlen_qkv"] = tuple(torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
                                 for shape in ((tq, ah, ad), (tk, ah, ad), (tk, ah, ad)))
        dx["varlen_cu"] = tuple(
            torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
            for lens in ([asq] * ab, list(ATTN_VARLEN_K)))
        dx["varlen_out"] = (torch.empty((ap, tq, ah, ad), device=dev),
                            torch.empty((ap, tq, ah), device=dev), torch.empty((ap, tq, ah), device=dev))
    if not args.no_next:
        # odd-stride rows and their aligned neighbours, drawn on the device
        # (standard normal, seeded); three sets each, so that consecutive
        # launches of one op touch well over the 256 MB of last-level cache
        gen = torch.Generator(device=dev)
        gen.manual_seed(9)
        for key, shape, dt in (("sum_47", (1048576, 47), torch.float32),
                               ("sum_1001", (65536, 1001), torch.float32),
                               ("sum_1000", (65536, 1000), torch.float32),
                               ("softmax_8191", (8192, 8191), torch.bfloat16)):
            dx[key] = [torch.randn(shape, generator=gen, device=dev).to(dt) for _ in range(3)]
        dx["softmax_8191_out"] = [torch.empty_like(dx["softmax_8191"][0]) for _ in range(3)]
        dx["sum_47_out"] = torch.empty(1048576, device=dev)
        dx["sum_1001_out"] = torch.empty(65536, device=dev)
    y_short_sum = torch.empty(1048576, dtype=torch.float32, device=dev)
    y_short_max = torch.empty(1048576, dtype=torch.float32, device=dev)
    y_long_f = torch.empty(16, dtype=torch.float32, device=dev)
    y_long_i = torch.empty(16, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    # algorithmic bytes per launch (inputs read once, outputs written once)
    B = _algo_bytes()
    ops = {
        "short_sum": lambda i: rr.reduce_rows(dx["short"][i % 5], "sum", out=y_short_sum),
        "short_max": lambda i: rr.reduce_rows(dx["short"][i % 5], "max", out=y_short_max),
        "softmax": lambda i: rr.softmax_rows(dx["softmax"][i % 4], out=dx["softmax_out"][i % 4]),
        "long_sum": lambda i: rr.reduce_rows(dx["long_f"][0], "sum", out=y_long_f),
        "long_max": lambda i: rr.reduce_rows(dx["long_i"][0], "max", out=y_long_i),
        "merge": lambda i: rr.splitk_lse_merge(*dx["merge"][i % 8], 1.0, torch.bfloat16,
                                               out=dx["merge_out"][i % 8]),
    }
    y_multi = {k: torch.empty(16, dtype=torch.float32, device=dev) for k in ("sum", "max", "min")}
    y_cols = torch.empty(16384, dtype=torch.float32, device=dev)
    next_ops = {
        "multi_long": lambda i: rr.reduce_rows_multi(dx["long_f"][0], out=y_multi),
        "axis_cols": lambda i: rr.reduce_axis(dx["long_f"][0].view(16384, 16384), 0, "sum",
                                              out=y_cols),
        "softmax_long": lambda i: rr.softmax_rows(dx["softmax_long"][i % 3],
                                                  out=dx["softmax_long_out"][i % 3]),
        "layernorm": lambda i: rr.layernorm_rows(dx["layernorm"][i % 4], *dx["layernorm_w"], 1e-5,
                                                 out=dx["layernorm_out"][i % 4],
                                                 mean_out=dx["layernorm_stats"][i % 4][0],
                                                 rstd_out=dx["layernorm_stats"][i % 4][1]),
        "attention": lambda i: rr.splitk_attention_partials(*dx["attn_qkv"], ATTN[5],
                                                            out=dx["attn_out"]),
        # the whole split-K attention: the partials above, then their LSE merge
        "attention_merged": lambda i: rr.splitk_lse_merge(
            *rr.splitk_attention_partials(*dx["attn_qkv"], ATTN[5], out=dx["attn_out"]), 1.0,
            torch.bfloat16, out=dx["attn_merged"]),
        # both in one launch, the partials combined by the last workgroup of each tile
        "attention_fused": lambda i: rr.splitk_attention(*dx["attn_qkv"], ATTN[5],
                                                         out=dx["attn_fused"],
                                                         workspace=dx["attn_ws"]),
        # the partials of packed sequences of mixed key lengths
        "attention_varlen": lambda i: rr.splitk_attention_partials_varlen(
            *dx["varlen_qkv"], *dx["varlen_cu"], ATTN[2], ATTN[5], out=dx["varlen_out"]),
        "sum_47": lambda i: rr.reduce_rows(dx["sum_47"][i % 3], "sum", out=dx["sum_47_out"]),
        "sum_1001": lambda i: rr.reduce_rows(dx["sum_1001"][i % 3], "sum", out=dx["sum_1001_out"]),
        "sum_1000": lambda i: rr.reduce_rows(dx["sum_1000"][i % 3], "sum", out=dx["sum_1001_out"]),
        "softmax_8191": lambda i: rr.softmax_rows(dx["softmax_8191"][i % 3],
                                                  out=dx["softmax_8191_out"][i % 3]),
    }
    only = args.only.split(",") if args.only else None
    names = [n for n in ops if only is None or n in only]
    next_names = [] if args.no_next else [n for n in next_ops if only is None or n in only]

    # ------------------------------------------------------------ parity
    parity = "skipped"
    bit_identical = None
    if not args.no_parity:
        import oracle

        log("parity check on sampled rows")
        for n in names:
            ops[n](0)
        for n in next_names:
            next_ops[n](0)
        torch.cuda.synchronize()
        ok = True
        if "softmax_long" in next_names:
            pick = [0, SOFTMAX_LONG[0] - 1]
            y = dx["softmax_long_out"][0][pick].cpu().view(torch.int16).numpy().view(np.uint16)
            r = oracle.softmax_rows(np.ascontiguousarray(host["softmax_long"][pick]), "bf16")
            ok &= bool(bf16_ulp_diff(y, r).max() <= 1)
        if "axis_cols" in next_names:
            r = oracle.reduce_axis(host["long_f"].reshape(1, 16384, 16384), "sum")[0]
            y = y_cols.cpu().numpy()
            ok &= bool(np.all(np.abs(y - r) <= 1e-6 + 1e-5 * np.abs(r)))
        if "multi_long" in next_names:
            for k in ("sum", "max", "min"):
                y = y_multi[k][:2].cpu().numpy()
                r = oracle.reduce_rows(host["long_f"][:2], k)
                ok &= bool(np.all(np.abs(y - r) <= 1e-6 + 1e-5 * np.abs(r)) if k == "sum"
                           else np.array_equal(y, r))
        if "layernorm" in next_names:
            xl, gl, bl = host["layernorm"]
            pick = np.linspace(0, LAYERNORM[0] - 1, 8).astype(np.int64)
            y = dx["layernorm_out"][0][pick].cpu().view(torch.int16).numpy().view(np.uint16)
            r, rm, rs = oracle.layernorm_rows(np.ascontiguousarray(xl[pick]), gl, bl, 1e-5, "bf16")
            yv = (y.astype(np.uint32) << 16).view(np.float32)
            rv = (r.astype(np.uint32) << 16).view(np.float32)
            # 1 bf16 ulp, or the float32 bar's absolute 1e-6 (cancellation near zero)
            ok &= bool(np.all((bf16_ulp_diff(y, r) <= 1) | (np.abs(yv - rv) <= 1e-6)))
            gm = dx["layernorm_stats"][0][0][pick].cpu().numpy()
            gs = dx["layernorm_stats"][0][1][pick].cpu().numpy()
            ok &= bool(np.all(np.abs(gm - rm) <= 1e-6 + 1e-5 * np.abs(rm)))
            ok &= bool(np.all(np.abs(gs - rs) <= 1e-6 + 1e-5 * np.abs(rs)))
        if "attention" in next_names:
            # one head against the oracle; bound from the kernel's arithmetic
            # (bf16 probabilities: 2^-8 of the weighted |v|, plus float32 terms)
            ab, ah, asq, ad, an, ap = ATTN
            bh = (ab - 1, ah - 1)
            bits = [t[bh[0]:bh[0] + 1, bh[1]:bh[1] + 1].contiguous().cpu().view(torch.int16)
                    .numpy().view(np.uint16) for t in dx["attn_qkv"]]
            sc = 1.0 / math.sqrt(ad)
            o_r, m_r, l_r = oracle.attention_partials(*bits, ap, sc)
            o_a, _, _ = oracle.attention_partials(bits[0], bits[1], bits[2] & np.uint16(0x7FFF),
                                                  ap, sc)
            rows = slice((bh[0] * ah + bh[1]) * asq, (bh[0] * ah + bh[1] + 1) * asq)
            og = dx["attn_out"][0][:, rows].cpu().numpy()
            mg = dx["attn_out"][1][:, rows].cpu().numpy()
            ok &= bool(np.all(np.abs(og - o_r) <= (2.0 ** -8 + 2.0 ** -12) * o_a + 1e-6))
            ok &= bool(np.all(np.abs(mg - m_r) <= 1e-5 * (1 + np.abs(m_r))))
        if "attention_varlen" in next_names:
            # the last sequence (the most keys) at its last head against the
            # oracle, with the dense row's bound
            ab, ah, asq, ad, an, ap = ATTN
            sb, hh = ab - 1, ah - 1
            q0, k0 = sb * asq, sum(ATTN_VARLEN_K[:sb])
            nk = ATTN_VARLEN_K[sb]
            qv, kv, vv = dx["varlen_qkv"]
            bits = [t[a:a + n, hh:hh + 1].contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
                    for t, a, n in ((qv, q0, asq), (kv, k0, nk), (vv, k0, nk))]
            cq, ck = np.array([0, asq], np.int32), np.array([0, nk], np.int32)
            sc = 1.0 / math.sqrt(ad)
            o_r, m_r, _ = oracle.attention_partials_varlen(*bits, cq, ck, ap, sc)
            o_a, _, _ = oracle.attention_partials_varlen(bits[0], bits[1], bits[2] & np.uint16(0x7FFF),
                                                         cq, ck, ap, sc)
            og = dx["varlen_out"][0][:, q0:q0 + asq, hh].cpu().numpy()
            mg = dx["varlen_out"][1][:, q0:q0 + asq, hh].cpu().numpy()
            ok &= bool(np.all(np.abs(og - o_r) <= (2.0 ** -8 + 2.0 ** -12) * o_a + 1e-6))
            ok &= bool(np.all(np.abs(mg - m_r) <= 1e-5 * (1 + np.abs(m_r))))
        if "attention_fused" in next_names and "attention_merged" in next_names:
            # the one-launch attention gives the bits of partials + merge
            ok &= bool(torch.equal(dx["attn_fused"].view(-1).view(torch.int16),
                                   dx["attn_merged"].view(-1).view(torch.int16)))
        # sampled rows of the full-size outputs of the pass above (no extra launches)
        xs = host["short"][:4096]
        if "short_sum" in names:
            y = y_short_sum[:4096].cpu().numpy()
            r = oracle.reduce_rows(xs, "sum")
            ok &= bool(np.all(np.abs(y - r) <= 1e-6 + 1e-5 * np.abs(r)))
        if "short_max" in names:
            ok &= bool(np.array_equal(y_short_max[:4096].cpu().numpy(), oracle.reduce_rows(xs, "max")))
        if "long_sum" in names:
            y = y_long_f.cpu().numpy()
            r = oracle.reduce_rows(host["long_f"][:2], "sum")
            ok &= bool(np.all(np.abs(y[:2] - r) <= 1e-6 + 1e-5 * np.abs(r)))
        if "long_max" in names:
            ok &= bool(np.array_equal(y_long_i.cpu().numpy()[:2], oracle.reduce_rows(host["long_i"][:2], "max")))
        if "softmax" in names:
            y = dx["softmax_out"][0][:8].cpu().view(torch.int16).numpy().view(np.uint16)
            r = oracle.softmax_rows(host["softmax"][:8], "bf16")
            ok &= bool(bf16_ulp_diff(y, r).max() <= 1)
        if "merge" in names:
            oh, mh, lh = host["merge"]
            y = dx["merge_out"][0].reshape(-1, 128)[:256].cpu().view(torch.int16).numpy().view(np.uint16)
            r = oracle.splitk_lse_merge(np.ascontiguousarray(oh.reshape(8, -1, 128)[:, :256]),
                                        np.ascontiguousarray(mh.reshape(8, -1)[:, :256]),
                                        np.ascontiguousarray(lh.reshape(8, -1)[:, :256]), 1.0, "bf16")
            ok &= bool(bf16_ulp_diff(y, r).max() <= 1)
        # run-to-run bit identity: each step op again into the same outputs
        outs = {"short_sum": lambda: y_short_sum, "short_max": lambda: y_short_max,
                "softmax": lambda: dx["softmax_out"][0], "long_sum": lambda: y_long_f,
                "long_max": lambda: y_long_i, "merge": lambda: dx["merge_out"][0]}
        first = {n: outs[n]().clone() for n in names}
        for n in names:
            ops[n](0)
        torch.cuda.synchronize()
        same = all(torch.equal(first[n].view(torch.int16) if first[n].element_size() == 2
                               else first[n].view(torch.int32),
                               outs[n]().view(torch.int16) if first[n].element_size() == 2
                               else outs[n]().view(torch.int32)) for n in names)
        ok &= same
        bit_identical = same
        parity = "ok" if ok else "FAILED"
        log("parity %s (repeat bit-identical: %s)" % (parity, same))
        if not ok:
            sys.exit(1)

    # ------------------------------------------------------------ timing
    stream = torch.cuda.current_stream(dev)

    def instrumented(nsteps, first):
        """Run nsteps steps with HIP events around every launch; per-op durations (ms)."""
        evs = {n: [] for n in names}
        for i in range(first, first + nsteps):
            for n in names:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                ops[n](i)
                b.record(stream)
                evs[n].append((a, b))
        torch.cuda.synchronize()
        return {n: [a.elapsed_time(b) for a, b in evs[n]] for n in names}

    # Warmup with every launch instrumented.  The dominant op is the one that
    # moves the most algorithmic bytes (every op is HBM-bound, so it is also
    # the longest); the first in step order on a tie (the f32 and i32 long-row
    # reductions move the same bytes), so the choice does not flip between runs.
    if not names and next_names:
        # a profiling run of operations outside the step (under rocprofv3):
        # each selected one launched warmup + steps times in a row, as the
        # next-row timing below runs them; nothing is timed
        for n in next_names:
            for i in range(args.warmup + args.steps):
                next_ops[n](i)
        torch.cuda.synchronize()
        print(json.dumps({"profile_run": next_names, "launches_each": args.warmup + args.steps}))
        return
    log("warmup %d steps" % args.warmup)
    if not names:
        sys.exit("bench.py: --only selected no operation of the step")
    # no garbage-collection pause of the host may hold back the launches the
    # HIP events time (the launches run at most a few steps ahead of it)
    gc.disable()
    instrumented(max(args.warmup, 1), 0)
    dom = max(names, key=lambda n: (B[n], -names.index(n)))

    # Timed region: exactly K steps; HIP events only around the dominant op
    # (an event pair costs a few microseconds of GPU time, so instrumenting
    # every launch would inflate the step).
    K = args.steps
    ev_dom = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(K)]
    log("timing %d steps" % K)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        for n in names:
            if n == dom:
                a, b = ev_dom[i]
                a.record(stream)
                ops[n](i)
                b.record(stream)
            else:
                ops[n](i)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    ms_per_step = t_total * 1e3 / K
    dom_ms = [a.elapsed_time(b) for a, b in ev_dom]

    # Per-op breakdown from a separate instrumented pass (not part of the timing).
    brk = instrumented(max(K, 10), K)
    per_op = {}
    for n in names:
        ts = sorted(dom_ms if n == dom else brk[n])
        mean = sum(ts) / len(ts)
        med = ts[len(ts) // 2]
        # rates from the median launch (mean, min and p90 beside it); the
        # roofline below divides by the mean launch instead
        per_op[n] = {"ms_mean": round(mean, 5), "ms_median": round(med, 5),
                     "ms_min": round(ts[0], 5),
                     "ms_p90": round(ts[min(len(ts) - 1, (9 * len(ts)) // 10)], 5), "bytes": B[n],
                     "GBps": round(B[n] / (med * 1e-3) / 1e9, 1),
                     "pct_peak": round(100 * B[n] / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 1),
                     "timed_in": "timed region" if n == dom else "instrumented pass"}
    # Operations outside the step: each timed alone with HIP events on the
    # stream -- its warmup launches, then its timed launches in a row (every
    # op rotates buffer sets larger than the last-level cache), before the
    # next op starts.
    next_rows = {}
    if next_names:
        log("timing next-row operations")
        reps = max(K, 10)
        evs = {n: [] for n in next_names}
        run_evs = {}
        for n in next_names:
            # warmup: at least --warmup launches and 20 ms of them, so that the
            # clocks have settled for the op before its timed launches
            t_w, i = time.perf_counter(), 0
            while i < max(args.warmup, 1) or time.perf_counter() - t_w < 0.02:
                next_ops[n](i)
                i += 1
                if i % 4 == 0:
                    torch.cuda.synchronize()
            torch.cuda.synchronize()
            for i in range(reps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                next_ops[n](i)
                b.record(stream)
                evs[n].append((a, b))
            # then the same launches back to back between one pair of events:
            # the sustained rate (no event between launches; clocks under
            # continuous load)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in range(reps):
                next_ops[n](i)
            b.record(stream)
            run_evs[n] = (a, b)
            torch.cuda.synchronize()
        for n in next_names:
            ts = sorted(a.elapsed_time(b) for a, b in evs[n])
            mean = sum(ts) / len(ts)
            med = ts[len(ts) // 2]
            gbs = NEXT_BYTES[n] / (med * 1e-3) / 1e9
            run_ms = run_evs[n][0].elapsed_time(run_evs[n][1]) / reps
            next_rows[n] = {"ms_mean": round(mean, 5), "ms_median": round(med, 5),
                            "ms_min": round(ts[0], 5), "bytes": NEXT_BYTES[n],
                            "GBps": round(gbs, 1), "pct_peak": round(100 * gbs / PEAK_HBM_GBS, 1),
                            "ms_back_to_back": round(run_ms, 5),
                            "pct_peak_back_to_back": round(
                                100 * NEXT_BYTES[n] / (run_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 1)}
        cu = rr.device_cu_count()
        if "axis_cols" in next_rows:
            pa = rr.plan_axis(1, 16384, 16384, torch.float32, "sum", cu_count=cu)
            next_rows["axis_cols"].update({
                "config": "f32 column sums of [16384, 16384] (reduce over a non-last axis), "
                          "split-K: %d slices, %d workgroups" % (pa["slices"], pa["grid"]),
                "kernels": [KERNEL_OF_OP["axis_cols_partial"], KERNEL_OF_OP["axis_cols_fold"]]})
        if "multi_long" in next_rows:
            pm = rr.plan_reduce(16, 1 << 24, torch.float32, "sum_max_min", cu_count=cu)
            next_rows["multi_long"].update({
                "config": "f32 sum, max and min over [16, 16777216] from one read, split-K "
                          "(G = %d, 16-byte partials)" % pm["slices"],
                "kernels": [KERNEL_OF_OP["multi_long"]]})
        if "layernorm" in next_rows:
            next_rows["layernorm"].update({
                "config": "bf16 layernorm [%d, %d] -> bf16, float32 gamma/beta, float32 "
                          "mean/rstd, block tier (persistent)" % LAYERNORM,
                "kernels": [KERNEL_OF_OP["layernorm"]]})
        if "attention" in next_rows:
            ab, ah, asq, ad, an, ap = ATTN
            t_s = next_rows["attention"]["ms_median"] * 1e-3
            next_rows["attention"].update({
                "config": "split-K attention partials: bf16 q [%d, %d, %d, %d], k and v over %d "
                          "keys in %d partitions -> float32 O, m, l (matrix cores, "
                          "v_mfma_f32_32x32x16_bf16)" % (ab, ah, asq, ad, an, ap),
                "kernels": [KERNEL_OF_OP["attention"]],
                "flops": _attn_flops(),
                "TFLOPs": round(_attn_flops() / t_s / 1e12, 1),
                "pct_peak_bf16_mfma": round(100 * _attn_flops() / t_s / 2.5e15, 1)})
        if "attention_varlen" in next_rows:
            ab, ah, asq, ad, an, ap = ATTN
            t_s = next_rows["attention_varlen"]["ms_median"] * 1e-3
            next_rows["attention_varlen"].update({
                "config": "split-K attention partials of %d packed sequences of %d queries, key "
                          "lengths %s, %d heads of depth %d, %d partitions per sequence -> float32 "
                          "O, m, l placed by (token, head)" % (ab, asq, list(ATTN_VARLEN_K), ah,
                                                               ad, ap),
                "kernels": [KERNEL_OF_OP["attention_varlen"]],
                "flops": _attn_flops(),
                "TFLOPs": round(_attn_flops() / t_s / 1e12, 1)})
            if "attention" in next_rows:
                next_rows["attention_varlen"]["frac_of_dense"] = round(
                    next_rows["attention"]["ms_median"] / next_rows["attention_varlen"]["ms_median"], 4)
        if "attention_merged" in next_rows:
            ab, ah, asq, ad, an, ap = ATTN
            t_s = next_rows["attention_merged"]["ms_median"] * 1e-3
            next_rows["attention_merged"].update({
                "config": "split-K attention end to end: the partials above, then their LSE merge "
                          "into bf16 [%d, %d, %d, %d] (two launches)" % (ab, ah, asq, ad),
                "kernels": [KERNEL_OF_OP["attention"], KERNEL_OF_OP["merge"]],
                "flops": _attn_flops(),
                "TFLOPs": round(_attn_flops() / t_s / 1e12, 1),
                "bytes_note": "bytes = q, k, v read once and the bf16 output written once; the "
                              "partials (130 MiB) go through HBM between the launches"})
        if "attention_fused" in next_rows:
            ab, ah, asq, ad, an, ap = ATTN
            t_s = next_rows["attention_fused"]["ms_median"] * 1e-3
            next_rows["attention_fused"].update({
                "config": "split-K attention in one launch: the partials of every (head, 128 "
                          "query rows) folded in partition order by the last of its %d "
                          "workgroups into bf16 [%d, %d, %d, %d]" % (ap, ab, ah, asq, ad),
                "kernels": [KERNEL_OF_OP["attention_fused"]],
                "flops": _attn_flops(),
                "TFLOPs": round(_attn_flops() / t_s / 1e12, 1),
                "bytes_note": "bytes = q, k, v read once and the bf16 output written once; the "
                              "partials go through the device-coherent level once each way"})
        for n, nb in NEIGHBOUR.items():
            if n in next_rows:
                ref = next_rows.get(nb) or per_op.get(nb)
                next_rows[n]["aligned_neighbour"] = nb
                if ref:
                    next_rows[n]["frac_of_neighbour"] = round(next_rows[n]["GBps"] / ref["GBps"], 4)
        for n, cfg in (("sum_47", "f32 row sum [1048576, 47] (row stride 47: rows at every "
                                  "offset from a 16-byte boundary), wave tier"),
                       ("sum_1001", "f32 row sum [65536, 1001] (odd row stride), block tier, "
                                    "persistent rows"),
                       ("sum_1000", "f32 row sum [65536, 1000] (aligned rows), block tier, "
                                    "persistent rows"),
                       ("softmax_8191", "bf16 softmax [8192, 8191] -> bf16 (odd row stride), "
                                        "block tier, persistent rows")):
            if n in next_rows:
                next_rows[n]["config"] = cfg
        if "softmax_long" in next_rows:
            r, c = SOFTMAX_LONG
            next_rows["softmax_long"].update({
                "config": "bf16 softmax [%d, %d] -> bf16, split-K tier (G = %d)" % (
                    r, c, rr.plan_softmax(r, c, cu_count=cu)["slices"]),
                "kernels": [KERNEL_OF_OP["softmax_long_stats"], KERNEL_OF_OP["softmax_long_map"]],
                "bytes_note": "bytes = x read once + y written once; the two-launch design reads "
                              "x twice (%d bytes moved)" % (B["softmax_long_stats"]
                                                            + B["softmax_long_map"])})

    # ------------------------------------------- achievable-bandwidth reference
    # Plain 128-bit non-temporal streams with no arithmetic (rr_test_stream):
    # what HBM delivers to a kernel that does nothing but move bytes, beside
    # the published 8 TB/s.  Read: the two 1 GiB long-row inputs alternated,
    # and the merge's 128 MiB inputs; copy: softmax-shaped 128 MiB -> 128 MiB
    # over the four softmax buffer sets, and 512 MiB -> 512 MiB; write: 1 GiB.
    ceilings = None
    if not args.no_ceilings:
        log("timing the reference streams")
        big = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        src_big = dx["long_f"][0].view(-1).view(torch.uint8)
        runs = {
            "read_1GiB": (1 << 30, lambda i: rr._test_stream(
                "read", (dx["long_f"][0] if i % 2 == 0 else dx["long_i"][0]))),
            "write_1GiB": (1 << 30, lambda i: rr._test_stream("write", None, big)),
            "copy_512MiB_each_way": (1 << 30, lambda i: rr._test_stream(
                "copy", src_big[:1 << 29], big[(i % 2) << 29:((i % 2) + 1) << 29])),
            "copy_128MiB_each_way": (1 << 28, lambda i: rr._test_stream(
                "copy", dx["softmax"][i % 4], dx["softmax_out"][i % 4])),
            # the LSE merge's partial outputs (128 MiB, the merge's eight sets
            # in turn): a kernel of the merge's size has a larger fixed share
            # (launch, ramp, drain) than a 1 GiB pass
            "read_128MiB": (1 << 27, lambda i: rr._test_stream(
                "read", dx["merge"][i % 8][0])),
        }
        ceilings = {}
        for name, (nbytes, fn) in runs.items():
            evs = []
            for i in range(23):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn(i)
                b.record(stream)
                if i >= 3:
                    evs.append((a, b))
            torch.cuda.synchronize()
            ts = sorted(a.elapsed_time(b) for a, b in evs)
            med = ts[len(ts) // 2]
            gbs = nbytes / (med * 1e-3) / 1e9
            ceilings[name] = {"ms_median": round(med, 5), "bytes": nbytes, "GBps": round(gbs, 1),
                              "pct_peak": round(100 * gbs / PEAK_HBM_GBS, 1)}
        del big
        torch.cuda.empty_cache()

    step_bytes = sum(B[n] for n in names)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # dominant kernel: the launch with the largest share of the step
    # achieved: algorithmic bytes over the dominant kernel's mean launch
    # duration in the timed region (HIP events on its stream)
    achieved = round(B[dom] / (per_op[dom]["ms_mean"] * 1e-3) / 1e9, 1)
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        ent = tr.get("kernels", {}).get(dom)
        if ent and tr.get("source_hash") == kernel_source_hash():
            traffic = ent.get("bytes_per_launch")
    if ceilings:
        # each step op beside the reference stream closest to its size and mix
        for n, ref in (("softmax", "copy_128MiB_each_way"), ("long_sum", "read_1GiB"),
                       ("long_max", "read_1GiB"), ("merge", "read_128MiB")):
            if n in per_op and ref in ceilings:
                per_op[n]["reference_stream"] = ref
                per_op[n]["frac_of_reference"] = round(per_op[n]["GBps"] / ceilings[ref]["GBps"], 4)
    roofline = {"bound": "hbm", "kernel": dom, "kernel_symbol": KERNEL_OF_OP[dom],
                "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "algorithmic_bytes": B[dom]}
    if ceilings:
        # the reference stream with the dominant kernel's mix of reads and writes
        ref = "copy_128MiB_each_way" if dom == "softmax" else "read_1GiB"
        roofline["reference_stream"] = ref
        roofline["reference_GBps"] = ceilings[ref]["GBps"]
        roofline["frac_of_reference"] = round(achieved / ceilings[ref]["GBps"], 4)

    # ------------------------------------------------------------ CPU baseline
    cpu = None
    gc.enable()  # the GPU timing is over
    if not args.no_cpu_baseline:
        import oracle

        log("timing the oracle on a sample")
        sample = {"short_rows": 1048576, "softmax_rows": 8192, "long_rows": 16, "lse_merge_rows": 32768}
        oh, mh, lh = host["merge"]
        o_s = np.ascontiguousarray(oh.reshape(8, -1, 128)[:, :sample["lse_merge_rows"]])
        m_s = np.ascontiguousarray(mh.reshape(8, -1)[:, :sample["lse_merge_rows"]])
        l_s = np.ascontiguousarray(lh.reshape(8, -1)[:, :sample["lse_merge_rows"]])
        xs = host["short"][:sample["short_rows"]]
        xsm = host["softmax"][:sample["softmax_rows"]]
        xlf = host["long_f"][:sample["long_rows"]]
        xli = host["long_i"][:sample["long_rows"]]
        nb = (2 * (xs.nbytes + 4 * xs.shape[0]) + 2 * xsm.nbytes + xlf.nbytes + 4 + xli.nbytes + 4
              + o_s.nbytes + m_s.nbytes + l_s.nbytes + o_s.shape[1] * 128 * 2)

        def oracle_step(jobs, pool=None):
            """One full step: every (function, args) job; on a pool when given."""
            c0 = time.perf_counter()
            if pool is None:
                for fn, a in jobs:
                    fn(*a)
            else:
                list(pool.map(lambda j: j[0](*j[1]), jobs))
            return time.perf_counter() - c0

        def step_jobs(blocks):
            """The step's oracle calls, each op's rows cut into `blocks` contiguous blocks
            (rows are independent, so the blocks together compute the same rows)."""
            def cut(n):
                k = min(blocks, n)
                return [(n * b // k, n * (b + 1) // k) for b in range(k)]
            jobs = []
            for a, b in cut(xs.shape[0]):
                jobs += [(oracle.reduce_rows, (xs[a:b], "sum")), (oracle.reduce_rows, (xs[a:b], "max"))]
            for a, b in cut(xsm.shape[0]):
                jobs.append((oracle.softmax_rows, (xsm[a:b], "bf16")))
            for a, b in cut(xlf.shape[0]):
                jobs += [(oracle.reduce_rows, (xlf[a:b], "sum")), (oracle.reduce_rows, (xli[a:b], "max"))]
            for a, b in cut(o_s.shape[1]):
                jobs.append((oracle.splitk_lse_merge,
                             (np.ascontiguousarray(o_s[:, a:b]), np.ascontiguousarray(m_s[:, a:b]),
                              np.ascontiguousarray(l_s[:, a:b]), 1.0, "bf16")))
            return jobs

        # one core: one full step of the oracle, repeated until ~10 s (at most 8 times)
        jobs1 = step_jobs(1)
        reps, c_s = 0, 0.0
        while reps < 8 and c_s < 10.0:
            c_s += oracle_step(jobs1)
            reps += 1
        c_s /= reps
        # T threads over rows (ctypes releases the GIL inside each oracle call); T is
        # the host CPUs this process may use, at most 16 (one GPU's share of the host)
        from concurrent.futures import ThreadPoolExecutor
        T = max(1, min(len(os.sched_getaffinity(0)), 16))
        jobsT = step_jobs(T)
        with ThreadPoolExecutor(max_workers=T) as pool:
            oracle_step(jobsT, pool)  # warm the pool and the page cache
            reps_t, c_t = 0, 0.0
            while reps_t < 8 and c_t < 5.0:
                c_t += oracle_step(jobsT, pool)
                reps_t += 1
        c_t /= reps_t
        sample = ("one full step of the same workload (short_rows %d of 1048576 rows sum+max, "
                  "softmax %d of 8192 rows, long_rows %d of 16 rows f32 sum + i32 max, "
                  "lse_merge %d of 32768 rows); the C oracle on %d threads, each op's rows cut "
                  "into %d contiguous blocks (the long-row op has 16 rows, so at most 16 threads "
                  "work on it)" % (sample["short_rows"], sample["softmax_rows"], sample["long_rows"],
                                   sample["lse_merge_rows"], T, T))
        cpu = {"value": round(nb / c_t / 1e9, 3), "unit": "GB/s", "cores": T, "kind": "oracle",
               "sample": sample, "seconds_per_step": round(c_t, 3), "repetitions": reps_t,
               "single_core": {"value": round(nb / c_s / 1e9, 3), "unit": "GB/s", "cores": 1,
                               "seconds_per_step": round(c_s, 3), "repetitions": reps}}

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32/f64 acc, bf16 io, i32",
        "data": "synthetic (seeded generators in split_deterministic_combine_amd/synth.py)",
        "config": {"workload": "rowwise suite: f32 sum+max [1048576,48] wave tier; bf16 softmax "
                               "[8192,8192] block tier; f32 sum + i32 max [16,2^24] split-K; "
                               "LSE merge P=8 O[8,32,128,128] -> bf16",
                   "ops": names, "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBS, 1),
                   "step_bytes": step_bytes, "parity": parity,
                   "repeat_bit_identical": bit_identical},
        "per_op": per_op,
        "next_rows": next_rows,
        "roofline": roofline,
        "reference_streams": ceilings,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
