"""C-ABI checks that need no GPU: the library loads, exports every symbol the
headers declare, plans tiers by the documented rule and rejects bad
arguments before it touches the device."""
import ctypes
import os
import subprocess
import re

import pytest
import torch

import split_deterministic_combine_amd as rr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("rr.h", "rr_test.h")]


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(rr_[a-z0-9_]+)\s*\(", text):
            names.add(m.group(1))
    return sorted(names)


def test_library_is_built_for_gfx950_and_loads():
    assert os.path.exists(rr.lib_path()), "run python -m split_deterministic_combine_amd.build"
    lib = ctypes.CDLL(rr.lib_path())
    assert lib.rr_version() == 1
    blob = open(rr.lib_path(), "rb").read()
    assert b"gfx950" in blob


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(rr.lib_path())
    declared = _declared_functions()
    assert {"rr_reduce_rows", "rr_softmax_rows", "rr_splitk_lse_merge"} <= set(declared)
    missing = [n for n in declared if not hasattr(lib, n)]
    assert not missing, missing


def test_plain_c_consumer_compiles_links_and_runs(tmp_path):
    # rr.h is a C header: a C11 program includes it, links librr.so and calls
    # the host-only entry points
    exe = str(tmp_path / "abi_consumer")
    libdir = os.path.dirname(rr.lib_path())
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_consumer.c"),
           "-o", exe, "-L", libdir, "-l:librr.so", "-Wl,-rpath," + libdir]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    assert "reduce tier=5 slices=32 grid=512 ws=4352" in out
    assert "softmax tier=2 block=256 grid=512" in out
    assert "layernorm tier=2 block=128 grid=1024" in out
    assert "axis tier=5 slices=2" in out
    assert "bad ld -> 2 (invalid shape" in out
    assert "empty softmax -> 0" in out and "P=0 merge -> 2" in out
    assert "noalloc bad ld -> 2" in out
    assert "varlen without buffers -> 1" in out
    assert "varlen heads not a multiple of kv heads -> 2" in out
    # one 4-byte ticket per (head, 128 query rows): 256 groups, 1024 bytes
    assert re.search(r"attention workspace 0 \d+ 1024\b", out), out


@pytest.mark.parametrize("rows,cols,op,block,lanes,grid", [
    (65536, 1000, "sum", 64, 0, 4096),    # 250 chunks: 64 threads x 4, 16 per CU
    (1024, 8192, "max", 512, 0, 512),     # 2048 chunks: 512 threads x 4, 2 per CU
    (20000, 65, "min", 64, 16, 4096),     # 17 chunks: 16 lanes x 4 per row, 4 rows a step
    (6000, 500, "sum", 64, 32, 3000),     # 125 chunks: 32 lanes x 4 per row, 2 rows a step
    (1023, 1000, "sum", 256, 0, 1023),    # fewer than 4 rows per CU: a workgroup per row
    (65536, 8193, "sum", 256, 0, 65536),  # beyond 2048 chunks
    (65536, 1000, "sum_max_min", 64, 0, 4096),   # the three statistics alike
])
def test_block_tier_reduce_persistent_plan(rows, cols, op, block, lanes, grid):
    p = rr.plan_reduce(rows, cols, torch.float32, op, cu_count=256)
    assert (p["tier"], p["block"], p["lanes_per_row"], p["grid"]) == \
        ("block", block, lanes, grid), p


def test_status_strings_are_distinct():
    lib = ctypes.CDLL(rr.lib_path())
    lib.rr_status_string.restype = ctypes.c_char_p
    texts = {lib.rr_status_string(s) for s in range(9)}
    assert len(texts) == 9 and all(texts)


# ------------------------------------------------------------- tier rules

@pytest.mark.parametrize("rows,cols,tier", [
    (64, 1024, "block"),           # small rows
    (1048576, 48, "wave"),         # short rows
    (16, 1 << 24, "splitk"),       # rows < CU and long rows
    (255, 65536, "splitk"),
    (256, 65536, "block"),         # rows == CU: not split-K
    (100, 65535, "block"),         # too short for split-K
    (1000, 8, "tiled"),
    (1000, 1, "tiled"),
    (1000, 9, "wave"),
    (1000, 64, "wave"),
    (1000, 65, "block"),
    (3, 0, "tiled"),
])
def test_auto_tier_rule(rows, cols, tier):
    assert rr.plan_reduce(rows, cols, cu_count=256)["tier"] == tier


def test_splitk_geometry_for_the_long_row_workload():
    p = rr.plan_reduce(16, 1 << 24, cu_count=256)
    assert p["slices"] == 32 and p["grid"] == 512 and p["tile_cols"] == 8192
    assert p["workspace_bytes"] == 256 + 16 * 32 * 8


@pytest.mark.parametrize("rows,cols", [(1, 65536), (7, 100003), (200, 1 << 20), (3, 70001),
                                       (16, 1 << 24), (1, 1 << 30)])
def test_splitk_every_workgroup_gets_a_tile(rows, cols):
    p = rr.plan_reduce(rows, cols, tier="splitk", cu_count=256)
    g, t = p["slices"], p["tile_cols"]
    assert 1 <= g <= 256 and t % 4 == 0
    assert g <= -(-cols // t)          # T >= G tiles: every run [g*T/G, (g+1)*T/G) is non-empty
    assert p["grid"] == rows * g


def test_multi_stat_plan_uses_16_byte_partials():
    p = rr.plan_reduce(16, 1 << 24, op="sum_max_min", cu_count=256)
    assert p["tier"] == "splitk" and p["slices"] == 32
    assert p["workspace_bytes"] == 256 + 16 * 32 * 16
    assert rr.plan_reduce(1000, 48, op="sum_max_min")["tier"] == "wave"


def test_multi_stat_entry_point_validates_before_touching_the_device():
    lib = ctypes.CDLL(rr.lib_path())
    vp, i64, it = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.rr_reduce_rows_multi.argtypes = [vp, vp, vp, vp, i64, i64, i64, it, it, vp,
                                         ctypes.c_size_t, vp]
    lib.rr_reduce_rows.argtypes = [vp, vp, i64, i64, i64, it, it, it, vp, ctypes.c_size_t, vp]
    one = ctypes.c_void_p(16)  # never dereferenced: validation fails or no-ops first
    assert lib.rr_reduce_rows_multi(None, one, None, None, -1, 4, 4, 0, 0, None, 0, None) == 2
    assert lib.rr_reduce_rows_multi(None, one, None, None, 4, 8, 4, 0, 0, None, 0, None) == 2
    assert lib.rr_reduce_rows_multi(None, one, None, None, 4, 8, 8, 2, 0, None, 0, None) == 3
    assert lib.rr_reduce_rows_multi(None, one, None, None, 4, 100, 100, 0, 1, None, 0, None) == 4
    assert lib.rr_reduce_rows_multi(None, one, None, None, 0, 8, 8, 0, 0, None, 0, None) == 0
    assert lib.rr_reduce_rows_multi(None, None, None, None, 4, 8, 8, 0, 0, None, 0, None) == 1
    assert lib.rr_reduce_rows_multi(None, one, None, None, 4, 8, 8, 0, 0, None, 0, None) == 1
    # the tuple op is only for the planner queries
    assert lib.rr_reduce_rows(None, None, 4, 8, 8, 0, 3, 0, None, 0, None) == 7


def test_axis_plan():
    # many outputs: tiled, 4 adjacent outputs per thread
    p = rr.plan_axis(1, 4096, 1 << 20)
    assert p["tier"] == "tiled" and p["lanes_per_row"] == 4 and p["grid"] == (1 << 20) // 4 // 256
    # few outputs, long axis: split-K over the axis
    p = rr.plan_axis(1, 1 << 20, 64, cu_count=256)
    # 16 output groups: one tile of 16 groups x 16 axis lanes; 2 workgroups
    # per CU, so 512 slices
    assert p["tier"] == "splitk" and p["slices"] == 512 and p["grid"] == 512
    assert p["workspace_bytes"] == 512 * 64 * 8 and p["tile_cols"] == 2048
    p = rr.plan_axis(1, 1000, 64, cu_count=256)
    # 16 groups: tiles of 16 groups x 16 axis lanes; slices of >= 32 steps per lane
    assert p["tier"] == "splitk" and p["slices"] == 2 and p["grid"] == 2
    p = rr.plan_axis(1024, 4096, 16, cu_count=256)                      # narrow inner
    assert p["tier"] == "splitk" and p["slices"] == 1 and p["grid"] == 1024
    p = rr.plan_axis(1, 1 << 16, 1024, cu_count=256)    # 256 groups: 4 tiles of 64 x 4 lanes
    assert p["slices"] == 128 and p["grid"] == 512
    assert rr.plan_axis(1, 100, 64)["tier"] == "tiled"                 # axis too short
    assert rr.plan_axis(3, 100, 7)["lanes_per_row"] == 1               # inner % 4 != 0
    assert rr.plan_axis(3, 100, 8, tier="serial")["lanes_per_row"] == 1
    for tier, status in (("block", 4), ("wave", 4)):
        with pytest.raises(rr.RRError) as e:
            rr.plan_axis(3, 100, 8, tier=tier)
        assert e.value.status == status
    with pytest.raises(rr.RRError) as e:
        rr.plan_axis(1 << 40, 1 << 20, 1 << 10)                        # size overflows
    assert e.value.status == 2


def test_axis_entry_point_validates_before_touching_the_device():
    lib = ctypes.CDLL(rr.lib_path())
    vp, i64, it = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.rr_reduce_axis.argtypes = [vp, vp, i64, i64, i64, it, it, it, vp, ctypes.c_size_t, vp]
    assert lib.rr_reduce_axis(None, None, -1, 4, 4, 0, 0, 0, None, 0, None) == 2
    assert lib.rr_reduce_axis(None, None, 4, 4, 4, 2, 0, 0, None, 0, None) == 3
    assert lib.rr_reduce_axis(None, None, 4, 4, 4, 0, 5, 0, None, 0, None) == 7
    assert lib.rr_reduce_axis(None, None, 4, 4, 4, 0, 0, 2, None, 0, None) == 4
    assert lib.rr_reduce_axis(None, None, 0, 4, 4, 0, 0, 0, None, 0, None) == 0
    assert lib.rr_reduce_axis(None, None, 4, 4, 0, 0, 0, 0, None, 0, None) == 0
    assert lib.rr_reduce_axis(None, None, 4, 4, 4, 0, 0, 0, None, 0, None) == 1


def test_splitk_forced_on_short_rows_has_one_slice():
    p = rr.plan_reduce(64, 1000, tier="splitk", cu_count=256)
    assert p["slices"] == 1 and p["grid"] == 64


def test_wave_lanes_per_row():
    assert rr.plan_reduce(10, 48)["lanes_per_row"] == 16
    assert rr.plan_reduce(10, 16, tier="wave")["lanes_per_row"] == 4
    assert rr.plan_reduce(10, 17, tier="wave")["lanes_per_row"] == 16
    assert rr.plan_reduce(10, 64, tier="wave")["lanes_per_row"] == 16
    assert rr.plan_softmax(10, 64, tier="wave")["lanes_per_row"] == 16   # bf16: 8 per chunk


def test_softmax_tier_rule():
    assert rr.plan_softmax(8192, 8192)["tier"] == "block"
    assert rr.plan_softmax(8192, 8192)["block"] == 256
    assert rr.plan_softmax(8192, 8192)["grid"] == 512        # persistent rows: 2 per CU
    assert rr.plan_softmax(8192, 8191)["grid"] == 512        # ragged rows: persistent too
    assert rr.plan_softmax(64, 16384)["block"] == 512        # 2048 chunks: 512 threads x 4
    assert rr.plan_softmax(65536, 1024)["block"] == 64       # 128 chunks: one wavefront x 2
    assert rr.plan_softmax(65536, 1024)["grid"] == 256 * 16  # 32 loads per lane per CU
    assert rr.plan_softmax(64, 16385, tier="block")["block"] == 512  # ragged, long: wider
    assert rr.plan_softmax(64, 8201)["block"] == 512         # 1026 chunks: 512 threads x 4
    assert rr.plan_softmax(64, 8200)["block"] == 512         # 1025 whole chunks: persistent
    assert rr.plan_softmax(100, 40)["tier"] == "wave"
    assert rr.plan_softmax(100, 4)["tier"] == "tiled"
    assert rr.plan_softmax(16, 1 << 20)["tier"] == "splitk"    # rows < CU and long rows
    assert rr.plan_softmax(16, 16384)["tier"] == "block"       # 2048 chunks stay in registers
    # rows too long for registers (more than 2048 16-byte chunks) go split-K at
    # any row count
    assert rr.plan_softmax(64, 16385)["tier"] == "splitk"
    assert rr.plan_softmax(256, 1 << 20)["tier"] == "splitk"
    assert rr.plan_softmax(8192, 16392)["tier"] == "splitk"
    assert rr.plan_softmax(8192, 8193, x_dtype=torch.float32)["tier"] == "splitk"
    assert rr.plan_softmax(8192, 8192, x_dtype=torch.float32)["tier"] == "block"
    assert rr.plan_softmax(16, 65535)["tier"] == "splitk"
    assert rr.plan_layernorm(4096, 32768)["tier"] == "splitk"
    assert rr.plan_layernorm(4096, 16384)["tier"] == "block"
    p = rr.plan_softmax(4096, 32768, cu_count=256)           # G = 1: a workgroup per row
    assert p["slices"] == 1 and p["grid"] == 4096


def test_softmax_splitk_geometry():
    # bf16 rows of 2^20: tiles of 4 x 256 threads x 8 elements; 64 workgroups
    # per row (16 rows x 64 = 4 per CU), 16 tiles each
    p = rr.plan_softmax(16, 1 << 20, cu_count=256)
    assert p["slices"] == 64 and p["grid"] == 1024 and p["tile_cols"] == 8192
    assert p["workspace_bytes"] == 16 * 64 * 8
    # float32 input: 4 elements per 16-byte chunk
    p = rr.plan_softmax(16, 1 << 20, x_dtype=torch.float32, cu_count=256)
    assert p["tile_cols"] == 4096 and p["slices"] == 64


@pytest.mark.parametrize("rows,cols", [(1, 65536), (3, 70001), (200, 1 << 20), (1, 1 << 30)])
def test_softmax_splitk_every_workgroup_gets_a_tile(rows, cols):
    p = rr.plan_softmax(rows, cols, tier="splitk", cu_count=256)
    g, t = p["slices"], p["tile_cols"]
    assert 1 <= g <= 256 and g <= -(-cols // t) and p["grid"] == rows * g


def test_layernorm_tier_rule_and_geometry():
    p = rr.plan_layernorm(16384, 4096)
    # 512 chunks: 128 threads x 4 chunks; 32 loads per lane in flight per CU
    # = 4 workgroups of 2 wavefronts x 4 chunks per CU
    assert p["tier"] == "block" and p["block"] == 128 and p["grid"] == 1024
    p = rr.plan_layernorm(262144, 512)
    assert p["block"] == 64 and p["grid"] == 256 * 32            # 64 chunks: 1 per lane
    p = rr.plan_layernorm(4096, 16384)
    assert p["block"] == 512 and p["grid"] == 256                # 2048 chunks: 4 per lane
    assert rr.plan_layernorm(4096, 16392)["grid"] == 4096        # too long: one row per workgroup
    # rows at any alignment are persistent too (per-row weights)
    assert rr.plan_layernorm(16384, 4095)["grid"] == 1024
    assert rr.plan_layernorm(16384, 4095)["block"] == 128
    assert rr.plan_layernorm(100, 40)["tier"] == "wave"
    assert rr.plan_layernorm(100, 8)["tier"] == "tiled"
    assert rr.plan_layernorm(16, 1 << 20)["tier"] == "splitk"
    p = rr.plan_layernorm(16, 1 << 20, cu_count=256)
    assert p["slices"] == 64 and p["tile_cols"] == 8192 and p["grid"] == 1024
    assert p["workspace_bytes"] == 16 * 64 * 16
    p = rr.plan_layernorm(16, 1 << 20, x_dtype=torch.float32, cu_count=256)
    assert p["tile_cols"] == 4096 and p["slices"] == 64
    assert rr.plan_layernorm(4, 1000, tier="splitk", cu_count=256)["slices"] == 1
    with pytest.raises(rr.RRError) as e:
        rr.plan_layernorm(4, 65, tier="wave")
    assert e.value.status == 4
    with pytest.raises(rr.RRError) as e:
        rr.plan_layernorm(4, 8, x_dtype=torch.int32)
    assert e.value.status == 3
    with pytest.raises(rr.RRError) as e:
        rr.plan_layernorm(4, 8, w_dtype=torch.int32)
    assert e.value.status == 3


def test_layernorm_entry_point_validates_before_touching_the_device():
    lib = ctypes.CDLL(rr.lib_path())
    vp, i64, it = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.rr_layernorm_rows.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, it, it, it,
                                      ctypes.c_float, it, vp, ctypes.c_size_t, vp]

    def call(rows=4, cols=8, ldx=8, ldy=8, xd=2, yd=2, wd=0, eps=1e-5, tier=0):
        return lib.rr_layernorm_rows(None, None, None, None, None, None, rows, cols, ldx, ldy,
                                     xd, yd, wd, eps, tier, None, 0, None)
    assert call(rows=-1) == 2
    assert call(ldx=7) == 2
    assert call(ldy=7) == 2
    assert call(eps=-1.0) == 2
    assert call(eps=float("nan")) == 2
    assert call(eps=float("inf")) == 2
    assert call(xd=1) == 3
    assert call(wd=1) == 3
    assert call(tier=6) == 4
    assert call(cols=65, ldx=65, ldy=65, tier=1) == 4
    assert call(rows=0) == 0          # no-op
    assert call(cols=0) == 0          # no-op
    assert call() == 1                # NULL x / y


@pytest.mark.parametrize("kw,status", [
    (dict(rows=-1, cols=4), 2),
    (dict(rows=4, cols=-1), 2),
    (dict(rows=4, cols=8, ld=7), 2),
    (dict(rows=4, cols=65, tier="wave"), 4),
    (dict(rows=4, cols=8, dtype=torch.bfloat16), 3),
    (dict(rows=4, cols=8, cu_count=0), 2),
])
def test_plan_rejects_bad_arguments(kw, status):
    with pytest.raises(rr.RRError) as e:
        rr.plan_reduce(**kw)
    assert e.value.status == status


def test_entry_points_validate_before_touching_the_device():
    # Invalid shapes come back as status codes with no HIP call (no GPU here).
    lib = ctypes.CDLL(rr.lib_path())
    vp = ctypes.c_void_p
    lib.rr_reduce_rows.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, ctypes.c_size_t, vp]
    lib.rr_softmax_rows.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp,
                                    ctypes.c_size_t, vp]
    lib.rr_splitk_lse_merge.argtypes = [vp, vp, vp, vp, ctypes.c_int32, ctypes.c_int64,
                                        ctypes.c_int32, ctypes.c_float, ctypes.c_int, vp]
    assert lib.rr_reduce_rows(None, None, -1, 4, 4, 0, 0, 0, None, 0, None) == 2
    assert lib.rr_reduce_rows(None, None, 4, 8, 4, 0, 0, 0, None, 0, None) == 2
    assert lib.rr_reduce_rows(None, None, 4, 8, 8, 2, 0, 0, None, 0, None) == 3
    assert lib.rr_reduce_rows(None, None, 4, 8, 8, 0, 9, 0, None, 0, None) == 7
    assert lib.rr_reduce_rows(None, None, 4, 100, 100, 0, 0, 1, None, 0, None) == 4
    assert lib.rr_reduce_rows(None, None, 0, 8, 8, 0, 0, 0, None, 0, None) == 0   # no-op
    assert lib.rr_reduce_rows(None, None, 4, 8, 8, 0, 0, 0, None, 0, None) == 1   # NULL
    assert lib.rr_softmax_rows(None, None, 4, 8, 8, 8, 1, 1, 0, None, 0, None) == 3   # int32
    assert lib.rr_softmax_rows(None, None, 4, 8, 8, 8, 2, 2, 6, None, 0, None) == 4   # bad tier
    assert lib.rr_softmax_rows(None, None, 4, 8, 8, 8, 2, 2, 5, None, 0, None) == 1   # NULL
    assert lib.rr_softmax_rows(None, None, 4, 8, 4, 8, 2, 2, 0, None, 0, None) == 2   # ld_x < cols
    assert lib.rr_softmax_rows(None, None, 4, 0, 8, 8, 2, 2, 0, None, 0, None) == 0   # no-op
    assert lib.rr_splitk_lse_merge(None, None, None, None, 0, 4, 8, 1.0, 2, None) == 2
    assert lib.rr_splitk_lse_merge(None, None, None, None, 257, 4, 8, 1.0, 2, None) == 2
    assert lib.rr_splitk_lse_merge(None, None, None, None, 8, 4, 0, 1.0, 2, None) == 2
    assert lib.rr_splitk_lse_merge(None, None, None, None, 8, 4, 8, 1.0, 1, None) == 3
    assert lib.rr_splitk_lse_merge(None, None, None, None, 8, 0, 8, 1.0, 2, None) == 0
    assert lib.rr_splitk_lse_merge(None, None, None, None, 8, 4, 8, 1.0, 2, None) == 1


def test_noalloc_entry_point_validates_before_touching_the_device():
    lib = ctypes.CDLL(rr.lib_path())
    vp, i64, it = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.rr_reduce_rows_noalloc.argtypes = [vp, vp, i64, i64, i64, it, it, it, vp]
    f = lib.rr_reduce_rows_noalloc
    assert f(None, None, -1, 4, 4, 0, 0, 0, None) == 2        # negative rows
    assert f(None, None, 4, 8, 4, 0, 0, 0, None) == 2         # ld < cols
    assert f(None, None, 4, 8, 8, 2, 0, 0, None) == 3         # bf16 reduce
    assert f(None, None, 4, 8, 8, 0, 3, 0, None) == 7         # the multi-statistic op
    assert f(None, None, 4, 100, 100, 0, 0, 1, None) == 4     # wave tier, cols > 64
    assert f(None, None, 0, 8, 8, 0, 0, 0, None) == 0         # no-op
    assert f(None, None, 4, 8, 8, 0, 0, 0, None) == 1         # NULL
    lib.rr_status_string.restype = ctypes.c_char_p
    assert b"scratch" in lib.rr_status_string(8)
    assert rr.NOALLOC_SCRATCH_BYTES == 1 << 20
    hdr = open(os.path.join(ROOT, "include", "rr.h")).read()
    assert "#define RR_NOALLOC_SCRATCH_BYTES (1 << 20)" in hdr


def test_noalloc_scratch_bound_matches_the_plans():
    # an automatic split-K plan (rows < CU) fits the library's scratch with
    # room to spare; a forced split-K over many rows does not, and the entry
    # point refuses it (RR_ERR_SCRATCH) rather than overrun the array
    for rows in (1, 16, 37, 255):
        for op in ("sum", "max"):
            need = rr.plan_reduce(rows, 1 << 20, torch.float32, op, cu_count=256)["workspace_bytes"]
            assert 0 < need <= 16384, (rows, need)
    big = rr.plan_reduce(200000, 64, torch.float32, "sum", "splitk", cu_count=256)
    assert big["workspace_bytes"] > rr.NOALLOC_SCRATCH_BYTES


def test_attention_partials_validate_before_touching_the_device():
    lib = ctypes.CDLL(rr.lib_path())
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.rr_splitk_attention_partials.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                                 i32, i32, ctypes.c_float, vp]
    f = lib.rr_splitk_attention_partials
    ok = dict(batch=1, heads=4, kv_heads=2, q_rows=8, kv_len=16, depth=128, P=2, scale=0.1)

    def call(ptr=16, **kw):
        a = dict(ok, **kw)
        return f(ptr, ptr, ptr, ptr, ptr, ptr, a["batch"], a["heads"], a["kv_heads"], a["q_rows"],
                 a["kv_len"], a["depth"], a["P"], a["scale"], None)

    assert call(depth=96) == 2                     # depth 64 or 128 only
    assert call(heads=3) == 2                      # heads % kv_heads
    assert call(kv_heads=0) == 2
    assert call(P=0) == 2 and call(P=257) == 2
    assert call(scale=float("nan")) == 2 and call(scale=float("inf")) == 2
    assert call(q_rows=-1) == 2 and call(kv_len=-1) == 2
    assert call(q_rows=1 << 23) == 2               # q_rows * depth * 2 >= 2^31
    assert call(batch=1 << 40, heads=1 << 40, kv_heads=1) == 2   # grid beyond 31 bits, no overflow
    assert call(batch=1 << 62, P=256) == 2
    assert call(ptr=None) == 1                     # NULL
    assert call(ptr=8) == 2                        # misaligned
    assert call(ptr=None, q_rows=0) == 0           # nothing to do


def test_varlen_attention_partials_validate_before_touching_the_device():
    lib = ctypes.CDLL(rr.lib_path())
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.rr_splitk_attention_partials_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64,
                                                        i64, i64, i64, i64, i32, i32,
                                                        ctypes.c_float, vp]
    f = lib.rr_splitk_attention_partials_varlen
    ok = dict(batch=3, heads=4, kv_heads=2, total_q=40, total_k=90, max_q=20, depth=128, P=2,
              scale=0.1)

    def call(ptr=16, cu=16, **kw):
        a = dict(ok, **kw)
        return f(ptr, ptr, ptr, cu, cu, ptr, ptr, ptr, a["batch"], a["heads"], a["kv_heads"],
                 a["total_q"], a["total_k"], a["max_q"], a["depth"], a["P"], a["scale"], None)

    assert call(depth=96) == 2 and call(heads=3) == 2 and call(P=0) == 2
    assert call(scale=float("nan")) == 2
    assert call(total_q=-1) == 2 and call(total_k=-1) == 2 and call(max_q=-1) == 2
    assert call(total_q=1 << 31) == 2 and call(total_k=1 << 31) == 2   # int32 offsets
    assert call(heads=1 << 15, kv_heads=1) == 2    # 128 query rows' bytes beyond 2^31
    assert call(heads=1 << 14, kv_heads=1, ptr=None) == 1
    assert call(batch=1 << 40, heads=1 << 12, kv_heads=1) == 2   # grid beyond 31 bits
    assert call(ptr=None) == 1 and call(cu=None) == 1
    assert call(ptr=8) == 2                        # misaligned
    assert call(ptr=None, cu=None, total_q=0) == 0 # nothing to do
    assert call(ptr=None, cu=None, batch=0) == 0
    assert call(ptr=None, cu=None, max_q=0) == 0


def test_fused_attention_validates_before_touching_the_device():
    lib = ctypes.CDLL(rr.lib_path())
    vp, i64, i32, st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    lib.rr_splitk_attention.argtypes = [vp, vp, vp, vp, st, i64, i64, i64, i64, i64, i32, i32,
                                        ctypes.c_float, vp, ctypes.c_size_t, vp]
    lib.rr_splitk_attention_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32, i32,
                                                        ctypes.POINTER(ctypes.c_size_t),
                                                        ctypes.POINTER(ctypes.c_size_t)]
    f = lib.rr_splitk_attention
    ok = dict(batch=2, heads=4, kv_heads=2, q_rows=200, kv_len=16, depth=128, P=8, scale=0.1,
              dtype=2)

    def need(**kw):
        a = dict(ok, **kw)
        n, t = ctypes.c_size_t(7), ctypes.c_size_t(7)
        s = lib.rr_splitk_attention_workspace_bytes(a["batch"], a["heads"], a["kv_heads"],
                                                    a["q_rows"], a["kv_len"], a["depth"], a["P"],
                                                    ctypes.byref(n), ctypes.byref(t))
        need.tickets = t.value
        return s, n.value

    # tickets for 2*4*2 (head, query tile) groups padded to 256 bytes, then
    # O_p, m_p and l_p for P whole 128-row tiles of every group
    cells = 2 * 4 * 2 * 8 * 128
    assert need() == (0, 256 + cells * 128 * 4 + 2 * cells * 4) and need.tickets == 256
    assert need(batch=40, q_rows=1)[0] == 0 and need.tickets == 768   # 160 tickets, 640 B
    assert need(P=17)[0] == 2 and need(depth=64, P=9)[0] == 2   # P <= depth / 8
    assert need(depth=64, P=8)[0] == 0
    assert need(q_rows=0) == (0, 0)
    assert lib.rr_splitk_attention_workspace_bytes(1, 1, 1, 1, 1, 128, 1, None, None) == 1
    n = ctypes.c_size_t(0)
    assert lib.rr_splitk_attention_workspace_bytes(1, 1, 1, 1, 1, 128, 1, ctypes.byref(n),
                                                   None) == 0 and n.value > 0
    ws_len = need()[1]

    def call(ptr=256, ws=4096, ws_len=ws_len, **kw):
        a = dict(ok, **kw)
        return f(ptr, ptr, ptr, ptr, a["dtype"], a["batch"], a["heads"], a["kv_heads"], a["q_rows"],
                 a["kv_len"], a["depth"], a["P"], a["scale"], ws, ws_len, None)

    assert call(depth=96) == 2 and call(heads=3) == 2 and call(P=0) == 2
    assert call(P=17) == 2 and call(depth=64, P=9) == 2
    assert call(scale=float("nan")) == 2
    assert call(dtype=1) == 3                      # int32 output
    assert call(ptr=None) == 1
    assert call(ptr=8) == 2                        # misaligned
    assert call(ws=None) == 5 and call(ws_len=ws_len - 1) == 5 and call(ws=4100) == 5
    assert call(ptr=None, ws=None, q_rows=0) == 0  # nothing to do


def test_stream_reference_validates_before_touching_the_device():
    lib = ctypes.CDLL(rr.lib_path())
    vp = ctypes.c_void_p
    lib.rr_test_stream.argtypes = [ctypes.c_int32, vp, vp, ctypes.c_size_t, ctypes.c_int32, vp]
    assert lib.rr_test_stream(3, 16, 16, 64, 0, None) == 2      # unknown mode
    assert lib.rr_test_stream(0, None, None, 64, 0, None) == 1  # read without x
    assert lib.rr_test_stream(1, None, None, 64, 0, None) == 1  # write without y
    assert lib.rr_test_stream(2, 16, None, 64, 0, None) == 1    # copy without y
    assert lib.rr_test_stream(2, 16, 32, 40, 0, None) == 2      # size not a multiple of 16
    assert lib.rr_test_stream(2, 8, 32, 64, 0, None) == 2       # misaligned x
    assert lib.rr_test_stream(0, 16, None, 64, 17, None) == 2   # blocks per CU out of range
    assert lib.rr_test_stream(2, 16, 32, 0, 0, None) == 0       # nothing to move


def test_product_path_has_no_cpu_fallback():
    # The binding must refuse CPU tensors rather than compute on the host.
    x = torch.zeros(4, 8)
    with pytest.raises(ValueError):
        rr.reduce_rows(x)
    with pytest.raises(ValueError):
        rr.softmax_rows(x.bfloat16())
    src = open(os.path.join(ROOT, "split_deterministic_combine_amd", "__init__.py")).read()
    assert "oracle" not in src


def test_binding_argtypes_match_the_header_prototypes():
    # every prototype in rr.h / rr_test.h against the ctypes argtypes the
    # binding sets for it: a drifted signature would pass garbage silently
    import re
    lib = rr._load()
    protos = {}
    for h in ("rr.h", "rr_test.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(?:rr_status|void|int|const char\*)\s+(rr_\w+)\s*\(([^)]*)\)\s*;", text):
            params = m.group(2).strip()
            protos[m.group(1)] = 0 if params in ("", "void") else params.count(",") + 1
    assert len(protos) >= 20
    checked = 0
    for name, n in protos.items():
        fn = getattr(lib, name)
        if fn.argtypes is None:
            continue
        assert len(fn.argtypes) == n, (name, len(fn.argtypes), n)
        checked += 1
    assert checked >= 15
