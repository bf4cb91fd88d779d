"""The C-ABI library on the host (no GPU): it loads, exports exactly what
include/norm.h declares, and its host logic (launch-shape tables, workspace
sizing, argument validation) behaves as documented.  Every call here returns
before the library makes any HIP call; no kernel is launched."""
import ctypes
import os
import re
import subprocess

import pytest

import row_normalization_persistent_amd as rn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "norm.h")

SUCCESS, INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE = 0, 1, 2, 3, 4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"NORM_API\s+[\w\s\*]+?\b(norm_\w+)\s*\(", text)))


def test_header_declares_the_four_operations():
    names = declared_functions()
    for op in ("norm_fused_add_rmsnorm", "norm_rmsnorm_fwd", "norm_layernorm_fwd",
               "norm_layernorm_bwd", "norm_rmsnorm_bwd", "norm_fused_add_rmsnorm_bwd"):
        assert op in names
    for op in list(names):
        if op.endswith("_ex"):
            assert op[:-3] in names  # every strided variant has a plain form
    for op in ("norm_fused_add_rmsnorm", "norm_rmsnorm_fwd", "norm_layernorm_fwd"):
        assert op + "_split" in names  # the row-split forward
    for op in ("norm_fused_add_rmsnorm", "norm_rmsnorm_fwd", "norm_layernorm_fwd",
               "norm_layernorm_bwd", "norm_rmsnorm_bwd", "norm_fused_add_rmsnorm_bwd"):
        assert op + "_f32" in names  # fp32 activations
    assert len(names) == 42


def test_library_exports_every_declared_symbol():
    L = rn.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", rn.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert exported == declared_functions(), "library exports more or less than the header"


def test_library_targets_gfx950_only():
    blob = open(rn.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa-[a-z+-]*gfx[0-9a-z]+", blob))
    assert targets == {b"amdgcn-amd-amdhsa--gfx950"}, targets


def test_status_strings():
    for code, name in rn.STATUS.items():
        assert rn.status_string(code).startswith(name)
    assert rn.status_string(99) == "unknown norm_status"


def test_compiled_shapes_cover_every_hidden_size():
    for op in rn.OPS:
        for h in rn.HIDDEN_SIZES:
            cfgs = [c for c in rn.list_configs(op, h) if not c.runtime_hidden]
            assert cfgs, (op, h)
            for c in cfgs:
                assert c.threads_per_row % 64 == 0
                assert h % (8 * c.threads_per_row) == 0
                assert c.threads_per_row * c.rows_per_block <= 1024
        assert rn.list_configs(op, 0) == []
        assert rn.list_configs(op, (1 << 20) + 8) == []
        # rows wider than the on-chip kernels hold: the streamed shape only
        stream = rn.Cfg(512 if rn.OPS[op] >= 3 else 1024, 1, 0, 8)
        assert rn.list_configs(op, 70000) == [stream]
        assert rn.list_configs(op, 1 << 20) == [stream]


def test_runtime_hidden_shapes():
    # any hidden gets run-time shapes at the widest access the row allows
    for op in rn.OPS:
        for h, w in ((1, 1), (3000, 8), (4100, 4), (130, 2), (127, 1), (4096, 8), (5120, 8)):
            cfgs = [c for c in rn.list_configs(op, h) if c.runtime_hidden]
            assert cfgs, (op, h)
            for c in cfgs:
                t = c.threads_per_row
                assert c.vector_elems == w
                assert t in (8, 16, 32, 64, 128, 256, 512, 1024)
                r = max(1, 256 // t)  # lane groups a workgroup; narrow rows: 1, 2 or 4 rows each
                assert c.rows_per_block in ((r, 2 * r, 4 * r) if t < 64 else (r,))
                assert t // 2 < max(h // w, 1) or t == 8  # no shape with half its lanes idle
            sel = rn.select_config(op, 4096, h, cu_count=256)
            assert sel.runtime_hidden == (h not in rn.HIDDEN_SIZES)
            if sel.runtime_hidden:
                assert sel in cfgs or rn.OPS[op] >= 3, (op, h, sel)
    # the widest rows each family holds on chip; past them the streamed kernels
    # take 16-byte rows up to 2^20, and narrower accesses stay unsupported
    assert rn.select_config("fused_add_rmsnorm", 64, 65536, cu_count=256).threads_per_row == 1024
    assert "stream" not in rn.describe_config("fused_add_rmsnorm", 64, 65536, cu_count=256)
    for op, h in (("layernorm_fwd", 49152 + 8), ("rmsnorm_fwd", 65536 + 8),
                  ("fused_add_rmsnorm", 65536 + 8), ("layernorm_bwd", 32768 + 8),
                  ("rmsnorm_bwd", 32768 + 8), ("fused_add_rmsnorm_bwd", 1 << 20)):
        c = rn.select_config(op, 64, h, cu_count=256)
        assert c.vector_elems == 8 and c.threads_per_row == (512 if "bwd" in op else 1024), op
        d = rn.describe_config(op, 64, h, cu_count=256)
        assert "stream_" in d or "stage_fwd_kernel" in d, d
    for op, h in (("layernorm_fwd", 49152 + 4), ("rmsnorm_fwd", 65536 + 2),
                  ("layernorm_bwd", 32768 + 4), ("rmsnorm_bwd", 8193),
                  ("fused_add_rmsnorm", (1 << 20) + 8)):
        with pytest.raises(rn.NormError) as e:
            rn.select_config(op, 64, h, cu_count=256)
        assert e.value.status == UNSUPPORTED
    # small-batch rule on the run-time path: fewer rows -> more lanes per row
    prev = 1 << 30
    for rows in (1, 16, 256, 1024, 2048):  # (from 16 * CUs rows on, at most 4 accesses a lane)
        c = rn.select_config("rmsnorm_fwd", rows, 5120, cu_count=256)
        assert c.threads_per_row <= prev
        prev = c.threads_per_row
    # tiny rows share a wave; backward rows get one access per lane
    assert rn.select_config("rmsnorm_fwd", 1 << 16, 64, cu_count=256).threads_per_row == 8
    # two rows per lane group from 8 workgroups per CU up
    assert rn.select_config("rmsnorm_fwd", 1 << 17, 128, cu_count=256).rows_per_block == 32
    assert rn.select_config("rmsnorm_fwd", 8192, 128, cu_count=256).rows_per_block == 16
    assert rn.select_config("rmsnorm_fwd", 1 << 17, 128, cu_count=256).threads_per_row == 16
    assert rn.select_config("layernorm_fwd", 2048, 1000, cu_count=256).threads_per_row == 64
    # LayerNorm below a wave: about three accesses a lane, four rows a lane group
    assert rn.select_config("layernorm_fwd", 1 << 15, 512, cu_count=256) == rn.Cfg(32, 32, 0, 8)
    assert rn.select_config("layernorm_fwd", 1 << 17, 128, cu_count=256) == rn.Cfg(8, 128, 0, 8)
    assert rn.select_config("layernorm_fwd", 1 << 14, 768, cu_count=256) == rn.Cfg(32, 8, 0, 8)
    assert rn.select_config("rmsnorm_bwd", 8192, 128).threads_per_row == 16
    assert rn.select_config("layernorm_bwd", 8192, 5120).threads_per_row == 256
    assert rn.select_config("layernorm_bwd", 8192, 1000).threads_per_row == 128
    assert rn.select_config("rmsnorm_bwd", 64, 16376).threads_per_row == 512


def test_describe_staged_forward_widths():
    """Fused add + RMSNorm and RMSNorm rows past the on-chip forward kernels go
    to the LDS-staged kernel while registers and LDS hold them whole, to the
    streamed kernel past that; LayerNorm rows always stream."""
    for op, first, last in (("fused_add_rmsnorm", 65544, 81920), ("rmsnorm_fwd", 69912, 114688)):
        for h in (first, last):
            d = rn.describe_config(op, 300, h, cu_count=256)
            assert "stage_fwd_kernel" in d and d.endswith("grid 256"), d
        assert "stage_fwd_kernel" in rn.describe_config(op, 7, first, cu_count=256)
        assert rn.describe_config(op, 7, first, cu_count=256).endswith("grid 7")
        assert "stream_fwd_kernel" in rn.describe_config(op, 300, last + 8, cu_count=256)
    # RMSNorm rows that the streamed kernel reads once but for under 1/16
    assert "stream_fwd_kernel" in rn.describe_config("rmsnorm_fwd", 300, 69904, cu_count=256)
    for h in (49160, 65536, 90112, 131072):
        assert "stream_fwd_kernel" in rn.describe_config("layernorm_fwd", 300, h, cu_count=256)


def test_select_config_small_batches_spread_rows_over_more_lanes():
    # the small-batch rule: fewer rows -> more lanes per row, never fewer
    small = rn.select_config("fused_add_rmsnorm", 1, 4096, cu_count=256)
    mid = rn.select_config("fused_add_rmsnorm", 1024, 4096, cu_count=256)
    assert small.threads_per_row > mid.threads_per_row == 64
    prev = 1 << 30
    for rows in (1, 4, 16, 64, 256, 512, 1024, 2048):
        c = rn.select_config("fused_add_rmsnorm", rows, 4096, cu_count=256)
        assert c.threads_per_row <= prev
        prev = c.threads_per_row
    # fewer CUs fill up with fewer rows
    assert (rn.select_config("fused_add_rmsnorm", 256, 4096, cu_count=64).threads_per_row
            <= rn.select_config("fused_add_rmsnorm", 256, 4096, cu_count=256).threads_per_row)
    for op in ("fused_add_rmsnorm", "rmsnorm_fwd", "layernorm_fwd"):
        for h in rn.HIDDEN_SIZES:
            for rows in (1, 64, 1024, 2048, 4096, 8192, 1 << 20):
                c = rn.select_config(op, rows, h, cu_count=256)
                listed = [(k.threads_per_row, k.rows_per_block, k.grid > 0)
                          for k in rn.list_configs(op, h)]
                assert (c.threads_per_row, c.rows_per_block, c.grid > 0) in listed, \
                    (op, h, rows, c)
                # at most 8 vectors per lane by the rules, 16 (the compiled cap)
                # for shapes from the measured table
                assert h // (8 * c.threads_per_row) <= 16
    # LayerNorm forward: the persistent ring kernel at hidden >= 8192 for large batches
    for h, rows in ((16384, 2048), (12288, 2048), (8192, 8192), (4096, 8192)):
        c = rn.select_config("layernorm_fwd", rows, h, cu_count=256)
        assert c.grid > 0 and c.rows_per_block == 1, (h, rows, c)
        assert (c.threads_per_row, 1) in [(k.threads_per_row, k.rows_per_block)
                                          for k in rn.list_configs("layernorm_fwd", h)
                                          if k.grid > 0]
        assert "layernorm_fwd_ring_kernel" in rn.describe_config("layernorm_fwd", rows, h, 256)
    for h, rows in ((16384, 256), (4096, 2048), (2048, 8192), (1024, 8192)):
        assert rn.select_config("layernorm_fwd", rows, h, cu_count=256).grid == 0
    assert rn.select_config("layernorm_fwd", 600, 16384, cu_count=256).grid == 256
    # the switches where walks of two rows start to win: 320 rows (LayerNorm at
    # hidden 16384; RMSNorm at 12288 and 16384, and at 8192 up to 511 rows, then
    # again from 2048)
    sel = lambda op, rows, h: rn.select_config(op, rows, h, cu_count=256).grid
    assert sel("layernorm_fwd", 319, 16384) == 0 and sel("layernorm_fwd", 320, 16384) == 256
    assert sel("layernorm_fwd", 320, 12288) == 0 and sel("layernorm_fwd", 320, 8192) == 0
    for h in (16384, 12288):
        assert sel("rmsnorm_fwd", 319, h) == 0 and sel("rmsnorm_fwd", 320, h) == 256
    assert sel("rmsnorm_fwd", 319, 8192) == 0 and sel("rmsnorm_fwd", 320, 8192) == 256
    assert sel("rmsnorm_fwd", 511, 8192) == 256 and sel("rmsnorm_fwd", 512, 8192) == 0
    assert sel("rmsnorm_fwd", 2047, 8192) == 0 and sel("rmsnorm_fwd", 2048, 8192) == 256
    for h in rn.HIDDEN_SIZES:
        c = rn.select_config("layernorm_bwd", 8192, h)
        assert rn.Cfg(c.threads_per_row, 1, 0, 0) in rn.list_configs("layernorm_bwd", h)
        assert c.grid == 256
        assert rn.select_config("layernorm_bwd", 5, h).grid == 5


def test_ring_depth_follows_the_walk():
    """The ring kernels (LayerNorm, RMSNorm forward) run the shallowest compiled
    depth that holds a workgroup's walk, ceil(rows / grid) rows, else the
    deepest; the same rows and grid always give the same kernel."""
    import re

    def depth(op, rows, h, cfg=None):
        d = rn.describe_config(op, rows, h, cu_count=256)
        m = re.search(r"ring of (\d+) rows", d)
        return int(m.group(1)) if m else None

    for op in ("layernorm_fwd", "rmsnorm_fwd"):
        # 256 workgroups: walks of 2, 3, 4, 8, 9, 32 rows
        assert depth(op, 512, 16384) == 2
        assert depth(op, 513, 16384) == 4
        assert depth(op, 1024, 16384) == 4
        assert depth(op, 2048, 16384) == 8
        assert depth(op, 2049, 16384) == 8   # past the deepest ring: the deepest
        assert depth(op, 8192, 16384) == 8
        assert depth(op, 1024, 12288) == 4
    assert depth("layernorm_fwd", 8192, 4096) == 2   # 64 lanes hold only depth 2
    assert depth("rmsnorm_fwd", 1024, 8192) is None  # not a ring for 512-2047 rows there
    assert depth("rmsnorm_fwd", 400, 8192) == 2
    assert depth("layernorm_fwd", 320, 16384) == 2


def test_describe_config():
    d = rn.describe_config("fused_add_rmsnorm", 8192, 4096, cu_count=256)
    c = rn.select_config("fused_add_rmsnorm", 8192, 4096, cu_count=256)
    assert f"fused_add_rmsnorm_kernel<4096,{c.threads_per_row},{c.rows_per_block}>" in d
    # the late-weights variant where it measured faster, the early one around it
    assert "layernorm_fwd_lw_kernel<4096,64,4>" in rn.describe_config("layernorm_fwd", 2048,
                                                                      4096, cu_count=256)
    assert "layernorm_fwd_kernel<4096,64,4>" in rn.describe_config("layernorm_fwd", 1024, 4096,
                                                                   cu_count=256)
    assert "rmsnorm_fwd_lw_kernel<2048,64,4>" in rn.describe_config("rmsnorm_fwd", 4096, 2048,
                                                                    cu_count=256)
    # rows are counted on a 256-CU part: half the rows on a 128-CU part
    assert "rmsnorm_fwd_lw_kernel<2048,64,4>" in rn.describe_config("rmsnorm_fwd", 2048, 2048,
                                                                    cu_count=128)
    assert "fused_add_rmsnorm_lw_kernel<4096,64,4>" in rn.describe_config(
        "fused_add_rmsnorm", 2048, 4096, cu_count=256)
    # run-time hidden: late weights exactly when the grid is 2 to 4 workgroups per CU
    seen = set()
    for rows in (256, 1024, 2048, 4096, 8192):
        d = rn.describe_config("rmsnorm_fwd", rows, 2560, cu_count=256)
        c = rn.select_config("rmsnorm_fwd", rows, 2560, cu_count=256)
        late = 512 <= -(-rows // c.rows_per_block) <= 1024
        assert ("rmsnorm_fwd_dyn_lw_kernel<" in d) == late, d
        seen.add(late)
    assert seen == {True, False}
    d = rn.describe_config("layernorm_bwd", 8192, 4096, cu_count=256)
    assert "persistent grid of 256" in d and f"workspace {rn.workspace_bytes(8192, 4096)}" in d
    with pytest.raises(rn.NormError):
        rn.describe_config("rmsnorm_fwd", 4, 70002, cu_count=256)
    d = rn.describe_config("layernorm_bwd", 1000, 65536, cu_count=256)
    assert "31 row walkers x 16 column tiles" in d and "exchanging partial row sums" in d and \
        f"workspace {rn.workspace_bytes(1000, 65536)}" in d
    # fewer CUs (a partition): the exchange's workgroups stay co-resident, two
    # a CU: 2 x 32 / 16 tiles = 4 walkers
    assert rn.select_config("layernorm_bwd", 1000, 65536, cu_count=32).grid == 4
    assert "4 row walkers x 16 column tiles" in \
        rn.describe_config("layernorm_bwd", 1000, 65536, cu_count=32)
    assert rn.select_config("layernorm_bwd", 1000, 65536).grid == 31  # no CU count: 256-CU caps
    d = rn.describe_config("rmsnorm_fwd", 4096, 5120, cu_count=256)
    c = rn.select_config("rmsnorm_fwd", 4096, 5120, cu_count=256)
    assert f"rmsnorm_fwd_dyn_kernel<8,{c.threads_per_row}," in d
    d = rn.describe_config("layernorm_bwd", 8192, 100)
    assert "norm_bwd_dyn_rows_kernel<4," in d and f"workspace {rn.workspace_bytes(8192, 100)}" in d
    L = rn.lib()
    buf = ctypes.create_string_buffer(8)  # truncated, still NUL-terminated
    n = L.norm_describe_config(0, 16, 4096, 256, buf, 8)
    full = rn.describe_config(0, 16, 4096, cu_count=256)
    assert n == len(full) and buf.value.decode() == full[:7]


def test_workspace_bytes():
    for h in rn.HIDDEN_SIZES:
        g = rn.select_config("rmsnorm_bwd", 8192, h).grid
        # without a shape: enough for the compiled kernels and for the
        # run-time kernels at any access width (strided or narrow-aligned rows)
        assert rn.workspace_bytes(8192, h, op="rmsnorm_bwd") >= g * h * 4  # one slab
        assert rn.workspace_bytes(8192, h, op="fused_add_rmsnorm_bwd") >= g * h * 4
        c = rn.select_config("layernorm_bwd", 8192, h)
        assert rn.workspace_bytes(8192, h) >= c.grid * 2 * h * 4
        assert rn.workspace_bytes(8192, h) == 2 * rn.workspace_bytes(8192, h, op="rmsnorm_bwd")
        assert rn.workspace_bytes(0, h) == 0
        assert rn.workspace_bytes(100, h, rn.Cfg(256, 1, 7)) == 7 * 2 * h * 4
    assert rn.workspace_bytes(3, 4096) == 3 * 2 * 4096 * 4  # never more slabs than rows
    # run-time shapes: one slab per row group, each output padded to 64 columns
    # run-time shapes: one slab per workgroup, whatever its rows per workgroup
    assert rn.workspace_bytes(100, 1000, rn.Cfg(16, 16, 7, 8)) == 7 * 2 * 1024 * 4
    assert rn.workspace_bytes(8192, 1000) >= 256 * 2 * 1024 * 4
    assert rn.workspace_bytes(10, (1 << 20) + 8) == 0
    # streamed rows: one slab per row walker (511 // column tiles of 4096, at
    # most the rows), then the tiles' exchange area: per walker 12 walk steps
    # of 16 bytes a tile
    assert rn.workspace_bytes(10, 70000) == 10 * 2 * 70016 * 4 + 10 * 12 * 18 * 16
    assert rn.workspace_bytes(1000, 65536) == 31 * 2 * 65536 * 4 + 31 * 12 * 16 * 16
    assert rn.workspace_bytes(1000, 65536, op="rmsnorm_bwd") == 31 * 65536 * 4 + 31 * 12 * 16 * 16
    assert rn.workspace_bytes(1000, 65536, rn.Cfg(512, 1, 5, 8)) == \
        5 * 2 * 65536 * 4 + 5 * 12 * 16 * 16
    # up to 64 tiles (262144 columns) the tiles exchange their partial sums;
    # wider rows take the row sums kernel (8 bytes a row) and 16384-column
    # tiles, 255 // tiles walkers
    assert rn.workspace_bytes(1000, 262144) == 7 * 2 * 262144 * 4 + 7 * 12 * 64 * 16
    assert rn.workspace_bytes(1000, 262152) == 15 * 2 * 262208 * 4 + 1000 * 8
    assert "exchanging partial row sums" in rn.describe_config("layernorm_bwd", 1000, 262144)
    d = rn.describe_config("rmsnorm_bwd", 1000, 262152)
    assert "stream_bwd_stats_kernel" in d and "15 row walkers x 17 column tiles" in d, d
    assert rn.workspace_bytes(-1, 4096) == 0


# ---- argument validation (fake device addresses; nothing is dereferenced)
A = 1 << 32  # a 16-byte aligned fake address
MB = 1 << 24


def fused(out=A, res=A + MB, x=A + 2 * MB, w=A + 3 * MB, rows=4, hidden=4096, eps=1e-6, cfg=None):
    return rn.lib().norm_fused_add_rmsnorm_cfg(out, res, x, w, rows, hidden, eps, cfg, None)


def test_fused_validation():
    assert fused(rows=0) == SUCCESS  # nothing to do, no launch
    assert fused(rows=-1) == INVALID
    assert fused(eps=float("nan")) == INVALID
    assert fused(eps=float("inf")) == INVALID
    assert fused(eps=-1e-6) == INVALID
    assert fused(hidden=(1 << 20) + 8) == UNSUPPORTED
    assert fused(hidden=70002) == UNSUPPORTED  # 4-byte accesses stop at 16384
    assert fused(hidden=0) == UNSUPPORTED
    assert fused(out=0) == INVALID
    assert fused(res=0) == INVALID
    assert fused(x=0) == INVALID
    assert fused(w=0) == INVALID
    assert fused(x=A + 2 * MB + 1) == MISALIGNED  # bf16 needs 2 bytes
    assert fused(res=A + MB + 1) == MISALIGNED
    assert fused(w=A + 3 * MB + 1) == MISALIGNED
    compiled = ctypes.byref(rn.LaunchCfg(64, 4, 0, 0))  # compiled shapes need 16 bytes
    assert fused(x=A + 2 * MB + 8, cfg=compiled) == MISALIGNED
    assert fused(w=A + 3 * MB + 4, cfg=compiled) == MISALIGNED
    assert fused(hidden=4000, cfg=compiled) == UNSUPPORTED
    assert fused(res=A + 2 * MB) == INVALID   # residual may alias nothing
    assert fused(out=A + MB) == INVALID       # out == residual
    assert fused(out=A + 2 * MB + 64) == INVALID  # partial overlap with x
    assert fused(w=A + 16) == INVALID         # weight inside out
    bad = rn.LaunchCfg(96, 1, 0)
    assert fused(cfg=ctypes.byref(bad)) == INVALID  # not a compiled shape
    assert fused(cfg=ctypes.byref(rn.LaunchCfg(64, 4, 3))) == INVALID  # no ring kernel here
    assert fused(cfg=ctypes.byref(rn.LaunchCfg(64, 1, -1))) == INVALID
    assert fused(cfg=ctypes.byref(rn.LaunchCfg(0, 1, 0))) == INVALID
    # run-time-hidden shapes
    assert fused(cfg=ctypes.byref(rn.LaunchCfg(64, 1, 0, 8))) == INVALID  # rows per block is 4
    assert fused(cfg=ctypes.byref(rn.LaunchCfg(64, 4, 0, 3))) == INVALID  # not an access width
    assert fused(cfg=ctypes.byref(rn.LaunchCfg(8, 32, 0, 8))) == INVALID  # row too wide for it
    assert fused(hidden=4100, cfg=ctypes.byref(rn.LaunchCfg(512, 1, 0, 8))) == INVALID
    assert fused(x=A + 2 * MB + 8, cfg=ctypes.byref(rn.LaunchCfg(512, 1, 0, 8))) == MISALIGNED


def rms(out=A, x=A + MB, w=A + 2 * MB, rows=4, hidden=2048, eps=1e-6):
    return rn.lib().norm_rmsnorm_fwd_cfg(out, x, w, rows, hidden, eps, None, None)


def test_rmsnorm_validation():
    assert rms(rows=0) == SUCCESS
    assert rms(hidden=65546) == UNSUPPORTED
    assert rms(out=0) == INVALID
    assert rms(out=A + 1) == MISALIGNED
    assert rms(out=A + MB + 16) == INVALID  # partial overlap with x
    assert rms(w=A + 32) == INVALID


def lnf(y=A, mean=A + MB, rstd=A + MB + 65536, x=A + 2 * MB, w=A + 3 * MB, b=A + 3 * MB + 65536,
        rows=4, hidden=1024, eps=1e-5):
    return rn.lib().norm_layernorm_fwd_cfg(y, mean, rstd, x, w, b, rows, hidden, eps, None, None)


def test_layernorm_fwd_validation():
    assert lnf(rows=0) == SUCCESS
    assert lnf(eps=-1.0) == INVALID
    assert lnf(hidden=(1 << 20) + 8) == UNSUPPORTED
    assert lnf(hidden=49152 + 4) == UNSUPPORTED  # past 49152 only 16-byte rows (streamed)
    assert lnf(b=0) == INVALID
    assert lnf(mean=0) == INVALID   # mean and rstd are both given or both null
    assert lnf(rstd=0) == INVALID
    assert lnf(mean=A + MB + 2) == MISALIGNED
    assert lnf(b=A + 3 * MB + 65536 + 1) == MISALIGNED
    assert lnf(mean=A + MB, rstd=A + MB + 8) == INVALID  # mean/rstd overlap
    L = rn.lib()
    ring = lambda c: L.norm_layernorm_fwd_cfg(A, A + MB, A + MB + 65536, A + 2 * MB, A + 3 * MB,
                                              A + 3 * MB + 65536, 4, 1024, 1e-5, ctypes.byref(c),
                                              None)
    assert ring(rn.LaunchCfg(128, 1, 4, 0)) == INVALID   # no ring kernel at hidden 1024
    assert ring(rn.LaunchCfg(128, 2, 4, 0)) == INVALID   # ring shapes hold one row a group
    assert ring(rn.LaunchCfg(128, 1, 4, 8)) == INVALID   # rings are compiled-hidden only
    rms_ring = lambda c, h: L.norm_rmsnorm_fwd_cfg(A, A + 2 * GB, A + 4 * GB, 4, h, 1e-6,
                                                   ctypes.byref(c), None)
    assert rms_ring(rn.LaunchCfg(512, 1, 4, 0), 2048) == INVALID   # RMSNorm rings from 8192 only
    assert rms_ring(rn.LaunchCfg(64, 1, 4, 0), 16384) == INVALID   # no ring of 64 lanes there
    assert rms_ring(rn.LaunchCfg(512, 2, 4, 0), 16384) == INVALID  # one row a group
    fused_ring = lambda c: L.norm_fused_add_rmsnorm_cfg(A, A + 2 * GB, A + 4 * GB, A + 6 * GB, 4,
                                                        16384, 1e-6, ctypes.byref(c), None)
    assert fused_ring(rn.LaunchCfg(512, 1, 4, 0)) == INVALID      # the fused op has no ring


GB = 1 << 30


def lnb(dx=A, dw=A + GB, db=A + GB + 65536, dy=A + 2 * GB, x=A + 3 * GB, mean=A + 4 * GB,
        rstd=A + 4 * GB + 65536, w=A + 5 * GB, ws=A + 6 * GB, ws_bytes=None, rows=8192,
        hidden=4096, eps=1e-5, cfg=None):
    if ws_bytes is None:
        ws_bytes = rn.workspace_bytes(rows, hidden) - 4
    return rn.lib().norm_layernorm_bwd_cfg(dx, dw, db, dy, x, mean, rstd, w, ws, ws_bytes, rows,
                                           hidden, eps, cfg, None)


def test_layernorm_bwd_validation():
    # all checks pass except the workspace size: proves the order of checks
    assert lnb() == WORKSPACE
    assert lnb(rows=-2) == INVALID
    assert lnb(eps=float("nan")) == INVALID
    assert lnb(hidden=32778) == UNSUPPORTED  # past 32768 only 16-byte rows (streamed)
    assert lnb(hidden=(1 << 20) + 8) == UNSUPPORTED
    assert lnb(hidden=5000) == WORKSPACE  # run-time kernels (workspace sized for 4096)
    assert lnb(dw=0) == INVALID
    assert lnb(ws=0) == INVALID
    assert lnb(dy=0) == INVALID
    assert lnb(mean=0) == INVALID
    assert lnb(dx=A + 1) == MISALIGNED
    assert lnb(dx=A + 4) == WORKSPACE  # 4-byte alignment: narrower accesses
    assert lnb(mean=A + 4 * GB + 2) == MISALIGNED
    assert lnb(ws=A + 6 * GB + 4) == MISALIGNED
    assert lnb(db=A + GB + 4 * 4096 - 8) == INVALID  # dweight overlaps dbias
    assert lnb(dx=A + 2 * GB) == WORKSPACE           # dx == dy is allowed
    assert lnb(dx=A + 2 * GB + 16) == INVALID        # partial overlap
    assert lnb(ws=A + 3 * GB) == INVALID             # workspace over x
    assert lnb(cfg=ctypes.byref(rn.LaunchCfg(96, 1, 0))) == INVALID
    assert lnb(cfg=ctypes.byref(rn.LaunchCfg(256, 2, 0))) == INVALID
    assert lnb(cfg=ctypes.byref(rn.LaunchCfg(256, 1, -1))) == INVALID
    small = rn.LaunchCfg(256, 1, 4)
    assert lnb(cfg=ctypes.byref(small), ws_bytes=4 * 2 * 4096 * 4 - 1) == WORKSPACE


def test_python_binding_rejects_bad_tensors():
    import torch
    x = torch.zeros(4, 4096, dtype=torch.bfloat16)
    w = torch.zeros(4096, dtype=torch.bfloat16)
    with pytest.raises(ValueError):  # host tensors are refused before any call
        rn.fused_add_rmsnorm(x, x.clone(), w, 1e-6)
    with pytest.raises(TypeError):
        rn.rmsnorm_fwd(x.float(), w, 1e-6)


def rmsb(dx=A, dw=A + GB, dy=A + 2 * GB, x=A + 3 * GB, w=A + 5 * GB, ws=A + 6 * GB,
         ws_bytes=None, rows=8192, hidden=4096, eps=1e-6, dres=None, cfg=None):
    if ws_bytes is None:
        ws_bytes = rn.workspace_bytes(rows, hidden, op="rmsnorm_bwd") - 4
    if dres is None:
        return rn.lib().norm_rmsnorm_bwd_cfg(dx, dw, dy, x, w, ws, ws_bytes, rows, hidden, eps,
                                             cfg, None)
    return rn.lib().norm_fused_add_rmsnorm_bwd_cfg(dx, dw, dy, dres, x, w, ws, ws_bytes, rows,
                                                   hidden, eps, cfg, None)


def test_rmsnorm_bwd_validation():
    assert rmsb() == WORKSPACE  # everything else valid: proves the order of checks
    assert rmsb(dres=A + 4 * GB) == WORKSPACE
    assert rmsb(rows=-1) == INVALID
    assert rmsb(eps=-1.0) == INVALID
    assert rmsb(eps=float("nan")) == INVALID
    assert rmsb(hidden=32778) == UNSUPPORTED
    assert rmsb(hidden=8193) == UNSUPPORTED  # odd rows: 2-byte accesses, at most 8192
    assert rmsb(hidden=4095) == WORKSPACE
    assert rmsb(dw=0) == INVALID
    assert rmsb(x=0) == INVALID
    assert rmsb(dy=A + 2 * GB + 1) == MISALIGNED
    assert rmsb(dres=A + 4 * GB + 1) == MISALIGNED
    assert rmsb(dy=A + 2 * GB + 8) == WORKSPACE
    assert rmsb(dx=A + 2 * GB) == WORKSPACE                 # dx == dy allowed
    assert rmsb(dx=A + 4 * GB, dres=A + 4 * GB) == WORKSPACE  # ds == dres allowed
    assert rmsb(dx=A + 3 * GB) == INVALID                   # dx == x is not
    assert rmsb(dx=A + 2 * GB + 16) == INVALID
    assert rmsb(ws=A + 1 * GB + 64) == INVALID              # workspace over dweight
    assert rmsb(cfg=ctypes.byref(rn.LaunchCfg(512, 1, 4)),
                ws_bytes=4 * 4096 * 4 - 1) == WORKSPACE


# ---- strided rows (the _ex entry points) ---------------------------------------------
def rmsb_ex(dx=A, ld_dx=4096, dw=A + GB, dy=A + 2 * GB, ld_dy=4096, x=A + 3 * GB, ld_x=4096,
            w=A + 5 * GB, ws=A + 6 * GB, rows=8192, hidden=4096, eps=1e-6, cfg=None):
    ws_bytes = rn.workspace_bytes(rows, hidden, op="rmsnorm_bwd") - 4
    return rn.lib().norm_rmsnorm_bwd_ex(dx, ld_dx, dw, dy, ld_dy, x, ld_x, w, ws, ws_bytes,
                                        rows, hidden, eps, cfg, None)


def test_strided_validation():
    assert rmsb_ex() == WORKSPACE
    assert rmsb_ex(ld_x=4095) == INVALID           # ld < hidden
    assert rmsb_ex(ld_x=1 << 41) == INVALID        # absurd stride
    # a legal stride whose span over all rows passes 2^47 bytes (offsets would
    # leave int64 long before an address could be that far)
    assert rmsb_ex(ld_x=1 << 40, rows=(1 << 31) - 1) == INVALID
    assert rmsb_ex(x=A + 7 * GB, ld_x=1 << 40, rows=64) == WORKSPACE  # just inside
    assert rmsb_ex(ld_x=3 * 4096) == WORKSPACE     # a column slice of a wider matrix
    # dx and dy as two column slices of one [rows, 2 * hidden] matrix: their rows
    # interleave without sharing an element
    assert rmsb_ex(dx=A + 2 * GB, ld_dx=8192, dy=A + 2 * GB + 8192, ld_dy=8192) == WORKSPACE
    # ... but shifted by half a row they do share elements
    assert rmsb_ex(dx=A + 2 * GB, ld_dx=8192, dy=A + 2 * GB + 4096, ld_dy=8192) == INVALID
    # the exact alias dx == dy needs equal strides
    assert rmsb_ex(dx=A + 2 * GB, ld_dx=4096, dy=A + 2 * GB, ld_dy=4096) == WORKSPACE
    assert rmsb_ex(dx=A + 2 * GB, ld_dx=8192, dy=A + 2 * GB, ld_dy=4096) == INVALID
    # odd strides force 2-byte accesses: still accepted
    assert rmsb_ex(ld_x=4097) == WORKSPACE
    compiled = ctypes.byref(rn.LaunchCfg(512, 1, 0, 0))
    assert rmsb_ex(ld_x=8192, cfg=compiled) == INVALID  # compiled shapes need contiguous rows
    L = rn.lib()
    # forward: out overlapping a slice of x, and a bad ld (rejected before any HIP call)
    assert L.norm_rmsnorm_fwd_ex(A, 4096, A + 2, 8192, A + GB, 4, 4096, 1e-6, None,
                                 None) == INVALID
    assert L.norm_rmsnorm_fwd_ex(A, 4000, A + GB, 4096, A + 2 * GB, 4, 4096, 1e-6, None,
                                 None) == INVALID
    assert L.norm_rmsnorm_fwd_ex(A, 4096, A + GB, 1 << 40, A + 2 * GB, (1 << 31) - 1, 4096,
                                 1e-6, None, None) == INVALID  # x spans past 2^47 bytes
    assert L.norm_fused_add_rmsnorm_ex(A, 4096, A + GB, 4096, A + 2 * GB, 4096, A + 3 * GB, 4,
                                       (1 << 20) + 8, 1e-6, None, None) == UNSUPPORTED
    assert L.norm_layernorm_fwd_ex(A, 4096, None, None, A + GB, 4095, A + 2 * GB, A + 3 * GB, 4,
                                   4096, 1e-5, None, None) == INVALID
    assert L.norm_layernorm_bwd_ex(A, 4096, A + GB, A + GB + 65536, A + 2 * GB, 4096,
                                   A + 3 * GB, 4096, A + 4 * GB, A + 4 * GB + 65536, A + 5 * GB,
                                   A + 6 * GB, 0, 8192, 4096, 1e-5, None, None) == WORKSPACE
    assert L.norm_fused_add_rmsnorm_bwd_ex(A, 4096, A + GB, A + 2 * GB, 4096, A + 4 * GB, 4095,
                                           A + 3 * GB, 4096, A + 5 * GB, A + 6 * GB, 0, 8192,
                                           4096, 1e-6, None, None) == INVALID  # ld_dres < hidden
    assert L.norm_fused_add_rmsnorm_bwd_ex(A, 4096, A + GB, A + 2 * GB, 4096, None, 0,
                                           A + 3 * GB, 4096, A + 5 * GB, A + 6 * GB, 0, 8192,
                                           4096, 1e-6, None, None) == WORKSPACE  # ld ignored


# ---- row-split forward --------------------------------------------------------------
def test_select_split():
    """Rows are split only when few and heavy: up to 8 rows that move >= 256
    KiB (fused, 8 * hidden bytes) or 192 KiB (4 * hidden) each, 9 to 32 rows
    that move >= 384 KiB, or up to 64 rows that no one-workgroup-per-row
    kernel holds (LayerNorm above 49152).  Chunks aim at ~64 KiB of traffic
    (8192 columns fused, 16384 RMSNorm, 12288 LayerNorm), at most
    max(4, 64 / rows) a row; hidden must be a multiple of 8."""
    sel = lambda op, rows, h, cu=256: rn.select_split(op, rows, h, cu_count=cu)
    F, R, L = "fused_add_rmsnorm", "rmsnorm_fwd", "layernorm_fwd"
    assert sel(F, 1, 65536) == (8, 4)       # 8 chunks of 8192 columns
    assert sel(F, 1, 32768) == (4, 4)
    assert sel(F, 1, 24576) == (1, 0)       # 192 KiB a row: a tie for the fused op
    assert sel(F, 1, 40960) == (5, 4)
    assert sel(F, 1, 16384) == (1, 0)       # 128 KiB a row: one workgroup is faster
    assert sel(F, 9, 32768) == (1, 0)       # 9-32 rows need 384 KiB a row
    assert sel(F, 16, 65536) == (4, 8)      # at most max(4, 64 / rows) chunks
    assert sel(F, 32, 49152) == (4, 6)
    assert sel(F, 33, 65536) == (1, 0)
    assert sel(F, 1, 65528) == (8, 4)       # the last chunk holds 8184 columns
    assert sel(R, 1, 65536) == (4, 8)       # 4 chunks of 16384 columns
    assert sel(R, 1, 49152) == (3, 8)
    assert sel(R, 1, 32768) == (1, 0)       # 128 KiB a row
    assert sel(R, 16, 65536) == (1, 0)      # 256 KiB < 384 KiB
    assert sel(L, 1, 49152) == (4, 6)       # 12288 columns a chunk
    assert sel(L, 9, 49152) == (1, 0)
    assert sel(L, 9, 57344) == (5, 6)       # no one-workgroup kernel holds it: split
    assert sel(L, 64, 65536) == (4, 8)      # ... up to 64 rows
    assert sel(L, 65, 65536) == (1, 0)
    assert sel(L, 2, 57344, cu=8) == (4, 7)
    assert sel(F, 1, 65540) == (1, 0)       # not a multiple of 8
    assert sel(F, 4, 65536, cu=4) == (1, 0)
    for op in (F, R, L):
        for rows in (1, 2, 3, 5, 8, 9, 17, 32, 64, 128, 512):
            for h in (8192, 8200, 12288, 16384, 24576, 30000, 32768, 49152, 57344, 65536):
                k, v = sel(op, rows, h)
                if k > 1:
                    chunk = 256 * v * 8
                    assert 1 <= v <= 8 and 2 <= k <= 64 and rows * k <= 256
                    assert (k - 1) * chunk < h <= k * chunk  # no empty chunk
    with pytest.raises(rn.NormError):
        rn.select_split("layernorm_bwd", 1, 16384, cu_count=256)


def test_split_workspace_bytes():
    assert rn.split_workspace_bytes(0) == 0
    assert rn.split_workspace_bytes(-3) == 0
    assert rn.split_workspace_bytes(1) == 256 + 144 * 8
    assert rn.split_workspace_bytes(512) == 256 + 512 * 144 * 8
    assert rn.split_workspace_bytes(10 ** 6) == rn.split_workspace_bytes(512)


WS = A + 8 * MB  # a workspace away from every other argument


def fused_split(out=A, res=A + MB, x=A + 2 * MB, w=A + 3 * MB, rows=4, hidden=16384, eps=1e-6,
                ws=WS, ws_bytes=1 << 20, split=2):
    return rn.lib().norm_fused_add_rmsnorm_split(out, res, x, w, rows, hidden, eps, ws, ws_bytes,
                                                 split, None)


def test_split_validation():
    """Checks that return before any HIP call (the CU count is the last one)."""
    assert fused_split(rows=0) == SUCCESS
    assert fused_split(split=-1) == INVALID
    assert fused_split(split=65) == INVALID
    assert fused_split(rows=-1) == INVALID
    assert fused_split(eps=float("nan")) == INVALID
    assert fused_split(hidden=(1 << 20) + 8) == UNSUPPORTED
    assert fused_split(x=0) == INVALID
    assert fused_split(res=A + 2 * MB) == INVALID              # residual aliases x
    assert fused_split(x=A + 2 * MB + 1) == MISALIGNED
    # explicit k: contiguous 16-byte rows of a multiple-of-8 hidden, <= 512 rows
    assert fused_split(x=A + 2 * MB + 8) == MISALIGNED
    assert fused_split(hidden=16380) == INVALID
    assert fused_split(rows=513) == INVALID
    assert fused_split(hidden=8192 * 8 + 8, split=2) == INVALID  # 2 chunks of 17 accesses
    assert fused_split(hidden=65536, split=2) == INVALID        # 16 accesses a lane
    assert fused_split(ws=0) == WORKSPACE
    assert fused_split(ws_bytes=rn.split_workspace_bytes(4) - 1) == WORKSPACE
    assert fused_split(ws=WS + 4) == MISALIGNED
    assert fused_split(ws=A + 2 * MB + 4096) == INVALID         # workspace inside x
    assert fused_split(ws=A + 3 * MB - 16) == INVALID           # overlaps the weight
    L = rn.lib()
    assert L.norm_rmsnorm_fwd_split(A, A + MB, A + 2 * MB, 4, 16384, 1e-6, 0, 0, 3,
                                    None) == WORKSPACE
    assert L.norm_rmsnorm_fwd_split(A, A, A + 2 * MB, 4, 16384, 1e-6, WS, 1 << 20, -2,
                                    None) == INVALID
    assert L.norm_layernorm_fwd_split(A, A + MB, A + MB + 8, A + 2 * MB, A + 3 * MB,
                                      A + 3 * MB + 65536, 4, 16384, 1e-5, WS, 1 << 20, 2,
                                      None) == INVALID  # rstd overlaps mean
    assert L.norm_layernorm_fwd_split(A, A + MB, A + MB + 65536, A + 2 * MB, A + 3 * MB,
                                      A + 3 * MB + 65536, 4, 16384, 1e-5, A + MB + 8, 1 << 20,
                                      2, None) == MISALIGNED


def test_split_status_and_spin_limit_host_side():
    """The error-word query rejects bad arguments before any HIP call; the
    spin limit is process-wide and returns the previous value."""
    L = rn.lib()
    st = ctypes.c_uint32(7)
    assert L.norm_split_status(None, 1, ctypes.byref(st), None) == INVALID
    assert L.norm_split_status(WS, 1, None, None) == INVALID
    assert L.norm_split_status(WS + 4, 1, ctypes.byref(st), None) == MISALIGNED
    assert st.value == 7  # untouched on error
    prev = rn.set_split_spin_limit(5)
    try:
        assert prev == 1 << 20
        assert rn.set_split_spin_limit(0) == 5
    finally:
        rn.set_split_spin_limit(prev)
    assert rn.set_split_spin_limit(prev) == prev


def test_noalloc_validation():
    """The allocation-free LayerNorm backward validates like
    norm_layernorm_bwd and refuses launches whose partial sums exceed its
    scratch array, all before any HIP call."""
    L = rn.lib()
    f = L.norm_layernorm_bwd_noalloc
    f.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                          ctypes.c_void_p]

    def call(dx=A, dw=A + MB, db=A + 2 * MB, dy=A + 3 * MB, x=A + 4 * MB, m=A + 5 * MB,
             r=A + 6 * MB, w=A + 7 * MB, rows=8, hidden=4096, eps=1e-5):
        return f(dx, dw, db, dy, x, m, r, w, rows, hidden, eps, None)

    assert call(rows=-1) == INVALID
    assert call(dw=0) == INVALID
    assert call(db=0) == INVALID
    assert call(x=0) == INVALID
    assert call(m=0) == INVALID
    assert call(eps=float("inf")) == INVALID
    assert call(hidden=0) == UNSUPPORTED
    assert call(dw=A + MB + 2) == MISALIGNED
    assert call(dx=A + 3 * MB + 64) == INVALID      # dx overlaps dy without equalling it
    assert call(dw=A + 5 * MB) == INVALID           # dweight aliases mean
    # 256 rows of 32768 columns: 256 slabs of 2 x 32768 fp32 = 64 MiB > 32 MiB
    big = 1 << 30
    assert call(dx=A, dy=A + big, x=A + 2 * big, m=A + 3 * big, r=A + 3 * big + MB,
                w=A + 3 * big + 2 * MB, dw=A + 3 * big + 3 * MB, db=A + 3 * big + 4 * MB,
                rows=256, hidden=32768) == WORKSPACE
    assert rn.NOALLOC_SCRATCH_BYTES == 32 << 20
    assert rn.workspace_bytes(512, 16384) == rn.NOALLOC_SCRATCH_BYTES  # the largest that fits


def test_f32_validation():
    """The fp32 entry points: contiguous rows, hidden a multiple of 4 up to
    2^20, 16-byte-aligned matrices and weight / bias vectors; every case here
    returns before any HIP call."""
    L = rn.lib()
    fa = L.norm_fused_add_rmsnorm_f32

    def fused(out=A, res=A + 4 * MB, x=A + 8 * MB, w=A + 12 * MB, rows=8, hidden=4096,
              eps=1e-6):
        return fa(out, res, x, w, rows, hidden, eps, None)

    assert fused(rows=0) == SUCCESS             # nothing to launch
    assert fused(rows=-1) == INVALID
    assert fused(eps=float("nan")) == INVALID
    assert fused(hidden=0) == UNSUPPORTED
    assert fused(hidden=4098) == UNSUPPORTED    # not a multiple of 4
    assert fused(hidden=2) == UNSUPPORTED
    assert fused(hidden=(1 << 20) + 4) == UNSUPPORTED
    assert fused(x=0) == INVALID
    assert fused(res=0) == INVALID
    assert fused(x=A + 8 * MB + 8) == MISALIGNED  # 8 bytes: fine for bf16, not here
    assert fused(w=A + 12 * MB + 4) == MISALIGNED
    assert fused(res=A + 8 * MB) == INVALID      # residual aliases x
    assert fused(out=A + 12 * MB) == INVALID     # out overlaps the weight
    assert fused(out=A + 8 * MB + 16) == INVALID  # out overlaps x without equalling it
    rf = L.norm_rmsnorm_fwd_f32
    assert rf(A, A + 4 * MB, A + 8 * MB, 8, 4102, 1e-6, None) == UNSUPPORTED
    assert rf(A, A + 4 * MB, A + 8 * MB + 16, 8, 4096, -1.0, None) == INVALID
    lf = L.norm_layernorm_fwd_f32
    assert lf(A, A + 4 * MB, 0, A + 8 * MB, A + 12 * MB, A + 13 * MB, 8, 4096, 1e-5,
              None) == INVALID                   # mean without rstd
    assert lf(A, A + 4 * MB, A + 4 * MB + 16, A + 8 * MB, A + 12 * MB, A + 13 * MB + 8, 8,
              4096, 1e-5, None) == MISALIGNED    # bias
    assert lf(A, A + 4 * MB, A + 4 * MB + 16, A + 8 * MB, A + 12 * MB, A + 13 * MB, 8, 4096,
              1e-5, None) == INVALID             # rstd overlaps mean (8 rows = 32 bytes)
    assert lf(A, A + 4 * MB + 2, A + 5 * MB, A + 8 * MB, A + 12 * MB, A + 13 * MB, 8, 4096,
              1e-5, None) == MISALIGNED          # mean 4-byte

    lb = L.norm_layernorm_bwd_f32
    WS = A + 64 * MB  # apart from every other argument below
    ws_need = rn.workspace_bytes_f32("layernorm_bwd", 8, 4096)

    def lbwd(dx=A, dw=A + 4 * MB, db=A + 5 * MB, dy=A + 8 * MB, x=A + 12 * MB, m=A + 16 * MB,
             r=A + 17 * MB, w=A + 18 * MB, ws=WS, ws_bytes=1 << 20, rows=8, hidden=4096):
        return lb(dx, dw, db, dy, x, m, r, w, ws, ws_bytes, rows, hidden, 0.0, None)

    assert lbwd(rows=-1) == INVALID
    assert lbwd(hidden=4094) == UNSUPPORTED
    assert lbwd(ws=0) == INVALID
    assert lbwd(db=0) == INVALID
    assert lbwd(m=0) == INVALID
    assert lbwd(dy=A + 8 * MB + 4) == MISALIGNED
    assert lbwd(ws=WS + 8) == MISALIGNED
    assert lbwd(dw=A + 4 * MB + 2) == MISALIGNED
    assert lbwd(dx=A + 8 * MB + 16) == INVALID   # dx overlaps dy without equalling it
    assert lbwd(dw=A + 16 * MB) == INVALID       # dweight aliases mean
    assert lbwd(ws=A + 12 * MB) == INVALID       # workspace inside x
    assert lbwd(ws_bytes=ws_need - 1) == WORKSPACE
    rb = L.norm_rmsnorm_bwd_f32
    assert rb(A, A + 4 * MB, A + 8 * MB, A + 12 * MB, A + 16 * MB, WS, 16, 8, 4096, 1e-6,
              None) == WORKSPACE
    assert rb(A, A + 4 * MB, A + 8 * MB, A + 12 * MB, A + 16 * MB + 8, WS, 1 << 20, 8, 4096,
              1e-6, None) == MISALIGNED          # weight
    fb = L.norm_fused_add_rmsnorm_bwd_f32
    assert fb(A, A + 4 * MB, A + 8 * MB, A + 12 * MB + 4, A + 16 * MB, A + 20 * MB, WS,
              1 << 20, 8, 4096, 1e-6, None) == MISALIGNED  # dres
    assert fb(A + 12 * MB, A + 4 * MB, A + 8 * MB, A + 12 * MB, A + 16 * MB, A + 20 * MB, WS,
              16, 8, 4096, 1e-6, None) == WORKSPACE  # ds == dres is allowed
    assert fb(A + 16 * MB, A + 4 * MB, A + 8 * MB, None, A + 16 * MB, A + 20 * MB, WS,
              1 << 20, 8, 4096, 1e-6, None) == INVALID   # ds aliases s


def test_f32_workspace_sizes():
    """Workspace of the fp32 backward: a slab of padded hidden fp32 per output
    column sum and row walker, plus the tiles' partial-sum exchange area (per
    walker 12 walk steps of 16 bytes a tile) over 16388 ... 262144 columns
    (tiles of 4096, at most 511 / tiles walkers), 8 bytes a row (the row
    sums) past that (tiles of 8192, at most 255 / tiles walkers); one tile
    up to 8192 columns (min(rows, 255) walkers); at 8196 ... 16384 columns
    min(rows, 256) walkers."""
    ws = rn.workspace_bytes_f32
    pad = lambda h: -(-h // 64) * 64
    assert ws("layernorm_bwd", 8192, 4096) == 255 * 2 * 4096 * 4
    assert ws("rmsnorm_bwd", 8192, 4096) == 255 * 4096 * 4
    assert ws("fused_add_rmsnorm_bwd", 3, 4100) == 3 * pad(4100) * 4
    assert ws("layernorm_bwd", 1000, 1 << 20) == 1 * 2 * (1 << 20) * 4 + 1000 * 8
    assert ws("layernorm_bwd", 1000, 1 << 18) == 7 * 2 * (1 << 18) * 4 + 7 * 12 * 64 * 16
    assert ws("layernorm_bwd", 1000, (1 << 18) + 4) == 7 * 2 * pad((1 << 18) + 4) * 4 + 1000 * 8
    assert ws("layernorm_bwd", 1000, 16384 + 4) == 102 * 2 * pad(16388) * 4 + 102 * 12 * 5 * 16
    # 8196 ... 16384 columns: the LDS-staged kernel, min(rows, 256) slabs
    assert ws("layernorm_bwd", 1000, 16384) == 256 * 2 * 16384 * 4
    assert ws("rmsnorm_bwd", 3, 8196) == 3 * pad(8196) * 4
    assert ws("fused_add_rmsnorm_bwd", 100, 12288) == 100 * 12288 * 4
    assert ws("layernorm_bwd", 1000, 8192) == 255 * 2 * 8192 * 4  # one tile
    assert ws("layernorm_bwd", 0, 4096) == 0
    assert ws("layernorm_bwd", 8, 4098) == 0
    assert ws("layernorm_fwd", 8, 4096) == 0      # a forward op
    # the largest any call needs stays under 32 MiB
    assert max(ws("layernorm_bwd", 1 << 20, h) for h in (4096, 8192, 8196, 65536, 1 << 20)) \
        < 32 << 20


def test_wide_backward_host_logic():
    """Backward rows above 16384 run on 512-lane workgroups with the row
    staged in LDS (5 to 8 16-byte accesses a lane, up to 32768; the fused op
    up to 7, 28672), then on the streamed kernels; narrower accesses stop at
    the register-resident kernels' widest rows."""
    for op in ("layernorm_bwd", "rmsnorm_bwd", "fused_add_rmsnorm_bwd"):
        for h in (16392, 20000, 24576, 28672) + ((32768,) if op != "fused_add_rmsnorm_bwd" else ()):
            c = rn.select_config(op, 8192, h)
            assert (c.threads_per_row, c.rows_per_block, c.grid, c.vector_elems) == \
                (512, 1, 256, 8), (op, h, c)
            v = -(-h // 4096)
            assert f"norm_bwd_wide_kernel<{v}," in rn.describe_config(op, 8192, h)
            assert rn.list_configs(op, h) == [rn.Cfg(512, 1, 0, 8)]
            outs = 2 if op == "layernorm_bwd" else 1
            padded = -(-h // 64) * 64
            assert rn.workspace_bytes(8192, h, op=op) == 256 * outs * padded * 4
            # (the RMSNorm query covers the fused op, which streams 32768)
            xch = 3 * 12 * 8 * 16 if op == "rmsnorm_bwd" and h == 32768 else 0
            assert rn.workspace_bytes(3, h, op=op) == 3 * outs * padded * 4 + xch
        # 9 accesses a lane: past the LDS-staged kernel, the streamed kernels
        c = rn.select_config(op, 8192, 32776)
        assert (c.threads_per_row, c.grid, c.vector_elems) == (512, 56, 8)  # 511 // 9 tiles
        assert "stream_bwd_tile_kernel" in rn.describe_config(op, 8192, 32776)
        with pytest.raises(rn.NormError):
            rn.select_config(op, 8192, 20002)   # 4-byte accesses: up to the run-time kernels
        assert rn.select_config(op, 8192, 16384 - 8).threads_per_row != 512 or \
            rn.select_config(op, 8192, 16384 - 8).rows_per_block == 1
    # the fused op at 8 accesses a lane (28680 ... 32768): the streamed kernels,
    # 8 column tiles of 4096, 511 // 8 walkers
    for h, tiles in ((28680, 8), (32768, 8)):
        c = rn.select_config("fused_add_rmsnorm_bwd", 8192, h)
        assert (c.threads_per_row, c.grid, c.vector_elems) == (512, 511 // tiles, 8), (h, c)
        d = rn.describe_config("fused_add_rmsnorm_bwd", 8192, h)
        assert "stream_bwd_tile_kernel" in d and "norm_bwd_wide_kernel" not in d
        assert rn.list_configs("fused_add_rmsnorm_bwd", h) == [rn.Cfg(512, 1, 0, 8)]
        # the query the two RMSNorm backward ops share covers both choices: the
        # plain op's 256 staged slabs, or (few rows) the fused op's walkers'
        # slabs and exchange slots
        padded = -(-h // 64) * 64
        assert rn.workspace_bytes(8192, h, op="fused_add_rmsnorm_bwd") == 256 * padded * 4
        assert rn.workspace_bytes(3, h, op="fused_add_rmsnorm_bwd") == \
            3 * padded * 4 + 3 * 12 * tiles * 16
        assert rn.workspace_bytes(3, h, op="rmsnorm_bwd") == \
            rn.workspace_bytes(3, h, op="fused_add_rmsnorm_bwd")
    assert "norm_bwd_wide_kernel<8," in rn.describe_config("rmsnorm_bwd", 8192, 32768)


def test_tuned_forward_table():
    """Measured launch shapes override the rules for some (op, compiled
    hidden, rows) cells, counted on a 256-CU part: entries measured at >= 1024
    rows stop at their row count (their gain needs whole workgroup waves)."""
    sel = lambda op, rows, h, cu=256: rn.select_config(op, rows, h, cu_count=cu)
    assert sel("rmsnorm_fwd", 2048, 2048) == rn.Cfg(256, 1, 0, 8)  # a run-time shape
    assert sel("rmsnorm_fwd", 1500, 2048) == rn.Cfg(256, 1, 0, 8)
    assert sel("rmsnorm_fwd", 2049, 2048) != rn.Cfg(256, 1, 0, 8)   # past the measured row count
    assert sel("rmsnorm_fwd", 1024, 2048, cu=128) == rn.Cfg(256, 1, 0, 8)  # = 2048 on 256 CUs
    assert sel("rmsnorm_fwd", 1024, 16384) == rn.Cfg(512, 1, 256, 0)  # the RMSNorm ring rule
    assert sel("rmsnorm_fwd", 1024, 8192) != rn.Cfg(512, 1, 256, 0)   # not below 2048 rows there
    assert sel("fused_add_rmsnorm", 64, 4096) == rn.Cfg(512, 1, 0, 8)  # the run-time kernel
    assert sel("fused_add_rmsnorm", 8192, 4096) == rn.Cfg(128, 2, 0, 0)  # the rules
    assert sel("layernorm_fwd", 64, 8192) == rn.Cfg(256, 1, 0, 0)
    assert sel("layernorm_fwd", 8192, 12288) == rn.Cfg(512, 1, 256, 0)  # the ring rule
    assert sel("layernorm_fwd", 1024, 12288) == rn.Cfg(512, 1, 256, 0)
    assert sel("layernorm_fwd", 64, 12288) == rn.Cfg(256, 1, 0, 0)  # an entry below the ring
    # every table choice runs: a listed shape of its (op, hidden)
    for op in ("fused_add_rmsnorm", "rmsnorm_fwd", "layernorm_fwd"):
        for h in rn.HIDDEN_SIZES:
            listed = rn.list_configs(op, h)
            for rows in (1, 3, 16, 40, 64, 100, 256, 300, 700, 1024, 1500, 2048, 3000, 4096,
                         6000, 8192):
                c = sel(op, rows, h)
                assert rn.Cfg(c.threads_per_row, c.rows_per_block, 0, c.vector_elems) in \
                    [rn.Cfg(k.threads_per_row, k.rows_per_block, 0, k.vector_elems)
                     for k in listed], (op, h, rows, c)


def test_missing_library_raises_and_product_never_touches_the_oracle(monkeypatch, tmp_path):
    """No fallback: without librownorm.so every entry of the binding raises,
    and no module of the package imports the oracle."""
    import ast
    import glob
    import os

    monkeypatch.setattr(rn, "_lib", None)
    monkeypatch.setattr(rn, "LIB_PATH", str(tmp_path / "librownorm.so"))
    with pytest.raises(ImportError, match="missing"):
        rn.lib()
    with pytest.raises(ImportError):
        rn.select_config("fused_add_rmsnorm", 8, 4096)
    pkg = os.path.dirname(os.path.abspath(rn.__file__))
    for path in glob.glob(os.path.join(pkg, "**", "*.py"), recursive=True):
        tree = ast.parse(open(path).read())
        for node in ast.walk(tree):
            names = [a.name for a in node.names] if isinstance(node, (ast.Import,
                                                                      ast.ImportFrom)) else []
            if isinstance(node, ast.ImportFrom) and node.module:
                names.append(node.module)
            assert not any(n == "oracle" or n.startswith("oracle.") for n in names), path
