"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle,
element by element, on the seeded workloads and on edge cases.  Rules in
parity.py.  Every test here needs an MI355X."""
import os

import numpy as np
import pytest
import torch

import oracle
import parity as P
import row_normalization_persistent_amd as rn
from row_normalization_persistent_amd import workloads as wl

pytestmark = pytest.mark.gpu

NT = min(16, os.cpu_count() or 1)
DEV = "cuda"


def dev(bits):
    return wl.to_device_bf16(bits, DEV)


def host(t):
    torch.cuda.synchronize()
    return wl.from_device_bf16(t)


# ------------------------------------------------------------------ fused
def run_fused(inp, cfg=None, out_is_x=False):
    x, r, w = dev(inp["x"]), dev(inp["r"]), dev(inp["w"])
    out = x if out_is_x else None
    out, res = rn.fused_add_rmsnorm(x, r, w, inp["eps"], out=out, cfg=cfg)
    return host(out), host(res)


def check_fused(inp, cfg=None, out_is_x=False, what="fused"):
    ref, res_ref, _ = oracle.fused_add_rmsnorm(inp["x"], inp["r"], inp["w"], inp["eps"], NT)
    out, res = run_fused(inp, cfg, out_is_x)
    P.assert_bits_equal(res, res_ref, f"{what}: residual")
    return P.assert_bf16_close(out, ref, f"{what}: out")


def test_fused_small_config():
    """rows=16, hidden=4096, seed 0."""
    check_fused(wl.fused_inputs(16, 4096, seed=0))


@pytest.mark.parametrize("rows", wl.FUSED_SWEEP_ROWS)
def test_fused_batch_sweep(rows):
    """hidden=4096, rows 1..8192, in the launch shape the library picks."""
    check_fused(wl.fused_inputs(rows, 4096, seed=0), what=f"fused rows={rows}")


@pytest.mark.parametrize("hidden", rn.HIDDEN_SIZES)
def test_fused_every_compiled_shape(hidden):
    """Every compiled (lanes, rows-per-workgroup) shape, on a ragged row count
    (not a multiple of any rows-per-workgroup) that spans several workgroups."""
    inp = wl.fused_inputs(37, hidden, seed=1)
    for c in rn.list_configs("fused_add_rmsnorm", hidden):
        check_fused(inp, cfg=c, what=f"fused h={hidden} {c}")


def test_fused_in_place_out():
    check_fused(wl.fused_inputs(64, 4096, seed=2), out_is_x=True, what="fused out==x")


# (op, rows, hidden) where the library runs the late-weights variant of the
# forward kernels on a 256-CU part (weight and bias loaded after the row's
# statistics), with ragged row counts where the bucket allows
LATE_WEIGHT_CASES = [("layernorm_fwd", 2047, 4096), ("rmsnorm_fwd", 4095, 1024),
                     ("rmsnorm_fwd", 4093, 2048), ("rmsnorm_fwd", 1023, 8192),
                     ("fused_add_rmsnorm", 2047, 1024), ("fused_add_rmsnorm", 4095, 1024),
                     ("fused_add_rmsnorm", 2046, 4096), ("fused_add_rmsnorm", 3, 8192),
                     ("fused_add_rmsnorm", 501, 12288), ("fused_add_rmsnorm", 1, 16384),
                     ("fused_add_rmsnorm", 61, 16384), ("fused_add_rmsnorm", 501, 16384),
                     # run-time hidden: 2 to 4 workgroups per CU
                     ("rmsnorm_fwd", 2047, 6144), ("layernorm_fwd", 1023, 7168),
                     ("fused_add_rmsnorm", 2045, 5120), ("rmsnorm_fwd", 1001, 5118),
                     ("layernorm_fwd", 999, 3070), ("fused_add_rmsnorm", 1001, 6142)]


@pytest.mark.parametrize("op,rows,hidden", LATE_WEIGHT_CASES)
def test_fwd_late_weight_variant(op, rows, hidden):
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    if cu != 256:
        pytest.skip(f"the late-weights buckets are given for 256 CUs; this part has {cu}")
    assert "_lw_kernel<" in rn.describe_config(op, rows, hidden), (op, rows, hidden)
    if op == "layernorm_fwd":
        check_lnf(wl.layernorm_fwd_inputs(rows, hidden, seed=21), what=f"late {rows}x{hidden}")
    elif op == "rmsnorm_fwd":
        check_rms(wl.rmsnorm_inputs(rows, hidden, seed=21), what=f"late {rows}x{hidden}")
    else:
        check_fused(wl.fused_inputs(rows, hidden, seed=21), what=f"late {rows}x{hidden}")


# ------------------------------------------------------------------ rmsnorm
def check_rms(inp, cfg=None, what="rmsnorm", in_place=False):
    ref, _ = oracle.rmsnorm_fwd(inp["x"], inp["w"], inp["eps"], NT)
    x, w = dev(inp["x"]), dev(inp["w"])
    out = rn.rmsnorm_fwd(x, w, inp["eps"], out=x if in_place else None, cfg=cfg)
    return P.assert_bf16_close(host(out), ref, what)


@pytest.mark.parametrize("hidden", wl.RMSNORM_HIDDEN)
@pytest.mark.parametrize("rows", wl.RMSNORM_ROWS)
def test_rmsnorm_config(hidden, rows):
    """x ~ N(0,1) with 1% outlier channels x50, w ~ N(1,0.1), eps 1e-6."""
    check_rms(wl.rmsnorm_inputs(rows, hidden, seed=0), what=f"rmsnorm {rows}x{hidden}")


@pytest.mark.parametrize("hidden", [8192, 12288, 16384])
def test_rmsnorm_fwd_ring_shapes_and_grids(hidden):
    """The RMSNorm persistent ring kernels: every compiled lane count, one
    workgroup, walks of 11, 8, 5, 4, 3 and 2 rows (75 rows over 7, 10, 15, 19,
    37 or 38 workgroups: every compiled ring depth, full and partial ring
    steps), idle
    workgroups (300 > rows); in place too.  Outlier channels as in the RMSNorm
    workload."""
    inp = wl.rmsnorm_inputs(75, hidden, seed=16)
    rings = [c for c in rn.list_configs("rmsnorm_fwd", hidden) if c.grid > 0]
    assert rings
    assert len({c.threads_per_row for c in rings}) == len(rings)
    for c in rings:
        for grid in (1, 7, 10, 15, 19, 37, 38, 300):
            cfg = rn.Cfg(c.threads_per_row, 1, grid, 0)
            check_rms(inp, cfg=cfg, what=f"rmsnorm ring h={hidden} {cfg}")
        check_rms(inp, cfg=rn.Cfg(c.threads_per_row, 1, 7, 0), in_place=True,
                  what=f"rmsnorm ring h={hidden} lanes={c.threads_per_row} in place")


@pytest.mark.parametrize("rows,hidden", [(1024, 16384), (2048, 12288), (4096, 8192),
                                         (1100, 16384), (320, 16384), (401, 12288),
                                         (511, 8192)])
def test_rmsnorm_fwd_ring_in_library_choice(rows, hidden):
    """Sizes where the library picks the RMSNorm ring kernel by itself."""
    assert rn.select_config("rmsnorm_fwd", rows, hidden).grid > 0
    assert "rmsnorm_fwd_ring_kernel" in rn.describe_config("rmsnorm_fwd", rows, hidden)
    check_rms(wl.rmsnorm_inputs(rows, hidden, seed=17), what=f"rmsnorm ring {rows}x{hidden}")


@pytest.mark.parametrize("hidden", rn.HIDDEN_SIZES)
def test_rmsnorm_every_compiled_shape(hidden):
    inp = wl.rmsnorm_inputs(37, hidden, seed=3)
    for c in rn.list_configs("rmsnorm_fwd", hidden):
        check_rms(inp, cfg=c, what=f"rmsnorm h={hidden} {c}")
    check_rms(inp, what="rmsnorm in place", in_place=True)


# ------------------------------------------------------------------ layernorm fwd
def check_lnf(inp, cfg=None, what="layernorm_fwd", with_stats=True):
    x_bits, w_bits, b_bits = inp["x"], inp["w"], inp["b"]
    ref, mean_ref, rstd_ref = oracle.layernorm_fwd(x_bits, w_bits, b_bits, inp["eps"], NT)
    y, mean, rstd = rn.layernorm_fwd(dev(x_bits), dev(w_bits), dev(b_bits), inp["eps"], cfg=cfg,
                                     with_stats=with_stats)
    xd, wd, bd = P.bits_to_f64(x_bits), P.bits_to_f64(w_bits), P.bits_to_f64(b_bits)
    scale = P.layernorm_y_scale(xd, mean_ref, rstd_ref, wd, bd)
    stats = P.assert_bf16_close(host(y), ref, f"{what}: y", floor_scale=scale)
    if with_stats:
        P.assert_f32_close(mean.cpu().numpy(), mean_ref, f"{what}: mean")
        P.assert_f32_close(rstd.cpu().numpy(), rstd_ref, f"{what}: rstd")
    return stats


@pytest.mark.parametrize("hidden", wl.LAYERNORM_FWD_HIDDEN)
def test_layernorm_fwd_config(hidden):
    """rows=2048, x ~ N(0.5,2), w ~ N(1,0.1), b ~ N(0,0.1), eps 1e-5."""
    stats = check_lnf(wl.layernorm_fwd_inputs(wl.LAYERNORM_FWD_ROWS, hidden, seed=0),
                      what=f"layernorm_fwd h={hidden}")
    P.report_floor(f"layernorm_fwd {wl.LAYERNORM_FWD_ROWS}x{hidden} y", stats)


@pytest.mark.parametrize("hidden", rn.HIDDEN_SIZES)
def test_layernorm_fwd_every_compiled_shape(hidden):
    inp = wl.layernorm_fwd_inputs(37, hidden, seed=4)
    for c in rn.list_configs("layernorm_fwd", hidden):
        check_lnf(inp, cfg=c, what=f"layernorm_fwd h={hidden} {c}")
    check_lnf(inp, what="layernorm_fwd without stats", with_stats=False)


@pytest.mark.parametrize("hidden", [2048, 4096, 8192, 12288, 16384])
def test_layernorm_fwd_ring_shapes_and_grids(hidden):
    """The persistent ring kernels: every compiled lane count, grids of one
    workgroup, ragged walks (75 rows over 7, 10, 15, 19, 37 or 38 workgroups:
    walks of 11, 8, 5, 4, 3 and 2 rows, so every compiled ring depth runs, with
    full and partial ring steps) and idle workgroups (300 > rows); in place too."""
    inp = wl.layernorm_fwd_inputs(75, hidden, seed=14)
    rings = [c for c in rn.list_configs("layernorm_fwd", hidden) if c.grid > 0]
    assert rings
    assert len({c.threads_per_row for c in rings}) == len(rings)  # one entry per lane count
    for c in rings:
        for grid in (1, 7, 10, 15, 19, 37, 38, 300):
            cfg = rn.Cfg(c.threads_per_row, 1, grid, 0)
            check_lnf(inp, cfg=cfg, what=f"layernorm ring h={hidden} {cfg}")
        check_lnf(inp, cfg=c, what=f"layernorm ring h={hidden} no stats", with_stats=False)
    ref, _, _ = oracle.layernorm_fwd(inp["x"], inp["w"], inp["b"], inp["eps"], NT)
    x = dev(inp["x"])
    rn.layernorm_fwd(x, dev(inp["w"]), dev(inp["b"]), inp["eps"], y=x,
                     cfg=rn.Cfg(rings[0].threads_per_row, 1, 7, 0))
    xd = P.bits_to_f64(inp["x"])
    _, mean_ref, rstd_ref = oracle.layernorm_fwd(inp["x"], inp["w"], inp["b"], inp["eps"], NT)
    scale = P.layernorm_y_scale(xd, mean_ref, rstd_ref, P.bits_to_f64(inp["w"]),
                                P.bits_to_f64(inp["b"]))
    P.assert_bf16_close(host(x), ref, "layernorm ring in place", floor_scale=scale)


@pytest.mark.parametrize("rows,hidden", [(2048, 16384), (1100, 12288), (8192, 4096),
                                         (320, 16384), (479, 16384)])
def test_layernorm_fwd_ring_in_library_choice(rows, hidden):
    """Sizes where the library picks the ring kernel by itself."""
    assert rn.select_config("layernorm_fwd", rows, hidden).grid > 0
    check_lnf(wl.layernorm_fwd_inputs(rows, hidden, seed=15),
              what=f"layernorm_fwd ring {rows}x{hidden}")


# ------------------------------------------------------------------ layernorm bwd
def lnb_inputs(rows, hidden, seed=0):
    inp = wl.layernorm_bwd_inputs(rows, hidden, seed)
    _, mean, rstd = oracle.layernorm_fwd(inp["x"], inp["w"], np.zeros(hidden, np.uint16),
                                         inp["eps"], NT)
    inp["mean"] = mean.astype(np.float32)
    inp["rstd"] = rstd.astype(np.float32)
    return inp


def run_lnb(inp, cfg=None, dx_is_dy=False):
    dy = dev(inp["dy"])
    args = (dy, dev(inp["x"]), torch.from_numpy(inp["mean"]).to(DEV),
            torch.from_numpy(inp["rstd"]).to(DEV), dev(inp["w"]))
    dx, dw, db = rn.layernorm_bwd(*args, eps=inp["eps"], dx=dy if dx_is_dy else None, cfg=cfg)
    return host(dx), dw.cpu().numpy(), db.cpu().numpy()


def check_lnb(inp, cfg=None, what="layernorm_bwd", dx_is_dy=False):
    dx_ref, dw_ref, db_ref = oracle.layernorm_bwd(inp["dy"], inp["x"], inp["mean"], inp["rstd"],
                                                  inp["w"], NT)
    dx, dw, db = run_lnb(inp, cfg, dx_is_dy)
    xd, dyd, wd = P.bits_to_f64(inp["x"]), P.bits_to_f64(inp["dy"]), P.bits_to_f64(inp["w"])
    mean, rstd = inp["mean"].astype(np.float64), inp["rstd"].astype(np.float64)
    scale = P.layernorm_dx_scale(xd, dyd, wd, mean, rstd)
    stats = P.assert_bf16_close(dx, dx_ref, f"{what}: dx", floor_scale=scale)
    xhat = (xd - mean[:, None]) * rstd[:, None]
    P.assert_colsum_close(dw, dw_ref, ((dyd * xhat) ** 2).sum(0), f"{what}: dweight")
    P.assert_colsum_close(db, db_ref, (dyd ** 2).sum(0), f"{what}: dbias")
    return stats, (dx, dw, db)


@pytest.mark.parametrize("hidden", wl.LAYERNORM_BWD_HIDDEN)
def test_layernorm_bwd_config(hidden):
    """rows=8192, x, dy ~ N(0,1), w ~ N(1,0.1), mean/rstd from x with eps 1e-5."""
    stats, _ = check_lnb(lnb_inputs(wl.LAYERNORM_BWD_ROWS, hidden, seed=0),
                         what=f"layernorm_bwd h={hidden}")
    P.report_floor(f"layernorm_bwd {wl.LAYERNORM_BWD_ROWS}x{hidden} dx", stats)


@pytest.mark.parametrize("hidden", rn.HIDDEN_SIZES)
def test_layernorm_bwd_every_compiled_shape(hidden):
    inp = lnb_inputs(75, hidden, seed=5)
    for c in rn.list_configs("layernorm_bwd", hidden):
        for grid in (1, 7, 75, 200):  # one slab, ragged, one row each, idle workgroups
            check_lnb(inp,
                      cfg=rn.Cfg(c.threads_per_row, c.rows_per_block, grid, c.vector_elems),
                      what=f"layernorm_bwd h={hidden} {c} grid={grid}")
    check_lnb(inp, what="layernorm_bwd dx==dy", dx_is_dy=True)


def test_layernorm_bwd_deterministic():
    inp = lnb_inputs(1024, 4096, seed=6)
    _, first = check_lnb(inp)
    for _ in range(2):
        again = run_lnb(inp)
        for a, b in zip(first, again):
            assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


def test_layernorm_bwd_zero_rows_zero_fills():
    h = 4096
    dw = torch.full((h,), float("nan"), device=DEV)
    db = torch.full((h,), float("nan"), device=DEV)
    e = torch.empty(0, h, dtype=torch.bfloat16, device=DEV)
    s = torch.empty(0, dtype=torch.float32, device=DEV)
    w = torch.ones(h, dtype=torch.bfloat16, device=DEV)
    rn.layernorm_bwd(e, e, s, s, w, dweight=dw, dbias=db)
    torch.cuda.synchronize()
    assert (dw.cpu() == 0).all() and (db.cpu() == 0).all()


# ------------------------------------------------------------------ edge cases
def test_edge_rows():
    """Constant, zero, one-hot, tiny and huge rows through every forward op."""
    h = 4096
    rng = np.random.default_rng(9)
    rows = np.zeros((8, h), np.float32)
    rows[0] = 1.0
    rows[1] = -3.5
    rows[2] = 0.0
    rows[3, 17] = 2.5
    rows[4] = rng.standard_normal(h) * 1e-30   # tiny: squares underflow fp32
    rows[5] = rng.standard_normal(h) * 1e15    # huge: squares stay finite in fp32
    rows[6] = rng.standard_normal(h) * 1e-3
    rows[7, ::2] = 1.0
    x = wl.bf16_bits(rows)
    w = wl.bf16_bits(1.0 + 0.1 * rng.standard_normal(h).astype(np.float32))
    b = wl.bf16_bits(0.1 * rng.standard_normal(h).astype(np.float32))
    eps = wl.EPS_RMS
    check_rms({"x": x, "w": w, "eps": eps}, what="rmsnorm edge rows")
    zero_r = np.zeros_like(x)
    check_fused({"x": x, "r": zero_r, "w": w, "eps": eps}, what="fused edge rows")
    check_lnf({"x": x, "w": w, "b": b, "eps": wl.EPS_LN}, what="layernorm edge rows")


def test_fused_residual_bit_exact_on_hard_sums():
    """Ties, cancellation, subnormal sums and wide exponent gaps in x + r."""
    h = 4096
    rng = np.random.default_rng(10)
    x = wl.bf16_bits(rng.standard_normal((64, h)).astype(np.float32))
    gaps = np.exp2(rng.integers(-40, 40, size=(64, h))).astype(np.float32)
    r = wl.bf16_bits(rng.standard_normal((64, h)).astype(np.float32) * gaps)
    r[:8] = x[:8] ^ np.uint16(0x8000)                      # exact cancellation
    sub = (rng.integers(1, 128, size=(8, h)) * np.float32(2.0 ** -133)).astype(np.float32)
    x[8:16] = wl.bf16_bits(sub)                             # bf16 subnormals
    r[8:16] = wl.bf16_bits(sub[::-1])
    x[16:24] = wl.bf16_bits(np.float32(1.0) + np.zeros((8, h), np.float32))
    r[16:24] = wl.bf16_bits(np.full((8, h), 2.0 ** -8, np.float32))  # ties at 1 + 2^-8
    inp = {"x": x, "r": r, "w": wl.bf16_bits(np.ones(h, np.float32)), "eps": wl.EPS_RMS}
    _, res_ref, _ = oracle.fused_add_rmsnorm(x, r, inp["w"], inp["eps"], NT)
    _, res = run_fused(inp)
    P.assert_bits_equal(res, res_ref, "residual on hard sums")


def test_rmsnorm_scale_invariance_on_gpu():
    """RMSNorm(2^k x) at eps = 0 stays within 2 ulp of the oracle's RMSNorm(x)."""
    inp = wl.rmsnorm_inputs(16, 8192, seed=11)
    ref, _ = oracle.rmsnorm_fwd(inp["x"], inp["w"], 0.0, NT)
    for k in (-6, 5):
        xs = wl.bf16_bits((P.bits_to_f64(inp["x"]) * 2.0 ** k).astype(np.float32))
        out = rn.rmsnorm_fwd(dev(xs), dev(inp["w"]), 0.0)
        P.assert_bf16_close(host(out), ref, f"scale 2^{k}")


def _guarded(n, pad=4096, fill=0x7FC1):
    """A bf16 buffer of n elements with `pad` guard elements on each side."""
    big = torch.full((n + 2 * pad,), fill, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    return big, big[pad:pad + n]


def _guards_intact(big, n, pad=4096, fill=0x7FC1):
    b = big.view(torch.int16).cpu().numpy()
    return (b[:pad] == fill).all() and (b[pad + n:] == fill).all()


@pytest.mark.parametrize("rows", [1, 5, 37, 300])
def test_no_write_outside_outputs_and_every_output_written(rows):
    """Guard regions around every bf16 output stay untouched, and outputs
    pre-filled with NaN are fully overwritten (parity would fail otherwise)."""
    h = 4096
    inp = wl.fused_inputs(rows, h, seed=12)
    n = rows * h
    ref, res_ref, _ = oracle.fused_add_rmsnorm(inp["x"], inp["r"], inp["w"], inp["eps"], NT)
    big_o, out = _guarded(n)
    big_r, res = _guarded(n)
    res.copy_(dev(inp["r"]).view(-1))
    for c in rn.list_configs("fused_add_rmsnorm", h):
        out.view(torch.int16).fill_(0x7FC1)
        res.copy_(dev(inp["r"]).view(-1))
        rn.fused_add_rmsnorm(dev(inp["x"]), res.view(rows, h), dev(inp["w"]), inp["eps"],
                             out=out.view(rows, h), cfg=c)
        torch.cuda.synchronize()
        assert _guards_intact(big_o, n) and _guards_intact(big_r, n), c
        P.assert_bits_equal(host(res).reshape(rows, h), res_ref, f"guarded residual {c}")
        P.assert_bf16_close(host(out).reshape(rows, h), ref, f"guarded out {c}")
    linp = lnb_inputs(rows, h, seed=13)
    big_dx, dx = _guarded(n)
    for c in rn.list_configs("layernorm_bwd", h):
        dx.view(torch.int16).fill_(0x7FC1)
        dy = dev(linp["dy"])
        rn.layernorm_bwd(dy, dev(linp["x"]), torch.from_numpy(linp["mean"]).to(DEV),
                         torch.from_numpy(linp["rstd"]).to(DEV), dev(linp["w"]),
                         dx=dx.view(rows, h),
                         cfg=rn.Cfg(c.threads_per_row, c.rows_per_block, 0, c.vector_elems))
        torch.cuda.synchronize()
        assert _guards_intact(big_dx, n), c
        assert not torch.isnan(dx.float()).any().item(), c


def test_binding_refuses_tensors_off_the_current_device(monkeypatch):
    """The library launches on the current device: the binding refuses a call
    whose tensors live elsewhere, before anything is enqueued (the current
    device is stubbed to another index, as a one-GPU machine has no second)."""
    x = torch.zeros(4, 4096, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(4096, dtype=torch.bfloat16, device=DEV)
    out = torch.full_like(x, 3.0)
    rn.rmsnorm_fwd(x, w, 1e-6, out=out)  # accepted on the current device
    torch.cuda.synchronize()
    assert bool((out == 0).all())
    out.fill_(3.0)
    monkeypatch.setattr(rn, "_current_device", lambda: x.get_device() + 1)
    with pytest.raises(ValueError, match="current device"):
        rn.rmsnorm_fwd(x, w, 1e-6, out=out)
    with pytest.raises(ValueError, match="current device"):
        rn.layernorm_bwd(x, x, torch.zeros(4, device=DEV), torch.ones(4, device=DEV), w)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())  # nothing ran
