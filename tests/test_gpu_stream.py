"""GPU parity of the streamed kernels (rows wider than one workgroup's
registers hold: forward past 65536 columns, LayerNorm forward past 49152,
the backward operations past 32768; 16-byte rows up to 2^20 columns) and of
the LDS-staged forward (the fused op's and RMSNorm's rows of those that
registers and LDS hold)
against the CPU oracle, through the C ABI: the library's own choice over
ragged widths and row counts, strided and in-place rows, explicit row-walker
counts of the backward, bitwise run-to-run determinism, the row-split entry
points falling back to them, and the allocation-free LayerNorm backward on
them.  Rules in parity.py."""
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


def strided(bits, ld):
    """A [rows, hidden] device view with row stride ld holding `bits`."""
    rows, h = bits.shape
    base = torch.full((rows, ld), 7.0, dtype=torch.bfloat16, device=DEV)
    base[:, :h] = dev(bits)
    return base[:, :h]


# ------------------------------------------------------------------ forward
FWD_CASES = [("fused_add_rmsnorm", 65544, 37), ("fused_add_rmsnorm", 131072, 300),
             ("fused_add_rmsnorm", 1 << 20, 3), ("rmsnorm_fwd", 65544, 3), ("rmsnorm_fwd", 73728, 5),
             ("rmsnorm_fwd", 73736, 4),
             ("rmsnorm_fwd", 100000, 37), ("rmsnorm_fwd", 262144, 64),
             ("layernorm_fwd", 49160, 37), ("layernorm_fwd", 65536, 300), ("layernorm_fwd", 65544, 9),
             ("fused_add_rmsnorm", 98304, 11), ("fused_add_rmsnorm", 98312, 5),
             ("layernorm_fwd", 100000, 1), ("layernorm_fwd", 1 << 20, 3)]


def fwd_inputs(op, rows, h, seed):
    if op == "fused_add_rmsnorm":
        return wl.fused_inputs(rows, h, seed)
    if op == "rmsnorm_fwd":
        return wl.rmsnorm_inputs(rows, h, seed)
    return wl.layernorm_fwd_inputs(rows, h, seed)


def check_fwd(op, inp, got, what):
    if op == "fused_add_rmsnorm":
        ref, res_ref, _ = oracle.fused_add_rmsnorm(inp["x"], inp["r"], inp["w"], inp["eps"], NT)
        P.assert_bits_equal(got["res"], res_ref, f"{what}: residual")
        P.assert_bf16_close(got["out"], ref, f"{what}: out")
    elif op == "rmsnorm_fwd":
        ref, _ = oracle.rmsnorm_fwd(inp["x"], inp["w"], inp["eps"], NT)
        P.assert_bf16_close(got["out"], ref, what)
    else:
        ref, mean_ref, rstd_ref = oracle.layernorm_fwd(inp["x"], inp["w"], inp["b"], inp["eps"],
                                                       NT)
        xd, wd, bd = P.bits_to_f64(inp["x"]), P.bits_to_f64(inp["w"]), P.bits_to_f64(inp["b"])
        scale = P.layernorm_y_scale(xd, mean_ref, rstd_ref, wd, bd)
        P.assert_bf16_close(got["out"], ref, f"{what}: y", floor_scale=scale)
        P.assert_f32_close(got["mean"], mean_ref, f"{what}: mean")
        P.assert_f32_close(got["rstd"], rstd_ref, f"{what}: rstd")


def run_fwd(op, inp, ld=None, in_place=False, split=None):
    h = inp["x"].shape[1]
    x = strided(inp["x"], ld) if ld else dev(inp["x"])
    kw = {} if split is None else {"split": split,
                                   "workspace": torch.zeros(rn.split_workspace_bytes(len(x)),
                                                            dtype=torch.uint8, device=DEV)}
    out = x if in_place else None
    if op == "fused_add_rmsnorm":
        r = strided(inp["r"], ld) if ld else dev(inp["r"])
        out, r = rn.fused_add_rmsnorm(x, r, dev(inp["w"]), inp["eps"], out=out, **kw)
        return {"out": host(out), "res": host(r)}
    if op == "rmsnorm_fwd":
        return {"out": host(rn.rmsnorm_fwd(x, dev(inp["w"]), inp["eps"], out=out, **kw))}
    y, mean, rstd = rn.layernorm_fwd(x, dev(inp["w"]), dev(inp["b"]), inp["eps"], y=out, **kw)
    return {"out": host(y), "mean": mean.cpu().numpy(), "rstd": rstd.cpu().numpy()}


@pytest.mark.parametrize("op,h,rows", FWD_CASES)
def test_stream_forward(op, h, rows):
    d = rn.describe_config(op, rows, h)
    assert "stream_fwd_kernel" in d or "stage_fwd_kernel" in d, d
    inp = fwd_inputs(op, rows, h, seed=h + rows)
    check_fwd(op, inp, run_fwd(op, inp), f"{op} {rows}x{h}")


# The LDS-staged forward (fused add + RMSNorm and RMSNorm rows past the
# on-chip kernels that registers and LDS hold whole): each at its first width
# (RMSNorm's: where the streamed kernel would read 1/16 of the row twice), a
# ragged width and its widest, over one row, fewer rows than workgroups,
# exactly as many, and walks of two and three rows; the widths just outside
# the band go to the streamed kernel.
STAGE_CASES = [("fused_add_rmsnorm", 65544, 300), ("fused_add_rmsnorm", 73736, 1),
               ("fused_add_rmsnorm", 81920, 600), ("rmsnorm_fwd", 69912, 257),
               ("rmsnorm_fwd", 98312, 37), ("rmsnorm_fwd", 114688, 513),
               ("rmsnorm_fwd", 73736, 256)]


@pytest.mark.parametrize("op,h,rows", STAGE_CASES)
def test_staged_forward(op, h, rows):
    assert "stage_fwd_kernel" in rn.describe_config(op, rows, h)
    inp = fwd_inputs(op, rows, h, seed=2 * h + rows)
    check_fwd(op, inp, run_fwd(op, inp), f"{op} staged {rows}x{h}")


@pytest.mark.parametrize("op,h", [("fused_add_rmsnorm", 81928), ("rmsnorm_fwd", 114696),
                                  ("rmsnorm_fwd", 69904)])
def test_first_width_past_the_staged_forward(op, h):
    assert "stream_fwd_kernel" in rn.describe_config(op, 300, h)
    inp = fwd_inputs(op, 300, h, seed=h)
    check_fwd(op, inp, run_fwd(op, inp), f"{op} streamed 300x{h}")


@pytest.mark.parametrize("op", ["fused_add_rmsnorm", "rmsnorm_fwd"])
def test_staged_forward_bitwise_run_to_run(op):
    """Outputs of two calls are bitwise equal (no order-dependent arithmetic),
    over a walk of several rows a workgroup."""
    h, rows = 73736, 700
    inp = fwd_inputs(op, rows, h, seed=11)
    a, b = run_fwd(op, inp), run_fwd(op, inp)
    for k in a:
        assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), f"{op} {k}"


@pytest.mark.parametrize("op", ["fused_add_rmsnorm", "rmsnorm_fwd", "layernorm_fwd"])
@pytest.mark.parametrize("h", [65536 + 64, 131072 + 64])  # LDS-staged (not LayerNorm), streamed
def test_stream_forward_strided_and_in_place(op, h):
    rows = 45 if h < 100000 else 9
    inp = fwd_inputs(op, rows, h, seed=3)
    check_fwd(op, inp, run_fwd(op, inp, ld=h + 136), f"{op} strided")
    check_fwd(op, inp, run_fwd(op, inp, in_place=True), f"{op} in place")


@pytest.mark.parametrize("op", ["fused_add_rmsnorm", "rmsnorm_fwd", "layernorm_fwd"])
def test_stream_forward_behind_the_row_split(op):
    """The row-split entry point splits few wide rows and hands the rest (too
    many rows to split) to the streamed kernel; both agree with the oracle."""
    h = 131072
    for rows in (2, 100):
        k, _ = rn.select_split(op, rows, h)
        assert (k > 1) == (rows == 2), (op, rows, k)
        inp = fwd_inputs(op, rows, h, seed=rows)
        check_fwd(op, inp, run_fwd(op, inp, split=0), f"{op} split entry {rows}x{h}")


# ------------------------------------------------------------------ backward
# both sides of 262144 columns: the widest rows whose tiles exchange partial
# row sums, and the first that take the row sums kernel and read x, dy again
BWD_CASES = [(32776, 37), (40000, 300), (65536, 300), (100000, 37), (131072, 1),
             (262144, 11), (262152, 5), (1 << 20, 3)]


def lnb_inputs(rows, h, seed):
    inp = wl.layernorm_bwd_inputs(rows, h, seed)
    _, mean, rstd = oracle.layernorm_fwd(inp["x"], inp["w"], np.zeros(h, np.uint16), inp["eps"],
                                         NT)
    inp["mean"], inp["rstd"] = mean.astype(np.float32), rstd.astype(np.float32)
    return inp


def run_lnb(inp, cfg=None, alias=False, noalloc=False):
    dy = dev(inp["dy"])
    args = (dy, dev(inp["x"]), torch.from_numpy(inp["mean"]).to(DEV),
            torch.from_numpy(inp["rstd"]).to(DEV), dev(inp["w"]))
    if noalloc:
        dx, dw, db = rn.layernorm_bwd_noalloc(*args)
    else:
        dx, dw, db = rn.layernorm_bwd(*args, dx=dy if alias else None, cfg=cfg)
    return host(dx), dw.cpu().numpy(), db.cpu().numpy()


def check_lnb(inp, got, what):
    dx_ref, dw_ref, db_ref = oracle.layernorm_bwd(inp["dy"], inp["x"], inp["mean"], inp["rstd"],
                                                  inp["w"], NT)
    xd, dyd, wd = P.bits_to_f64(inp["x"]), P.bits_to_f64(inp["dy"]), P.bits_to_f64(inp["w"])
    mean, rstd = inp["mean"].astype(np.float64), inp["rstd"].astype(np.float64)
    scale = P.layernorm_dx_scale(xd, dyd, wd, mean, rstd)
    P.assert_bf16_close(got[0], dx_ref, f"{what}: dx", floor_scale=scale)
    xhat = (xd - mean[:, None]) * rstd[:, None]
    P.assert_colsum_close(got[1], dw_ref, ((dyd * xhat) ** 2).sum(0), f"{what}: dweight")
    P.assert_colsum_close(got[2], db_ref, (dyd ** 2).sum(0), f"{what}: dbias")


def run_rmsb(inp, fused, cfg=None, alias=False):
    dy, x, w = dev(inp["dy"]), dev(inp["x"]), dev(inp["w"])
    if fused:
        dres = dev(inp["dres"]) if inp.get("dres") is not None else None
        out, dw = rn.fused_add_rmsnorm_bwd(dy, x, w, inp["eps"], dres=dres,
                                           ds=dy if alias else None, cfg=cfg)
    else:
        out, dw = rn.rmsnorm_bwd(dy, x, w, inp["eps"], dx=dy if alias else None, cfg=cfg)
    return host(out), dw.cpu().numpy()


def check_rmsb(inp, fused, got, what):
    dres = inp.get("dres") if fused else None
    dx_ref, dw_ref, rstd = oracle.rmsnorm_bwd(inp["dy"], inp["x"], inp["w"], inp["eps"],
                                              dres=dres, nthreads=NT)
    xd, dyd, wd = P.bits_to_f64(inp["x"]), P.bits_to_f64(inp["dy"]), P.bits_to_f64(inp["w"])
    scale = P.rmsnorm_dx_scale(xd, dyd, wd, rstd,
                               P.bits_to_f64(dres) if dres is not None else None)
    P.assert_bf16_close(got[0], dx_ref, f"{what}: dx", floor_scale=scale)
    xhat = xd * rstd[:, None]
    P.assert_colsum_close(got[1], dw_ref, ((dyd * xhat) ** 2).sum(0), f"{what}: dweight")


@pytest.mark.parametrize("h,rows", BWD_CASES)
def test_stream_layernorm_bwd(h, rows):
    d = rn.describe_config("layernorm_bwd", rows, h)
    assert "stream_bwd_tile_kernel" in d
    assert ("exchanging partial row sums" in d) == (h <= 262144), d
    inp = lnb_inputs(rows, h, seed=h + rows)
    check_lnb(inp, run_lnb(inp), f"layernorm_bwd {rows}x{h}")


@pytest.mark.parametrize("h,rows", BWD_CASES)
def test_stream_rmsnorm_and_fused_bwd(h, rows):
    inp = wl.rmsnorm_bwd_inputs(rows, h, seed=h + rows)
    check_rmsb(inp, False, run_rmsb(inp, False), f"rmsnorm_bwd {rows}x{h}")
    check_rmsb(inp, True, run_rmsb(inp, True), f"fused bwd {rows}x{h}")
    nodres = dict(inp, dres=None)
    check_rmsb(nodres, True, run_rmsb(nodres, True), f"fused bwd no dres {rows}x{h}")


def test_stream_bwd_walkers_aliasing_and_determinism():
    """Explicit row-walker counts (one slab each), dx == dy, and bitwise equal
    results from repeated calls."""
    h, rows = 65536 + 8, 75
    inp = lnb_inputs(rows, h, seed=9)
    for walkers in (1, 7, 75, 200):
        cfg = rn.Cfg(512, 1, walkers, 8)
        check_lnb(inp, run_lnb(inp, cfg=cfg), f"layernorm_bwd walkers {walkers}")
    check_lnb(inp, run_lnb(inp, alias=True), "layernorm_bwd dx == dy")
    first = run_lnb(inp)
    for _ in range(2):
        for a, b in zip(first, run_lnb(inp)):
            assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
    rinp = wl.rmsnorm_bwd_inputs(rows, h, seed=10)
    for walkers in (1, 13):
        cfg = rn.Cfg(512, 1, walkers, 8)
        check_rmsb(rinp, True, run_rmsb(rinp, True, cfg=cfg), f"fused bwd walkers {walkers}")
    check_rmsb(rinp, True, run_rmsb(rinp, True, alias=True), "fused bwd ds == dout")
    check_rmsb(rinp, False, run_rmsb(rinp, False, alias=True), "rmsnorm bwd dx == dy")


@pytest.mark.parametrize("h,rows", [(40000, 300), (65544, 75), (262144, 9)])
def test_stream_bwd_reread_path_is_bitwise_the_exchange(h, rows):
    """The column tiles of a row exchange their partial row sums (up to 32
    tiles: 262144 columns, the widest case here); a tile that stops waiting
    (spin limit 0: never wait) reads the other tiles of each row itself and
    forms their partials as their own workgroups do.  Both paths give the
    same bits, and agree with the oracle."""
    inp = lnb_inputs(rows, h, seed=h + 3)
    rinp = wl.rmsnorm_bwd_inputs(rows, h, seed=h + 4)
    fast = (run_lnb(inp), run_rmsb(rinp, False), run_rmsb(rinp, True))
    # 0: every tile re-reads; 1 and 4 polls: some tiles give up while others
    # still take their partners' partials (which ones varies run to run)
    for limit in (0, 1, 4):
        old = rn.set_bwd_spin_limit(limit)
        try:
            slow = (run_lnb(inp), run_rmsb(rinp, False), run_rmsb(rinp, True))
        finally:
            rn.set_bwd_spin_limit(old)
        for what, a, b in zip(("layernorm_bwd", "rmsnorm_bwd", "fused bwd"), fast, slow):
            for k, (u, v) in enumerate(zip(a, b)):
                assert np.array_equal(np.asarray(u).view(np.uint8),
                                      np.asarray(v).view(np.uint8)), \
                    f"{what} output {k}: spin limit {limit} differs from the exchange"
    check_lnb(inp, slow[0], f"layernorm_bwd re-read {rows}x{h}")
    check_rmsb(rinp, True, slow[2], f"fused bwd re-read {rows}x{h}")


def test_stream_bwd_zero_rows_and_noalloc():
    h = 65536
    dw = torch.full((h,), float("nan"), device=DEV)
    db = torch.full((h,), float("nan"), device=DEV)
    e = torch.empty(0, h, dtype=torch.bfloat16, device=DEV)
    s = torch.empty(0, device=DEV)
    rn.layernorm_bwd(e, e, s, s, torch.ones(h, dtype=torch.bfloat16, device=DEV), dweight=dw,
                     dbias=db)
    torch.cuda.synchronize()
    assert bool((dw == 0).all()) and bool((db == 0).all())
    # the allocation-free entry point runs the streamed kernels too, bitwise
    # as the workspace entry point
    inp = lnb_inputs(300, h, seed=12)
    assert rn.workspace_bytes(300, h) <= rn.NOALLOC_SCRATCH_BYTES
    a, b = run_lnb(inp, noalloc=True), run_lnb(inp)
    for x, y in zip(a, b):
        assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))
    check_lnb(inp, a, "layernorm_bwd_noalloc streamed")
