"""GPU parity of RMSNorm backward and the fused residual-add + RMSNorm
backward (through the C ABI) against the CPU oracle.  Rules in parity.py."""
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


def run(inp, fused, cfg=None, alias=None):
    dy, x, w = dev(inp["dy"]), dev(inp["x"]), dev(inp["w"])
    if fused:
        dres = dev(inp["dres"]) if inp.get("dres") is not None else None
        ds = {"dout": dy, "dres": dres}.get(alias)
        out, dw = rn.fused_add_rmsnorm_bwd(dy, x, w, inp["eps"], dres=dres, ds=ds, cfg=cfg)
    else:
        out, dw = rn.rmsnorm_bwd(dy, x, w, inp["eps"], dx=dy if alias == "dout" else None,
                                 cfg=cfg)
    torch.cuda.synchronize()
    return wl.from_device_bf16(out), dw.cpu().numpy()


def check(inp, fused, cfg=None, alias=None, what="rmsnorm_bwd"):
    dres = inp.get("dres") if fused else None
    dx_ref, dw_ref, rstd = oracle.rmsnorm_bwd(inp["dy"], inp["x"], inp["w"], inp["eps"],
                                              dres=dres, nthreads=NT)
    dx, dw = run(inp, fused, cfg, alias)
    xd, dyd, wd = P.bits_to_f64(inp["x"]), P.bits_to_f64(inp["dy"]), P.bits_to_f64(inp["w"])
    scale = P.rmsnorm_dx_scale(xd, dyd, wd, rstd,
                               P.bits_to_f64(dres) if dres is not None else None)
    stats = P.assert_bf16_close(dx, dx_ref, f"{what}: dx", floor_scale=scale)
    xhat = xd * rstd[:, None]
    P.assert_colsum_close(dw, dw_ref, ((dyd * xhat) ** 2).sum(0), f"{what}: dweight")
    return stats, (dx, dw)


@pytest.mark.parametrize("hidden", wl.RMSNORM_BWD_HIDDEN)
def test_rmsnorm_bwd_config(hidden):
    """rows=8192, x, dy ~ N(0,1), w ~ N(1,0.1), eps 1e-6."""
    inp = wl.rmsnorm_bwd_inputs(wl.RMSNORM_BWD_ROWS, hidden, seed=0)
    stats, _ = check(inp, fused=False, what=f"rmsnorm_bwd h={hidden}")
    P.report_floor(f"rmsnorm_bwd {wl.RMSNORM_BWD_ROWS}x{hidden} dx", stats)


@pytest.mark.parametrize("hidden", wl.RMSNORM_BWD_HIDDEN)
def test_fused_add_rmsnorm_bwd_config(hidden):
    """The fused op's backward at its residual output, with the residual gradient."""
    inp = wl.rmsnorm_bwd_inputs(wl.RMSNORM_BWD_ROWS, hidden, seed=1)
    stats, _ = check(inp, fused=True, what=f"fused_add_rmsnorm_bwd h={hidden}")
    P.report_floor(f"fused_add_rmsnorm_bwd {wl.RMSNORM_BWD_ROWS}x{hidden} ds", stats)


@pytest.mark.parametrize("hidden", rn.HIDDEN_SIZES)
def test_every_compiled_shape_and_grid(hidden):
    inp = wl.rmsnorm_bwd_inputs(75, hidden, seed=2)
    nodres = dict(inp, dres=None)
    for c in rn.list_configs("rmsnorm_bwd", hidden):
        for grid in (1, 7, 75, 200):
            cfg = rn.Cfg(c.threads_per_row, c.rows_per_block, grid, c.vector_elems)
            check(inp, fused=False, cfg=cfg, what=f"rmsnorm_bwd h={hidden} {cfg}")
            check(inp, fused=True, cfg=cfg, what=f"fused bwd h={hidden} {cfg}")
            check(nodres, fused=True, cfg=cfg, what=f"fused bwd no dres h={hidden} {cfg}")


def test_in_place_outputs():
    inp = wl.rmsnorm_bwd_inputs(300, 4096, seed=3)
    check(inp, fused=False, alias="dout", what="rmsnorm_bwd dx==dy")
    check(inp, fused=True, alias="dout", what="fused bwd ds==dout")
    check(inp, fused=True, alias="dres", what="fused bwd ds==dres")


def test_deterministic_and_fused_without_dres_equals_plain():
    inp = wl.rmsnorm_bwd_inputs(1024, 8192, seed=4)
    _, first = check(inp, fused=True)
    for _ in range(2):
        again = run(inp, fused=True)
        for a, b in zip(first, again):
            assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
    plain = run(inp, fused=False)
    nodres = run(dict(inp, dres=None), fused=True)
    for a, b in zip(plain, nodres):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


def test_zero_rows_zero_fills_dweight():
    h = 2048
    dw = torch.full((h,), float("nan"), device=DEV)
    e = torch.empty(0, h, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(h, dtype=torch.bfloat16, device=DEV)
    rn.rmsnorm_bwd(e, e, w, 1e-6, dweight=dw)
    torch.cuda.synchronize()
    assert (dw.cpu() == 0).all()
