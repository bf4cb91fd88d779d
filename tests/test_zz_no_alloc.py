"""The allocation-free LayerNorm backward entry point (partial sums in the
library's per-device scratch array) through the C ABI: two calls in a row,
the second smaller, each bitwise equal to norm_layernorm_bwd with a caller
workspace on the same inputs and within the oracle's tolerances; the largest
partial-sum size that fits, the first that does not, and zero rows."""
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


def case(rows, hidden, seed):
    b = wl.layernorm_bwd_inputs(rows, hidden, seed=seed)
    _, mean, rstd = oracle.layernorm_fwd(b["x"], b["w"], np.zeros(hidden, np.uint16), b["eps"],
                                         NT)
    b["mean"], b["rstd"] = mean.astype(np.float32), rstd.astype(np.float32)
    d = {k: wl.to_device_bf16(b[k], DEV) for k in ("dy", "x", "w")}
    d["mean"] = torch.from_numpy(b["mean"]).to(DEV)
    d["rstd"] = torch.from_numpy(b["rstd"]).to(DEV)
    return b, d


def both(d):
    """(no-alloc outputs, workspace-entry outputs), as host arrays."""
    dx0, dw0, db0 = rn.layernorm_bwd_noalloc(d["dy"], d["x"], d["mean"], d["rstd"], d["w"])
    dx1, dw1, db1 = rn.layernorm_bwd(d["dy"], d["x"], d["mean"], d["rstd"], d["w"])
    torch.cuda.synchronize()
    return ((wl.from_device_bf16(dx0), dw0.cpu().numpy(), db0.cpu().numpy()),
            (wl.from_device_bf16(dx1), dw1.cpu().numpy(), db1.cpu().numpy()))


def check_oracle(b, got, what):
    dx_ref, dw_ref, db_ref = oracle.layernorm_bwd(b["dy"], b["x"], b["mean"], b["rstd"], b["w"],
                                                  NT)
    xd, dyd, wd = P.bits_to_f64(b["x"]), P.bits_to_f64(b["dy"]), P.bits_to_f64(b["w"])
    scale = P.layernorm_dx_scale(xd, dyd, wd, b["mean"].astype(np.float64),
                                 b["rstd"].astype(np.float64))
    P.assert_bf16_close(got[0], dx_ref, f"{what}: dx", floor_scale=scale)
    xhat = (xd - b["mean"].astype(np.float64)[:, None]) * b["rstd"].astype(np.float64)[:, None]
    P.assert_colsum_close(got[1], dw_ref, ((dyd * xhat) ** 2).sum(0), f"{what}: dweight")
    P.assert_colsum_close(got[2], db_ref, (dyd ** 2).sum(0), f"{what}: dbias")


@pytest.mark.parametrize("first,second", [((512, 16384), (300, 1024)),
                                          ((8192, 4096), (37, 4096)),
                                          ((1000, 5120), (45, 100))])
def test_noalloc_matches_workspace_entry_twice(first, second):
    print(f"noalloc pair {first} then {second}", flush=True)
    for k, (rows, hidden) in enumerate((first, second)):
        b, d = case(rows, hidden, seed=rows + hidden)
        noalloc, ws = both(d)
        for a, c, name in zip(noalloc, ws, ("dx", "dweight", "dbias")):
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  c.view(np.uint32) if c.dtype == np.float32 else c), \
                f"call {k} {rows}x{hidden}: {name} differs from norm_layernorm_bwd"
        if rows * hidden <= 8 << 20:
            check_oracle(b, noalloc, f"noalloc call {k} {rows}x{hidden}")


def test_noalloc_scratch_limit_and_zero_rows():
    # 256 workgroups x 2 x 16384 fp32 is exactly the scratch size: accepted (above);
    # 32768-wide rows need 256 x 2 x 32768 x 4 = 64 MiB from 256 rows: refused
    assert rn.NOALLOC_SCRATCH_BYTES == 32 << 20
    rows, hidden = 256, 32768
    assert rn.workspace_bytes(rows, hidden) > rn.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(rows, hidden, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(hidden, dtype=torch.bfloat16, device=DEV)
    m = torch.zeros(rows, device=DEV)
    r = torch.ones(rows, device=DEV)
    dx = torch.full_like(x, 7.0)
    with pytest.raises(rn.NormError) as e:
        rn.layernorm_bwd_noalloc(x, x, m, r, w, dx=dx)
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert bool((dx == 7.0).all()), "a refused call wrote its output"
    # 128 such rows fit (128 x 2 x 32768 x 4 bytes = 32 MiB)
    b, d = case(128, 32768, seed=11)
    noalloc, ws = both(d)
    for a, c in zip(noalloc, ws):
        assert np.array_equal(a, c)
    # zero rows: column sums of nothing are zero
    dw = torch.full((1024,), 5.0, device=DEV)
    db = torch.full((1024,), 5.0, device=DEV)
    e0 = torch.empty(0, 1024, dtype=torch.bfloat16, device=DEV)
    rn.layernorm_bwd_noalloc(e0, e0, torch.empty(0, device=DEV), torch.empty(0, device=DEV),
                             torch.ones(1024, dtype=torch.bfloat16, device=DEV), dweight=dw,
                             dbias=db)
    torch.cuda.synchronize()
    assert bool((dw == 0).all()) and bool((db == 0).all())
