"""GPU parity of the run-time-hidden kernels against the CPU oracle: hidden
sizes outside the compiled set (tiny, odd, not a multiple of 8, up to each
family's widest row), rows given with a row stride (column slices of wider
matrices), pointers aligned to fewer than 16 bytes, and every run-time launch
shape.  Outputs written through a stride must leave the elements between the
rows untouched.  Rules in parity.py."""
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
FILL = 0x7FC1  # a NaN pattern: any stray read would poison a result, any stray write shows

# hidden sizes and the access width each implies for contiguous rows
FWD_HIDDEN = [1, 7, 64, 100, 127, 128, 130, 256, 320, 1000, 1536, 3000, 4100, 5120, 7168]
BWD_HIDDEN = [1, 7, 64, 100, 127, 130, 320, 1000, 3000, 4100, 5120]


def dev(bits):
    return wl.to_device_bf16(bits, DEV)


def host(t):
    torch.cuda.synchronize()
    return wl.from_device_bf16(t)


class Strided:
    """A [rows, h] bf16 view with row stride `ld` that starts `off` elements
    into a buffer filled with FILL; knows which buffer elements are its own."""

    def __init__(self, rows, h, ld=None, off=0, bits=None):
        self.rows, self.h, self.ld, self.off = rows, h, ld or h, off
        n = off + (rows - 1) * self.ld + h if rows else off
        self.big = torch.full((n + 64,), FILL, dtype=torch.int16, device=DEV)
        flat = self.big.view(torch.bfloat16)[off:off + rows * self.ld]
        if rows * self.ld > flat.numel():  # the last row's tail past the buffer is not needed
            flat = self.big.view(torch.bfloat16)[off:]
        self.t = torch.as_strided(flat, (rows, h), (self.ld, 1))
        if bits is not None:
            self.t.copy_(dev(bits))

    def guards_intact(self):
        b = self.big.cpu().numpy()
        mask = np.ones(b.size, bool)
        for i in range(self.rows):
            s = self.off + i * self.ld
            mask[s:s + self.h] = False
        return bool((b[mask] == np.int16(FILL)).all())

    def bits(self):
        return host(self.t)


def runtime_cfgs(op, h):
    return [c for c in rn.list_configs(op, h) if c.runtime_hidden]


# ------------------------------------------------------------------ forward
def check_fwd(op, inp, cfg=None, layout=None, what=""):
    """One forward op on `inp`; layout = (ld multiple, element offset) for
    every matrix argument (None: contiguous tensors)."""
    rows, h = inp["x"].shape
    what = f"{op} {rows}x{h} {what}"
    mk = (lambda bits=None: Strided(rows, h, h * layout[0] + layout[1], layout[1], bits)) \
        if layout else None
    if op == "fused_add_rmsnorm":
        ref, res_ref, _ = oracle.fused_add_rmsnorm(inp["x"], inp["r"], inp["w"], inp["eps"], NT)
        if mk:
            x, r, o = mk(inp["x"]), mk(inp["r"]), mk()
            rn.fused_add_rmsnorm(x.t, r.t, dev(inp["w"]), inp["eps"], out=o.t, cfg=cfg)
            out, res = o.bits(), r.bits()
            assert o.guards_intact() and r.guards_intact() and x.guards_intact(), what
        else:
            out, res = rn.fused_add_rmsnorm(dev(inp["x"]), dev(inp["r"]), dev(inp["w"]),
                                            inp["eps"], cfg=cfg)
            out, res = host(out), host(res)
        P.assert_bits_equal(res, res_ref, f"{what}: residual")
        P.assert_bf16_close(out, ref, f"{what}: out")
    elif op == "rmsnorm_fwd":
        ref, _ = oracle.rmsnorm_fwd(inp["x"], inp["w"], inp["eps"], NT)
        if mk:
            x, o = mk(inp["x"]), mk()
            rn.rmsnorm_fwd(x.t, dev(inp["w"]), inp["eps"], out=o.t, cfg=cfg)
            out = o.bits()
            assert o.guards_intact(), what
        else:
            out = host(rn.rmsnorm_fwd(dev(inp["x"]), dev(inp["w"]), inp["eps"], cfg=cfg))
        P.assert_bf16_close(out, ref, what)
    else:
        ref, mean_ref, rstd_ref = oracle.layernorm_fwd(inp["x"], inp["w"], inp["b"], inp["eps"],
                                                       NT)
        if mk:
            x, o = mk(inp["x"]), mk()
            _, mean, rstd = rn.layernorm_fwd(x.t, dev(inp["w"]), dev(inp["b"]), inp["eps"],
                                             y=o.t, cfg=cfg)
            y = o.bits()
            assert o.guards_intact(), what
        else:
            y, mean, rstd = rn.layernorm_fwd(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]),
                                             inp["eps"], cfg=cfg)
            y = host(y)
        xd, wd, bd = P.bits_to_f64(inp["x"]), P.bits_to_f64(inp["w"]), P.bits_to_f64(inp["b"])
        scale = P.layernorm_y_scale(xd, mean_ref, rstd_ref, wd, bd)
        P.assert_bf16_close(y, ref, f"{what}: y", floor_scale=scale)
        P.assert_f32_close(mean.cpu().numpy(), mean_ref, f"{what}: mean")
        P.assert_f32_close(rstd.cpu().numpy(), rstd_ref, f"{what}: rstd")


def fwd_inputs(op, rows, h, seed):
    if op == "fused_add_rmsnorm":
        return wl.fused_inputs(rows, h, seed)
    if op == "rmsnorm_fwd":
        return wl.rmsnorm_inputs(rows, h, seed)
    return wl.layernorm_fwd_inputs(rows, h, seed)


FWD_OPS = ["fused_add_rmsnorm", "rmsnorm_fwd", "layernorm_fwd"]


@pytest.mark.parametrize("h", FWD_HIDDEN)
def test_fwd_runtime_hidden(h):
    """Ragged row counts in the library's own launch choice."""
    for op in FWD_OPS:
        assert rn.select_config(op, 37, h).runtime_hidden
        for rows in (1, 37, 300):
            check_fwd(op, fwd_inputs(op, rows, h, seed=h + rows))


@pytest.mark.parametrize("h", [64, 256, 1000, 4096, 5120])
def test_fwd_every_runtime_shape(h):
    """Every run-time shape, from 8-lane rows (32 to a workgroup) to 1024 lanes,
    on 37 rows (a partial last workgroup for every rows-per-workgroup)."""
    for op in FWD_OPS:
        cfgs = runtime_cfgs(op, h)
        assert cfgs
        inp = fwd_inputs(op, 37, h, seed=7)
        for c in cfgs:
            check_fwd(op, inp, cfg=c, what=str(c))


# (hidden, ld multiple, offset): ld = hidden * multiple + offset elements and the
# first row starts `offset` elements into a 256-byte-aligned buffer
@pytest.mark.parametrize("h,ld_mult,off", [
    (4096, 3, 4096),   # a column slice of a [rows, 3h + h] matrix: 16-byte accesses
    (4096, 1, 1),      # odd stride, 2-byte offset: 2-byte accesses
    (4096, 2, 2),      # 4-byte accesses
    (4096, 2, 4),      # 8-byte accesses
    (1000, 2, 1000),   # a slice at a hidden size outside the compiled set
    (127, 3, 5),       # odd width, odd stride
])
def test_fwd_strided_and_misaligned(h, ld_mult, off):
    for op in FWD_OPS:
        check_fwd(op, fwd_inputs(op, 45, h, seed=3), layout=(ld_mult, off),
                  what=f"ld={ld_mult}h off={off}")


def test_fwd_widest_rows():
    """The widest row each forward family holds: 65536 (fused, RMSNorm) and
    49152 (LayerNorm), at 1024 lanes."""
    for op, h in (("fused_add_rmsnorm", 65536), ("rmsnorm_fwd", 65536 - 8),
                  ("layernorm_fwd", 49152)):
        c = rn.select_config(op, 3, h)
        assert c.runtime_hidden and c.threads_per_row == 1024, (op, c)
        check_fwd(op, fwd_inputs(op, 3, h, seed=5))


def test_fwd_in_place_runtime():
    """out == x (same pointer and stride) on the run-time path."""
    h = 5120
    inp = wl.rmsnorm_inputs(33, h, seed=8)
    ref, _ = oracle.rmsnorm_fwd(inp["x"], inp["w"], inp["eps"], NT)
    x = Strided(33, h, 2 * h, h, inp["x"])
    rn.rmsnorm_fwd(x.t, dev(inp["w"]), inp["eps"], out=x.t)
    P.assert_bf16_close(x.bits(), ref, "rmsnorm in place, strided")
    assert x.guards_intact()


def test_qk_norm_slices_of_one_projection():
    """RMSNorm over head-sized rows normalized in place inside a fused
    [tokens, q | k | v] projection: each head's column slice is a [tokens, 128]
    matrix with row stride 3 * heads * 128.  q and k change, v is untouched."""
    tokens, heads, hd = 40, 4, 128
    rng = np.random.default_rng(21)
    qkv_f = rng.standard_normal((tokens, 3 * heads * hd)).astype(np.float32)
    qkv = dev(wl.bf16_bits(qkv_f))
    before = host(qkv)
    w = wl.bf16_bits((1.0 + 0.1 * rng.standard_normal(hd)).astype(np.float32))
    for head in range(2 * heads):  # the q heads, then the k heads
        view = qkv[:, head * hd:(head + 1) * hd]
        rn.rmsnorm_fwd(view, dev(w), wl.EPS_RMS, out=view)
    after = host(qkv)
    for part in (0, 1):
        sl = slice(part * heads * hd, (part + 1) * heads * hd)
        x_bits = np.ascontiguousarray(before[:, sl]).reshape(tokens * heads, hd)
        ref, _ = oracle.rmsnorm_fwd(x_bits, w, wl.EPS_RMS, NT)
        got = np.ascontiguousarray(after[:, sl]).reshape(tokens * heads, hd)
        P.assert_bf16_close(got, ref, f"qk-norm part {part}")
    assert np.array_equal(after[:, 2 * heads * hd:], before[:, 2 * heads * hd:])


# ------------------------------------------------------------------ backward
def lnb_inputs(rows, h, seed):
    inp = wl.layernorm_bwd_inputs(rows, h, seed)
    _, mean, rstd = oracle.layernorm_fwd(inp["x"], inp["w"], np.zeros(h, np.uint16), inp["eps"],
                                         NT)
    inp["mean"], inp["rstd"] = mean.astype(np.float32), rstd.astype(np.float32)
    return inp


def check_bwd(op, inp, cfg=None, layout=None, alias=False, what=""):
    """op in layernorm_bwd, rmsnorm_bwd, fused_add_rmsnorm_bwd (with inp's dres,
    or without when it is None).  alias: dx written over dy."""
    rows, h = inp["x"].shape
    what = f"{op} {rows}x{h} {what}"
    mk = (lambda bits=None: Strided(rows, h, h * layout[0] + layout[1], layout[1], bits)) \
        if layout else (lambda bits=None: Strided(rows, h, h, 0, bits))
    dy, x = mk(inp["dy"]), mk(inp["x"])
    dx = dy if alias else mk()
    w = dev(inp["w"])
    xd, dyd, wd = P.bits_to_f64(inp["x"]), P.bits_to_f64(inp["dy"]), P.bits_to_f64(inp["w"])
    if op == "layernorm_bwd":
        dx_ref, dw_ref, db_ref = oracle.layernorm_bwd(inp["dy"], inp["x"], inp["mean"],
                                                      inp["rstd"], inp["w"], NT)
        _, dw, db = rn.layernorm_bwd(dy.t, x.t, torch.from_numpy(inp["mean"]).to(DEV),
                                     torch.from_numpy(inp["rstd"]).to(DEV), w, dx=dx.t, cfg=cfg)
        mean, rstd = inp["mean"].astype(np.float64), inp["rstd"].astype(np.float64)
        scale = P.layernorm_dx_scale(xd, dyd, wd, mean, rstd)
        xhat = (xd - mean[:, None]) * rstd[:, None]
        P.assert_colsum_close(db.cpu().numpy(), db_ref, (dyd ** 2).sum(0), f"{what}: dbias")
    else:
        dres = inp.get("dres") if op == "fused_add_rmsnorm_bwd" else None
        dx_ref, dw_ref, rstd = oracle.rmsnorm_bwd(inp["dy"], inp["x"], inp["w"], inp["eps"],
                                                  dres=dres, nthreads=NT)
        if op == "rmsnorm_bwd":
            _, dw = rn.rmsnorm_bwd(dy.t, x.t, w, inp["eps"], dx=dx.t, cfg=cfg)
        else:
            dr = mk(dres) if dres is not None else None
            _, dw = rn.fused_add_rmsnorm_bwd(dy.t, x.t, w, inp["eps"],
                                             dres=dr.t if dr is not None else None, ds=dx.t,
                                             cfg=cfg)
        scale = P.rmsnorm_dx_scale(xd, dyd, wd, rstd,
                                   P.bits_to_f64(dres) if dres is not None else None)
        xhat = xd * rstd[:, None]
    P.assert_bf16_close(dx.bits(), dx_ref, f"{what}: dx", floor_scale=scale)
    P.assert_colsum_close(dw.cpu().numpy(), dw_ref, ((dyd * xhat) ** 2).sum(0),
                          f"{what}: dweight")
    assert dx.guards_intact() and dy.guards_intact() and x.guards_intact(), what
    return dx.bits(), dw.cpu().numpy()


def bwd_inputs(op, rows, h, seed):
    if op == "layernorm_bwd":
        return lnb_inputs(rows, h, seed)
    inp = wl.rmsnorm_bwd_inputs(rows, h, seed)
    if op == "rmsnorm_bwd":
        inp["dres"] = None
    return inp


BWD_OPS = ["layernorm_bwd", "rmsnorm_bwd", "fused_add_rmsnorm_bwd"]


@pytest.mark.parametrize("h", BWD_HIDDEN)
def test_bwd_runtime_hidden(h):
    for op in BWD_OPS:
        assert rn.select_config(op, 300, h).runtime_hidden
        for rows in (1, 300):
            check_bwd(op, bwd_inputs(op, rows, h, seed=h + rows))


@pytest.mark.parametrize("h", [128, 1000, 4096])
def test_bwd_every_runtime_shape_and_grid(h):
    """Every run-time backward shape with one walker slab, ragged walks and
    idle walkers; the fused op also without its residual gradient."""
    for op in BWD_OPS:
        inp = bwd_inputs(op, 75, h, seed=9)
        for c in runtime_cfgs(op, h):
            for grid in (1, 7, 0):
                cfg = rn.Cfg(c.threads_per_row, c.rows_per_block, grid, c.vector_elems)
                check_bwd(op, inp, cfg=cfg, what=str(cfg))
        if op == "fused_add_rmsnorm_bwd":
            check_bwd(op, dict(inp, dres=None), what="no dres")


@pytest.mark.parametrize("h,ld_mult,off", [(4096, 3, 4096), (4096, 2, 2), (1000, 2, 1000),
                                           (127, 3, 5)])
def test_bwd_strided_and_misaligned(h, ld_mult, off):
    for op in BWD_OPS:
        check_bwd(op, bwd_inputs(op, 90, h, seed=4), layout=(ld_mult, off),
                  what=f"ld={ld_mult}h off={off}")
        check_bwd(op, bwd_inputs(op, 90, h, seed=5), layout=(ld_mult, off), alias=True,
                  what=f"dx==dy ld={ld_mult}h off={off}")


def test_bwd_widest_rows():
    """Widest backward rows: 16384 - 8 (16-byte accesses, not the compiled
    16384) and 8191 (odd: 2-byte accesses)."""
    for op in BWD_OPS:
        for h in (16384 - 8, 8191):
            c = rn.select_config(op, 40, h)
            assert c.runtime_hidden, (op, h, c)
            check_bwd(op, bwd_inputs(op, 40, h, seed=6))


@pytest.mark.parametrize("h", [16392, 20000, 24576, 28672, 28680, 32768])
def test_bwd_wide_rows_staged_in_lds(h):
    """Rows wider than the register-resident backward holds (16392 ... 32768):
    512-lane workgroups with x and dy staged in LDS, 5 to 8 accesses a lane
    (the fused op up to 7, 28672: its wider rows take the streamed tiles);
    one row, a ragged 37 and 300 rows over the 256-workgroup grid."""
    for op in BWD_OPS:
        c = rn.select_config(op, 300, h)
        assert (c.threads_per_row, c.rows_per_block, c.vector_elems) == (512, 1, 8), (op, c)
        streamed = op == "fused_add_rmsnorm_bwd" and h > 28672
        assert ("stream_bwd_tile_kernel" if streamed else "norm_bwd_wide_kernel") in \
            rn.describe_config(op, 300, h)
        for rows in (1, 37, 300):
            check_bwd(op, bwd_inputs(op, rows, h, seed=h + rows))
        if op == "fused_add_rmsnorm_bwd":
            check_bwd(op, dict(bwd_inputs(op, 37, h, seed=3), dres=None), what="no dres")


def test_bwd_wide_grids_strides_alias_and_determinism():
    h = 20000
    for op in BWD_OPS:
        inp = bwd_inputs(op, 75, h, seed=12)
        for grid in (1, 7, 0):
            check_bwd(op, inp, cfg=rn.Cfg(512, 1, grid, 8), what=f"grid {grid}")
        first = check_bwd(op, inp)
        again = check_bwd(op, inp)
        for x, y in zip(first, again):
            assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))
        # rows of a wider matrix (ld = 2h + 8), and dx written over dy
        check_bwd(op, bwd_inputs(op, 40, h, seed=13), layout=(2, 8), what="strided")
        check_bwd(op, bwd_inputs(op, 40, h, seed=14), layout=(2, 8), alias=True,
                  what="dx==dy strided")


def test_bwd_runtime_deterministic():
    for op in BWD_OPS:
        inp = bwd_inputs(op, 2000, 5120, seed=10)
        first = check_bwd(op, inp)
        again = check_bwd(op, inp)
        for a, b in zip(first, again):
            assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8)), op


@pytest.mark.parametrize("h", [4096, 5120])
def test_rmsnorm_bwd_eps_zero_with_partial_ring(h):
    """eps = 0 with a row count that leaves the last ring step of most
    workgroups partial: the rows past the end must add nothing (no NaN from
    0 * inf) to dweight, on the compiled (4096) and run-time (5120) kernels."""
    for op in ("rmsnorm_bwd", "fused_add_rmsnorm_bwd"):
        inp = bwd_inputs(op, 1001, h, seed=11)
        inp["eps"] = 0.0
        check_bwd(op, inp, what="eps=0")


def test_bwd_runtime_zero_rows_zero_fills():
    h = 1000
    e = torch.empty(0, h, dtype=torch.bfloat16, device=DEV)
    s = torch.empty(0, dtype=torch.float32, device=DEV)
    w = torch.ones(h, dtype=torch.bfloat16, device=DEV)
    dw = torch.full((h,), float("nan"), device=DEV)
    db = torch.full((h,), float("nan"), device=DEV)
    rn.layernorm_bwd(e, e, s, s, w, dweight=dw, dbias=db)
    torch.cuda.synchronize()
    assert (dw.cpu() == 0).all() and (db.cpu() == 0).all()
    dw.fill_(float("nan"))
    rn.rmsnorm_bwd(e, e, w, 1e-6, dweight=dw)
    torch.cuda.synchronize()
    assert (dw.cpu() == 0).all()
