"""GPU parity of the fp32-activation entry points (`norm_*_f32`) against the
CPU oracle's fp32 functions, through the C ABI: the six operations over
widths from 4 to 2^20 columns (ragged tails of the 16-byte accesses, the
4096- and 8192-column tiles of the backward and the 1024-lane passes of the
forward), row counts from 1 to the thousands, in-place calls, LayerNorm without
statistics, zero rows, memory past the outputs left untouched, bitwise
run-to-run determinism, and graph replays.  Rules (the fp32 bound derived
from the kernels' summation order) in parity.py."""
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


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy().astype(np.float64)


def f64(a):
    return np.asarray(a, np.float64)


def walkers(rows, h):
    if 8196 <= h <= 16384:  # the LDS-staged kernel: one slab per workgroup
        return max(1, min(rows, 256))
    if 16388 <= h <= 262144:  # exchange tiles of 4096 columns, two workgroups a CU
        return max(1, min(rows, 511 // -(-h // 4096)))
    return max(1, min(rows, 255 // -(-h // 8192)))


# ------------------------------------------------------------------ forward
# one shape per launch-shape bucket of the fp32 forward (rows of up to 1024
# columns several to a wave; then lanes x accesses held: up to 2048, 4096,
# 8192, 16384 columns, then 1024 lanes x 8 / x 4; the LDS-staged rows past
# those: fused 34956-40960, RMSNorm 34956-69632, with walks of two rows a
# workgroup)
FWD_SHAPES = [(4, 1), (12, 37), (32, 1000), (64, 517), (100, 33), (128, 300), (200, 77),
              (256, 64), (500, 33), (512, 19), (516, 7), (1024, 300), (2048, 45), (4096, 64),
              (4100, 37), (8192, 11), (16384, 9), (16388, 5), (32768, 7), (32772, 5),
              (34956, 4), (40960, 300), (45056, 257), (65536, 17), (69632, 3), (100004, 3),
              (1 << 20, 2)]


def check_fused(inp, out, res, h, what):
    ref, res_ref, _ = oracle.fused_add_rmsnorm_f32(inp["x"], inp["r"], inp["w"], inp["eps"], NT)
    assert np.array_equal(np.asarray(res, np.float32).view(np.uint32),
                          res_ref.view(np.uint32)), f"{what}: residual differs from fp32(x + r)"
    P.assert_f32_scaled(out, ref, np.abs(ref), h, f"{what}: out")


@pytest.mark.parametrize("h,rows", FWD_SHAPES)
def test_fused_add_rmsnorm_f32(h, rows):
    inp = wl.fused_inputs(rows, h, seed=h + rows, f32=True)
    x, r, w = dev(inp["x"]), dev(inp["r"]), dev(inp["w"])
    out, r = rn.fused_add_rmsnorm_f32(x, r, w, inp["eps"])
    torch.cuda.synchronize()
    check_fused(inp, host(out), r.cpu().numpy(), h, f"fused f32 {rows}x{h}")


@pytest.mark.parametrize("h,rows", FWD_SHAPES)
def test_rmsnorm_fwd_f32(h, rows):
    inp = wl.rmsnorm_inputs(rows, h, seed=h + rows + 1, f32=True)
    out = rn.rmsnorm_fwd_f32(dev(inp["x"]), dev(inp["w"]), inp["eps"])
    ref, _ = oracle.rmsnorm_fwd_f32(inp["x"], inp["w"], inp["eps"], NT)
    P.assert_f32_scaled(host(out), ref, np.abs(ref), h, f"rmsnorm f32 {rows}x{h}")


def check_ln_fwd(inp, y, mean, rstd, h, what):
    ref, mean_ref, rstd_ref = oracle.layernorm_fwd_f32(inp["x"], inp["w"], inp["b"], inp["eps"],
                                                       NT)
    xd, wd, bd = f64(inp["x"]), f64(inp["w"]), f64(inp["b"])
    scale = P.layernorm_y_scale(xd, mean_ref, rstd_ref, wd, bd)
    P.assert_f32_scaled(y, ref, scale, h, f"{what}: y")
    if mean is not None:
        P.assert_f32_scaled(mean, mean_ref, np.abs(xd).mean(axis=1), h, f"{what}: mean")
        P.assert_f32_scaled(rstd, rstd_ref, rstd_ref, h, f"{what}: rstd")


@pytest.mark.parametrize("h,rows", FWD_SHAPES)
def test_layernorm_fwd_f32(h, rows):
    inp = wl.layernorm_fwd_inputs(rows, h, seed=h + rows + 2, f32=True)
    y, mean, rstd = rn.layernorm_fwd_f32(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]), inp["eps"])
    check_ln_fwd(inp, host(y), host(mean), host(rstd), h, f"layernorm f32 {rows}x{h}")


@pytest.mark.parametrize("h", [512, 4096, 20000, 40960])  # group, streamed, streamed, LDS-staged
def test_forward_f32_in_place_and_without_stats(h):
    rows = 19
    inp = wl.fused_inputs(rows, h, seed=5, f32=True)
    x, r, w = dev(inp["x"]), dev(inp["r"]), dev(inp["w"])
    out, r = rn.fused_add_rmsnorm_f32(x, r, w, inp["eps"], out=x)
    assert out.data_ptr() == x.data_ptr()
    check_fused(inp, host(out), r.cpu().numpy(), h, "fused f32 in place")

    inp = wl.rmsnorm_inputs(rows, h, seed=6, f32=True)
    x = dev(inp["x"])
    rn.rmsnorm_fwd_f32(x, dev(inp["w"]), inp["eps"], out=x)
    ref, _ = oracle.rmsnorm_fwd_f32(inp["x"], inp["w"], inp["eps"], NT)
    P.assert_f32_scaled(host(x), ref, np.abs(ref), h, "rmsnorm f32 in place")

    inp = wl.layernorm_fwd_inputs(rows, h, seed=7, f32=True)
    x = dev(inp["x"])
    y, mean, rstd = rn.layernorm_fwd_f32(x, dev(inp["w"]), dev(inp["b"]), inp["eps"], y=x,
                                         with_stats=False)
    assert mean is None and rstd is None
    check_ln_fwd(inp, host(y), None, None, h, "layernorm f32 in place, no stats")


def test_forward_f32_leaves_memory_past_the_outputs_alone():
    rows, h = 7, 8196
    inp = wl.layernorm_fwd_inputs(rows, h, seed=8, f32=True)
    canary = np.float32(-12345.5)
    ybuf = torch.full((rows * h + 4096,), float(canary), device=DEV)
    sbuf = torch.full((2 * rows + 64,), float(canary), device=DEV)
    y = ybuf[:rows * h].view(rows, h)
    mean, rstd = sbuf[:rows], sbuf[rows:2 * rows]
    rn.layernorm_fwd_f32(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]), inp["eps"], y=y,
                         mean=mean, rstd=rstd)
    torch.cuda.synchronize()
    assert torch.all(ybuf[rows * h:] == float(canary))
    assert torch.all(sbuf[2 * rows:] == float(canary))
    check_ln_fwd(inp, host(y), host(mean), host(rstd), h, "layernorm f32 canary")


def test_forward_f32_zero_rows():
    w = torch.ones(4096, device=DEV)
    x = torch.empty((0, 4096), device=DEV)
    assert rn.rmsnorm_fwd_f32(x, w, 1e-6).shape == (0, 4096)
    y, mean, rstd = rn.layernorm_fwd_f32(x, w, torch.zeros_like(w), 1e-5)
    assert y.shape == (0, 4096) and mean.numel() == 0


def test_forward_f32_deterministic():
    rows, h = 64, 65540
    inp = wl.layernorm_fwd_inputs(rows, h, seed=9, f32=True)
    x, w, b = dev(inp["x"]), dev(inp["w"]), dev(inp["b"])
    first = rn.layernorm_fwd_f32(x, w, b, inp["eps"])
    for _ in range(3):
        again = rn.layernorm_fwd_f32(x, w, b, inp["eps"])
        for a, c in zip(first, again):
            assert torch.equal(a.view(torch.int32), c.view(torch.int32))


# ------------------------------------------------------------------ backward
# one-tile rows (up to 8192), LDS-staged rows (8196 ... 16384: 5 ... 8 accesses
# a lane), tiled rows beyond
BWD_SHAPES = [(4, 1), (12, 7), (1024, 300), (4096, 1000), (4100, 37), (8192, 45), (8196, 65),
              (10244, 33), (12288, 300), (16384, 300), (16388, 40), (65536, 17), (262144, 5),
              (262148, 3), (1 << 20, 2)]


def ln_stats_f32(x, eps):
    """The given statistics of the backward: the oracle's forward rounded to fp32."""
    _, mean, rstd = oracle.layernorm_fwd_f32(x, np.ones(x.shape[1], np.float32),
                                             np.zeros(x.shape[1], np.float32), eps, NT)
    return mean.astype(np.float32), rstd.astype(np.float32)


def check_ln_bwd(inp, mean32, rstd32, dx, dw, db, what):
    rows, h = inp["x"].shape
    dx_ref, dw_ref, db_ref = oracle.layernorm_bwd_f32(inp["dy"], inp["x"], mean32, rstd32,
                                                      inp["w"], NT)
    xd, dyd, wd = f64(inp["x"]), f64(inp["dy"]), f64(inp["w"])
    m, q = f64(mean32), f64(rstd32)
    P.assert_f32_scaled(dx, dx_ref, P.layernorm_dx_scale(xd, dyd, wd, m, q), h, f"{what}: dx")
    xhat = (xd - m[:, None]) * q[:, None]
    p = walkers(rows, h)
    P.assert_colsum_f32(dw, dw_ref, np.abs(dyd * xhat).sum(axis=0), rows, p, h,
                        f"{what}: dweight")
    P.assert_colsum_f32(db, db_ref, np.abs(dyd).sum(axis=0), rows, p, h, f"{what}: dbias")


@pytest.mark.parametrize("h,rows", BWD_SHAPES)
def test_layernorm_bwd_f32(h, rows):
    inp = wl.layernorm_bwd_inputs(rows, h, seed=h + rows + 3, f32=True)
    mean32, rstd32 = ln_stats_f32(inp["x"], inp["eps"])
    dx, dw, db = rn.layernorm_bwd_f32(dev(inp["dy"]), dev(inp["x"]), dev(mean32), dev(rstd32),
                                      dev(inp["w"]))
    check_ln_bwd(inp, mean32, rstd32, host(dx), host(dw), host(db),
                 f"layernorm bwd f32 {rows}x{h}")


def check_rms_bwd(inp, dx, dw, dres, what):
    rows, h = inp["x"].shape
    dx_ref, dw_ref, rstd_ref = oracle.rmsnorm_bwd_f32(inp["dy"], inp["x"], inp["w"], inp["eps"],
                                                      dres, NT)
    xd, dyd, wd = f64(inp["x"]), f64(inp["dy"]), f64(inp["w"])
    scale = P.rmsnorm_dx_scale(xd, dyd, wd, rstd_ref, None if dres is None else f64(dres))
    P.assert_f32_scaled(dx, dx_ref, scale, h, f"{what}: dx")
    P.assert_colsum_f32(dw, dw_ref, np.abs(dyd * xd * rstd_ref[:, None]).sum(axis=0), rows,
                        walkers(rows, h), h, f"{what}: dweight")


@pytest.mark.parametrize("h,rows", BWD_SHAPES)
def test_rmsnorm_bwd_f32(h, rows):
    inp = wl.rmsnorm_bwd_inputs(rows, h, seed=h + rows + 4, f32=True)
    dx, dw = rn.rmsnorm_bwd_f32(dev(inp["dy"]), dev(inp["x"]), dev(inp["w"]), inp["eps"])
    check_rms_bwd(inp, host(dx), host(dw), None, f"rmsnorm bwd f32 {rows}x{h}")


@pytest.mark.parametrize("h,rows", BWD_SHAPES)
def test_fused_add_rmsnorm_bwd_f32(h, rows):
    inp = wl.rmsnorm_bwd_inputs(rows, h, seed=h + rows + 5, f32=True)
    ds, dw = rn.fused_add_rmsnorm_bwd_f32(dev(inp["dy"]), dev(inp["x"]), dev(inp["w"]),
                                          inp["eps"], dres=dev(inp["dres"]))
    check_rms_bwd(inp, host(ds), host(dw), inp["dres"], f"fused bwd f32 {rows}x{h}")


@pytest.mark.parametrize("h", [4096, 40000])
def test_backward_f32_in_place(h):
    rows = 33
    inp = wl.rmsnorm_bwd_inputs(rows, h, seed=10, f32=True)
    dout, dres = dev(inp["dy"]), dev(inp["dres"])
    ds, dw = rn.fused_add_rmsnorm_bwd_f32(dout, dev(inp["x"]), dev(inp["w"]), inp["eps"],
                                          dres=dres, ds=dres)       # ds == dres
    assert ds.data_ptr() == dres.data_ptr()
    check_rms_bwd(inp, host(ds), host(dw), inp["dres"], "fused bwd f32, ds = dres")
    ds, dw = rn.fused_add_rmsnorm_bwd_f32(dout, dev(inp["x"]), dev(inp["w"]), inp["eps"],
                                          dres=dev(inp["dres"]), ds=dout)  # ds == dout
    check_rms_bwd(inp, host(ds), host(dw), inp["dres"], "fused bwd f32, ds = dout")

    inp = wl.layernorm_bwd_inputs(rows, h, seed=11, f32=True)
    mean32, rstd32 = ln_stats_f32(inp["x"], inp["eps"])
    dy = dev(inp["dy"])
    dx, dw, db = rn.layernorm_bwd_f32(dy, dev(inp["x"]), dev(mean32), dev(rstd32),
                                      dev(inp["w"]), dx=dy)
    assert dx.data_ptr() == dy.data_ptr()
    check_ln_bwd(inp, mean32, rstd32, host(dx), host(dw), host(db), "layernorm bwd f32 in place")


def test_backward_f32_zero_rows_zero_fill():
    h = 8196
    w = torch.ones(h, device=DEV)
    x = torch.empty((0, h), device=DEV)
    stat = torch.empty(0, device=DEV)
    dw = torch.full((h,), 3.0, device=DEV)
    db = torch.full((h,), 3.0, device=DEV)
    rn.layernorm_bwd_f32(x, x, stat, stat, w, dweight=dw, dbias=db)
    torch.cuda.synchronize()
    assert torch.all(dw == 0) and torch.all(db == 0)
    dw.fill_(5.0)
    rn.rmsnorm_bwd_f32(x, x, w, 1e-6, dweight=dw)
    torch.cuda.synchronize()
    assert torch.all(dw == 0)


def test_backward_f32_deterministic_and_dirty_workspace():
    rows, h = 700, 20000
    inp = wl.layernorm_bwd_inputs(rows, h, seed=12, f32=True)
    mean32, rstd32 = ln_stats_f32(inp["x"], inp["eps"])
    args = (dev(inp["dy"]), dev(inp["x"]), dev(mean32), dev(rstd32), dev(inp["w"]))
    need = rn.workspace_bytes_f32("layernorm_bwd", rows, h)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=DEV)  # NaN patterns
    first = rn.layernorm_bwd_f32(*args, workspace=ws)
    check_ln_bwd(inp, mean32, rstd32, host(first[0]), host(first[1]), host(first[2]),
                 "layernorm bwd f32, dirty workspace")
    for _ in range(3):
        ws.fill_(0xFF)
        again = rn.layernorm_bwd_f32(*args, workspace=ws)
        for a, c in zip(first, again):
            assert torch.equal(a.view(torch.int32), c.view(torch.int32))


def test_backward_f32_reread_path_is_bitwise_the_exchange():
    """Rows of several column tiles: the tiles' exchanged partial row sums and
    the re-read path (spin limit 0: no tile waits; 1 or 4 polls: some tiles
    give up while others wait) give the same bits."""
    rows, h = 300, 40004
    inp = wl.layernorm_bwd_inputs(rows, h, seed=15, f32=True)
    mean32, rstd32 = ln_stats_f32(inp["x"], inp["eps"])
    args = (dev(inp["dy"]), dev(inp["x"]), dev(mean32), dev(rstd32), dev(inp["w"]))
    rin = wl.rmsnorm_bwd_inputs(rows, h, seed=16, f32=True)
    rargs = (dev(rin["dy"]), dev(rin["x"]), dev(rin["w"]), rin["eps"])

    def run():
        ln = rn.layernorm_bwd_f32(*args)
        rms = rn.rmsnorm_bwd_f32(*rargs)
        fused = rn.fused_add_rmsnorm_bwd_f32(*rargs, dres=dev(rin["dres"]))
        torch.cuda.synchronize()
        return [t.clone() for t in (*ln, *rms, *fused)]

    fast = run()
    # 0: no tile waits; 1 and 4 polls: some tiles give up, others do not
    for limit in (1, 4, 0):
        old = rn.set_bwd_spin_limit(limit)
        try:
            slow = run()
        finally:
            rn.set_bwd_spin_limit(old)
        for k, (a, c) in enumerate(zip(fast, slow)):
            assert torch.equal(a.view(torch.int32), c.view(torch.int32)), \
                f"spin limit {limit}, output {k}"
    check_ln_bwd(inp, mean32, rstd32, host(slow[0]), host(slow[1]), host(slow[2]),
                 "layernorm bwd f32, re-read path")


def test_f32_graph_replays_match_eager():
    """Forward and backward captured in one HIP graph: every replay bitwise
    equal to the eager calls (no memset nodes: the kernels write every slab
    they read)."""
    rows, h = 96, 24580
    fin = wl.fused_inputs(rows, h, seed=13, f32=True)
    bin_ = wl.layernorm_bwd_inputs(rows, h, seed=14, f32=True)
    mean32, rstd32 = ln_stats_f32(bin_["x"], bin_["eps"])
    x, r0, w = dev(fin["x"]), dev(fin["r"]), dev(fin["w"])
    dy, bx, bm, bq, bw = (dev(bin_["dy"]), dev(bin_["x"]), dev(mean32), dev(rstd32),
                          dev(bin_["w"]))
    out = torch.empty_like(x)
    r = r0.clone()
    dx = torch.empty_like(bx)
    dw = torch.empty(h, device=DEV)
    db = torch.empty(h, device=DEV)
    ws = torch.empty(rn.workspace_bytes_f32("layernorm_bwd", rows, h), dtype=torch.uint8,
                     device=DEV)

    def step():
        rn.fused_add_rmsnorm_f32(x, r, w, fin["eps"], out=out)
        rn.layernorm_bwd_f32(dy, bx, bm, bq, bw, dx=dx, dweight=dw, dbias=db, workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # eager, on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (out, r, dx, dw, db)]
    check_fused(fin, host(out), r.cpu().numpy(), h, "fused f32 eager before capture")
    g = torch.cuda.CUDAGraph()
    r.copy_(r0)
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        r.copy_(r0)
        out.zero_(); dx.zero_(); dw.zero_(); db.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, e in zip((out, r, dx, dw, db), eager):
            assert torch.equal(a.view(torch.int32), e.view(torch.int32)), f"replay {i}"


# ------------------------------------------------------------ a large call
def test_f32_fused_8192_rows():
    """8192 x 4096 fp32 (the fused operation's largest row count at its
    hidden size), every row against the oracle."""
    rows, h = 8192, 4096
    inp = wl.fused_inputs(rows, h, seed=15, f32=True)
    x, r, w = dev(inp["x"]), dev(inp["r"]), dev(inp["w"])
    out, r = rn.fused_add_rmsnorm_f32(x, r, w, inp["eps"])
    check_fused(inp, host(out), r.cpu().numpy(), h, "fused f32 8192x4096")


# ------------------------------------------------------------ seeded random sweep
def _random_cases(n=36, seed=20251203):
    """(op, rows, hidden, seed): hidden a multiple of 4 drawn log-uniformly
    from 4 to 2^18 (every launch bucket of the fp32 kernels, one-tile and
    tiled backward rows), rows log-uniform up to 4000, at most 8 Mi elements."""
    rng = np.random.default_rng(seed)
    ops = ("fused", "rms", "ln", "ln_bwd", "rms_bwd", "fused_bwd")
    out = []
    for k in range(n):
        h = 4 * max(1, int(np.exp(rng.uniform(0.0, np.log(1 << 16)))))
        rows = max(1, int(np.exp(rng.uniform(0.0, np.log(4000.0)))))
        rows = max(1, min(rows, (8 << 20) // h))
        out.append((ops[k % len(ops)], rows, h, int(rng.integers(0, 1 << 30))))
    return out


RANDOM_CASES = _random_cases()


@pytest.mark.parametrize("op,rows,h,seed", RANDOM_CASES,
                         ids=[f"{o}-{r}x{h}" for o, r, h, _ in RANDOM_CASES])
def test_f32_random_case(op, rows, h, seed):
    what = f"random fp32 {op} {rows}x{h} seed {seed}"
    if op == "fused":
        inp = wl.fused_inputs(rows, h, seed=seed, f32=True)
        out, r = rn.fused_add_rmsnorm_f32(dev(inp["x"]), dev(inp["r"]), dev(inp["w"]), inp["eps"])
        check_fused(inp, host(out), r.cpu().numpy(), h, what)
    elif op == "rms":
        inp = wl.rmsnorm_inputs(rows, h, seed=seed, f32=True)
        out = rn.rmsnorm_fwd_f32(dev(inp["x"]), dev(inp["w"]), inp["eps"])
        ref, _ = oracle.rmsnorm_fwd_f32(inp["x"], inp["w"], inp["eps"], NT)
        P.assert_f32_scaled(host(out), ref, np.abs(ref), h, what)
    elif op == "ln":
        inp = wl.layernorm_fwd_inputs(rows, h, seed=seed, f32=True)
        y, mean, rstd = rn.layernorm_fwd_f32(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]),
                                             inp["eps"])
        check_ln_fwd(inp, host(y), host(mean), host(rstd), h, what)
    elif op == "ln_bwd":
        inp = wl.layernorm_bwd_inputs(rows, h, seed=seed, f32=True)
        mean32, rstd32 = ln_stats_f32(inp["x"], inp["eps"])
        dx, dw, db = rn.layernorm_bwd_f32(dev(inp["dy"]), dev(inp["x"]), dev(mean32),
                                          dev(rstd32), dev(inp["w"]))
        check_ln_bwd(inp, mean32, rstd32, host(dx), host(dw), host(db), what)
    else:
        inp = wl.rmsnorm_bwd_inputs(rows, h, seed=seed, f32=True)
        fused = op == "fused_bwd"
        if fused:
            dx, dw = rn.fused_add_rmsnorm_bwd_f32(dev(inp["dy"]), dev(inp["x"]), dev(inp["w"]),
                                                  inp["eps"], dres=dev(inp["dres"]))
        else:
            dx, dw = rn.rmsnorm_bwd_f32(dev(inp["dy"]), dev(inp["x"]), dev(inp["w"]), inp["eps"])
        check_rms_bwd(inp, host(dx), host(dw), inp["dres"] if fused else None, what)
