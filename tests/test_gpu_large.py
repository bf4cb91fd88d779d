"""GPU parity past 4 GiB per matrix: every kernel family's 64-bit row
addressing (row offsets beyond 2^31 and 2^32 bytes), through the C ABI,
for bf16 and fp32 activations.

The matrices are drawn on the device from seeded generators
(workloads.device_normal_bf16); the oracle recomputes sampled rows: the first
rows, the rows on either side of the 2^31- and 2^32-byte offsets, the ragged
last rows and a few seeded random rows.  Outputs are filled with NaN before
each call, so an element the kernels never wrote fails the all-finite check
on the whole output.  Column sums (dweight, dbias) cover every row: the
oracle's backward runs over the whole matrix in row chunks (copied to the
host), and its per-chunk column sums are added in fp64.  Rules in
parity.py."""
import os

import numpy as np
import pytest
import torch

import oracle
import parity as P
import row_normalization_persistent_amd as rn
from row_normalization_persistent_amd import workloads as wl

pytestmark = pytest.mark.gpu

# The largest case holds about 20 GiB at once (three or four 4 GiB matrices
# and fp64 column-sum chunks).
NEED_BYTES = 24 << 30


@pytest.fixture(autouse=True)
def _enough_device_memory():
    total = torch.cuda.get_device_properties(0).total_memory
    if total < NEED_BYTES:
        pytest.skip(f"needs {NEED_BYTES >> 30} GiB of device memory, the device has "
                    f"{total >> 30} GiB")

NT = min(16, os.cpu_count() or 1)
DEV = "cuda"
GIB4 = 1 << 32


def rows_past_4gib(hidden: int, extra: int, ld: int | None = None) -> int:
    """Rows of a bf16 matrix with row stride ld (default hidden) whose last
    rows lie past 2^32 bytes."""
    return GIB4 // (2 * (ld or hidden)) + extra


def sample_rows(rows: int, row_bytes: int, seed: int) -> np.ndarray:
    picks = {0, 1, rows - 2, rows - 1}
    for edge in (1 << 31, 1 << 32):
        r = edge // row_bytes
        picks.update({r - 1, r, r + 1})
    picks.update(np.random.default_rng(seed).integers(0, rows, 6).tolist())
    return np.array(sorted(p for p in picks if 0 <= p < rows), np.int64)


def take(t: torch.Tensor, idx: np.ndarray) -> np.ndarray:
    """Rows idx of a bf16 device matrix as host bf16 bits."""
    sel = t.index_select(0, torch.from_numpy(idx).to(t.device))
    return wl.from_device_bf16(sel)


def assert_all_finite(t: torch.Tensor, what: str):
    bad = int((~torch.isfinite(t.float() if t.dtype == torch.bfloat16 else t)).sum().item())
    assert bad == 0, f"{what}: {bad} elements not written (still NaN) or not finite"


def nan_like(t: torch.Tensor) -> torch.Tensor:
    return torch.full(t.shape, float("nan"), dtype=t.dtype, device=t.device)


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def weight(hidden, seed, mean=1.0, std=0.1):
    rng = np.random.default_rng(seed)
    bits = wl.bf16_bits((rng.standard_normal(hidden) * std + mean).astype(np.float32))
    return bits, wl.to_device_bf16(bits, DEV)


def oracle_colsums(n_rows, chunk_fn, chunk=1 << 15):
    """Column sums over all rows from the oracle: chunk_fn(a, b) runs the
    oracle's backward on rows a..b (host copies) and returns, per output,
    (its column sums, a per-column scale of the summed terms: their squares'
    sums for the bf16 rule, their absolute values' sums for the fp32 one);
    both are added over the chunks in fp64.  The scale enters the tolerance
    only."""
    tot = None
    for k, a in enumerate(range(0, n_rows, chunk)):
        part = chunk_fn(a, min(n_rows, a + chunk))
        tot = part if tot is None else [(s + ps, q + pq) for (s, q), (ps, pq) in zip(tot, part)]
        if k % 4 == 0:
            print(f"  oracle column sums: rows {a} .. {min(n_rows, a + chunk)} of {n_rows}",
                  flush=True)
    return tot


def f64_rows(bits: np.ndarray) -> torch.Tensor:
    """bf16 bit rows on the host as an fp64 CPU tensor (exact)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).double()


def test_fused_add_rmsnorm_past_4gib():
    """hidden 4096 (compiled kernels): x, residual, out of 4 GiB + 77 rows each."""
    h = 4096
    rows = rows_past_4gib(h, 77)
    idx = sample_rows(rows, 2 * h, seed=1)
    x = wl.device_normal_bf16(rows, h, 0.0, 1.0, seed=101)
    r = wl.device_normal_bf16(rows, h, 0.0, 1.0, seed=102)
    w_bits, w = weight(h, 103)
    xs, rs = take(x, idx), take(r, idx)
    out = nan_like(x)
    rn.fused_add_rmsnorm(x, r, w, wl.EPS_RMS, out=out)
    torch.cuda.synchronize()
    ref, res_ref, _ = oracle.fused_add_rmsnorm(xs, rs, w_bits, wl.EPS_RMS, NT)
    P.assert_bits_equal(take(r, idx), res_ref, "fused past 4 GiB: residual")
    P.assert_bf16_close(take(out, idx), ref, "fused past 4 GiB: out")
    assert_all_finite(out, "fused past 4 GiB: out")
    del x, r, out
    free()


def test_fused_add_rmsnorm_runtime_hidden_past_4gib():
    """hidden 5120 (run-time-hidden kernels): 4 GiB + 3 rows each."""
    h = 5120
    rows = rows_past_4gib(h, 3)
    idx = sample_rows(rows, 2 * h, seed=2)
    x = wl.device_normal_bf16(rows, h, 0.0, 1.0, seed=201)
    r = wl.device_normal_bf16(rows, h, 0.0, 1.0, seed=202)
    w_bits, w = weight(h, 203)
    xs, rs = take(x, idx), take(r, idx)
    out = nan_like(x)
    rn.fused_add_rmsnorm(x, r, w, wl.EPS_RMS, out=out)
    torch.cuda.synchronize()
    ref, res_ref, _ = oracle.fused_add_rmsnorm(xs, rs, w_bits, wl.EPS_RMS, NT)
    P.assert_bits_equal(take(r, idx), res_ref, "run-time fused past 4 GiB: residual")
    P.assert_bf16_close(take(out, idx), ref, "run-time fused past 4 GiB: out")
    assert_all_finite(out, "run-time fused past 4 GiB: out")
    del x, r, out
    free()


def test_rmsnorm_fwd_past_4gib():
    """hidden 2048: 2^20 + 3 rows (4 GiB + 12 KiB per matrix)."""
    h = 2048
    rows = rows_past_4gib(h, 3)
    idx = sample_rows(rows, 2 * h, seed=3)
    x = wl.device_normal_bf16(rows, h, 0.0, 1.0, seed=301)
    w_bits, w = weight(h, 302)
    out = nan_like(x)
    rn.rmsnorm_fwd(x, w, wl.EPS_RMS, out=out)
    torch.cuda.synchronize()
    ref, _ = oracle.rmsnorm_fwd(take(x, idx), w_bits, wl.EPS_RMS, NT)
    P.assert_bf16_close(take(out, idx), ref, "rmsnorm past 4 GiB")
    assert_all_finite(out, "rmsnorm past 4 GiB")
    del x, out
    free()


def test_rmsnorm_fwd_ring_past_4gib():
    """hidden 16384 (the persistent ring kernel, deepest ring): 4 GiB + 5 rows."""
    h = 16384
    rows = rows_past_4gib(h, 5)
    idx = sample_rows(rows, 2 * h, seed=8)
    x = wl.device_normal_bf16(rows, h, 0.0, 1.0, seed=801)
    w_bits, w = weight(h, 802)
    assert "rmsnorm_fwd_ring_kernel" in rn.describe_config("rmsnorm_fwd", rows, h)
    out = nan_like(x)
    rn.rmsnorm_fwd(x, w, wl.EPS_RMS, out=out)
    torch.cuda.synchronize()
    ref, _ = oracle.rmsnorm_fwd(take(x, idx), w_bits, wl.EPS_RMS, NT)
    P.assert_bf16_close(take(out, idx), ref, "rmsnorm ring past 4 GiB")
    assert_all_finite(out, "rmsnorm ring past 4 GiB")
    del x, out
    free()


def test_rmsnorm_fwd_column_slice_past_4gib():
    """In place on the first 128 columns of a [rows, 384] matrix of 4 GiB + 5
    rows (narrow rows share one buffer descriptor per set of rows)."""
    h, ld = 128, 384
    rows = rows_past_4gib(h, 5, ld)
    idx = sample_rows(rows, 2 * ld, seed=4)
    xv = wl.device_normal_bf16(rows, h, 0.0, 1.0, seed=401, ld=ld)
    w_bits, w = weight(h, 402)
    xs = take(xv, idx)
    full = xv.as_strided((rows, ld), (ld, 1))
    rest = full[:, h:].clone()
    rn.rmsnorm_fwd(xv, w, wl.EPS_RMS, out=xv)
    torch.cuda.synchronize()
    ref, _ = oracle.rmsnorm_fwd(xs, w_bits, wl.EPS_RMS, NT)
    P.assert_bf16_close(take(xv, idx), ref, "rmsnorm slice past 4 GiB")
    assert torch.equal(full[:, h:], rest), "columns outside the slice changed"
    del xv, full, rest
    free()


def test_layernorm_fwd_past_4gib():
    """hidden 16384 (the persistent ring kernel): 4 GiB + 5 rows per matrix."""
    h = 16384
    rows = rows_past_4gib(h, 5)
    idx = sample_rows(rows, 2 * h, seed=5)
    x = wl.device_normal_bf16(rows, h, 0.5, 2.0, seed=501)
    w_bits, w = weight(h, 502)
    b_bits, b = weight(h, 503, mean=0.0, std=0.1)
    y = nan_like(x)
    mean = torch.full((rows,), float("nan"), dtype=torch.float32, device=DEV)
    rstd = torch.full((rows,), float("nan"), dtype=torch.float32, device=DEV)
    assert "ring" in rn.describe_config("layernorm_fwd", rows, h)
    rn.layernorm_fwd(x, w, b, wl.EPS_LN, y=y, mean=mean, rstd=rstd)
    torch.cuda.synchronize()
    xs = take(x, idx)
    ref, mean_ref, rstd_ref = oracle.layernorm_fwd(xs, w_bits, b_bits, wl.EPS_LN, NT)
    xd, wd, bd = P.bits_to_f64(xs), P.bits_to_f64(w_bits), P.bits_to_f64(b_bits)
    scale = P.layernorm_y_scale(xd, mean_ref, rstd_ref, wd, bd)
    P.assert_bf16_close(take(y, idx), ref, "layernorm past 4 GiB: y", floor_scale=scale)
    ti = torch.from_numpy(idx).to(DEV)
    P.assert_f32_close(mean[ti].cpu().numpy(), mean_ref, "layernorm past 4 GiB: mean")
    P.assert_f32_close(rstd[ti].cpu().numpy(), rstd_ref, "layernorm past 4 GiB: rstd")
    assert_all_finite(y, "layernorm past 4 GiB: y")
    assert_all_finite(mean, "layernorm past 4 GiB: mean")
    assert_all_finite(rstd, "layernorm past 4 GiB: rstd")
    del x, y, mean, rstd
    free()


def test_layernorm_bwd_past_4gib():
    """hidden 4096: x, dy, dx of 4 GiB + 77 rows.  mean and rstd are drawn
    (inputs of the backward, used as given by both sides), not computed from x."""
    h = 4096
    rows = rows_past_4gib(h, 77)
    idx = sample_rows(rows, 2 * h, seed=6)
    x = wl.device_normal_bf16(rows, h, 0.0, 1.0, seed=601)
    dy = wl.device_normal_bf16(rows, h, 0.0, 1.0, seed=602)
    mean = wl.device_normal_f32(rows, 0.0, 0.02, seed=603)
    rstd = wl.device_normal_f32(rows, 1.0, 0.05, seed=604)
    w_bits, w = weight(h, 605)
    dx = nan_like(x)
    dw = torch.full((h,), float("nan"), dtype=torch.float32, device=DEV)
    db = torch.full((h,), float("nan"), dtype=torch.float32, device=DEV)
    rn.layernorm_bwd(dy, x, mean, rstd, w, dx=dx, dweight=dw, dbias=db)
    torch.cuda.synchronize()
    ti = torch.from_numpy(idx).to(DEV)
    xs, dys = take(x, idx), take(dy, idx)
    ms, rs = mean[ti].cpu().numpy(), rstd[ti].cpu().numpy()
    dx_ref, _, _ = oracle.layernorm_bwd(dys, xs, ms, rs, w_bits, NT)
    xd, dyd, wd = P.bits_to_f64(xs), P.bits_to_f64(dys), P.bits_to_f64(w_bits)
    scale = P.layernorm_dx_scale(xd, dyd, wd, ms.astype(np.float64), rs.astype(np.float64))
    P.assert_bf16_close(take(dx, idx), dx_ref, "layernorm bwd past 4 GiB: dx", floor_scale=scale)
    assert_all_finite(dx, "layernorm bwd past 4 GiB: dx")

    def chunk(a, b):
        xs, dys = wl.from_device_bf16(x[a:b]), wl.from_device_bf16(dy[a:b])
        ms, rs = mean[a:b].cpu().numpy(), rstd[a:b].cpu().numpy()
        _, cdw, cdb = oracle.layernorm_bwd(dys, xs, ms, rs, w_bits, NT)
        dyt = f64_rows(dys)
        xhat = (f64_rows(xs) - torch.from_numpy(ms).double()[:, None]) * \
            torch.from_numpy(rs).double()[:, None]
        return [(cdw, ((dyt * xhat) ** 2).sum(0).numpy()), (cdb, (dyt * dyt).sum(0).numpy())]

    (dw_ref, dw_q), (db_ref, db_q) = oracle_colsums(rows, chunk)
    P.assert_colsum_close(dw.cpu().numpy(), dw_ref, dw_q, "layernorm bwd past 4 GiB: dweight")
    P.assert_colsum_close(db.cpu().numpy(), db_ref, db_q, "layernorm bwd past 4 GiB: dbias")
    del x, dy, dx, mean, rstd
    free()


def test_fused_add_rmsnorm_bwd_past_4gib():
    """hidden 4096, with the residual gradient: s, dout, dres, ds of 4 GiB + 7 rows."""
    h = 4096
    rows = rows_past_4gib(h, 7)
    idx = sample_rows(rows, 2 * h, seed=7)
    s = wl.device_normal_bf16(rows, h, 0.0, 1.0, seed=701)
    dout = wl.device_normal_bf16(rows, h, 0.0, 1.0, seed=702)
    dres = wl.device_normal_bf16(rows, h, 0.0, 1.0, seed=703)
    w_bits, w = weight(h, 704)
    ds = nan_like(s)
    dw = torch.full((h,), float("nan"), dtype=torch.float32, device=DEV)
    rn.fused_add_rmsnorm_bwd(dout, s, w, wl.EPS_RMS, dres=dres, ds=ds, dweight=dw)
    torch.cuda.synchronize()
    ss, dos, drs = take(s, idx), take(dout, idx), take(dres, idx)
    dx_ref, _, rstd = oracle.rmsnorm_bwd(dos, ss, w_bits, wl.EPS_RMS, dres=drs, nthreads=NT)
    xd, dyd, wd = P.bits_to_f64(ss), P.bits_to_f64(dos), P.bits_to_f64(w_bits)
    scale = P.rmsnorm_dx_scale(xd, dyd, wd, rstd, P.bits_to_f64(drs))
    P.assert_bf16_close(take(ds, idx), dx_ref, "fused bwd past 4 GiB: ds", floor_scale=scale)
    assert_all_finite(ds, "fused bwd past 4 GiB: ds")

    def chunk(a, b):
        sc, dc = wl.from_device_bf16(s[a:b]), wl.from_device_bf16(dout[a:b])
        # dres does not enter dweight: the oracle adds it to ds only
        _, cdw, crstd = oracle.rmsnorm_bwd(dc, sc, w_bits, wl.EPS_RMS, nthreads=NT)
        t = f64_rows(dc) * f64_rows(sc) * torch.from_numpy(crstd)[:, None]
        return [(cdw, (t * t).sum(0).numpy())]

    ((dw_ref, dw_q),) = oracle_colsums(rows, chunk)
    P.assert_colsum_close(dw.cpu().numpy(), dw_ref, dw_q, "fused bwd past 4 GiB: dweight")
    del s, dout, dres, ds
    free()


def test_streamed_fused_add_rmsnorm_past_4gib():
    """hidden 131072 (the streamed two-pass kernel): x, residual, out of 4 GiB
    + 3 rows each."""
    h = 131072
    rows = rows_past_4gib(h, 3)
    idx = sample_rows(rows, 2 * h, seed=9)
    assert "stream_fwd_kernel" in rn.describe_config("fused_add_rmsnorm", rows, h)
    x = wl.device_normal_bf16(rows, h, 0.0, 1.0, seed=901)
    r = wl.device_normal_bf16(rows, h, 0.0, 1.0, seed=902)
    w_bits, w = weight(h, 903)
    xs, rs = take(x, idx), take(r, idx)
    out = nan_like(x)
    rn.fused_add_rmsnorm(x, r, w, wl.EPS_RMS, out=out)
    torch.cuda.synchronize()
    ref, res_ref, _ = oracle.fused_add_rmsnorm(xs, rs, w_bits, wl.EPS_RMS, NT)
    P.assert_bits_equal(take(r, idx), res_ref, "streamed fused past 4 GiB: residual")
    P.assert_bf16_close(take(out, idx), ref, "streamed fused past 4 GiB: out")
    assert_all_finite(out, "streamed fused past 4 GiB: out")
    del x, r, out
    free()


def test_streamed_layernorm_bwd_past_4gib():
    """hidden 65536 (row reductions, then column tiles): x, dy, dx of 4 GiB + 5
    rows; column sums over every row against chunked oracle calls."""
    h = 65536
    rows = rows_past_4gib(h, 5)
    idx = sample_rows(rows, 2 * h, seed=10)
    assert "stream_bwd_tile_kernel" in rn.describe_config("layernorm_bwd", rows, h)
    x = wl.device_normal_bf16(rows, h, 0.0, 1.0, seed=1001)
    dy = wl.device_normal_bf16(rows, h, 0.0, 1.0, seed=1002)
    mean = wl.device_normal_f32(rows, 0.0, 0.02, seed=1003)
    rstd = wl.device_normal_f32(rows, 1.0, 0.05, seed=1004)
    w_bits, w = weight(h, 1005)
    dx = nan_like(x)
    dw = torch.full((h,), float("nan"), dtype=torch.float32, device=DEV)
    db = torch.full((h,), float("nan"), dtype=torch.float32, device=DEV)
    rn.layernorm_bwd(dy, x, mean, rstd, w, dx=dx, dweight=dw, dbias=db)
    torch.cuda.synchronize()
    ti = torch.from_numpy(idx).to(DEV)
    xs, dys = take(x, idx), take(dy, idx)
    ms, rs = mean[ti].cpu().numpy(), rstd[ti].cpu().numpy()
    dx_ref, _, _ = oracle.layernorm_bwd(dys, xs, ms, rs, w_bits, NT)
    xd, dyd, wd = P.bits_to_f64(xs), P.bits_to_f64(dys), P.bits_to_f64(w_bits)
    scale = P.layernorm_dx_scale(xd, dyd, wd, ms.astype(np.float64), rs.astype(np.float64))
    P.assert_bf16_close(take(dx, idx), dx_ref, "streamed layernorm bwd past 4 GiB: dx",
                        floor_scale=scale)
    assert_all_finite(dx, "streamed layernorm bwd past 4 GiB: dx")

    def chunk(a, b):
        xc, dc = wl.from_device_bf16(x[a:b]), wl.from_device_bf16(dy[a:b])
        mc, rc = mean[a:b].cpu().numpy(), rstd[a:b].cpu().numpy()
        _, cdw, cdb = oracle.layernorm_bwd(dc, xc, mc, rc, w_bits, NT)
        dyt = f64_rows(dc)
        xhat = (f64_rows(xc) - torch.from_numpy(mc).double()[:, None]) * \
            torch.from_numpy(rc).double()[:, None]
        return [(cdw, ((dyt * xhat) ** 2).sum(0).numpy()), (cdb, (dyt * dyt).sum(0).numpy())]

    (dw_ref, dw_q), (db_ref, db_q) = oracle_colsums(rows, chunk, chunk=1 << 12)
    P.assert_colsum_close(dw.cpu().numpy(), dw_ref, dw_q,
                          "streamed layernorm bwd past 4 GiB: dweight")
    P.assert_colsum_close(db.cpu().numpy(), db_ref, db_q,
                          "streamed layernorm bwd past 4 GiB: dbias")
    del x, dy, dx, mean, rstd
    free()


# ------------------------------------------------------------- fp32 activations
def device_normal_f32_rows(rows: int, hidden: int, mean: float, std: float,
                           seed: int) -> torch.Tensor:
    """A [rows, hidden] fp32 matrix ~ N(mean, std) drawn on the device."""
    return wl.device_normal_f32(rows * hidden, mean, std, seed, DEV).view(rows, hidden)


def take_f32(t: torch.Tensor, idx: np.ndarray) -> np.ndarray:
    return t.index_select(0, torch.from_numpy(idx).to(t.device)).cpu().numpy()


def test_f32_fused_add_rmsnorm_past_4gib():
    """fp32 hidden 4096: x, residual, out of 4 GiB + 77 rows each."""
    h = 4096
    rows = GIB4 // (4 * h) + 77
    idx = sample_rows(rows, 4 * h, seed=11)
    x = device_normal_f32_rows(rows, h, 0.0, 1.0, seed=1101)
    r = device_normal_f32_rows(rows, h, 0.0, 1.0, seed=1102)
    w = wl.device_normal_f32(h, 1.0, 0.1, 1103, DEV)
    xs, rs = take_f32(x, idx), take_f32(r, idx)
    out = nan_like(x)
    rn.fused_add_rmsnorm_f32(x, r, w, wl.EPS_RMS, out=out)
    torch.cuda.synchronize()
    ref, res_ref, _ = oracle.fused_add_rmsnorm_f32(xs, rs, w.cpu().numpy(), wl.EPS_RMS, NT)
    assert np.array_equal(take_f32(r, idx).view(np.uint32), res_ref.view(np.uint32)), \
        "fp32 fused past 4 GiB: residual"
    P.assert_f32_scaled(take_f32(out, idx), ref, np.abs(ref), h, "fp32 fused past 4 GiB: out")
    assert_all_finite(out, "fp32 fused past 4 GiB: out")
    del x, r, out
    free()


def test_f32_layernorm_bwd_past_4gib():
    """fp32 hidden 4096: x, dy, dx of 4 GiB + 77 rows (one-tile rows reduced
    in the tile kernel); mean and rstd drawn (inputs used as given)."""
    h = 4096
    rows = GIB4 // (4 * h) + 77
    idx = sample_rows(rows, 4 * h, seed=12)
    x = device_normal_f32_rows(rows, h, 0.0, 1.0, seed=1201)
    dy = device_normal_f32_rows(rows, h, 0.0, 1.0, seed=1202)
    mean = wl.device_normal_f32(rows, 0.0, 0.02, 1203, DEV)
    rstd = wl.device_normal_f32(rows, 1.0, 0.05, 1204, DEV)
    w = wl.device_normal_f32(h, 1.0, 0.1, 1205, DEV)
    w_h = w.cpu().numpy()
    dx = nan_like(x)
    dw = torch.full((h,), float("nan"), dtype=torch.float32, device=DEV)
    db = torch.full((h,), float("nan"), dtype=torch.float32, device=DEV)
    rn.layernorm_bwd_f32(dy, x, mean, rstd, w, dx=dx, dweight=dw, dbias=db)
    torch.cuda.synchronize()
    ti = torch.from_numpy(idx).to(DEV)
    xs, dys = take_f32(x, idx), take_f32(dy, idx)
    ms, rs = mean[ti].cpu().numpy(), rstd[ti].cpu().numpy()
    dx_ref, _, _ = oracle.layernorm_bwd_f32(dys, xs, ms, rs, w_h, NT)
    scale = P.layernorm_dx_scale(xs.astype(np.float64), dys.astype(np.float64),
                                 w_h.astype(np.float64), ms.astype(np.float64),
                                 rs.astype(np.float64))
    P.assert_f32_scaled(take_f32(dx, idx), dx_ref, scale, h, "fp32 layernorm bwd past 4 GiB: dx")
    assert_all_finite(dx, "fp32 layernorm bwd past 4 GiB: dx")

    def chunk(a, b):
        xc, dyc = x[a:b].cpu().numpy(), dy[a:b].cpu().numpy()
        mc, rc = mean[a:b].cpu().numpy(), rstd[a:b].cpu().numpy()
        _, cdw, cdb = oracle.layernorm_bwd_f32(dyc, xc, mc, rc, w_h, NT)
        dyt = torch.from_numpy(dyc).double()
        xhat = (torch.from_numpy(xc).double() - torch.from_numpy(mc).double()[:, None]) * \
            torch.from_numpy(rc).double()[:, None]
        return [(cdw, (dyt * xhat).abs().sum(0).numpy()), (cdb, dyt.abs().sum(0).numpy())]

    (dw_ref, dw_a), (db_ref, db_a) = oracle_colsums(rows, chunk)
    p = max(1, min(rows, 255))  # row walkers of a one-tile fp32 row
    P.assert_colsum_f32(dw.cpu().numpy(), dw_ref, dw_a, rows, p, h,
                        "fp32 layernorm bwd past 4 GiB: dweight")
    P.assert_colsum_f32(db.cpu().numpy(), db_ref, db_a, rows, p, h,
                        "fp32 layernorm bwd past 4 GiB: dbias")
    del x, dy, dx, mean, rstd
    free()
