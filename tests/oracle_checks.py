"""Pins for the CPU oracle: checks that tie it to something other than itself.

Each ``check_*`` takes an ``oracle.Oracle`` and raises AssertionError on a
mismatch.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutants.py`` runs them on builds of the oracle with a mistake
planted in the C source and requires that some check fails for every mistake.

What each pin compares against:
  * bf16 codec      -- torch's own fp32<->bf16 conversions (a library routine).
  * residual        -- torch fp32 add then bf16 rounding: both routes must give
                       the same bits for every finite bf16 pair.
  * RMSNorm         -- torch.nn.functional.rms_norm in float64 (library routine);
                       closed forms (constant, one-hot and zero rows); exact
                       scale invariance at eps = 0.
  * LayerNorm fwd   -- torch.nn.functional.layer_norm / var_mean in float64;
                       invariants (zero mean, closed-form second moment,
                       constant row -> bias, affine consistency).
  * LayerNorm bwd   -- torch autograd in float64; central finite differences of
                       sum(dy * LayerNorm(x)) with the statistics recomputed
                       from x; column sums against math.fsum.
  * RMSNorm bwd     -- torch autograd of rms_norm in float64 (with and without
                       the fused op's residual gradient); central finite
                       differences; fsum column sums; closed forms (constant
                       row, orthogonality to x at eps = 0).
  * all operations  -- brute force: 50-digit decimal arithmetic on tiny rows.
"""
from __future__ import annotations

import math

import numpy as np
import torch

F = torch.nn.functional


# ---------------------------------------------------------------- helpers
def torch_bf16_bits(values_f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def torch_bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def rand_bf16(rng, shape, mean=0.0, std=1.0) -> np.ndarray:
    return torch_bf16_bits((rng.standard_normal(shape) * std + mean).astype(np.float32))


def close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    err = np.abs(a - b)
    lim = atol + rtol * np.abs(b)
    bad = ~(err <= lim)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                           f"max err {float(err.max()):.3e}")


def ln_np(x, w, b, eps):
    """LayerNorm in float64 numpy, statistics recomputed from x (test-side)."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * w + b


def stats_np(x, eps):
    mu = x.mean(axis=-1)
    var = ((x - mu[:, None]) ** 2).mean(axis=-1)
    return mu, 1.0 / np.sqrt(var + eps)


# ---------------------------------------------------------------- bf16 codec
def check_bf16_decode(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = o.bf16_decode(bits)
    ref = torch_bf16_to_f64(bits)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan_ref), "NaN patterns differ"
    assert np.array_equal(mine[~nan_ref], ref[~nan_ref]), "decoded values differ"
    assert np.array_equal(np.signbit(mine[~nan_ref]), np.signbit(ref[~nan_ref])), "zero signs"


def _encode_cases(rng) -> np.ndarray:
    cases = []
    hi = np.arange(65536, dtype=np.uint32) << 16
    # exact bf16 values, exact ties, just below / above ties
    for low in (0x0000, 0x8000, 0x7FFF, 0x8001, 0x4000, 0xC000, 0xFFFF, 0x0001):
        cases.append(hi | np.uint32(low))
    # fp32 subnormals and the smallest normals
    cases.append(np.arange(0, 1 << 20, 37, dtype=np.uint32))
    cases.append(np.arange(0x007F0000, 0x00810000, 3, dtype=np.uint32))
    # the overflow boundary: largest finite bf16 .. fp32 max
    cases.append(np.arange(0x7F7F0000, 0x7F800000, 1, dtype=np.uint32))
    cases.append(rng.integers(0, 1 << 32, size=1_000_000, dtype=np.uint64).astype(np.uint32))
    u = np.concatenate(cases)
    u = np.concatenate([u, u ^ np.uint32(0x80000000)])
    f = u.view(np.float32)
    return f[np.isfinite(f)]


def check_bf16_encode(o):
    rng = np.random.default_rng(1234)
    f = _encode_cases(rng)
    mine = o.bf16_encode(f.astype(np.float64))
    ref = torch_bf16_bits(f)
    bad = mine != ref
    assert not bad.any(), (f"{int(bad.sum())} encodings differ, e.g. fp32 bits "
                           f"{hex(f[bad][0].view(np.uint32))}: {hex(mine[bad][0])} vs "
                           f"{hex(ref[bad][0])}")


# ---------------------------------------------------------------- fused residual
def _wide_pairs(rng, n):
    """bf16 pairs (x, r) covering equal, near and far exponents and cancellation."""
    x = rand_bf16(rng, (n,))
    scale = np.exp2(rng.integers(-30, 31, size=n)).astype(np.float32)
    r = torch_bf16_bits(torch_bf16_to_f64(rand_bf16(rng, (n,))).astype(np.float32) * scale)
    r[: n // 8] = x[: n // 8] ^ np.uint16(0x8000)  # exact cancellation -> +0
    # sums past the largest finite bf16 / fp32 (must overflow to +-inf)
    big = np.array([0x7F7F, 0x7F7E, 0x7F00, 0xFF7F, 0x7F7F], np.uint16)
    x[n // 8: n // 8 + 5] = big
    r[n // 8: n // 8 + 5] = np.array([0x7F7F, 0x7F7F, 0x7F7F, 0xFF7F, 0x7F70], np.uint16)
    return x, r


def check_fused_residual(o):
    rng = np.random.default_rng(7)
    x, r = _wide_pairs(rng, 64 * 512)
    x = x.reshape(64, 512)
    r = r.reshape(64, 512)
    w = rand_bf16(rng, (512,), 1.0, 0.1)
    _, res, _ = o.fused_add_rmsnorm(x, r, w, 1e-6)
    with np.errstate(over="ignore"):
        s32 = torch_bf16_to_f64(x).astype(np.float32) + torch_bf16_to_f64(r).astype(np.float32)
    ref = torch_bf16_bits(s32)
    bad = res != ref
    assert not bad.any(), f"{int(bad.sum())} residual bits differ"
    assert (res.reshape(-1)[: (64 * 512) // 8] == 0).all(), "x + (-x) must give +0"


# ---------------------------------------------------------------- RMSNorm
def check_rms_library(o):
    rng = np.random.default_rng(11)
    for rows, hidden in ((5, 64), (3, 1000), (2, 4096)):
        x = rand_bf16(rng, (rows, hidden))
        r = rand_bf16(rng, (rows, hidden))
        w = rand_bf16(rng, (hidden,), 1.0, 0.1)
        eps = float(np.float32(1e-6))
        xd, rd, wd = (torch.from_numpy(torch_bf16_to_f64(a)) for a in (x, r, w))
        out, rstd = o.rmsnorm_fwd(x, w, eps)
        ref = F.rms_norm(xd, (hidden,), wd, eps).numpy()
        close(out, ref, 1e-13, 1e-300, "rmsnorm vs torch rms_norm")
        ref_rstd = torch.rsqrt((xd * xd).mean(-1) + eps).numpy()
        close(rstd, ref_rstd, 1e-13, 0, "rmsnorm rstd")
        fout, _, _ = o.fused_add_rmsnorm(x, r, w, eps)
        fref = F.rms_norm(xd + rd, (hidden,), wd, eps).numpy()
        close(fout, fref, 1e-13, 1e-300, "fused vs torch rms_norm(x + r)")


def check_rms_closed_forms(o):
    hidden = 256
    eps = float(np.float32(1e-6))
    rng = np.random.default_rng(3)
    w = rand_bf16(rng, (hidden,), 1.0, 0.1)
    wd = torch_bf16_to_f64(w)
    consts = np.array([1.0, -3.5, 0.0078125, 96.0], np.float32)
    x = torch_bf16_bits(np.repeat(consts[:, None], hidden, axis=1))
    out, _ = o.rmsnorm_fwd(x, w, eps)
    c = consts.astype(np.float64)[:, None]
    close(out, c / np.sqrt(c * c + eps) * wd, 1e-15, 0, "constant row")
    out0, _ = o.rmsnorm_fwd(x, w, 0.0)
    assert np.array_equal(out0, np.sign(c) * wd), "constant row at eps=0 must equal sign*w"
    a = np.float64(2.5)
    xh = np.zeros((3, hidden), np.float32)
    ks = [0, 17, hidden - 1]
    for i, k in enumerate(ks):
        xh[i, k] = a
    out, _ = o.rmsnorm_fwd(torch_bf16_bits(xh), w, eps)
    for i, k in enumerate(ks):
        exp = a / math.sqrt(a * a / hidden + eps) * wd[k]
        close(out[i, k], exp, 1e-15, 0, "one-hot value")
        others = np.delete(out[i], k)
        assert (others == 0).all(), "one-hot: other outputs must be exactly 0"
    out, _ = o.rmsnorm_fwd(np.zeros((2, hidden), np.uint16), w, eps)
    assert (out == 0).all(), "zero row"
    # fused: r = -x + c gives the constant row c
    xr = rand_bf16(rng, (4, hidden))
    xrd = torch_bf16_to_f64(xr).astype(np.float32)
    r = torch_bf16_bits(np.repeat(consts[:, None], hidden, axis=1) - xrd)
    fout, res, _ = o.fused_add_rmsnorm(xr, r, w, eps)
    sd = torch_bf16_to_f64(xr) + torch_bf16_to_f64(r)
    close(fout, sd / np.sqrt((sd * sd).mean(1, keepdims=True) + eps) * wd, 1e-14, 1e-300,
          "fused near-constant rows")


def _scale_bits(bits, k):
    return torch_bf16_bits((torch_bf16_to_f64(bits) * 2.0 ** k).astype(np.float32))


def check_rms_scale_invariance(o):
    rng = np.random.default_rng(5)
    x = rand_bf16(rng, (6, 512))
    r = rand_bf16(rng, (6, 512))
    w = rand_bf16(rng, (512,), 1.0, 0.1)
    base, _ = o.rmsnorm_fwd(x, w, 0.0)
    fbase, _, _ = o.fused_add_rmsnorm(x, r, w, 0.0)
    for k in (-7, -1, 3, 12):
        out, _ = o.rmsnorm_fwd(_scale_bits(x, k), w, 0.0)
        assert np.array_equal(out, base), f"RMSNorm(2^{k} x) != RMSNorm(x) at eps=0"
        fout, _, _ = o.fused_add_rmsnorm(_scale_bits(x, k), _scale_bits(r, k), w, 0.0)
        assert np.array_equal(fout, fbase), f"fused not scale invariant at 2^{k}"
    # eps > 0: scaling by alpha is the same as dividing eps by alpha^2
    eps = 1e-2
    out_a, _ = o.rmsnorm_fwd(_scale_bits(x, 3), w, eps)
    out_b, _ = o.rmsnorm_fwd(x, w, eps / 64.0)
    close(out_a, out_b, 1e-14, 1e-300, "scaling vs eps/alpha^2")


# ---------------------------------------------------------------- LayerNorm forward
def check_ln_library(o):
    rng = np.random.default_rng(13)
    for rows, hidden in ((4, 64), (3, 768), (2, 12288)):
        x = rand_bf16(rng, (rows, hidden), 0.5, 2.0)
        w = rand_bf16(rng, (hidden,), 1.0, 0.1)
        b = rand_bf16(rng, (hidden,), 0.0, 0.1)
        eps = float(np.float32(1e-5))
        xd, wd, bd = (torch.from_numpy(torch_bf16_to_f64(a)) for a in (x, w, b))
        y, mean, rstd = o.layernorm_fwd(x, w, b, eps)
        ref = F.layer_norm(xd, (hidden,), wd, bd, eps).numpy()
        close(y, ref, 1e-12, 1e-13, "layernorm vs torch layer_norm")
        var, mu = torch.var_mean(xd, dim=-1, unbiased=False)
        close(mean, mu.numpy(), 1e-13, 1e-15, "mean vs torch var_mean")
        close(rstd, (1.0 / torch.sqrt(var + eps)).numpy(), 1e-13, 0, "rstd vs torch var_mean")


def check_ln_invariants(o):
    rng = np.random.default_rng(17)
    eps = float(np.float32(1e-5))
    for hidden in (64, 1024, 12288):
        x = rand_bf16(rng, (3, hidden), 0.5, 2.0)
        ones = torch_bf16_bits(np.ones(hidden, np.float32))
        zeros = np.zeros(hidden, np.uint16)
        y, mean, rstd = o.layernorm_fwd(x, ones, zeros, eps)
        assert (np.abs(y.sum(1)) <= 1e-12 * hidden).all(), "sum of y must be 0"
        xd = torch_bf16_to_f64(x)
        var = ((xd - xd.mean(1, keepdims=True)) ** 2).mean(1)
        close((y * y).mean(1), var / (var + eps), 1e-12, 0, "second moment var/(var+eps)")
        w = rand_bf16(rng, (hidden,), 1.0, 0.1)
        b = rand_bf16(rng, (hidden,), 0.0, 0.1)
        yab, _, _ = o.layernorm_fwd(x, w, b, eps)
        close(yab, y * torch_bf16_to_f64(w) + torch_bf16_to_f64(b), 1e-13, 1e-14,
              "affine consistency")
        const = torch_bf16_bits(np.full((2, hidden), -1.75, np.float32))
        yc, mc, rc = o.layernorm_fwd(const, w, b, eps)
        assert np.array_equal(yc, np.broadcast_to(torch_bf16_to_f64(b), yc.shape)), \
            "constant row must give y = b"
        assert (mc == -1.75).all() and np.allclose(rc, 1 / math.sqrt(eps), rtol=1e-15)


# ---------------------------------------------------------------- LayerNorm backward
def check_lnb_autograd(o):
    rng = np.random.default_rng(19)
    eps = float(np.float32(1e-5))
    for rows, hidden in ((5, 64), (7, 1024), (3, 4096)):
        x = rand_bf16(rng, (rows, hidden))
        dy = rand_bf16(rng, (rows, hidden))
        w = rand_bf16(rng, (hidden,), 1.0, 0.1)
        b = rand_bf16(rng, (hidden,), 0.0, 0.1)
        xd = torch_bf16_to_f64(x)
        mu, rstd = stats_np(xd, eps)
        dx, dw, db = o.layernorm_bwd(dy, x, mu, rstd, w)
        xt = torch.from_numpy(xd.copy()).requires_grad_(True)
        wt = torch.from_numpy(torch_bf16_to_f64(w)).requires_grad_(True)
        bt = torch.from_numpy(torch_bf16_to_f64(b)).requires_grad_(True)
        F.layer_norm(xt, (hidden,), wt, bt, eps).backward(torch.from_numpy(torch_bf16_to_f64(dy)))
        scale = np.abs(xt.grad.numpy()).max()
        close(dx, xt.grad.numpy(), 1e-10, 1e-12 * scale, "dx vs autograd")
        close(dw, wt.grad.numpy(), 1e-10, 1e-11, "dweight vs autograd")
        close(db, bt.grad.numpy(), 1e-12, 1e-12, "dbias vs autograd")


def check_lnb_finite_differences(o):
    rng = np.random.default_rng(23)
    eps = float(np.float32(1e-5))
    for rows, hidden in ((1, 8), (3, 16), (3, 64)):
        x = rand_bf16(rng, (rows, hidden), 0.5, 2.0)
        dy = rand_bf16(rng, (rows, hidden))
        w = rand_bf16(rng, (hidden,), 1.0, 0.1)
        b = rand_bf16(rng, (hidden,), 0.0, 0.1)
        xd, dyd, wd, bd = (torch_bf16_to_f64(a) for a in (x, dy, w, b))
        mu, rstd = stats_np(xd, eps)
        dx, dw, db = o.layernorm_bwd(dy, x, mu, rstd, w)

        def loss_row(i, xrow, wv=wd, bv=bd):
            return float(np.sum(dyd[i] * ln_np(xrow[None, :], wv, bv, eps)[0]))

        fd = np.empty_like(xd)
        for i in range(rows):
            for j in range(hidden):
                h = 1e-5 * max(1.0, abs(xd[i, j]))
                xp = xd[i].copy()
                xm = xd[i].copy()
                xp[j] += h
                xm[j] -= h
                fd[i, j] = (loss_row(i, xp) - loss_row(i, xm)) / (2 * h)
        close(dx, fd, 1e-6, 1e-6 * np.abs(fd).max(), "dx vs central finite differences")
        fdw = np.empty(hidden)
        fdb = np.empty(hidden)
        for j in range(hidden):
            wp, wm, bp, bm = wd.copy(), wd.copy(), bd.copy(), bd.copy()
            wp[j] += 1e-3
            wm[j] -= 1e-3
            bp[j] += 1e-3
            bm[j] -= 1e-3
            fdw[j] = sum(loss_row(i, xd[i], wp, bd) - loss_row(i, xd[i], wm, bd)
                         for i in range(rows)) / 2e-3
            fdb[j] = sum(loss_row(i, xd[i], wd, bp) - loss_row(i, xd[i], wd, bm)
                         for i in range(rows)) / 2e-3
        close(dw, fdw, 1e-8, 1e-9, "dweight vs finite differences")
        close(db, fdb, 1e-8, 1e-9, "dbias vs finite differences")


def check_lnb_column_sums(o):
    rng = np.random.default_rng(29)
    eps = float(np.float32(1e-5))
    rows, hidden = 3000, 96
    x = rand_bf16(rng, (rows, hidden))
    dy = rand_bf16(rng, (rows, hidden))
    w = rand_bf16(rng, (hidden,), 1.0, 0.1)
    xd, dyd = torch_bf16_to_f64(x), torch_bf16_to_f64(dy)
    mu, rstd = stats_np(xd, eps)
    dx, dw, db = o.layernorm_bwd(dy, x, mu, rstd, w)
    xhat = (xd - mu[:, None]) * rstd[:, None]
    for j in range(hidden):
        assert db[j] == math.fsum(dyd[:, j]), f"dbias[{j}] != fsum"
        ref = math.fsum(dyd[:, j] * xhat[:, j])
        assert abs(dw[j] - ref) <= 1e-12 * math.fsum(np.abs(dyd[:, j] * xhat[:, j])), \
            f"dweight[{j}] vs fsum"
    # inner-reduction invariants: sum_j dx = 0 and sum_j dx * xhat = rstd*H*c2*eps/(var+eps)
    g = dyd * torch_bf16_to_f64(w)
    c2 = (g * xhat).mean(1)
    var = 1.0 / rstd ** 2 - eps
    close(dx.sum(1), np.zeros(rows), 0, 1e-11 * np.abs(dx).sum(1).max(), "sum_j dx = 0")
    close((dx * xhat).sum(1), rstd * hidden * c2 * eps / (var + eps), 1e-6,
          1e-11 * np.abs(dx * xhat).sum(1).max(), "sum_j dx*xhat closed form")


def check_thread_count_independence(o):
    rng = np.random.default_rng(31)
    x = rand_bf16(rng, (37, 256))
    r = rand_bf16(rng, (37, 256))
    w = rand_bf16(rng, (256,), 1.0, 0.1)
    b = rand_bf16(rng, (256,), 0.0, 0.1)
    a1 = o.fused_add_rmsnorm(x, r, w, 1e-6, nthreads=1)
    a7 = o.fused_add_rmsnorm(x, r, w, 1e-6, nthreads=7)
    for u, v in zip(a1, a7):
        assert np.array_equal(u, v)
    y1 = o.layernorm_fwd(x, w, b, 1e-5, nthreads=1)
    y5 = o.layernorm_fwd(x, w, b, 1e-5, nthreads=5)
    for u, v in zip(y1, y5):
        assert np.array_equal(u, v)
    d1 = o.layernorm_bwd(r, x, y1[1], y1[2], w, nthreads=1)
    d6 = o.layernorm_bwd(r, x, y1[1], y1[2], w, nthreads=6)
    for u, v in zip(d1, d6):
        assert np.array_equal(u, v)


# ---------------------------------------------------------------- RMSNorm backward
def rms_np(x, w, eps):
    """RMSNorm in float64 numpy, statistic recomputed from x (test-side)."""
    return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps) * w


def check_rmsb_autograd(o):
    rng = np.random.default_rng(37)
    eps = float(np.float32(1e-6))
    for rows, hidden in ((5, 64), (7, 1024), (3, 4096)):
        x = rand_bf16(rng, (rows, hidden))
        dy = rand_bf16(rng, (rows, hidden))
        dres = rand_bf16(rng, (rows, hidden))
        w = rand_bf16(rng, (hidden,), 1.0, 0.1)
        xt = torch.from_numpy(torch_bf16_to_f64(x)).requires_grad_(True)
        wt = torch.from_numpy(torch_bf16_to_f64(w)).requires_grad_(True)
        F.rms_norm(xt, (hidden,), wt, eps).backward(torch.from_numpy(torch_bf16_to_f64(dy)))
        dx, dw, rstd = o.rmsnorm_bwd(dy, x, w, eps)
        scale = np.abs(xt.grad.numpy()).max()
        close(dx, xt.grad.numpy(), 1e-10, 1e-12 * scale, "rmsnorm dx vs autograd")
        close(dw, wt.grad.numpy(), 1e-10, 1e-11, "rmsnorm dweight vs autograd")
        xd = torch_bf16_to_f64(x)
        close(rstd, 1.0 / np.sqrt((xd * xd).mean(1) + eps), 1e-14, 0, "rmsnorm bwd rstd")
        # the fused op: s = x + r feeds both out and the residual output, so the
        # residual gradient adds to the normalization's input gradient
        st = torch.from_numpy(xd.copy()).requires_grad_(True)
        out = F.rms_norm(st, (hidden,), torch.from_numpy(torch_bf16_to_f64(w)), eps)
        (out * torch.from_numpy(torch_bf16_to_f64(dy))).sum().add(
            (st * torch.from_numpy(torch_bf16_to_f64(dres))).sum()).backward()
        fdx, fdw, _ = o.rmsnorm_bwd(dy, x, w, eps, dres=dres)
        close(fdx, st.grad.numpy(), 1e-10, 1e-12 * scale, "fused bwd ds vs autograd")
        assert np.array_equal(fdw, dw), "the residual gradient must not touch dweight"


def check_rmsb_finite_differences(o):
    rng = np.random.default_rng(41)
    eps = 1e-3
    for rows, hidden in ((1, 8), (3, 16), (2, 64)):
        x = rand_bf16(rng, (rows, hidden))
        dy = rand_bf16(rng, (rows, hidden))
        w = rand_bf16(rng, (hidden,), 1.0, 0.1)
        xd, dyd, wd = (torch_bf16_to_f64(a) for a in (x, dy, w))
        dx, dw, _ = o.rmsnorm_bwd(dy, x, w, eps)

        def loss_row(i, xrow, wv=wd):
            return float(np.sum(dyd[i] * rms_np(xrow[None, :], wv, eps)[0]))

        fd = np.empty_like(xd)
        for i in range(rows):
            for j in range(hidden):
                h = 1e-5 * max(1.0, abs(xd[i, j]))
                xp, xm = xd[i].copy(), xd[i].copy()
                xp[j] += h
                xm[j] -= h
                fd[i, j] = (loss_row(i, xp) - loss_row(i, xm)) / (2 * h)
        close(dx, fd, 1e-6, 1e-6 * np.abs(fd).max(), "rmsnorm dx vs finite differences")
        fdw = np.empty(hidden)
        for j in range(hidden):
            wp, wm = wd.copy(), wd.copy()
            wp[j] += 1e-3
            wm[j] -= 1e-3
            fdw[j] = sum(loss_row(i, xd[i], wp) - loss_row(i, xd[i], wm) for i in range(rows)) / 2e-3
        close(dw, fdw, 1e-8, 1e-9, "rmsnorm dweight vs finite differences")


def check_rmsb_sums_and_closed_forms(o):
    rng = np.random.default_rng(43)
    rows, hidden = 2000, 96
    eps = float(np.float32(1e-6))
    x = rand_bf16(rng, (rows, hidden))
    dy = rand_bf16(rng, (rows, hidden))
    w = rand_bf16(rng, (hidden,), 1.0, 0.1)
    xd, dyd, wd = (torch_bf16_to_f64(a) for a in (x, dy, w))
    dx, dw, rstd = o.rmsnorm_bwd(dy, x, w, eps)
    xhat = xd * rstd[:, None]
    for j in range(hidden):
        ref = math.fsum(dyd[:, j] * xhat[:, j])
        assert abs(dw[j] - ref) <= 1e-12 * math.fsum(np.abs(dyd[:, j] * xhat[:, j])), \
            f"rmsnorm dweight[{j}] vs fsum"
    # sum_j dx * x = rstd * sum_j(g x) * eps / (mean(x^2) + eps)
    g = dyd * wd
    ms = (xd * xd).mean(1)
    close((dx * xd).sum(1), rstd * (g * xd).sum(1) * eps / (ms + eps), 1e-6,
          1e-12 * np.abs(dx * xd).sum(1).max(), "sum_j dx*x closed form")
    # constant row c > 0 at eps = 0: xhat = 1, dx = (g - mean(g)) / c
    c = 2.5
    xc = torch_bf16_bits(np.full((3, hidden), c, np.float32))
    dxc, _, _ = o.rmsnorm_bwd(dy[:3], xc, w, 0.0)
    gc = dyd[:3] * wd
    close(dxc, (gc - gc.mean(1, keepdims=True)) / c, 1e-13, 1e-15, "constant row dx")
    # the residual gradient is added once, unchanged
    dres = rand_bf16(rng, (rows, hidden))
    fdx, _, _ = o.rmsnorm_bwd(dy, x, w, eps, dres=dres)
    assert np.array_equal(fdx, dx + torch_bf16_to_f64(dres)), "dres must be added as is"


# ---------------------------------------------------------------- brute force
def _dec(a):
    """float64 array -> nested lists of exact Decimals."""
    import decimal
    return [[decimal.Decimal(float(v)) for v in row] for row in np.atleast_2d(a)]


def check_decimal_brute_force(o):
    """Every operation on tiny rows recomputed with 50-digit decimal
    arithmetic from the textbook formulas (RMSNorm: Zhang & Sennrich 2019,
    eq. 4; LayerNorm: Ba, Kiros & Hinton 2016, eq. 4, and their gradients),
    element by element; the fp64 oracle must agree to ~1e-13 relative."""
    import decimal
    ctx = decimal.Context(prec=50)
    D = decimal.Decimal
    rng = np.random.default_rng(53)
    for rows, hidden in ((1, 8), (3, 16), (4, 24)):
        eps_r, eps_l = float(np.float32(1e-6)), float(np.float32(1e-5))
        x = rand_bf16(rng, (rows, hidden))
        r = rand_bf16(rng, (rows, hidden))
        dy = rand_bf16(rng, (rows, hidden))
        dres = rand_bf16(rng, (rows, hidden))
        w = rand_bf16(rng, (hidden,), 1.0, 0.1)
        b = rand_bf16(rng, (hidden,), 0.0, 0.1)
        X, R, DY, DR = (_dec(torch_bf16_to_f64(a)) for a in (x, r, dy, dres))
        W, B = _dec(torch_bf16_to_f64(w))[0], _dec(torch_bf16_to_f64(b))[0]
        H = D(hidden)
        er, el = D(eps_r), D(eps_l)

        def rms_rows(M):
            outs, rstds = [], []
            for row in M:
                ms = ctx.divide(sum((ctx.multiply(v, v) for v in row), D(0)), H)
                rs = ctx.divide(D(1), ctx.sqrt(ctx.add(ms, er)))
                rstds.append(rs)
                outs.append([ctx.multiply(ctx.multiply(v, rs), W[j]) for j, v in enumerate(row)])
            return outs, rstds

        def as_f64(M):
            return np.array([[float(v) for v in row] for row in M])

        # RMSNorm forward
        ref, _ = rms_rows(X)
        out, _ = o.rmsnorm_fwd(x, w, eps_r)
        close(out, as_f64(ref), 1e-13, 1e-300, "rmsnorm vs decimal")
        # fused: s = x + r exactly, then RMSNorm of s
        S = [[ctx.add(a, c) for a, c in zip(ra, rc)] for ra, rc in zip(X, R)]
        ref, _ = rms_rows(S)
        out, _, _ = o.fused_add_rmsnorm(x, r, w, eps_r)
        close(out, as_f64(ref), 1e-13, 1e-300, "fused out vs decimal")
        # LayerNorm forward (statistics of the exact row)
        ys, mus, rstds = [], [], []
        for row in X:
            mu = ctx.divide(sum(row, D(0)), H)
            var = ctx.divide(sum((ctx.multiply(v - mu, v - mu) for v in row), D(0)), H)
            rs = ctx.divide(D(1), ctx.sqrt(ctx.add(var, el)))
            mus.append(mu)
            rstds.append(rs)
            ys.append([ctx.add(ctx.multiply(ctx.multiply(v - mu, rs), W[j]), B[j])
                       for j, v in enumerate(row)])
        y, mean, rstd = o.layernorm_fwd(x, w, b, eps_l)
        scale = np.abs(as_f64(ys)).max()
        close(y, as_f64(ys), 1e-13, 1e-14 * scale, "layernorm y vs decimal")
        close(mean, [float(m) for m in mus], 1e-13, 1e-15, "layernorm mean vs decimal")
        close(rstd, [float(v) for v in rstds], 1e-13, 0, "layernorm rstd vs decimal")
        # LayerNorm backward with the given (fp64) statistics
        MEAN, RSTD = [D(float(m)) for m in mean], [D(float(v)) for v in rstd]
        dx_ref, dw_ref, db_ref = [], [D(0)] * hidden, [D(0)] * hidden
        for i in range(rows):
            xh = [ctx.multiply(X[i][j] - MEAN[i], RSTD[i]) for j in range(hidden)]
            g = [ctx.multiply(DY[i][j], W[j]) for j in range(hidden)]
            c1 = ctx.divide(sum(g, D(0)), H)
            c2 = ctx.divide(sum((ctx.multiply(g[j], xh[j]) for j in range(hidden)), D(0)), H)
            dx_ref.append([ctx.multiply(RSTD[i], g[j] - c1 - ctx.multiply(xh[j], c2))
                           for j in range(hidden)])
            for j in range(hidden):
                dw_ref[j] = ctx.add(dw_ref[j], ctx.multiply(DY[i][j], xh[j]))
                db_ref[j] = ctx.add(db_ref[j], DY[i][j])
        dx, dw, db = o.layernorm_bwd(dy, x, mean, rstd, w)
        scale = np.abs(as_f64(dx_ref)).max()
        close(dx, as_f64(dx_ref), 1e-12, 1e-13 * scale, "layernorm dx vs decimal")
        close(dw, [float(v) for v in dw_ref], 1e-12, 1e-13, "layernorm dweight vs decimal")
        close(db, [float(v) for v in db_ref], 1e-13, 1e-14, "layernorm dbias vs decimal")
        # RMSNorm backward (statistic recomputed), with the fused op's residual gradient
        _, RS = rms_rows(X)
        dx_ref, dw_ref = [], [D(0)] * hidden
        for i in range(rows):
            xh = [ctx.multiply(X[i][j], RS[i]) for j in range(hidden)]
            g = [ctx.multiply(DY[i][j], W[j]) for j in range(hidden)]
            c = ctx.divide(sum((ctx.multiply(g[j], xh[j]) for j in range(hidden)), D(0)), H)
            dx_ref.append([ctx.add(ctx.multiply(RS[i], g[j] - ctx.multiply(xh[j], c)), DR[i][j])
                           for j in range(hidden)])
            for j in range(hidden):
                dw_ref[j] = ctx.add(dw_ref[j], ctx.multiply(DY[i][j], xh[j]))
        dx, dw, _ = o.rmsnorm_bwd(dy, x, w, eps_r, dres=dres)
        scale = np.abs(as_f64(dx_ref)).max()
        close(dx, as_f64(dx_ref), 1e-12, 1e-13 * scale, "rmsnorm bwd dx vs decimal")
        close(dw, [float(v) for v in dw_ref], 1e-12, 1e-13, "rmsnorm bwd dweight vs decimal")


ALL_CHECKS = [
    check_bf16_decode,
    check_bf16_encode,
    check_fused_residual,
    check_rms_library,
    check_rms_closed_forms,
    check_rms_scale_invariance,
    check_ln_library,
    check_ln_invariants,
    check_lnb_autograd,
    check_lnb_finite_differences,
    check_lnb_column_sums,
    check_rmsb_autograd,
    check_rmsb_finite_differences,
    check_rmsb_sums_and_closed_forms,
    check_decimal_brute_force,
    check_thread_count_independence,
]
