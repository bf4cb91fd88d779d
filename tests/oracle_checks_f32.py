"""Pins for the oracle's fp32-activation functions (oracle_f32.c): checks that
tie them to something other than themselves.  Each ``check_*`` takes an
``oracle.Oracle`` and raises AssertionError on a mismatch;
``test_oracle_pins.py`` runs them on the real oracle and
``test_oracle_mutants.py`` on builds with a mistake planted in oracle_f32.c.

What each pin compares against:
  * residual       -- torch's float32 add (a library routine): bit for bit,
                      over ties, wide exponent gaps, cancellation, overflow.
  * bf16 oracle    -- on binary32 inputs that are bf16 values, every output of
                      every function equals the bf16 oracle's (pinned on its
                      own in oracle_checks.py) bit for bit: the same sums in
                      the same order.
  * library        -- on general binary32 inputs: torch rms_norm / layer_norm
                      in float64 and torch autograd in float64 for both
                      backward passes (with and without the residual
                      gradient).
  * closed forms   -- constant rows (RMSNorm: c / sqrt(c^2 + eps) * w;
                      LayerNorm: y = b), zero rows of dy (dx = 0).
"""
from __future__ import annotations

import numpy as np
import torch

from oracle_checks import close, rand_bf16, torch_bf16_to_f64

F = torch.nn.functional


def _f32(rng, shape, mean=0.0, std=1.0):
    return (rng.standard_normal(shape) * std + mean).astype(np.float32)


def check_f32_residual(o):
    rng = np.random.default_rng(21)
    rows, hidden = 8, 512
    x = _f32(rng, (rows, hidden))
    r = _f32(rng, (rows, hidden))
    # row 1: ties (x = 1 + k ulp, r = half an ulp), row 2: wide gaps, row 3:
    # cancellation, row 4: overflow
    ulp = np.float32(2.0 ** -23)
    x[1] = np.float32(1.0) + ulp * np.arange(hidden, dtype=np.float32) % 64
    r[1] = ulp / 2
    x[2] = np.float32(1e30)
    r[2] = _f32(rng, (hidden,)) * np.float32(1e-10)
    r[3] = -x[3]
    x[4, :8] = np.float32(3e38)
    r[4, :8] = np.float32(3e38)
    w = _f32(rng, (hidden,), 1.0, 0.1)
    _, res, _ = o.fused_add_rmsnorm_f32(x, r, w, 1e-6)
    with np.errstate(over="ignore"):
        ref = (torch.from_numpy(x) + torch.from_numpy(r)).numpy()
    assert np.array_equal(res.view(np.uint32), ref.view(np.uint32)), \
        f"{int((res.view(np.uint32) != ref.view(np.uint32)).sum())} residual bits differ"
    assert (res[3].view(np.uint32) == 0).all(), "x + (-x) must give +0"
    assert np.isinf(res[4, :8]).all()


def check_f32_matches_bf16_oracle(o):
    rng = np.random.default_rng(22)
    rows, hidden = 6, 300
    bits = {k: rand_bf16(rng, (rows, hidden)) for k in ("x", "r", "dy", "dres")}
    wb = rand_bf16(rng, (hidden,), 1.0, 0.1)
    bb = rand_bf16(rng, (hidden,), 0.0, 0.1)
    f = {k: torch_bf16_to_f64(v).astype(np.float32) for k, v in bits.items()}
    w, b = torch_bf16_to_f64(wb).astype(np.float32), torch_bf16_to_f64(bb).astype(np.float32)
    eps = float(np.float32(1e-6))

    def same(a, c, what):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(c).view(np.uint8)), what

    o32, _, rs32 = o.fused_add_rmsnorm_f32(f["x"], f["r"], w, eps)
    o16, _, rs16 = o.fused_add_rmsnorm(bits["x"], bits["r"], wb, eps)
    same(o32, o16, "fused out"), same(rs32, rs16, "fused rstd")
    same(o.rmsnorm_fwd_f32(f["x"], w, eps)[0], o.rmsnorm_fwd(bits["x"], wb, eps)[0], "rmsnorm")
    for a, c, n in zip(o.layernorm_fwd_f32(f["x"], w, b, eps),
                       o.layernorm_fwd(bits["x"], wb, bb, eps), ("y", "mean", "rstd")):
        same(a, c, f"layernorm {n}")
    _, mean, rstd = o.layernorm_fwd(bits["x"], wb, bb, eps)
    for a, c, n in zip(o.layernorm_bwd_f32(f["dy"], f["x"], mean, rstd, w),
                       o.layernorm_bwd(bits["dy"], bits["x"], mean, rstd, wb),
                       ("dx", "dweight", "dbias")):
        same(a, c, f"layernorm bwd {n}")
    for dres32, dres16 in ((None, None), (f["dres"], bits["dres"])):
        for a, c, n in zip(o.rmsnorm_bwd_f32(f["dy"], f["x"], w, eps, dres=dres32),
                           o.rmsnorm_bwd(bits["dy"], bits["x"], wb, eps, dres=dres16),
                           ("dx", "dweight", "rstd")):
            same(a, c, f"rmsnorm bwd {n} (dres {dres32 is not None})")


def check_f32_library(o):
    rng = np.random.default_rng(23)
    rows, hidden = 5, 777
    x, r = _f32(rng, (rows, hidden), 0.3, 1.5), _f32(rng, (rows, hidden))
    w, b = _f32(rng, (hidden,), 1.0, 0.1), _f32(rng, (hidden,), 0.0, 0.1)
    dy, dres = _f32(rng, (rows, hidden)), _f32(rng, (rows, hidden))
    eps = float(np.float32(1e-5))
    t = {k: torch.from_numpy(v).double() for k, v in
         dict(x=x, r=r, w=w, b=b, dy=dy, dres=dres).items()}
    out, res, _ = o.fused_add_rmsnorm_f32(x, r, w, eps)
    s = torch.from_numpy(x.astype(np.float64) + r.astype(np.float64))
    close(out, F.rms_norm(s, (hidden,), t["w"], eps).numpy(), 1e-12, 1e-300, "fused f32")
    close(o.rmsnorm_fwd_f32(x, w, eps)[0], F.rms_norm(t["x"], (hidden,), t["w"], eps).numpy(),
          1e-12, 1e-300, "rmsnorm f32")
    y, mean, rstd = o.layernorm_fwd_f32(x, w, b, eps)
    close(y, F.layer_norm(t["x"], (hidden,), t["w"], t["b"], eps).numpy(), 1e-12, 1e-12,
          "layernorm f32")
    var, mu = torch.var_mean(t["x"], -1, unbiased=False)
    close(mean, mu.numpy(), 1e-12, 1e-15, "layernorm mean f32")
    close(rstd, torch.rsqrt(var + eps).numpy(), 1e-12, 0, "layernorm rstd f32")
    # LayerNorm backward: the given statistics are the exact ones, so autograd
    # (statistics recomputed from x) must agree
    xa = t["x"].clone().requires_grad_(True)
    wa = t["w"].clone().requires_grad_(True)
    ba = t["b"].clone().requires_grad_(True)
    F.layer_norm(xa, (hidden,), wa, ba, eps).backward(t["dy"])
    dx, dw, db = o.layernorm_bwd_f32(dy, x, mean, rstd, w)
    close(dx, xa.grad.numpy(), 1e-10, 1e-12, "layernorm bwd dx f32")
    close(dw, wa.grad.numpy(), 1e-10, 1e-12, "layernorm bwd dweight f32")
    close(db, ba.grad.numpy(), 1e-10, 1e-12, "layernorm bwd dbias f32")
    for with_dres in (False, True):
        xa = t["x"].clone().requires_grad_(True)
        wa = t["w"].clone().requires_grad_(True)
        F.rms_norm(xa, (hidden,), wa, eps).backward(t["dy"])
        dx, dw, _ = o.rmsnorm_bwd_f32(dy, x, w, eps, dres=dres if with_dres else None)
        ref = xa.grad.numpy() + (dres.astype(np.float64) if with_dres else 0.0)
        close(dx, ref, 1e-10, 1e-12, f"rmsnorm bwd dx f32 (dres {with_dres})")
        close(dw, wa.grad.numpy(), 1e-10, 1e-12, "rmsnorm bwd dweight f32")


def check_f32_closed_forms(o):
    hidden = 96
    w = np.linspace(0.5, 1.5, hidden).astype(np.float32)
    b = np.linspace(-0.2, 0.3, hidden).astype(np.float32)
    eps = float(np.float32(1e-6))
    for c in (np.float32(0.75), np.float32(-3.0)):
        x = np.full((2, hidden), c, np.float32)
        out, _ = o.rmsnorm_fwd_f32(x, w, eps)
        cd = float(c)
        close(out, np.broadcast_to(cd / np.sqrt(cd * cd + eps) * w.astype(np.float64),
                                   out.shape), 1e-15, 0, "rmsnorm f32 constant row")
        y, mean, _ = o.layernorm_fwd_f32(x, w, b, eps)
        assert np.array_equal(y, np.broadcast_to(b.astype(np.float64), y.shape)), \
            "layernorm f32 constant row must give the bias"
        assert (mean == cd).all()
    x = _f32(np.random.default_rng(24), (3, hidden))
    _, mean, rstd = o.layernorm_fwd_f32(x, w, b, eps)
    dx, dw, db = o.layernorm_bwd_f32(np.zeros_like(x), x, mean, rstd, w)
    assert not dx.any() and not dw.any() and not db.any(), "dy = 0 must give zero gradients"


F32_CHECKS = [
    check_f32_residual,
    check_f32_matches_bf16_oracle,
    check_f32_library,
    check_f32_closed_forms,
]
