"""Comparison rules between the HIP path and the oracle.

* bf16 residual of the fused op: bit-exact (exactly one correct rounding of
  x + r exists, and the oracle's exact sum rounded once equals the kernel's
  fp32 sum rounded once for every finite input).
* bf16 normalized outputs: |gpu - ref| <= 2 ulp_bf16(ref), ref the unrounded
  fp64 oracle value; ulp_bf16(v) = 2^max(floor(log2|v|) - 7, -133).
  For the outputs formed by cancellation (LayerNorm y and dx, RMSNorm and
  fused residual-add + RMSNorm dx, where rstd * (g - xhat * c) subtracts two
  terms of the row's scale) a floor of 2^-16 * M is added, M the magnitude of
  the terms that cancel (fp32 sums over the row leave errors of order
  2^-24 * sum|terms|; 2^-16 is 256x that and is at most 1/256 bf16 ulp at
  scale M, so it only matters for outputs cancelled far below the row's
  scale).  Every element that passes only by the floor must be such an
  output: |ref| <= 2^-6 * M (there 2 ulp are at most 2^-13 * M, so the floor
  can add a real share of the budget); a floor-only pass at a larger |ref|
  fails, since the floor is not meant to cover it.
* fp32 statistics (LayerNorm mean, rstd): |gpu - ref| <= 1e-6 + 1e-5 |ref|.
* fp32 column sums (dweight, dbias): |gpu - ref| <= 1e-3 |ref| + 1e-3 sqrt(sum_i t_i^2),
  t the summed terms (dy * xhat or dy): relative 1e-3, with the column's RMS
  scale as the absolute floor for columns that cancel to near zero.
* fp32 activations (the `_f32` entry points), from the arithmetic: every
  output is a short formula over the row's fp32 sums, so its error is the
  sums' relative error times the magnitude M of the terms it combines, plus a
  few roundings.  The longest sequential fp32 sum one lane forms in a row
  reduction is n(H) = max(32, 4 ceil(H / 4096)) values: up to 32768 columns
  the launch shapes give a lane at most 8 16-byte accesses of a row (4 values
  each), a wider row is walked by 1024 lanes; the lanes then meet in a tree of
  at most 16 levels.  Bound:
  |gpu - ref| <= (n(H) + 64) 2^-24 M, 64 covering the tree, the output
  formula's roundings, the hardware rsqrt (1 ulp) and the rounding of
  x + r to fp32 (the oracle normalizes the exact sum).  M: |ref| for the
  pure products (fused and RMSNorm out), the cancellation scales below for
  LayerNorm y and the dx of every backward, mean_j |x| for the LayerNorm mean,
  rstd itself for rstd.  Column sums over rows: each of the P row walkers sums
  ceil(rows / P) terms in order, then the walkers meet in a fixed pairwise
  tree, and each term carries its row's statistic error:
  |gpu - ref| <= (ceil(rows / P) + n(H) + 64) 2^-24 sum_i |t_i|.
"""
from __future__ import annotations

import numpy as np
import torch

FLOOR = 2.0 ** -16
CANCELLED = 2.0 ** -6  # floor-only passes must have |ref| <= CANCELLED * M


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def ulp_bf16(ref: np.ndarray) -> np.ndarray:
    a = np.abs(ref)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(a > 0, e, -126.0)
    return np.exp2(np.maximum(e - 7.0, -133.0))


def assert_bits_equal(got: np.ndarray, exp: np.ndarray, what: str):
    got = np.asarray(got).view(np.uint16)
    exp = np.asarray(exp).view(np.uint16)
    assert got.shape == exp.shape, what
    bad = got != exp
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} bits differ; first at "
                             f"{tuple(idx)}: {hex(got[tuple(idx)])} vs {hex(exp[tuple(idx)])}")


def assert_bf16_close(got_bits: np.ndarray, ref: np.ndarray, what: str, ulps: float = 2.0,
                      floor_scale: np.ndarray | None = None) -> dict:
    got = bits_to_f64(got_bits)
    assert got.shape == ref.shape, what
    err = np.abs(got - ref)
    lim = ulps * ulp_bf16(ref)
    if floor_scale is not None:
        lim = lim + FLOOR * floor_scale
    bad = ~(err <= lim)  # NaN in got fails
    if bad.any():
        idx = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside {ulps} bf16 ulp; "
                             f"first at {idx}: got {got[idx]!r} ref {ref[idx]!r}")
    with np.errstate(invalid="ignore", divide="ignore"):
        e = err / ulp_bf16(ref)
    only_floor, ratio = 0, 0.0
    if floor_scale is not None:
        only = err > ulps * ulp_bf16(ref)
        only_floor = int(only.sum())
        if only_floor:
            m = np.broadcast_to(floor_scale, ref.shape)[only]
            r = np.abs(ref[only]) / m
            ratio = float(r.max())
            if ratio > CANCELLED:
                k = int(np.argmax(r))
                raise AssertionError(
                    f"{what}: an element passed only by the cancellation floor although its "
                    f"value is not cancelled: |ref| = {abs(ref[only][k])!r} is "
                    f"{r[k]:.3g} x its term scale M (limit {CANCELLED})")
    return {"max_err_ulp": float(np.nanmax(e)), "passed_only_by_floor": only_floor,
            "elements": int(ref.size), "floor_max_ref_over_m": ratio}


def report_floor(what: str, stats: dict) -> None:
    """One line per checked output with the floor's use (shown with -s)."""
    print(f"FLOOR {what}: {stats['passed_only_by_floor']} of {stats['elements']} elements "
          f"passed only by the cancellation floor (max |ref|/M among them "
          f"{stats['floor_max_ref_over_m']:.3g}); max error {stats['max_err_ulp']:.3f} bf16 ulp",
          flush=True)


def assert_f32_close(got: np.ndarray, ref: np.ndarray, what: str, rtol=1e-5, atol=1e-6):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    bad = ~(err <= atol + rtol * np.abs(ref))
    if bad.any():
        i = int(np.argwhere(bad.reshape(-1))[0][0])
        raise AssertionError(f"{what}: {int(bad.sum())} outside rtol {rtol} atol {atol}; "
                             f"first {i}: {got.reshape(-1)[i]!r} vs {ref.reshape(-1)[i]!r}")


def assert_colsum_close(got: np.ndarray, ref: np.ndarray, terms_sq_sum: np.ndarray, what: str,
                        rtol=1e-3):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    lim = rtol * np.abs(ref) + rtol * np.sqrt(terms_sq_sum)
    bad = ~(err <= lim)
    if bad.any():
        j = int(np.argwhere(bad)[0][0])
        raise AssertionError(f"{what}: {int(bad.sum())} columns outside tolerance; first {j}: "
                             f"{got[j]!r} vs {ref[j]!r} (limit {lim[j]!r})")


def layernorm_y_scale(xd, mean, rstd, wd, bd):
    """M for LayerNorm y: rstd * (|x - mu| + mean_j |x|) * |w| + |b|."""
    mabs = np.abs(xd).mean(axis=1, keepdims=True)
    return rstd[:, None] * (np.abs(xd - mean[:, None]) + mabs) * np.abs(wd) + np.abs(bd)


def layernorm_dx_scale(xd, dyd, wd, mean, rstd):
    """M for LayerNorm dx: q (|g| + |c1| + |xhat||c2| + mean|g| + |xhat| mean|g xhat|)."""
    xhat = (xd - mean[:, None]) * rstd[:, None]
    g = dyd * wd
    c1 = g.mean(axis=1, keepdims=True)
    gx = g * xhat
    c2 = gx.mean(axis=1, keepdims=True)
    return rstd[:, None] * (np.abs(g) + np.abs(c1) + np.abs(xhat) * np.abs(c2)
                            + np.abs(g).mean(axis=1, keepdims=True)
                            + np.abs(xhat) * np.abs(gx).mean(axis=1, keepdims=True))


def rmsnorm_dx_scale(xd, dyd, wd, rstd, dresd=None):
    """M for RMSNorm dx: rstd (|g| + |xhat||c| + |xhat| mean|g xhat|) [+ |dres|]."""
    xhat = xd * rstd[:, None]
    g = dyd * wd
    gx = g * xhat
    c = gx.mean(axis=1, keepdims=True)
    m = rstd[:, None] * (np.abs(g) + np.abs(xhat) * np.abs(c)
                         + np.abs(xhat) * np.abs(gx).mean(axis=1, keepdims=True))
    if dresd is not None:
        m = m + np.abs(dresd)
    return m


U32 = 2.0 ** -24


def f32_seq(hidden: int) -> int:
    """n(H): the longest sequential fp32 sum one lane of a row reduction forms."""
    return max(32, 4 * -(-hidden // 4096))


def assert_f32_scaled(got, ref, scale, hidden: int, what: str) -> float:
    """|gpu - ref| <= (n(H) + 64) 2^-24 M; returns the largest err / (2^-24 M)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, what
    m = np.broadcast_to(np.asarray(scale, np.float64), ref.shape)
    err = np.abs(got - ref)
    lim = (f32_seq(hidden) + 64) * U32 * m
    bad = ~(err <= lim)
    if bad.any():
        idx = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside (n(H) + 64) "
                             f"2^-24 M; first at {idx}: got {got[idx]!r} ref {ref[idx]!r} "
                             f"(M {m[idx]!r})")
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.where(m > 0, err / (U32 * m), 0.0)
    return float(r.max()) if r.size else 0.0


def assert_colsum_f32(got, ref, terms_abs_sum, rows: int, walkers: int, hidden: int,
                      what: str) -> None:
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    lim = (-(-rows // walkers) + f32_seq(hidden) + 64) * U32 * np.asarray(terms_abs_sum)
    bad = ~(err <= lim)
    if bad.any():
        j = int(np.argwhere(bad)[0][0])
        raise AssertionError(f"{what}: {int(bad.sum())} columns outside tolerance; first {j}: "
                             f"{got[j]!r} vs {ref[j]!r} (limit {lim[j]!r})")

