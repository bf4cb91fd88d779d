"""Seeded synthetic workloads shaped like LLM hidden-state activations.

This module only draws random numbers and rounds them to bf16 with torch's own
fp32 -> bf16 conversion (round-to-nearest-even); it holds none of the
normalization arithmetic.  The same generators feed the HIP path, the oracle,
the tests and the benchmark.

Recipe (one ``numpy.random.default_rng(seed)`` per workload point, fp32 draws in
a fixed order, then bf16 rounding):

* fused residual-add + RMSNorm: x, r ~ N(0, 1); w ~ N(1, 0.1); eps = fp32(1e-6)
* RMSNorm: x ~ N(0, 1) with round(0.01 * hidden) outlier *columns* (chosen by a
  seeded permutation) multiplied by 50 in every row; w ~ N(1, 0.1); eps = fp32(1e-6)
* LayerNorm forward: x ~ N(0.5, 2); w ~ N(1, 0.1); b ~ N(0, 0.1); eps = fp32(1e-5)
* LayerNorm backward: x, dy ~ N(0, 1); w ~ N(1, 0.1); the per-row mean/rstd are
  computed by the caller from x with eps = fp32(1e-5)
* RMSNorm backward (and the fused residual-add + RMSNorm backward): x, dy ~ N(0, 1);
  w ~ N(1, 0.1); dres ~ N(0, 1) (gradient of the fused op's residual output);
  eps = fp32(1e-6)

``N(m, s)`` means mean m and standard deviation s.  With ``f32=True`` a
generator returns the same fp32 draws without the bf16 rounding (the inputs of
the fp32-activation entry points).
"""
from __future__ import annotations

import numpy as np
import torch

EPS_RMS = float(np.float32(1e-6))
EPS_LN = float(np.float32(1e-5))

FUSED_HIDDEN = 4096
FUSED_SWEEP_ROWS = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192)
FUSED_SMALL_ROWS = 16
RMSNORM_HIDDEN = (2048, 8192, 16384)
RMSNORM_ROWS = (1, 64, 1024, 4096)
LAYERNORM_FWD_HIDDEN = (1024, 4096, 12288, 16384)
LAYERNORM_FWD_ROWS = 2048
LAYERNORM_BWD_HIDDEN = (4096, 8192)
LAYERNORM_BWD_ROWS = 8192
RMSNORM_BWD_HIDDEN = (4096, 8192)
RMSNORM_BWD_ROWS = 8192


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), rounded by torch (RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _keep_f32(a: np.ndarray) -> np.ndarray:
    """The fp32 draws themselves (the generators' ``f32=True``)."""
    return np.ascontiguousarray(a, dtype=np.float32).copy()


def _normal(rng: np.random.Generator, shape, mean: float, std: float) -> np.ndarray:
    z = rng.standard_normal(shape, dtype=np.float32)
    return z * np.float32(std) + np.float32(mean)


def fused_inputs(rows: int, hidden: int = FUSED_HIDDEN, seed: int = 0, f32: bool = False) -> dict:
    q = _keep_f32 if f32 else bf16_bits
    rng = np.random.default_rng(seed)
    x = _normal(rng, (rows, hidden), 0.0, 1.0)
    r = _normal(rng, (rows, hidden), 0.0, 1.0)
    w = _normal(rng, (hidden,), 1.0, 0.1)
    return {"x": q(x), "r": q(r), "w": q(w), "eps": EPS_RMS}


def outlier_columns(hidden: int, seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng(seed + 0x5EED)
    k = int(round(0.01 * hidden))
    return np.sort(rng.permutation(hidden)[:k])


def rmsnorm_inputs(rows: int, hidden: int, seed: int = 0, f32: bool = False) -> dict:
    q = _keep_f32 if f32 else bf16_bits
    rng = np.random.default_rng(seed)
    x = _normal(rng, (rows, hidden), 0.0, 1.0)
    cols = outlier_columns(hidden, seed)
    x[:, cols] *= np.float32(50.0)
    w = _normal(rng, (hidden,), 1.0, 0.1)
    return {"x": q(x), "w": q(w), "eps": EPS_RMS, "outlier_cols": cols}


def layernorm_fwd_inputs(rows: int, hidden: int, seed: int = 0, f32: bool = False) -> dict:
    q = _keep_f32 if f32 else bf16_bits
    rng = np.random.default_rng(seed)
    x = _normal(rng, (rows, hidden), 0.5, 2.0)
    w = _normal(rng, (hidden,), 1.0, 0.1)
    b = _normal(rng, (hidden,), 0.0, 0.1)
    return {"x": q(x), "w": q(w), "b": q(b), "eps": EPS_LN}


def layernorm_bwd_inputs(rows: int, hidden: int, seed: int = 0, f32: bool = False) -> dict:
    q = _keep_f32 if f32 else bf16_bits
    rng = np.random.default_rng(seed)
    x = _normal(rng, (rows, hidden), 0.0, 1.0)
    dy = _normal(rng, (rows, hidden), 0.0, 1.0)
    w = _normal(rng, (hidden,), 1.0, 0.1)
    return {"x": q(x), "dy": q(dy), "w": q(w), "eps": EPS_LN}


def rmsnorm_bwd_inputs(rows: int, hidden: int, seed: int = 0, f32: bool = False) -> dict:
    q = _keep_f32 if f32 else bf16_bits
    rng = np.random.default_rng(seed)
    x = _normal(rng, (rows, hidden), 0.0, 1.0)
    dy = _normal(rng, (rows, hidden), 0.0, 1.0)
    w = _normal(rng, (hidden,), 1.0, 0.1)
    dres = _normal(rng, (rows, hidden), 0.0, 1.0)
    return {"x": q(x), "dy": q(dy), "w": q(w), "dres": q(dres),
            "eps": EPS_RMS}


def device_normal_bf16(rows: int, hidden: int, mean: float, std: float, seed: int,
                       device="cuda", ld: int | None = None) -> torch.Tensor:
    """A [rows, hidden] bf16 matrix ~ N(mean, std) drawn on the device from a
    seeded torch generator, for matrices too large to draw on the host: fp32
    draws in chunks of rows, rounded to bf16 by torch.  With ``ld`` > hidden the
    matrix is the first ``hidden`` columns of a [rows, ld] allocation whose
    other columns hold draws of the same distribution."""
    cols = hidden if ld is None else ld
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    full = torch.empty((rows, cols), dtype=torch.bfloat16, device=device)
    chunk = max(1, (1 << 26) // cols)
    for a in range(0, rows, chunk):
        b = min(rows, a + chunk)
        z = torch.randn((b - a, cols), generator=g, device=device, dtype=torch.float32)
        full[a:b] = (z * std + mean).to(torch.bfloat16)
    return full if ld is None else full[:, :hidden]


def device_normal_f32(n: int, mean: float, std: float, seed: int, device="cuda") -> torch.Tensor:
    """n fp32 values ~ N(mean, std) drawn on the device from a seeded torch generator."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(n, generator=g, device=device, dtype=torch.float32) * std + mean


def to_device_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """bf16 bit patterns (uint16) -> torch.bfloat16 tensor on `device`."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def from_device_bf16(t: torch.Tensor) -> np.ndarray:
    """torch.bfloat16 tensor -> bf16 bit patterns (uint16) on the host."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
