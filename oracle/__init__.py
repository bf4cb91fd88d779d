"""CPU oracle for inner-persistent row normalization -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never imports it and
shares no code with it.

The arithmetic lives in ``oracle.c`` (plain fp64 loops over bf16 operands, built
with gcc -O2 and no fast-math) and ``oracle_f32.c`` (the same definitions over
binary32 operands, for the fp32-activation entry points); this module only
marshals numpy arrays into them.  Definitions:

* fused residual-add + RMSNorm forward -- "optimize inner persistent scheduler
  for static fusion" (nvFuser PR 5281), author description and changes
  walkthrough (in-place residual update); formula: RMSNorm, Zhang & Sennrich
  (2019) eq. 4, applied to ``x + r``;
* RMSNorm / LayerNorm forward -- "TMA inner persistent scheduler" (nvFuser
  PR 5587), description summary; LayerNorm per Ba, Kiros & Hinton (2016)
  eq. 4 with biased variance and eps inside the square root;
* LayerNorm backward as a combined inner + outer reduction -- "Llu/ln bwd"
  (nvFuser PR 207), author note and review thread;
* RMSNorm backward (and the fused residual-add + RMSNorm backward) -- the same
  combined inner + outer reduction applied to RMSNorm; the gradient of
  Zhang & Sennrich (2019) eq. 4 with the statistic recomputed from x.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SOURCES = [os.path.join(_HERE, "oracle.c"), os.path.join(_HERE, "oracle_f32.c")]
F32_SOURCE = _SOURCES[1]

def build(force: bool = True, sources=None, out_path: str | None = None,
          defines=()) -> str:
    """Compile the oracle with gcc (-O2, strict IEEE: no fast-math, no FMA
    contraction).  ``sources``/``out_path`` let a test build a modified copy."""
    out_path = out_path or LIB_PATH
    if not force and os.path.exists(out_path):
        return out_path
    tmp = out_path + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-pthread", "-Wall", "-Wextra", *[f"-D{d}" for d in defines],
           *(sources or _SOURCES), "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def _bind(lib):
    lib.orc_bf16_decode.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_decode.restype = ctypes.c_double
    lib.orc_bf16_encode.argtypes = [ctypes.c_double]
    lib.orc_bf16_encode.restype = ctypes.c_uint16
    lib.orc_bf16_decode_n.argtypes = [_u16p, _f64p, _i64]
    lib.orc_bf16_decode_n.restype = None
    lib.orc_bf16_encode_n.argtypes = [_f64p, _u16p, _i64]
    lib.orc_bf16_encode_n.restype = None
    lib.orc_fused_add_rmsnorm.argtypes = [_u16p, _u16p, _u16p, _i64, _i64, ctypes.c_double,
                                          _f64p, _u16p, _f64p, ctypes.c_int]
    lib.orc_rmsnorm_fwd.argtypes = [_u16p, _u16p, _i64, _i64, ctypes.c_double, _f64p, _f64p,
                                    ctypes.c_int]
    lib.orc_layernorm_fwd.argtypes = [_u16p, _u16p, _u16p, _i64, _i64, ctypes.c_double,
                                      _f64p, _f64p, _f64p, ctypes.c_int]
    lib.orc_layernorm_bwd.argtypes = [_u16p, _u16p, _f64p, _f64p, _u16p, _i64, _i64,
                                      _f64p, _f64p, _f64p, ctypes.c_int]
    lib.orc_rmsnorm_bwd.argtypes = [_u16p, _u16p, _u16p, _u16p, _i64, _i64, ctypes.c_double,
                                    _f64p, _f64p, _f64p, ctypes.c_int]
    for name in ("orc_fused_add_rmsnorm", "orc_rmsnorm_fwd", "orc_layernorm_fwd",
                 "orc_layernorm_bwd", "orc_rmsnorm_bwd"):
        getattr(lib, name).restype = ctypes.c_int
    if hasattr(lib, "orc_fused_add_rmsnorm_f32"):  # builds without oracle_f32.c lack them
        lib.orc_fused_add_rmsnorm_f32.argtypes = [_f32p, _f32p, _f32p, _i64, _i64,
                                                  ctypes.c_double, _f64p, _f32p, _f64p,
                                                  ctypes.c_int]
        lib.orc_rmsnorm_fwd_f32.argtypes = [_f32p, _f32p, _i64, _i64, ctypes.c_double, _f64p,
                                            _f64p, ctypes.c_int]
        lib.orc_layernorm_fwd_f32.argtypes = [_f32p, _f32p, _f32p, _i64, _i64, ctypes.c_double,
                                              _f64p, _f64p, _f64p, ctypes.c_int]
        lib.orc_layernorm_bwd_f32.argtypes = [_f32p, _f32p, _f64p, _f64p, _f32p, _i64, _i64,
                                              _f64p, _f64p, _f64p, ctypes.c_int]
        lib.orc_rmsnorm_bwd_f32.argtypes = [_f32p, _f32p, _f32p, _f32p, _i64, _i64,
                                            ctypes.c_double, _f64p, _f64p, _f64p, ctypes.c_int]
        for name in ("orc_fused_add_rmsnorm_f32", "orc_rmsnorm_fwd_f32",
                     "orc_layernorm_fwd_f32", "orc_layernorm_bwd_f32", "orc_rmsnorm_bwd_f32"):
            getattr(lib, name).restype = ctypes.c_int
    return lib


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected bf16 bit patterns as uint16, got {a.dtype}")
    return a


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _p16(a):
    return a.ctypes.data_as(_u16p)


def _p64(a):
    return a.ctypes.data_as(_f64p)


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.float32:
        raise TypeError(f"expected float32 values, got {a.dtype}")
    return a


def _p32(a):
    return a.ctypes.data_as(_f32p)


def _check(rc: int, name: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {name}: invalid arguments")


def _shape(x: np.ndarray):
    if x.ndim != 2:
        raise ValueError("expected a [rows, hidden] matrix")
    return x.shape


class Oracle:
    """numpy front end over one build of the oracle library."""

    def __init__(self, lib_path: str = LIB_PATH):
        if lib_path == LIB_PATH and not os.path.exists(lib_path):
            build()
        self.lib = _bind(ctypes.CDLL(lib_path))

    def bf16_decode(self, bits) -> np.ndarray:
        """bf16 bit patterns (uint16) -> exact float64 values."""
        b = _u16(bits)
        out = np.empty(b.shape, dtype=np.float64)
        self.lib.orc_bf16_decode_n(_p16(b), _p64(out), b.size)
        return out

    def bf16_encode(self, values) -> np.ndarray:
        """float64 values -> nearest bf16 bit patterns (ties to even)."""
        v = _f64(values)
        out = np.empty(v.shape, dtype=np.uint16)
        self.lib.orc_bf16_encode_n(_p64(v), _p16(out), v.size)
        return out

    def fused_add_rmsnorm(self, x, r, w, eps: float, nthreads: int = 1):
        """Returns (out_f64, residual_bf16_bits, rstd_f64)."""
        x, r, w = _u16(x), _u16(r), _u16(w)
        rows, hidden = _shape(x)
        assert r.shape == x.shape and w.shape == (hidden,)
        out = np.empty((rows, hidden), np.float64)
        res = np.empty((rows, hidden), np.uint16)
        rstd = np.empty((rows,), np.float64)
        _check(self.lib.orc_fused_add_rmsnorm(_p16(x), _p16(r), _p16(w), rows, hidden,
                                              float(eps), _p64(out), _p16(res), _p64(rstd),
                                              nthreads), "fused_add_rmsnorm")
        return out, res, rstd

    def rmsnorm_fwd(self, x, w, eps: float, nthreads: int = 1):
        """Returns (out_f64, rstd_f64)."""
        x, w = _u16(x), _u16(w)
        rows, hidden = _shape(x)
        assert w.shape == (hidden,)
        out = np.empty((rows, hidden), np.float64)
        rstd = np.empty((rows,), np.float64)
        _check(self.lib.orc_rmsnorm_fwd(_p16(x), _p16(w), rows, hidden, float(eps), _p64(out),
                                        _p64(rstd), nthreads), "rmsnorm_fwd")
        return out, rstd

    def layernorm_fwd(self, x, w, b, eps: float, nthreads: int = 1):
        """Returns (y_f64, mean_f64, rstd_f64)."""
        x, w, b = _u16(x), _u16(w), _u16(b)
        rows, hidden = _shape(x)
        assert w.shape == (hidden,) and b.shape == (hidden,)
        y = np.empty((rows, hidden), np.float64)
        mean = np.empty((rows,), np.float64)
        rstd = np.empty((rows,), np.float64)
        _check(self.lib.orc_layernorm_fwd(_p16(x), _p16(w), _p16(b), rows, hidden, float(eps),
                                          _p64(y), _p64(mean), _p64(rstd), nthreads),
               "layernorm_fwd")
        return y, mean, rstd

    def layernorm_bwd(self, dy, x, mean, rstd, w, nthreads: int = 1):
        """mean/rstd are the given per-row statistics (any float dtype, widened
        exactly to float64).  Returns (dx_f64, dweight_f64, dbias_f64)."""
        dy, x, w = _u16(dy), _u16(x), _u16(w)
        rows, hidden = _shape(x)
        assert dy.shape == x.shape and w.shape == (hidden,)
        mean = _f64(mean)
        rstd = _f64(rstd)
        assert mean.shape == (rows,) and rstd.shape == (rows,)
        dx = np.empty((rows, hidden), np.float64)
        dw = np.empty((hidden,), np.float64)
        db = np.empty((hidden,), np.float64)
        _check(self.lib.orc_layernorm_bwd(_p16(dy), _p16(x), _p64(mean), _p64(rstd), _p16(w),
                                          rows, hidden, _p64(dx), _p64(dw), _p64(db),
                                          nthreads), "layernorm_bwd")
        return dx, dw, db


    def rmsnorm_bwd(self, dy, x, w, eps: float, dres=None, nthreads: int = 1):
        """RMSNorm backward with rstd recomputed from x; dres (optional bf16
        bits) is added to dx (the fused residual-add + RMSNorm backward).
        Returns (dx_f64, dweight_f64, rstd_f64)."""
        dy, x, w = _u16(dy), _u16(x), _u16(w)
        rows, hidden = _shape(x)
        assert dy.shape == x.shape and w.shape == (hidden,)
        dres_p = None
        if dres is not None:
            dres = _u16(dres)
            assert dres.shape == x.shape
            dres_p = _p16(dres)
        dx = np.empty((rows, hidden), np.float64)
        dw = np.empty((hidden,), np.float64)
        rstd = np.empty((rows,), np.float64)
        _check(self.lib.orc_rmsnorm_bwd(_p16(dy), _p16(x), _p16(w), dres_p, rows, hidden,
                                        float(eps), _p64(dx), _p64(dw), _p64(rstd), nthreads),
               "rmsnorm_bwd")
        return dx, dw, rstd


    # ---- fp32 activations (oracle_f32.c) ------------------------------------
    def fused_add_rmsnorm_f32(self, x, r, w, eps: float, nthreads: int = 1):
        """float32 x, r, w.  Returns (out_f64, residual_f32, rstd_f64)."""
        x, r, w = _f32(x), _f32(r), _f32(w)
        rows, hidden = _shape(x)
        assert r.shape == x.shape and w.shape == (hidden,)
        out = np.empty((rows, hidden), np.float64)
        res = np.empty((rows, hidden), np.float32)
        rstd = np.empty((rows,), np.float64)
        _check(self.lib.orc_fused_add_rmsnorm_f32(_p32(x), _p32(r), _p32(w), rows, hidden,
                                                  float(eps), _p64(out), _p32(res), _p64(rstd),
                                                  nthreads), "fused_add_rmsnorm_f32")
        return out, res, rstd

    def rmsnorm_fwd_f32(self, x, w, eps: float, nthreads: int = 1):
        """Returns (out_f64, rstd_f64)."""
        x, w = _f32(x), _f32(w)
        rows, hidden = _shape(x)
        assert w.shape == (hidden,)
        out = np.empty((rows, hidden), np.float64)
        rstd = np.empty((rows,), np.float64)
        _check(self.lib.orc_rmsnorm_fwd_f32(_p32(x), _p32(w), rows, hidden, float(eps),
                                            _p64(out), _p64(rstd), nthreads), "rmsnorm_fwd_f32")
        return out, rstd

    def layernorm_fwd_f32(self, x, w, b, eps: float, nthreads: int = 1):
        """Returns (y_f64, mean_f64, rstd_f64)."""
        x, w, b = _f32(x), _f32(w), _f32(b)
        rows, hidden = _shape(x)
        assert w.shape == (hidden,) and b.shape == (hidden,)
        y = np.empty((rows, hidden), np.float64)
        mean = np.empty((rows,), np.float64)
        rstd = np.empty((rows,), np.float64)
        _check(self.lib.orc_layernorm_fwd_f32(_p32(x), _p32(w), _p32(b), rows, hidden,
                                              float(eps), _p64(y), _p64(mean), _p64(rstd),
                                              nthreads), "layernorm_fwd_f32")
        return y, mean, rstd

    def layernorm_bwd_f32(self, dy, x, mean, rstd, w, nthreads: int = 1):
        """mean/rstd: the given statistics, widened exactly to float64.
        Returns (dx_f64, dweight_f64, dbias_f64)."""
        dy, x, w = _f32(dy), _f32(x), _f32(w)
        rows, hidden = _shape(x)
        assert dy.shape == x.shape and w.shape == (hidden,)
        mean, rstd = _f64(mean), _f64(rstd)
        assert mean.shape == (rows,) and rstd.shape == (rows,)
        dx = np.empty((rows, hidden), np.float64)
        dw = np.empty((hidden,), np.float64)
        db = np.empty((hidden,), np.float64)
        _check(self.lib.orc_layernorm_bwd_f32(_p32(dy), _p32(x), _p64(mean), _p64(rstd), _p32(w),
                                              rows, hidden, _p64(dx), _p64(dw), _p64(db),
                                              nthreads), "layernorm_bwd_f32")
        return dx, dw, db

    def rmsnorm_bwd_f32(self, dy, x, w, eps: float, dres=None, nthreads: int = 1):
        """Returns (dx_f64, dweight_f64, rstd_f64); dres (float32) is added to dx."""
        dy, x, w = _f32(dy), _f32(x), _f32(w)
        rows, hidden = _shape(x)
        assert dy.shape == x.shape and w.shape == (hidden,)
        dres_p = None
        if dres is not None:
            dres = _f32(dres)
            assert dres.shape == x.shape
            dres_p = _p32(dres)
        dx = np.empty((rows, hidden), np.float64)
        dw = np.empty((hidden,), np.float64)
        rstd = np.empty((rows,), np.float64)
        _check(self.lib.orc_rmsnorm_bwd_f32(_p32(dy), _p32(x), _p32(w), dres_p, rows, hidden,
                                            float(eps), _p64(dx), _p64(dw), _p64(rstd), nthreads),
               "rmsnorm_bwd_f32")
        return dx, dw, rstd


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def bf16_decode(bits):
    return default().bf16_decode(bits)


def bf16_encode(values):
    return default().bf16_encode(values)


def fused_add_rmsnorm(x, r, w, eps, nthreads=1):
    return default().fused_add_rmsnorm(x, r, w, eps, nthreads)


def rmsnorm_fwd(x, w, eps, nthreads=1):
    return default().rmsnorm_fwd(x, w, eps, nthreads)


def layernorm_fwd(x, w, b, eps, nthreads=1):
    return default().layernorm_fwd(x, w, b, eps, nthreads)


def layernorm_bwd(dy, x, mean, rstd, w, nthreads=1):
    return default().layernorm_bwd(dy, x, mean, rstd, w, nthreads)


def rmsnorm_bwd(dy, x, w, eps, dres=None, nthreads=1):
    return default().rmsnorm_bwd(dy, x, w, eps, dres, nthreads)


def fused_add_rmsnorm_f32(x, r, w, eps, nthreads=1):
    return default().fused_add_rmsnorm_f32(x, r, w, eps, nthreads)


def rmsnorm_fwd_f32(x, w, eps, nthreads=1):
    return default().rmsnorm_fwd_f32(x, w, eps, nthreads)


def layernorm_fwd_f32(x, w, b, eps, nthreads=1):
    return default().layernorm_fwd_f32(x, w, b, eps, nthreads)


def layernorm_bwd_f32(dy, x, mean, rstd, w, nthreads=1):
    return default().layernorm_bwd_f32(dy, x, mean, rstd, w, nthreads)


def rmsnorm_bwd_f32(dy, x, w, eps, dres=None, nthreads=1):
    return default().rmsnorm_bwd_f32(dy, x, w, eps, dres, nthreads)
