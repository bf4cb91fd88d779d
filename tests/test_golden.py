"""The oracle reproduces its stored regression fixture bit for bit (CPU only).
The fixture is written by tests/golden/make_golden.py, which calls only the
oracle."""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "oracle_regression.json")


def _u16(v, shape):
    return np.array(v, np.uint16).reshape(shape)


def _f64(v, shape=None):
    a = np.array([float.fromhex(s) for s in v], np.float64)
    return a.reshape(shape) if shape else a


def test_oracle_matches_regression_fixture():
    g = json.load(open(GOLDEN))
    c = g["fused_add_rmsnorm"]
    sh = (c["rows"], c["hidden"])
    out, res, rstd = oracle.fused_add_rmsnorm(_u16(c["x"], sh), _u16(c["r"], sh),
                                              _u16(c["w"], sh[1]), c["eps"])
    assert np.array_equal(out, _f64(c["out"], sh))
    assert np.array_equal(res, _u16(c["residual"], sh))
    assert np.array_equal(rstd, _f64(c["rstd"]))
    c = g["rmsnorm_fwd"]
    sh = (c["rows"], c["hidden"])
    out, rstd = oracle.rmsnorm_fwd(_u16(c["x"], sh), _u16(c["w"], sh[1]), c["eps"])
    assert np.array_equal(out, _f64(c["out"], sh))
    assert np.array_equal(rstd, _f64(c["rstd"]))
    c = g["layernorm_fwd"]
    sh = (c["rows"], c["hidden"])
    y, mean, rstd = oracle.layernorm_fwd(_u16(c["x"], sh), _u16(c["w"], sh[1]),
                                         _u16(c["b"], sh[1]), c["eps"])
    assert np.array_equal(y, _f64(c["y"], sh))
    assert np.array_equal(mean, _f64(c["mean"]))
    assert np.array_equal(rstd, _f64(c["rstd"]))
    c = g["layernorm_bwd"]
    sh = (c["rows"], c["hidden"])
    dx, dw, db = oracle.layernorm_bwd(_u16(c["dy"], sh), _u16(c["x"], sh), _f64(c["mean"]),
                                      _f64(c["rstd"]), _u16(c["w"], sh[1]))
    assert np.array_equal(dx, _f64(c["dx"], sh))
    assert np.array_equal(dw, _f64(c["dweight"]))
    assert np.array_equal(db, _f64(c["dbias"]))
