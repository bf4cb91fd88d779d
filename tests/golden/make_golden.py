"""Write tests/golden/oracle_regression.json: small oracle outputs kept as a
regression fixture, so a later edit of the oracle that changes any result (even
by one rounding) is noticed.  Calls only the oracle and the seeded input
generators; run from the repository root:  python tests/golden/make_golden.py

The pages print no worked example, so this fixture pins the oracle against its
own earlier, pinned state; the pins against mathematics and library routines
live in tests/oracle_checks.py."""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from row_normalization_persistent_amd import workloads as wl  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.json")


def hexes(a):
    return [float(v).hex() for v in np.asarray(a, np.float64).reshape(-1)]


def bits(a):
    return [int(v) for v in np.asarray(a).reshape(-1)]


def main():
    cases = {}
    f = wl.fused_inputs(rows=3, hidden=16, seed=0)
    out, res, rstd = oracle.fused_add_rmsnorm(f["x"], f["r"], f["w"], f["eps"])
    cases["fused_add_rmsnorm"] = {"rows": 3, "hidden": 16, "eps": f["eps"],
                                  "x": bits(f["x"]), "r": bits(f["r"]), "w": bits(f["w"]),
                                  "out": hexes(out), "residual": bits(res), "rstd": hexes(rstd)}
    g = wl.rmsnorm_inputs(rows=2, hidden=200, seed=0)
    out, rstd = oracle.rmsnorm_fwd(g["x"], g["w"], g["eps"])
    cases["rmsnorm_fwd"] = {"rows": 2, "hidden": 200, "eps": g["eps"], "x": bits(g["x"]),
                            "w": bits(g["w"]), "out": hexes(out), "rstd": hexes(rstd)}
    h = wl.layernorm_fwd_inputs(rows=2, hidden=24, seed=0)
    y, mean, rstd = oracle.layernorm_fwd(h["x"], h["w"], h["b"], h["eps"])
    cases["layernorm_fwd"] = {"rows": 2, "hidden": 24, "eps": h["eps"], "x": bits(h["x"]),
                              "w": bits(h["w"]), "b": bits(h["b"]), "y": hexes(y),
                              "mean": hexes(mean), "rstd": hexes(rstd)}
    k = wl.layernorm_bwd_inputs(rows=3, hidden=16, seed=0)
    _, m, q = oracle.layernorm_fwd(k["x"], k["w"], np.zeros(16, np.uint16), k["eps"])
    m32, q32 = m.astype(np.float32), q.astype(np.float32)
    dx, dw, db = oracle.layernorm_bwd(k["dy"], k["x"], m32, q32, k["w"])
    cases["layernorm_bwd"] = {"rows": 3, "hidden": 16, "x": bits(k["x"]), "dy": bits(k["dy"]),
                              "w": bits(k["w"]), "mean": hexes(m32), "rstd": hexes(q32),
                              "dx": hexes(dx), "dweight": hexes(dw), "dbias": hexes(db)}
    with open(OUT, "w") as fh:
        json.dump(cases, fh, indent=0)
        fh.write("\n")


if __name__ == "__main__":
    main()
