"""Parity on both sides of every switch in the library's own launch choice.

For each forward operation and hidden size (compiled and run-time), the row
counts where the chosen kernel changes (another launch shape, the
late-weights variant, the persistent ring or another ring depth) are found
from the library's description of its choice on this device, and the rows
just below and at each switch run through the library's choice against the
oracle.  Switches past 17 M elements are left to the large-matrix and random
tests."""
import pytest

import row_normalization_persistent_amd as rn
from row_normalization_persistent_amd import workloads as wl

import test_gpu_parity as TP

pytestmark = pytest.mark.gpu

MAX_ELEMS = 17 << 20
MAX_ROWS = 16384


def _kernel(op, rows, hidden):
    d = rn.describe_config(op, rows, hidden)  # this device's compute-unit count
    return d.split(": ", 1)[1].split(" (")[0]


def switch_rows(op, hidden):
    """Row counts r where the kernel for r differs from the kernel for r - 1."""
    out, prev = [], _kernel(op, 1, hidden)
    for r in range(2, min(MAX_ROWS, MAX_ELEMS // hidden) + 1):
        k = _kernel(op, r, hidden)
        if k != prev:
            out.append(r)
        prev = k
    return out


CHECK = {
    "fused_add_rmsnorm": lambda r, h, s, what: TP.check_fused(wl.fused_inputs(r, h, seed=s),
                                                              what=what),
    "rmsnorm_fwd": lambda r, h, s, what: TP.check_rms(wl.rmsnorm_inputs(r, h, seed=s), what=what),
    "layernorm_fwd": lambda r, h, s, what: TP.check_lnf(wl.layernorm_fwd_inputs(r, h, seed=s),
                                                        what=what),
}


# compiled hidden sizes, then run-time ones (not multiples of 64: 1000, 3080; wide: 5120, 7168)
HIDDEN = tuple(rn.HIDDEN_SIZES) + (1000, 3080, 5120, 7168)


@pytest.mark.parametrize("hidden", HIDDEN)
@pytest.mark.parametrize("op", sorted(CHECK))
def test_both_sides_of_every_switch(op, hidden):
    switches = switch_rows(op, hidden)
    assert switches, (op, hidden)  # every operation changes shape somewhere below 17 M elements
    for r in switches:
        for rows in (r - 1, r):
            what = f"{op} {rows}x{hidden}: {_kernel(op, rows, hidden)}"
            print(what, flush=True)
            CHECK[op](rows, hidden, rows * 7 + hidden, what)
