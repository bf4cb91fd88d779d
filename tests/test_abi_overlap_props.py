"""Property tests of the C ABI's overlap checks (host only, no GPU): random
layouts of small strided matrices at fake addresses, checked against a
brute-force model of the bytes each argument covers.

* Safety: a call the library accepts never has two arguments sharing a byte,
  except the exact aliases the header allows (out == x, dx == dy).
* No false rejection: arguments whose address ranges are disjoint are always
  accepted.

On a host without a GPU an accepted call stops at its first HIP call (the
device query: NORM_ERROR_DEVICE, or the launch: NORM_ERROR_LAUNCH); a
rejected one returns NORM_ERROR_INVALID_VALUE before any HIP call.  No memory
is touched at the fake addresses.  With a GPU present an accepted call would
launch a kernel on them, so the module runs only where there is none."""
import pytest
import torch
from hypothesis import given, settings, strategies as st

import row_normalization_persistent_amd as rn

pytestmark = pytest.mark.skipif(
    torch.cuda.device_count() > 0,
    reason="accepted calls would launch kernels at fake addresses on a GPU")

INVALID, LAUNCH, DEVICE = 1, 5, 6
ACCEPTED = (LAUNCH, DEVICE)
BASE = 1 << 36  # fake, 4 KiB aligned


def matrix_bytes(off, rows, ld, cols, elem):
    """The set of byte addresses of a [rows, cols] matrix with row stride ld
    (elements) at byte offset off from BASE."""
    out = set()
    for i in range(rows):
        start = off + i * ld * elem
        out.update(range(start, start + cols * elem))
    return out


def extent(off, rows, ld, cols, elem):
    return off, off + ((rows - 1) * ld + cols) * elem


def disjoint(a, b):
    return a[1] <= b[0] or b[1] <= a[0]


@st.composite
def fused_layout(draw):
    hidden = draw(st.integers(1, 24))
    rows = draw(st.integers(1, 5))
    lds = [draw(st.integers(hidden, hidden + 24)) for _ in range(3)]
    offs = [2 * draw(st.integers(0, 600)) for _ in range(4)]  # out, residual, x, weight
    if draw(st.booleans()):  # the allowed exact alias out == x
        offs[0], lds[0] = offs[2], lds[2]
    return hidden, rows, lds, offs


@settings(max_examples=400, deadline=None)
@given(fused_layout())
def test_fused_forward_overlap_rules(layout):
    hidden, rows, (ld_o, ld_r, ld_x), (o_off, r_off, x_off, w_off) = layout
    L = rn.lib()
    st_ = L.norm_fused_add_rmsnorm_ex(BASE + o_off, ld_o, BASE + r_off, ld_r, BASE + x_off, ld_x,
                                      BASE + w_off, rows, hidden, 1e-6, None, None)
    assert st_ == INVALID or st_ in ACCEPTED, rn.status_string(st_)
    regions = {"out": (o_off, rows, ld_o, hidden), "res": (r_off, rows, ld_r, hidden),
               "x": (x_off, rows, ld_x, hidden), "w": (w_off, 1, hidden, hidden)}
    pairs = [("out", "x"), ("out", "w"), ("out", "res"), ("res", "x"), ("res", "w")]
    exact_alias = o_off == x_off and ld_o == ld_x
    if st_ in ACCEPTED:  # accepted: no pair shares a byte (out == x exactly aside)
        for a, b in pairs:
            if (a, b) == ("out", "x") and exact_alias:
                continue
            shared = matrix_bytes(*regions[a], 2) & matrix_bytes(*regions[b], 2)
            assert not shared, f"accepted with {a} and {b} sharing bytes: {layout}"
    if all(disjoint(extent(*regions[a], 2), extent(*regions[b], 2)) or
           ((a, b) == ("out", "x") and exact_alias) for a, b in pairs):
        assert st_ in ACCEPTED, f"rejected a layout with disjoint address ranges: {layout}"


@st.composite
def lnbwd_layout(draw):
    hidden = draw(st.integers(1, 24))
    rows = draw(st.integers(1, 5))
    lds = [draw(st.integers(hidden, hidden + 24)) for _ in range(3)]  # dx, dy, x
    # dx, dy, x (bf16); mean, rstd, dweight, dbias (fp32); weight (bf16); workspace
    offs = [2 * draw(st.integers(0, 500)) for _ in range(3)]
    offs += [4 * draw(st.integers(0, 250)) for _ in range(2)]
    offs += [2 * draw(st.integers(0, 500))]
    offs += [4 * draw(st.integers(0, 250)) for _ in range(2)]
    offs += [16 * draw(st.integers(0, 80))]
    if draw(st.booleans()):  # the allowed exact alias dx == dy
        offs[0], lds[0] = offs[1], lds[1]
    return hidden, rows, lds, offs


@settings(max_examples=400, deadline=None)
@given(lnbwd_layout())
def test_layernorm_backward_overlap_rules(layout):
    hidden, rows, (ld_dx, ld_dy, ld_x), offs = layout
    dx, dy, x, mean, rstd, w, dw, db, ws = offs
    L = rn.lib()
    ws_bytes = L.norm_layernorm_bwd_workspace_bytes(rows, hidden)
    st_ = L.norm_layernorm_bwd_ex(BASE + dx, ld_dx, BASE + dw, BASE + db, BASE + dy, ld_dy,
                                  BASE + x, ld_x, BASE + mean, BASE + rstd, BASE + w,
                                  BASE + ws, ws_bytes, rows, hidden, 1e-5, None, None)
    assert st_ == INVALID or st_ in ACCEPTED, rn.status_string(st_)
    regions = {"dx": ((dx, rows, ld_dx, hidden), 2), "dy": ((dy, rows, ld_dy, hidden), 2),
               "x": ((x, rows, ld_x, hidden), 2), "mean": ((mean, 1, rows, rows), 4),
               "rstd": ((rstd, 1, rows, rows), 4), "w": ((w, 1, hidden, hidden), 2),
               "dw": ((dw, 1, hidden, hidden), 4), "db": ((db, 1, hidden, hidden), 4),
               "ws": ((ws, 1, ws_bytes, ws_bytes), 1)}
    outputs = ("dx", "dw", "db", "ws")
    inputs = ("dy", "x", "mean", "rstd", "w")
    pairs = [(o, i) for o in outputs for i in inputs] + \
            [(a, b) for k, a in enumerate(outputs) for b in outputs[k + 1:]]
    exact_alias = dx == dy and ld_dx == ld_dy

    def allowed(a, b):
        return {a, b} == {"dx", "dy"} and exact_alias

    def bytes_of(name):
        (off, r, ld, cols), elem = regions[name]
        return matrix_bytes(off, r, ld, cols, elem)

    def ext(name):
        (off, r, ld, cols), elem = regions[name]
        return extent(off, r, ld, cols, elem)

    if st_ in ACCEPTED:
        for a, b in pairs:
            if not allowed(a, b):
                assert not (bytes_of(a) & bytes_of(b)), \
                    f"accepted with {a} and {b} sharing bytes: {layout}"
    if all(disjoint(ext(a), ext(b)) or allowed(a, b) for a, b in pairs):
        assert st_ in ACCEPTED, f"rejected a layout with disjoint address ranges: {layout}"


@settings(max_examples=300, deadline=None)
@given(st.integers(1, 6), st.sampled_from([4, 8, 12, 16, 20]),
       st.lists(st.integers(0, 200), min_size=4, max_size=4), st.booleans())
def test_f32_fused_forward_overlap_rules(rows, hidden, offs16, alias):
    """The fp32 entry points: 16-byte-aligned fake pointers, the same rules."""
    o, r, x, w = (16 * v for v in offs16)
    if alias:
        o = x
    L = rn.lib()
    st_ = L.norm_fused_add_rmsnorm_f32(BASE + o, BASE + r, BASE + x, BASE + w, rows, hidden,
                                       1e-6, None)
    assert st_ == INVALID or st_ in ACCEPTED, rn.status_string(st_)
    regions = {"out": (o, rows, hidden, hidden), "res": (r, rows, hidden, hidden),
               "x": (x, rows, hidden, hidden), "w": (w, 1, hidden, hidden)}
    pairs = [("out", "x"), ("out", "w"), ("out", "res"), ("res", "x"), ("res", "w")]
    if st_ in ACCEPTED:
        for a, b in pairs:
            if (a, b) == ("out", "x") and o == x:
                continue
            assert not (matrix_bytes(*regions[a], 4) & matrix_bytes(*regions[b], 4)), (a, b)
    if all(disjoint(extent(*regions[a], 4), extent(*regions[b], 4)) or
           ((a, b) == ("out", "x") and o == x) for a, b in pairs):
        assert st_ in ACCEPTED
