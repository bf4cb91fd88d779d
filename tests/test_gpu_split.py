"""GPU parity of the row-split forward (one row over k workgroups that meet in
a workspace) against the CPU oracle: the library's own choices, explicit
chunk counts (a ragged last chunk, one chunk), constant rows, repeated calls
and HIP-graph replays on one workspace (which every call must leave zero),
and the errors that need the device's CU count.  Rules in parity.py."""
import os

import numpy as np
import pytest
import torch

import oracle
import parity as P
import row_normalization_persistent_amd as rn
from row_normalization_persistent_amd import workloads as wl

pytestmark = pytest.mark.gpu

NT = min(16, os.cpu_count() or 1)
DEV = "cuda"
OPS = ["fused_add_rmsnorm", "rmsnorm_fwd", "layernorm_fwd"]


def dev(bits):
    return wl.to_device_bf16(bits, DEV)


def host(t):
    torch.cuda.synchronize()
    return wl.from_device_bf16(t)


def inputs(op, rows, h, seed):
    if op == "fused_add_rmsnorm":
        return wl.fused_inputs(rows, h, seed)
    if op == "rmsnorm_fwd":
        return wl.rmsnorm_inputs(rows, h, seed)
    return wl.layernorm_fwd_inputs(rows, h, seed)


def workspace(rows):
    return torch.zeros(rn.split_workspace_bytes(rows), dtype=torch.uint8, device=DEV)


def run(op, inp, ws, split):
    """The op through the row-split entry point; host bits of its outputs."""
    if op == "fused_add_rmsnorm":
        out, res = rn.fused_add_rmsnorm(dev(inp["x"]), dev(inp["r"]), dev(inp["w"]), inp["eps"],
                                        workspace=ws, split=split)
        return {"out": host(out), "res": host(res)}
    if op == "rmsnorm_fwd":
        return {"out": host(rn.rmsnorm_fwd(dev(inp["x"]), dev(inp["w"]), inp["eps"],
                                           workspace=ws, split=split))}
    y, mean, rstd = rn.layernorm_fwd(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]), inp["eps"],
                                     workspace=ws, split=split)
    return {"out": host(y), "mean": mean.cpu().numpy(), "rstd": rstd.cpu().numpy()}


def check(op, inp, got, what):
    if op == "fused_add_rmsnorm":
        ref, res_ref, _ = oracle.fused_add_rmsnorm(inp["x"], inp["r"], inp["w"], inp["eps"], NT)
        P.assert_bits_equal(got["res"], res_ref, f"{what}: residual")
        P.assert_bf16_close(got["out"], ref, f"{what}: out")
    elif op == "rmsnorm_fwd":
        ref, _ = oracle.rmsnorm_fwd(inp["x"], inp["w"], inp["eps"], NT)
        P.assert_bf16_close(got["out"], ref, what)
    else:
        ref, mean_ref, rstd_ref = oracle.layernorm_fwd(inp["x"], inp["w"], inp["b"], inp["eps"],
                                                       NT)
        xd, wd, bd = P.bits_to_f64(inp["x"]), P.bits_to_f64(inp["w"]), P.bits_to_f64(inp["b"])
        scale = P.layernorm_y_scale(xd, mean_ref, rstd_ref, wd, bd)
        P.assert_bf16_close(got["out"], ref, f"{what}: y", floor_scale=scale)
        P.assert_f32_close(got["mean"], mean_ref, f"{what}: mean")
        P.assert_f32_close(got["rstd"], rstd_ref, f"{what}: rstd")


def cu_count():
    return torch.cuda.get_device_properties(0).multi_processor_count


# (rows, hidden) for the library's own choice: every shape is split for at
# least one op (heavy rows; LayerNorm rows wider than one workgroup holds)
CHOSEN = [(1, 65536), (4, 65536), (16, 65536), (3, 65528), (1, 32768), (2, 57344),
          (64, 65536), (32, 49152), (7, 40960), (5, 49152)]
# explicit chunk counts: (rows, hidden, split, effective k)
EXPLICIT = [(2, 32768, 5, 4), (1, 65536, 64, 32), (5, 30000, 3, 3), (2, 16, 2, 1),
            (4, 8192, 2, 2), (1, 4096, 16, 2), (17, 12288, 6, 6), (64, 16384, 4, 4)]


@pytest.mark.parametrize("rows,h", CHOSEN)
def test_split_library_choice(rows, h):
    split_any = False
    for op in OPS:
        k, v = rn.select_split(op, rows, h)
        split_any |= k > 1
        assert rows * k <= cu_count()
        ws = workspace(rows)
        inp = inputs(op, rows, h, seed=rows * 7 + h)
        check(op, inp, run(op, inp, ws, 0), f"{op} {rows}x{h} split {k}x{v}")
        assert int(torch.count_nonzero(ws)) == 0, "the workspace must be left zero-filled"
    assert split_any, (rows, h)


@pytest.mark.parametrize("rows,h,split,k", EXPLICIT)
def test_split_explicit(rows, h, split, k):
    acc = h // 8
    v = -(-acc // (256 * split))
    assert -(-acc // (256 * v)) == k  # the chunk count the library derives
    for op in OPS:
        ws = workspace(rows)
        inp = inputs(op, rows, h, seed=split + h)
        check(op, inp, run(op, inp, ws, split), f"{op} {rows}x{h} split={split}")
        assert int(torch.count_nonzero(ws)) == 0


def test_split_constant_rows():
    """Degenerate rows: a constant row has variance exactly 0 in every chunk,
    so LayerNorm gives y = bias exactly; RMSNorm gives w * x / sqrt(x^2 + eps)."""
    rows, h = 4, 16384
    for op in OPS:
        inp = inputs(op, rows, h, seed=5)
        inp["x"] = np.repeat(inp["x"][:, :1], h, axis=1).copy()
        if "r" in inp:
            inp["r"] = np.zeros_like(inp["r"])
        got = run(op, inp, workspace(rows), 8)
        check(op, inp, got, f"{op} constant rows")
        if op == "layernorm_fwd":
            P.assert_bits_equal(got["out"], np.broadcast_to(inp["b"], (rows, h)).copy(),
                                "constant rows: y == bias")


def test_split_not_chosen_runs_usual_kernels():
    """Rows the library does not split run the usual kernels; the workspace
    is not touched and may be absent."""
    for rows, h in ((1, 4096), (300, 16384), (2, 8196), (1, 16384)):
        assert rn.select_split("rmsnorm_fwd", rows, h)[0] == 1
        for op in OPS:
            inp = inputs(op, rows, h, seed=h)
            ws = torch.full((rn.split_workspace_bytes(rows),), 0x5A, dtype=torch.uint8,
                            device=DEV)
            check(op, inp, run(op, inp, ws, 0), f"{op} {rows}x{h} unsplit")
            assert bool((ws == 0x5A).all()), "an unsplit call must not touch the workspace"
            check(op, inp, run(op, inp, None, 0), f"{op} {rows}x{h} no workspace")


def test_split_in_place():
    """out == x (and y == x): each workgroup reads its chunk before any
    workgroup writes, and the chunks are disjoint, so in-place calls work."""
    rows, h = 3, 65536
    for op in ("fused_add_rmsnorm", "rmsnorm_fwd", "layernorm_fwd"):
        assert rn.select_split(op, rows, h)[0] > 1
        inp = inputs(op, rows, h, seed=21)
        x, w = dev(inp["x"]), dev(inp["w"])
        ws = workspace(rows)
        if op == "fused_add_rmsnorm":
            r = dev(inp["r"])
            rn.fused_add_rmsnorm(x, r, w, inp["eps"], out=x, workspace=ws)
            got = {"out": host(x), "res": host(r)}
        elif op == "rmsnorm_fwd":
            rn.rmsnorm_fwd(x, w, inp["eps"], out=x, workspace=ws)
            got = {"out": host(x)}
        else:
            _, mean, rstd = rn.layernorm_fwd(x, w, dev(inp["b"]), inp["eps"], y=x, workspace=ws)
            got = {"out": host(x), "mean": mean.cpu().numpy(), "rstd": rstd.cpu().numpy()}
        check(op, inp, got, f"{op} in place")
        assert int(torch.count_nonzero(ws)) == 0


def test_split_stats_optional():
    rows, h = 2, 57344
    assert rn.select_split("layernorm_fwd", rows, h)[0] > 1
    inp = inputs("layernorm_fwd", rows, h, seed=9)
    ws = workspace(rows)
    y, mean, rstd = rn.layernorm_fwd(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]), inp["eps"],
                                     with_stats=False, workspace=ws, split=0)
    assert mean is None and rstd is None
    ref, mean_ref, rstd_ref = oracle.layernorm_fwd(inp["x"], inp["w"], inp["b"], inp["eps"], NT)
    xd, wd, bd = P.bits_to_f64(inp["x"]), P.bits_to_f64(inp["w"]), P.bits_to_f64(inp["b"])
    P.assert_bf16_close(host(y), ref, "y", floor_scale=P.layernorm_y_scale(xd, mean_ref,
                                                                          rstd_ref, wd, bd))


def test_split_repeated_calls_and_graph_replays():
    """One workspace, many calls of different shapes and ops in stream order,
    then the same calls captured in a HIP graph and replayed with poisoned
    outputs between replays: every result is bitwise the first eager one."""
    shapes = [("fused_add_rmsnorm", 1, 65536), ("layernorm_fwd", 64, 65536),
              ("rmsnorm_fwd", 3, 65536), ("fused_add_rmsnorm", 16, 49152),
              ("layernorm_fwd", 2, 57344)]
    for op, rows, h in shapes:
        assert rn.select_split(op, rows, h)[0] > 1
    ws = workspace(64)
    s = torch.cuda.Stream()
    bufs = []
    for op, rows, h in shapes:
        inp = inputs(op, rows, h, seed=rows + h)
        b = {"op": op, "x": dev(inp["x"]), "w": dev(inp["w"]), "eps": inp["eps"],
             "out": torch.empty(rows, h, dtype=torch.bfloat16, device=DEV)}
        if op == "fused_add_rmsnorm":
            b["r0"] = dev(inp["r"])
            b["r"] = torch.empty_like(b["r0"])
        if op == "layernorm_fwd":
            b["b"] = dev(inp["b"])
            b["mean"] = torch.empty(rows, device=DEV)
            b["rstd"] = torch.empty(rows, device=DEV)
        bufs.append(b)

    def step():
        for b in bufs:
            if b["op"] == "fused_add_rmsnorm":
                b["r"].copy_(b["r0"])
                rn.fused_add_rmsnorm(b["x"], b["r"], b["w"], b["eps"], out=b["out"], stream=s,
                                     workspace=ws, split=0)
            elif b["op"] == "rmsnorm_fwd":
                rn.rmsnorm_fwd(b["x"], b["w"], b["eps"], out=b["out"], stream=s, workspace=ws,
                               split=0)
            else:
                rn.layernorm_fwd(b["x"], b["w"], b["b"], b["eps"], y=b["out"], mean=b["mean"],
                                 rstd=b["rstd"], stream=s, workspace=ws, split=0)

    def outputs():
        torch.cuda.synchronize()
        res = []
        for b in bufs:
            for key in ("out", "r", "mean", "rstd"):
                if key in b:
                    t = b[key]
                    res.append(t.view(torch.int16).cpu().numpy().copy() if t.dtype ==
                               torch.bfloat16 else t.cpu().numpy().copy())
        return res

    with torch.cuda.stream(s):
        step()
    first = outputs()
    for _ in range(3):
        with torch.cuda.stream(s):
            step()
        for a, b in zip(outputs(), first):
            assert np.array_equal(a, b), "repeated eager calls differ"
    assert int(torch.count_nonzero(ws)) == 0

    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for replay in range(4):
        for b in bufs:
            b["out"].view(torch.int16).fill_(0x7FC1)
            if "mean" in b:
                b["mean"].fill_(float("nan"))
                b["rstd"].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        for k, (a, b) in enumerate(zip(outputs(), first)):
            assert np.array_equal(a, b), f"replay {replay}: output {k} differs"
        assert int(torch.count_nonzero(ws)) == 0


def test_split_errors_that_need_the_device():
    rows, h = 200, 16384
    inp = inputs("rmsnorm_fwd", rows, h, seed=1)
    x, w = dev(inp["x"]), dev(inp["w"])
    with pytest.raises(rn.NormError) as e:  # 400 workgroups cannot all be resident
        rn.rmsnorm_fwd(x, w, 1e-6, workspace=workspace(rows), split=2)
    assert e.value.status == 1
    small = torch.zeros(rn.split_workspace_bytes(1), dtype=torch.uint8, device=DEV)
    x64 = dev(inputs("rmsnorm_fwd", 4, 65536, seed=2)["x"])
    w64 = dev(inputs("rmsnorm_fwd", 4, 65536, seed=2)["w"])
    with pytest.raises(rn.NormError) as e:
        rn.rmsnorm_fwd(x64, w64, 1e-6, workspace=small, split=0)
    assert e.value.status == 4
    with pytest.raises(rn.NormError) as e:  # the library splits these rows: a workspace is needed
        rn.rmsnorm_fwd(x64, w64, 1e-6, workspace=None, split=0)
    assert e.value.status == 4


@pytest.mark.parametrize("op,rows,h,split", [("fused_add_rmsnorm", 2, 32768, 4),
                                             ("rmsnorm_fwd", 3, 65536, 4),
                                             ("layernorm_fwd", 2, 57344, 5)])
def test_split_give_up_is_visible(op, rows, h, split):
    """A partner wait that gives up (forced from the host: a spin limit of 0
    polls, so every split workgroup gives up at once and every kernel still
    exits) writes NaN for its chunk, never a wrong finite value; the fused
    op's residual is still exact; the error word reports it until cleared,
    the rest of the workspace is zero again, and the next call on the same
    workspace is correct."""
    inp = inputs(op, rows, h, seed=5 + rows)
    ws = workspace(rows)
    prev = rn.set_split_spin_limit(0)
    try:
        got = run(op, inp, ws, split)
        assert rn.set_split_spin_limit(0) == 0
        with pytest.raises(rn.SplitGaveUpError):
            if op == "rmsnorm_fwd":
                rn.rmsnorm_fwd(dev(inp["x"]), dev(inp["w"]), inp["eps"], workspace=ws,
                               split=split, check_split=True)
            elif op == "fused_add_rmsnorm":
                rn.fused_add_rmsnorm(dev(inp["x"]), dev(inp["r"]), dev(inp["w"]), inp["eps"],
                                     workspace=ws, split=split, check_split=True)
            else:
                rn.layernorm_fwd(dev(inp["x"]), dev(inp["w"]), dev(inp["b"]), inp["eps"],
                                 workspace=ws, split=split, check_split=True)
    finally:
        rn.set_split_spin_limit(prev)
    assert prev == 1 << 20
    out = P.bits_to_f64(got["out"])
    assert np.isnan(out).all(), f"{op}: a chunk that gave up holds finite values"
    if op == "fused_add_rmsnorm":
        _, res_ref, _ = oracle.fused_add_rmsnorm(inp["x"], inp["r"], inp["w"], inp["eps"], NT)
        P.assert_bits_equal(got["res"], res_ref, f"{op}: residual after a give-up")
    if op == "layernorm_fwd":
        assert np.isnan(got["mean"]).all() and np.isnan(got["rstd"]).all()
    # check_split cleared the word of the second call; the first call's bit was
    # the same bit, so the word is 0 now and the row words were zeroed
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws)) == 0
    assert rn.split_status(ws) == 0
    # a give-up without check_split: the word reports it, clear=False keeps it
    prev = rn.set_split_spin_limit(0)
    try:
        run(op, inp, ws, split)
    finally:
        rn.set_split_spin_limit(prev)
    assert rn.split_status(ws, clear=False) == 1
    assert int(torch.count_nonzero(ws[4:])) == 0
    assert rn.split_status(ws) == 1
    assert rn.split_status(ws) == 0
    # the same workspace, default limit: correct, and no error reported
    got = run(op, inp, ws, split)
    check(op, inp, got, f"{op} {rows}x{h} after a give-up")
    assert rn.split_status(ws) == 0


def test_split_status_untouched_when_not_split():
    """Rows the library does not split leave the workspace (and its error
    word) alone, whatever the spin limit."""
    inp = inputs("fused_add_rmsnorm", 64, 4096, seed=3)
    assert rn.select_split("fused_add_rmsnorm", 64, 4096)[0] == 1
    ws = workspace(64)
    prev = rn.set_split_spin_limit(0)
    try:
        got = run("fused_add_rmsnorm", inp, ws, 0)
    finally:
        rn.set_split_spin_limit(prev)
    check("fused_add_rmsnorm", inp, got, "not split, spin limit 0")
    assert rn.split_status(ws) == 0
