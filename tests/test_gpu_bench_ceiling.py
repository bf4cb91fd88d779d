"""The benchmark's same-traffic kernel (libnormceiling.so) moves exactly the
bytes it stands for: in every launch shape it writes the old x to the residual
buffer and the old residual to out, bit for bit, for ragged row counts, and
touches nothing past the last row.  It is a measurement kernel, not part of
the normalization library."""
import ctypes
import os

import numpy as np
import pytest
import torch

import row_normalization_persistent_amd as rn

pytestmark = pytest.mark.gpu

PATH = os.path.join(os.path.dirname(os.path.abspath(rn.__file__)), "libnormceiling.so")


@pytest.mark.parametrize("lanes,rpb", [(64, 4), (128, 2), (256, 1), (512, 1)])
def test_same_traffic_kernel_copies(lanes, rpb):
    if not os.path.exists(PATH):
        pytest.fail("libnormceiling.so is not built")
    f = ctypes.CDLL(PATH).normceil_same_traffic_h4096
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    f.restype = ctypes.c_int
    h = 4096
    g = torch.Generator(device="cuda")
    g.manual_seed(lanes)
    for rows in (1, 37, 1001):
        x = torch.randn(rows + 1, h, generator=g, device="cuda").to(torch.bfloat16)
        r = torch.randn(rows + 1, h, generator=g, device="cuda").to(torch.bfloat16)
        out = torch.full((rows + 1, h), 7.0, dtype=torch.bfloat16, device="cuda")
        x0, r0 = x.clone(), r.clone()
        stream = torch.cuda.current_stream().cuda_stream
        assert f(out.data_ptr(), r.data_ptr(), x.data_ptr(), rows, lanes, rpb, stream) == 0
        torch.cuda.synchronize()
        assert torch.equal(r[:rows].view(torch.int16), x0[:rows].view(torch.int16))
        assert torch.equal(out[:rows].view(torch.int16), r0[:rows].view(torch.int16))
        assert torch.equal(x.view(torch.int16), x0.view(torch.int16))  # x is only read
        assert torch.equal(r[rows].view(torch.int16), r0[rows].view(torch.int16))  # the row past
        assert bool((out[rows] == 7.0).all())
    assert f(out.data_ptr(), r.data_ptr(), x.data_ptr(), 4, 96, 1, stream) == 1  # no such shape
    assert f(out.data_ptr() + 2, r.data_ptr(), x.data_ptr(), 4, lanes, rpb, stream) == 1
    assert f(0, r.data_ptr(), x.data_ptr(), 4, lanes, rpb, stream) == 1
    assert np.isfinite(out[:rows].float().cpu().numpy()).all()


def _lib():
    if not os.path.exists(PATH):
        pytest.fail("libnormceiling.so is not built")
    L = ctypes.CDLL(PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.normceil_stream.argtypes = [ctypes.POINTER(vp), i32, ctypes.POINTER(vp), i32, i64, i32,
                                  i32, vp]
    L.normceil_stream.restype = ctypes.c_int
    L.normceil_rows.argtypes = [ctypes.POINTER(vp), i32, vp, i64, i64, i32, i32, i64, i32, vp]
    L.normceil_rows.restype = ctypes.c_int
    return L


def _ptrs(ts, n):
    return (ctypes.c_void_p * n)(*([t.data_ptr() for t in ts] + [None] * (n - len(ts))))


@pytest.mark.parametrize("nr,nw", [(1, 0), (0, 1), (1, 1), (2, 1), (2, 2), (3, 1)])
def test_stream_kernel_moves_exactly_its_buffers(nr, nw):
    """Every output vector i is the XOR of the inputs' vector i (the vector
    index when there is no input); read-only launches write nothing; nothing
    past the end is touched.  Sizes are ragged against every grid x unroll."""
    L = _lib()
    stream = torch.cuda.current_stream().cuda_stream
    g = torch.Generator(device="cuda")
    g.manual_seed(nr * 4 + nw)
    for n_vec, grid, unroll in ((1, 1, 1), (1000, 3, 8), (123457, 64, 4), (1 << 20, 1024, 2)):
        ins = [torch.randint(-2 ** 31, 2 ** 31 - 1, (n_vec + 4, 4), dtype=torch.int32,
                             generator=g, device="cuda") for _ in range(nr)]
        outs = [torch.full((n_vec + 4, 4), 7, dtype=torch.int32, device="cuda")
                for _ in range(nw)]
        sink = torch.full((grid + 1, 4), 7, dtype=torch.int32, device="cuda")
        ins0 = [t.clone() for t in ins]
        o = outs if nw else [sink]
        assert L.normceil_stream(_ptrs(ins, 3), nr, _ptrs(o, 2), nw, n_vec * 16, grid, unroll,
                                 stream) == 0
        torch.cuda.synchronize()
        if nr:
            exp = ins0[0][:n_vec].clone()
            for t in ins0[1:]:
                exp ^= t[:n_vec]
        else:
            i = torch.arange(n_vec, dtype=torch.int64, device="cuda")
            exp = torch.stack([i.to(torch.int32), (i >> 32).to(torch.int32),
                               torch.zeros_like(i, dtype=torch.int32),
                               torch.zeros_like(i, dtype=torch.int32)], 1)
        for t in outs:
            assert torch.equal(t[:n_vec], exp)
            assert bool((t[n_vec:] == 7).all()), "wrote past the end"
        for a, b in zip(ins, ins0):
            assert torch.equal(a, b), "an input changed"
        if not nw:
            assert bool((sink == 7).all()), "a read-only launch wrote its sink"
    assert L.normceil_stream(_ptrs([], 3), 0, _ptrs([], 2), 0, 16, 1, 1, stream) == 1
    assert L.normceil_stream(_ptrs(ins, 3), nr, _ptrs(o, 2), nw, 24, 1, 1, stream) == 1
    assert L.normceil_stream(_ptrs(ins, 3), nr, _ptrs(o, 2), nw, 16, 1, 3, stream) == 1


@pytest.mark.parametrize("nr,lanes,vecs,grid,depth", [
    (2, 512, 1, 256, 4), (2, 1024, 1, 256, 3), (3, 512, 1, 256, 4), (1, 512, 4, 256, 8),
    (2, 512, 8, 256, 1), (2, 512, 1, 0, 1), (1, 128, 2, 7, 2)])
def test_row_traffic_kernel_moves_exactly_its_rows(nr, lanes, vecs, grid, depth):
    """Every output row is the XOR of its input rows, for ragged row counts
    against the walk's grid and ring; rows past the end and the inputs are
    untouched."""
    L = _lib()
    stream = torch.cuda.current_stream().cuda_stream
    h = vecs * 8 * lanes
    g = torch.Generator(device="cuda")
    g.manual_seed(lanes + vecs + depth)
    for rows in (1, 37, 1000):
        ins = [torch.randint(-2 ** 15, 2 ** 15 - 1, (rows + 1, h), dtype=torch.int16,
                             generator=g, device="cuda") for _ in range(nr)]
        out = torch.full((rows + 1, h), 7, dtype=torch.int16, device="cuda")
        ins0 = [t.clone() for t in ins]
        assert L.normceil_rows(_ptrs(ins, 3), nr, out.data_ptr(), rows, h, lanes, vecs, grid,
                               depth, stream) == 0
        torch.cuda.synchronize()
        exp = ins0[0][:rows].clone()
        for t in ins0[1:]:
            exp ^= t[:rows]
        assert torch.equal(out[:rows], exp)
        assert bool((out[rows] == 7).all()), "wrote past the last row"
        for a, b in zip(ins, ins0):
            assert torch.equal(a, b)
    assert L.normceil_rows(_ptrs(ins, 3), nr, out.data_ptr(), rows, h + 8, lanes, vecs, grid,
                           depth, stream) == 1
    assert L.normceil_rows(_ptrs(ins, 3), nr, out.data_ptr(), rows, h, lanes, vecs, 0, 2,
                           stream) == 1
    assert L.normceil_rows(_ptrs(ins, 3), 3, out.data_ptr(), rows, 4 * 8 * 512, 512, 4, 256, 8,
                           stream) == 1  # a ring that would not fit the registers


@pytest.mark.parametrize("lanes,rpb", [(64, 4), (128, 2), (256, 1), (512, 1)])
def test_fused_shape_parts(lanes, rpb):
    """Reads-only launches write nothing, writes-only launches write exactly
    out and the residual (the vector index) for the rows given, and the empty
    grid touches nothing."""
    L = ctypes.CDLL(PATH)
    f = L.normceil_fused_shape_part
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    f.restype = ctypes.c_int
    h = 4096
    stream = torch.cuda.current_stream().cuda_stream
    for rows in (1, 37, 1001):
        x = torch.randint(-2 ** 31, 2 ** 31 - 1, (rows + 1, h // 2), dtype=torch.int32,
                          device="cuda")
        r0 = torch.randint(-2 ** 31, 2 ** 31 - 1, (rows + 1, h // 2), dtype=torch.int32,
                           device="cuda")
        for mode in (1, 3):
            r, out = r0.clone(), torch.full_like(x, 7)
            assert f(out.data_ptr(), r.data_ptr(), x.data_ptr(), rows, lanes, rpb, mode,
                     stream) == 0
            torch.cuda.synchronize()
            assert torch.equal(r, r0) and bool((out == 7).all()), mode
        r, out = r0.clone(), torch.full_like(x, 7)
        assert f(out.data_ptr(), r.data_ptr(), x.data_ptr(), rows, lanes, rpb, 2, stream) == 0
        torch.cuda.synchronize()
        idx = torch.arange(rows * h // 8, dtype=torch.int32, device="cuda")
        exp = idx.repeat_interleave(4).view(rows, h // 2)
        assert torch.equal(out[:rows], exp) and torch.equal(r[:rows], exp)
        assert torch.equal(r[rows], r0[rows]) and bool((out[rows] == 7).all())
    assert f(out.data_ptr(), r.data_ptr(), x.data_ptr(), 4, lanes, rpb, 0, stream) == 1
    assert f(out.data_ptr(), r.data_ptr(), x.data_ptr(), 4, 96, 1, 1, stream) == 1
