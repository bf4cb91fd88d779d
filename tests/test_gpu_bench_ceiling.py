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
