"""Inner-persistent row normalization for MI355X (gfx950): Python binding.

A thin ctypes layer over ``librownorm.so`` (C ABI declared in
``include/norm.h``).  It only checks tensor metadata and marshals pointers,
sizes and the current HIP stream; every step of the computation runs in the
library's HIP kernels.  There is no fallback: if the library is missing the
import of an op raises.

Operations (names as in the C ABI):
  * ``fused_add_rmsnorm``  -- residual <- bf16(x + residual);
                              out <- bf16(RMSNorm(x + residual) * w)
  * ``rmsnorm_fwd``        -- out <- bf16(RMSNorm(x) * w)
  * ``layernorm_fwd``      -- y <- bf16(LayerNorm(x) * w + b), fp32 mean/rstd
  * ``layernorm_bwd``      -- dx (bf16), dweight/dbias (fp32) from dy, x, mean, rstd, w
  * ``rmsnorm_bwd``        -- dx (bf16), dweight (fp32) from dy, x, w (rstd recomputed)
  * ``fused_add_rmsnorm_bwd`` -- ds = RMSNorm backward of dout at s, plus dres;
                              the gradient of both the x and residual inputs

Each op has an fp32 twin with the suffix ``_f32`` (fp32 activations, weights
and gradients; contiguous rows, hidden a multiple of 4 up to 2^20).

The three forward ops also take ``workspace=`` (a zero-filled uint8 device
tensor of ``split_workspace_bytes(rows)``) and ``split=``: the row-split entry
points, which may spread each of few wide rows over several workgroups.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librownorm.so")

# hidden sizes of the compiled-hidden kernels; any other hidden runs on the
# run-time-hidden kernels
HIDDEN_SIZES = (1024, 2048, 4096, 8192, 12288, 16384)

OP_FUSED_ADD_RMSNORM = 0
OP_RMSNORM_FWD = 1
OP_LAYERNORM_FWD = 2
OP_LAYERNORM_BWD = 3
OP_RMSNORM_BWD = 4
OP_FUSED_ADD_RMSNORM_BWD = 5
OPS = {"fused_add_rmsnorm": 0, "rmsnorm_fwd": 1, "layernorm_fwd": 2, "layernorm_bwd": 3,
       "rmsnorm_bwd": 4, "fused_add_rmsnorm_bwd": 5}

STATUS = {
    0: "NORM_SUCCESS",
    1: "NORM_ERROR_INVALID_VALUE",
    2: "NORM_ERROR_UNSUPPORTED_HIDDEN",
    3: "NORM_ERROR_MISALIGNED",
    4: "NORM_ERROR_WORKSPACE",
    5: "NORM_ERROR_LAUNCH",
    6: "NORM_ERROR_DEVICE",
}


class NormError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class LaunchCfg(ctypes.Structure):
    _fields_ = [("threads_per_row", ctypes.c_int32), ("rows_per_block", ctypes.c_int32),
                ("grid", ctypes.c_int32), ("vector_elems", ctypes.c_int32)]

    def astuple(self):
        return (self.threads_per_row, self.rows_per_block, self.grid, self.vector_elems)

    def __repr__(self):
        return (f"LaunchCfg(threads_per_row={self.threads_per_row}, "
                f"rows_per_block={self.rows_per_block}, grid={self.grid}, "
                f"vector_elems={self.vector_elems})")


@dataclass(frozen=True)
class Cfg:
    """A launch shape.  vector_elems == 0: a compiled-hidden shape; 1, 2, 4, 8:
    a run-time-hidden shape with accesses of that many bf16 elements."""
    threads_per_row: int
    rows_per_block: int = 1
    grid: int = 0
    vector_elems: int = 0

    @property
    def runtime_hidden(self) -> bool:
        return self.vector_elems != 0

    def c(self) -> LaunchCfg:
        return LaunchCfg(self.threads_per_row, self.rows_per_block, self.grid, self.vector_elems)


_lib = None
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_i32 = ctypes.c_int32
_cfgp = ctypes.POINTER(LaunchCfg)


def lib() -> ctypes.CDLL:
    """Load librownorm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m row_normalization_persistent_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.norm_status_string.argtypes = [ctypes.c_int]
    L.norm_status_string.restype = ctypes.c_char_p
    _sz = ctypes.c_size_t
    sigs = {
        "norm_fused_add_rmsnorm_cfg": [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _cfgp, _vp],
        "norm_rmsnorm_fwd_cfg": [_vp, _vp, _vp, _i64, _i64, _f32, _cfgp, _vp],
        "norm_layernorm_fwd_cfg": [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _cfgp, _vp],
        "norm_layernorm_bwd_cfg": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64,
                                   _f32, _cfgp, _vp],
        "norm_fused_add_rmsnorm": [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _vp],
        "norm_rmsnorm_fwd": [_vp, _vp, _vp, _i64, _i64, _f32, _vp],
        "norm_layernorm_fwd": [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _vp],
        "norm_layernorm_bwd": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64,
                               _f32, _vp],
        "norm_rmsnorm_bwd_cfg": [_vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64, _f32, _cfgp,
                                 _vp],
        "norm_rmsnorm_bwd": [_vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64, _f32, _vp],
        "norm_fused_add_rmsnorm_bwd_cfg": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64,
                                           _f32, _cfgp, _vp],
        "norm_fused_add_rmsnorm_bwd": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64, _f32,
                                       _vp],
        # strided variants: every matrix pointer is followed by its leading dimension
        "norm_fused_add_rmsnorm_ex": [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _f32,
                                      _cfgp, _vp],
        "norm_rmsnorm_fwd_ex": [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _f32, _cfgp, _vp],
        "norm_layernorm_fwd_ex": [_vp, _i64, _vp, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _f32,
                                  _cfgp, _vp],
        "norm_layernorm_bwd_ex": [_vp, _i64, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp,
                                  _sz, _i64, _i64, _f32, _cfgp, _vp],
        "norm_rmsnorm_bwd_ex": [_vp, _i64, _vp, _vp, _i64, _vp, _i64, _vp, _vp, _sz, _i64, _i64,
                                _f32, _cfgp, _vp],
        "norm_fused_add_rmsnorm_bwd_ex": [_vp, _i64, _vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                                          _vp, _sz, _i64, _i64, _f32, _cfgp, _vp],
        # row-split forward: workspace, workspace bytes, workgroups per row
        "norm_fused_add_rmsnorm_split": [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _vp, _sz, _i32,
                                         _vp],
        "norm_rmsnorm_fwd_split": [_vp, _vp, _vp, _i64, _i64, _f32, _vp, _sz, _i32, _vp],
        "norm_layernorm_fwd_split": [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _vp, _sz,
                                     _i32, _vp],
        # LayerNorm backward with the library's per-device scratch (no workspace)
        "norm_layernorm_bwd_noalloc": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32,
                                       _vp],
        # fp32 activations (contiguous rows)
        "norm_fused_add_rmsnorm_f32": [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _vp],
        "norm_rmsnorm_fwd_f32": [_vp, _vp, _vp, _i64, _i64, _f32, _vp],
        "norm_layernorm_fwd_f32": [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _f32, _vp],
        "norm_layernorm_bwd_f32": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64,
                                   _f32, _vp],
        "norm_rmsnorm_bwd_f32": [_vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64, _f32, _vp],
        "norm_fused_add_rmsnorm_bwd_f32": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64,
                                           _f32, _vp],
    }
    for n, args in sigs.items():
        fn = getattr(L, n)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.norm_rmsnorm_bwd_workspace_bytes.argtypes = [_i64, _i64]
    L.norm_rmsnorm_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.norm_rmsnorm_bwd_workspace_bytes_cfg.argtypes = [_i64, _i64, _cfgp]
    L.norm_rmsnorm_bwd_workspace_bytes_cfg.restype = ctypes.c_size_t
    L.norm_layernorm_bwd_workspace_bytes.argtypes = [_i64, _i64]
    L.norm_layernorm_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.norm_layernorm_bwd_workspace_bytes_cfg.argtypes = [_i64, _i64, _cfgp]
    L.norm_layernorm_bwd_workspace_bytes_cfg.restype = ctypes.c_size_t
    L.norm_bwd_workspace_bytes_f32.argtypes = [ctypes.c_int, _i64, _i64]
    L.norm_bwd_workspace_bytes_f32.restype = ctypes.c_size_t
    L.norm_split_workspace_bytes.argtypes = [_i64]
    L.norm_split_workspace_bytes.restype = ctypes.c_size_t
    L.norm_select_split.argtypes = [ctypes.c_int, _i64, _i64, _i32, ctypes.POINTER(_i32),
                                    ctypes.POINTER(_i32)]
    L.norm_select_split.restype = ctypes.c_int
    L.norm_split_status.argtypes = [_vp, _i32, ctypes.POINTER(ctypes.c_uint32), _vp]
    L.norm_split_status.restype = ctypes.c_int
    L.norm_split_set_spin_limit.argtypes = [ctypes.c_uint32]
    L.norm_split_set_spin_limit.restype = ctypes.c_uint32
    L.norm_bwd_set_spin_limit.argtypes = [ctypes.c_uint32]
    L.norm_bwd_set_spin_limit.restype = ctypes.c_uint32
    L.norm_select_config.argtypes = [ctypes.c_int, _i64, _i64, ctypes.c_int32, _cfgp]
    L.norm_select_config.restype = ctypes.c_int
    L.norm_list_configs.argtypes = [ctypes.c_int, _i64, _cfgp, ctypes.c_int32]
    L.norm_list_configs.restype = ctypes.c_int32
    L.norm_describe_config.argtypes = [ctypes.c_int, _i64, _i64, ctypes.c_int32, ctypes.c_char_p,
                                       ctypes.c_size_t]
    L.norm_describe_config.restype = ctypes.c_int32
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().norm_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise NormError(status, f"{what}: {status_string(status)}")


def _cfg_ptr(cfg):
    if cfg is None:
        return None
    c = cfg.c() if isinstance(cfg, Cfg) else cfg
    return ctypes.byref(c)


# The current stream's handle without building a torch.cuda.Stream object
# (the public route costs about 2 us a call); falls back to it where absent.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_current_device = getattr(torch._C, "_cuda_getDevice", None)


def _stream(stream, *tensors) -> int:
    """The stream handle to launch on.  The library launches on the current
    HIP device, so every tensor of the call must live there."""
    cur = _current_device() if _current_device is not None else torch.cuda.current_device()
    for t in tensors:
        if t is not None and t.get_device() != cur:
            raise ValueError(f"every tensor must be on the current device cuda:{cur}; "
                             f"got one on {t.device}")
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(cur)
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _tensor(t, name: str, dtype=torch.bfloat16) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t


def _mat(t, name: str, dtype=torch.bfloat16) -> torch.Tensor:
    """A contiguous device tensor."""
    _tensor(t, name, dtype)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _rows(t, name: str, hidden: int | None = None, dtype=torch.bfloat16):
    """A [..., hidden] bf16 device tensor viewed as rows: returns (rows,
    hidden, ld), ld the row stride in elements.  The last dimension must be
    unit-stride and the leading dimensions must collapse to one stride (any
    contiguous tensor, a column slice of a wider matrix, ...)."""
    _tensor(t, name, dtype)
    if t.dim() < 1:
        raise ValueError(f"{name} must have a hidden dimension")
    h = t.shape[-1]
    if hidden is not None and h != hidden:
        raise ValueError(f"{name} must have hidden={hidden} columns, got {h}")
    rows = t.numel() // h if h else 0
    if t.is_contiguous() or rows <= 1:
        return rows, h, h
    if t.stride(-1) != 1:
        raise ValueError(f"{name} needs a unit stride along its last dimension")
    try:
        v = t.view(rows, h)
    except RuntimeError as e:
        raise ValueError(f"{name}: leading dimensions do not collapse to one row stride") from e
    return rows, h, v.stride(0)


def _rows_hidden(x: torch.Tensor):
    if x.dim() < 1:
        raise ValueError("x must have a hidden dimension")
    hidden = x.shape[-1]
    rows = x.numel() // hidden if hidden else 0
    return rows, hidden


def _vec(t, hidden, name, dtype=torch.bfloat16):
    _mat(t, name, dtype)
    if t.numel() != hidden:
        raise ValueError(f"{name} must hold hidden={hidden} elements")
    return t


def _like(t, out, name):
    """`out` (validated, shape of t, any row stride) or a new contiguous tensor."""
    if out is None:
        return torch.empty(t.shape, dtype=t.dtype, device=t.device)
    if out.shape != t.shape:
        raise ValueError(f"{name} must have shape {tuple(t.shape)}")
    return out


def split_workspace_bytes(rows: int) -> int:
    """Bytes of workspace the row-split forward needs for `rows` rows."""
    return int(lib().norm_split_workspace_bytes(rows))


def select_split(op, rows: int, hidden: int, cu_count: int = 0):
    """(workgroups per row, 16-byte accesses per lane) the library would use
    for a row-split forward; (1, 0) means no split."""
    k, v = _i32(), _i32()
    _check(lib().norm_select_split(int(OPS.get(op, op)), rows, hidden, cu_count,
                                   ctypes.byref(k), ctypes.byref(v)), "norm_select_split")
    return k.value, v.value


class SplitGaveUpError(NormError):
    """A row-split call's workgroup gave up waiting for its row's partners:
    the chunks it owned were written as NaN."""


def split_status(workspace, clear: bool = True, stream=None) -> int:
    """The row-split workspace's error word after every call enqueued on the
    stream so far (synchronizes with it): 0, or bit 0 set when a workgroup
    gave up waiting for its row's partners.  clear: reset it to 0."""
    _mat(workspace, "workspace", torch.uint8)
    st = ctypes.c_uint32()
    _check(lib().norm_split_status(workspace.data_ptr(), int(bool(clear)), ctypes.byref(st),
                                   _stream(stream, workspace)), "norm_split_status")
    return st.value


def set_split_spin_limit(polls: int) -> int:
    """Polls a row-split partner wait makes before giving up (process-wide;
    0 makes every split workgroup give up at once).  Returns the previous
    value.  For tests and diagnostics."""
    return int(lib().norm_split_set_spin_limit(int(polls)))


def set_bwd_spin_limit(polls: int) -> int:
    """Polls a streamed-backward column tile makes waiting for its row's
    other tiles before it re-reads them itself (process-wide; 0: never wait;
    results are the same bits either way).  Returns the previous value.  For
    tests and diagnostics."""
    return int(lib().norm_bwd_set_spin_limit(int(polls)))


def _split_check(workspace, stream, what: str) -> None:
    """check_split=True: wait for the call and raise if any workgroup gave up."""
    if workspace is not None and split_status(workspace, True, stream) != 0:
        raise SplitGaveUpError(6, f"{what}: a workgroup gave up waiting for its row's "
                                  "partners; the chunks it owned are NaN")


def _split_ws(workspace):
    """(pointer, bytes) of a row-split workspace (a zero-filled uint8 device
    tensor), or (None, 0)."""
    if workspace is None:
        return None, 0
    _mat(workspace, "workspace", torch.uint8)
    return workspace.data_ptr(), workspace.numel()


def fused_add_rmsnorm(x, residual, weight, eps: float, out=None, cfg=None, stream=None,
                      workspace=None, split=None, check_split: bool = False):
    """residual <- bf16(x + residual) in place; returns (out, residual).
    x, residual and out may be row-strided views (e.g. column slices).  With
    `workspace` (zero-filled uint8, split_workspace_bytes(rows)) or `split`,
    runs the row-split entry point on contiguous rows (split None/0: the
    library's choice, 1: never, k: about k workgroups a row).  check_split:
    wait for the call and raise SplitGaveUpError if a workgroup gave up."""
    if workspace is not None or split is not None:
        if cfg is not None:
            raise ValueError("cfg does not apply to the row-split entry point")
        rows, hidden = _rows_hidden(_mat(x, "x"))
        _mat(residual, "residual")
        if residual.shape != x.shape:
            raise ValueError("residual must have x's shape")
        _vec(weight, hidden, "weight")
        out = _mat(_like(x, out, "out"), "out")
        wp, wb = _split_ws(workspace)
        _check(lib().norm_fused_add_rmsnorm_split(out.data_ptr(), residual.data_ptr(),
                                                  x.data_ptr(), weight.data_ptr(), rows, hidden,
                                                  float(eps), wp, wb, int(split or 0),
                                                  _stream(stream, x, residual, weight, out,
                                                          workspace)),
               "norm_fused_add_rmsnorm_split")
        if check_split:
            _split_check(workspace, stream, "norm_fused_add_rmsnorm_split")
        return out, residual
    rows, hidden, ld_x = _rows(x, "x")
    if residual.shape != x.shape:
        raise ValueError("residual must have x's shape")
    _, _, ld_r = _rows(residual, "residual")
    _vec(weight, hidden, "weight")
    out = _like(x, out, "out")
    _, _, ld_o = _rows(out, "out")
    _check(lib().norm_fused_add_rmsnorm_ex(out.data_ptr(), ld_o, residual.data_ptr(), ld_r,
                                           x.data_ptr(), ld_x, weight.data_ptr(), rows, hidden,
                                           float(eps), _cfg_ptr(cfg),
                                           _stream(stream, x, residual, weight, out)),
           "norm_fused_add_rmsnorm")
    return out, residual


def rmsnorm_fwd(x, weight, eps: float, out=None, cfg=None, stream=None, workspace=None,
                split=None, check_split: bool = False):
    """workspace / split / check_split: the row-split entry point, as for
    fused_add_rmsnorm."""
    if workspace is not None or split is not None:
        if cfg is not None:
            raise ValueError("cfg does not apply to the row-split entry point")
        rows, hidden = _rows_hidden(_mat(x, "x"))
        _vec(weight, hidden, "weight")
        out = _mat(_like(x, out, "out"), "out")
        wp, wb = _split_ws(workspace)
        _check(lib().norm_rmsnorm_fwd_split(out.data_ptr(), x.data_ptr(), weight.data_ptr(),
                                            rows, hidden, float(eps), wp, wb, int(split or 0),
                                            _stream(stream, x, weight, out, workspace)),
               "norm_rmsnorm_fwd_split")
        if check_split:
            _split_check(workspace, stream, "norm_rmsnorm_fwd_split")
        return out
    rows, hidden, ld_x = _rows(x, "x")
    _vec(weight, hidden, "weight")
    out = _like(x, out, "out")
    _, _, ld_o = _rows(out, "out")
    _check(lib().norm_rmsnorm_fwd_ex(out.data_ptr(), ld_o, x.data_ptr(), ld_x, weight.data_ptr(),
                                     rows, hidden, float(eps), _cfg_ptr(cfg),
                                     _stream(stream, x, weight, out)),
           "norm_rmsnorm_fwd")
    return out


def layernorm_fwd(x, weight, bias, eps: float, y=None, mean=None, rstd=None,
                  with_stats: bool = True, cfg=None, stream=None, workspace=None, split=None,
                  check_split: bool = False):
    """Returns (y, mean, rstd); mean/rstd are None when with_stats is False.
    workspace / split / check_split: the row-split entry point, as for
    fused_add_rmsnorm."""
    use_split = workspace is not None or split is not None
    if use_split:
        if cfg is not None:
            raise ValueError("cfg does not apply to the row-split entry point")
        _mat(x, "x")
    rows, hidden, ld_x = _rows(x, "x")
    _vec(weight, hidden, "weight")
    _vec(bias, hidden, "bias")
    y = _like(x, y, "y")
    _, _, ld_y = _rows(y, "y")
    if with_stats:
        mean = torch.empty(rows, dtype=torch.float32, device=x.device) if mean is None else mean
        rstd = torch.empty(rows, dtype=torch.float32, device=x.device) if rstd is None else rstd
        _mat(mean, "mean", torch.float32)
        _mat(rstd, "rstd", torch.float32)
        if mean.numel() != rows or rstd.numel() != rows:
            raise ValueError("mean/rstd must hold one value per row")
        mp, rp = mean.data_ptr(), rstd.data_ptr()
    else:
        mean = rstd = None
        mp = rp = None
    if use_split:
        _mat(y, "y")
        wp, wb = _split_ws(workspace)
        _check(lib().norm_layernorm_fwd_split(y.data_ptr(), mp, rp, x.data_ptr(),
                                              weight.data_ptr(), bias.data_ptr(), rows, hidden,
                                              float(eps), wp, wb, int(split or 0),
                                              _stream(stream, x, weight, bias, y, mean, rstd,
                                                      workspace)),
               "norm_layernorm_fwd_split")
        if check_split:
            _split_check(workspace, stream, "norm_layernorm_fwd_split")
        return y, mean, rstd
    _check(lib().norm_layernorm_fwd_ex(y.data_ptr(), ld_y, mp, rp, x.data_ptr(), ld_x,
                                       weight.data_ptr(), bias.data_ptr(), rows, hidden,
                                       float(eps), _cfg_ptr(cfg),
                                       _stream(stream, x, weight, bias, y, mean, rstd)),
           "norm_layernorm_fwd")
    return y, mean, rstd


def workspace_bytes(rows: int, hidden: int, cfg=None, op: str = "layernorm_bwd") -> int:
    """Workspace bytes a backward op needs (LayerNorm: two partial slabs per
    row walker; the RMSNorm backward ops: one).  Without cfg: enough for any
    layout of this hidden size."""
    rms = OPS.get(op, op) in (OP_RMSNORM_BWD, OP_FUSED_ADD_RMSNORM_BWD)
    if cfg is None:
        fn = lib().norm_rmsnorm_bwd_workspace_bytes if rms else \
            lib().norm_layernorm_bwd_workspace_bytes
        return int(fn(rows, hidden))
    fn = lib().norm_rmsnorm_bwd_workspace_bytes_cfg if rms else \
        lib().norm_layernorm_bwd_workspace_bytes_cfg
    return int(fn(rows, hidden, _cfg_ptr(cfg)))


def _bwd_common(dy, x, weight, dx, dweight, workspace, cfg, op):
    rows, hidden, ld_x = _rows(x, "x")
    if dy.shape != x.shape:
        raise ValueError("dy must have x's shape")
    _, _, ld_dy = _rows(dy, "dy")
    _vec(weight, hidden, "weight")
    dx = _like(x, dx, "dx")
    _, _, ld_dx = _rows(dx, "dx")
    dweight = torch.empty(hidden, dtype=torch.float32, device=x.device) if dweight is None \
        else dweight
    _vec(dweight, hidden, "dweight", torch.float32)
    need = workspace_bytes(rows, hidden, cfg, op)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _mat(workspace, "workspace", workspace.dtype)
    wsb = workspace.numel() * workspace.element_size()
    return rows, hidden, (ld_dx, ld_dy, ld_x), dx, dweight, workspace, wsb


def layernorm_bwd(dy, x, mean, rstd, weight, eps: float = 0.0, dx=None, dweight=None,
                  dbias=None, workspace=None, cfg=None, stream=None):
    """Returns (dx, dweight, dbias).  ``workspace`` (uint8 device tensor) is
    allocated when not given."""
    rows, hidden, (ld_dx, ld_dy, ld_x), dx, dweight, workspace, wsb = _bwd_common(
        dy, x, weight, dx, dweight, workspace, cfg, "layernorm_bwd")
    _mat(mean, "mean", torch.float32)
    _mat(rstd, "rstd", torch.float32)
    if mean.numel() != rows or rstd.numel() != rows:
        raise ValueError("mean/rstd must hold one value per row")
    dbias = torch.empty(hidden, dtype=torch.float32, device=x.device) if dbias is None else dbias
    _vec(dbias, hidden, "dbias", torch.float32)
    _check(lib().norm_layernorm_bwd_ex(dx.data_ptr(), ld_dx, dweight.data_ptr(),
                                       dbias.data_ptr(), dy.data_ptr(), ld_dy, x.data_ptr(), ld_x,
                                       mean.data_ptr(), rstd.data_ptr(), weight.data_ptr(),
                                       workspace.data_ptr(), wsb, rows, hidden, float(eps),
                                       _cfg_ptr(cfg),
                                       _stream(stream, dy, x, mean, rstd, weight, dx, dweight,
                                               dbias, workspace)),
           "norm_layernorm_bwd")
    return dx, dweight, dbias


# bytes of the per-device scratch array norm_layernorm_bwd_noalloc uses
NOALLOC_SCRATCH_BYTES = 32 << 20


def layernorm_bwd_noalloc(dy, x, mean, rstd, weight, eps: float = 0.0, dx=None, dweight=None,
                          dbias=None, stream=None):
    """layernorm_bwd through the entry point that allocates nothing: its
    partial sums go to the library's per-device scratch array, so calls that
    overlap in time on one device race.  Contiguous tensors; pass dx, dweight
    and dbias to keep the binding from allocating them.  Returns (dx,
    dweight, dbias)."""
    rows, hidden = _rows_hidden(_mat(x, "x"))
    _mat(dy, "dy")
    if dy.shape != x.shape:
        raise ValueError("dy must have x's shape")
    _vec(weight, hidden, "weight")
    _mat(mean, "mean", torch.float32)
    _mat(rstd, "rstd", torch.float32)
    if mean.numel() != rows or rstd.numel() != rows:
        raise ValueError("mean/rstd must hold one value per row")
    dx = _mat(_like(x, dx, "dx"), "dx")
    dweight = torch.empty(hidden, dtype=torch.float32, device=x.device) if dweight is None \
        else dweight
    dbias = torch.empty(hidden, dtype=torch.float32, device=x.device) if dbias is None else dbias
    _vec(dweight, hidden, "dweight", torch.float32)
    _vec(dbias, hidden, "dbias", torch.float32)
    _check(lib().norm_layernorm_bwd_noalloc(dx.data_ptr(), dweight.data_ptr(), dbias.data_ptr(),
                                            dy.data_ptr(), x.data_ptr(), mean.data_ptr(),
                                            rstd.data_ptr(), weight.data_ptr(), rows, hidden,
                                            float(eps),
                                            _stream(stream, dy, x, mean, rstd, weight, dx,
                                                    dweight, dbias)),
           "norm_layernorm_bwd_noalloc")
    return dx, dweight, dbias


def rmsnorm_bwd(dy, x, weight, eps: float, dx=None, dweight=None, workspace=None, cfg=None,
                stream=None):
    """Returns (dx, dweight); rstd is recomputed from x with eps."""
    rows, hidden, (ld_dx, ld_dy, ld_x), dx, dweight, workspace, wsb = _bwd_common(
        dy, x, weight, dx, dweight, workspace, cfg, "rmsnorm_bwd")
    _check(lib().norm_rmsnorm_bwd_ex(dx.data_ptr(), ld_dx, dweight.data_ptr(), dy.data_ptr(),
                                     ld_dy, x.data_ptr(), ld_x, weight.data_ptr(),
                                     workspace.data_ptr(), wsb, rows, hidden, float(eps),
                                     _cfg_ptr(cfg),
                                     _stream(stream, dy, x, weight, dx, dweight, workspace)),
           "norm_rmsnorm_bwd")
    return dx, dweight


def fused_add_rmsnorm_bwd(dout, s, weight, eps: float, dres=None, ds=None, dweight=None,
                          workspace=None, cfg=None, stream=None):
    """Backward of fused_add_rmsnorm at its residual output s: returns (ds,
    dweight), ds the gradient of both the x and residual inputs."""
    rows, hidden, (ld_ds, ld_dout, ld_s), ds, dweight, workspace, wsb = _bwd_common(
        dout, s, weight, ds, dweight, workspace, cfg, "fused_add_rmsnorm_bwd")
    ld_dres = hidden
    if dres is not None:
        if dres.shape != s.shape:
            raise ValueError("dres must have s's shape")
        _, _, ld_dres = _rows(dres, "dres")
    _check(lib().norm_fused_add_rmsnorm_bwd_ex(ds.data_ptr(), ld_ds, dweight.data_ptr(),
                                               dout.data_ptr(), ld_dout,
                                               dres.data_ptr() if dres is not None else None,
                                               ld_dres, s.data_ptr(), ld_s, weight.data_ptr(),
                                               workspace.data_ptr(), wsb, rows, hidden,
                                               float(eps), _cfg_ptr(cfg),
                                               _stream(stream, dout, dres, s, weight, ds,
                                                       dweight, workspace)),
           "norm_fused_add_rmsnorm_bwd")
    return ds, dweight


def select_config(op, rows: int, hidden: int, cu_count: int = 0) -> Cfg:
    op = OPS.get(op, op)
    c = LaunchCfg()
    _check(lib().norm_select_config(int(op), rows, hidden, cu_count, ctypes.byref(c)),
           "norm_select_config")
    return Cfg(*c.astuple())


def describe_config(op, rows: int, hidden: int, cu_count: int = 0) -> str:
    """The launch the library would make, as text (kernel, lanes, grid, ...)."""
    op = OPS.get(op, op)
    n = lib().norm_describe_config(int(op), rows, hidden, cu_count, None, 0)
    if n < 0:
        raise NormError(1, f"norm_describe_config: invalid arguments ({op}, {rows}, {hidden})")
    buf = ctypes.create_string_buffer(n + 1)
    lib().norm_describe_config(int(op), rows, hidden, cu_count, buf, n + 1)
    return buf.value.decode()


def list_configs(op, hidden: int):
    op = OPS.get(op, op)
    n = lib().norm_list_configs(int(op), hidden, None, 0)
    arr = (LaunchCfg * max(n, 1))()
    lib().norm_list_configs(int(op), hidden, arr, n)
    return [Cfg(*arr[i].astuple()) for i in range(n)]


# ---- fp32 activations -----------------------------------------------------------
# Contiguous fp32 tensors throughout; the library requires hidden % 4 == 0 and
# 16-byte-aligned matrices and weight / bias vectors (it reports a violation).
def _f32_rows(x, name):
    _mat(x, name, torch.float32)
    return _rows_hidden(x)


def _f32_same(t, ref, name):
    _mat(t, name, torch.float32)
    if t.shape != ref.shape:
        raise ValueError(f"{name} must have shape {tuple(ref.shape)}")
    return t


def _f32_out(t, ref, name):
    return _f32_same(torch.empty_like(ref) if t is None else t, ref, name)


def _f32_colsum(t, hidden, name, device):
    t = torch.empty(hidden, dtype=torch.float32, device=device) if t is None else t
    return _vec(t, hidden, name, torch.float32)


def fused_add_rmsnorm_f32(x, residual, weight, eps: float, out=None, stream=None):
    """fp32 fused_add_rmsnorm: residual <- x + residual (fp32) in place;
    returns (out, residual)."""
    rows, hidden = _f32_rows(x, "x")
    _f32_same(residual, x, "residual")
    _vec(weight, hidden, "weight", torch.float32)
    out = _f32_out(out, x, "out")
    _check(lib().norm_fused_add_rmsnorm_f32(out.data_ptr(), residual.data_ptr(), x.data_ptr(),
                                            weight.data_ptr(), rows, hidden, float(eps),
                                            _stream(stream, x, residual, weight, out)),
           "norm_fused_add_rmsnorm_f32")
    return out, residual


def rmsnorm_fwd_f32(x, weight, eps: float, out=None, stream=None):
    rows, hidden = _f32_rows(x, "x")
    _vec(weight, hidden, "weight", torch.float32)
    out = _f32_out(out, x, "out")
    _check(lib().norm_rmsnorm_fwd_f32(out.data_ptr(), x.data_ptr(), weight.data_ptr(), rows,
                                      hidden, float(eps), _stream(stream, x, weight, out)),
           "norm_rmsnorm_fwd_f32")
    return out


def layernorm_fwd_f32(x, weight, bias, eps: float, y=None, mean=None, rstd=None,
                      with_stats: bool = True, stream=None):
    """Returns (y, mean, rstd); mean/rstd are None when with_stats is False."""
    rows, hidden = _f32_rows(x, "x")
    _vec(weight, hidden, "weight", torch.float32)
    _vec(bias, hidden, "bias", torch.float32)
    y = _f32_out(y, x, "y")
    if with_stats:
        mean = torch.empty(rows, dtype=torch.float32, device=x.device) if mean is None else mean
        rstd = torch.empty(rows, dtype=torch.float32, device=x.device) if rstd is None else rstd
        _mat(mean, "mean", torch.float32)
        _mat(rstd, "rstd", torch.float32)
        if mean.numel() != rows or rstd.numel() != rows:
            raise ValueError("mean/rstd must hold one value per row")
        mp, rp = mean.data_ptr(), rstd.data_ptr()
    else:
        mean = rstd = None
        mp = rp = None
    _check(lib().norm_layernorm_fwd_f32(y.data_ptr(), mp, rp, x.data_ptr(), weight.data_ptr(),
                                        bias.data_ptr(), rows, hidden, float(eps),
                                        _stream(stream, x, weight, bias, y, mean, rstd)),
           "norm_layernorm_fwd_f32")
    return y, mean, rstd


def workspace_bytes_f32(op, rows: int, hidden: int) -> int:
    """Workspace bytes of an fp32 backward op."""
    return int(lib().norm_bwd_workspace_bytes_f32(int(OPS.get(op, op)), rows, hidden))


def _f32_ws(workspace, op, rows, hidden, device):
    if workspace is None:
        workspace = torch.empty(max(workspace_bytes_f32(op, rows, hidden), 16),
                                dtype=torch.uint8, device=device)
    _mat(workspace, "workspace", workspace.dtype)
    return workspace, workspace.numel() * workspace.element_size()


def layernorm_bwd_f32(dy, x, mean, rstd, weight, eps: float = 0.0, dx=None, dweight=None,
                      dbias=None, workspace=None, stream=None):
    """Returns (dx, dweight, dbias)."""
    rows, hidden = _f32_rows(x, "x")
    _f32_same(dy, x, "dy")
    _vec(weight, hidden, "weight", torch.float32)
    _mat(mean, "mean", torch.float32)
    _mat(rstd, "rstd", torch.float32)
    if mean.numel() != rows or rstd.numel() != rows:
        raise ValueError("mean/rstd must hold one value per row")
    dx = _f32_out(dx, x, "dx")
    dweight = _f32_colsum(dweight, hidden, "dweight", x.device)
    dbias = _f32_colsum(dbias, hidden, "dbias", x.device)
    workspace, wsb = _f32_ws(workspace, "layernorm_bwd", rows, hidden, x.device)
    _check(lib().norm_layernorm_bwd_f32(dx.data_ptr(), dweight.data_ptr(), dbias.data_ptr(),
                                        dy.data_ptr(), x.data_ptr(), mean.data_ptr(),
                                        rstd.data_ptr(), weight.data_ptr(), workspace.data_ptr(),
                                        wsb, rows, hidden, float(eps),
                                        _stream(stream, dy, x, mean, rstd, weight, dx, dweight,
                                                dbias, workspace)),
           "norm_layernorm_bwd_f32")
    return dx, dweight, dbias


def rmsnorm_bwd_f32(dy, x, weight, eps: float, dx=None, dweight=None, workspace=None,
                    stream=None):
    """Returns (dx, dweight); rstd is recomputed from x with eps."""
    rows, hidden = _f32_rows(x, "x")
    _f32_same(dy, x, "dy")
    _vec(weight, hidden, "weight", torch.float32)
    dx = _f32_out(dx, x, "dx")
    dweight = _f32_colsum(dweight, hidden, "dweight", x.device)
    workspace, wsb = _f32_ws(workspace, "rmsnorm_bwd", rows, hidden, x.device)
    _check(lib().norm_rmsnorm_bwd_f32(dx.data_ptr(), dweight.data_ptr(), dy.data_ptr(),
                                      x.data_ptr(), weight.data_ptr(), workspace.data_ptr(), wsb,
                                      rows, hidden, float(eps),
                                      _stream(stream, dy, x, weight, dx, dweight, workspace)),
           "norm_rmsnorm_bwd_f32")
    return dx, dweight


def fused_add_rmsnorm_bwd_f32(dout, s, weight, eps: float, dres=None, ds=None, dweight=None,
                              workspace=None, stream=None):
    """Backward of fused_add_rmsnorm_f32 at its residual output s: returns
    (ds, dweight)."""
    rows, hidden = _f32_rows(s, "s")
    _f32_same(dout, s, "dout")
    if dres is not None:
        _f32_same(dres, s, "dres")
    _vec(weight, hidden, "weight", torch.float32)
    ds = _f32_out(ds, s, "ds")
    dweight = _f32_colsum(dweight, hidden, "dweight", s.device)
    workspace, wsb = _f32_ws(workspace, "fused_add_rmsnorm_bwd", rows, hidden, s.device)
    _check(lib().norm_fused_add_rmsnorm_bwd_f32(ds.data_ptr(), dweight.data_ptr(),
                                                dout.data_ptr(),
                                                dres.data_ptr() if dres is not None else None,
                                                s.data_ptr(), weight.data_ptr(),
                                                workspace.data_ptr(), wsb, rows, hidden,
                                                float(eps),
                                                _stream(stream, dout, dres, s, weight, ds,
                                                        dweight, workspace)),
           "norm_fused_add_rmsnorm_bwd_f32")
    return ds, dweight
