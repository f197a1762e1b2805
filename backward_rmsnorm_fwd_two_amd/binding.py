"""ctypes binding of the gfx950 RMSNorm library (``librmsnorm_mi355x.so``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory (outputs,
workspace) and the current HIP stream.  There is no fallback path: if the
library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librmsnorm_mi355x.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -m backward_rmsnorm_fwd_two_amd.build` "
        "(or __graft_entry__.build()) first")

# torch is imported first so that its HIP runtime (same soname) is the one
# the library binds to: streams from torch are then valid in the library.
_lib = ctypes.CDLL(LIB_PATH)

RMSN_F32, RMSN_F16, RMSN_BF16 = 0, 1, 2
RMSN_OP_FWD, RMSN_OP_FUSED, RMSN_OP_VJP, RMSN_OP_GRAD, RMSN_OP_FUSED_VJP, RMSN_OP_GATE = 0, 1, 2, 3, 4, 5
RMSN_MAX_D = 1 << 24
RMSN_MAX_GATE_D = 1 << 28
RMSN_NOALLOC_SCRATCH_BYTES = 16 << 20

STATUS = {
    0: "RMSN_OK", -1: "RMSN_E_NULLPTR", -2: "RMSN_E_SHAPE", -3: "RMSN_E_DTYPE",
    -4: "RMSN_E_WORKSPACE", -5: "RMSN_E_OVERLAP", -6: "RMSN_E_HIP", -7: "RMSN_E_ALIGN",
    -8: "RMSN_E_CONFIG",
}

_DT = {torch.float32: RMSN_F32, torch.float16: RMSN_F16, torch.bfloat16: RMSN_BF16}


class Config(ctypes.Structure):
    """Mirror of ``rmsn_config_t`` (0 in a field = automatic)."""
    _fields_ = [
        ("lanes_per_row", ctypes.c_int32),
        ("vecs_per_lane", ctypes.c_int32),
        ("vec_bytes", ctypes.c_int32),
        ("block_threads", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
    ]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_vp, _i64, _int, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_cfgp = ctypes.POINTER(Config)

_lib.rmsnorm_fwd.argtypes = [_vp, _vp, _vp, _i64, _i64, _int, _f32, _f32, _vp]
_lib.rmsnorm_fwd_cfg.argtypes = [_vp, _vp, _vp, _i64, _i64, _int, _f32, _f32, _cfgp, _vp]
_lib.fused_add_rmsnorm_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _int, _f32, _f32, _vp]
_lib.fused_add_rmsnorm_fwd_cfg.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _int, _f32, _f32,
                                           _cfgp, _vp]
_lib.rmsnorm_vjp_workspace_bytes.argtypes = [_i64, _i64, _int]
_lib.rmsnorm_vjp_workspace_bytes.restype = _sz
_lib.rmsnorm_vjp.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64, _int, _f32, _f32, _vp]
_lib.rmsnorm_vjp_cfg.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64, _int, _f32, _f32,
                                 _cfgp, _vp]
_lib.rmsnorm_vjp_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _int, _f32, _f32, _vp]
_lib.rmsnorm_fwd_vjp.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64, _int, _f32, _f32,
                                 _vp]
_lib.rmsnorm_fwd_vjp_cfg.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64, _int, _f32,
                                     _f32, _cfgp, _vp]
_lib.fused_add_rmsnorm_vjp.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64, _int, _f32,
                                       _f32, _vp]
_lib.fused_add_rmsnorm_vjp_cfg.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64, _int,
                                           _f32, _f32, _cfgp, _vp]
_lib.rmsnorm_backward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _vp, _sz, _i64, _i64, _int,
                                  _f32, _f32, _cfgp, _vp]
_lib.silu_gate.argtypes = [_vp, _vp, _i64, _i64, _int, _vp]
_lib.silu_gate_cfg.argtypes = [_vp, _vp, _i64, _i64, _int, _cfgp, _vp]
_lib.silu_gate_vjp.argtypes = [_vp, _vp, _vp, _i64, _i64, _int, _vp]
_lib.silu_gate_vjp_cfg.argtypes = [_vp, _vp, _vp, _i64, _i64, _int, _cfgp, _vp]
_lib.rmsn_query_config.argtypes = [_int, _i64, _i64, _int, _int, _cfgp]
_lib.rmsn_status_str.argtypes = [_int]
_lib.rmsn_status_str.restype = ctypes.c_char_p
for _name in ("rmsnorm_fwd", "rmsnorm_fwd_cfg", "fused_add_rmsnorm_fwd", "fused_add_rmsnorm_fwd_cfg",
              "rmsnorm_vjp", "rmsnorm_vjp_cfg", "rmsnorm_vjp_noalloc", "rmsnorm_fwd_vjp", "rmsnorm_fwd_vjp_cfg",
              "fused_add_rmsnorm_vjp", "fused_add_rmsnorm_vjp_cfg", "silu_gate", "silu_gate_cfg",
              "silu_gate_vjp", "silu_gate_vjp_cfg", "rmsnorm_backward", "rmsn_query_config"):
    getattr(_lib, _name).restype = _int

raw = _lib  # the C functions themselves (pointer-level access for tests)


class RMSNormError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} "
                         f"({_lib.rmsn_status_str(status).decode()})")


def _check(status: int, where: str) -> None:
    if status != 0:
        raise RMSNormError(status, where)


def _stream(t: torch.Tensor):
    """The current stream of t's device, which must be the current device:
    the library plans and launches on the current device."""
    cur = torch.cuda.current_device()
    if t.device.index != cur:
        raise ValueError(f"tensors are on {t.device} but the current device is cuda:{cur}; "
                         "call inside torch.cuda.device(...) of the tensors' device")
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _rows_d(x: torch.Tensor) -> Tuple[int, int]:
    if x.dim() < 1:
        raise ValueError("expected a tensor whose last axis is normalised")
    D = x.shape[-1]
    rows = x.numel() // D if D else 0
    return rows, D


def _req(t: torch.Tensor, name: str, dtype, device, numel=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def _cfg(cfg) -> Optional[ctypes.pointer]:
    if cfg is None:
        return None
    if isinstance(cfg, dict):
        cfg = Config(**cfg)
    return ctypes.pointer(cfg)


def _dt(x: torch.Tensor) -> int:
    if x.dtype not in _DT:
        raise ValueError(f"unsupported dtype {x.dtype}")
    return _DT[x.dtype]


def rmsnorm_fwd(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-5, weight_bias: float = 0.0,
                out: Optional[torch.Tensor] = None, cfg=None) -> torch.Tensor:
    """y = x * rsqrt(mean(x^2, -1) + eps) * (weight_bias + w)."""
    dt = _dt(x)
    rows, D = _rows_d(x)
    _req(x, "x", x.dtype, x.device)
    _req(w, "w", x.dtype, x.device, D)
    if out is None:
        out = torch.empty_like(x)
    _req(out, "out", x.dtype, x.device, x.numel())
    if cfg is None:
        st = _lib.rmsnorm_fwd(x.data_ptr(), w.data_ptr(), out.data_ptr(), rows, D, dt,
                              float(eps), float(weight_bias), _stream(x))
    else:
        st = _lib.rmsnorm_fwd_cfg(x.data_ptr(), w.data_ptr(), out.data_ptr(), rows, D, dt,
                                  float(eps), float(weight_bias), _cfg(cfg), _stream(x))
    _check(st, "rmsnorm_fwd")
    return out


def fused_add_rmsnorm_fwd(x: torch.Tensor, residual: torch.Tensor, w: torch.Tensor,
                          eps: float = 1e-6, weight_bias: float = 0.0,
                          normed: Optional[torch.Tensor] = None,
                          new_residual: Optional[torch.Tensor] = None,
                          cfg=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """new_residual = x + residual; normed = rmsnorm(x + residual) * (weight_bias + w)."""
    dt = _dt(x)
    rows, D = _rows_d(x)
    _req(x, "x", x.dtype, x.device)
    _req(residual, "residual", x.dtype, x.device, x.numel())
    _req(w, "w", x.dtype, x.device, D)
    if normed is None:
        normed = torch.empty_like(x)
    if new_residual is None:
        new_residual = torch.empty_like(x)
    _req(normed, "normed", x.dtype, x.device, x.numel())
    _req(new_residual, "new_residual", x.dtype, x.device, x.numel())
    args = (x.data_ptr(), residual.data_ptr(), w.data_ptr(), normed.data_ptr(),
            new_residual.data_ptr(), rows, D, dt, float(eps), float(weight_bias))
    if cfg is None:
        st = _lib.fused_add_rmsnorm_fwd(*args, _stream(x))
    else:
        st = _lib.fused_add_rmsnorm_fwd_cfg(*args, _cfg(cfg), _stream(x))
    _check(st, "fused_add_rmsnorm_fwd")
    return normed, new_residual


def rmsnorm_vjp_workspace_bytes(rows: int, D: int, dtype: torch.dtype) -> int:
    n = _lib.rmsnorm_vjp_workspace_bytes(int(rows), int(D), _DT[dtype])
    if n == 0:
        raise ValueError("invalid shape for rmsnorm_vjp_workspace_bytes")
    return int(n)


def workspace_for(rows: int, D: int, dtype: torch.dtype, device, cfg=None) -> torch.Tensor:
    """A device workspace large enough for rmsnorm_vjp on this shape (and for
    `cfg`'s grid when one is given)."""
    n = rmsnorm_vjp_workspace_bytes(rows, D, dtype)
    if cfg is not None:
        c = cfg if isinstance(cfg, dict) else cfg.as_dict()
        if c.get("vecs_per_lane", 0) == -2:
            # column split: row statistics [rows, slices, 2] fp32 (a slice is
            # 1024 vectors of at least one element), then the chunks' dw rows
            slices = -(-D // 1024)
            n = max(n, -(-(rows * slices * 8) // 256) * 256 + (c.get("num_blocks", 0) or 1024) * D * 4)
        else:
            nb = c.get("num_blocks", 0) or 2048
            n = max(n, nb * D * 4)
    return torch.empty(n, dtype=torch.uint8, device=device)


def rmsnorm_vjp(x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, eps: float = 1e-5,
                weight_bias: float = 0.0, dx: Optional[torch.Tensor] = None,
                dw: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                cfg=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Returns (dx, dw): dx in x's dtype, dw fp32 summed over every row."""
    dt = _dt(x)
    rows, D = _rows_d(x)
    _req(x, "x", x.dtype, x.device)
    _req(w, "w", x.dtype, x.device, D)
    _req(dy, "dy", x.dtype, x.device, x.numel())
    if dx is None:
        dx = torch.empty_like(x)
    if dw is None:
        dw = torch.empty(D, dtype=torch.float32, device=x.device)
    _req(dx, "dx", x.dtype, x.device, x.numel())
    _req(dw, "dw", torch.float32, x.device, D)
    if workspace is None:
        workspace = workspace_for(rows, D, x.dtype, x.device, cfg)
    _req(workspace, "workspace", workspace.dtype, x.device)
    nbytes = workspace.numel() * workspace.element_size()
    args = (x.data_ptr(), w.data_ptr(), dy.data_ptr(), dx.data_ptr(), dw.data_ptr(),
            workspace.data_ptr(), nbytes, rows, D, dt, float(eps), float(weight_bias))
    if cfg is None:
        st = _lib.rmsnorm_vjp(*args, _stream(x))
    else:
        st = _lib.rmsnorm_vjp_cfg(*args, _cfg(cfg), _stream(x))
    _check(st, "rmsnorm_vjp")
    return dx, dw


def rmsnorm_vjp_noalloc(x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, dx: torch.Tensor,
                        dw: torch.Tensor, eps: float = 1e-5, weight_bias: float = 0.0) -> Tuple[torch.Tensor, torch.Tensor]:
    """rmsnorm_vjp into caller-provided dx and dw (fp32) with the library's own
    device scratch: the call allocates nothing.  Calls that overlap on one
    GPU share that scratch and race."""
    dt = _dt(x)
    rows, D = _rows_d(x)
    _req(x, "x", x.dtype, x.device)
    _req(w, "w", x.dtype, x.device, D)
    _req(dy, "dy", x.dtype, x.device, x.numel())
    _req(dx, "dx", x.dtype, x.device, x.numel())
    _req(dw, "dw", torch.float32, x.device, D)
    st = _lib.rmsnorm_vjp_noalloc(x.data_ptr(), w.data_ptr(), dy.data_ptr(), dx.data_ptr(), dw.data_ptr(),
                                  rows, D, dt, float(eps), float(weight_bias), _stream(x))
    _check(st, "rmsnorm_vjp_noalloc")
    return dx, dw


def prepare(fn_name: str, *args):
    """Marshal the arguments of one C entry point once and return a callable
    that re-issues the call (same tensors, same stream) with no per-call
    Python checks -- for tight loops where the host must stay ahead of the
    GPU.  The tensors must stay alive while the callable is used."""
    fn = getattr(_lib, fn_name)
    conv = []
    for a, t in zip(args, fn.argtypes):
        conv.append(a if isinstance(a, ctypes._SimpleCData) else t(a))

    def call():
        st = fn(*conv)
        if st != 0:
            raise RMSNormError(st, fn_name)
    return call


def prepared_fwd(x, w, out, eps, weight_bias):
    rows, D = _rows_d(x)
    _req(x, "x", x.dtype, x.device)
    _req(w, "w", x.dtype, x.device, D)
    _req(out, "out", x.dtype, x.device, x.numel())
    return prepare("rmsnorm_fwd", x.data_ptr(), w.data_ptr(), out.data_ptr(), rows, D, _dt(x),
                   float(eps), float(weight_bias), _stream(x))


def prepared_fused(x, residual, w, normed, new_residual, eps, weight_bias):
    rows, D = _rows_d(x)
    for t, n in ((x, "x"), (residual, "residual"), (normed, "normed"), (new_residual, "new_residual")):
        _req(t, n, x.dtype, x.device, x.numel())
    _req(w, "w", x.dtype, x.device, D)
    return prepare("fused_add_rmsnorm_fwd", x.data_ptr(), residual.data_ptr(), w.data_ptr(),
                   normed.data_ptr(), new_residual.data_ptr(), rows, D, _dt(x), float(eps),
                   float(weight_bias), _stream(x))


def prepared_vjp(x, w, dy, dx, dw, workspace, eps, weight_bias):
    rows, D = _rows_d(x)
    for t, n in ((x, "x"), (dy, "dy"), (dx, "dx")):
        _req(t, n, x.dtype, x.device, x.numel())
    _req(w, "w", x.dtype, x.device, D)
    _req(dw, "dw", torch.float32, x.device, D)
    nbytes = workspace.numel() * workspace.element_size()
    return prepare("rmsnorm_vjp", x.data_ptr(), w.data_ptr(), dy.data_ptr(), dx.data_ptr(),
                   dw.data_ptr(), workspace.data_ptr(), nbytes, rows, D, _dt(x), float(eps),
                   float(weight_bias), _stream(x))


def rmsnorm_fwd_vjp(x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, eps: float = 1e-5,
                    weight_bias: float = 0.0, y: Optional[torch.Tensor] = None,
                    dx: Optional[torch.Tensor] = None, dw: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None,
                    cfg=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Grad call in one pass: returns (y, dx, dw)."""
    dt = _dt(x)
    rows, D = _rows_d(x)
    _req(x, "x", x.dtype, x.device)
    _req(w, "w", x.dtype, x.device, D)
    _req(dy, "dy", x.dtype, x.device, x.numel())
    y = torch.empty_like(x) if y is None else y
    dx = torch.empty_like(x) if dx is None else dx
    dw = torch.empty(D, dtype=torch.float32, device=x.device) if dw is None else dw
    _req(y, "y", x.dtype, x.device, x.numel())
    _req(dx, "dx", x.dtype, x.device, x.numel())
    _req(dw, "dw", torch.float32, x.device, D)
    if workspace is None:
        workspace = workspace_for(rows, D, x.dtype, x.device, cfg)
    nbytes = workspace.numel() * workspace.element_size()
    args = (x.data_ptr(), w.data_ptr(), dy.data_ptr(), y.data_ptr(), dx.data_ptr(), dw.data_ptr(),
            workspace.data_ptr(), nbytes, rows, D, dt, float(eps), float(weight_bias))
    if cfg is None:
        st = _lib.rmsnorm_fwd_vjp(*args, _stream(x))
    else:
        st = _lib.rmsnorm_fwd_vjp_cfg(*args, _cfg(cfg), _stream(x))
    _check(st, "rmsnorm_fwd_vjp")
    return y, dx, dw


def fused_add_rmsnorm_vjp(h: torch.Tensor, w: torch.Tensor, dy: torch.Tensor,
                          d_new_residual: torch.Tensor, eps: float = 1e-6, weight_bias: float = 0.0,
                          dh: Optional[torch.Tensor] = None, dw: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None,
                          cfg=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Backward of fused_add_rmsnorm_fwd at h = new_residual: returns (dh, dw);
    dh is the gradient of both x and residual."""
    dt = _dt(h)
    rows, D = _rows_d(h)
    _req(h, "h", h.dtype, h.device)
    _req(w, "w", h.dtype, h.device, D)
    _req(dy, "dy", h.dtype, h.device, h.numel())
    _req(d_new_residual, "d_new_residual", h.dtype, h.device, h.numel())
    dh = torch.empty_like(h) if dh is None else dh
    dw = torch.empty(D, dtype=torch.float32, device=h.device) if dw is None else dw
    _req(dh, "dh", h.dtype, h.device, h.numel())
    _req(dw, "dw", torch.float32, h.device, D)
    if workspace is None:
        workspace = workspace_for(rows, D, h.dtype, h.device, cfg)
    nbytes = workspace.numel() * workspace.element_size()
    args = (h.data_ptr(), w.data_ptr(), dy.data_ptr(), d_new_residual.data_ptr(), dh.data_ptr(),
            dw.data_ptr(), workspace.data_ptr(), nbytes, rows, D, dt, float(eps), float(weight_bias))
    if cfg is None:
        st = _lib.fused_add_rmsnorm_vjp(*args, _stream(h))
    else:
        st = _lib.fused_add_rmsnorm_vjp_cfg(*args, _cfg(cfg), _stream(h))
    _check(st, "fused_add_rmsnorm_vjp")
    return dh, dw


def prepared_fused_vjp(h, w, dy, d_new_residual, dh, dw, workspace, eps, weight_bias):
    rows, D = _rows_d(h)
    for t, n in ((h, "h"), (dy, "dy"), (d_new_residual, "d_new_residual"), (dh, "dh")):
        _req(t, n, h.dtype, h.device, h.numel())
    _req(w, "w", h.dtype, h.device, D)
    _req(dw, "dw", torch.float32, h.device, D)
    nbytes = workspace.numel() * workspace.element_size()
    return prepare("fused_add_rmsnorm_vjp", h.data_ptr(), w.data_ptr(), dy.data_ptr(),
                   d_new_residual.data_ptr(), dh.data_ptr(), dw.data_ptr(), workspace.data_ptr(),
                   nbytes, rows, D, _dt(h), float(eps), float(weight_bias), _stream(h))


def prepared_grad(x, w, dy, y, dx, dw, workspace, eps, weight_bias):
    rows, D = _rows_d(x)
    for t, n in ((x, "x"), (dy, "dy"), (y, "y"), (dx, "dx")):
        _req(t, n, x.dtype, x.device, x.numel())
    _req(w, "w", x.dtype, x.device, D)
    _req(dw, "dw", torch.float32, x.device, D)
    nbytes = workspace.numel() * workspace.element_size()
    return prepare("rmsnorm_fwd_vjp", x.data_ptr(), w.data_ptr(), dy.data_ptr(), y.data_ptr(),
                   dx.data_ptr(), dw.data_ptr(), workspace.data_ptr(), nbytes, rows, D, _dt(x),
                   float(eps), float(weight_bias), _stream(x))


def rmsnorm_backward(x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, eps: float = 1e-5,
                     weight_bias: float = 0.0, d_new_residual: Optional[torch.Tensor] = None,
                     y: Optional[torch.Tensor] = None, dx: Optional[torch.Tensor] = None,
                     dw: Optional[torch.Tensor] = None, dw_dtype: Optional[torch.dtype] = None,
                     want_y: bool = False, workspace: Optional[torch.Tensor] = None,
                     cfg=None) -> Tuple[Optional[torch.Tensor], torch.Tensor, torch.Tensor]:
    """The general backward: returns (y or None, dx, dw).  `d_new_residual`
    selects the fused backward (x is then h), `y` / `want_y` the grad call;
    `dw_dtype` is torch.float32 (default) or x's dtype."""
    dt = _dt(x)
    rows, D = _rows_d(x)
    dw_dtype = torch.float32 if dw_dtype is None else dw_dtype
    if dw_dtype not in (torch.float32, x.dtype):
        raise ValueError(f"dw_dtype must be torch.float32 or {x.dtype}")
    _req(x, "x", x.dtype, x.device)
    _req(w, "w", x.dtype, x.device, D)
    _req(dy, "dy", x.dtype, x.device, x.numel())
    if d_new_residual is not None:
        _req(d_new_residual, "d_new_residual", x.dtype, x.device, x.numel())
    if y is None and want_y:
        y = torch.empty_like(x)
    if y is not None:
        _req(y, "y", x.dtype, x.device, x.numel())
    if dx is None:
        dx = torch.empty_like(x)
    if dw is None:
        dw = torch.empty(D, dtype=dw_dtype, device=x.device)
    _req(dx, "dx", x.dtype, x.device, x.numel())
    _req(dw, "dw", dw_dtype, x.device, D)
    if workspace is None:
        workspace = workspace_for(rows, D, x.dtype, x.device, cfg)
    _req(workspace, "workspace", workspace.dtype, x.device)
    nbytes = workspace.numel() * workspace.element_size()
    st = _lib.rmsnorm_backward(x.data_ptr(), w.data_ptr(), dy.data_ptr(),
                               None if d_new_residual is None else d_new_residual.data_ptr(),
                               None if y is None else y.data_ptr(), dx.data_ptr(), dw.data_ptr(),
                               _DT[dw_dtype], workspace.data_ptr(), nbytes, rows, D, dt, float(eps),
                               float(weight_bias), _cfg(cfg), _stream(x))
    _check(st, "rmsnorm_backward")
    return y, dx, dw


def silu_gate(x: torch.Tensor, out: Optional[torch.Tensor] = None, cfg=None) -> torch.Tensor:
    """y = silu(x[..., :d]) * x[..., d:2d] for x of last axis 2d; y has last axis d."""
    dt = _dt(x)
    rows, two_d = _rows_d(x)
    if two_d % 2:
        raise ValueError("the last axis of x must be even (2d)")
    d = two_d // 2
    _req(x, "x", x.dtype, x.device)
    if out is None:
        out = torch.empty(tuple(x.shape[:-1]) + (d,), dtype=x.dtype, device=x.device)
    _req(out, "out", x.dtype, x.device, rows * d)
    if cfg is None:
        st = _lib.silu_gate(x.data_ptr(), out.data_ptr(), rows, d, dt, _stream(x))
    else:
        st = _lib.silu_gate_cfg(x.data_ptr(), out.data_ptr(), rows, d, dt, _cfg(cfg), _stream(x))
    _check(st, "silu_gate")
    return out


def silu_gate_vjp(x: torch.Tensor, dy: torch.Tensor, out: Optional[torch.Tensor] = None,
                  cfg=None) -> torch.Tensor:
    """Gradient of sum(dy * silu_gate(x)) with respect to x (x's shape)."""
    dt = _dt(x)
    rows, two_d = _rows_d(x)
    if two_d % 2:
        raise ValueError("the last axis of x must be even (2d)")
    d = two_d // 2
    _req(x, "x", x.dtype, x.device)
    _req(dy, "dy", x.dtype, x.device, rows * d)
    if out is None:
        out = torch.empty_like(x)
    _req(out, "out", x.dtype, x.device, x.numel())
    if cfg is None:
        st = _lib.silu_gate_vjp(x.data_ptr(), dy.data_ptr(), out.data_ptr(), rows, d, dt, _stream(x))
    else:
        st = _lib.silu_gate_vjp_cfg(x.data_ptr(), dy.data_ptr(), out.data_ptr(), rows, d, dt, _cfg(cfg),
                                    _stream(x))
    _check(st, "silu_gate_vjp")
    return out


def prepared_gate_vjp(x, dy, out):
    rows, two_d = _rows_d(x)
    _req(x, "x", x.dtype, x.device)
    _req(dy, "dy", x.dtype, x.device, rows * (two_d // 2))
    _req(out, "out", x.dtype, x.device, x.numel())
    return prepare("silu_gate_vjp", x.data_ptr(), dy.data_ptr(), out.data_ptr(), rows, two_d // 2, _dt(x),
                   _stream(x))


def prepared_gate(x, out):
    rows, two_d = _rows_d(x)
    _req(x, "x", x.dtype, x.device)
    _req(out, "out", x.dtype, x.device, rows * (two_d // 2))
    return prepare("silu_gate", x.data_ptr(), out.data_ptr(), rows, two_d // 2, _dt(x), _stream(x))


def query_config(op: int, rows: int, D: int, dtype: torch.dtype, align_bytes: int = 16) -> dict:
    """The configuration the automatic choice makes for this shape."""
    c = Config()
    _check(_lib.rmsn_query_config(op, int(rows), int(D), _DT[dtype], int(align_bytes),
                                  ctypes.byref(c)), "rmsn_query_config")
    return c.as_dict()
