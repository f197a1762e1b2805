"""Python front end of the fp64 CPU oracle (``rmsnorm_oracle.c``).

TEST INFRASTRUCTURE ONLY.  The product path (the HIP library and its binding)
never imports this module; only the tests, the smoke check and the
benchmark's CPU-baseline leg do.  It imports nothing from the product
package.

Inputs are torch CPU tensors or numpy arrays in a storage dtype (float32,
float16, bfloat16).  They are widened exactly to fp64 here; every result is
the unrounded fp64 value (callers round with :func:`round_to` when they need
the storage-dtype value).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rmsnorm_oracle.c")
_LIB = os.path.join(_HERE, "librmsnorm_oracle.so")
_lock = threading.Lock()
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def build(force: bool = False) -> str:
    """Compile the oracle with the host C compiler (plain -O2, no vector
    intrinsics, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off",
                               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path: str):
    lib = ctypes.CDLL(path)
    i64, dbl = ctypes.c_int64, ctypes.c_double
    lib.orc_rmsnorm_fwd.argtypes = [i64, i64, _dp, _dp, dbl, dbl, _dp, _dp]
    lib.orc_fused_add_rmsnorm_fwd.argtypes = [i64, i64, _dp, _dp, _dp, dbl, dbl, _dp, _dp]
    lib.orc_rmsnorm_vjp.argtypes = [i64, i64, _dp, _dp, _dp, dbl, dbl, _dp, _dp]
    lib.orc_fused_add_rmsnorm_vjp.argtypes = [i64, i64, _dp, _dp, _dp, _dp, dbl, dbl, _dp, _dp]
    lib.orc_silu_gate.argtypes = [i64, i64, _dp, _dp]
    lib.orc_silu_gate_vjp.argtypes = [i64, i64, _dp, _dp, _dp]
    lib.orc_round_array.argtypes = [ctypes.c_int, i64, _dp, _dp]
    for name in ("orc_round_f16", "orc_round_bf16", "orc_round_f32"):
        getattr(lib, name).argtypes = [dbl]
        getattr(lib, name).restype = dbl
    for name in ("orc_rmsnorm_fwd", "orc_fused_add_rmsnorm_fwd", "orc_rmsnorm_vjp",
                 "orc_fused_add_rmsnorm_vjp", "orc_silu_gate", "orc_silu_gate_vjp", "orc_round_array"):
        getattr(lib, name).restype = None
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            _lib = _bind(build())
    return _lib


def swap_library(path):
    """Test hook: route every oracle call through the library at `path`
    (a deliberately mutated build, to show that the pins catch mistakes);
    ``None`` restores the real oracle.  Returns nothing."""
    global _lib
    with _lock:
        _lib = _bind(path) if path is not None else None


def widen(a) -> np.ndarray:
    """Exact widening of a storage-dtype tensor/array to a C-contiguous fp64
    numpy array.  bfloat16 torch tensors are widened through their bit
    pattern (a bf16 value is the top half of an fp32 with the same bits)."""
    try:
        import torch
    except ImportError:  # pragma: no cover
        torch = None
    if torch is not None and isinstance(a, torch.Tensor):
        a = a.detach().cpu()
        if a.dtype == torch.bfloat16:
            bits = a.contiguous().view(torch.int16).numpy().astype(np.uint16)
            a = (bits.astype(np.uint32) << 16).view(np.float32)
        else:
            a = a.numpy()
    a = np.asarray(a)
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def _check2d(x: np.ndarray):
    if x.ndim != 2:
        raise ValueError("expected a [rows, D] array")
    return x.shape


def rmsnorm_fwd(x, w, eps: float, weight_bias: float):
    """y = x * rsqrt(mean(x^2) + eps) * (weight_bias + w), fp64.
    Returns (y, rstd).  eps and weight_bias are taken as fp32 scalars (the
    precision the library's interface carries), widened to fp64."""
    x = widen(x)
    w = widen(w)
    rows, D = _check2d(x)
    y = np.empty_like(x)
    rstd = np.empty(rows, dtype=np.float64)
    _load().orc_rmsnorm_fwd(rows, D, _p(x), _p(w), float(np.float32(eps)),
                            float(np.float32(weight_bias)), _p(y), _p(rstd))
    return y, rstd


def fused_add_rmsnorm_fwd(x, residual, w, eps: float, weight_bias: float):
    """Returns (normed, new_residual) in fp64, new_residual unrounded."""
    x = widen(x)
    res = widen(residual)
    w = widen(w)
    rows, D = _check2d(x)
    normed = np.empty_like(x)
    newres = np.empty_like(x)
    _load().orc_fused_add_rmsnorm_fwd(rows, D, _p(x), _p(res), _p(w), float(np.float32(eps)),
                                      float(np.float32(weight_bias)), _p(normed), _p(newres))
    return normed, newres


def rmsnorm_vjp(x, w, dy, eps: float, weight_bias: float):
    """Returns (dx, dw) in fp64; dw is summed over every row."""
    x = widen(x)
    w = widen(w)
    dy = widen(dy)
    rows, D = _check2d(x)
    dx = np.empty_like(x)
    dw = np.empty(D, dtype=np.float64)
    _load().orc_rmsnorm_vjp(rows, D, _p(x), _p(w), _p(dy), float(np.float32(eps)),
                            float(np.float32(weight_bias)), _p(dx), _p(dw))
    return dx, dw


def fused_add_rmsnorm_vjp(h, w, dy, d_new_residual, eps: float, weight_bias: float):
    """Backward of the fused form: returns (dh, dw) in fp64, where dh is the
    gradient reaching h = x + residual (and so both x and residual)."""
    h = widen(h)
    w = widen(w)
    dy = widen(dy)
    dr = widen(d_new_residual)
    rows, D = _check2d(h)
    dh = np.empty_like(h)
    dw = np.empty(D, dtype=np.float64)
    _load().orc_fused_add_rmsnorm_vjp(rows, D, _p(h), _p(w), _p(dy), _p(dr), float(np.float32(eps)),
                                      float(np.float32(weight_bias)), _p(dh), _p(dw))
    return dh, dw


def silu_gate(x):
    """y = silu(x[:, :d]) * x[:, d:2d] for x of shape [rows, 2d]; fp64."""
    x = widen(x)
    rows, two_d = _check2d(x)
    if two_d % 2:
        raise ValueError("last axis must be even (2d)")
    d = two_d // 2
    y = np.empty((rows, d), dtype=np.float64)
    _load().orc_silu_gate(rows, d, _p(x), _p(y))
    return y


def silu_gate_vjp(x, dy):
    """Gradient [rows, 2d] of sum(dy * silu_gate(x)) with respect to x; fp64."""
    x, dy = widen(x), widen(dy)
    rows, two_d = _check2d(x)
    if two_d % 2 or dy.shape != (rows, two_d // 2):
        raise ValueError("x must be [rows, 2d] and dy [rows, d]")
    dx = np.empty((rows, two_d), dtype=np.float64)
    _load().orc_silu_gate_vjp(rows, two_d // 2, _p(x), _p(dy), _p(dx))
    return dx


_KIND = {"float32": 0, "float16": 1, "bfloat16": 2}


def round_to(a, dtype: str) -> np.ndarray:
    """Round fp64 values to the nearest value of `dtype` (ties to even),
    directly from fp64; the result is returned as fp64."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    out = np.empty_like(a)
    _load().orc_round_array(_KIND[dtype], a.size, _p(a), _p(out))
    return out


def round_scalar(v: float, dtype: str) -> float:
    lib = _load()
    return {"float32": lib.orc_round_f32, "float16": lib.orc_round_f16,
            "bfloat16": lib.orc_round_bf16}[dtype](float(v))
