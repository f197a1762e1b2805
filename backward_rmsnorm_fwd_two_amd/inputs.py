"""Seeded synthetic inputs for the RMSNorm workloads.

This module only draws random numbers and casts them to a storage dtype; it
holds none of RMSNorm's arithmetic, and it is the one module that both the
GPU path's callers (tests, benchmark) and the oracle's callers use.

Recipe (identical for every workload):
  * ``numpy.random.default_rng(seed)``; tensors are drawn in the order the
    workload lists them, each in chunks of 1024 rows (the stream is consumed
    in row-major order, so the chunk size does not change the values);
  * draws are made in float32 (``rng.random`` / ``rng.standard_normal`` with
    ``dtype=float32``); U(a, b) = a + (b - a) * u and N(0, s) = s * z are
    formed in float32;
  * the float32 values are cast to the storage dtype by torch (round to
    nearest, ties to even).  N(mu, s) takes s as the standard deviation.

Workloads (shapes and distributions of the pages' benchmarks):
  * ``poc_small``    fp32  x[64,512], w[512], dy[64,512] ~ U(0,1), eps 1e-5
  * ``poc_8192x4096`` fp16 x[8192,4096], w[4096], dy ~ U(0,1), eps 1e-5 --
    the tensors of the MLX PR's POC timing script
  * ``decode``       bf16 x, residual [B,H] ~ N(0,1), w[H] ~ N(0,0.1), eps 1e-6
    -- the (batch, hidden) grid of the fused add+RMSNorm microbenchmark
  * ``axis_sweep``   fp16 x, dy [rows,D] ~ N(0,1), w ~ U(0.5,1.5), eps 1e-6 --
    the small-axis band of the CUDA regression report
  * ``prefill``      bf16 x, residual [R,D] ~ N(0,1), dy ~ N(0,0.01),
    w ~ N(0,0.1), weight_bias 1.0, eps 1e-6 -- prefill-scale fused add+norm
    followed by the backward pass
  * ``gate``         x[rows, 2d] ~ N(0,2) (both halves) -- the gated
    activation silu(x[:, :d]) * x[:, d:2d]; d = 14336 is the MLP width of
    the Llama-3 8B model (the decoder family the fused-kernel issue adopts
    first), rows 8192 (prefill chunk) or 1 / 4 / 8 (decode batch)
"""
from __future__ import annotations

import numpy as np
import torch

CHUNK_ROWS = 1024

_TORCH_DTYPES = {
    "float32": torch.float32,
    "float16": torch.float16,
    "bfloat16": torch.bfloat16,
}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPES[name]


def _draw(rng: np.random.Generator, shape, dtype: str, kind: str, a: float, b: float) -> torch.Tensor:
    """Draw a tensor of `shape` chunk by chunk (1024 leading-axis rows per
    chunk).  kind 'u': U(a, b);  kind 'n': N(a, b), b the standard deviation."""
    out = torch.empty(shape, dtype=torch_dtype(dtype))
    flat = out.reshape(-1)
    nrows = shape[0] if len(shape) > 1 else 1
    row_elems = int(np.prod(shape[1:])) if len(shape) > 1 else int(np.prod(shape))
    a32, b32 = np.float32(a), np.float32(b)
    for r0 in range(0, nrows, CHUNK_ROWS):
        r1 = min(nrows, r0 + CHUNK_ROWS)
        n = (r1 - r0) * row_elems
        if kind == "u":
            v = a32 + (b32 - a32) * rng.random(n, dtype=np.float32)
        elif kind == "n":
            v = a32 + b32 * rng.standard_normal(n, dtype=np.float32)
        else:
            raise ValueError(kind)
        flat[r0 * row_elems:r1 * row_elems] = torch.from_numpy(v).to(out.dtype)
    return out


def uniform(rng, shape, lo, hi, dtype):
    return _draw(rng, tuple(shape), dtype, "u", lo, hi)


def normal(rng, shape, mean, std, dtype):
    return _draw(rng, tuple(shape), dtype, "n", mean, std)


def poc_small(seed: int = 0):
    rng = np.random.default_rng(seed)
    x = uniform(rng, (64, 512), 0.0, 1.0, "float32")
    w = uniform(rng, (512,), 0.0, 1.0, "float32")
    dy = uniform(rng, (64, 512), 0.0, 1.0, "float32")
    return dict(x=x, w=w, dy=dy, eps=1e-5, weight_bias=0.0, dtype="float32")


def poc_8192x4096(seed: int = 0, rows: int = 8192, D: int = 4096):
    rng = np.random.default_rng(seed)
    x = uniform(rng, (rows, D), 0.0, 1.0, "float16")
    w = uniform(rng, (D,), 0.0, 1.0, "float16")
    dy = uniform(rng, (rows, D), 0.0, 1.0, "float16")
    return dict(x=x, w=w, dy=dy, eps=1e-5, weight_bias=0.0, dtype="float16")


def decode(B: int, H: int, weight_bias: float, seed: int = 0):
    rng = np.random.default_rng(seed)
    x = normal(rng, (B, H), 0.0, 1.0, "bfloat16")
    res = normal(rng, (B, H), 0.0, 1.0, "bfloat16")
    w = normal(rng, (H,), 0.0, 0.1, "bfloat16")
    return dict(x=x, residual=res, w=w, eps=1e-6, weight_bias=float(weight_bias), dtype="bfloat16")


def axis_sweep(rows: int, D: int, seed: int = 0, dtype: str = "float16"):
    rng = np.random.default_rng(seed)
    x = normal(rng, (rows, D), 0.0, 1.0, dtype)
    dy = normal(rng, (rows, D), 0.0, 1.0, dtype)
    w = uniform(rng, (D,), 0.5, 1.5, dtype)
    return dict(x=x, dy=dy, w=w, eps=1e-6, weight_bias=0.0, dtype=dtype)


def prefill(seed: int = 0, rows: int = 32768, D: int = 8192):
    rng = np.random.default_rng(seed)
    x = normal(rng, (rows, D), 0.0, 1.0, "bfloat16")
    res = normal(rng, (rows, D), 0.0, 1.0, "bfloat16")
    dy = normal(rng, (rows, D), 0.0, 0.01, "bfloat16")
    w = normal(rng, (D,), 0.0, 0.1, "bfloat16")
    return dict(x=x, residual=res, dy=dy, w=w, eps=1e-6, weight_bias=1.0, dtype="bfloat16")


def generic(rows: int, D: int, dtype: str, seed: int = 0, dist: str = "normal"):
    """A generic case for shape sweeps: x, dy ~ N(0,1) (or U(0,1)),
    w ~ U(0.5, 1.5)."""
    rng = np.random.default_rng(seed)
    if dist == "normal":
        x = normal(rng, (rows, D), 0.0, 1.0, dtype)
        dy = normal(rng, (rows, D), 0.0, 1.0, dtype)
    else:
        x = uniform(rng, (rows, D), 0.0, 1.0, dtype)
        dy = uniform(rng, (rows, D), 0.0, 1.0, dtype)
    res = normal(rng, (rows, D), 0.0, 1.0, dtype)
    w = uniform(rng, (D,), 0.5, 1.5, dtype)
    return dict(x=x, dy=dy, residual=res, w=w, eps=1e-6, weight_bias=0.0, dtype=dtype)


def gate(rows: int, d: int, dtype: str = "bfloat16", seed: int = 0, std: float = 2.0):
    rng = np.random.default_rng(seed)
    x = normal(rng, (rows, 2 * d), 0.0, std, dtype)
    return dict(x=x, d=d, dtype=dtype)
