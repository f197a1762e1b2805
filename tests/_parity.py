"""Comparison rules shared by the GPU parity tests.

The reference value is the oracle's unrounded fp64 result.  For each output
element the error measure is |out - ref| / max(1, |ref|):
  fp32 outputs          <= 1e-5
  fp16 / bf16 outputs   <= 4e-3
  dw (fp32, [D])        max_j |dw_j - ref_j| <= 1e-3 * max_j |ref_j|
NaN must sit exactly where the reference has NaN, and infinities must match
exactly.  Outputs are widened to fp64 with torch's exact conversions.
"""
from __future__ import annotations

import numpy as np
import torch

TOL = {torch.float32: 1e-5, torch.float16: 4e-3, torch.bfloat16: 4e-3}
DW_TOL = 1e-3


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def rel_err(out: np.ndarray, ref: np.ndarray) -> np.ndarray:
    with np.errstate(invalid="ignore"):
        return np.abs(out - ref) / np.maximum(1.0, np.abs(ref))


def assert_close(out_t: torch.Tensor, ref: np.ndarray, what: str, tol: float = None):
    tol = TOL[out_t.dtype] if tol is None else tol
    out = to64(out_t).reshape(ref.shape)
    nan_ref = np.isnan(ref)
    nan_out = np.isnan(out)
    assert np.array_equal(nan_ref, nan_out), f"{what}: NaN positions differ ({nan_ref.sum()} vs {nan_out.sum()})"
    inf_ref = np.isinf(ref)
    assert np.array_equal(out[inf_ref], ref[inf_ref]) and np.array_equal(np.isinf(out), inf_ref), \
        f"{what}: infinities differ"
    fin = np.isfinite(ref)
    if fin.any():
        err = rel_err(out[fin], ref[fin])
        worst = float(err.max())
        assert worst <= tol, f"{what}: max err {worst:.3e} > {tol:.1e} (at flat index {int(np.argmax(err))})"
        return worst
    return 0.0


def assert_dw_close(dw_t: torch.Tensor, ref: np.ndarray, what: str = "dw", tol: float = DW_TOL):
    assert dw_t.dtype == torch.float32
    dw = to64(dw_t)
    assert np.array_equal(np.isnan(dw), np.isnan(ref)), f"{what}: NaN positions differ"
    fin = np.isfinite(ref)
    scale = float(np.max(np.abs(ref[fin]))) if fin.any() else 0.0
    err = float(np.max(np.abs(dw[fin] - ref[fin]))) if fin.any() else 0.0
    assert err <= tol * max(scale, 1e-30), f"{what}: max |err| {err:.3e} > {tol:.0e} * {scale:.3e}"
    return err / max(scale, 1e-30)


def ulp_report(out_t: torch.Tensor, ref: np.ndarray, rounded: np.ndarray) -> dict:
    """Informational: how many outputs differ from the round-to-nearest-even
    of the reference (`rounded`, the oracle's own rounding), and by how many
    units in the last place at most (ulps counted on the storage format's bit
    patterns; fp16/bf16/fp32 are sign-magnitude, so patterns are mapped to a
    monotone integer line first)."""
    out = out_t.detach().cpu().contiguous()
    bits = {torch.float16: torch.int16, torch.bfloat16: torch.int16, torch.float32: torch.int32}[out.dtype]
    ro = torch.from_numpy(np.ascontiguousarray(rounded)).to(out.dtype)

    def line(t):
        i = t.view(bits).to(torch.int64)
        sign_bit = 1 << (8 * t.element_size() - 1)
        mag = i & (sign_bit - 1)
        return torch.where(i < 0, -mag, mag)

    d = (line(out) - line(ro)).abs().reshape(-1)
    fin = torch.from_numpy(np.isfinite(ref).reshape(-1))
    d = d[fin]
    return {"n": int(d.numel()), "differ": int((d != 0).sum()), "max_ulp": int(d.max()) if d.numel() else 0}
