"""GPU: the general backward entry point rmsnorm_backward -- the VJP, the
grad call and the fused backward through one call, with dw in fp32 or in the
weight dtype (rounded once from the fp32 sum).  Checks: outputs bit-identical
to the dedicated entry points; dw in the weight dtype equal to the
round-to-nearest-even of the fp32 dw and within the oracle's tolerance plus
half an ulp of that dtype; one-block grids (staged through the workspace),
the streaming kernel, rows = 0, and the error codes."""
import ctypes
import sys

import numpy as np
import pytest
import torch

from _parity import DW_TOL, assert_close, to64
from backward_rmsnorm_fwd_two_amd import inputs as I
from oracle import oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
# unit roundoff (half an ulp, relative) of the storage formats
UNIT_ROUNDOFF = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8, torch.float32: 2.0 ** -24}


@pytest.fixture(scope="module")
def R():
    import backward_rmsnorm_fwd_two_amd as pkg
    return pkg


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def assert_typed_dw_close(dw_t, ref, what="dw"):
    """dw stored in a 16-bit dtype: |dw - ref| <= 1e-3 * max|ref| + u * |ref|."""
    dw = to64(dw_t)
    u = UNIT_ROUNDOFF[dw_t.dtype]
    scale = float(np.max(np.abs(ref)))
    err = np.abs(dw - ref)
    bound = DW_TOL * scale + u * np.abs(ref)
    assert np.all(err <= bound), f"{what}: worst excess {float(np.max(err - bound)):.3e}"


CASES = [
    (8192, 4096, "float16", None),
    (37, 1000, "bfloat16", None),
    (3, 64, "bfloat16", None),                       # one-block grid
    (40, 512, "float16", dict(num_blocks=1)),        # forced one-block grid
    (2, 70000, "bfloat16", None),                    # streaming kernel
    (9, 300, "float32", None),                       # fp32: dw_dt = dt = fp32
]


def _id(c):
    return f"{c[0]}x{c[1]}-{c[2]}" + ("-grid1" if c[3] else "")


@pytest.mark.parametrize("case", CASES, ids=_id)
@pytest.mark.parametrize("mode", ["vjp", "grad", "fused"])
def test_backward_matches_dedicated_calls(R, case, mode):
    rows, D, dtype, cfg = case
    _say(f"rmsnorm_backward {mode} {rows}x{D} {dtype} cfg={cfg}")
    c = I.generic(rows, D, dtype, seed=rows + 3 * D)
    x, w, dy, dr = (c[k].to(DEV) for k in ("x", "w", "dy", "residual"))
    eps, wb = c["eps"], (1.0 if mode == "fused" else 0.0)
    tdt = x.dtype
    if mode == "vjp":
        dx0, dw0 = R.rmsnorm_vjp(x, w, dy, eps, wb, cfg=cfg)
        y0 = None
    elif mode == "grad":
        y0, dx0, dw0 = R.rmsnorm_fwd_vjp(x, w, dy, eps, wb, cfg=cfg)
    else:
        dx0, dw0 = R.fused_add_rmsnorm_vjp(x, w, dy, dr, eps, wb, cfg=cfg)
        y0 = None
    kw = dict(d_new_residual=dr if mode == "fused" else None, want_y=mode == "grad", cfg=cfg)
    y1, dx1, dw1 = R.rmsnorm_backward(x, w, dy, eps, wb, **kw)
    y2, dx2, dw2 = R.rmsnorm_backward(x, w, dy, eps, wb, dw_dtype=tdt, **kw)
    torch.cuda.synchronize()
    assert torch.equal(dx1, dx0) and torch.equal(dx2, dx0)
    assert torch.equal(dw1, dw0)
    if y0 is not None:
        assert torch.equal(y1, y0) and torch.equal(y2, y0)
    assert dw2.dtype == tdt
    # the weight-dtype dw is the fp32 sum rounded once (RNE, as torch's cast)
    assert torch.equal(dw2, dw0.to(tdt))
    if mode == "fused":
        _, dwref = O.fused_add_rmsnorm_vjp(c["x"], c["w"], c["dy"], c["residual"], eps, wb)
    else:
        _, dwref = O.rmsnorm_vjp(c["x"], c["w"], c["dy"], eps, wb)
    assert_typed_dw_close(dw2, dwref)


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_backward_rows_zero_typed_dw(R, dtype):
    tdt = I.torch_dtype(dtype)
    x = torch.empty(0, 333, dtype=tdt, device=DEV)
    w = torch.ones(333, dtype=tdt, device=DEV)
    dw = torch.full((333,), float("nan"), dtype=tdt, device=DEV)
    R.rmsnorm_backward(x, w, x, dw=dw, dw_dtype=tdt)
    torch.cuda.synchronize()
    assert torch.all(dw == 0)


def test_backward_error_codes(R):
    lib = R.raw
    x = torch.zeros(4, 64, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(64, dtype=torch.bfloat16, device=DEV)
    dx = torch.empty_like(x)
    y = torch.empty_like(x)
    dwb = torch.empty(65, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: t.data_ptr()
    args = lambda dnr, yy, dw, dwdt, wsp, wsn: (p(x), p(w), p(x), dnr, yy, p(dx), dw, dwdt, wsp, wsn,
                                               4, 64, 2, 1e-5, 0.0, None, s)
    assert lib.rmsnorm_backward(*args(None, None, p(dwb), 2, p(ws), ws.numel())) == 0
    assert lib.rmsnorm_backward(*args(None, None, p(dwb), 1, p(ws), ws.numel())) == -3   # fp16 dw, bf16 x
    assert lib.rmsnorm_backward(*args(p(x), p(y), p(dwb), 2, p(ws), ws.numel())) == -8   # y and d_new_residual
    assert lib.rmsnorm_backward(*args(None, None, p(dwb) + 1, 2, p(ws), ws.numel())) == -7
    assert lib.rmsnorm_backward(*args(None, None, p(dwb), 2, None, 0)) == -4             # staged sum needs a workspace
    assert lib.rmsnorm_backward(*args(None, None, None, 2, p(ws), ws.numel())) == -1
    torch.cuda.synchronize()
    with pytest.raises(ValueError):
        R.rmsnorm_backward(x, w, x, dw_dtype=torch.float16)
