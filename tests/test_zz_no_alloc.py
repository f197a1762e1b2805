"""GPU: rmsnorm_vjp_noalloc -- the VJP with the library's own device scratch
instead of a caller workspace (for callers that cannot allocate).  Called
through the C ABI twice in a row, the second call on a smaller input, each
checked bit for bit against rmsnorm_vjp on the same arguments and against the
fp64 oracle within the usual tolerances; a shape whose partial rows exceed
the scratch is refused before any launch."""
import ctypes
import sys

import numpy as np
import pytest
import torch

from _parity import assert_close, assert_dw_close
from backward_rmsnorm_fwd_two_amd import inputs as I
from oracle import oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _raw_noalloc(R, x, w, dy, dx, dw, eps, wb):
    rows, D = x.shape
    dt = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}[x.dtype]
    stream = ctypes.c_void_p(torch.cuda.current_stream(x.device).cuda_stream)
    return R.raw.rmsnorm_vjp_noalloc(x.data_ptr(), w.data_ptr(), dy.data_ptr(), dx.data_ptr(), dw.data_ptr(),
                                     rows, D, dt, float(eps), float(wb), stream)


# two calls in a row: the headline shape, then a smaller ragged one
CALLS = [("poc 8192x4096 fp16", lambda: I.poc_8192x4096()),
         ("37x1000 bf16", lambda: I.axis_sweep(37, 1000, dtype="bfloat16", seed=5))]


def test_noalloc_matches_vjp_two_calls():
    import backward_rmsnorm_fwd_two_amd as R
    for name, make in CALLS:
        _say(f"noalloc call: {name}")
        c = make()
        x, w, dy = c["x"].to(DEV), c["w"].to(DEV), c["dy"].to(DEV)
        eps, wb = c["eps"], c["weight_bias"]
        dx_ref, dw_ref = R.rmsnorm_vjp(x, w, dy, eps, wb)
        dx = torch.full_like(x, float("nan"))
        dw = torch.full_like(dw_ref, float("nan"))
        assert _raw_noalloc(R, x, w, dy, dx, dw, eps, wb) == 0
        torch.cuda.synchronize()
        assert torch.equal(dx.view(torch.int16 if x.element_size() == 2 else torch.int32),
                           dx_ref.view(torch.int16 if x.element_size() == 2 else torch.int32)), name
        assert torch.equal(dw.view(torch.int32), dw_ref.view(torch.int32)), name
        dxo, dwo = O.rmsnorm_vjp(c["x"], c["w"], c["dy"], eps, wb)
        assert_close(dx, dxo, f"{name} dx")
        assert_dw_close(dw, dwo, f"{name} dw")


def test_noalloc_refuses_shapes_beyond_the_scratch():
    import backward_rmsnorm_fwd_two_amd as R
    # 2048 rows of 32768 bf16 (the streaming kernel, one persistent block per
    # CU): 256 partial rows of 128 KiB, beyond the 16 MiB scratch.  Real
    # buffers (never filled), so that a wrong acceptance could not touch
    # memory outside them.
    rows, D = 2048, 32768
    assert R.rmsnorm_vjp_workspace_bytes(rows, D, torch.bfloat16) > R.RMSN_NOALLOC_SCRATCH_BYTES
    x = torch.empty(rows, D, dtype=torch.bfloat16, device=DEV)
    dy, dx = torch.empty_like(x), torch.empty_like(x)
    w = torch.empty(D, dtype=torch.bfloat16, device=DEV)
    dw = torch.empty(D, dtype=torch.float32, device=DEV)
    _say("noalloc refusal: 2048 x 32768 bf16")
    assert _raw_noalloc(R, x, w, dy, dx, dw, 1e-6, 0.0) == -4  # RMSN_E_WORKSPACE


def test_noalloc_rows_zero_writes_zero_dw():
    import backward_rmsnorm_fwd_two_amd as R
    dw = torch.full((300,), float("nan"), dtype=torch.float32, device=DEV)
    w = torch.ones(300, dtype=torch.float16, device=DEV)
    assert R.raw.rmsnorm_vjp_noalloc(None, w.data_ptr(), None, None, dw.data_ptr(), 0, 300, 1, 1e-5, 0.0,
                                     None) == 0
    torch.cuda.synchronize()
    assert torch.equal(dw.cpu(), torch.zeros(300))
