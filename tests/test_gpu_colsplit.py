"""GPU: the column-split backward forms -- a statistics kernel over (column
slice, row) blocks and an apply kernel over (column tile, row chunk) blocks,
taken automatically for few rows of a wide D and forced with vecs_per_lane =
-2 at any shape.  Every form is compared with the fp64 oracle on every
element: forced at small shapes (ragged slices and tiles, one row, chunks
that do not divide the rows, narrow loads), automatic at wide rows, with dw
in the weight dtype, in place, repeated bitwise, and through the exact
workspace size the library reports."""
import sys

import numpy as np
import pytest
import torch

from _parity import assert_close, assert_dw_close, to64
from backward_rmsnorm_fwd_two_amd import inputs as I
from oracle import oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def R():
    import backward_rmsnorm_fwd_two_amd as pkg
    return pkg


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check(R, rows, D, dtype, seed, cfg, wb=1.0):
    c = I.generic(rows, D, dtype, seed=seed)
    rng = np.random.default_rng(seed)
    dr = I.normal(rng, (rows, D), 0.0, 0.5, dtype)
    xg, wg, dyg, drg = c["x"].to(DEV), c["w"].to(DEV), c["dy"].to(DEV), dr.to(DEV)
    eps = c["eps"]
    what = f"{dtype} {rows}x{D} cfg={cfg}"
    dx, dw = R.rmsnorm_vjp(xg, wg, dyg, eps, wb, cfg=cfg)
    gy, gdx, gdw = R.rmsnorm_fwd_vjp(xg, wg, dyg, eps, wb, cfg=cfg)
    dh, hdw = R.fused_add_rmsnorm_vjp(xg, wg, dyg, drg, eps, wb, cfg=cfg)
    torch.cuda.synchronize()
    yref, _ = O.rmsnorm_fwd(c["x"], c["w"], eps, wb)
    dxref, dwref = O.rmsnorm_vjp(c["x"], c["w"], c["dy"], eps, wb)
    dhref, hdwref = O.fused_add_rmsnorm_vjp(c["x"], c["w"], c["dy"], dr, eps, wb)
    assert_close(dx, dxref, f"{what} dx")
    assert_dw_close(dw, dwref, f"{what} dw")
    assert_close(gy, yref, f"{what} grad y")
    assert_close(gdx, dxref, f"{what} grad dx")
    assert_dw_close(gdw, dwref, f"{what} grad dw")
    assert_close(dh, dhref, f"{what} dh")
    assert_dw_close(hdw, hdwref, f"{what} fused dw")
    return c, (dx, dw)


@pytest.mark.parametrize("rows,D,dtype,chunks", [
    (1, 4096, "bfloat16", 0), (7, 5000, "float16", 3), (33, 3000, "float32", 5), (64, 8192, "bfloat16", 0),
    (100, 1000, "float16", 7), (5, 7, "float16", 2), (13, 1025, "float32", 0), (300, 2048, "bfloat16", 16),
    (2, 70001, "bfloat16", 0), (513, 256, "float16", 0)])
def test_forced_every_form(R, rows, D, dtype, chunks):
    cfg = dict(vecs_per_lane=-2, num_blocks=chunks)
    q = R.query_config(2, rows, D, I.torch_dtype(dtype))
    _say(f"column split forced {dtype} {rows}x{D} chunks={chunks} (automatic plan {q})")
    _check(R, rows, D, dtype, seed=rows + D, cfg=cfg)


@pytest.mark.parametrize("rows,D,dtype", [(17, 1 << 20, "bfloat16"), (100, 65536, "float16"),
                                          (3, 100000, "float32"), (255, 16392, "bfloat16")])
def test_automatic_wide_rows(R, rows, D, dtype):
    q = R.query_config(2, rows, D, I.torch_dtype(dtype))
    _say(f"column split automatic {dtype} {rows}x{D}: {q}")
    assert q["vecs_per_lane"] == -2 and q["block_threads"] == 256, q
    for op in (3, 4):
        assert R.query_config(op, rows, D, I.torch_dtype(dtype))["vecs_per_lane"] == -2
    _check(R, rows, D, dtype, seed=D % 1000 + rows, cfg=None, wb=0.0)


def test_many_rows_keep_the_streaming_grid(R):
    for rows, D in ((8192, 1 << 16), (2048, 32768), (1024, 16392)):
        q = R.query_config(2, rows, D, torch.bfloat16)
        assert q["vecs_per_lane"] == -1, (rows, D, q)
    for rows, D in ((4096, 1 << 16), (1024, 32768), (511, 16392)):
        q = R.query_config(2, rows, D, torch.bfloat16)
        assert q["vecs_per_lane"] == -2, (rows, D, q)


def test_typed_dw_in_place_repeat_and_exact_workspace(R):
    rows, D, dtype = 40, 40000, "bfloat16"
    c = I.generic(rows, D, dtype, seed=11)
    td = I.torch_dtype(dtype)
    assert R.query_config(2, rows, D, td)["vecs_per_lane"] == -2
    xg, wg, dyg = c["x"].to(DEV), c["w"].to(DEV), c["dy"].to(DEV)
    nbytes = R.rmsnorm_vjp_workspace_bytes(rows, D, td)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    dx, dw = R.rmsnorm_vjp(xg, wg, dyg, c["eps"], 0.5, workspace=ws)
    dx2, dw2 = R.rmsnorm_vjp(xg, wg, dyg, c["eps"], 0.5, workspace=ws)
    # dw in the weight dtype (the fp32 sum rounded once by the combine)
    _, dx3, dwt = R.rmsnorm_backward(xg, wg, dyg, c["eps"], 0.5, dw_dtype=td, workspace=ws)
    # in place: dx over dy, then over x
    dyi = dyg.clone()
    R.rmsnorm_vjp(xg, wg, dyi, c["eps"], 0.5, dx=dyi, workspace=ws)
    xi = xg.clone()
    R.rmsnorm_vjp(xi, wg, dyg, c["eps"], 0.5, dx=xi, workspace=ws)
    torch.cuda.synchronize()
    dxref, dwref = O.rmsnorm_vjp(c["x"], c["w"], c["dy"], c["eps"], 0.5)
    assert_close(dx, dxref, "dx")
    assert_dw_close(dw, dwref)
    assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16))
    assert torch.equal(dw.view(torch.int32), dw2.view(torch.int32))
    assert torch.equal(dx3.view(torch.int16), dx.view(torch.int16))
    np.testing.assert_array_equal(to64(dwt), O.round_to(to64(dw), dtype))
    assert torch.equal(dyi.view(torch.int16), dx.view(torch.int16))
    assert torch.equal(xi.view(torch.int16), dx.view(torch.int16))


def test_forced_rejections(R):
    c = I.generic(4, 1024, "float16", seed=1)
    xg, wg, dyg = c["x"].to(DEV), c["w"].to(DEV), c["dy"].to(DEV)
    for bad in (dict(vecs_per_lane=-2, lanes_per_row=64), dict(vecs_per_lane=-2, block_threads=512)):
        with pytest.raises(R.RMSNormError) as ei:
            R.rmsnorm_vjp(xg, wg, dyg, c["eps"], 0.0, cfg=bad)
        assert ei.value.status == -8, bad
    # the forward forms have no column split
    with pytest.raises(R.RMSNormError) as ei:
        R.rmsnorm_fwd(xg, wg, c["eps"], 0.0, cfg=dict(vecs_per_lane=-2))
    assert ei.value.status == -8
