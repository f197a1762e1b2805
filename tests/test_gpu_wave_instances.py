"""GPU: every compiled wave-row instance (rows of W = 3, 5, 6, 7, 9, 10, 11,
12, 13, 14 or 15 waves, one or two 16-byte vectors per lane), every wide 16-bit instance
(four vectors per lane: 384, 448 or 512 lanes for the VJP, 448 or 512 for
the grad call and the fused backward) and the fp32 four-vector instances
(512 lanes) run, forced
through the *_cfg entry points, and matches the fp64 oracle on a few rows,
one and two rows per block; combinations without an instance return
RMSN_E_CONFIG.  The automatic plan selects only some of these instances,
so without forcing them several would never run.

The D of each case is lanes x vectors per lane x elements per 16-byte
vector, so the row tiles exactly."""
import sys

import pytest
import torch

from _parity import assert_close, assert_dw_close
from backward_rmsnorm_fwd_two_amd import inputs as I
from oracle import oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
WAVE_LANES = [192, 320, 384, 448, 576, 640, 704, 768, 832, 896, 960]
E_CONFIG = -8


@pytest.fixture(scope="module")
def R():
    import backward_rmsnorm_fwd_two_amd as pkg
    return pkg


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _backward_instance(dtype, lanes, k, op):
    """Whether a pipelined instance exists for a backward form (mirror of the
    library's instance table): 16-bit rows with two vectors per lane stop at
    768 lanes (wider would spill), the wide four-vector 16-bit instances
    serve the VJP on 384, 448 and 512 lanes and the other two forms on 448
    and 512, and fp32 rows take four vectors per lane on 512 lanes only."""
    if k == 4:
        if dtype == "float32":
            return lanes == 512
        return (op == "vjp" and lanes in (384, 448, 512)) or (op != "vjp" and lanes in (448, 512))
    if dtype != "float32" and k == 2 and lanes > 640:
        # 11 and 12 waves fit (147-168 VGPRs; the fused backward with one
        # d_new_residual buffer); 13 to 15 waves fit none
        return lanes in (704, 768)
    return True


CASES = [(dt, lanes, k) for dt in ("float32", "float16", "bfloat16") for lanes in WAVE_LANES for k in (1, 2)]
CASES += [(dt, lanes, 4) for dt in ("float16", "bfloat16") for lanes in (384, 448, 512)]
CASES += [("float32", 512, 4), ("float32", 448, 4)]


def _id(c):
    return f"{c[0]}-{c[1]}x{c[2]}"


@pytest.mark.parametrize("dtype,lanes,k", CASES, ids=[_id(c) for c in CASES])
def test_wave_instance_parity(R, dtype, lanes, k):
    nv = 4 if dtype == "float32" else 8
    D = lanes * k * nv
    _say(f"wave instance {dtype} lanes={lanes} k={k} D={D}")
    # 13 rows in one-row blocks, and in two-row blocks (a ragged last group)
    for rows, slots in ((13, 1), (13, 2)):
        c = I.generic(rows, D, dtype, seed=lanes * 7 + k + rows)
        x, w, dy, res = (c[n].to(DEV) for n in ("x", "w", "dy", "residual"))
        eps, wb = c["eps"], 0.5
        cfg = dict(lanes_per_row=lanes, vecs_per_lane=k, vec_bytes=16, block_threads=slots * lanes, num_blocks=0)
        yref, _ = O.rmsnorm_fwd(c["x"], c["w"], eps, wb)
        nref, href = O.fused_add_rmsnorm_fwd(c["x"], c["residual"], c["w"], eps, wb)
        dxref, dwref = O.rmsnorm_vjp(c["x"], c["w"], c["dy"], eps, wb)
        dhref, dwhref = O.fused_add_rmsnorm_vjp(c["x"], c["w"], c["dy"], c["residual"], eps, wb)

        # forward forms: an instance for every wave width and one or two
        # vectors per lane, blocks of up to 1024 threads
        if k in (1, 2) and slots * lanes <= 1024:
            y = R.rmsnorm_fwd(x, w, eps, wb, cfg=cfg)
            n, h = R.fused_add_rmsnorm_fwd(x, res, w, eps, wb, cfg=cfg)
            torch.cuda.synchronize()
            assert_close(y, yref, f"y {cfg}")
            assert_close(n, nref, f"normed {cfg}")
            assert_close(h, href, f"new_residual {cfg}")

        # backward forms: one row per block always; two rows while the
        # registers allow (blocks of at most 768 threads, not the wide rows)
        elems = k * nv
        two_ok = elems <= 16 and 2 * lanes <= 768
        for op in ("vjp", "grad", "fused"):
            exists = _backward_instance(dtype, lanes, k, op) and (slots == 1 or two_ok)
            if k == 4 and lanes == 512:
                # a power of two: a form or block the pipelined instances do
                # not serve takes the plain loop, within its register budget
                # (16 elements per lane, fp32: 1024 threads; 32, 16-bit: 512)
                exists = slots == 1 or dtype == "float32"
            try:
                if op == "vjp":
                    dx, dw = R.rmsnorm_vjp(x, w, dy, eps, wb, cfg=cfg)
                elif op == "grad":
                    yg, dx, dw = R.rmsnorm_fwd_vjp(x, w, dy, eps, wb, cfg=cfg)
                else:
                    dx, dw = R.fused_add_rmsnorm_vjp(x, w, dy, res, eps, wb, cfg=cfg)
                torch.cuda.synchronize()
            except R.RMSNormError as e:
                assert not exists, f"{op} {cfg}: {e}"
                assert e.status == E_CONFIG, f"{op} {cfg}: {e}"
                continue
            assert exists, f"{op} {cfg}: ran without an instance"
            if op == "fused":
                assert_close(dx, dhref, f"dh {cfg}")
                assert_dw_close(dw, dwhref, f"fused dw {cfg}")
            else:
                assert_close(dx, dxref, f"{op} dx {cfg}")
                assert_dw_close(dw, dwref, f"{op} dw {cfg}")
                if op == "grad":
                    assert_close(yg, yref, f"grad y {cfg}")
