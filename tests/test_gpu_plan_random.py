"""GPU: the automatic plan on seeded random shapes.

Plan queries launch nothing; about 3000 random (op, rows, D, dtype) are
checked against the invariants every plan must keep: the row is covered by
the lanes and vectors, blocks are whole waves holding whole row slots, the
persistent backward grids never hold one dw partial row per row and stay
within the partial-row bound, the VJP workspace is smaller than a [rows, D]
fp32 temporary (beyond its 256-byte floor), and forward calls on no more
rows than compute units take one row per block on 64..768 whole 16-byte
vectors, and the backward forms on few rows (<= 32 KiB per tensor) one
block with one vector per lane.  Then 40
random shapes (up to ~1.5 M elements) run through every form and are
compared with the fp64 oracle on every element."""
import sys

import numpy as np
import pytest
import torch

from _parity import assert_close, assert_dw_close, to64
from backward_rmsnorm_fwd_two_amd import inputs as I
from oracle import oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DTYPES = ("float32", "float16", "bfloat16")


@pytest.fixture(scope="module")
def R():
    import backward_rmsnorm_fwd_two_amd as pkg
    return pkg


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _shape(rng):
    """Rows and D drawn log-uniformly, with a bias towards the boundaries the
    plan rules sit on (multiples of 64 vectors, powers of two, +-1)."""
    D = int(np.exp(rng.uniform(0.0, np.log(300000))))
    if rng.random() < 0.4:
        base = int(2 ** rng.integers(4, 17))
        D = max(1, base + int(rng.integers(-1, 2)) * (1 if rng.random() < 0.5 else 64))
    rows = int(np.exp(rng.uniform(0.0, np.log(40000))))
    if rng.random() < 0.3:
        rows = int(rng.choice([1, 2, 3, 255, 256, 257, 511, 512, 513, 4096]))
    return max(1, rows), max(1, D)


def _np2(n):
    p = 1
    while p < n:
        p *= 2
    return p


def test_plan_invariants_random_shapes(R):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rng = np.random.default_rng(20261202)
    checked = 0
    for _ in range(3000):
        rows, D = _shape(rng)
        dtype = DTYPES[int(rng.integers(0, 3))]
        td = I.torch_dtype(dtype)
        s = td.itemsize
        for op in range(5):
            what = (op, rows, D, dtype)
            q = R.query_config(op, rows, D, td)
            k, lanes, vb, block, nb = (q["vecs_per_lane"], q["lanes_per_row"], q["vec_bytes"],
                                       q["block_threads"], q["num_blocks"])
            assert vb in (2, 4, 8, 16) and vb >= s, (what, q)
            nv = vb // s
            assert 64 <= block <= 1024 and block % 64 == 0, (what, q)
            assert nb >= 1, (what, q)
            if k > 0:
                assert k in (1, 2, 4, 8), (what, q)
                assert 1 <= lanes <= 1024 and block % lanes == 0, (what, q)
                assert lanes * k * nv >= D, (what, q)            # the row is covered
                if D * s % vb:                                    # overlapped last vector
                    assert vb == 16 and D * s > 16, (what, q)
            elif k == -1:
                assert lanes == 0 and D * s % vb == 0, (what, q)     # streaming: whole vectors only
            else:
                assert k == -2 and op >= 2 and block == 256 and rows <= 65535, (what, q)
            if op >= 2:
                assert nb <= 2048, (what, q)
                ovl = D * s % 16 != 0 and D * s > 16
                nvec16 = -(-D * s // 16)
                if ((D * s % 16 == 0 or ovl) and rows * D * s <= 32768 and
                        nvec16 <= (1024 if s == 2 and not ovl else 512)):
                    # few rows: one block looping over them, one vector per lane
                    assert k == 1 and vb == 16 and nb == 1 and lanes in (nvec16, _np2(nvec16)), (what, q)
                    cap = 512 if lanes <= 16 else 256
                    assert block == max(64, lanes * min(_np2(rows), max(1, cap // lanes))), (what, q)
                if rows >= 2:
                    # never one dw partial row per row (the [rows, D] temporary)
                    assert nb <= (rows + 1) // 2, (what, q)
                    ws = R.rmsnorm_vjp_workspace_bytes(rows, D, td)
                    assert ws == 256 or ws < rows * D * 4, (what, q, ws)    # 256: the size floor
            elif rows <= cus and D * s % 16 == 0 and 64 <= D * s // 16 <= 768 and (D * s // 16) % 64 == 0:
                assert (lanes, k, vb, block, nb) == (D * s // 16, 1, 16, max(D * s // 16, 64), rows), (what, q)
            checked += 1
    _say(f"plan invariants: {checked} plans")
    assert checked == 15000


def _parity_case(R, rows, D, dtype, seed):
    c = I.generic(rows, D, dtype, seed=seed)
    rng = np.random.default_rng(seed)
    dr = I.normal(rng, (rows, D), 0.0, 0.5, dtype)
    wb = float(rng.choice([0.0, 1.0]))
    xg, wg, dyg, rg, drg = (t.to(DEV) for t in (c["x"], c["w"], c["dy"], c["residual"], dr))
    eps = c["eps"]
    what = f"{dtype} {rows}x{D} wb={wb}"
    y = R.rmsnorm_fwd(xg, wg, eps, wb)
    n, h = R.fused_add_rmsnorm_fwd(xg, rg, wg, eps, wb)
    dx, dw = R.rmsnorm_vjp(xg, wg, dyg, eps, wb)
    gy, gdx, gdw = R.rmsnorm_fwd_vjp(xg, wg, dyg, eps, wb)
    dh, hdw = R.fused_add_rmsnorm_vjp(xg, wg, dyg, drg, eps, wb)
    torch.cuda.synchronize()
    yref, _ = O.rmsnorm_fwd(c["x"], c["w"], eps, wb)
    nref, href = O.fused_add_rmsnorm_fwd(c["x"], c["residual"], c["w"], eps, wb)
    dxref, dwref = O.rmsnorm_vjp(c["x"], c["w"], c["dy"], eps, wb)
    dhref, _ = O.fused_add_rmsnorm_vjp(c["x"], c["w"], c["dy"], dr, eps, wb)
    assert_close(y, yref, f"{what} y")
    assert_close(n, nref, f"{what} normed")
    np.testing.assert_array_equal(to64(h), O.round_to(href, dtype), err_msg=f"{what} new_residual")
    assert_close(dx, dxref, f"{what} dx")
    assert_dw_close(dw, dwref, f"{what} dw")
    assert_close(gy, yref, f"{what} grad y")
    assert_close(gdx, dxref, f"{what} grad dx")
    assert_dw_close(gdw, dwref, f"{what} grad dw")
    assert_close(dh, dhref, f"{what} dh")
    assert_dw_close(hdw, dwref, f"{what} fused dw")


def test_random_shapes_every_form_matches_oracle(R):
    rng = np.random.default_rng(7)
    done = 0
    while done < 40:
        rows, D = _shape(rng)
        if rows * D > 1_500_000:
            continue
        dtype = DTYPES[int(rng.integers(0, 3))]
        _say(f"random shape {done}: {dtype} {rows}x{D}")
        _parity_case(R, rows, D, dtype, seed=1000 + done)
        done += 1
