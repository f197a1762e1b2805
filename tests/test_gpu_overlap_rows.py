"""GPU: rows that are not a whole number of 16-byte vectors (D * itemsize not
a multiple of 16: D = 257, 500, 511, 513 of the small-axis sweep in 16-bit
storage, odd fp32 widths).  They run on 16-byte vectors with the row's last
vector shifted back to end at the row's end; its leading elements, which the
previous vector also holds, stay out of the row sums and of dw.  Every form
is compared with the fp64 oracle on every element, at row counts that make
every block loop over several row groups and at one row; rows too wide for
the register kernels fall back to narrower loads."""
import sys

import numpy as np
import pytest
import torch

from _parity import assert_close, assert_dw_close, to64
from backward_rmsnorm_fwd_two_amd import inputs as I
from oracle import oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
OPS = {"fwd": 0, "fused": 1, "vjp": 2, "grad": 3, "fused_vjp": 4}


@pytest.fixture(scope="module")
def R():
    import backward_rmsnorm_fwd_two_amd as pkg
    return pkg


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _gpu(t):
    return t.to(DEV)


def _itemsize(dtype):
    return 4 if dtype == "float32" else 2


def _check_every_form(R, rows, D, dtype, seed, cfg=None, wb=1.0):
    """Every form against the oracle; with a forced cfg, a form whose
    instance cannot take the block (register budget: RMSN_E_CONFIG) is
    skipped.  Returns the forms checked."""
    c = I.generic(rows, D, dtype, seed=seed)
    rng = np.random.default_rng(seed)
    dr = I.normal(rng, (rows, D), 0.0, 0.5, dtype)
    xg, wg, dyg, drg = _gpu(c["x"]), _gpu(c["w"]), _gpu(c["dy"]), _gpu(dr)
    eps = c["eps"]
    what = f"{dtype} {rows}x{D} cfg={cfg}"
    calls = {
        "fwd": lambda: R.rmsnorm_fwd(xg, wg, eps, wb, cfg=cfg),
        "fused": lambda: R.fused_add_rmsnorm_fwd(xg, drg, wg, eps, wb, cfg=cfg),
        "vjp": lambda: R.rmsnorm_vjp(xg, wg, dyg, eps, wb, cfg=cfg),
        "grad": lambda: R.rmsnorm_fwd_vjp(xg, wg, dyg, eps, wb, cfg=cfg),
        "fused_vjp": lambda: R.fused_add_rmsnorm_vjp(xg, wg, dyg, drg, eps, wb, cfg=cfg),
    }
    out = {}
    for name, call in calls.items():
        try:
            out[name] = call()
        except R.RMSNormError as e:
            if cfg is None or e.status != -8 or cfg.get("block_threads", 0) <= 256:
                raise
    torch.cuda.synchronize()
    yref, _ = O.rmsnorm_fwd(c["x"], c["w"], eps, wb)
    if "fwd" in out:
        assert_close(out["fwd"], yref, f"{what} y")
    if "fused" in out:
        nref, href = O.fused_add_rmsnorm_fwd(c["x"], dr, c["w"], eps, wb)
        normed, newres = out["fused"]
        assert_close(normed, nref, f"{what} normed")
        np.testing.assert_array_equal(to64(newres), O.round_to(href, dtype), err_msg=f"{what} new_residual")
    if "vjp" in out or "grad" in out:
        dxref, dwref = O.rmsnorm_vjp(c["x"], c["w"], c["dy"], eps, wb)
        if "vjp" in out:
            assert_close(out["vjp"][0], dxref, f"{what} dx")
            assert_dw_close(out["vjp"][1], dwref, f"{what} dw")
        if "grad" in out:
            gy, gdx, gdw = out["grad"]
            assert_close(gy, yref, f"{what} grad y")
            assert_close(gdx, dxref, f"{what} grad dx")
            assert_dw_close(gdw, dwref, f"{what} grad dw")
    if "fused_vjp" in out:
        dhref, hdwref = O.fused_add_rmsnorm_vjp(c["x"], c["w"], c["dy"], dr, eps, wb)
        assert_close(out["fused_vjp"][0], dhref, f"{what} dh")
        assert_dw_close(out["fused_vjp"][1], hdwref, f"{what} fused dw")
    return sorted(out)


@pytest.mark.parametrize("dtype,D", [("float16", 257), ("float16", 500), ("float16", 511), ("float16", 513),
                                     ("bfloat16", 513), ("float32", 1023), ("float32", 97)])
def test_plan_takes_16_byte_vectors(R, dtype, D):
    td = I.torch_dtype(dtype)
    for name, op in OPS.items():
        q = R.query_config(op, 16384, D, td)
        assert q["vec_bytes"] == 16, (name, q)
        assert q["vecs_per_lane"] > 0 and q["lanes_per_row"] * q["vecs_per_lane"] * 16 >= D * _itemsize(dtype), q


def test_plan_narrow_below_one_vector(R):
    # 7 fp16 elements (14 bytes) are less than one 16-byte vector
    q = R.query_config(2, 64, 7, torch.float16)
    assert q["vec_bytes"] == 2, q


@pytest.mark.parametrize("dtype,D", [
    ("float16", 9), ("float16", 15), ("float16", 17), ("float16", 257), ("float16", 500),
    ("float16", 511), ("float16", 513), ("bfloat16", 1025), ("bfloat16", 3001), ("float16", 4097),
    ("float16", 8191), ("bfloat16", 12289), ("float32", 5), ("float32", 97), ("float32", 1023),
    ("float32", 4099), ("float16", 1500), ("float16", 2049), ("float16", 4500), ("bfloat16", 4700),
    ("float32", 2251)])
@pytest.mark.parametrize("rows", [1, 300])
def test_every_form_matches_oracle(R, dtype, D, rows):
    _say(f"overlapped rows {dtype} {rows}x{D}")
    _check_every_form(R, rows, D, dtype, seed=D + rows)


# (dtype, D): the forward's and the fused forward's (lanes, vectors per lane)
# on rows of a whole number of waves, or None where the power-of-two layout
# stays
WAVE_FWD = [("float16", 1500, None, (192, 1)), ("float16", 1300, None, (192, 1)), ("float16", 2049, (320, 1), None),
            ("bfloat16", 3001, (192, 2), None), ("float16", 4500, (576, 1), (576, 1)),
            ("bfloat16", 4700, (320, 2), (320, 2)), ("float32", 2251, (576, 1), (576, 1)),
            ("float16", 7001, None, None), ("float16", 8191, None, None)]


@pytest.mark.parametrize("dtype,D,fwd,fused", WAVE_FWD)
def test_forward_wave_rows_plan(R, dtype, D, fwd, fused):
    """The forward forms on overlapped rows take a whole number of waves
    (lanes 64 W, W not a power of two) where the row fills most of its slots
    and the power-of-two layout would leave many masked; elsewhere they keep
    the power-of-two layout."""
    td = I.torch_dtype(dtype)
    for op, want in ((0, fwd), (1, fused)):
        q = R.query_config(op, 4096, D, td)
        got = (q["lanes_per_row"], q["vecs_per_lane"])
        lanes = q["lanes_per_row"]
        wave = lanes > 64 and lanes & (lanes - 1) != 0
        if want is None:
            assert not wave, (op, q)
        else:
            assert got == want, (op, q)
            assert q["block_threads"] in (lanes, 2 * lanes), q
        assert lanes * q["vecs_per_lane"] * 16 >= D * _itemsize(dtype), q


@pytest.mark.parametrize("dtype,D,geoms", [
    ("float16", 2049, [(192, 2, 0), (320, 1, 0), (320, 1, 640), (576, 1, 0), (960, 1, 0), (320, 2, 0)]),
    ("bfloat16", 4097, [(576, 1, 0), (320, 2, 0), (704, 1, 0), (960, 1, 0), (576, 0, 0)]),
    ("float32", 1001, [(192, 2, 384), (320, 1, 0), (448, 1, 896)])])
def test_forced_forward_wave_rows(R, dtype, D, geoms):
    """Requested whole-wave geometries (lanes 64 W, one or two vectors per
    lane, one or two rows per block) of the forward forms on overlapped rows,
    every element against the oracle at a ragged row count."""
    rows = 301
    c = I.generic(rows, D, dtype, seed=D + 7)
    rng = np.random.default_rng(D)
    dr = I.normal(rng, (rows, D), 0.0, 0.5, dtype)
    xg, wg, drg = _gpu(c["x"]), _gpu(c["w"]), _gpu(dr)
    eps = c["eps"]
    yref, _ = O.rmsnorm_fwd(c["x"], c["w"], eps, 1.0)
    nref, href = O.fused_add_rmsnorm_fwd(c["x"], dr, c["w"], eps, 1.0)
    for lanes, k, block in geoms:
        cfg = dict(lanes_per_row=lanes, vecs_per_lane=k, vec_bytes=16, block_threads=block, num_blocks=0)
        _say(f"forced forward wave rows {dtype} {rows}x{D} {cfg}")
        y = R.rmsnorm_fwd(xg, wg, eps, 1.0, cfg=cfg)
        normed, newres = R.fused_add_rmsnorm_fwd(xg, drg, wg, eps, 1.0, cfg=cfg)
        torch.cuda.synchronize()
        assert_close(y, yref, f"{cfg} y")
        assert_close(normed, nref, f"{cfg} normed")
        np.testing.assert_array_equal(to64(newres), O.round_to(href, dtype), err_msg=f"{cfg} new_residual")
    # a lane count too small for the row, and three vectors per lane, are refused
    for bad in (dict(lanes_per_row=192, vecs_per_lane=1), dict(lanes_per_row=192, vecs_per_lane=4)):
        with pytest.raises(R.RMSNormError):
            R.rmsnorm_fwd(xg, wg, eps, 1.0, cfg=dict(vec_bytes=16, block_threads=0, num_blocks=0, **bad))


def test_small_axis_sweep_widths_full_size(R):
    """The sweep's odd widths at their full 16384 rows, every element."""
    for D in (257, 500, 511, 513):
        _say(f"overlapped rows float16 16384x{D}")
        _check_every_form(R, 16384, D, "float16", seed=D, wb=0.0)


@pytest.mark.parametrize("dtype,D", [("float16", 513), ("bfloat16", 257), ("float32", 1023)])
def test_forced_geometries(R, dtype, D):
    """Every lanes / vectors-per-lane / block the overlapped instances take,
    on 16-byte vectors, with small grids that make blocks loop."""
    s = _itemsize(dtype)
    nv = 16 // s
    nvec = -(-D // nv)
    cfgs = []
    for k in (1, 2, 4, 8):
        for lanes in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512):
            if lanes * k < nvec or (lanes * k >= 4 * nvec and lanes > 1):
                continue
            for block in (64, 256, 512):
                if block < lanes or block % lanes:
                    continue
                cfgs.append(dict(lanes_per_row=lanes, vecs_per_lane=k, vec_bytes=16, block_threads=block,
                                 num_blocks=0))
    _say(f"overlapped forced geometries {dtype} D={D}: {len(cfgs)}")
    assert cfgs
    checked = 0
    for cfg in cfgs:
        for nb in (0, 5):
            checked += len(_check_every_form(R, 77, D, dtype, seed=D, cfg=dict(cfg, num_blocks=nb)))
    assert checked >= 2 * len(cfgs) * 3


def test_forced_streaming_with_16_byte_vectors_rejected(R):
    c = I.generic(4, 513, "float16", seed=1)
    xg, wg = _gpu(c["x"]), _gpu(c["w"])
    with pytest.raises(R.RMSNormError) as ei:
        R.rmsnorm_fwd(xg, wg, c["eps"], 0.0, cfg=dict(vecs_per_lane=-1, vec_bytes=16, block_threads=256))
    assert ei.value.status == -8
    # the streaming kernel itself takes the row on narrower loads
    y = R.rmsnorm_fwd(xg, wg, c["eps"], 0.0, cfg=dict(vecs_per_lane=-1, block_threads=256))
    torch.cuda.synchronize()
    assert_close(y, O.rmsnorm_fwd(c["x"], c["w"], c["eps"], 0.0)[0], "streaming y")


def test_wide_odd_row_falls_back_to_narrow_loads(R):
    # 8192 * 8 + 1 fp16 elements: more vectors than the register kernels hold;
    # the forward streams them, the backward forms on 3 rows split columns
    D = 65537
    q = R.query_config(0, 3, D, torch.float16)
    assert q["vecs_per_lane"] == -1 and q["vec_bytes"] == 2, q
    q = R.query_config(2, 3, D, torch.float16)
    assert q["vecs_per_lane"] == -2 and q["vec_bytes"] == 2, q
    _check_every_form(R, 3, D, "float16", seed=3)
