"""GPU parity of the gated activation y = silu(x[:, :d]) * x[:, d:2d] (the
candidate-fusion list of the mlxcel fused-kernel issue): the HIP library
through its C ABI against the fp64 CPU oracle on the same seeded inputs --
every half width d from 1 to 600 in each dtype, the decode and prefill-scale
Llama-3 8B MLP shapes (the full 8192 x 14336 output compared element by
element), forced kernel configurations (load width, vectors per thread,
block, a grid smaller than the chunk count), misaligned pointers, IEEE
special values, and the error codes."""
import ctypes
import sys

import numpy as np
import pytest
import torch

from _parity import assert_close, to64
from backward_rmsnorm_fwd_two_amd import inputs as I
from oracle import oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DTYPES = ["float32", "float16", "bfloat16"]
MLP_D = 14336


@pytest.fixture(scope="module")
def R():
    import backward_rmsnorm_fwd_two_amd as pkg
    return pkg


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(R, x, what, cfg=None, out=None):
    y = R.silu_gate(x.to(DEV), out=out, cfg=cfg)
    torch.cuda.synchronize()
    ref = O.silu_gate(x)
    return assert_close(y, ref, what)


@pytest.mark.parametrize("dtype", DTYPES)
def test_gate_every_d_1_to_600(R, dtype):
    _say(f"gate every d 1..600 {dtype}")
    worst = 0.0
    for d in range(1, 601):
        x = I.gate(3, d, dtype, seed=d)["x"]
        worst = max(worst, check(R, x, f"{dtype} d={d}"))
    _say(f"  worst err {worst:.2e}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rows,d", [(1, MLP_D), (4, MLP_D), (8, MLP_D), (37, 4104), (129, 1000),
                                    (1000, 24), (4097, 8), (3, 1 << 16), (2, 100003)])
def test_gate_shapes(R, dtype, rows, d):
    _say(f"gate rows={rows} d={d} {dtype}")
    x = I.gate(rows, d, dtype, seed=rows + d)["x"]
    check(R, x, f"{dtype} rows={rows} d={d}")


def test_gate_full_prefill_chunk_every_element(R):
    """8192 x 14336 bf16 (x is 448 MiB): every output element against the
    oracle, 512 rows at a time."""
    rows, d = 8192, MLP_D
    _say(f"gate full size rows={rows} d={d} bfloat16")
    x = I.gate(rows, d, "bfloat16", seed=0)["x"]
    y = R.silu_gate(x.to(DEV))
    torch.cuda.synchronize()
    yc = y.cpu()
    worst = 0.0
    for r0 in range(0, rows, 512):
        ref = O.silu_gate(x[r0:r0 + 512])
        worst = max(worst, assert_close(yc[r0:r0 + 512], ref, f"rows {r0}.."))
    _say(f"  worst err {worst:.2e}")


def _configs(d, s):
    out = []
    for vb in (16, 8, 4, 2):
        if vb < s or (d * s) % vb:
            continue
        for u in (1, 2, 4, 8):
            for block in (64, 256, 1024):
                for nb in (0, 1, 7):
                    out.append(dict(vec_bytes=vb, vecs_per_lane=u, block_threads=block, num_blocks=nb))
    return out


@pytest.mark.parametrize("dtype,rows,d", [("bfloat16", 5, 1000), ("float16", 33, 96),
                                          ("float32", 7, 520), ("bfloat16", 3, 8200)])
def test_gate_forced_configs(R, dtype, rows, d):
    x = I.gate(rows, d, dtype, seed=7)["x"]
    s = x.element_size()
    ref = O.silu_gate(x)
    xg = x.to(DEV)
    cfgs = _configs(d, s)
    _say(f"gate forced configs {dtype} rows={rows} d={d}: {len(cfgs)}")
    for cfg in cfgs:
        y = R.silu_gate(xg, cfg=cfg)
        torch.cuda.synchronize()
        assert_close(y, ref, f"cfg {cfg}")


@pytest.mark.parametrize("dtype", ["float16", "bfloat16", "float32"])
@pytest.mark.parametrize("xoff,yoff", [(1, 0), (0, 1), (3, 5), (2, 2)])
def test_gate_misaligned(R, dtype, xoff, yoff):
    rows, d = 9, 776
    x = I.gate(rows, d, dtype, seed=11)["x"]
    tdt = I.torch_dtype(dtype)
    xb = torch.zeros(rows * 2 * d + 16, dtype=tdt, device=DEV)
    xb[xoff:xoff + rows * 2 * d] = x.reshape(-1).to(DEV)
    yb = torch.full((rows * d + 16,), 7.0, dtype=tdt, device=DEV)
    xv = xb[xoff:xoff + rows * 2 * d].view(rows, 2 * d)
    yv = yb[yoff:yoff + rows * d].view(rows, d)
    R.silu_gate(xv, out=yv)
    torch.cuda.synchronize()
    assert_close(yv, O.silu_gate(x), f"{dtype} xoff={xoff} yoff={yoff}")
    yc = to64(yb)
    assert np.all(yc[:yoff] == 7.0) and np.all(yc[yoff + rows * d:] == 7.0), "wrote outside y"


def test_gate_writes_exactly_y(R):
    rows, d = 17, 333
    x = I.gate(rows, d, "bfloat16", seed=3)["x"]
    yb = torch.full((rows * d + 512,), -3.0, dtype=torch.bfloat16, device=DEV)
    for cfg in (None, dict(vecs_per_lane=8, block_threads=1024), dict(num_blocks=1)):
        y = yb[:rows * d].view(rows, d)
        R.silu_gate(x.to(DEV), out=y, cfg=cfg)
        torch.cuda.synchronize()
        assert torch.all(yb[rows * d:] == -3.0)
        assert_close(y, O.silu_gate(x), f"cfg {cfg}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_gate_special_values(R, dtype):
    # a: first half; b: second half.  Combinations stay clear of overflow in
    # the storage dtype and of b = inf with a below -88.7 (silu there is -0).
    a_vals = [0.0, -0.0, 1.0, -1.0, 0.5, -0.5, 5.0, -5.0, 30.0, -30.0, 80.0, -80.0,
              float("inf"), float("-inf"), float("nan")]
    if dtype != "float16":
        a_vals += [88.0, -88.0, 89.0, -89.0, 100.0, -100.0, 1e30 if dtype == "float32" else 1e20]
    b_vals = [1.0, -2.0, 0.0, 0.25]
    pairs = [(a, b) for a in a_vals for b in b_vals]
    pairs += [(2.0, float("inf")), (-2.0, float("inf")), (3.0, float("nan"))]
    d = len(pairs)
    x = torch.tensor([[p[0] for p in pairs] + [p[1] for p in pairs]], dtype=torch.float64)
    x = x.to(I.torch_dtype(dtype))
    check(R, x, f"{dtype} special values")


def test_gate_matches_prepared_call(R):
    x = I.gate(64, 2048, "bfloat16", seed=5)["x"].to(DEV)
    y1 = R.silu_gate(x)
    y2 = torch.empty_like(y1)
    R.prepared_gate(x, y2)()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_gate_errors(R):
    lib = R.raw
    x = torch.zeros(4, 16, dtype=torch.bfloat16, device=DEV)
    y = torch.zeros(4, 8, dtype=torch.bfloat16, device=DEV)
    xp, yp = x.data_ptr(), y.data_ptr()
    assert lib.silu_gate(xp, yp, 0, 8, 2, None) == 0
    assert lib.silu_gate(None, yp, 4, 8, 2, None) == -1
    assert lib.silu_gate(xp, yp, 4, 0, 2, None) == -2
    assert lib.silu_gate(xp, yp, -1, 8, 2, None) == -2
    assert lib.silu_gate(xp, yp, 4, (1 << 28) + 1, 2, None) == -2
    assert lib.silu_gate(xp, yp, 1 << 40, 1 << 27, 2, None) == -2
    assert lib.silu_gate(xp, yp, 4, 8, 5, None) == -3
    assert lib.silu_gate(xp + 1, yp, 4, 8, 2, None) == -7
    # y inside x
    assert lib.silu_gate(xp, xp + 32, 4, 8, 2, None) == -5
    for bad in (dict(lanes_per_row=1), dict(vecs_per_lane=3), dict(vecs_per_lane=-1),
                dict(block_threads=100), dict(block_threads=2048), dict(vec_bytes=32)):
        c = R.Config(**bad)
        assert lib.silu_gate_cfg(xp, yp, 4, 8, 2, ctypes.byref(c), None) == -8, bad
    # 8 bf16 = 16 bytes per half row: 16-byte loads allowed; d = 12 is 24 bytes
    c = R.Config(vec_bytes=16)
    assert lib.silu_gate_cfg(xp, yp, 4, 8, 2, ctypes.byref(c), None) == 0
    assert lib.silu_gate_cfg(xp, yp, 2, 12, 2, ctypes.byref(c), None) == -8
    with pytest.raises(ValueError):
        R.silu_gate(torch.zeros(2, 7, dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()


# ------------------------------------------------------------ backward

def _dy(rows, d, dtype, seed):
    return I.normal(np.random.default_rng(seed), (rows, d), 0.0, 1.0, dtype)


def check_vjp(R, x, dy, what, cfg=None, out=None):
    g = R.silu_gate_vjp(x.to(DEV), dy.to(DEV), out=out, cfg=cfg)
    torch.cuda.synchronize()
    return assert_close(g, O.silu_gate_vjp(x, dy), what)


@pytest.mark.parametrize("dtype", DTYPES)
def test_gate_vjp_every_d_1_to_300(R, dtype):
    _say(f"gate vjp every d 1..300 {dtype}")
    for d in range(1, 301):
        x = I.gate(3, d, dtype, seed=d)["x"]
        check_vjp(R, x, _dy(3, d, dtype, d), f"{dtype} d={d}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rows,d", [(1, MLP_D), (8, MLP_D), (129, 1000), (4097, 8), (2, 100003)])
def test_gate_vjp_shapes(R, dtype, rows, d):
    _say(f"gate vjp rows={rows} d={d} {dtype}")
    x = I.gate(rows, d, dtype, seed=rows + d)["x"]
    check_vjp(R, x, _dy(rows, d, dtype, rows), f"{dtype} rows={rows} d={d}")


def test_gate_vjp_full_prefill_chunk_every_element(R):
    rows, d = 8192, MLP_D
    _say(f"gate vjp full size rows={rows} d={d} bfloat16")
    x = I.gate(rows, d, "bfloat16", seed=1)["x"]
    dy = _dy(rows, d, "bfloat16", 2)
    g = R.silu_gate_vjp(x.to(DEV), dy.to(DEV))
    torch.cuda.synchronize()
    gc = g.cpu()
    for r0 in range(0, rows, 512):
        assert_close(gc[r0:r0 + 512], O.silu_gate_vjp(x[r0:r0 + 512], dy[r0:r0 + 512]), f"rows {r0}..")


@pytest.mark.parametrize("dtype,rows,d", [("bfloat16", 5, 1000), ("float32", 7, 520), ("float16", 33, 96)])
def test_gate_vjp_forced_configs_and_in_place(R, dtype, rows, d):
    x = I.gate(rows, d, dtype, seed=17)["x"]
    dy = _dy(rows, d, dtype, 18)
    ref = O.silu_gate_vjp(x, dy)
    xg, dyg = x.to(DEV), dy.to(DEV)
    base = R.silu_gate_vjp(xg, dyg)
    for cfg in _configs(d, x.element_size()):
        g = R.silu_gate_vjp(xg, dyg, cfg=cfg)
        torch.cuda.synchronize()
        assert_close(g, ref, f"cfg {cfg}")
    # in place: dx over x, bit-identical to the out-of-place result
    xi = xg.clone()
    R.silu_gate_vjp(xi, dyg, out=xi)
    torch.cuda.synchronize()
    assert torch.equal(xi, base)


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
@pytest.mark.parametrize("xoff,dyoff,dxoff", [(1, 0, 0), (0, 3, 0), (0, 0, 5), (2, 2, 2)])
def test_gate_vjp_misaligned(R, dtype, xoff, dyoff, dxoff):
    rows, d = 9, 776
    x = I.gate(rows, d, dtype, seed=19)["x"]
    dy = _dy(rows, d, dtype, 20)
    tdt = I.torch_dtype(dtype)

    def place(t, off):
        flat = torch.zeros(t.numel() + 16, dtype=tdt, device=DEV)
        flat[off:off + t.numel()] = t.reshape(-1).to(DEV)
        return flat, flat[off:off + t.numel()].view(t.shape)

    _, xv = place(x, xoff)
    _, dyv = place(dy, dyoff)
    gb = torch.full((rows * 2 * d + 16,), 7.0, dtype=tdt, device=DEV)
    gv = gb[dxoff:dxoff + rows * 2 * d].view(rows, 2 * d)
    R.silu_gate_vjp(xv, dyv, out=gv)
    torch.cuda.synchronize()
    assert_close(gv, O.silu_gate_vjp(x, dy), "dx")
    gc = to64(gb)
    assert np.all(gc[:dxoff] == 7.0) and np.all(gc[dxoff + rows * 2 * d:] == 7.0)


@pytest.mark.parametrize("dtype", DTYPES)
def test_gate_vjp_special_values(R, dtype):
    a_vals = [0.0, -0.0, 1.0, -1.0, 5.0, -5.0, 30.0, -30.0, float("inf"), float("-inf"), float("nan")]
    if dtype != "float16":
        a_vals += [88.0, -88.0, 100.0, -100.0]
    b_vals = [1.0, -2.0, 0.0]
    g_vals = [1.0, -0.5]
    trip = [(a, b, g) for a in a_vals for b in b_vals for g in g_vals]
    d = len(trip)
    x = torch.tensor([[t[0] for t in trip] + [t[1] for t in trip]], dtype=torch.float64).to(I.torch_dtype(dtype))
    dy = torch.tensor([[t[2] for t in trip]], dtype=torch.float64).to(I.torch_dtype(dtype))
    check_vjp(R, x, dy, f"{dtype} special values")


def test_gate_vjp_errors_and_autograd(R):
    lib = R.raw
    x = torch.zeros(4, 16, dtype=torch.bfloat16, device=DEV)
    dy = torch.zeros(4, 8, dtype=torch.bfloat16, device=DEV)
    dx = torch.empty_like(x)
    p = lambda t: t.data_ptr()
    assert lib.silu_gate_vjp(p(x), p(dy), p(dx), 0, 8, 2, None) == 0
    assert lib.silu_gate_vjp(p(x), None, p(dx), 4, 8, 2, None) == -1
    assert lib.silu_gate_vjp(p(x), p(dy), p(x) + 32, 4, 8, 2, None) == -5      # partial overlap with x
    assert lib.silu_gate_vjp(p(x), p(dy), p(dy), 2, 8, 2, None) == -5          # dx over dy
    assert lib.silu_gate_vjp(p(x), p(dy), p(x), 4, 8, 2, None) == 0            # in place
    torch.cuda.synchronize()
    # autograd through silu_gate_op
    c = I.gate(16, 512, "float32", seed=21)
    xg = c["x"].to(DEV).requires_grad_(True)
    y = R.silu_gate_op(xg)
    dyc = _dy(16, 512, "float32", 22)
    y.backward(dyc.to(DEV))
    torch.cuda.synchronize()
    assert_close(y.detach(), O.silu_gate(c["x"]), "y")
    assert_close(xg.grad, O.silu_gate_vjp(c["x"], dyc), "dx")
