"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU
oracle on the same seeded inputs, for the five workloads and the dispatch
edge cases (every D in the (256, 512] band the CUDA regression report names,
small and large D, misaligned pointers, forced kernel configurations)."""
import sys

import numpy as np
import pytest
import torch

from _parity import DW_TOL, TOL, assert_close, assert_dw_close, to64, ulp_report
from backward_rmsnorm_fwd_two_amd import inputs as I
from oracle import oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def R():
    import backward_rmsnorm_fwd_two_amd as pkg
    return pkg


def _gpu(t):
    return t.to(DEV)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_fwd_vjp(R, x, w, dy, eps, wb, cfg_f=None, cfg_v=None):
    xg, wg, dyg = _gpu(x), _gpu(w), _gpu(dy)
    y = R.rmsnorm_fwd(xg, wg, eps, wb, cfg=cfg_f)
    dx, dw = R.rmsnorm_vjp(xg, wg, dyg, eps, wb, cfg=cfg_v)
    torch.cuda.synchronize()
    return y, dx, dw


def check_fwd_vjp(R, x, w, dy, eps, wb, what, cfg_f=None, cfg_v=None):
    y, dx, dw = run_fwd_vjp(R, x, w, dy, eps, wb, cfg_f, cfg_v)
    yref, _ = O.rmsnorm_fwd(x, w, eps, wb)
    dxref, dwref = O.rmsnorm_vjp(x, w, dy, eps, wb)
    ey = assert_close(y, yref, f"{what} y")
    edx = assert_close(dx, dxref, f"{what} dx")
    edw = assert_dw_close(dw, dwref, f"{what} dw")
    return ey, edx, edw


def test_single_hip_runtime_mapped(R):
    # torch and the library must share one HIP runtime (streams cross over).
    torch.zeros(1, device=DEV)
    maps = open("/proc/self/maps").read().splitlines()
    libs = {line.split()[-1] for line in maps if "libamdhip64" in line}
    assert len(libs) == 1, libs


def test_poc_small_fp32(R):
    c = I.poc_small()
    _say("poc_small fp32 64x512")
    check_fwd_vjp(R, c["x"], c["w"], c["dy"], c["eps"], c["weight_bias"], "poc_small")


def test_poc_8192x4096_fp16(R):
    c = I.poc_8192x4096()
    _say("poc 8192x4096 fp16")
    ey, edx, edw = check_fwd_vjp(R, c["x"], c["w"], c["dy"], c["eps"], c["weight_bias"], "poc")
    _say(f"  max err y {ey:.2e} dx {edx:.2e} dw {edw:.2e}")
    # informational: disagreements with the round-to-nearest-even of the
    # reference (each within tolerance by the checks above)
    y, dx, _ = run_fwd_vjp(R, c["x"], c["w"], c["dy"], c["eps"], c["weight_bias"])
    yref, _ = O.rmsnorm_fwd(c["x"], c["w"], c["eps"], c["weight_bias"])
    dxref, _ = O.rmsnorm_vjp(c["x"], c["w"], c["dy"], c["eps"], c["weight_bias"])
    ry = ulp_report(y, yref, O.round_to(yref, "float16"))
    rdx = ulp_report(dx, dxref, O.round_to(dxref, "float16"))
    _say(f"  y: {ry['differ']} of {ry['n']} differ from RNE(ref), max {ry['max_ulp']} ulp; "
         f"dx: {rdx['differ']} of {rdx['n']}, max {rdx['max_ulp']} ulp")


@pytest.mark.parametrize("B", [1, 4, 8])
@pytest.mark.parametrize("H", [2048, 4096, 8192])
@pytest.mark.parametrize("wb", [0.0, 1.0])
def test_decode_fused_bf16(R, B, H, wb):
    c = I.decode(B, H, wb)
    x, res, w = _gpu(c["x"]), _gpu(c["residual"]), _gpu(c["w"])
    normed, newres = R.fused_add_rmsnorm_fwd(x, res, w, c["eps"], wb)
    torch.cuda.synchronize()
    nref, hres = O.fused_add_rmsnorm_fwd(c["x"], c["residual"], c["w"], c["eps"], wb)
    assert_close(normed, nref, "normed")
    # new_residual is the sum rounded once: bit-exact against the oracle's
    # round-to-nearest-even of the fp64 sum.
    np.testing.assert_array_equal(to64(newres), O.round_to(hres, "bfloat16"))
    # The unfused composition (sum rounded to bf16, then the forward kernel)
    # normalises the rounded sum: it is held to the same tolerance against
    # the oracle of that composition.  (Against the fused reference it also
    # carries the rounding of the sum, which can exceed 4e-3.)
    y2 = R.rmsnorm_fwd(newres, w, c["eps"], wb)
    torch.cuda.synchronize()
    uref, _ = O.rmsnorm_fwd(newres.cpu(), c["w"], c["eps"], wb)
    assert_close(y2, uref, "unfused normed")


AXIS_LIST = [128, 256, 257, 320, 384, 448, 500, 511, 512, 513, 1024]


@pytest.mark.parametrize("D", AXIS_LIST)
def test_axis_sweep_fp16_16384_rows(R, D):
    c = I.axis_sweep(16384, D)
    _say(f"axis sweep D={D}")
    check_fwd_vjp(R, c["x"], c["w"], c["dy"], c["eps"], c["weight_bias"], f"D={D}")


@pytest.mark.parametrize("D", AXIS_LIST)
def test_axis_sweep_single_row_matches_row0(R, D):
    big = I.axis_sweep(16384, D)
    x1, dy1 = big["x"][:1].clone(), big["dy"][:1].clone()
    y1, dx1, dw1 = run_fwd_vjp(R, x1, big["w"], dy1, big["eps"], 0.0)
    yref, _ = O.rmsnorm_fwd(x1, big["w"], big["eps"], 0.0)
    dxref, dwref = O.rmsnorm_vjp(x1, big["w"], dy1, big["eps"], 0.0)
    assert_close(y1, yref, "y rows=1")
    assert_close(dx1, dxref, "dx rows=1")
    assert_dw_close(dw1, dwref, "dw rows=1")
    yb, dxb, _ = run_fwd_vjp(R, big["x"], big["w"], big["dy"], big["eps"], 0.0)
    # row 0 of the full run agrees with the single-row run within tolerance
    assert_close(yb[:1], to64(y1), "row0 vs rows=1 y")
    assert_close(dxb[:1], to64(dx1), "row0 vs rows=1 dx")


@pytest.mark.parametrize("D", list(range(257, 514)))
def test_band_257_513_fp16(R, D):
    # the band of the CUDA regression report, at the sweep's 16384 rows
    c = I.axis_sweep(16384, D, seed=D)
    check_fwd_vjp(R, c["x"], c["w"], c["dy"], c["eps"], c["weight_bias"], f"band D={D}")


@pytest.mark.parametrize("dtype", ["float32", "float16", "bfloat16"])
@pytest.mark.parametrize("rows", [1, 3, 64])
def test_every_D_1_to_1100(R, dtype, rows):
    _say(f"D sweep 1..1100 {dtype} rows={rows}")
    for D in range(1, 1101):
        c = I.generic(rows, D, dtype, seed=D)
        check_fwd_vjp(R, c["x"], c["w"], c["dy"], c["eps"], 0.0, f"{dtype} rows={rows} D={D}")


@pytest.mark.parametrize("dtype", ["float32", "float16", "bfloat16"])
@pytest.mark.parametrize("D", [2048, 4096, 8192, 12289, 16384, 32768, 65536, 65537, 100000])
def test_large_D(R, dtype, D):
    rows = 24 if D <= 16384 else 5
    c = I.generic(rows, D, dtype, seed=7)
    _say(f"large D={D} {dtype}")
    check_fwd_vjp(R, c["x"], c["w"], c["dy"], c["eps"], 0.25, f"{dtype} D={D}")


@pytest.mark.parametrize("dtype", ["float32", "float16", "bfloat16"])
@pytest.mark.parametrize("offset", [1, 2, 3, 4, 5, 6, 7])
def test_misaligned_base_pointers(R, dtype, offset):
    rows, D = 37, 512
    c = I.generic(rows, D, dtype, seed=offset)
    td = I.torch_dtype(dtype)
    n = rows * D

    def shifted(t, off):
        buf = torch.empty(t.numel() + 16, dtype=td, device=DEV)
        v = buf[off:off + t.numel()]
        v.copy_(_gpu(t).reshape(-1))
        return v.view(t.shape)

    x, dy = shifted(c["x"], offset), shifted(c["dy"], (offset + 3) % 8)
    w = shifted(c["w"], (offset + 5) % 8)
    y = torch.empty(n + 16, dtype=td, device=DEV)[offset:offset + n].view(rows, D)
    dx = torch.empty(n + 16, dtype=td, device=DEV)[(offset + 1) % 8:(offset + 1) % 8 + n].view(rows, D)
    R.rmsnorm_fwd(x, w, c["eps"], 0.5, out=y)
    _, dw = R.rmsnorm_vjp(x, w, dy, c["eps"], 0.5, dx=dx)
    torch.cuda.synchronize()
    yref, _ = O.rmsnorm_fwd(c["x"], c["w"], c["eps"], 0.5)
    dxref, dwref = O.rmsnorm_vjp(c["x"], c["w"], c["dy"], c["eps"], 0.5)
    assert_close(y, yref, "y")
    assert_close(dx, dxref, "dx")
    assert_dw_close(dw, dwref)


@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
@pytest.mark.parametrize("D", [4096, 3072, 14336])
@pytest.mark.parametrize("offset", [1, 3])
def test_misaligned_pointers_every_form_bitwise(R, dtype, D, offset):
    """Row vectors are read and written at element alignment, so the plan
    (16-byte vectors; the pipelined fixed-width backward instances at these
    widths) does not depend on the pointers: each form run on buffers shifted
    by a few elements gives bitwise the results of the aligned run, and both
    match the oracle on every element."""
    rows = 600
    c = I.generic(rows, D, dtype, seed=D + offset)
    rng = np.random.default_rng(offset)
    dr = I.normal(rng, (rows, D), 0.0, 0.5, dtype)
    td = I.torch_dtype(dtype)

    def placed(t, off):
        buf = torch.zeros(t.numel() + 16, dtype=td, device=DEV)
        v = buf[off:off + t.numel()]
        v.copy_(_gpu(t).reshape(-1))
        return v.view(t.shape)

    def empty(shape, off):
        n = int(np.prod(shape))
        return torch.empty(n + 16, dtype=td, device=DEV)[off:off + n].view(shape)

    def run(o):
        x, w, dy, drg = (placed(c["x"], o), placed(c["w"], (o + 5) % 8), placed(c["dy"], (o + 3) % 8),
                         placed(dr, (o + 6) % 8))
        out = {}
        out["y"] = R.rmsnorm_fwd(x, w, c["eps"], 0.5, out=empty((rows, D), (o + 1) % 8))
        out["dx"], out["dw"] = R.rmsnorm_vjp(x, w, dy, c["eps"], 0.5, dx=empty((rows, D), (o + 2) % 8))
        out["gy"], out["gdx"], out["gdw"] = R.rmsnorm_fwd_vjp(
            x, w, dy, c["eps"], 0.5, y=empty((rows, D), (o + 4) % 8), dx=empty((rows, D), (o + 7) % 8))
        out["dh"], out["hdw"] = R.fused_add_rmsnorm_vjp(x, w, dy, drg, c["eps"], 0.5,
                                                        dh=empty((rows, D), (o + 1) % 8))
        out["normed"] = empty((rows, D), (o + 2) % 8)
        out["newres"] = empty((rows, D), (o + 3) % 8)
        R.fused_add_rmsnorm_fwd(x, drg, w, c["eps"], 0.5, normed=out["normed"], new_residual=out["newres"])
        return out

    _say(f"misaligned every form {dtype} D={D} offset={offset}")
    for op in (2, 3, 4):
        assert R.query_config(op, rows, D, td, align_bytes=2)["vec_bytes"] == 16
    base, moved = run(0), run(offset)
    torch.cuda.synchronize()
    for k in base:
        a, b = base[k], moved[k]
        iv = torch.int32 if a.dtype == torch.float32 else torch.int16
        assert torch.equal(a.contiguous().view(iv), b.contiguous().view(iv)), k
    yref, _ = O.rmsnorm_fwd(c["x"], c["w"], c["eps"], 0.5)
    dxref, dwref = O.rmsnorm_vjp(c["x"], c["w"], c["dy"], c["eps"], 0.5)
    dhref, hdwref = O.fused_add_rmsnorm_vjp(c["x"], c["w"], c["dy"], dr, c["eps"], 0.5)
    nref, href = O.fused_add_rmsnorm_fwd(c["x"], dr, c["w"], c["eps"], 0.5)
    assert_close(moved["y"], yref, "y")
    assert_close(moved["gy"], yref, "grad y")
    assert_close(moved["dx"], dxref, "dx")
    assert_close(moved["gdx"], dxref, "grad dx")
    assert_dw_close(moved["dw"], dwref)
    assert_dw_close(moved["gdw"], dwref, "grad dw")
    assert_close(moved["dh"], dhref, "dh")
    assert_dw_close(moved["hdw"], hdwref, "fused dw")
    assert_close(moved["normed"], nref, "normed")
    np.testing.assert_array_equal(to64(moved["newres"]), O.round_to(href, dtype))


def _max_block(op, k, nv, itemsize):
    """Mirrors the library's register budget (0 forward, 1 fused forward, 2
    and 3 the VJP forms)."""
    elems = k * nv
    lim = 32 if op == 0 else ((16 if k > 4 else 32) if op == 1 else (8 if k > 4 else 16))
    return 1024 if elems <= lim else (512 if elems <= 2 * lim else 256)


def _legal_configs(op, D, itemsize):
    """Every (lanes, K, vec_bytes, block) combination the register kernels
    accept for D, plus the streaming kernel at two block sizes.  16-byte
    vectors on a row that is not a whole number of them overlap the last
    vector (backward forms then in blocks of at most 512 threads)."""
    out = []
    for vb in (16, 8, 4, 2):
        ovl = (D * itemsize) % vb != 0
        if vb < itemsize or (ovl and (vb != 16 or D * itemsize < 16)):
            continue
        nv = vb // itemsize
        nvec = -(-D // nv)
        for k in (1, 2, 4, 8):
            maxb = _max_block(op, k, nv, itemsize)
            if ovl and op >= 2:
                maxb = min(maxb, 512)
            for lanes in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024):
                if lanes * k < nvec or lanes > maxb:
                    continue
                if lanes * k >= 4 * nvec and lanes > 1:
                    continue  # grossly oversized; covered by smaller cases
                for block in (64, 256, 1024):
                    if block < lanes or block > maxb or block % lanes:
                        continue
                    out.append(dict(lanes_per_row=lanes, vecs_per_lane=k, vec_bytes=vb,
                                    block_threads=block, num_blocks=0))
    for block in (256, 1024):
        out.append(dict(lanes_per_row=0, vecs_per_lane=-1, vec_bytes=0, block_threads=block, num_blocks=0))
    return out


@pytest.mark.parametrize("dtype,D", [("float16", 512), ("float16", 500), ("bfloat16", 384),
                                     ("float32", 320), ("float16", 4096), ("float32", 97)])
def test_forced_configs_agree(R, dtype, D):
    rows = 77
    c = I.generic(rows, D, dtype, seed=D)
    s = 4 if dtype == "float32" else 2
    cfgs = _legal_configs(0, D, s)
    _say(f"forced configs {dtype} D={D}: {len(cfgs)}")
    yref, _ = O.rmsnorm_fwd(c["x"], c["w"], c["eps"], 1.0)
    dxref, dwref = O.rmsnorm_vjp(c["x"], c["w"], c["dy"], c["eps"], 1.0)
    xg, wg, dyg = _gpu(c["x"]), _gpu(c["w"]), _gpu(c["dy"])
    for cfg in cfgs:
        y = R.rmsnorm_fwd(xg, wg, c["eps"], 1.0, cfg=cfg)
        torch.cuda.synchronize()
        assert_close(y, yref, f"fwd {cfg}")
    for cfg in _legal_configs(2, D, s):
        for nb in (0, 1, 3):
            cc = dict(cfg, num_blocks=nb)
            dx, dw = R.rmsnorm_vjp(xg, wg, dyg, c["eps"], 1.0, cfg=cc)
            torch.cuda.synchronize()
            assert_close(dx, dxref, f"vjp dx {cc}")
            assert_dw_close(dw, dwref, f"vjp dw {cc}")


def test_deterministic_bitwise(R):
    c = I.poc_8192x4096(rows=2048)
    xg, wg, dyg = _gpu(c["x"]), _gpu(c["w"]), _gpu(c["dy"])
    outs = []
    for _ in range(2):
        y = R.rmsnorm_fwd(xg, wg, c["eps"], 0.0)
        dx, dw = R.rmsnorm_vjp(xg, wg, dyg, c["eps"], 0.0)
        torch.cuda.synchronize()
        outs.append((y.clone(), dx.clone(), dw.clone()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.float32 else a.view(torch.int32),
                           b.view(torch.uint8) if b.dtype != torch.float32 else b.view(torch.int32))


@pytest.mark.parametrize("dtype", ["float16", "bfloat16", "float32"])
@pytest.mark.parametrize("rows,D", [(5, 300), (64, 4096), (3, 70001)])
def test_canaries_and_nan_prefill(R, dtype, rows, D):
    # Outputs sit between guard bands of a sentinel and are pre-filled with
    # NaN: every element must be written, nothing outside may change.
    td = I.torch_dtype(dtype)
    c = I.generic(rows, D, dtype, seed=3)
    G = 4096
    n = rows * D

    def guarded(numel, dt):
        buf = torch.full((numel + 2 * G,), float("nan"), dtype=dt, device=DEV)
        buf[:G] = 7.0
        buf[G + numel:] = 7.0
        return buf

    ybuf, dxbuf, dwbuf = guarded(n, td), guarded(n, td), guarded(D, torch.float32)
    xg, wg, dyg = _gpu(c["x"]), _gpu(c["w"]), _gpu(c["dy"])
    R.rmsnorm_fwd(xg, wg, c["eps"], 0.0, out=ybuf[G:G + n].view(rows, D))
    R.rmsnorm_vjp(xg, wg, dyg, c["eps"], 0.0, dx=dxbuf[G:G + n].view(rows, D), dw=dwbuf[G:G + D])
    torch.cuda.synchronize()
    for buf, numel in ((ybuf, n), (dxbuf, n), (dwbuf, D)):
        assert torch.all(buf[:G] == 7.0) and torch.all(buf[G + numel:] == 7.0), "guard band written"
        assert not torch.isnan(buf[G:G + numel]).any(), "an output element was not written"


def test_workspace_bounded_and_no_allocation(R):
    # The dw partial buffer is bounded independently of rows: never a
    # [rows, D] temporary, and the library allocates no device memory.
    D = 4096
    sizes = [R.rmsnorm_vjp_workspace_bytes(r, D, torch.float16) for r in (1, 512, 8192, 65536, 1 << 20)]
    assert max(sizes) <= 2048 * D * 4 + 256
    assert sizes[-1] == sizes[-2]
    c = I.poc_8192x4096()
    xg, wg, dyg = _gpu(c["x"]), _gpu(c["w"]), _gpu(c["dy"])
    dx = torch.empty_like(xg)
    dw = torch.empty(D, dtype=torch.float32, device=DEV)
    ws = R.workspace_for(8192, D, torch.float16, DEV)
    assert ws.numel() <= 8192 * D * 2 // 4   # far below a [rows, D] temporary
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    R.rmsnorm_vjp(xg, wg, dyg, c["eps"], 0.0, dx=dx, dw=dw, workspace=ws)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == before


def test_rows_zero(R):
    x = torch.empty(0, 64, dtype=torch.float16, device=DEV)
    w = torch.ones(64, dtype=torch.float16, device=DEV)
    y = R.rmsnorm_fwd(x, w)
    assert y.shape == (0, 64)
    dw = torch.full((64,), float("nan"), device=DEV)
    R.rmsnorm_vjp(x, w, x, dw=dw)
    torch.cuda.synchronize()
    assert torch.all(dw == 0)


def test_nan_inf_propagation(R):
    c = I.generic(6, 256, "float16", seed=9)
    x = c["x"].clone()
    x[1, 5] = float("nan")
    x[3, 7] = float("inf")
    dy = c["dy"].clone()
    dy[4, 9] = float("nan")
    y, dx, dw = run_fwd_vjp(R, x, c["w"], dy, c["eps"], 0.0)
    yref, _ = O.rmsnorm_fwd(x, c["w"], c["eps"], 0.0)
    dxref, dwref = O.rmsnorm_vjp(x, c["w"], dy, c["eps"], 0.0)
    assert_close(y, yref, "y")
    assert_close(dx, dxref, "dx")
    assert np.array_equal(np.isnan(to64(dw)), np.isnan(dwref))


def test_zero_row_eps_zero_gives_nan_like_oracle(R):
    x = torch.zeros(2, 128, dtype=torch.float32)
    x[1] = 1.0
    w = torch.ones(128)
    dy = torch.ones(2, 128)
    y, dx, dw = run_fwd_vjp(R, x, w, dy, 0.0, 0.0)
    yref, _ = O.rmsnorm_fwd(x, w, 0.0, 0.0)
    dxref, _ = O.rmsnorm_vjp(x, w, dy, 0.0, 0.0)
    assert np.array_equal(np.isnan(to64(y)), np.isnan(yref))
    assert np.array_equal(np.isnan(to64(dx)), np.isnan(dxref))


def test_error_codes(R):
    import ctypes
    lib = R.raw
    x = torch.zeros(4, 64, dtype=torch.float16, device=DEV)
    w = torch.ones(64, dtype=torch.float16, device=DEV)
    y = torch.empty_like(x)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: t.data_ptr()
    assert lib.rmsnorm_fwd(None, p(w), p(y), 4, 64, 1, 1e-5, 0.0, s) == -1
    assert lib.rmsnorm_fwd(p(x), p(w), p(y), -1, 64, 1, 1e-5, 0.0, s) == -2
    assert lib.rmsnorm_fwd(p(x), p(w), p(y), 4, 0, 1, 1e-5, 0.0, s) == -2
    assert lib.rmsnorm_fwd(p(x), p(w), p(y), 4, 64, 7, 1e-5, 0.0, s) == -3
    # y one row into x: a partial overlap (y == x exactly would be in place)
    assert lib.rmsnorm_fwd(p(x), p(w), p(x) + 128, 3, 64, 1, 1e-5, 0.0, s) == -5
    assert lib.rmsnorm_fwd(p(x) + 1, p(w), p(y), 2, 64, 1, 1e-5, 0.0, s) == -7
    dx = torch.empty_like(x)
    dw = torch.empty(64, dtype=torch.float32, device=DEV)
    assert lib.rmsnorm_vjp(p(x), p(w), p(x), p(dx), p(dw), None, 0, 4, 64, 1, 1e-5, 0.0, s) == -4 or \
        R.rmsnorm_vjp_workspace_bytes(4, 64, torch.float16) <= 256
    assert lib.rmsnorm_vjp(p(x), p(w), p(x), p(x) + 128, p(dw), None, 0, 3, 64, 1, 1e-5, 0.0, s) == -5
    assert lib.rmsnorm_vjp(p(x), p(w), p(x), p(dx), p(x), None, 0, 4, 64, 1, 1e-5, 0.0, s) == -5
    assert lib.rmsnorm_vjp(p(x), p(w), p(x), p(dx), None, None, 0, 4, 64, 1, 1e-5, 0.0, s) == -1
    # a workspace smaller than the plan needs is refused before any launch
    x2 = torch.zeros(8192, 64, dtype=torch.float16, device=DEV)
    dx2 = torch.empty_like(x2)
    tiny = torch.empty(256, dtype=torch.uint8, device=DEV)
    need = R.rmsnorm_vjp_workspace_bytes(8192, 64, torch.float16)
    assert need > 256
    assert lib.rmsnorm_vjp(p(x2), p(w), p(x2), p(dx2), p(dw), p(tiny), 8, 8192, 64, 1,
                           1e-5, 0.0, s) == -4
    torch.cuda.synchronize()


def test_prefill_fused_then_vjp_bf16_full_size(R):
    # [32768, 8192] bf16, weight_bias 1 (Gemma), in the launch configuration
    # the benchmark times.  Every row is checked, streaming the oracle in row
    # chunks: normed within tolerance, new_residual bit-exactly, dx within
    # tolerance, and dw over every row (dw is additive over row splits).  The
    # VJP runs on the GPU's new_residual, checked first in the same chunk.
    _say("prefill 32768x8192 bf16: generating")
    c = I.prefill()
    rows, D = c["x"].shape
    x, res, w, dy = _gpu(c["x"]), _gpu(c["residual"]), _gpu(c["w"]), _gpu(c["dy"])
    normed, newres = R.fused_add_rmsnorm_fwd(x, res, w, c["eps"], c["weight_bias"])
    dx, dw = R.rmsnorm_vjp(newres, w, dy, c["eps"], c["weight_bias"])
    torch.cuda.synchronize()
    del x, res, dy
    _say("prefill: every row against the oracle")
    dwref = np.zeros(D)
    CH = 2048
    for r0 in range(0, rows, CH):
        sl = slice(r0, r0 + CH)
        nref, href = O.fused_add_rmsnorm_fwd(c["x"][sl], c["residual"][sl], c["w"], c["eps"], c["weight_bias"])
        assert_close(normed[sl], nref, f"normed rows {r0}..{r0 + CH}")
        nr = newres[sl].cpu()
        np.testing.assert_array_equal(to64(nr), O.round_to(href, "bfloat16"), f"new_residual rows {r0}..")
        dxref, part = O.rmsnorm_vjp(nr, c["w"], c["dy"][sl], c["eps"], c["weight_bias"])
        assert_close(dx[sl], dxref, f"dx rows {r0}..{r0 + CH}")
        dwref += part
    assert_dw_close(dw, dwref, "dw (all rows)")


def test_max_D_and_beyond(R):
    Dmax = R.RMSN_MAX_D
    c = I.generic(2, Dmax, "float16", seed=1)
    check_fwd_vjp(R, c["x"], c["w"], c["dy"], c["eps"], 0.0, "D=2^24")
    x = torch.zeros(1, Dmax + 1, dtype=torch.float16, device=DEV)
    w = torch.zeros(Dmax + 1, dtype=torch.float16, device=DEV)
    with pytest.raises(R.RMSNormError) as ei:
        R.rmsnorm_fwd(x, w)
    assert ei.value.status == -2


# ------------------------------------------------------------- grad call

def check_grad(R, x, w, dy, eps, wb, what, cfg=None):
    xg, wg, dyg = _gpu(x), _gpu(w), _gpu(dy)
    y, dx, dw = R.rmsnorm_fwd_vjp(xg, wg, dyg, eps, wb, cfg=cfg)
    torch.cuda.synchronize()
    yref, _ = O.rmsnorm_fwd(x, w, eps, wb)
    dxref, dwref = O.rmsnorm_vjp(x, w, dy, eps, wb)
    assert_close(y, yref, f"{what} grad y")
    assert_close(dx, dxref, f"{what} grad dx")
    assert_dw_close(dw, dwref, f"{what} grad dw")
    return y, dx, dw


def test_grad_call_poc_small_and_8192x4096(R):
    c = I.poc_small()
    check_grad(R, c["x"], c["w"], c["dy"], c["eps"], c["weight_bias"], "poc_small")
    c = I.poc_8192x4096()
    _, dx, dw = check_grad(R, c["x"], c["w"], c["dy"], c["eps"], c["weight_bias"], "poc")
    # the grad call's dx is the VJP's, bit for bit (same row geometry, same
    # arithmetic); dw too when both use the same grid (the same partial rows)
    dx2, dw2 = R.rmsnorm_vjp(_gpu(c["x"]), _gpu(c["w"]), _gpu(c["dy"]), c["eps"], c["weight_bias"])
    torch.cuda.synchronize()
    assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16))
    rows, D = c["x"].shape
    if R.query_config(3, rows, D, dx.dtype)["num_blocks"] == R.query_config(2, rows, D, dx.dtype)["num_blocks"]:
        assert torch.equal(dw.view(torch.int32), dw2.view(torch.int32))


@pytest.mark.parametrize("D", AXIS_LIST + [4096, 8192, 70001])
@pytest.mark.parametrize("dtype", ["float16", "bfloat16", "float32"])
def test_grad_call_axis_sweep(R, D, dtype):
    rows = 1024 if D <= 8192 else 3
    c = I.generic(rows, D, dtype, seed=D)
    check_grad(R, c["x"], c["w"], c["dy"], c["eps"], 1.0, f"{dtype} D={D}")


@pytest.mark.parametrize("dtype,D", [("float16", 512), ("bfloat16", 500), ("float32", 97)])
def test_grad_call_forced_configs(R, dtype, D):
    rows = 77
    c = I.generic(rows, D, dtype, seed=D)
    s = 4 if dtype == "float32" else 2
    for cfg in _legal_configs(2, D, s):
        for nb in (0, 3):
            check_grad(R, c["x"], c["w"], c["dy"], c["eps"], 0.5, f"{cfg}", cfg=dict(cfg, num_blocks=nb))


def test_grad_call_rows_zero_and_errors(R):
    import ctypes
    x = torch.empty(0, 64, dtype=torch.float16, device=DEV)
    w = torch.ones(64, dtype=torch.float16, device=DEV)
    dw = torch.full((64,), float("nan"), device=DEV)
    R.rmsnorm_fwd_vjp(x, w, x, dw=dw)
    torch.cuda.synchronize()
    assert torch.all(dw == 0)
    x = torch.zeros(4, 64, dtype=torch.float16, device=DEV)
    dx = torch.empty_like(x)
    dwv = torch.empty(64, dtype=torch.float32, device=DEV)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: t.data_ptr()
    lib = R.raw
    assert lib.rmsnorm_fwd_vjp(p(x), p(w), p(x), None, p(dx), p(dwv), None, 0, 4, 64, 1, 1e-5, 0.0, s) == -1
    assert lib.rmsnorm_fwd_vjp(p(x), p(w), p(x), p(dx), p(dx), p(dwv), None, 0, 4, 64, 1, 1e-5, 0.0, s) == -5
    assert lib.rmsnorm_fwd_vjp(p(x), p(w), p(x), p(x) + 128, p(dx), p(dwv), None, 0, 3, 64, 1, 1e-5, 0.0, s) == -5
    torch.cuda.synchronize()


# -------------------------------------- fused backward (residual gradient)

def check_fused_vjp(R, h, w, dy, dr, eps, wb, what, cfg=None):
    hg, wg, dyg, drg = _gpu(h), _gpu(w), _gpu(dy), _gpu(dr)
    dh, dw = R.fused_add_rmsnorm_vjp(hg, wg, dyg, drg, eps, wb, cfg=cfg)
    torch.cuda.synchronize()
    dhref, dwref = O.fused_add_rmsnorm_vjp(h, w, dy, dr, eps, wb)
    assert_close(dh, dhref, f"{what} dh")
    assert_dw_close(dw, dwref, f"{what} dw")
    return dh, dw


@pytest.mark.parametrize("dtype", ["bfloat16", "float16", "float32"])
@pytest.mark.parametrize("rows,D", [(1, 2048), (8, 4096), (512, 8192), (300, 512), (77, 513), (5, 70001)])
def test_fused_vjp_parity(R, dtype, rows, D):
    c = I.generic(rows, D, dtype, seed=rows + D)
    rng = np.random.default_rng(D)
    dr = I.normal(rng, (rows, D), 0.0, 0.5, dtype)
    check_fused_vjp(R, c["x"], c["w"], c["dy"], dr, c["eps"], 1.0, f"{dtype} {rows}x{D}")


def test_fused_vjp_zero_residual_grad_equals_vjp_bitwise(R):
    c = I.generic(1000, 4096, "bfloat16", seed=3)
    hg, wg, dyg = _gpu(c["x"]), _gpu(c["w"]), _gpu(c["dy"])
    dh, dw = R.fused_add_rmsnorm_vjp(hg, wg, dyg, torch.zeros_like(hg), c["eps"], 1.0)
    dx, dw2 = R.rmsnorm_vjp(hg, wg, dyg, c["eps"], 1.0)
    torch.cuda.synchronize()
    assert torch.equal(dh.view(torch.int16), dx.view(torch.int16))
    assert torch.equal(dw.view(torch.int32), dw2.view(torch.int32))


@pytest.mark.parametrize("dtype,D", [("bfloat16", 512), ("float16", 500), ("float32", 97)])
def test_fused_vjp_forced_configs(R, dtype, D):
    rows = 53
    c = I.generic(rows, D, dtype, seed=D)
    dr = I.normal(np.random.default_rng(1), (rows, D), 0.0, 1.0, dtype)
    s = 4 if dtype == "float32" else 2
    for cfg in _legal_configs(3, D, s):
        check_fused_vjp(R, c["x"], c["w"], c["dy"], dr, c["eps"], 0.0, f"{cfg}", cfg=dict(cfg, num_blocks=3))


def test_prefill_full_training_step_bf16(R):
    # The prefill workload end to end: fused forward, then its backward with a
    # residual-stream gradient (seeded N(0, 0.01)).  Every row against the
    # oracle in row chunks: normed, new_residual (bit-exact), dh, and dw.
    _say("prefill training step 32768x8192 bf16")
    c = I.prefill()
    rows, D = c["x"].shape
    dr_cpu = I.normal(np.random.default_rng(11), (rows, D), 0.0, 0.01, "bfloat16")
    x, res, w, dy = _gpu(c["x"]), _gpu(c["residual"]), _gpu(c["w"]), _gpu(c["dy"])
    normed, h = R.fused_add_rmsnorm_fwd(x, res, w, c["eps"], c["weight_bias"])
    del x, res
    dr = _gpu(dr_cpu)
    dh, dw = R.fused_add_rmsnorm_vjp(h, w, dy, dr, c["eps"], c["weight_bias"])
    torch.cuda.synchronize()
    del dy, dr
    dwref = np.zeros(D)
    CH = 2048
    for r0 in range(0, rows, CH):
        sl = slice(r0, r0 + CH)
        nref, href = O.fused_add_rmsnorm_fwd(c["x"][sl], c["residual"][sl], c["w"], c["eps"], c["weight_bias"])
        assert_close(normed[sl], nref, f"normed rows {r0}..{r0 + CH}")
        hs = h[sl].cpu()
        np.testing.assert_array_equal(to64(hs), O.round_to(href, "bfloat16"), f"new_residual rows {r0}..")
        dhref, part = O.fused_add_rmsnorm_vjp(hs, c["w"], c["dy"][sl], dr_cpu[sl], c["eps"], c["weight_bias"])
        assert_close(dh[sl], dhref, f"dh rows {r0}..{r0 + CH}")
        dwref += part
    assert_dw_close(dw, dwref, "dw (all rows)")


# ------------------------------------------------- fused forward coverage

def check_fused(R, x, res, w, eps, wb, what, cfg=None, out=None):
    xg, rg, wg = _gpu(x), _gpu(res), _gpu(w)
    if out is None:
        normed, newres = R.fused_add_rmsnorm_fwd(xg, rg, wg, eps, wb, cfg=cfg)
    else:
        normed, newres = R.fused_add_rmsnorm_fwd(xg, rg, wg, eps, wb, normed=out[0], new_residual=out[1], cfg=cfg)
    torch.cuda.synchronize()
    nref, href = O.fused_add_rmsnorm_fwd(x, res, w, eps, wb)
    assert_close(normed, nref, f"{what} normed")
    np.testing.assert_array_equal(to64(newres).reshape(href.shape),
                                  O.round_to(href, str(x.dtype).replace("torch.", "")), err_msg=f"{what} new_residual")


@pytest.mark.parametrize("dtype", ["float32", "float16", "bfloat16"])
def test_fused_every_D_1_to_700(R, dtype):
    for D in range(1, 701):
        c = I.generic(3, D, dtype, seed=D)
        check_fused(R, c["x"], c["residual"], c["w"], c["eps"], 1.0, f"{dtype} D={D}")


@pytest.mark.parametrize("dtype,D", [("bfloat16", 512), ("float16", 500), ("float32", 97), ("bfloat16", 8192)])
def test_fused_forced_configs(R, dtype, D):
    rows = 37
    c = I.generic(rows, D, dtype, seed=D)
    s = 4 if dtype == "float32" else 2
    cfgs = _legal_configs(1, D, s)
    _say(f"fused forced configs {dtype} D={D}: {len(cfgs)}")
    for cfg in cfgs:
        check_fused(R, c["x"], c["residual"], c["w"], c["eps"], 0.0, f"{cfg}", cfg=cfg)


@pytest.mark.parametrize("dtype", ["float32", "float16", "bfloat16"])
@pytest.mark.parametrize("offset", [1, 3, 5])
def test_fused_misaligned(R, dtype, offset):
    rows, D = 21, 1024
    c = I.generic(rows, D, dtype, seed=offset)
    td = I.torch_dtype(dtype)
    n = rows * D

    def shifted(t, off):
        buf = torch.empty(t.numel() + 16, dtype=td, device=DEV)
        v = buf[off:off + t.numel()]
        v.copy_(_gpu(t).reshape(-1))
        return v.view(t.shape)

    x, res, w = shifted(c["x"], offset), shifted(c["residual"], (offset + 2) % 8), shifted(c["w"], 0)
    normed = torch.empty(n + 16, dtype=td, device=DEV)[offset:offset + n].view(rows, D)
    newres = torch.empty(n + 16, dtype=td, device=DEV)[7 - offset:7 - offset + n].view(rows, D)
    R.fused_add_rmsnorm_fwd(x, res, w, c["eps"], 1.0, normed=normed, new_residual=newres)
    torch.cuda.synchronize()
    nref, href = O.fused_add_rmsnorm_fwd(c["x"], c["residual"], c["w"], c["eps"], 1.0)
    assert_close(normed, nref, "normed")
    np.testing.assert_array_equal(to64(newres), O.round_to(href, dtype))
