"""GPU: the two VJP row loops.  Blocks of at most 256 threads (or a whole
512-lane row in a 512-thread block) whose rows are exactly lanes x K
vectors run the software-pipelined loop (unmasked; a ragged last row group
is masked on the loop's exit path), and so do rows of a whole number of
waves that is not a power of two (wave rows: 3, 5, 6, 7, 10 waves ...,
one to four rows per block); every other register-resident shape runs
the plain loop.  Checks, on both sides of that rule: parity with the
fp64 oracle on every row (the last row group of every block goes through
the loop's exit path) and dw over all rows; dx of
the pipelined loop bit-identical to the plain loop's (forced through a
512-thread block, same row geometry) for the VJP and the fused backward;
and for wave rows, the plan's geometry and dx bit-identical across rows
per block and grids.  Few rows (rows x D x itemsize <= 32 KiB) take one
vector per lane in one block that loops over them: plan, every form against
the oracle, and the grad call's dx and dw equal to the VJP's."""
import sys

import numpy as np
import pytest
import torch

from _parity import assert_close, assert_dw_close
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


# (rows, D, dtype): pipelined shapes (D tiles exactly; full or ragged last
# row groups) next to plain ones (D that does not tile)
CASES = [
    (8192, 4096, "float16"),    # pipelined: 512 lanes x 1 vector, one row per block
    (8191, 4096, "float16"),    # still pipelined (one slot), odd row count
    (4096, 512, "bfloat16"),    # pipelined: 32 lanes, 8 row slots
    (4093, 512, "bfloat16"),    # pipelined, 8 slots: the last group is ragged (masked exit path)
    (2048, 1024, "float32"),    # pipelined: 128 lanes x 2 x 4 floats, 2 slots
    (2047, 1024, "float32"),    # pipelined, ragged last group
    (3000, 3072, "float16"),    # wave rows: 3 waves x 2 vectors, two rows per block
    (1200, 1536, "bfloat16"),   # wave rows: 3 waves x 1 vector, four rows per block
    (1202, 1536, "float16"),    # wave rows, four rows per block, rows % 4 == 2: ragged last group
    (601, 2560, "float16"),     # wave rows: 5 waves x 1, two rows per block, odd rows: ragged
    (1001, 5120, "bfloat16"),   # wave rows: 10 waves x 1
    (700, 6144, "float16"),     # wave rows: 12 waves x 1
    (513, 3584, "bfloat16"),    # wave rows: 7 waves x 1, two blocks per CU
    (257, 7168, "float16"),     # wave rows: 14 waves x 1
    (300, 10240, "bfloat16"),   # wave rows: 10 waves x 2
    (300, 4608, "bfloat16"),    # wave rows: 9 waves x 1
    (200, 9216, "float16"),     # wave rows: 9 waves x 2
    (900, 3072, "float32"),     # wave rows: 6 waves x 2 x 4 floats
    (333, 7168, "float32"),     # wave rows: 14 waves x 2 x 4 floats
    (130, 12288, "float16"),    # 12 waves x 2, one row per block
    (100, 14336, "bfloat16"),   # wide: 7 waves x 4 vectors
    (99, 16384, "float16"),     # wide: 8 waves x 4 vectors (512 lanes)
    (64, 12288, "float32"),     # plain loop: 1024 lanes x 3 of 4 vectors (no wave instance)
    (200, 8192, "float32"),     # fp32: 512 lanes x 4 vectors, one row per block
    (1000, 1024, "bfloat16"),   # pipelined: 64 lanes, 4 slots
    (1024, 8192, "bfloat16"),   # pipelined: a 1024-lane row (one vector per lane) per block
    (1023, 8192, "float16"),    # pipelined, odd row count
    (512, 4096, "float32"),     # pipelined: 512 lanes x 2 x 4 floats
    (300, 11264, "bfloat16"),   # wave rows: 11 waves x 2
    (401, 6656, "float16"),     # wave rows: 13 waves x 1
    (350, 7680, "bfloat16"),    # wave rows: 15 waves x 1
    (300, 5632, "float32"),     # wave rows: 11 waves x 2 x 4 floats
    (257, 3328, "float32"),     # wave rows: 13 waves x 1 x 4 floats
]


@pytest.mark.parametrize("rows,D,dtype", CASES)
def test_vjp_paths_match_oracle(R, rows, D, dtype):
    _say(f"vjp paths rows={rows} D={D} {dtype}")
    c = I.generic(rows, D, dtype, seed=rows + 7 * D)
    x, w, dy, dr = (c[k].to(DEV) for k in ("x", "w", "dy", "residual"))
    dx, dw = R.rmsnorm_vjp(x, w, dy, c["eps"], 0.5)
    dh, dwf = R.fused_add_rmsnorm_vjp(x, w, dy, dr, c["eps"], 0.5)
    torch.cuda.synchronize()
    # every row (dx, dh) and dw over every row, in slabs
    dwref = np.zeros(D)
    for r0 in range(0, rows, 1024):
        sl = slice(r0, r0 + 1024)
        dxref, part = O.rmsnorm_vjp(c["x"][sl], c["w"], c["dy"][sl], c["eps"], 0.5)
        assert_close(dx[sl], dxref, f"dx rows {r0}..")
        dhref, _ = O.fused_add_rmsnorm_vjp(c["x"][sl], c["w"], c["dy"][sl], c["residual"][sl], c["eps"], 0.5)
        assert_close(dh[sl], dhref, f"dh rows {r0}..")
        dwref += part
    assert_dw_close(dw, dwref, "dw")
    assert_dw_close(dwf, dwref, "fused dw")


# The shapes of CASES whose pipelined row geometry also has a plain-loop
# instance in a wider block (power-of-two lanes up to 512, at most 16
# elements per lane); wave rows, four-vector rows and 16-bit rows of 1024
# vectors (1024 lanes x 1, one row per block) have no plain-loop twin at
# their width, and their dx is checked bitwise across rows per block and
# grids by test_wave_rows_geometry_and_bitwise and the repeat tests.
PLAIN_TWIN = [c for c in CASES if (c[0], c[1]) in {
    (8192, 4096), (8191, 4096), (4096, 512), (4093, 512), (2048, 1024), (2047, 1024), (200, 8192),
    (1000, 1024), (512, 4096)}]


@pytest.mark.parametrize("rows,D,dtype", PLAIN_TWIN)
def test_pipelined_dx_equals_plain_loop(R, rows, D, dtype):
    """dx does not depend on the grid or on which loop ran: forcing a block
    with two row slots (same lanes, vectors and load width) selects the plain
    loop."""
    c = I.generic(rows, D, dtype, seed=3 * rows + D)
    x, w, dy, dr = (c[k].to(DEV) for k in ("x", "w", "dy", "residual"))
    q = R.query_config(2, rows, D, x.dtype)
    elems = q["vecs_per_lane"] * q["vec_bytes"] // x.element_size()
    assert q["vecs_per_lane"] > 0 and _is_pow2(q["lanes_per_row"]) and q["lanes_per_row"] <= 512, q
    assert elems <= 16, q
    plain = dict(lanes_per_row=q["lanes_per_row"], vecs_per_lane=q["vecs_per_lane"],
                 vec_bytes=q["vec_bytes"], block_threads=max(512, 2 * q["lanes_per_row"]), num_blocks=0)
    _say(f"pipelined vs plain rows={rows} D={D} {dtype} plan={q}")
    dx_a, _ = R.rmsnorm_vjp(x, w, dy, c["eps"], 0.0)
    dx_b, _ = R.rmsnorm_vjp(x, w, dy, c["eps"], 0.0, cfg=plain)
    dh_a, _ = R.fused_add_rmsnorm_vjp(x, w, dy, dr, c["eps"], 1.0)
    dh_b, _ = R.fused_add_rmsnorm_vjp(x, w, dy, dr, c["eps"], 1.0, cfg=plain)
    _, dx_g, _ = R.rmsnorm_fwd_vjp(x, w, dy, c["eps"], 0.0)
    torch.cuda.synchronize()
    assert torch.equal(dx_a, dx_b)
    assert torch.equal(dh_a, dh_b)
    assert torch.equal(dx_g, dx_a)


def _is_pow2(v):
    return v > 0 and (v & (v - 1)) == 0


def _grid(groups, cap):
    """The backward forms' persistent grid: at most `cap` blocks, and at
    least two row groups per block whenever there are two (so the dw partial
    rows are never one per row)."""
    g = min(groups, cap)
    if groups > 1:
        g = min(g, (groups + 1) // 2)
    return max(g, 1)


# (rows, D, dtype, lanes, vectors per lane, rows per block, blocks per CU) of
# the automatic plan for the VJP; None: not wave rows
WAVE = [
    (3000, 3072, "float16", 192, 2, 2, 1),
    (1200, 1536, "bfloat16", 192, 1, 4, 1),
    (1202, 1536, "float16", 192, 1, 4, 1),
    (601, 2560, "float16", 320, 1, 2, 1),
    (1001, 5120, "bfloat16", 640, 1, 1, 1),
    (700, 6144, "float16", 768, 1, 1, 1),
    (257, 7168, "float16", 896, 1, 1, 1),
    (513, 3584, "bfloat16", 448, 1, 1, 2),
    (300, 10240, "bfloat16", 640, 2, 1, 1),
    (300, 4608, "bfloat16", 576, 1, 1, 1),
    (200, 9216, "float16", 576, 2, 1, 1),
    (900, 3072, "float32", 384, 2, 1, 1),
    (333, 7168, "float32", 896, 2, 1, 1),
    (130, 12288, "float16", 768, 2, 1, 1),
    (100, 14336, "bfloat16", 448, 4, 1, 1),
    (99, 16384, "float16", 512, 4, 1, 1),
    (64, 12288, "float32", None, None, None, None),
    (200, 8192, "float32", 512, 4, 1, 1),
    (300, 11264, "bfloat16", 704, 2, 1, 1),
    (401, 6656, "float16", 832, 1, 1, 1),
    (350, 7680, "bfloat16", 960, 1, 1, 1),
    (300, 5632, "float32", 704, 2, 1, 1),
    (257, 3328, "float32", 832, 1, 1, 1),
]


@pytest.mark.parametrize("rows,D,dtype,lanes,k,slots,per_cu", WAVE)
def test_wave_rows_geometry_and_bitwise(R, rows, D, dtype, lanes, k, slots, per_cu):
    """The automatic plan tiles rows of a whole number of waves exactly (lanes
    x K = D / vector elements) with the rows per block and grid of its
    in-flight rule; dx and the fused backward's dh do not depend on the rows
    per block or on the grid (each row is reduced inside its own slot)."""
    c = I.generic(rows, D, dtype, seed=5 * rows + D)
    x, w, dy, dr = (c[kk].to(DEV) for kk in ("x", "w", "dy", "residual"))
    q = R.query_config(2, rows, D, x.dtype)
    _say(f"wave rows rows={rows} D={D} {dtype} plan={q}")
    nvec = D * x.element_size() // 16
    if lanes is None:
        assert _is_pow2(q["lanes_per_row"]), q
        return
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    # wide 16-bit rows (four vectors per lane) hold one row per block
    wide = k == 4 and dtype != "float32"
    assert q["vec_bytes"] == 16 and q["lanes_per_row"] == lanes and q["vecs_per_lane"] == k, q
    assert lanes * k == nvec and (k == 4 or not _is_pow2(lanes))
    assert q["block_threads"] == slots * lanes, q
    groups = (rows + slots - 1) // slots
    assert q["num_blocks"] == _grid(groups, per_cu * cus), q
    # the fused backward and the grad call lay these rows out alike
    qf = R.query_config(4, rows, D, x.dtype)
    assert qf["lanes_per_row"] == lanes and qf["vecs_per_lane"] == k, qf
    dx_a, dw_a = R.rmsnorm_vjp(x, w, dy, c["eps"], 0.25)
    dh_a, _ = R.fused_add_rmsnorm_vjp(x, w, dy, dr, c["eps"], 1.0)
    # the grad call gives the VJP's dx bit for bit, dw too on the same grid
    # (fp16 included: every kernel rounds dx from the same fp32 value)
    qg = R.query_config(3, rows, D, x.dtype)
    _, dx_g, dw_g = R.rmsnorm_fwd_vjp(x, w, dy, c["eps"], 0.25)
    torch.cuda.synchronize()
    assert (qg["lanes_per_row"], qg["vecs_per_lane"]) == (lanes, k), qg
    # the grad call stores as many rows as it reads (y and dx for x and dy):
    # one persistent block per CU at every width (the VJP may take two)
    gslots = qg["block_threads"] // lanes
    assert qg["num_blocks"] == _grid((rows + gslots - 1) // gslots, cus), qg
    assert torch.equal(dx_g, dx_a)
    if qg["num_blocks"] == q["num_blocks"]:
        assert torch.equal(dw_g, dw_a)
    variants = [dict(lanes_per_row=lanes, vecs_per_lane=k, vec_bytes=16, block_threads=lanes, num_blocks=37)]
    for s in (2, 4):
        if not wide and s * lanes <= 768:
            variants.append(dict(lanes_per_row=lanes, vecs_per_lane=k, vec_bytes=16,
                                 block_threads=s * lanes, num_blocks=0))
    for v in variants:
        dx_b, dw_b = R.rmsnorm_vjp(x, w, dy, c["eps"], 0.25, cfg=v)
        dh_b, _ = R.fused_add_rmsnorm_vjp(x, w, dy, dr, c["eps"], 1.0, cfg=v)
        torch.cuda.synchronize()
        assert torch.equal(dx_a, dx_b), v
        assert torch.equal(dh_a, dh_b), v
    dhref, _ = O.fused_add_rmsnorm_vjp(c["x"], c["w"], c["dy"], c["residual"], c["eps"], 1.0)
    assert_close(dh_a, dhref, "dh")
    dxref, dwref = O.rmsnorm_vjp(c["x"], c["w"], c["dy"], c["eps"], 0.25)
    assert_close(dx_a, dxref, "dx")
    assert_close(dx_b, dxref, "dx (forced geometry)")
    assert_dw_close(dw_b, dwref, "dw (forced geometry)")
    assert_dw_close(dw_a, dwref, "dw")


@pytest.mark.parametrize("rows,D,dtype", [(1200, 20480, "bfloat16"), (1600, 32768, "float16"),
                                          (1100, 20480, "float32")])
def test_streaming_vjp_grid_follows_occupancy(R, rows, D, dtype):
    """Rows past the register path stream (one 1024-thread block per row
    iteration, dw in registers) once there are enough of them (fewer take
    the column split); the instances that keep 4 vectors of dw per thread
    (16-bit) or 8 (fp32) hold more than 64 VGPRs, so only one such block
    resides per CU and the persistent grid is one block per CU (a second
    round of blocks would only add partial rows), at most half the rows.
    Parity with the oracle at that grid."""
    c = I.generic(rows, D, dtype, seed=rows + D)
    x, w, dy, dr = (c[k].to(DEV) for k in ("x", "w", "dy", "residual"))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for op in (2, 3, 4):
        q = R.query_config(op, rows, D, x.dtype)
        _say(f"streaming vjp op={op} rows={rows} D={D} {dtype} plan={q}")
        assert q["vecs_per_lane"] == -1 and q["block_threads"] == 1024, q
        assert q["num_blocks"] == _grid(rows, cus), q
    dx, dw = R.rmsnorm_vjp(x, w, dy, c["eps"], 0.5)
    dh, dwf = R.fused_add_rmsnorm_vjp(x, w, dy, dr, c["eps"], 0.5)
    torch.cuda.synchronize()
    dxref, dwref = O.rmsnorm_vjp(c["x"], c["w"], c["dy"], c["eps"], 0.5)
    assert_close(dx, dxref, "dx")
    assert_dw_close(dw, dwref, "dw")
    dhref, _ = O.fused_add_rmsnorm_vjp(c["x"], c["w"], c["dy"], c["residual"], c["eps"], 0.5)
    assert_close(dh, dhref, "dh")
    assert_dw_close(dwf, dwref, "fused dw")


# (rows, D, dtype, op -> expected (lanes, vectors per lane) of the automatic
# backward plan): dense 16-bit rows of 1536..2048 vectors without a pipelined
# instance run the plain loop on 256 lanes x 8, one block per CU; sparser
# rows that 9 waves x 2 hold (1025..1152 vectors) run the duplicate-slot
# instance there
EIGHT = [
    (200, 13312, "bfloat16", {2: (256, 8), 3: (256, 8), 4: (256, 8)}),
    (150, 14336, "float16", {2: (448, 4), 3: (448, 4), 4: (448, 4)}),
    (130, 16384, "bfloat16", {2: (512, 4), 3: (512, 4), 4: (512, 4)}),
    (300, 8200, "float16", {2: (576, 2), 3: (576, 2), 4: (576, 2)}),
]


@pytest.mark.parametrize("rows,D,dtype,plans", EIGHT)
def test_dense_wide_rows_eight_vectors(R, rows, D, dtype, plans):
    c = I.generic(rows, D, dtype, seed=rows * 3 + D)
    x, w, dy, dr = (c[k].to(DEV) for k in ("x", "w", "dy", "residual"))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for op, (lanes, k) in plans.items():
        q = R.query_config(op, rows, D, x.dtype)
        _say(f"eight-wide op={op} rows={rows} D={D} {dtype} plan={q}")
        assert (q["lanes_per_row"], q["vecs_per_lane"]) == (lanes, k), q
        if (lanes, k) == (256, 8):
            assert q["block_threads"] == 256 and q["num_blocks"] == _grid(rows, cus), q
    dx, dw = R.rmsnorm_vjp(x, w, dy, c["eps"], 0.5)
    y, dxg, dwg = R.rmsnorm_fwd_vjp(x, w, dy, c["eps"], 0.5)
    dh, dwf = R.fused_add_rmsnorm_vjp(x, w, dy, dr, c["eps"], 0.5)
    torch.cuda.synchronize()
    dxref, dwref = O.rmsnorm_vjp(c["x"], c["w"], c["dy"], c["eps"], 0.5)
    yref, _ = O.rmsnorm_fwd(c["x"], c["w"], c["eps"], 0.5)
    dhref, _ = O.fused_add_rmsnorm_vjp(c["x"], c["w"], c["dy"], c["residual"], c["eps"], 0.5)
    assert_close(dx, dxref, "dx")
    assert_close(dxg, dxref, "grad dx")
    assert_close(y, yref, "grad y")
    assert_close(dh, dhref, "dh")
    for d, what in ((dw, "dw"), (dwg, "grad dw"), (dwf, "fused dw")):
        assert_dw_close(d, dwref, what)


@pytest.mark.parametrize("D,dtype,lanes", [(14336, "bfloat16", 448), (16384, "float16", 512), (14336, "float16", 448)])
def test_wide_rows_steady_state_many_rows_per_block(R, D, dtype, lanes):
    """The pipelined four-vector instances (one row per block) with many
    rows per block: 200 rows on a forced 7-block grid, so the loop body
    (and the fused backward's single d_new_residual buffer, reloaded inside
    the loop) runs in its steady state for ~28 iterations per block.  VJP,
    grad call (y and dx) and fused backward against the oracle on every
    row, and dw."""
    rows = 200
    c = I.generic(rows, D, dtype, seed=D + 17)
    x, w, dy, dr = (c[k].to(DEV) for k in ("x", "w", "dy", "residual"))
    cfg = dict(lanes_per_row=lanes, vecs_per_lane=4, vec_bytes=16, block_threads=lanes, num_blocks=7)
    _say(f"wide rows steady state D={D} {dtype} cfg={cfg}")
    dx, dw = R.rmsnorm_vjp(x, w, dy, c["eps"], 0.5, cfg=cfg)
    y, dxg, dwg = R.rmsnorm_fwd_vjp(x, w, dy, c["eps"], 0.5, cfg=cfg)
    dh, dwf = R.fused_add_rmsnorm_vjp(x, w, dy, dr, c["eps"], 0.5, cfg=cfg)
    torch.cuda.synchronize()
    dxref, dwref = O.rmsnorm_vjp(c["x"], c["w"], c["dy"], c["eps"], 0.5)
    yref, _ = O.rmsnorm_fwd(c["x"], c["w"], c["eps"], 0.5)
    dhref, _ = O.fused_add_rmsnorm_vjp(c["x"], c["w"], c["dy"], c["residual"], c["eps"], 0.5)
    assert_close(dx, dxref, "dx")
    assert_close(dxg, dxref, "grad dx")
    assert_close(y, yref, "grad y")
    assert_close(dh, dhref, "dh")
    assert torch.equal(dxg, dx)
    for d, what in ((dw, "dw"), (dwg, "grad dw"), (dwf, "fused dw")):
        assert_dw_close(d, dwref, what)


@pytest.mark.parametrize("dtype", ["float32", "float16", "bfloat16"])
def test_partial_rows_never_one_per_row(R, dtype):
    """Every backward form's plan, over a sweep of row counts and widths:
    whenever there are two rows or more, the dw partial rows (the persistent
    grid, or the column split's row chunks) number fewer than the rows, and
    the workspace is at most half a [rows, D] fp32 buffer -- the gw_temp
    layout the MLX pull request removes -- plus, for the column split, the
    rows' statistics (two floats per slice of 1024 vectors)."""
    dt = getattr(torch, dtype)
    for rows in (2, 3, 7, 64, 255, 256, 257, 511, 1000, 5000, 100000):
        for D in (1, 64, 257, 512, 1000, 4096, 8192, 14336, 16384, 20480, 70000, 1 << 20):
            for op in (2, 3, 4):
                q = R.query_config(op, rows, D, dt)
                assert q["num_blocks"] < rows, (op, rows, D, q)
            ws = R.rmsnorm_vjp_workspace_bytes(rows, D, dt)
            stats = -(-(rows * -(-D // 1024) * 8) // 256) * 256
            assert ws <= max(256, ((rows + 1) // 2) * D * 4 + stats), (rows, D, ws)


def _np2(n):
    p = 1
    while p < n:
        p *= 2
    return p


def _few_rows_block(lanes, rows):
    cap = 512 if lanes <= 16 else 256
    return max(64, lanes * min(_np2(rows), max(1, cap // lanes)))


# Few rows for the backward forms: rows x D x itemsize <= 32 KiB and at most
# 1024 16-byte vectors per row in 16-bit storage (512 in fp32 or with the
# last vector overlapped): one block looping over the rows (no combine
# launch), one vector per lane, lanes x min(next_pow2(rows), cap / lanes)
# threads (cap 512 for rows of 16 lanes or fewer, else 256).
FEW = [(1, 128, "float16"), (2, 256, "bfloat16"), (1, 4096, "float16"), (16, 512, "float16"), (64, 128, "bfloat16"),
       (3, 1024, "bfloat16"), (4, 2048, "float16"), (1, 1536, "bfloat16"), (2, 2560, "float16"), (5, 64, "float32"),
       (1, 2048, "float32"), (7, 256, "float32"), (4, 1536, "float16"),
       (32, 512, "float16"), (128, 128, "float16"), (8, 2048, "bfloat16"), (4, 4096, "bfloat16"),
       (1, 8192, "float16"), (2, 6144, "bfloat16"), (1, 5120, "float16"), (2, 7168, "float16"),
       # overlapped last vector
       (1, 257, "float16"), (2, 513, "float16"), (4, 500, "bfloat16"), (1, 2049, "bfloat16"), (3, 97, "float32"),
       (8, 1001, "float16")]


@pytest.mark.parametrize("rows,D,dtype", FEW)
def test_few_rows_one_block_every_form(R, rows, D, dtype):
    td = I.torch_dtype(dtype)
    nvec = -(-D * td.itemsize // 16)   # the last vector overlapped when D * itemsize is not a multiple of 16
    for op in (2, 3, 4):
        q = R.query_config(op, rows, D, td)
        _say(f"few-row backward op={op} {dtype} {rows}x{D} plan={q}")
        assert q["vecs_per_lane"] == 1 and q["vec_bytes"] == 16, q
        assert q["lanes_per_row"] in (nvec, _np2(nvec)), q
        assert q["num_blocks"] == 1 and q["block_threads"] == _few_rows_block(q["lanes_per_row"], rows), q
    c = I.generic(rows, D, dtype, seed=rows * 7 + D)
    x, w, dy, dr = (c[k].to(DEV) for k in ("x", "w", "dy", "residual"))
    dx, dw = R.rmsnorm_vjp(x, w, dy, c["eps"], 1.0)
    y, dxg, dwg = R.rmsnorm_fwd_vjp(x, w, dy, c["eps"], 1.0)
    dh, dwf = R.fused_add_rmsnorm_vjp(x, w, dy, dr, c["eps"], 1.0)
    torch.cuda.synchronize()
    dxref, dwref = O.rmsnorm_vjp(c["x"], c["w"], c["dy"], c["eps"], 1.0)
    yref, _ = O.rmsnorm_fwd(c["x"], c["w"], c["eps"], 1.0)
    dhref, _ = O.fused_add_rmsnorm_vjp(c["x"], c["w"], c["dy"], c["residual"], c["eps"], 1.0)
    assert_close(dx, dxref, "dx")
    assert_dw_close(dw, dwref, "dw")
    assert_close(y, yref, "grad y")
    assert_close(dh, dhref, "dh")
    assert_dw_close(dwf, dwref, "fused dw")
    # the three forms share the plan: the grad call's dx and dw are the VJP's, bit for bit
    assert torch.equal(dxg, dx) and torch.equal(dwg, dw)


def test_few_rows_rule_stops_where_rows_do_not_fit_one_block(R):
    bf = torch.bfloat16
    assert R.query_config(2, 5, 3840, bf)["vecs_per_lane"] == 2       # 38 KiB (256 x 2, duplicate slots)
    assert R.query_config(2, 6, 3072, bf)["vecs_per_lane"] == 2       # 36 KiB (192 x 2)
    assert R.query_config(2, 129, 128, bf)["vecs_per_lane"] == 2      # 33 KiB
    assert R.query_config(2, 1, 4096, torch.float32)["vecs_per_lane"] == 2   # fp32 rows of 1024 vectors
    q = R.query_config(2, 17, 1001, torch.float16)                     # overlapped, 34 KiB
    assert (q["lanes_per_row"], q["vecs_per_lane"]) == (64, 2), q
    q = R.query_config(2, 1, 1000, torch.float16)                      # 125 whole vectors: inside
    assert (q["lanes_per_row"], q["vecs_per_lane"], q["block_threads"], q["num_blocks"]) == (128, 1, 128, 1), q
    # one row of 256 vectors: inside the rule
    assert R.query_config(2, 1, 2048, bf)["vecs_per_lane"] == 1