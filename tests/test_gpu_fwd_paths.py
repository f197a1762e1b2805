"""GPU: the plain forward of rows of 1025..2048 16-byte vectors takes 256
lanes x 8 vectors in 256-thread blocks; longer rows that need 1024 lanes
but fill under 70 % of their vector slots take the streaming kernel
(512-thread blocks); full rows and the 4-vector fp32 instance stay in
registers.  Checks the automatic plan on
both sides of that rule and parity of the forward with the fp64 oracle on
every row, plus the same rows forced through the register kernel.  Rows of a whole number of waves that is not a power of two (wave
rows) with two 16-byte vectors per lane take an exact-tiling instance of
up to 768 lanes (two three-wave rows per block); its plan, parity of the
forward and the fused forward, forced one-vector and 896-lane instances,
and outputs bit-identical across rows per block.  Few rows (at most one per
CU) of 64..768 16-byte vectors in a multiple of 64 take one vector per lane,
one row per block, in both forward forms."""
import sys

import numpy as np
import pytest
import torch

from _parity import assert_close, to64
from backward_rmsnorm_fwd_two_amd import inputs as I
from oracle import oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def R():
    import backward_rmsnorm_fwd_two_amd as pkg
    return pkg


# (rows, D, dtype, the automatic plan: "256x8" for rows of 1025..2048
# 16-byte vectors, "stream" for sparser 1024-lane rows, "reg" otherwise)
CASES = [(600, 8200, "bfloat16", "256x8"), (500, 10248, "float16", "256x8"), (300, 16392, "bfloat16", "stream"),
         (700, 4100, "float32", "256x8"), (400, 16384, "bfloat16", "256x8"), (300, 8200, "float32", "reg"),
         (500, 12288, "bfloat16", "256x8"), (250, 20480, "bfloat16", "stream"), (200, 22000, "float16", "stream")]


@pytest.mark.parametrize("rows,D,dtype,plan", CASES)
def test_sparse_forward_rows_stream(R, rows, D, dtype, plan):
    print(f"forward paths rows={rows} D={D} {dtype}", flush=True)
    sys.stdout.flush()
    c = I.generic(rows, D, dtype, seed=rows + D)
    x, w = c["x"].to(DEV), c["w"].to(DEV)
    q = R.query_config(0, rows, D, x.dtype)
    if plan == "stream":
        assert q["vecs_per_lane"] == -1 and q["block_threads"] == 512, q
    elif plan == "256x8":
        assert (q["lanes_per_row"], q["vecs_per_lane"], q["block_threads"]) == (256, 8, 256), q
    else:
        assert q["vecs_per_lane"] > 0 and q["lanes_per_row"] == 1024, q
    y = R.rmsnorm_fwd(x, w, c["eps"], 1.0)
    reg = dict(lanes_per_row=1024, vecs_per_lane=0, vec_bytes=0, block_threads=1024, num_blocks=0)
    y_reg = R.rmsnorm_fwd(x, w, c["eps"], 1.0, cfg=reg)
    torch.cuda.synchronize()
    yref, _ = O.rmsnorm_fwd(c["x"], c["w"], c["eps"], 1.0)
    assert_close(y, yref, "y")
    assert_close(y_reg, yref, "y (register kernel)")


def _is_pow2(v):
    return v > 0 and (v & (v - 1)) == 0


# (rows, D, dtype, lanes, rows per block) of the automatic forward plan;
# lanes None: the power-of-two layout
WAVE = [(4000, 3072, "float16", 192, 2), (4001, 3072, "bfloat16", 192, 2), (1001, 5120, "bfloat16", 320, 1),
        (700, 6144, "float16", 384, 1), (333, 12288, "bfloat16", 768, 1), (500, 10240, "float16", 640, 1),
        (700, 3072, "float32", 384, 1), (500, 3584, "bfloat16", None, None), (200, 14336, "bfloat16", None, None),
        (300, 11264, "bfloat16", 704, 1)]


@pytest.mark.parametrize("rows,D,dtype,lanes,slots", WAVE)
def test_wave_rows_forward(R, rows, D, dtype, lanes, slots):
    print(f"forward wave rows rows={rows} D={D} {dtype}", flush=True)
    sys.stdout.flush()
    c = I.generic(rows, D, dtype, seed=2 * rows + D)
    x, w, res = c["x"].to(DEV), c["w"].to(DEV), c["residual"].to(DEV)
    nvec = D * x.element_size() // 16
    for op in (0, 1):
        q = R.query_config(op, rows, D, x.dtype)
        if lanes is None:
            assert _is_pow2(q["lanes_per_row"]) or q["vecs_per_lane"] == -1, q
        elif op == 0 and nvec > 1024:
            # the plain forward of longer rows takes 256 lanes x 8 instead
            assert (q["lanes_per_row"], q["vecs_per_lane"]) == (256, 8), q
        else:
            assert q["lanes_per_row"] == lanes and q["vecs_per_lane"] == 2 and q["vec_bytes"] == 16, q
            assert q["block_threads"] == slots * lanes and q["num_blocks"] == (rows + slots - 1) // slots, q
    # the automatic plan (the wave-row geometry forced where the plain
    # forward's automatic plan is 256 x 8), and (power-of-two plans) the
    # wave-row instance the row also tiles, forced: one vector per lane on
    # 64 W lanes
    cfgs = [None]
    if lanes is not None and nvec > 1024:
        cfgs = [dict(lanes_per_row=lanes, vecs_per_lane=2, vec_bytes=16, block_threads=slots * lanes, num_blocks=0)]
    if lanes is None:
        for k in (1, 2):
            wl = nvec // k
            if nvec % k == 0 and wl % 64 == 0 and not _is_pow2(wl) and wl <= 1024:
                cfgs.append(dict(lanes_per_row=wl, vecs_per_lane=k, vec_bytes=16, block_threads=wl, num_blocks=0))
    else:
        for s_ in (1, 2, 4):
            if s_ != slots and s_ * lanes <= 1024:
                cfgs.append(dict(lanes_per_row=lanes, vecs_per_lane=2, vec_bytes=16, block_threads=s_ * lanes,
                                 num_blocks=0))
    assert lanes is not None or len(cfgs) > 1
    yref, _ = O.rmsnorm_fwd(c["x"], c["w"], c["eps"], 1.0)
    nref, href = O.fused_add_rmsnorm_fwd(c["x"], c["residual"], c["w"], c["eps"], 1.0)
    first = None
    for cfg in cfgs:
        y = R.rmsnorm_fwd(x, w, c["eps"], 1.0, cfg=cfg)
        n, h = R.fused_add_rmsnorm_fwd(x, res, w, c["eps"], 1.0, cfg=cfg)
        torch.cuda.synchronize()
        assert_close(y, yref, f"y cfg={cfg}")
        assert_close(n, nref, f"normed cfg={cfg}")
        np.testing.assert_array_equal(to64(h), O.round_to(href, dtype), f"new_residual cfg={cfg}")
        if lanes is not None:
            # same lanes and vectors: rows per block change nothing
            if first is None:
                first = (y, n, h)
            else:
                assert torch.equal(y, first[0]) and torch.equal(n, first[1]) and torch.equal(h, first[2]), cfg


# (rows, D, dtype, expected (lanes, vectors per lane) of the plain forward):
# rows of 129..1024 16-byte vectors that a power-of-two layout with 2 vectors
# per lane would leave under 90 % full take 4 vectors per lane on half the
# lanes; full rows and wave rows keep 2
SHORT = [(300, 4608, "bfloat16", (256, 4)), (301, 2560, "float16", (128, 4)), (300, 1536, "bfloat16", (64, 4)),
         (257, 3584, "float16", (128, 4)), (300, 4096, "bfloat16", (256, 2)), (300, 3072, "float16", (192, 2))]


@pytest.mark.parametrize("rows,D,dtype,plan", SHORT)
def test_sparse_short_forward_rows(R, rows, D, dtype, plan):
    print(f"short forward rows={rows} D={D} {dtype}", flush=True)
    sys.stdout.flush()
    c = I.generic(rows, D, dtype, seed=rows + 5 * D)
    x, w = c["x"].to(DEV), c["w"].to(DEV)
    q = R.query_config(0, rows, D, x.dtype)
    assert (q["lanes_per_row"], q["vecs_per_lane"]) == plan, q
    y = R.rmsnorm_fwd(x, w, c["eps"], 1.0)
    torch.cuda.synchronize()
    yref, _ = O.rmsnorm_fwd(c["x"], c["w"], c["eps"], 1.0)
    assert_close(y, yref, "y")


# Few rows (at most one per CU) of 64..768 whole 16-byte vectors, a multiple
# of 64: both forward forms take one vector per lane on as many lanes as the
# row has vectors, one row per block (decode batches are latency-bound).
FEW = [(1, 2048, "bfloat16"), (8, 512, "float16"), (4, 1536, "bfloat16"), (64, 2560, "float16"),
       (8, 3072, "bfloat16"), (3, 1024, "float32"), (17, 768, "float32"), (5, 1536, "float32"),
       (2, 3584, "float16"), (1, 4096, "bfloat16"), (7, 4608, "bfloat16"), (3, 5120, "float16"),
       (4, 5632, "bfloat16"), (8, 6144, "bfloat16"), (2, 2048, "float32"), (6, 3072, "float32")]


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("rows,D,dtype", FEW)
def test_few_rows_one_vector_per_lane(R, rows, D, dtype):
    print(f"few-row forward rows={rows} D={D} {dtype}", flush=True)
    sys.stdout.flush()
    td = I.torch_dtype(dtype)
    nvec = D * td.itemsize // 16
    for op in (0, 1):
        q = R.query_config(op, rows, D, td)
        assert (q["lanes_per_row"], q["vecs_per_lane"], q["vec_bytes"]) == (nvec, 1, 16), (op, q)
        assert q["block_threads"] == max(nvec, 64) and q["num_blocks"] == rows, (op, q)
        # more rows than CUs: the bandwidth layouts (two or four vectors per lane)
        qb = R.query_config(op, _cus() + 1, D, td)
        assert qb["vecs_per_lane"] in (2, 4), (op, qb)
    c = I.generic(rows, D, dtype, seed=rows + 7 * D)
    x, res, w = c["x"].to(DEV), c["residual"].to(DEV), c["w"].to(DEV)
    for wb in (0.0, 1.0):
        y = R.rmsnorm_fwd(x, w, c["eps"], wb)
        n, h = R.fused_add_rmsnorm_fwd(x, res, w, c["eps"], wb)
        torch.cuda.synchronize()
        assert_close(y, O.rmsnorm_fwd(c["x"], c["w"], c["eps"], wb)[0], f"y wb={wb}")
        nref, href = O.fused_add_rmsnorm_fwd(c["x"], c["residual"], c["w"], c["eps"], wb)
        assert_close(n, nref, f"normed wb={wb}")
        np.testing.assert_array_equal(to64(h), O.round_to(href, dtype), f"new_residual wb={wb}")


def test_few_rows_rule_limits(R):
    """Outside the rule the plans are the bandwidth ones: at the CU count
    plus one, at 1024 vectors, at 32 vectors, for a count that is not a
    multiple of 64, and for the backward forms."""
    cus = _cus()
    bf = torch.bfloat16
    assert R.query_config(1, cus, 2048, bf)["vecs_per_lane"] == 1
    assert R.query_config(1, cus + 1, 2048, bf)["vecs_per_lane"] == 2
    assert R.query_config(0, 8, 8192, bf)["vecs_per_lane"] == 2          # 1024 vectors
    assert R.query_config(1, 8, 8192, bf)["vecs_per_lane"] == 2
    q = R.query_config(0, 8, 256, bf)                                     # 32 vectors
    assert (q["lanes_per_row"], q["vecs_per_lane"], q["block_threads"]) == (16, 2, 256), q
    q = R.query_config(1, 8, 1280, bf)                                    # 160 vectors
    assert (q["lanes_per_row"], q["vecs_per_lane"]) == (128, 2), q
    # the backward forms have their own few-rows rule (one block up to 32 KiB
    # per tensor); beyond it they keep two vectors per lane
    for op in (2, 3, 4):
        assert R.query_config(op, 16, 2048, bf)["vecs_per_lane"] == 2


@pytest.mark.parametrize("D,block", [(3072, 256), (2048, 128)])
def test_few_rows_with_a_requested_block(R, D, block):
    """A configuration that fixes only the block size keeps the layout that
    block fits (the few-rows rule applies to a fully automatic geometry)."""
    rows = 4
    c = I.generic(rows, D, "bfloat16", seed=D + block)
    x, res, w = c["x"].to(DEV), c["residual"].to(DEV), c["w"].to(DEV)
    cfg = dict(block_threads=block)
    y = R.rmsnorm_fwd(x, w, c["eps"], 1.0, cfg=cfg)
    n, h = R.fused_add_rmsnorm_fwd(x, res, w, c["eps"], 1.0, cfg=cfg)
    torch.cuda.synchronize()
    assert_close(y, O.rmsnorm_fwd(c["x"], c["w"], c["eps"], 1.0)[0], "y")
    nref, href = O.fused_add_rmsnorm_fwd(c["x"], c["residual"], c["w"], c["eps"], 1.0)
    assert_close(n, nref, "normed")
    np.testing.assert_array_equal(to64(h), O.round_to(href, "bfloat16"), "new_residual")
    # the automatic plan of the same shape is the few-rows one
    assert R.query_config(0, rows, D, torch.bfloat16)["vecs_per_lane"] == 1


@pytest.mark.parametrize("D,dtype", [(8192, "bfloat16"), (8192, "float16"), (16384, "bfloat16"), (4096, "float32"),
                                     (8192, "float32")])
def test_few_rows_wide_fused_fixed_width_matches_runtime_width(R, D, dtype):
    """The fused forward of 512- and 1024-lane rows runs the instance with the
    lanes fixed at compile time on no more rows than CUs, the runtime-width
    kernel on more: the same lanes, vectors and reduction order, so a row
    comes out bit for bit the same either way."""
    few, many = 5, _cus() + 45
    c = I.generic(many, D, dtype, seed=D + few)
    td = I.torch_dtype(dtype)
    nvec = D * td.itemsize // 16
    for rows in (few, many):
        q = R.query_config(1, rows, D, td)
        assert q["lanes_per_row"] * q["vecs_per_lane"] == nvec and q["lanes_per_row"] >= 512, q
    x, res, w = c["x"].to(DEV), c["residual"].to(DEV), c["w"].to(DEV)
    n_few, h_few = R.fused_add_rmsnorm_fwd(x[:few].contiguous(), res[:few].contiguous(), w, c["eps"], 1.0)
    n_many, h_many = R.fused_add_rmsnorm_fwd(x, res, w, c["eps"], 1.0)
    torch.cuda.synchronize()
    nref, href = O.fused_add_rmsnorm_fwd(c["x"][:few], c["residual"][:few], c["w"], c["eps"], 1.0)
    assert_close(n_few, nref, "normed (few rows)")
    np.testing.assert_array_equal(to64(h_few), O.round_to(href, dtype), "new_residual (few rows)")
    assert torch.equal(n_few, n_many[:few]) and torch.equal(h_few, h_many[:few])
