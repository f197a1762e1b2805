"""GPU: forward rows that need 1024 lanes but fill under 70 % of their
vector slots take the streaming kernel (512-thread blocks); full rows and
the 4-vector fp32 instance stay in registers.  Checks the automatic plan on
both sides of that rule and parity of the forward with the fp64 oracle on
the first and last rows, plus the same rows forced through the register
kernel."""
import sys

import pytest
import torch

from _parity import assert_close
from backward_rmsnorm_fwd_two_amd import inputs as I
from oracle import oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def R():
    import backward_rmsnorm_fwd_two_amd as pkg
    return pkg


# (rows, D, dtype, streamed by the automatic plan)
CASES = [(600, 8200, "bfloat16", True), (500, 10240, "float16", True), (300, 16392, "bfloat16", True),
         (700, 4100, "float32", True), (400, 16384, "bfloat16", False), (300, 8200, "float32", False),
         (500, 12288, "bfloat16", False)]


@pytest.mark.parametrize("rows,D,dtype,streamed", CASES)
def test_sparse_forward_rows_stream(R, rows, D, dtype, streamed):
    print(f"forward paths rows={rows} D={D} {dtype}", flush=True)
    sys.stdout.flush()
    c = I.generic(rows, D, dtype, seed=rows + D)
    x, w = c["x"].to(DEV), c["w"].to(DEV)
    q = R.query_config(0, rows, D, x.dtype)
    assert (q["vecs_per_lane"] == -1) == streamed, q
    if streamed:
        assert q["block_threads"] == 512, q
    y = R.rmsnorm_fwd(x, w, c["eps"], 1.0)
    reg = dict(lanes_per_row=1024, vecs_per_lane=0, vec_bytes=0, block_threads=1024, num_blocks=0)
    y_reg = R.rmsnorm_fwd(x, w, c["eps"], 1.0, cfg=reg)
    torch.cuda.synchronize()
    idx = list(range(32)) + list(range(rows - 32, rows))
    yref, _ = O.rmsnorm_fwd(c["x"][idx], c["w"], c["eps"], 1.0)
    assert_close(y[idx], yref, "y")
    assert_close(y_reg[idx], yref, "y (register kernel)")
