"""GPU: the library on several streams and inside a captured HIP graph.

The entry points keep no state between calls and allocate nothing, so
(a) two host threads driving two streams (default priority) with their own
buffers and workspaces must reproduce the single-stream results bit for bit,
and (b) a graph captured from the calls (all buffers allocated beforehand)
must, on every replay, reproduce what the eager calls give on the inputs of
that replay -- with eager work and synchronisation between the replays."""
import threading

import pytest
import torch

from backward_rmsnorm_fwd_two_amd import inputs as I

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def R():
    import backward_rmsnorm_fwd_two_amd as pkg
    return pkg


def _buffers(R, rows, D, seed):
    c = I.generic(rows, D, "bfloat16", seed=seed)
    b = {k: c[k].to(DEV) for k in ("x", "w", "dy", "residual")}
    b["y"] = torch.empty_like(b["x"])
    b["dx"] = torch.empty_like(b["x"])
    b["normed"] = torch.empty_like(b["x"])
    b["newres"] = torch.empty_like(b["x"])
    b["dw"] = torch.empty(D, dtype=torch.float32, device=DEV)
    b["ws"] = R.workspace_for(rows, D, torch.bfloat16, DEV)
    return b


def _run(R, b):
    R.rmsnorm_fwd(b["x"], b["w"], 1e-6, 1.0, out=b["y"])
    R.rmsnorm_vjp(b["x"], b["w"], b["dy"], 1e-6, 1.0, dx=b["dx"], dw=b["dw"], workspace=b["ws"])
    R.fused_add_rmsnorm_fwd(b["x"], b["residual"], b["w"], 1e-6, 1.0, normed=b["normed"],
                            new_residual=b["newres"])


OUTS = ("y", "dx", "dw", "normed", "newres")


def test_two_threads_two_streams(R):
    rows, D = 2048, 4096
    bufs = [_buffers(R, rows, D, seed) for seed in (1, 2)]
    # reference: one stream, sequential
    ref = []
    for b in bufs:
        _run(R, b)
        torch.cuda.synchronize()
        ref.append({k: b[k].clone() for k in OUTS})
        for k in OUTS:
            b[k].fill_(float("nan"))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=DEV) for _ in bufs]   # default priority
    errors = []

    def worker(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(25):
                    _run(R, bufs[i])
            streams[i].synchronize()
        except Exception as e:  # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(bufs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for b, r in zip(bufs, ref):
        for k in OUTS:
            assert torch.equal(b[k], r[k]), k


def test_graph_capture_replays_match_eager(R):
    rows, D = 1024, 4096
    b = _buffers(R, rows, D, seed=5)
    d = 2048
    gx = I.gate(rows, d, "bfloat16", seed=5)["x"].to(DEV)
    gy = torch.empty(rows, d, dtype=torch.bfloat16, device=DEV)

    def step():
        _run(R, b)
        R.silu_gate(gx, out=gy)

    # warm up on a side stream, then capture
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(4):
        # new inputs for this replay (eager work between replays)
        c = I.generic(rows, D, "bfloat16", seed=100 + rep)
        for k in ("x", "dy", "residual"):
            b[k].copy_(c[k].to(DEV))
        gx.copy_(I.gate(rows, d, "bfloat16", seed=100 + rep)["x"].to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {k: b[k].clone() for k in OUTS}
        got_gate = gy.clone()
        # eager on the same inputs
        step()
        torch.cuda.synchronize()
        for k in OUTS:
            assert torch.equal(got[k], b[k]), (rep, k)
        assert torch.equal(got_gate, gy), rep
