#!/usr/bin/env python3
"""Benchmark: RMSNorm forward + VJP on one MI355X through the C ABI.

One step = rmsnorm_fwd + rmsnorm_vjp (dx and the fp32 weight gradient dw)
over one [8192, 4096] fp16 batch (the tensors of the MLX pull request's POC
timing script: x, w, dy ~ U(0,1), eps 1e-5, weight_bias 0).  Throughput is
algorithmic bytes moved per step / time:
    forward  2*R*D*s + D*s        (read x, write y, read w)
    VJP      3*R*D*s + D*s + 4*D  (read x and dy, write dx, read w, write dw)
Inputs are resident in HBM before the timed region.  Calls go straight to
the C ABI with arguments marshalled once per buffer set.  Consecutive steps use
different buffer sets (rotating through enough copies that a set is touched
again only after >= 1 GiB of other traffic), so no step is served from the
256 MB last-level cache left warm by the step before it.

Prints one JSON line (rank 0); its `prefill` key holds the fused add+RMSNorm
forward + VJP at [32768, 8192] bf16 (the prefill-scale workload), measured the
same way.  `--workload prefill` prints that one alone;
`--workload gate` the gated activation silu(x[:, :d]) * x[:, d:2d] at the
Llama-3 8B MLP width (d = 14336) in bf16, prefill chunk and decode batches.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) for RMSNorm fwd+VJP, 8192x4096 fp16"
HBM_PEAK_GBPS = 8000.0
KERNEL_SOURCES = ["rmsn_kernels.hpp", "rmsn_device.hpp", "rmsn_launch.hpp", "rmsn_vjp.hip", "rmsn_vjp_lanes.hip",
                  "rmsn_vjp_waves.hip", "rmsn_vjp_dup.hip", "rmsn_vjp_dup_ovl.hip", "rmsn_fwd.hip", "rmsn_fwd_waves.hip", "rmsn_fwd_waves_ovl.hip", "rmsn_ovl.hip",
                  "rmsn_colsplit.hip", "rmsn_api.hip"]
GATE_SOURCES = ["rmsn_gate.hip", "rmsn_device.hpp", "rmsn_api.hip"]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(files=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "backward_rmsnorm_fwd_two_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(name: str, src_hash: str):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    (scaled by a copy kernel of known size), read from the committed summary
    profiles/<name>.md -- only if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", name + ".md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel source hash:\s*`?([0-9a-f]{16})", text)
    m_val = re.search(r"traffic per launch \(bytes\):\s*`?([0-9]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != src_hash:
        return None
    return int(m_val.group(1))


def elapsed_ms(a: torch.cuda.Event, b: torch.cuda.Event) -> float:
    return a.elapsed_time(b)


def copy_ceiling(nbytes: int = 256 << 20, reps: int = 20) -> float:
    """Device-to-device copy throughput (read + write bytes / time), GB/s."""
    src = torch.empty(nbytes // 2, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = elapsed_ms(e0, e1) / reps
    return 2 * nbytes / (ms * 1e-3) / 1e9


def cpu_threads():
    """(threads, affinity): the host cores this process may run on
    (sched_getaffinity), capped by OMP_NUM_THREADS when the environment sets
    it (the CPU share a shared host declares for this job)."""
    affinity = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    threads = min(affinity, int(cap)) if cap.isdigit() and int(cap) > 0 else affinity
    return max(1, threads), affinity


def cpu_oracle_baseline(c, rows, D, fwd_bytes, vjp_bytes, fused=False, seconds=8.0):
    """The fp64 CPU oracle as it stands, on a bounded sample of the same
    workload (its first `sample_rows` rows, repeated for about `seconds`),
    in GB/s on the same algorithmic byte model.  The inputs are widened to
    fp64 before the clock starts.  Headline figure: the same oracle calls on
    a static row split over one thread per host core (the C oracle runs
    without the GIL); also the single-thread figure."""
    import concurrent.futures as cf
    from oracle import oracle as O
    sample_rows = min(rows, 2048 if fused else 8192)
    w = O.widen(c["w"])
    x = O.widen(c["x"][:sample_rows])
    dy = O.widen(c["dy"][:sample_rows])
    res = O.widen(c["residual"][:sample_rows]) if fused else None
    eps, wb = c["eps"], c["weight_bias"]
    per_row_bytes = (fwd_bytes + vjp_bytes) / rows

    def work(lo, hi):
        if fused:
            _, h = O.fused_add_rmsnorm_fwd(x[lo:hi], res[lo:hi], w, eps, wb)
            O.rmsnorm_vjp(h, w, dy[lo:hi], eps, wb)
        else:
            O.rmsnorm_fwd(x[lo:hi], w, eps, wb)
            O.rmsnorm_vjp(x[lo:hi], w, dy[lo:hi], eps, wb)

    def timed(fn):
        t0 = time.perf_counter()
        passes = 0
        while True:
            fn()
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= seconds or passes >= 400:
                return passes, dt

    threads, affinity = cpu_threads()
    bounds = [(i * sample_rows // threads, (i + 1) * sample_rows // threads) for i in range(threads)]
    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda b: work(*b), bounds))  # first touch of the output buffers' pages
        passes, dt = timed(lambda: list(ex.map(lambda b: work(*b), bounds)))
    p1, dt1 = timed(lambda: work(0, sample_rows))
    return {
        "value": round(passes * sample_rows * per_row_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
        "kind": "oracle",
        "sample": f"{passes} pass(es) of fwd+VJP over the first {sample_rows} of {rows} rows (D={D}) split into "
                  f"{threads} row shards, one thread each; fp64 C oracle on inputs widened before timing; "
                  f"{dt:.1f} s",
        "affinity_cores": affinity,
        "single_thread": {"value": round(p1 * sample_rows * per_row_bytes / dt1 / 1e9, 4), "unit": "GB/s",
                          "cores": 1, "sample": f"{p1} pass(es) over the same rows, {dt1:.1f} s"},
    }


BENCHSRC = os.path.join(ROOT, "benchsrc")


def bench_tool(name: str, link_library: bool = False) -> str:
    """The measurement program benchsrc/<name>.hip (not part of the library),
    compiled for gfx950 into benchsrc/bin/ when it is missing or older than
    its sources.  link_library: it also includes the library's kernel headers
    and links librmsnorm_mi355x.so (which must be built)."""
    import subprocess
    from backward_rmsnorm_fwd_two_amd import build as B
    src = os.path.join(BENCHSRC, name + ".hip")
    exe = os.path.join(BENCHSRC, "bin", name)
    deps = [src]
    if link_library:
        if not os.path.exists(B.LIB_PATH):
            raise RuntimeError(f"{B.LIB_PATH} is not built; run __graft_entry__.build() first")
        deps += [B.LIB_PATH] + [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC) if f.endswith(".hpp")]
    if os.path.exists(exe) and os.path.getmtime(exe) >= max(os.path.getmtime(d) for d in deps):
        return exe
    os.makedirs(os.path.dirname(exe), exist_ok=True)
    cmd = [B.hipcc()] + B.HIPCC_FLAGS + [src, "-o", exe + ".tmp"]
    if link_library:
        cmd += [f"-L{B.HERE}", "-lrmsnorm_mi355x", "-Wl,-rpath,$ORIGIN/../../backward_rmsnorm_fwd_two_amd"]
    log(f"building {exe}")
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    os.replace(exe + ".tmp", exe)
    return exe


def ceiling_bench() -> int:
    """HBM throughput of trivial streaming kernels for each traffic mix the
    RMSNorm kernels have (benchsrc/stream_ceiling.hip): the practical ceiling
    each kernel is measured against."""
    import subprocess
    exe = bench_tool("stream_ceiling")
    out = subprocess.run([exe], capture_output=True, text=True, timeout=240)
    if out.returncode != 0:
        print(out.stdout + out.stderr, file=sys.stderr)
        return out.returncode
    best = {}
    for line in out.stdout.splitlines():
        f = dict(kv.split("=") for kv in line.split())
        key = (f["mix"], f["policy"], int(f["stream_MiB"]))
        best[key] = max(best.get(key, 0.0), float(f["GBps_med"]))
        log(line)
    grid = [{"mix": m, "policy": p, "stream_MiB": s, "median_GBps_best_grid": v}
            for (m, p, s), v in sorted(best.items())]
    cold = max(v for (m, p, s), v in best.items() if s == 512 and m == "1R1W")
    print(json.dumps({"metric": "HBM ceiling of trivial streaming kernels (1R1W, 512 MiB streams)",
                      "value": cold, "unit": "GB/s", "n_gpus": 1, "higher_is_better": True,
                      "data": "synthetic", "config": {"workload": "stream ceiling", "grid": grid}}))
    return 0


def dwreduce_bench() -> int:
    """Ways of finishing the VJP's dw reduction at [8192, 4096] fp16
    (benchsrc/dw_reduction.hip): the library's separate combine launch
    against a deterministic last-arrival reduction inside the row kernel's
    launch, with per-block timestamps of each stage."""
    import subprocess
    exe = bench_tool("dw_reduction", link_library=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=240)
    if out.returncode != 0:
        print(out.stdout + out.stderr, file=sys.stderr)
        return out.returncode
    res = json.loads(out.stdout.strip().splitlines()[-1])
    lib = res["library"]
    print(json.dumps({
        "metric": "RMSNorm fwd+VJP step, 8192x4096 fp16, by way of finishing the dw reduction",
        "value": round(335577088 / (lib["step_us"] * 1e-6) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "higher_is_better": True, "data": "synthetic",
        "config": {"workload": "dw reduction variants, [8192, 4096] fp16, U(0,1), eps 1e-5"},
        "probe": res}), flush=True)
    return 0


def grad_bench(R, I, dev, args) -> int:
    """The grad call in one launch (rmsnorm_fwd_vjp: y, dx, dw from one pass
    over x and dy) on the [8192, 4096] fp16 POC tensors.  Its HBM bytes:
    read x, dy; write y, dx (4*R*D*s) + w + fp32 dw.  Also reported: the
    same work done as rmsnorm_fwd + rmsnorm_vjp, timed the same way."""
    c = I.poc_8192x4096()
    rows, D = c["x"].shape
    s = c["x"].element_size()
    grad_bytes = 4 * rows * D * s + D * s + 4 * D
    sep_bytes = 5 * rows * D * s + 2 * D * s + 4 * D
    set_bytes = 4 * rows * D * s
    nsets = args.sets or (-(-(1 << 30) // set_bytes) + 1)
    w = c["w"].to(dev)
    dw = torch.empty(D, dtype=torch.float32, device=dev)
    ws = R.workspace_for(rows, D, c["x"].dtype, dev)
    sets = [{"x": c["x"].to(dev), "dy": c["dy"].to(dev), "y": torch.empty(rows, D, dtype=c["x"].dtype, device=dev),
             "dx": torch.empty(rows, D, dtype=c["x"].dtype, device=dev)} for _ in range(nsets)]
    g_calls = [R.prepared_grad(st["x"], w, st["dy"], st["y"], st["dx"], dw, ws, c["eps"], c["weight_bias"])
               for st in sets]
    f_calls = [R.prepared_fwd(st["x"], w, st["y"], c["eps"], c["weight_bias"]) for st in sets]
    v_calls = [R.prepared_vjp(st["x"], w, st["dy"], st["dx"], dw, ws, c["eps"], c["weight_bias"]) for st in sets]

    def run(fn, K, W):
        for i in range(W):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / K

    t_grad = run(lambda i: g_calls[i % nsets](), args.steps, args.warmup)
    t_sep = run(lambda i: (f_calls[i % nsets](), v_calls[i % nsets]()), args.steps, args.warmup)
    value = grad_bytes / t_grad / 1e9
    print(json.dumps({
        "metric": "achieved HBM GB/s for the one-launch RMSNorm grad call (y, dx, dw), 8192x4096 fp16",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(t_grad * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "grad call rmsnorm_fwd_vjp, [8192, 4096] fp16, U(0,1), eps 1e-5",
                   "bytes_per_step": grad_bytes, "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
                   "separate_fwd_plus_vjp_us": round(t_sep * 1e6, 3),
                   "separate_GBps_on_their_bytes": round(sep_bytes / t_sep / 1e9, 1),
                   "grad_call_us": round(t_grad * 1e6, 3)},
    }), flush=True)
    return 0


def decode_layers_graph(R, dev, x, res0, w, eps, wb, fused: bool, layers: int = 32, reps: int = 50):
    """A decoder's residual stream through `layers` norms, captured in one HIP
    graph: layer i adds its sublayer output x to the running residual and
    normalises the sum (fused: one call; unfused: torch add, then
    rmsnorm_fwd), and its new_residual is layer i+1's residual.  Returns the
    per-call time of graph replays (us) -- the GPU-side latency with the host
    launch path taken out, as a decode loop captured once and replayed per
    token runs -- after checking a replay against the same chain run eagerly,
    bit for bit."""
    newres = [torch.empty_like(x) for _ in range(layers)]
    normed = [torch.empty_like(x) for _ in range(layers)]

    def chain():
        r = res0
        for i in range(layers):
            if fused:
                R.fused_add_rmsnorm_fwd(x, r, w, eps, wb, normed=normed[i], new_residual=newres[i])
            else:
                torch.add(x, r, out=newres[i])
                R.rmsnorm_fwd(newres[i], w, eps, wb, out=normed[i])
            r = newres[i]

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        chain()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain()
    torch.cuda.synchronize()
    for t in normed + newres:
        t.zero_()
    graph.replay()
    torch.cuda.synchronize()
    got = (normed[-1].clone(), newres[-1].clone())
    chain()
    torch.cuda.synchronize()
    if not (torch.equal(got[0], normed[-1]) and torch.equal(got[1], newres[-1])):
        raise RuntimeError("graph replay differs from the eager chain")
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * layers)


def decode_bench(R, I, dev, args) -> int:
    """Decode-shaped fused add+RMSNorm: latency per call, fused (one launch)
    against the unfused composition (torch add, then rmsnorm_fwd) over the
    (batch, hidden) grid of the fused-kernel microbenchmark; bf16, eps 1e-6,
    weight_bias 0 and 1.  Per-call time = events around N back-to-back calls
    / N (launch-bound: the host path is part of the latency); and the same
    calls chained through a 32-layer residual stream and replayed from one
    HIP graph (`decode_layers_graph`)."""
    N = max(args.steps, 100)
    rows = []
    for wb in (0.0, 1.0):
        for B in (1, 4, 8):
            for H in (2048, 4096, 8192):
                c = I.decode(B, H, wb)
                x, res, w = c["x"].to(dev), c["residual"].to(dev), c["w"].to(dev)
                normed, newres = torch.empty_like(x), torch.empty_like(x)
                tmp, y = torch.empty_like(x), torch.empty_like(x)
                fused = R.prepared_fused(x, res, w, normed, newres, c["eps"], wb)
                fwd = R.prepared_fwd(tmp, w, y, c["eps"], wb)

                def unfused():
                    torch.add(x, res, out=tmp)
                    fwd()

                out = {}
                for name, fn in (("fused", fused), ("unfused", unfused)):
                    for _ in range(20):
                        fn()
                    torch.cuda.synchronize()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(N):
                        fn()
                    e1.record()
                    torch.cuda.synchronize()
                    out[name] = e0.elapsed_time(e1) * 1e3 / N
                gf = decode_layers_graph(R, dev, x, res, w, c["eps"], wb, fused=True)
                gu = decode_layers_graph(R, dev, x, res, w, c["eps"], wb, fused=False)
                rows.append({"B": B, "H": H, "weight_bias": wb, "fused_us": round(out["fused"], 3),
                             "unfused_us": round(out["unfused"], 3),
                             "speedup": round(out["unfused"] / out["fused"], 3),
                             "graph_fused_us": round(gf, 3), "graph_unfused_us": round(gu, 3),
                             "graph_speedup": round(gu / gf, 3)})
                log(f"decode B={B} H={H} wb={wb}: fused {out['fused']:.2f} us, unfused {out['unfused']:.2f} us; "
                    f"32-layer graph: fused {gf:.2f} us, unfused {gu:.2f} us per layer")
    mean_fused = float(np.mean([r["fused_us"] for r in rows]))
    mean_graph = float(np.mean([r["graph_fused_us"] for r in rows]))
    mean_graph_unfused = float(np.mean([r["graph_unfused_us"] for r in rows]))
    print(json.dumps({
        "metric": "fused add+RMSNorm decode latency per call (bf16)", "value": round(mean_fused, 3),
        "unit": "us", "n_gpus": 1, "steps": N, "warmup": 20, "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "graph_fused_us": round(mean_graph, 3), "graph_unfused_us": round(mean_graph_unfused, 3),
        "config": {"workload": "decode fused add+RMSNorm, B in {1,4,8} x H in {2048,4096,8192}, "
                               "weight_bias in {0,1}", "grid": rows},
    }), flush=True)
    return 0


def gate_bench(R, I, dev, args) -> int:
    """Gated activation y = silu(x[:, :d]) * x[:, d:2d], bf16, d = 14336 (the
    Llama-3 8B MLP width), x ~ N(0, 2).  Headline: the [8192, 2d] prefill
    chunk (x 448 MiB, y 224 MiB; algorithmic bytes 3 * rows * d * s, two
    reads and one write per output element), rotating buffer sets so that
    each call reads cold data.  Also: per-call latency at decode batches 1,
    4 and 8 (back-to-back prepared calls), and the backward dx = [da | db]
    at the prefill shape (5 * rows * d * s bytes per call)."""
    rows, d = 8192, 14336
    c = I.gate(rows, d, "bfloat16")
    s = 2
    nbytes = 3 * rows * d * s
    set_bytes = 3 * rows * d * s
    nsets = args.sets or (-(-(1 << 30) // set_bytes) + 1)
    log(f"uploading {nsets} buffer set(s) of {set_bytes / 2**20:.0f} MiB")
    xs = [c["x"].to(dev) for _ in range(nsets)]
    ys = [torch.empty(rows, d, dtype=torch.bfloat16, device=dev) for _ in range(nsets)]
    calls = [R.prepared_gate(x, y) for x, y in zip(xs, ys)]
    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        calls[i % nsets]()
    torch.cuda.synchronize()
    # the timed region holds only gate launches: one event pair around it
    # (on the launch stream) gives the kernel's average launch duration
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record(stream)
    for i in range(args.steps):
        calls[i % nsets]()
    g1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k_us = g0.elapsed_time(g1) * 1e3 / args.steps
    ms_per_step = wall * 1e3 / args.steps
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (k_us * 1e-6) / 1e9
    src_hash = kernel_source_hash(GATE_SOURCES)
    traffic = stored_traffic("gate_8192x14336_bf16", src_hash)
    del xs, ys, calls

    # backward: dx [rows, 2d] from x and dy [rows, d]; 5 * rows * d * s
    # algorithmic bytes (reads of x and dy, the write of dx), two rotating
    # sets of 1.1 GiB each so that every call reads cold data
    vbytes = 5 * rows * d * s
    dy_cpu = I.normal(np.random.default_rng(1), (rows, d), 0.0, 1.0, "bfloat16")
    vx = [c["x"].to(dev) for _ in range(2)]
    vdy = [dy_cpu.to(dev) for _ in range(2)]
    vdx = [torch.empty_like(v) for v in vx]
    vcalls = [R.prepared_gate_vjp(a, b, o) for a, b, o in zip(vx, vdy, vdx)]
    for i in range(args.warmup):
        vcalls[i % 2]()
    torch.cuda.synchronize()
    v0, v1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    v0.record(stream)
    for i in range(args.steps):
        vcalls[i % 2]()
    v1.record(stream)
    torch.cuda.synchronize()
    v_us = v0.elapsed_time(v1) * 1e3 / args.steps
    vjp = {"kernel": "silu_gate_vjp_kernel", "algorithmic_bytes": vbytes, "avg_us": round(v_us, 3),
           "achieved_gbps": round(vbytes / (v_us * 1e-6) / 1e9, 2),
           "frac": round(vbytes / (v_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    log(f"gate backward: {vjp['avg_us']} us, {vjp['achieved_gbps']} GB/s")
    del vx, vdy, vdx, vcalls

    decode = []
    N = max(args.steps, 200)
    for B in (1, 4, 8):
        cb = I.gate(B, d, "bfloat16", seed=B)
        x = cb["x"].to(dev)
        y = torch.empty(B, d, dtype=torch.bfloat16, device=dev)
        fn = R.prepared_gate(x, y)
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(N):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        decode.append({"B": B, "us_per_call": round(e0.elapsed_time(e1) * 1e3 / N, 3)})
        log(f"decode B={B}: {decode[-1]['us_per_call']} us per call")

    out = {
        "metric": "achieved HBM GB/s for the gated activation silu(x[:, :d]) * x[:, d:2d], 8192x14336 bf16",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "silu gate, x [8192, 28672] bf16 ~ N(0,2) -> y [8192, 14336]",
                   "rows": rows, "d": d, "bytes_per_step": nbytes, "buffer_sets": nsets,
                   "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2), "decode": decode,
                   "backward": vjp},
        "roofline": {"kernel": "silu_gate_kernel", "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes": nbytes, "avg_us": round(k_us, 3),
                     "method": "events around the whole timed region / steps"},
        "kernel_source_hash": src_hash,
    }
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        sample = 512
        xs_cpu = c["x"][:sample]
        t0 = time.perf_counter()
        passes = 0
        while True:
            O.silu_gate(xs_cpu)
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= 10.0 or passes >= 20:
                break
        out["cpu_baseline"] = {
            "value": round(passes * 3 * sample * d * s / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{passes} pass(es) over the first {sample} of {rows} rows (d={d}), "
                      f"fp64 C oracle incl. widening, {dt:.1f} s"}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


def sweep_bench(R, I, dev, args) -> int:
    """The small-axis dispatch sweep and the small fp32 case: fwd + VJP per
    call at 16384 rows x D for the D list of the CUDA regression report's
    band (fp16; the tensors fit in the 256 MB last-level cache, so the GB/s
    are effective, not HBM), the same D at rows = 1 (latency), and the
    [64, 512] fp32 POC case (latency).  Back-to-back prepared calls between
    one event pair per measurement."""
    stream = torch.cuda.current_stream(dev)
    N = max(50, min(args.steps, 400))

    def timed(fn):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(N):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / N

    def fwd_vjp_calls(c):
        x, w, dy = c["x"].to(dev), c["w"].to(dev), c["dy"].to(dev)
        rows, D = x.shape
        y, dx = torch.empty_like(x), torch.empty_like(x)
        dw = torch.empty(D, dtype=torch.float32, device=dev)
        ws = R.workspace_for(rows, D, x.dtype, dev)
        f = R.prepared_fwd(x, w, y, c["eps"], c["weight_bias"])
        v = R.prepared_vjp(x, w, dy, dx, dw, ws, c["eps"], c["weight_bias"])
        keep = (x, w, dy, y, dx, dw, ws)

        def step():
            f()
            v()
        return step, keep

    grid = []
    for D in (128, 256, 257, 320, 384, 448, 500, 511, 512, 513, 1024):
        c = I.axis_sweep(16384, D)
        step, keep = fwd_vjp_calls(c)
        us = timed(step)
        nbytes = 5 * 16384 * D * 2 + 2 * D * 2 + 4 * D
        c1 = I.axis_sweep(1, D)
        step1, keep1 = fwd_vjp_calls(c1)
        us1 = timed(step1)
        grid.append({"D": D, "rows16384_us": round(us, 3), "effective_GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "rows1_us": round(us1, 3)})
        log(f"D={D}: {us:.2f} us ({grid[-1]['effective_GBps']} GB/s effective), rows=1 {us1:.2f} us")
        del keep, keep1
    cs = I.poc_small()
    step, keep = fwd_vjp_calls(cs)
    small_us = timed(step)
    worst = min(g["effective_GBps"] for g in grid)
    print(json.dumps({
        "metric": "RMSNorm fwd+VJP over the small-axis D list, 16384 rows fp16 (effective, cache-resident)",
        "value": worst, "unit": "GB/s", "n_gpus": 1, "steps": N, "warmup": 5, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "axis sweep fp16 16384 x D (value = the worst D) and rows = 1; "
                               "POC small case fp32 64 x 512", "grid": grid,
                   "poc_small_fp32_fwd_plus_vjp_us": round(small_us, 3)},
    }), flush=True)
    return 0


def measure_ops(R, dev, rows, D, nsets, timed, gen, dt=torch.bfloat16) -> dict:
    """Every RMSNorm op on [rows, D] (nsets rotating buffer sets of seeded
    device-drawn inputs: x, residual ~ N(0, 1), dy ~ N(0, 0.01), w ~ N(0,
    0.1); weight_bias 1, eps 1e-6): per op the plan (lanes x vectors per
    lane, block, grid; vectors per lane -1 is the streaming kernel, -2 the
    column split) and the algorithmic GB/s of back-to-back prepared calls."""
    sets = []
    for _ in range(nsets):
        x = torch.empty(rows, D, dtype=dt, device=dev).normal_(generator=gen)
        sets.append(dict(x=x, res=torch.empty_like(x).normal_(generator=gen),
                         dy=torch.empty_like(x).normal_(0.0, 0.01, generator=gen),
                         o1=torch.empty_like(x), o2=torch.empty_like(x)))
    w = torch.empty(D, dtype=dt, device=dev).normal_(0.0, 0.1, generator=gen)
    dw = torch.empty(D, dtype=torch.float32, device=dev)
    ws = R.workspace_for(rows, D, dt, dev)
    el = rows * D * sets[0]["x"].element_size()
    ops = {
        "fwd": (0, 2, [R.prepared_fwd(t["x"], w, t["o1"], 1e-6, 1.0) for t in sets]),
        "fused_fwd": (1, 4, [R.prepared_fused(t["x"], t["res"], w, t["o1"], t["o2"], 1e-6, 1.0) for t in sets]),
        "vjp": (2, 3, [R.prepared_vjp(t["x"], w, t["dy"], t["o1"], dw, ws, 1e-6, 1.0) for t in sets]),
        "grad": (3, 4, [R.prepared_grad(t["x"], w, t["dy"], t["o2"], t["o1"], dw, ws, 1e-6, 1.0) for t in sets]),
        "fused_bwd": (4, 4, [R.prepared_fused_vjp(t["x"], w, t["dy"], t["res"], t["o1"], dw, ws, 1e-6, 1.0)
                             for t in sets]),
    }
    row = {"D": D, "rows": rows}
    for name, (op, tensors, calls) in ops.items():
        us = timed(calls)
        q = R.query_config(op, rows, D, dt)
        row[name] = {"us": round(us, 2), "GBps": round((tensors * el + 2 * D) / (us * 1e-6) / 1e9, 1),
                     "plan": f"{q['lanes_per_row']}x{q['vecs_per_lane']} b{q['block_threads']} g{q['num_blocks']}"}
    log(f"{rows}x{D}: " + " | ".join(f"{n} {row[n]['us']} us {row[n]['GBps']} GB/s ({row[n]['plan']})" for n in ops))
    del sets, ops
    torch.cuda.empty_cache()
    return row


def wide_bench(R, dev, args) -> int:
    """Few rows of a very wide D (bf16, four rotating buffer sets; the
    backward forms take the column split there): every op per shape as in
    the widths mode."""
    stream = torch.cuda.current_stream(dev)
    N = max(10, min(args.steps, 30))
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)

    def timed(calls):
        for i in range(2):
            calls[i % len(calls)]()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(N):
            calls[i % len(calls)]()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / N

    grid = [measure_ops(R, dev, rows, D, 4, timed, gen)
            for rows, D in ((16, 1 << 20), (128, 1 << 20), (256, 1 << 20), (511, 262144), (1024, 65536),
                            (4096, 65536))]
    worst = min(r["vjp"]["GBps"] for r in grid)
    print(json.dumps({
        "metric": "achieved HBM GB/s of the RMSNorm VJP on few rows of a wide D, bf16 (value = worst shape)",
        "value": worst, "unit": "GB/s", "n_gpus": 1, "steps": N, "warmup": 2, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "fwd, fused fwd, VJP, grad call, fused backward at bf16 [rows, D], 16..4096 rows, "
                               "D = 65536 .. 2^20", "grid": grid},
    }), flush=True)
    return 0


def widths_bench(R, dev, args) -> int:
    """Every RMSNorm op across model widths (bf16, D = 1152 .. 16384, among
    them widths that no lane count tiles exactly -- 1152, 2304, 3840, 5376 --
    rows = 2^25 / D: 64 MiB per row tensor; then fp16 odd widths whose rows
    end in an overlapped vector, D = 2049, 4097, 6001, 8191), cold: buffer
    sets rotate so that
    no call finds its inputs in the 256 MB last-level cache.  Inputs
    are drawn on the device from a seeded generator (x, residual ~ N(0, 1),
    dy, d_new_residual ~ N(0, 0.01), w ~ N(0, 0.1); weight_bias 1, eps
    1e-6).  Per op: the plan (lanes x vectors per lane, block, grid) and the
    algorithmic GB/s of back-to-back prepared calls between one event pair.
    Ten buffer sets rotate (each op's cycle touches 1.25-2.5 GiB, five to ten
    times the last-level cache)."""
    stream = torch.cuda.current_stream(dev)
    N = max(20, min(args.steps, 60))
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)

    def timed(calls):
        for i in range(4):
            calls[i % len(calls)]()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(N):
            calls[i % len(calls)]()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / N

    grid = []
    for D in (1152, 1536, 2048, 2304, 2560, 3072, 3584, 3840, 4096, 4608, 5120, 5376, 5632, 6144, 6656, 7168, 7680,
              8192, 9216, 10240, 11264, 12288, 14336, 16384):
        grid.append(measure_ops(R, dev, (1 << 25) // D, D, 10, timed, gen))
    # odd widths (fp16 rows whose last 16-byte vector is overlapped), same
    # 64 MiB tensors
    odd = [measure_ops(R, dev, (1 << 25) // D, D, 10, timed, gen, dt=torch.float16) for D in (2049, 4097, 6001, 8191)]
    worst = min(r["vjp"]["GBps"] for r in grid)
    print(json.dumps({
        "metric": "achieved HBM GB/s of the RMSNorm VJP across model widths, bf16, 64 MiB tensors (value = worst D)",
        "value": worst, "unit": "GB/s", "n_gpus": 1, "steps": N, "warmup": 4, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "fwd, fused fwd, VJP, grad call, fused backward at bf16 [2^25 / D, D], "
                               "D = 1152 .. 16384 (and fp16 odd widths D = 2049, 4097, 6001, 8191 under odd_grid)",
                   "grid": grid, "odd_grid": odd},
    }), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", choices=["poc", "prefill", "decode", "grad", "gate", "sweep", "widths", "wide",
                                           "ceiling", "dwreduce"],
                    default="poc")
    ap.add_argument("--sets", type=int, default=0, help="rotating buffer sets (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(rows would shard across GPUs with one all-reduce of dw). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2
    if args.workload == "ceiling":
        return ceiling_bench()
    if args.workload == "dwreduce":
        return dwreduce_bench()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2

    import backward_rmsnorm_fwd_two_amd as R
    from backward_rmsnorm_fwd_two_amd import inputs as I

    dev = torch.device("cuda:0")
    if args.workload == "decode":
        return decode_bench(R, I, dev, args)
    if args.workload == "grad":
        return grad_bench(R, I, dev, args)
    if args.workload == "gate":
        return gate_bench(R, I, dev, args)
    if args.workload == "sweep":
        return sweep_bench(R, I, dev, args)
    if args.workload == "widths":
        return widths_bench(R, dev, args)
    if args.workload == "wide":
        return wide_bench(R, dev, args)
    fused = args.workload == "prefill"
    out = step_bench(R, I, dev, args, fused)
    if not fused:
        # the second headline (fused add+RMSNorm fwd + VJP at prefill scale)
        # as an extra key of the same line
        out["prefill"] = step_bench(R, I, dev, args, True, nested=True)
    print(json.dumps(out), flush=True)
    return 0


def timed_b2b(calls, n, stream):
    """Average duration (us) of `n` back-to-back calls rotating through
    `calls`, from one HIP event pair on the stream the kernels run on."""
    for i in range(3):
        calls[i % len(calls)]()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        calls[i % len(calls)]()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def step_bench(R, I, dev, args, fused, nested=False):
    """One step = forward (fused add+RMSNorm for the prefill workload) +
    VJP over one batch; value = algorithmic bytes per step / wall time per
    step over exactly args.steps steps between device syncs.  The timed
    region holds nothing but the steps; per-op figures come from separate
    passes after it."""
    log(f"generating inputs ({'prefill' if fused else 'poc'})")
    if fused:
        c = I.prefill()
        workload = "fused add+RMSNorm fwd + VJP, [32768, 8192] bf16, weight_bias 1, eps 1e-6"
    else:
        c = I.poc_8192x4096()
        workload = "RMSNorm fwd + VJP, [8192, 4096] fp16, x/w/dy ~ U(0,1), eps 1e-5, weight_bias 0"
    rows, D = c["x"].shape
    s = c["x"].element_size()
    eps, wb = c["eps"], c["weight_bias"]
    if fused:
        fwd_bytes = 4 * rows * D * s + D * s          # read x, res; write normed, new_residual; read w
    else:
        fwd_bytes = 2 * rows * D * s + D * s          # read x; write y; read w
    vjp_bytes = 3 * rows * D * s + D * s + 4 * D      # read x, dy; write dx; read w; write dw (fp32)
    step_bytes = fwd_bytes + vjp_bytes

    set_bytes = (4 * rows * D * s) + (2 * rows * D * s if fused else 0)
    nsets = args.sets or (max(1, -(-(1 << 30) // set_bytes) + 1) if set_bytes < (1 << 30) else 1)
    log(f"uploading {nsets} buffer set(s) of {set_bytes / 2**20:.0f} MiB")
    w = c["w"].to(dev)
    sets = []
    for _ in range(nsets):
        st = {"x": c["x"].to(dev), "dy": c["dy"].to(dev)}
        if fused:
            st["res"] = c["residual"].to(dev)
            st["normed"] = torch.empty_like(st["x"])
            st["newres"] = torch.empty_like(st["x"])
        else:
            st["y"] = torch.empty_like(st["x"])
        st["dx"] = torch.empty_like(st["x"])
        sets.append(st)
    dw = torch.empty(D, dtype=torch.float32, device=dev)
    ws = R.workspace_for(rows, D, c["x"].dtype, dev)
    stream = torch.cuda.current_stream(dev)

    # Arguments are marshalled once per buffer set (prepared C calls), so
    # the host enqueues faster than the GPU drains and no step waits on Python.
    f_calls, v_calls = [], []
    for st in sets:
        if fused:
            f_calls.append(R.prepared_fused(st["x"], st["res"], w, st["normed"], st["newres"], eps, wb))
        else:
            f_calls.append(R.prepared_fwd(st["x"], w, st["y"], eps, wb))
        xin = st["newres"] if fused else st["x"]
        v_calls.append(R.prepared_vjp(xin, w, st["dy"], st["dx"], dw, ws, eps, wb))

    def step(i):
        k = i % nsets
        f_calls[k]()
        v_calls[k]()

    log(f"warmup {args.warmup}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps bracketed by device syncs, nothing else.
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # After the timed region: per-op event figures.  (1) Sampled steps with
    # event pairs around each op: an event record costs the GPU a few
    # microseconds, so these run high.  (2) Each op back to back on the
    # rotating sets with one event pair around 100 calls: the launch
    # durations the roofline uses (they agree with the kernel trace).
    nsamp = 20
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nsamp)]
    for i in range(nsamp):
        k = i % nsets
        evs[i][0].record(stream)
        f_calls[k]()
        evs[i][1].record(stream)
        v_calls[k]()
        evs[i][2].record(stream)
    torch.cuda.synchronize()
    fwd_ms = np.array([elapsed_ms(e[0], e[1]) for e in evs])
    vjp_ms = np.array([elapsed_ms(e[1], e[2]) for e in evs])
    NB = 100
    vjp_b2b_us = timed_b2b(v_calls, NB, stream)
    fwd_b2b_us = timed_b2b(f_calls, NB, stream)

    extra = {}
    if fused:
        # The backward of the fused form with a residual-stream gradient
        # (fused_add_rmsnorm_vjp): reads h, dy and d_new_residual, writes dh.
        dr = torch.empty_like(sets[0]["x"]).normal_(0.0, 0.01)
        rg = R.prepared_fused_vjp(sets[0]["newres"], w, sets[0]["dy"], dr, sets[0]["dx"], dw, ws, eps, wb)
        t_rg = timed_b2b([rg], 10, stream) * 1e-6
        rg_bytes = 4 * rows * D * s + D * s + 4 * D
        extra = {"fused_vjp_with_residual_grad_us": round(t_rg * 1e6, 2),
                 "fused_vjp_with_residual_grad_GBps": round(rg_bytes / t_rg / 1e9, 1)}
        del dr
    else:
        # Warm ("effective") figure: the same buffer set every step, so the
        # 256 MB last-level cache serves part of the traffic -- not an HBM number.
        warm_us = timed_b2b([lambda: step(0)], 100, stream)
        extra["warm_effective"] = {
            "step_us": round(warm_us, 3), "GBps": round(step_bytes / (warm_us * 1e-6) / 1e9, 1),
            "note": "one buffer set reused every step: partly served by the last-level cache"}
        # The same outputs (y, dx, dw) from the one-launch grad call, which
        # reads x and dy once (4*R*D*s + w + dw bytes instead of 5*R*D*s).
        g_calls = [R.prepared_grad(st["x"], w, st["dy"], st["y"], st["dx"], dw, ws, eps, wb) for st in sets]
        g_us = timed_b2b(g_calls, NB, stream)
        g_bytes = 4 * rows * D * s + D * s + 4 * D
        extra["grad_call_same_outputs"] = {
            "us_per_call": round(g_us, 3), "GBps_on_its_bytes": round(g_bytes / (g_us * 1e-6) / 1e9, 1),
            "note": "rmsnorm_fwd_vjp: the same y, dx, dw in one launch; not the headline"}

    src_hash = kernel_source_hash()
    vjp_gbps = vjp_bytes / (vjp_b2b_us * 1e-6) / 1e9
    vjp_roofline = {
        "kernel": "rmsnorm_vjp (vjp_rows + dw_combine launches)", "bound": "hbm",
        "achieved": round(vjp_gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": round(vjp_gbps / HBM_PEAK_GBPS, 4),
        "traffic": stored_traffic("vjp_prefill_32768x8192_bf16" if fused else "vjp_poc_8192x4096_fp16", src_hash),
        "algorithmic_bytes": vjp_bytes, "avg_us": round(vjp_b2b_us, 3),
        "method": "events around 100 back-to-back VJP calls on the launch stream, after the timed region"}
    fwd_gbps = fwd_bytes / (fwd_b2b_us * 1e-6) / 1e9
    fwd_roofline = {
        "kernel": "fused_add_rmsnorm_fwd (fwd_rows<FUSED>)" if fused else "rmsnorm_fwd (fwd_rows)",
        "bound": "hbm", "achieved": round(fwd_gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": round(fwd_gbps / HBM_PEAK_GBPS, 4),
        "traffic": stored_traffic("fused_fwd_prefill_32768x8192_bf16" if fused else "fwd_poc_8192x4096_fp16", src_hash),
        "algorithmic_bytes": fwd_bytes, "avg_us": round(fwd_b2b_us, 3),
        "method": "events around 100 back-to-back forward calls on the launch stream, after the timed region"}
    # the roofline object is the dominant kernel's: the one that takes the
    # larger share of the step
    roofline, other = (vjp_roofline, fwd_roofline) if vjp_b2b_us >= fwd_b2b_us else (fwd_roofline, vjp_roofline)
    ops = {
        "fwd_sampled_mean": round(float(fwd_ms.mean()) * 1e3, 3),
        "vjp_sampled_mean": round(float(vjp_ms.mean()) * 1e3, 3),
        "sampled_steps": nsamp,
        "fwd_back_to_back": round(fwd_b2b_us, 3), "vjp_back_to_back": round(vjp_b2b_us, 3),
        "summed_back_to_back_GBps": round(step_bytes / ((fwd_b2b_us + vjp_b2b_us) * 1e-6) / 1e9, 1),
        "note": "after the timed region; sampled_* carry per-call event overhead, back_to_back_* do not"}
    if nested:
        res = {"workload": workload, "rows": rows, "D": D, "storage_dtype": str(c["x"].dtype).replace("torch.", ""),
               "bytes_per_step": step_bytes, "buffer_sets": nsets, "steps": args.steps, "warmup": args.warmup,
               "ms_per_step": round(ms_per_step, 5), "value": round(value, 2), "unit": "GB/s",
               "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2), "roofline": roofline,
               "other_kernel": other, "ops_event_us": ops, **extra}
        del sets, f_calls, v_calls
        torch.cuda.empty_cache()
        return res

    log("copy ceiling")
    ceiling = copy_ceiling()
    out = {
        "metric": METRIC if not fused else "achieved HBM GB/s for fused add+RMSNorm fwd + VJP, 32768x8192 bf16",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": workload, "rows": rows, "D": D,
            "storage_dtype": str(c["x"].dtype).replace("torch.", ""),
            "bytes_per_step": step_bytes, "buffer_sets": nsets,
            "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        },
        "roofline": roofline,
        "other_kernel": other,
        "ops_event_us": ops,
        "copy_ceiling_GBps": round(ceiling, 1),
        "pct_of_copy_ceiling": round(100.0 * value / ceiling, 2),
        **extra,
        "kernel_source_hash": src_hash,
        "context": "MLX PR POC, Metal, model not stated: ~1.65 ms per grad call at this shape "
                   "(= %.0f GB/s on this byte model); not comparable hardware" % (step_bytes / 1.65e-3 / 1e9)
                   if not fused else None,
    }
    del sets, f_calls, v_calls
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle)")
        out["cpu_baseline"] = cpu_oracle_baseline(c, rows, D, fwd_bytes, vjp_bytes, fused)
    else:
        out["cpu_baseline"] = None
    return out


if __name__ == "__main__":
    sys.exit(main())
