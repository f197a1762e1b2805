"""CPU: the host logic of bench.py that needs no GPU.

- Every profile the bench reads HBM traffic from was taken on the current
  kernel sources (its recorded source hash is the one bench.py computes), so
  the bench line's `traffic` fields are not silently null.
- The stored-traffic reader returns the recorded bytes only for a matching
  hash.
- The algorithmic bytes the rooflines use equal the per-element counts of
  the method: forward 2RDs + Ds, VJP 3RDs + Ds + 4D, fused forward 4RDs + Ds.
- More than one GPU is refused with a message, before anything touches a GPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

# profiles whose `traffic per launch` lines feed the bench line, with the
# sources they depend on
TRAFFIC_PROFILES = {
    "vjp_poc_8192x4096_fp16": bench.KERNEL_SOURCES,
    "fwd_poc_8192x4096_fp16": bench.KERNEL_SOURCES,
    "vjp_prefill_32768x8192_bf16": bench.KERNEL_SOURCES,
    "fused_fwd_prefill_32768x8192_bf16": bench.KERNEL_SOURCES,
    "gate_8192x14336_bf16": bench.GATE_SOURCES,
}


@pytest.mark.parametrize("name", sorted(TRAFFIC_PROFILES))
def test_traffic_profiles_match_the_sources(name):
    h = bench.kernel_source_hash(TRAFFIC_PROFILES[name])
    t = bench.stored_traffic(name, h)
    assert t is not None, f"profiles/{name}.md was not taken on the current sources (hash {h})"
    assert t > 0


def test_stored_traffic_needs_the_matching_hash():
    h = bench.kernel_source_hash()
    assert bench.stored_traffic("vjp_poc_8192x4096_fp16", "0" * 16) is None
    assert bench.stored_traffic("no_such_profile", h) is None


def test_traffic_is_close_to_the_algorithmic_bytes():
    """The measured bytes per launch stay within a few percent above the
    algorithmic bytes (the dw partial rows are the only overhead)."""
    R, D, s = 8192, 4096, 2
    fwd = 2 * R * D * s + D * s
    vjp = 3 * R * D * s + D * s + 4 * D
    assert (fwd, vjp, fwd + vjp) == (134225920, 201351168, 335577088)
    Rp, Dp = 32768, 8192
    ffwd = 4 * Rp * Dp * 2 + Dp * 2
    pvjp = 3 * Rp * Dp * 2 + Dp * 2 + 4 * Dp
    assert ffwd + pvjp == 3758161920
    h = bench.kernel_source_hash()
    for name, alg, hi in (("vjp_poc_8192x4096_fp16", vjp, 1.05), ("fwd_poc_8192x4096_fp16", fwd, 1.01),
                          ("vjp_prefill_32768x8192_bf16", pvjp, 1.02),
                          ("fused_fwd_prefill_32768x8192_bf16", ffwd, 1.01)):
        t = bench.stored_traffic(name, h)
        assert t is not None and 0.999 * alg <= t <= hi * alg, (name, t, alg)


def test_more_than_one_gpu_is_refused():
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, env=env, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
