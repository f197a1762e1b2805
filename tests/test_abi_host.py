"""Host-side checks (no GPU): the C-ABI library loads and exports every
function include/rmsnorm_mi355x.h declares; the header compiles as strict
C99 and a C program links against the library; the product path and the
oracle share no code and never import each other."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rmsnorm_mi355x.h")
PKG = os.path.join(ROOT, "backward_rmsnorm_fwd_two_amd")
LIB = os.path.join(PKG, "librmsnorm_mi355x.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_three_operations():
    names = declared_functions()
    for n in ("rmsnorm_fwd", "fused_add_rmsnorm_fwd", "rmsnorm_vjp", "rmsnorm_vjp_workspace_bytes",
              "rmsn_status_str"):
        assert n in names, names


def test_library_exports_every_declared_symbol():
    if not os.path.exists(LIB):
        from backward_rmsnorm_fwd_two_amd import build
        build.build(verbose=False)
    lib = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported


def test_status_strings_without_gpu():
    lib = ctypes.CDLL(LIB)
    lib.rmsn_status_str.restype = ctypes.c_char_p
    for st in range(-8, 1):
        s = lib.rmsn_status_str(st).decode()
        assert s and s != "unknown status"
    # argument errors are reported before any device call
    lib.rmsnorm_fwd.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                                        ctypes.c_float, ctypes.c_float, ctypes.c_void_p]
    assert lib.rmsnorm_fwd(None, None, None, 4, 8, 1, 1e-5, 0.0, None) == -1
    assert lib.rmsnorm_fwd(None, None, None, 4, 8, 9, 1e-5, 0.0, None) == -3
    assert lib.rmsnorm_fwd(None, None, None, -1, 8, 1, 1e-5, 0.0, None) == -2
    assert lib.rmsnorm_fwd(None, None, None, 0, 8, 1, 1e-5, 0.0, None) == 0
    lib.rmsnorm_vjp_noalloc.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                                                 ctypes.c_float, ctypes.c_float, ctypes.c_void_p]
    assert lib.rmsnorm_vjp_noalloc(None, None, None, None, None, 4, 8, 9, 1e-5, 0.0, None) == -3
    assert lib.rmsnorm_vjp_noalloc(None, None, None, None, None, 4, 0, 1, 1e-5, 0.0, None) == -2


def _py_sources(d):
    for base, _, files in os.walk(d):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".c", ".h")):
                yield os.path.join(base, f)


def test_product_never_references_the_oracle():
    for path in _py_sources(PKG):
        text = open(path, errors="ignore").read()
        assert not re.search(r"\boracle\b", text.replace("the oracle", "")), path


def test_oracle_never_imports_the_product():
    for path in _py_sources(os.path.join(ROOT, "oracle")):
        text = open(path, errors="ignore").read()
        assert "backward_rmsnorm_fwd_two_amd" not in text, path
        assert "rmsn_device" not in text and "rmsn_kernels" not in text, path


def test_gpu_marker_registered(pytestconfig):
    markers = pytestconfig.getini("markers")
    assert any(m.startswith("gpu") for m in markers)


def test_gate_argument_errors_and_plan_without_gpu():
    lib = ctypes.CDLL(LIB)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.silu_gate.argtypes = [vp, vp, i64, i64, ctypes.c_int, vp]
    assert lib.silu_gate(None, None, 4, 8, 2, None) == -1
    assert lib.silu_gate(None, None, 4, 8, 9, None) == -3
    assert lib.silu_gate(None, None, 4, 0, 2, None) == -2
    assert lib.silu_gate(None, None, 4, (1 << 28) + 1, 2, None) == -2
    assert lib.silu_gate(None, None, 0, 8, 2, None) == 0

    class Cfg(ctypes.Structure):
        _fields_ = [(n, ctypes.c_int32) for n in
                    ("lanes_per_row", "vecs_per_lane", "vec_bytes", "block_threads", "num_blocks")]

    lib.rmsn_query_config.argtypes = [ctypes.c_int, i64, i64, ctypes.c_int, ctypes.c_int,
                                      ctypes.POINTER(Cfg)]

    def plan(rows, d, dt, align=16):
        c = Cfg()
        st = lib.rmsn_query_config(5, rows, d, dt, align, ctypes.byref(c))
        assert st == 0, st
        return (c.lanes_per_row, c.vecs_per_lane, c.vec_bytes, c.block_threads, c.num_blocks)

    # Llama-3 8B MLP width, bf16: 16-byte loads, one vector per thread,
    # 14336 * 2 / 16 = 1792 vectors per row, 64 per chunk (one-wave blocks)
    assert plan(8192, 14336, 2) == (0, 1, 16, 64, 8192 * 1792 // 64)
    assert plan(1, 14336, 2) == (0, 1, 16, 64, 28)
    # odd d in bf16: element loads
    assert plan(3, 1001, 2)[2] == 2 and plan(3, 1001, 2)[1] == 8
    # the load width follows the row pitch, not the pointers' alignment
    for align in (16, 8, 4):
        assert plan(3, 1000, 0, align=align)[2] == 16
    assert plan(3, 1002, 0)[2] == 8


def test_in_place_alias_rules_without_gpu():
    """Argument checks run before any device call: without a GPU, a call that
    passes them fails at the first HIP call (-6); an overlap the rules refuse
    returns -5.  Pointers are fake addresses (never dereferenced)."""
    lib = ctypes.CDLL(LIB)
    vp, i64, f32, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    lib.rmsnorm_fwd.argtypes = [vp, vp, vp, i64, i64, ci, f32, f32, vp]
    lib.fused_add_rmsnorm_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, ci, f32, f32, vp]
    lib.rmsnorm_fwd_vjp.argtypes = [vp] * 7 + [ctypes.c_size_t, i64, i64, ci, f32, f32, vp]
    lib.fused_add_rmsnorm_vjp.argtypes = [vp] * 7 + [ctypes.c_size_t, i64, i64, ci, f32, f32, vp]
    R, D = 4, 64
    tb = R * D * 2                                   # fp16 [4, 64]
    X, RES, W, DY, OUT, OUT2, DW, WS = (0x100000 * (i + 1) for i in range(8))
    HIP, OVL = -6, -5
    # forward: y over x allowed; y one row into x, or over w, refused
    assert lib.rmsnorm_fwd(X, W, X, R, D, 1, 1e-5, 0.0, None) == HIP
    assert lib.rmsnorm_fwd(X, W, X + 2 * D, R, D, 1, 1e-5, 0.0, None) == OVL
    assert lib.rmsnorm_fwd(X, W, W, 1, D, 1, 1e-5, 0.0, None) == OVL
    # fused: each output over x or residual; outputs never over each other
    for normed, newres in ((X, RES), (RES, X), (X, OUT), (OUT, RES)):
        assert lib.fused_add_rmsnorm_fwd(X, RES, W, normed, newres, R, D, 1, 1e-5, 0.0, None) == HIP
    assert lib.fused_add_rmsnorm_fwd(X, RES, W, X, X, R, D, 1, 1e-5, 0.0, None) == OVL
    assert lib.fused_add_rmsnorm_fwd(X, RES, W, OUT, OUT, R, D, 1, 1e-5, 0.0, None) == OVL
    assert lib.fused_add_rmsnorm_fwd(X, RES, W, RES + 2, OUT, R, D, 1, 1e-5, 0.0, None) == OVL
    # grad call: y and dx each over x or dy, not over each other, not partial
    ws_bytes = 1 << 20
    for y, dx in ((X, DY), (DY, X), (OUT, X), (DY, OUT2)):
        assert lib.rmsnorm_fwd_vjp(X, W, DY, y, dx, DW, WS, ws_bytes, R, D, 1, 1e-5, 0.0, None) == HIP
    assert lib.rmsnorm_fwd_vjp(X, W, DY, X, X, DW, WS, ws_bytes, R, D, 1, 1e-5, 0.0, None) == OVL
    assert lib.rmsnorm_fwd_vjp(X, W, DY, OUT, DY + tb // 2, DW, WS, ws_bytes, R, D, 1, 1e-5, 0.0, None) == OVL
    # dw never overlaps a row buffer
    assert lib.rmsnorm_fwd_vjp(X, W, DY, OUT, OUT2, X, WS, ws_bytes, R, D, 1, 1e-5, 0.0, None) == OVL
    # fused backward: dh over h, dy or d_new_residual
    for dh in (X, DY, RES, OUT):
        assert lib.fused_add_rmsnorm_vjp(X, W, DY, RES, dh, DW, WS, ws_bytes, R, D, 1, 1e-5, 0.0, None) == HIP
    assert lib.fused_add_rmsnorm_vjp(X, W, DY, RES, RES + 64, DW, WS, ws_bytes, R, D, 1, 1e-5, 0.0, None) == OVL


C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "rmsnorm_mi355x.h"

int main(void) {
    /* every status has a message */
    for (int st = -8; st <= 0; ++st) {
        const char *s = rmsn_status_str(st);
        if (s == NULL || strlen(s) == 0) return 10;
    }
    /* host-side argument checks, before any device call */
    if (rmsnorm_fwd(NULL, NULL, NULL, 4, 8, RMSN_F16, 1e-5f, 0.0f, NULL) != RMSN_E_NULLPTR) return 11;
    if (rmsnorm_fwd(NULL, NULL, NULL, -1, 8, RMSN_F16, 1e-5f, 0.0f, NULL) != RMSN_E_SHAPE) return 12;
    if (rmsnorm_fwd(NULL, NULL, NULL, 0, 8, RMSN_F16, 1e-5f, 0.0f, NULL) != RMSN_OK) return 13;
    if (fused_add_rmsnorm_fwd(NULL, NULL, NULL, NULL, NULL, 4, 8, 7, 1e-6f, 1.0f, NULL) != RMSN_E_DTYPE) return 14;
    if (rmsnorm_vjp(NULL, NULL, NULL, NULL, NULL, NULL, 0, 4, 0, RMSN_BF16, 1e-6f, 0.0f, NULL) != RMSN_E_SHAPE)
        return 15;
    if (rmsnorm_vjp_workspace_bytes(-1, 4096, RMSN_F16) != 0) return 16;
    printf("c abi ok\n");
    return 0;
}
"""


def test_header_is_plain_c_and_links_from_c(tmp_path):
    """The header compiles as strict C99 (no C++ in the declarations) and a C
    program links against the library and calls it: status strings and the
    argument checks that run before any device call."""
    if not os.path.exists(LIB):
        from backward_rmsnorm_fwd_two_amd import build
        build.build(verbose=False)
    src = tmp_path / "abi.c"
    exe = tmp_path / "abi"
    src.write_text(C_PROGRAM)
    cc = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                         "-I", os.path.join(ROOT, "include"), str(src), "-L", PKG, "-lrmsnorm_mi355x",
                         f"-Wl,-rpath,{PKG}", "-o", str(exe)], capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, (run.returncode, run.stdout, run.stderr)
    assert run.stdout.strip() == "c abi ok"
