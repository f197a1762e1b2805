"""Pins for the fp64 CPU oracle, checked against what the pages and the
mathematics fix -- never against the oracle's own formula retyped.

Forward  (MLX PR "RMSNormVJP backward writes a full {n_rows, D} gw_temp
intermediate", POC reference expression; mlxcel issue "Fused residual-add
RMSNorm ...", FusedAddRMSNorm bullet and Regression guard):
  closed forms (unit weight mean-square identity, constant row, zero row,
  D = 1), eps-inside-the-root homogeneity, scaled weight, Gemma 1+w,
  row-permutation equivariance, a hand-worked exact example.
Backward: central finite differences of L = sum(dy * y) in fp64, torch fp64
  autograd of the POC expression (a library routine), the identity
  <x, dx> = eps r^3 S, D = 1 and zero-row closed forms, linearity in dy,
  additivity of dw over row splits, dw independent of w and weight_bias.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


def _case(rows, D, seed=0, scale=1.0):
    r = _rng(seed)
    x = r.standard_normal((rows, D)) * scale
    w = r.uniform(0.5, 1.5, D)
    dy = r.standard_normal((rows, D))
    return x, w, dy


# --------------------------------------------------------------- forward pins

@pytest.mark.parametrize("eps", [1e-5, 1e-6, 0.25, 3.0])
@pytest.mark.parametrize("D", [1, 2, 7, 64, 513])
def test_fwd_unit_weight_mean_square(eps, D):
    # w = 1, weight_bias = 0: mean_j y^2 = ms / (ms + eps), ms = mean_j x^2.
    # A wrong denominator (D-1) or eps outside the root breaks this.
    x, _, _ = _case(5, D, seed=D)
    eps32 = float(np.float32(eps))
    y, _ = O.rmsnorm_fwd(x, np.ones(D), eps, 0.0)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.mean(y * y, axis=1), ms / (ms + eps32), rtol=1e-13)


@pytest.mark.parametrize("c", [0.5, 3.0, -2.0, 1e-3])
def test_fwd_constant_row(c):
    D, eps = 37, 1e-5
    w = _rng(1).uniform(-1, 2, D)
    eps32 = float(np.float32(eps))
    for wb in (0.0, 1.0):
        y, rstd = O.rmsnorm_fwd(np.full((1, D), c), w, eps, wb)
        np.testing.assert_allclose(y[0], (wb + w) * c / np.sqrt(c * c + eps32), rtol=1e-14)
        np.testing.assert_allclose(rstd[0], 1 / np.sqrt(c * c + eps32), rtol=1e-14)


def test_fwd_zero_row_and_D1():
    w = np.array([0.7])
    y, _ = O.rmsnorm_fwd(np.zeros((3, 1)), w, 1e-6, 0.0)
    assert np.all(y == 0)
    x = np.array([[2.0], [-0.5], [1e-4]])
    eps = 2.0 ** -12
    y, _ = O.rmsnorm_fwd(x, w, eps, 1.0)
    np.testing.assert_allclose(y[:, 0], 1.7 * x[:, 0] / np.sqrt(x[:, 0] ** 2 + eps), rtol=1e-14)


@pytest.mark.parametrize("c", [2.0, 4.0, 0.5])
def test_fwd_eps_inside_root_homogeneity(c):
    # y(c x; c^2 eps) == y(x; eps) holds only with eps inside the root next to
    # the mean.  Powers of two keep every scaled operand exact.
    x, w, _ = _case(6, 33, seed=3)
    eps = 2.0 ** -10
    y1, _ = O.rmsnorm_fwd(x, w, eps, 0.25)
    y2, _ = O.rmsnorm_fwd(c * x, w, c * c * eps, 0.25)
    np.testing.assert_allclose(y2, y1, rtol=1e-15, atol=0)


def test_fwd_scaled_weight_and_gemma():
    # weight scaled by k scales y by k (weight_bias 0); weight_bias 1 equals
    # weight_bias 0 with w + 1 (Gemma convention).
    x, w, _ = _case(4, 50, seed=4)
    y, _ = O.rmsnorm_fwd(x, w, 1e-6, 0.0)
    yk, _ = O.rmsnorm_fwd(x, 3.0 * w, 1e-6, 0.0)
    np.testing.assert_allclose(yk, 3.0 * y, rtol=1e-14)
    yg, _ = O.rmsnorm_fwd(x, w, 1e-6, 1.0)
    y1, _ = O.rmsnorm_fwd(x, w + 1.0, 1e-6, 0.0)
    np.testing.assert_array_equal(yg, y1)


def test_fwd_row_permutation():
    x, w, _ = _case(9, 21, seed=5)
    p = _rng(9).permutation(9)
    y, _ = O.rmsnorm_fwd(x, w, 1e-5, 0.0)
    yp, _ = O.rmsnorm_fwd(x[p], w, 1e-5, 0.0)
    np.testing.assert_array_equal(yp, y[p])


def test_hand_worked_examples():
    # Exact rational examples worked by hand from the POC reference
    # expression with eps = 0 (see tests/golden/hand_worked.json).
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.array(c["x"], dtype=np.float64)[None, :]
        w = np.array(c["w"], dtype=np.float64)
        dy = np.array(c["dy"], dtype=np.float64)[None, :]
        y, _ = O.rmsnorm_fwd(x, w, c["eps"], c["weight_bias"])
        np.testing.assert_allclose(y[0], c["y"], rtol=1e-15)
        dx, dw = O.rmsnorm_vjp(x, w, dy, c["eps"], c["weight_bias"])
        np.testing.assert_allclose(dx[0], c["dx"], rtol=1e-14, atol=1e-16)
        np.testing.assert_allclose(dw, c["dw"], rtol=1e-14, atol=1e-16)


# ----------------------------------------------------------------- fused pins

def test_fused_is_add_then_norm_of_unrounded_sum():
    r = _rng(7)
    x = r.standard_normal((5, 40)).astype(np.float32)
    res = r.standard_normal((5, 40)).astype(np.float32)
    w = r.normal(0, 0.1, 40)
    normed, newres = O.fused_add_rmsnorm_fwd(x, res, w, 1e-6, 1.0)
    h = x.astype(np.float64) + res.astype(np.float64)
    np.testing.assert_array_equal(newres, h)
    y, _ = O.rmsnorm_fwd(h, w, 1e-6, 1.0)
    np.testing.assert_array_equal(normed, y)


# -------------------------------------------------------------- backward pins

def _loss(x, w, dy, eps, wb):
    y, _ = O.rmsnorm_fwd(x, w, eps, wb)
    return float(np.sum(dy * y))


@pytest.mark.parametrize("rows", [1, 2, 3])
@pytest.mark.parametrize("D", [1, 2, 3, 5, 8, 17])
@pytest.mark.parametrize("wb", [0.0, 1.0])
def test_vjp_finite_differences(rows, D, wb):
    x, w, dy = _case(rows, D, seed=10 * rows + D)
    eps = 2.0 ** -8
    dx, dw = O.rmsnorm_vjp(x, w, dy, eps, wb)
    h = 1e-6
    fd_x = np.zeros_like(x)
    for i in range(rows):
        for j in range(D):
            xp, xm = x.copy(), x.copy()
            xp[i, j] += h
            xm[i, j] -= h
            fd_x[i, j] = (_loss(xp, w, dy, eps, wb) - _loss(xm, w, dy, eps, wb)) / (2 * h)
    fd_w = np.zeros(D)
    for j in range(D):
        wp, wm = w.copy(), w.copy()
        wp[j] += h
        wm[j] -= h
        fd_w[j] = (_loss(x, wp, dy, eps, wb) - _loss(x, wm, dy, eps, wb)) / (2 * h)
    scale_x = max(1.0, np.max(np.abs(dx)))
    scale_w = max(1.0, np.max(np.abs(dw)))
    assert np.max(np.abs(fd_x - dx)) <= 1e-7 * scale_x
    assert np.max(np.abs(fd_w - dw)) <= 1e-7 * scale_w


@pytest.mark.parametrize("wb", [0.0, 1.0])
def test_vjp_torch_fp64_autograd(wb):
    # Library cross-check: torch autograd (fp64, CPU) of the POC reference
    # expression gives the gradients for x and w.
    x, w, dy = _case(16, 96, seed=11)
    eps = 1e-5
    eps32 = float(np.float32(eps))
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    dyt = torch.tensor(dy)
    y = torch.rsqrt(xt.square().mean(-1, keepdim=True) + eps32) * xt * (wb + wt)
    (y * dyt).sum().backward()
    dx, dw = O.rmsnorm_vjp(x, w, dy, eps, wb)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_vjp_projection_identity():
    # <x_i, dx_i> = eps * r_i^3 * S_i,  S_i = sum_j dy_ij g_j x_ij.
    x, w, dy = _case(8, 64, seed=12)
    eps = 0.5
    wb = 0.3
    dx, _ = O.rmsnorm_vjp(x, w, dy, eps, wb)
    _, rstd = O.rmsnorm_fwd(x, w, eps, wb)
    eps32 = float(np.float32(eps))
    S = np.sum(dy * (np.float32(wb) + w) * x, axis=1)
    lhs = np.sum(x * dx, axis=1)
    np.testing.assert_allclose(lhs, eps32 * rstd ** 3 * S, rtol=1e-10, atol=1e-13)
    # eps = 0: RMSNorm is homogeneous of degree 0, so <x, dx> = 0.
    dx0, _ = O.rmsnorm_vjp(x, w, dy, 0.0, wb)
    assert np.max(np.abs(np.sum(x * dx0, axis=1))) < 1e-12


def test_vjp_D1_and_zero_row():
    w = np.array([0.8])
    x = np.array([[1.5], [-0.25]])
    dy = np.array([[2.0], [-3.0]])
    eps = 2.0 ** -6
    dx, dw = O.rmsnorm_vjp(x, w, dy, eps, 1.0)
    g = 1.8
    np.testing.assert_allclose(dx[:, 0], g * dy[:, 0] * eps * (x[:, 0] ** 2 + eps) ** -1.5, rtol=1e-13)
    np.testing.assert_allclose(dw[0], np.sum(dy[:, 0] * x[:, 0] / np.sqrt(x[:, 0] ** 2 + eps)), rtol=1e-13)
    # zero row: dx = g dy / sqrt(eps), no dw contribution.
    w = _rng(3).uniform(0.5, 1.5, 6)
    dy = _rng(4).standard_normal((1, 6))
    dx, dw = O.rmsnorm_vjp(np.zeros((1, 6)), w, dy, eps, 0.0)
    np.testing.assert_allclose(dx[0], w * dy[0] / np.sqrt(eps), rtol=1e-14)
    assert np.all(dw == 0)


def test_vjp_linear_in_dy():
    x, w, dy = _case(4, 30, seed=13)
    dy2 = _rng(14).standard_normal(dy.shape)
    a = O.rmsnorm_vjp(x, w, dy, 1e-5, 0.0)
    b = O.rmsnorm_vjp(x, w, dy2, 1e-5, 0.0)
    c = O.rmsnorm_vjp(x, w, dy + 2.0 * dy2, 1e-5, 0.0)
    for k in range(2):
        np.testing.assert_allclose(c[k], a[k] + 2.0 * b[k], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("k", [0, 1, 5, 11, 12])
def test_dw_additive_over_row_splits(k):
    # dw(X) = dw(X[:k]) + dw(X[k:]): the row sum that a cross-block combine
    # has to reproduce.
    x, w, dy = _case(12, 19, seed=15)
    _, dw = O.rmsnorm_vjp(x, w, dy, 1e-5, 0.0)
    _, dwa = O.rmsnorm_vjp(x[:k], w, dy[:k], 1e-5, 0.0)
    _, dwb = O.rmsnorm_vjp(x[k:], w, dy[k:], 1e-5, 0.0)
    np.testing.assert_allclose(dwa + dwb, dw, rtol=1e-13, atol=1e-14)


def test_dw_independent_of_weight():
    x, w, dy = _case(7, 23, seed=16)
    _, dw1 = O.rmsnorm_vjp(x, w, dy, 1e-5, 0.0)
    _, dw2 = O.rmsnorm_vjp(x, 5.0 * w - 1.0, dy, 1e-5, 1.0)
    np.testing.assert_array_equal(dw1, dw2)


def test_vjp_empty_rows():
    dx, dw = O.rmsnorm_vjp(np.zeros((0, 8)), np.ones(8), np.zeros((0, 8)), 1e-5, 0.0)
    assert dx.shape == (0, 8) and np.all(dw == 0)


def test_oracle_widening_is_exact():
    # fp16 / bf16 / fp32 storage values widen to fp64 without change.
    t = torch.tensor([1.0 + 2 ** -10, -3.140625, 6.1e-5, 65504.0], dtype=torch.float16)
    np.testing.assert_array_equal(O.widen(t), t.double().numpy())
    b = torch.tensor([1.0 + 2 ** -7, -3.140625, 1e-38, 3.3e38], dtype=torch.bfloat16)
    np.testing.assert_array_equal(O.widen(b), b.double().numpy())


# ------------------------------------------- fused backward (residual grad)

@pytest.mark.parametrize("rows,D", [(1, 1), (2, 3), (3, 8), (2, 17)])
@pytest.mark.parametrize("wb", [0.0, 1.0])
def test_fused_vjp_finite_differences(rows, D, wb):
    # L = sum(dy * normed(x + res)) + sum(dr * (x + res)); dL/dx = dL/dres = dh.
    r = _rng(20 + D)
    x = r.standard_normal((rows, D))
    res = r.standard_normal((rows, D))
    w = r.uniform(0.5, 1.5, D)
    dy = r.standard_normal((rows, D))
    dr = r.standard_normal((rows, D))
    eps = 2.0 ** -8

    def loss(xx, rr, ww):
        normed, h = O.fused_add_rmsnorm_fwd(xx, rr, ww, eps, wb)
        return float(np.sum(dy * normed) + np.sum(dr * h))

    dh, dw = O.fused_add_rmsnorm_vjp(x + res, w, dy, dr, eps, wb)
    hstep = 1e-6
    for i in range(rows):
        for j in range(D):
            for which in (0, 1):
                xp, xm, rp, rm = x.copy(), x.copy(), res.copy(), res.copy()
                if which == 0:
                    xp[i, j] += hstep
                    xm[i, j] -= hstep
                else:
                    rp[i, j] += hstep
                    rm[i, j] -= hstep
                fd = (loss(xp, rp, w) - loss(xm, rm, w)) / (2 * hstep)
                assert abs(fd - dh[i, j]) <= 1e-7 * max(1.0, abs(dh[i, j]))
    for j in range(D):
        wp, wm = w.copy(), w.copy()
        wp[j] += hstep
        wm[j] -= hstep
        fd = (loss(x, res, wp) - loss(x, res, wm)) / (2 * hstep)
        assert abs(fd - dw[j]) <= 1e-7 * max(1.0, abs(dw[j]))


def test_fused_vjp_zero_residual_grad_is_the_vjp():
    x, w, dy = _case(5, 33, seed=21)
    dh, dw = O.fused_add_rmsnorm_vjp(x, w, dy, np.zeros_like(x), 1e-5, 1.0)
    dx, dw2 = O.rmsnorm_vjp(x, w, dy, 1e-5, 1.0)
    np.testing.assert_array_equal(dh, dx)
    np.testing.assert_array_equal(dw, dw2)


# ---------------------------------------------------------- gated activation

def test_silu_gate_odd_part_identity():
    # silu(a) - silu(-a) = a, so y(a, b) - y(-a, b) = a * b exactly in the
    # mathematics (to rounding in fp64).
    r = _rng(30)
    a = r.standard_normal((7, 33)) * 4
    b = r.standard_normal((7, 33))
    y1 = O.silu_gate(np.concatenate([a, b], axis=1))
    y2 = O.silu_gate(np.concatenate([-a, b], axis=1))
    np.testing.assert_allclose(y1 - y2, a * b, rtol=1e-12, atol=1e-14)


def test_silu_gate_special_values_and_torch():
    a = np.array([[0.0, 1.0, -1.0, 30.0, -30.0, 800.0, -800.0]])
    b = np.ones_like(a)
    y = O.silu_gate(np.concatenate([a, b], axis=1))[0]
    assert y[0] == 0.0
    np.testing.assert_allclose(y[1], 1.0 / (1.0 + np.exp(-1.0)), rtol=1e-15)
    np.testing.assert_allclose(y[3], 30.0, rtol=1e-12)      # ~a for large a
    assert abs(y[4]) < 1e-11                                  # ~0 for very negative a
    assert y[5] == 800.0 and y[6] == 0.0
    # library cross-check: torch's silu in fp64
    r = _rng(31)
    x = r.standard_normal((5, 2 * 40)) * 3
    ref = (torch.nn.functional.silu(torch.tensor(x[:, :40])) * torch.tensor(x[:, 40:])).numpy()
    np.testing.assert_allclose(O.silu_gate(x), ref, rtol=1e-13, atol=1e-15)


def test_silu_gate_vjp_finite_differences():
    # central differences of L = sum(dy * y) with respect to every element of x
    r = _rng(32)
    rows, d = 3, 5
    x = r.standard_normal((rows, 2 * d)) * 3
    dy = r.standard_normal((rows, d))
    g = O.silu_gate_vjp(x, dy)
    h = 1e-6
    fd = np.empty_like(x)
    for i in range(rows):
        for j in range(2 * d):
            xp, xm = x.copy(), x.copy()
            xp[i, j] += h
            xm[i, j] -= h
            fd[i, j] = (np.sum(dy * O.silu_gate(xp)) - np.sum(dy * O.silu_gate(xm))) / (2 * h)
    np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8)


def test_silu_gate_vjp_torch_and_special_values():
    r = _rng(33)
    x = r.standard_normal((4, 2 * 24)) * 4
    dy = r.standard_normal((4, 24))
    xt = torch.tensor(x, requires_grad=True)
    y = torch.nn.functional.silu(xt[:, :24]) * xt[:, 24:]
    y.backward(torch.tensor(dy))
    np.testing.assert_allclose(O.silu_gate_vjp(x, dy), xt.grad.numpy(), rtol=1e-12, atol=1e-14)
    # a = 0: silu'(0) = 1/2 and silu(0) = 0
    x0 = np.array([[0.0, 0.0, 3.0, -5.0]])
    g0 = O.silu_gate_vjp(x0, np.array([[2.0, 1.0]]))[0]
    assert g0[0] == 3.0 and g0[1] == -2.5 and g0[2] == 0.0 and g0[3] == 0.0
