"""Pins for the optimizer-step oracle (CPU only, float64).

Each function is checked against something other than itself: closed forms
of the schedule, of the clipped norm and of AdamW under a constant gradient,
and the Newton-Schulz iteration against the scalar quintic applied to the
singular values of a matrix assembled from random orthogonal factors.
"""

import math

import numpy as np
import pytest

from oracle import optim

R = np.random.default_rng(4321)
A_, B_, C_ = optim.NS_COEFFS


# ---------------------------------------------------------------- schedule
def test_cosine_lr_closed_form_points():
    peak, warm, total, f = 0.02, 10, 110, 0.1
    assert optim.cosine_lr(0, peak, warm, total, f) == pytest.approx(peak / warm, rel=1e-15)
    assert optim.cosine_lr(warm - 1, peak, warm, total, f) == pytest.approx(peak, rel=1e-15)
    assert optim.cosine_lr(warm, peak, warm, total, f) == pytest.approx(peak, rel=1e-15)
    # halfway through the decay cos(pi/2) = 0: the mean of peak and the floor
    assert optim.cosine_lr(warm + 50, peak, warm, total, f) == pytest.approx(peak * (f + (1 - f) / 2), rel=1e-12)
    # the end of the decay (and beyond) sits on the floor
    assert optim.cosine_lr(total, peak, warm, total, f) == pytest.approx(peak * f, rel=1e-12)
    assert optim.cosine_lr(total + 7, peak, warm, total, f) == pytest.approx(peak * f, rel=1e-12)


def test_cosine_lr_monotone_after_warmup():
    lrs = [optim.cosine_lr(s, 1.0, 5, 60, 0.0) for s in range(0, 70)]
    assert all(lrs[i] <= lrs[i + 1] for i in range(4))
    assert all(lrs[i] >= lrs[i + 1] - 1e-15 for i in range(5, 69))


# ---------------------------------------------------------------- clipping
def test_clip_scale_closed_form():
    # constant-valued tensors: the global norm is |c| sqrt(n1 + n2) exactly
    g = [np.full((3, 4), -2.5), np.full(20, -2.5)]
    norm, s = optim.clip_scale(g, 1.0)
    assert norm == pytest.approx(2.5 * math.sqrt(32), rel=1e-14)
    assert s == pytest.approx(1.0 / (norm + 1e-6), rel=1e-14)
    # clipped gradients have norm ~ clip; small ones are left alone
    assert norm * s == pytest.approx(1.0, rel=1e-6)
    _, s_small = optim.clip_scale([np.full(4, 0.01)], 1.0)
    assert s_small == 1.0


# ---------------------------------------------------------------- AdamW
def test_adamw_first_step_closed_form():
    th = R.standard_normal(50)
    g = R.standard_normal(50)
    lr, b1, b2, eps, wd = 1e-3, 0.9, 0.95, 1e-8, 0.1
    th1, m, v = optim.adamw_update(th, g, np.zeros(50), np.zeros(50), 1, lr, b1, b2, eps, wd)
    # bias correction makes m_hat = g and v_hat = g^2 after one step
    np.testing.assert_allclose(th1, th - lr * (g / (np.abs(g) + eps) + wd * th), rtol=1e-13)
    np.testing.assert_allclose(m, (1 - b1) * g, rtol=1e-15)
    np.testing.assert_allclose(v, (1 - b2) * g * g, rtol=1e-15)


def test_adamw_constant_gradient_steps():
    th0 = R.standard_normal(30)
    g = R.standard_normal(30)
    lr, b1, b2, eps = 2e-3, 0.9, 0.999, 1e-8
    th, m, v = th0.copy(), np.zeros(30), np.zeros(30)
    for t in range(1, 6):
        th, m, v = optim.adamw_update(th, g, m, v, t, lr, b1, b2, eps, 0.0)
    # m = (1 - b1^t) g and v = (1 - b2^t) g^2: every step moves by lr g / (|g| + eps)
    np.testing.assert_allclose(th, th0 - 5 * lr * g / (np.abs(g) + eps), rtol=1e-12)


# ---------------------------------------------------------------- Newton-Schulz
def _orthogonal(n):
    q, r = np.linalg.qr(R.standard_normal((n, n)))
    return q * np.sign(np.diag(r))


def _phi(x, steps):
    for _ in range(steps):
        x = A_ * x + B_ * x ** 3 + C_ * x ** 5
    return x


def _ns_by_svd(P, s, Q, steps):
    """NS of P diag(s) Q^T (P [m,k], Q [n,k] orthonormal columns) from the
    scalar map of its singular values."""
    sn = s / (np.linalg.norm(s) + 1e-7)
    return (P * _phi(sn, steps)) @ Q.T


@pytest.mark.parametrize("m,n", [(12, 12), (8, 20), (24, 9)])
def test_newton_schulz_matches_singular_value_map(m, n):
    k = min(m, n)
    P, Q = _orthogonal(m)[:, :k], _orthogonal(n)[:, :k]
    s = np.exp(R.uniform(-1.0, 0.5, k))
    U = (P * s) @ Q.T
    for steps in (1, 5):
        np.testing.assert_allclose(optim.newton_schulz5(U, steps), _ns_by_svd(P, s, Q, steps), rtol=1e-9,
                                   atol=1e-12)


def test_newton_schulz_transpose_and_scale():
    U = R.standard_normal((10, 16))
    np.testing.assert_allclose(optim.newton_schulz5(U.T), optim.newton_schulz5(U).T, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(optim.newton_schulz5(7.0 * U), optim.newton_schulz5(U), rtol=1e-6, atol=1e-9)


def test_newton_schulz_scalar_polynomial_value():
    # a 1x1 input normalises to x0 = 3 / (3 + 1e-7) ~ 1; one step gives the
    # quintic at x0, close to a + b + c = 0.701
    x0 = 3.0 / (3.0 + 1e-7)
    y = optim.newton_schulz5(np.array([[3.0]]), 1)[0, 0]
    assert y == pytest.approx(A_ * x0 + B_ * x0 ** 3 + C_ * x0 ** 5, rel=1e-13)
    assert y == pytest.approx(0.701, abs=1e-6)


# ---------------------------------------------------------------- Muon
def test_muon_first_and_second_step_closed_form():
    m, n = 16, 6
    k = min(m, n)
    P, Q = _orthogonal(m)[:, :k], _orthogonal(n)[:, :k]
    s = np.exp(R.uniform(-0.5, 0.5, k))
    G = (P * s) @ Q.T
    W = R.standard_normal((m, n))
    lr, mu, wd = 0.02, 0.95, 0.1
    # step 1 from a zero buffer: U = (1 + mu) G, singular values (1 + mu) s
    O1 = _ns_by_svd(P, (1 + mu) * s, Q, 5)
    W1, b1 = optim.muon_update(W, G, np.zeros((m, n)), lr, mu, wd)
    np.testing.assert_allclose(b1, G, rtol=1e-15)
    np.testing.assert_allclose(W1, W - lr * (math.sqrt(m / n) * O1 + wd * W), rtol=1e-9, atol=1e-12)
    # step 2 with the same gradient: U = (1 + mu + mu^2) G, the same direction
    O2 = _ns_by_svd(P, (1 + mu + mu * mu) * s, Q, 5)
    W2, b2 = optim.muon_update(W1, G, b1, lr, mu, wd)
    np.testing.assert_allclose(b2, (1 + mu) * G, rtol=1e-14)
    np.testing.assert_allclose(W2, W1 - lr * (math.sqrt(m / n) * O2 + wd * W1), rtol=1e-9, atol=1e-12)
    # the update is orthogonal-like: its singular values sit near 1
    sv = np.linalg.svd(O1, compute_uv=False)
    assert sv.min() > 0.6 and sv.max() < 1.25


# ---------------------------------------------------------------- full step
def _tiny():
    shapes = {"E": (40, 8), "layers.0.W_qkv": (24, 8), "layers.0.W_o": (8, 8), "layers.0.W_1": (32, 8),
              "layers.0.W_2": (8, 32), "W_lm": (40, 8)}
    master = {k: R.standard_normal(v) * 0.02 for k, v in shapes.items()}
    grads = {k: R.standard_normal(v) for k, v in shapes.items()}
    hp = dict(lr_adamw=3e-3, lr_muon=0.02, warmup=4, total=40, final_frac=0.1, clip=1.0, wd=0.1, beta1=0.9,
              beta2=0.95, eps=1e-8, momentum=0.95, ns_steps=5)
    return master, grads, hp


def test_optimizer_step_groups_and_clipping():
    master, grads, hp = _tiny()
    st0 = {"m": {}, "v": {}, "buf": {}}
    new, st, norm, mult = optim.optimizer_step(master, grads, st0, hp, 0)
    assert mult == pytest.approx(1 / 4)
    assert set(st["m"]) == {"E", "W_lm"} and set(st["buf"]) == {k for k in master if k.startswith("layers.")}
    # the gradients are far above the clip: scaling them by 10 changes nothing
    g10 = {k: 10.0 * v for k, v in grads.items()}
    new10, _, norm10, _ = optim.optimizer_step(master, g10, st0, hp, 0)
    assert norm10 == pytest.approx(10 * norm, rel=1e-13)
    for k in master:
        np.testing.assert_allclose(new10[k], new[k], rtol=1e-6, atol=1e-12)
    # the AdamW tensors follow the first-step closed form with the clipped gradient
    s = 1.0 / (norm + 1e-6)
    lr = hp["lr_adamw"] * mult
    for k in ("E", "W_lm"):
        g = grads[k] * s
        np.testing.assert_allclose(new[k], master[k] - lr * (g / (np.abs(g) + hp["eps"]) + hp["wd"] * master[k]),
                                   rtol=1e-12)
