"""Pins for the per-operation oracle functions (CPU only, float64).

Each op is checked against something other than itself: closed forms,
invariants the pages state, torch library routines, finite differences and
brute force on tiny inputs.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import ops

R = np.random.default_rng(1234)


def fd_dir(f, x, d, h=1e-6):
    return (f(x + h * d) - f(x - h * d)) / (2 * h)


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_rms_closed_form():
    x = R.standard_normal((7, 96)) * 3.0
    eps = 1e-6
    y, r = ops.rmsnorm(x, eps)
    ms = np.mean(x * x, axis=-1)
    # rms(y) = sqrt(m/(m+eps)) with m = mean(x^2)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, -1)), np.sqrt(ms / (ms + eps)), rtol=1e-12)
    np.testing.assert_allclose(r, 1 / np.sqrt(ms + eps), rtol=1e-12)


def test_rmsnorm_scale_invariance_and_euler():
    x = R.standard_normal((5, 64))
    y1, _ = ops.rmsnorm(x, 0.0)
    y2, _ = ops.rmsnorm(3.7 * x, 0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-12, atol=1e-14)
    # degree-0 homogeneity at eps = 0 => x . dx = 0 for any upstream dy
    y, r = ops.rmsnorm(x, 0.0)
    dx = ops.rmsnorm_bwd(R.standard_normal(x.shape), y, r)
    assert np.max(np.abs(np.sum(x * dx, -1))) < 1e-12


def test_rmsnorm_matches_torch():
    x = R.standard_normal((9, 128))
    y, _ = ops.rmsnorm(x, 1e-6)
    yt = F.rms_norm(torch.from_numpy(x), (128,), eps=1e-6).numpy()
    np.testing.assert_allclose(y, yt, rtol=1e-12, atol=1e-14)


def test_rmsnorm_bwd_fd():
    x = R.standard_normal((4, 32))
    dy = R.standard_normal(x.shape)
    d = R.standard_normal(x.shape)
    y, r = ops.rmsnorm(x, 1e-6)
    an = np.sum(ops.rmsnorm_bwd(dy, y, r) * d)
    fd = fd_dir(lambda z: np.sum(ops.rmsnorm(z, 1e-6)[0] * dy), x, d)
    assert abs(an - fd) <= 1e-8 * max(1.0, abs(an))


# ---------------------------------------------------------------- RoPE
def test_rope_identity_at_zero_and_orthogonal():
    T, hd = 16, 32
    cos, sin = ops.rope_angles(T, hd, 10000.0)
    u = R.standard_normal((3, T, hd))
    v = ops.rope(u, cos, sin)
    np.testing.assert_allclose(v[:, 0], u[:, 0], rtol=0, atol=0)  # R_0 = I
    np.testing.assert_allclose(np.linalg.norm(v, axis=-1), np.linalg.norm(u, axis=-1), rtol=1e-13)
    np.testing.assert_allclose(ops.rope_bwd(v, cos, sin), u, rtol=1e-12, atol=1e-13)  # R^T R = I


def test_rope_relative_position_property():
    # "RoPE Intuition": q.k after rotation depends only on the distance m - n
    T, hd = 64, 32
    cos, sin = ops.rope_angles(T, hd, 10000.0)
    q = R.standard_normal(hd)
    k = R.standard_normal(hd)
    Q = ops.rope(np.broadcast_to(q, (T, hd)), cos, sin)
    K = ops.rope(np.broadcast_to(k, (T, hd)), cos, sin)
    for m, n, s in [(5, 2, 7), (10, 10, 30), (3, 9, 40), (0, 1, 50)]:
        assert abs(Q[m] @ K[n] - Q[m + s] @ K[n + s]) < 1e-12


def test_rope_layout_closed_form():
    # theta_0 = 1: unit vector e_0 at position t maps to cos(t) e_0 + sin(t) e_{hd/2};
    # the last pair turns by t * base^(-(hd-2)/hd).
    T, hd, base = 8, 16, 10000.0
    cos, sin = ops.rope_angles(T, hd, base)
    e0 = np.zeros((T, hd)); e0[:, 0] = 1.0
    v = ops.rope(e0, cos, sin)
    t = np.arange(T)
    np.testing.assert_allclose(v[:, 0], np.cos(t), atol=1e-15)
    np.testing.assert_allclose(v[:, hd // 2], np.sin(t), atol=1e-15)
    el = np.zeros((T, hd)); el[:, hd // 2 - 1] = 1.0
    w = ops.rope(el, cos, sin)
    ang = t * base ** (-(hd - 2) / hd)
    np.testing.assert_allclose(w[:, hd // 2 - 1], np.cos(ang), atol=1e-15)
    np.testing.assert_allclose(w[:, hd - 1], np.sin(ang), atol=1e-15)


def test_rope_matches_complex_rotation():
    # independent formulation: (a + i b) * exp(i t theta)
    T, hd = 12, 24
    cos, sin = ops.rope_angles(T, hd, 500.0)
    u = R.standard_normal((2, T, hd))
    c = torch.complex(torch.from_numpy(u[..., : hd // 2]), torch.from_numpy(u[..., hd // 2:]))
    theta = 500.0 ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    rot = torch.polar(torch.ones(T, hd // 2, dtype=torch.float64), torch.arange(T, dtype=torch.float64)[:, None] * theta)
    out = c * rot
    ref = torch.cat([out.real, out.imag], -1).numpy()
    np.testing.assert_allclose(ops.rope(u, cos, sin), ref, rtol=1e-12, atol=1e-13)


def test_qknorm_rope_bwd_fd():
    T, hd = 6, 16
    cos, sin = ops.rope_angles(T, hd, 10000.0)
    u = R.standard_normal((2, 3, T, hd))
    dv = R.standard_normal(u.shape)
    d = R.standard_normal(u.shape)
    v, r = ops.qknorm_rope(u, cos, sin, 1e-6)
    an = np.sum(ops.qknorm_rope_bwd(dv, v, r, cos, sin) * d)
    fd = fd_dir(lambda z: np.sum(ops.qknorm_rope(z, cos, sin, 1e-6)[0] * dv), u, d)
    assert abs(an - fd) <= 1e-8 * max(1.0, abs(an))


# ---------------------------------------------------------------- attention
def test_attention_single_position_returns_v():
    q = R.standard_normal((2, 3, 1, 8)); k = R.standard_normal(q.shape); v = R.standard_normal(q.shape)
    o, lse = ops.attention(q, k, v)
    np.testing.assert_allclose(o, v, rtol=1e-15, atol=0)
    np.testing.assert_allclose(lse[..., 0], np.sum(q * k, -1)[..., 0] / np.sqrt(8), rtol=1e-13)


def test_attention_identical_keys_prefix_mean():
    T, hd = 10, 8
    q = R.standard_normal((T, hd))
    k = np.broadcast_to(R.standard_normal(hd), (T, hd)).copy()
    v = R.standard_normal((T, hd))
    o, _ = ops.attention(q, k, v)
    ref = np.cumsum(v, 0) / np.arange(1, T + 1)[:, None]
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-14)


def test_attention_probs_rows_sum_to_one_and_causal():
    q = R.standard_normal((2, 16, 8)); k = R.standard_normal((2, 16, 8))
    p, _ = ops.attention_probs(q, k)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=1e-13)
    assert np.all(p[:, np.triu_indices(16, 1)[0], np.triu_indices(16, 1)[1]] == 0.0)


def test_attention_matches_torch_sdpa():
    q = R.standard_normal((2, 3, 20, 16)); k = R.standard_normal(q.shape); v = R.standard_normal(q.shape)
    o, _ = ops.attention(q, k, v)
    ot = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True).numpy()
    np.testing.assert_allclose(o, ot, rtol=1e-11, atol=1e-13)


def test_attention_bwd_fd():
    q = R.standard_normal((2, 9, 8)); k = R.standard_normal(q.shape); v = R.standard_normal(q.shape)
    do = R.standard_normal(q.shape)
    o, _ = ops.attention(q, k, v)
    dq, dk, dv = ops.attention_bwd(do, q, k, v, o)
    for which, an_g in ((0, dq), (1, dk), (2, dv)):
        d = R.standard_normal(q.shape)

        def f(z, which=which):
            args = [q, k, v]
            args[which] = z
            return np.sum(ops.attention(*args)[0] * do)

        an = np.sum(an_g * d)
        fd = fd_dir(f, [q, k, v][which], d)
        assert abs(an - fd) <= 1e-8 * max(1.0, abs(an)), which


# ---------------------------------------------------------------- ReLU^2
def test_relu2_values_and_bwd():
    u = np.array([-2.0, -0.0, 0.0, 0.5, 3.0])
    np.testing.assert_array_equal(ops.relu2(u), [0.0, 0.0, 0.0, 0.25, 9.0])
    np.testing.assert_array_equal(ops.relu2_bwd(np.ones(5), u), [0.0, 0.0, 0.0, 1.0, 6.0])


def test_relu2_half_zero_on_symmetric_input():
    # "ReLU² Sparsity": negatives map to exactly zero
    u = R.standard_normal(200000)
    frac = np.mean(ops.relu2(u) == 0.0)
    assert 0.49 < frac < 0.51


# ---------------------------------------------------------------- cross-entropy
@pytest.mark.parametrize("V", [512, 65536])
def test_ce_uniform_logits_is_ln_v(V):
    loss, _ = ops.cross_entropy(np.zeros((3, V)), np.array([0, 5, V - 1]))
    assert loss == pytest.approx(math.log(V), abs=1e-12)


def test_ce_matches_torch_and_rows_sum_zero():
    l = R.standard_normal((11, 37)) * 4
    y = R.integers(0, 37, 11)
    loss, lse = ops.cross_entropy(l, y)
    lt = F.cross_entropy(torch.from_numpy(l), torch.from_numpy(y)).item()
    assert loss == pytest.approx(lt, rel=1e-13)
    g = ops.cross_entropy_bwd(l, y, lse)
    np.testing.assert_allclose(g.sum(-1), 0.0, atol=1e-16)
    d = R.standard_normal(l.shape)
    an = np.sum(g * d)
    fd = fd_dir(lambda z: ops.cross_entropy(z, y)[0], l, d)
    assert abs(an - fd) <= 1e-8 * max(1.0, abs(an))


# ---------------------------------------------------------------- embedding
def test_embedding_bwd_brute_force_and_conservation():
    V, d, N = 13, 5, 40
    tok = R.integers(0, V - 3, N)  # the top 3 ids never occur
    dx = R.standard_normal((N, d))
    dE = ops.embedding_bwd(dx, tok, V)
    brute = np.zeros((V, d))
    for n in range(N):
        brute[tok[n]] += dx[n]
    np.testing.assert_allclose(dE, brute, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dE.sum(0), dx.sum(0), rtol=1e-12)
    assert np.all(dE[V - 3:] == 0.0)


# ---------------------------------------------------------------- input rounding
def test_bf16_round_is_rne():
    import synth
    # halfway cases go to the even neighbour
    assert synth.bf16_round(np.float32([1.0 + 2 ** -8]))[0] == 1.0
    assert synth.bf16_round(np.float32([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6
    assert synth.bf16_round(np.float32([1.0 + 2 ** -8 + 2 ** -20]))[0] == 1.0 + 2 ** -7
    x = R.standard_normal(100000).astype(np.float32) * 7
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(synth.bf16_round(x), ref)


# ---------------------------------------------------------------- masked cross-entropy
def test_ce_masked_matches_torch_ignore_index_and_fd():
    l = R.standard_normal((13, 29)) * 3
    y = R.integers(0, 29, 13)
    y[[0, 4, 5, 11]] = -1
    loss, lse = ops.cross_entropy(l, y)
    lt = F.cross_entropy(torch.from_numpy(l), torch.from_numpy(y), ignore_index=-1).item()
    assert loss == pytest.approx(lt, rel=1e-13)
    g = ops.cross_entropy_bwd(l, y, lse)
    assert np.all(g[y < 0] == 0.0)
    np.testing.assert_allclose(g.sum(-1), 0.0, atol=1e-16)
    d = R.standard_normal(l.shape)
    fd = fd_dir(lambda z: ops.cross_entropy(z, y)[0], l, d)
    assert abs(np.sum(g * d) - fd) <= 1e-8 * max(1.0, abs(fd))
    # the masked loss is the unmasked loss of the kept rows alone
    keep = y >= 0
    assert loss == pytest.approx(ops.cross_entropy(l[keep], y[keep])[0], rel=1e-14)


def test_ce_all_masked_is_zero():
    l = R.standard_normal((4, 9))
    y = np.full(4, -1)
    loss, lse = ops.cross_entropy(l, y)
    assert loss == 0.0
    assert np.all(ops.cross_entropy_bwd(l, y, lse) == 0.0)
