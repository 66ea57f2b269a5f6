"""Pins for the whole-model oracle (CPU only, float64).

* central finite differences along random directions of every tensor;
* an independent torch float64 autograd model built from library routines
  (rms_norm, scaled_dot_product_attention, cross_entropy, complex rotation);
* causality, uniform logits, batch linearity, init-loss and ReLU² sparsity
  invariants;
* the page-stated depth dial and parameter count (tests/golden/depth_dial.txt).
"""

import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import ops
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

TINY = oracle.derive_config(2, vocab=512, seq_len=64, d_model=128, n_heads=2, head_dim=64, d_ff=512)
MICRO = oracle.derive_config(2, vocab=40, seq_len=8, d_model=32, n_heads=2, head_dim=16, d_ff=64)


def make(cfg, B, seed=0, std=0.02):
    p = synth.weights(oracle.param_shapes(cfg), seed=seed, std=std)
    tok, tgt = synth.uniform_tokens(B, cfg.seq_len, cfg.vocab, seed=seed)
    return {k: v.astype(np.float64) for k, v in p.items()}, tok, tgt


# ---------------------------------------------------------------- golden: depth dial
def read_golden(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            out[k] = float(v)
    return out


def test_depth_dial_and_param_count():
    g = read_golden("depth_dial.txt")
    for depth in (20, 26):
        c = oracle.derive_config(depth, vocab=int(g["vocab"]))
        assert c.d_model == depth * g["rule_d_model_per_depth"]
        assert c.head_dim == g["rule_head_dim"]
        assert c.n_heads * c.head_dim == c.d_model
        assert c.d_ff == g["rule_ffn_mult"] * c.d_model
    c20 = oracle.derive_config(20)
    assert (c20.d_model, c20.n_heads, c20.d_ff) == (1280, 10, 5120)
    n = oracle.param_count(c20)
    assert n == 560_988_160
    assert abs(n / (g["approx_params_millions"] * 1e6) - 1) < g["approx_params_rel_tol"]
    assert 2 ** 16 == g["vocab"]


# ---------------------------------------------------------------- finite differences
@pytest.mark.parametrize("cfg,B", [(MICRO, 2), (TINY, 2)])
def test_grads_central_finite_differences(cfg, B):
    # larger weights than init so every path carries signal
    params, tok, tgt = make(cfg, B, seed=3, std=0.2)
    loss, grads = oracle.forward_backward(cfg, params, tok, tgt)
    rng = np.random.default_rng(7)
    h = 1e-5
    for name, _ in oracle.param_shapes(cfg):
        d = rng.standard_normal(params[name].shape)
        if name == "E":  # only rows that occur carry gradient
            d *= np.isin(np.arange(cfg.vocab), tok)[:, None]
        d /= np.linalg.norm(d)
        pp = dict(params); pm = dict(params)
        pp[name] = params[name] + h * d
        pm[name] = params[name] - h * d
        fd = (oracle.forward(cfg, pp, tok, tgt) - oracle.forward(cfg, pm, tok, tgt)) / (2 * h)
        an = float(np.sum(grads[name] * d))
        assert abs(fd - an) <= 1e-6 * max(abs(an), 1e-3), (name, fd, an)


# ---------------------------------------------------------------- torch float64 autograd
def torch_model_loss(cfg, P, tok, tgt, ignore_index=-100):
    """The same model written with torch library routines; autograd gives grads."""
    B, T = tok.shape
    H, hd = cfg.n_heads, cfg.head_dim
    d = cfg.d_model
    x = F.embedding(tok, P["E"])
    theta = cfg.rope_base ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    rot = torch.polar(torch.ones(T, hd // 2, dtype=torch.float64),
                      torch.arange(T, dtype=torch.float64)[:, None] * theta)

    def rotate(u):  # u [B, H, T, hd], split-half pairs as a complex number
        c = torch.complex(u[..., : hd // 2], u[..., hd // 2:]) * rot
        return torch.cat([c.real, c.imag], -1)

    Hk = cfg.kv_heads
    for l in range(cfg.depth):
        a = F.rms_norm(x, (d,), eps=cfg.eps)
        qkv = F.linear(a, P[f"layers.{l}.W_qkv"])
        q, k, v = torch.split(qkv, [H * hd, Hk * hd, Hk * hd], dim=-1)
        q = q.view(B, T, H, hd).transpose(1, 2)
        k = k.view(B, T, Hk, hd).transpose(1, 2)
        v = v.view(B, T, Hk, hd).transpose(1, 2)
        q = rotate(F.rms_norm(q, (hd,), eps=cfg.eps))
        k = rotate(F.rms_norm(k, (hd,), eps=cfg.eps))
        o = F.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=Hk != H)
        x = x + F.linear(o.transpose(1, 2).reshape(B, T, H * hd), P[f"layers.{l}.W_o"])
        m = F.rms_norm(x, (d,), eps=cfg.eps)
        x = x + F.linear(F.relu(F.linear(m, P[f"layers.{l}.W_1"])).square(), P[f"layers.{l}.W_2"])
    logits = F.linear(F.rms_norm(x, (d,), eps=cfg.eps), P["W_lm"])
    return F.cross_entropy(logits.reshape(-1, cfg.vocab), tgt.reshape(-1), ignore_index=ignore_index)


def test_matches_torch_float64_autograd_tiny():
    params, tok, tgt = make(TINY, 2, seed=0)
    loss, grads = oracle.forward_backward(TINY, params, tok, tgt)
    P = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in params.items()}
    lt = torch_model_loss(TINY, P, torch.from_numpy(tok).long(), torch.from_numpy(tgt).long())
    lt.backward()
    assert abs(loss - lt.item()) <= 1e-12 * abs(loss)
    for k, v in grads.items():
        ref = P[k].grad.numpy()
        err = np.linalg.norm(v - ref) / np.linalg.norm(ref)
        assert err <= 1e-10, (k, err)


# ---------------------------------------------------------------- invariants
def test_causality_bitwise():
    params, tok, tgt = make(TINY, 1, seed=1)
    t0 = 30
    l1 = oracle.forward_logits(TINY, params, tok)
    tok2 = tok.copy()
    tok2[:, t0 + 1:] = (tok2[:, t0 + 1:] + 17) % TINY.vocab
    l2 = oracle.forward_logits(TINY, params, tok2)
    assert np.array_equal(l1[:, : t0 + 1], l2[:, : t0 + 1])
    assert not np.array_equal(l1[:, t0 + 1:], l2[:, t0 + 1:])


def test_uniform_logits_loss_is_ln_v():
    params, tok, tgt = make(TINY, 2, seed=2)
    params["W_lm"] = np.zeros_like(params["W_lm"])
    assert oracle.forward(TINY, params, tok, tgt) == pytest.approx(math.log(512), abs=1e-12)
    assert math.log(512) == pytest.approx(6.238324625039508, abs=1e-15)


def test_batch_linearity():
    params, tok, tgt = make(TINY, 2, seed=4)
    loss, grads = oracle.forward_backward(TINY, params, tok, tgt)
    l0, g0 = oracle.forward_backward(TINY, params, tok[:1], tgt[:1])
    l1, g1 = oracle.forward_backward(TINY, params, tok[1:], tgt[1:])
    assert loss == pytest.approx((l0 + l1) / 2, rel=1e-13)
    for k in grads:
        np.testing.assert_allclose(grads[k], (g0[k] + g1[k]) / 2, rtol=1e-9, atol=1e-15)


def test_init_loss_and_relu2_sparsity():
    params, tok, tgt = make(TINY, 2, seed=5)
    loss = oracle.forward(TINY, params, tok, tgt)
    sigma2 = 0.02 ** 2 * TINY.d_model  # logit variance with an rms-1 input
    assert abs(loss - (math.log(TINY.vocab) + sigma2 / 2)) < 0.05
    # g = relu2(u) is exactly zero for about half of the pre-activations
    x = ops.embedding(params["E"], tok)
    m, _ = ops.rmsnorm(x, TINY.eps)
    g = ops.relu2(m @ params["layers.0.W_1"].T)
    assert 0.45 < np.mean(g == 0.0) < 0.55


def test_embedding_grad_conservation_full_model():
    params, tok, tgt = make(TINY, 2, seed=6)
    _, grads = oracle.forward_backward(TINY, params, tok, tgt)
    absent = np.setdiff1d(np.arange(TINY.vocab), tok)
    assert absent.size > 0 and np.all(grads["E"][absent] == 0.0)


# ---------------------------------------------------------------- loss mask
def masked_targets(tgt, seed, frac=0.5):
    rng = np.random.default_rng(seed)
    t = tgt.copy()
    t[rng.random(t.shape) < frac] = -1
    return t


def test_masked_matches_torch_float64_autograd_and_fd():
    params, tok, tgt = make(TINY, 2, seed=6)
    tgt = masked_targets(tgt, 6)
    tgt[1, :] = -1  # a whole sequence outside the loss
    loss, grads = oracle.forward_backward(TINY, params, tok, tgt)
    P2 = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in params.items()}
    lt = torch_model_loss(TINY, P2, torch.from_numpy(tok).long(), torch.from_numpy(tgt).long(), ignore_index=-1)
    lt.backward()
    assert abs(loss - lt.item()) <= 1e-12 * abs(loss)
    for k, v in grads.items():
        ref = P2[k].grad.numpy()
        err = np.linalg.norm(v - ref) / max(np.linalg.norm(ref), 1e-300)
        assert err <= 1e-10, (k, err)
    # finite differences of the masked loss along one direction per tensor
    p2, tok2, tgt2 = make(MICRO, 2, seed=8, std=0.2)
    tgt2 = masked_targets(tgt2, 8)
    l2, g2 = oracle.forward_backward(MICRO, p2, tok2, tgt2)
    rng = np.random.default_rng(9)
    h = 1e-5
    for name, _ in oracle.param_shapes(MICRO):
        d = rng.standard_normal(p2[name].shape)
        d /= np.linalg.norm(d)
        pp = dict(p2); pm = dict(p2)
        pp[name] = p2[name] + h * d
        pm[name] = p2[name] - h * d
        fd = (oracle.forward(MICRO, pp, tok2, tgt2) - oracle.forward(MICRO, pm, tok2, tgt2)) / (2 * h)
        an = float(np.sum(g2[name] * d))
        assert abs(fd - an) <= 1e-6 * max(abs(an), 1e-3), (name, fd, an)


def test_mask_is_token_weighted_union_of_single_positions():
    # loss(S) |S| = sum over t in S of loss({t}); the same for every gradient
    params, tok, tgt = make(MICRO, 2, seed=10, std=0.2)
    S = [(0, 1), (0, 6), (1, 0), (1, 7)]
    ts = np.full_like(tgt, -1)
    for b, t in S:
        ts[b, t] = tgt[b, t]
    loss, grads = oracle.forward_backward(MICRO, params, tok, ts)
    acc_l, acc_g = 0.0, {k: 0.0 for k in grads}
    for b, t in S:
        t1 = np.full_like(tgt, -1)
        t1[b, t] = tgt[b, t]
        l1, g1 = oracle.forward_backward(MICRO, params, tok, t1)
        acc_l += l1
        for k in grads:
            acc_g[k] = acc_g[k] + g1[k]
    assert loss * len(S) == pytest.approx(acc_l, rel=1e-12)
    for k in grads:
        np.testing.assert_allclose(grads[k] * len(S), acc_g[k], rtol=1e-9, atol=1e-14)


def test_masked_batch_is_weighted_mean_of_microbatches_and_empty_mask():
    # gradient accumulation: the loss of a batch = token-weighted mean of its microbatches
    params, tok, tgt = make(TINY, 3, seed=11)
    tgt = masked_targets(tgt, 11, frac=0.3)
    loss, grads = oracle.forward_backward(TINY, params, tok, tgt)
    parts = [oracle.forward_backward(TINY, params, tok[i:i + 1], tgt[i:i + 1]) for i in range(3)]
    n = [(tgt[i] >= 0).sum() for i in range(3)]
    assert loss == pytest.approx(sum(p[0] * k for p, k in zip(parts, n)) / sum(n), rel=1e-12)
    for key in grads:
        np.testing.assert_allclose(grads[key], sum(p[1][key] * k for p, k in zip(parts, n)) / sum(n),
                                   rtol=1e-9, atol=1e-15)
    # nothing counted: loss 0 and every gradient 0
    l0, g0 = oracle.forward_backward(TINY, params, tok, np.full_like(tgt, -1))
    assert l0 == 0.0 and all(np.all(v == 0.0) for v in g0.values())



# ---------------------------------------------------------------- grouped-query attention
GQA = oracle.derive_config(2, vocab=512, seq_len=64, d_model=256, n_heads=4, head_dim=64, d_ff=512, n_kv_heads=2)
MQA_MICRO = oracle.derive_config(2, vocab=40, seq_len=8, d_model=64, n_heads=4, head_dim=16, d_ff=64, n_kv_heads=1)


def test_gqa_matches_torch_sdpa_enable_gqa_autograd():
    params, tok, tgt = make(GQA, 2, seed=12)
    assert params["layers.0.W_qkv"].shape == ((4 + 2 * 2) * 64, 256)
    loss, grads = oracle.forward_backward(GQA, params, tok, tgt)
    P = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in params.items()}
    lt = torch_model_loss(GQA, P, torch.from_numpy(tok).long(), torch.from_numpy(tgt).long())
    lt.backward()
    assert abs(loss - lt.item()) <= 1e-12 * abs(loss)
    for k, v in grads.items():
        ref = P[k].grad.numpy()
        assert np.linalg.norm(v - ref) <= 1e-10 * np.linalg.norm(ref), k


def test_mqa_finite_differences():
    params, tok, tgt = make(MQA_MICRO, 2, seed=13, std=0.2)
    loss, grads = oracle.forward_backward(MQA_MICRO, params, tok, tgt)
    rng = np.random.default_rng(14)
    h = 1e-5
    for name, _ in oracle.param_shapes(MQA_MICRO):
        d = rng.standard_normal(params[name].shape)
        if name == "E":
            d *= np.isin(np.arange(MQA_MICRO.vocab), tok)[:, None]
        d /= np.linalg.norm(d)
        pp = dict(params); pm = dict(params)
        pp[name] = params[name] + h * d
        pm[name] = params[name] - h * d
        fd = (oracle.forward(MQA_MICRO, pp, tok, tgt) - oracle.forward(MQA_MICRO, pm, tok, tgt)) / (2 * h)
        an = float(np.sum(grads[name] * d))
        assert abs(fd - an) <= 1e-6 * max(abs(an), 1e-3), (name, fd, an)


def test_gqa_equals_mha_with_repeated_kv_heads():
    # a GQA model is the MHA model whose key/value heads are copies within each
    # group; its key/value weight gradients are the sums over the copies
    params, tok, tgt = make(GQA, 2, seed=15)
    H, Hk, hd = GQA.n_heads, GQA.kv_heads, GQA.head_dim
    G = H // Hk
    mha = oracle.derive_config(2, vocab=512, seq_len=64, d_model=256, n_heads=4, head_dim=64, d_ff=512)
    pm = dict(params)
    for l in range(GQA.depth):
        W = params[f"layers.{l}.W_qkv"]
        q, k, v = W[:H * hd], W[H * hd:(H + Hk) * hd], W[(H + Hk) * hd:]
        rep = lambda m: np.repeat(m.reshape(Hk, hd, -1), G, axis=0).reshape(H * hd, -1)  # noqa: E731
        pm[f"layers.{l}.W_qkv"] = np.concatenate([q, rep(k), rep(v)])
    lg, gg = oracle.forward_backward(GQA, params, tok, tgt)
    lm, gm = oracle.forward_backward(mha, pm, tok, tgt)
    assert lg == pytest.approx(lm, rel=1e-13)
    for l in range(GQA.depth):
        a, b = gg[f"layers.{l}.W_qkv"], gm[f"layers.{l}.W_qkv"]
        fold = lambda m: m.reshape(Hk, G, hd, -1).sum(axis=1).reshape(Hk * hd, -1)  # noqa: E731
        np.testing.assert_allclose(a[:H * hd], b[:H * hd], rtol=1e-10, atol=1e-16)
        np.testing.assert_allclose(a[H * hd:(H + Hk) * hd], fold(b[H * hd:2 * H * hd]), rtol=1e-10, atol=1e-16)
        np.testing.assert_allclose(a[(H + Hk) * hd:], fold(b[2 * H * hd:]), rtol=1e-10, atol=1e-16)
