"""Float64 oracle model: forward, hand-derived backward, and logits.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Model ("nanochat explainer", Modern architecture choices; The 'One Dial'
Design; Pretraining), per sequence b with positions t = 0..T-1:

    x = E[tok]
    for each layer:
        a = rho(x)
        q, k, v = a W_q^T, a W_k^T, a W_v^T            (H query heads of hd; Hk
                                                         key/value heads, Hk divides H)
        qh = R_t rho_hd(q); kh = R_t rho_hd(k)           (QK-norm, RoPE)
        o  = causal softmax(qh kh^T / sqrt(hd)) v        (query head h with kv head h // (H/Hk))
        x += concat_h(o) W_o^T
        m = rho(x); u = m W_1^T; g = max(u, 0)^2; x += g W_2^T
    z = rho(x); l = z W_lm^T
    loss = mean_n [logsumexp(l_n) - l_{n, y_n}]   over the positions with y_n >= 0

A negative target leaves its position out of the loss (the loss mask of
supervised fine-tuning, "nanochat explainer", Supervised Fine-Tuning); with
every target >= 0 the mean runs over all B*T positions, as in pretraining.

Parameters are a dict of float64 arrays named as in ``param_shapes``; every
weight is [out, in].  W_qkv stacks the q rows, then the k rows, then the v
rows; within each, head h owns rows h*hd .. h*hd + hd - 1.
"""

from dataclasses import dataclass

import numpy as np

from . import ops

F64 = np.float64


@dataclass(frozen=True)
class Config:
    depth: int
    d_model: int
    n_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    seq_len: int
    eps: float = 1e-6
    rope_base: float = 10000.0
    n_kv_heads: int = 0  # key/value heads; 0 means n_heads (multi-head attention)

    @property
    def kv_heads(self):
        return self.n_kv_heads or self.n_heads


def derive_config(depth, vocab=65536, seq_len=2048, d_model=0, n_heads=0,
                  head_dim=0, d_ff=0, eps=1e-6, rope_base=10000.0, n_kv_heads=0):
    """Apply the depth dial ("nanochat explainer", How dimensions are derived).

    d_model = 64*depth, head_dim = 128, n_heads = d_model/128, d_ff = 4*d_model.
    A nonzero override replaces the derived value (the tiny test model uses
    2 heads of 64).  n_kv_heads < n_heads gives grouped-query attention
    ("nanochat explainer", Inference & KV Cache: several query heads share one
    key/value head; one shared head is multi-query attention).  Pinned by the
    page-printed depth-20 figures in tests/golden/depth_dial.txt.
    """
    d = d_model or 64 * depth
    hd = head_dim or 128
    h = n_heads or d // hd
    f = d_ff or 4 * d
    if n_kv_heads and h % n_kv_heads:
        raise ValueError(f"{h} heads do not split into groups of {n_kv_heads} key/value heads")
    return Config(depth, d, h, hd, f, vocab, seq_len, eps, rope_base, n_kv_heads)


def param_shapes(cfg):
    """Ordered (name, shape) list: E, then per layer W_qkv, W_o, W_1, W_2, then W_lm.

    W_qkv stacks the n_heads query heads, then the kv_heads key heads, then the
    kv_heads value heads."""
    d, hh, f, V = cfg.d_model, cfg.n_heads * cfg.head_dim, cfg.d_ff, cfg.vocab
    hk = cfg.kv_heads * cfg.head_dim
    out = [("E", (V, d))]
    for l in range(cfg.depth):
        out += [
            (f"layers.{l}.W_qkv", (hh + 2 * hk, d)),
            (f"layers.{l}.W_o", (d, hh)),
            (f"layers.{l}.W_1", (f, d)),
            (f"layers.{l}.W_2", (d, f)),
        ]
    out.append(("W_lm", (V, d)))
    return out


def param_count(cfg):
    return int(sum(np.prod(s) for _, s in param_shapes(cfg)))


def _heads(t, B, T, H, hd):
    """[B, T, H*hd] -> [B, H, T, hd]."""
    return t.reshape(B, T, H, hd).transpose(0, 2, 1, 3)


def _unheads(t):
    """[B, H, T, hd] -> [B, T, H*hd]."""
    B, H, T, hd = t.shape
    return t.transpose(0, 2, 1, 3).reshape(B, T, H * hd)


def _wgrad(dY, X):
    """dW = dY^T X summed over all positions (for Y = X W^T)."""
    return dY.reshape(-1, dY.shape[-1]).T @ X.reshape(-1, X.shape[-1])


def _forward(cfg, params, tokens, keep):
    p = {k: np.asarray(v, dtype=F64) for k, v in params.items()}
    tokens = np.asarray(tokens)
    B, T = tokens.shape
    H, Hk, hd, eps = cfg.n_heads, cfg.kv_heads, cfg.head_dim, cfg.eps
    hh, hk = H * hd, Hk * hd
    G = H // Hk  # query heads per key/value head
    cos, sin = ops.rope_angles(T, hd, cfg.rope_base)
    x = ops.embedding(p["E"], tokens)  # [B, T, d]
    caches = []
    for l in range(cfg.depth):
        Wqkv = p[f"layers.{l}.W_qkv"]
        a, r1 = ops.rmsnorm(x, eps)
        q = _heads(a @ Wqkv[:hh].T, B, T, H, hd)
        k = _heads(a @ Wqkv[hh:hh + hk].T, B, T, Hk, hd)
        v = _heads(a @ Wqkv[hh + hk:].T, B, T, Hk, hd)
        qh, rq = ops.qknorm_rope(q, cos, sin, eps)
        kh, rk = ops.qknorm_rope(k, cos, sin, eps)
        # query head h attends with key/value head h // G
        o, lse = ops.attention(qh, np.repeat(kh, G, axis=1), np.repeat(v, G, axis=1))
        O = _unheads(o)
        x = x + O @ p[f"layers.{l}.W_o"].T
        m, r2 = ops.rmsnorm(x, eps)
        u = m @ p[f"layers.{l}.W_1"].T
        g = ops.relu2(u)
        x = x + g @ p[f"layers.{l}.W_2"].T
        if keep:
            caches.append(dict(a=a, r1=r1, qh=qh, kh=kh, v=v, rq=rq, rk=rk,
                               o=o, O=O, m=m, r2=r2, u=u, g=g))
    z, rf = ops.rmsnorm(x, eps)
    logits = z @ p["W_lm"].T  # [B, T, V]
    return p, logits, dict(layers=caches, z=z, rf=rf, cos=cos, sin=sin)


def forward_logits(cfg, params, tokens):
    """Logits [B, T, V] in float64."""
    _, logits, _ = _forward(cfg, params, tokens, keep=False)
    return logits


def forward(cfg, params, tokens, targets):
    """Mean next-token cross-entropy over the positions with a target >= 0 (nats)."""
    _, logits, _ = _forward(cfg, params, tokens, keep=False)
    V = logits.shape[-1]
    loss, _ = ops.cross_entropy(logits.reshape(-1, V), np.asarray(targets).reshape(-1))
    return loss


def forward_backward(cfg, params, tokens, targets):
    """Return (loss, grads) with grads a dict of float64 arrays like params.

    The backward is derived by hand from the forward above:
    linear Y = X W^T gives dX = dY W, dW = dY^T X; the residual stream passes
    its gradient through unchanged and adds each branch's input gradient.
    Pinned by central finite differences and an independent torch float64
    autograd model (tests/test_oracle_model.py).
    """
    p, logits, c = _forward(cfg, params, tokens, keep=True)
    tokens = np.asarray(tokens)
    B, T = tokens.shape
    H, Hk, hd = cfg.n_heads, cfg.kv_heads, cfg.head_dim
    hh, hk = H * hd, Hk * hd
    G = H // Hk
    V = logits.shape[-1]
    cos, sin = c["cos"], c["sin"]
    flat = logits.reshape(-1, V)
    y = np.asarray(targets).reshape(-1)
    loss, lse = ops.cross_entropy(flat, y)
    dl = ops.cross_entropy_bwd(flat, y, lse).reshape(B, T, V)

    grads = {}
    z = c["z"]
    grads["W_lm"] = _wgrad(dl, z)
    dz = dl @ p["W_lm"]
    dx = ops.rmsnorm_bwd(dz, z, c["rf"])
    for l in reversed(range(cfg.depth)):
        L = c["layers"][l]
        W1, W2 = p[f"layers.{l}.W_1"], p[f"layers.{l}.W_2"]
        Wo, Wqkv = p[f"layers.{l}.W_o"], p[f"layers.{l}.W_qkv"]
        # MLP branch: x += relu2(rho(x) W_1^T) W_2^T
        grads[f"layers.{l}.W_2"] = _wgrad(dx, L["g"])
        dg = dx @ W2
        du = ops.relu2_bwd(dg, L["u"])
        grads[f"layers.{l}.W_1"] = _wgrad(du, L["m"])
        dm = du @ W1
        dx = dx + ops.rmsnorm_bwd(dm, L["m"], L["r2"])
        # attention branch: x += attn(rho(x)) W_o^T
        grads[f"layers.{l}.W_o"] = _wgrad(dx, L["O"])
        dO = dx @ Wo
        do = _heads(dO, B, T, H, hd)
        dqh, dkh, dv = ops.attention_bwd(do, L["qh"], np.repeat(L["kh"], G, axis=1),
                                         np.repeat(L["v"], G, axis=1), L["o"])
        # a shared key/value head collects the gradients of its G query heads
        dkh = dkh.reshape(B, Hk, G, T, hd).sum(axis=2)
        dv = dv.reshape(B, Hk, G, T, hd).sum(axis=2)
        dq = ops.qknorm_rope_bwd(dqh, L["qh"], L["rq"], cos, sin)
        dk = ops.qknorm_rope_bwd(dkh, L["kh"], L["rk"], cos, sin)
        dqkv = np.concatenate([_unheads(dq), _unheads(dk), _unheads(dv)], axis=-1)
        grads[f"layers.{l}.W_qkv"] = _wgrad(dqkv, L["a"])
        da = dqkv @ Wqkv
        dx = dx + ops.rmsnorm_bwd(da, L["a"], L["r1"])
        assert dqkv.shape[-1] == hh + 2 * hk
    grads["E"] = ops.embedding_bwd(dx, tokens, V)
    return loss, grads
