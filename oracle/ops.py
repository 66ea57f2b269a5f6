"""Per-operation float64 definitions used by the oracle model.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Every function takes
and returns numpy float64 arrays; there is no blocking, fusion or reordering
beyond what each definition states.
"""

import numpy as np

F64 = np.float64


# --------------------------------------------------------------------------
# RMSNorm ("nanochat explainer", Modern architecture choices: RMSNorm).
# Parameter-free: y = x / sqrt(mean(x^2) + eps) over the last axis.
# Pinned by: rms(y) = sqrt(m / (m + eps)); scale invariance at eps = 0;
# x . dx = 0 at eps = 0; torch.nn.functional.rms_norm; finite differences.
# --------------------------------------------------------------------------
def rmsnorm(x, eps):
    """Return (y, r) with r = 1/sqrt(mean(x^2) + eps) over the last axis."""
    x = np.asarray(x, dtype=F64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r, r[..., 0]


def rmsnorm_bwd(dy, y, r):
    """Gradient of rmsnorm w.r.t. its input.

    With y = x*r and r = (mean(x^2)+eps)^(-1/2), differentiating gives
    dx = r * (dy - y * mean(dy * y)).
    """
    r = r[..., None]
    return r * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))


# --------------------------------------------------------------------------
# RoPE ("nanochat explainer", Architecture Choices -> RoPE Intuition).
# Split-half pairs (i, i + hd/2); theta_i = base^(-2i/hd); angle t*theta_i.
# Pinned by: norm preservation, R_0 = I, R^T R = I, and the relative-distance
# property <R_m q, R_n k> = <R_{m+s} q, R_{n+s} k> the page states.
# --------------------------------------------------------------------------
def rope_angles(seq_len, head_dim, base):
    """Return (cos, sin), each [seq_len, head_dim/2], of t * theta_i."""
    half = head_dim // 2
    i = np.arange(half, dtype=F64)
    theta = base ** (-2.0 * i / head_dim)
    t = np.arange(seq_len, dtype=F64)
    phi = t[:, None] * theta[None, :]
    return np.cos(phi), np.sin(phi)


def rope(u, cos, sin):
    """Rotate the last axis of u; u is [..., T, hd], cos/sin [T, hd/2]."""
    half = u.shape[-1] // 2
    a, b = u[..., :half], u[..., half:]
    return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)


def rope_bwd(dv, cos, sin):
    """Apply R_t^T (rotation by -phi): the gradient of rope w.r.t. u."""
    half = dv.shape[-1] // 2
    da, db = dv[..., :half], dv[..., half:]
    return np.concatenate([da * cos + db * sin, -da * sin + db * cos], axis=-1)


# --------------------------------------------------------------------------
# Causal softmax attention ("nanochat explainer", Pretraining: causal
# next-token prediction; Inference & KV Cache: full multi-head attention).
# Query t attends to keys j <= t; the keys j > t are excluded from the sum.
# Pinned by: T = 1 gives o = v; identical keys give prefix means of v;
# rows of P sum to 1; torch scaled_dot_product_attention(is_causal=True).
# --------------------------------------------------------------------------
def causal_mask(T):
    return np.tril(np.ones((T, T), dtype=bool))


def attention_probs(qh, kh):
    """P[..., t, j] = softmax over j <= t of qh_t . kh_j / sqrt(hd); 0 for j > t.

    Also returns lse[..., t] = log sum_{j<=t} exp(s_tj) (natural log).
    """
    hd = qh.shape[-1]
    T = qh.shape[-2]
    s = np.matmul(qh, np.swapaxes(kh, -1, -2)) / np.sqrt(hd)
    mask = causal_mask(T)
    s_masked = np.where(mask, s, -np.inf)
    mx = np.max(s_masked, axis=-1, keepdims=True)
    e = np.where(mask, np.exp(np.where(mask, s, 0.0) - mx), 0.0)
    den = np.sum(e, axis=-1, keepdims=True)
    p = e / den
    lse = (mx + np.log(den))[..., 0]
    return p, lse


def attention(qh, kh, v):
    """Return (o, lse); qh, kh, v are [..., T, hd]."""
    p, lse = attention_probs(qh, kh)
    return np.matmul(p, v), lse


def attention_bwd(do, qh, kh, v, o):
    """Gradients (dqh, dkh, dv) of o = attention(qh, kh, v).

    P is recomputed from qh and kh.  With D_t = sum_h do_th * o_th:
    dv = P^T do; dP = do v^T; dS = P * (dP - D); dqh = dS kh / sqrt(hd);
    dkh = dS^T qh / sqrt(hd).
    """
    hd = qh.shape[-1]
    p, _ = attention_probs(qh, kh)
    dv = np.matmul(np.swapaxes(p, -1, -2), do)
    dp = np.matmul(do, np.swapaxes(v, -1, -2))
    D = np.sum(do * o, axis=-1, keepdims=True)
    ds = p * (dp - D)
    dqh = np.matmul(ds, kh) / np.sqrt(hd)
    dkh = np.matmul(np.swapaxes(ds, -1, -2), qh) / np.sqrt(hd)
    return dqh, dkh, dv


# --------------------------------------------------------------------------
# QK-norm then RoPE ("nanochat explainer", Modern architecture choices).
# --------------------------------------------------------------------------
def qknorm_rope(u, cos, sin, eps):
    """u is [B, H, T, hd]. Returns (R_t rho(u), r) with r [B, H, T]."""
    y, r = rmsnorm(u, eps)
    return rope(y, cos, sin), r


def qknorm_rope_bwd(dv, v, r, cos, sin):
    """Gradient w.r.t. the pre-norm u, given v = R_t rho(u) and r."""
    dy = rope_bwd(dv, cos, sin)
    y = rope_bwd(v, cos, sin)  # R_t^T v = rho(u)
    return rmsnorm_bwd(dy, y, r)


# --------------------------------------------------------------------------
# ReLU-squared ("nanochat explainer", Architecture Choices -> ReLU² Sparsity).
# --------------------------------------------------------------------------
def relu2(u):
    return np.maximum(u, 0.0) ** 2


def relu2_bwd(dg, u):
    return dg * 2.0 * np.maximum(u, 0.0)


# --------------------------------------------------------------------------
# Next-token softmax cross-entropy ("nanochat explainer", Pretraining), with
# the loss mask of supervised fine-tuning ("nanochat explainer", Supervised
# Fine-Tuning: the same cross-entropy, counted only on the assistant's
# tokens).  A negative target marks a position outside the loss:
# loss = (1/|S|) sum_{n in S} [logsumexp(l_n) - l_{n, y_n}] in nats over the
# set S of positions with a target >= 0; 0 when S is empty.
# Pinned by: zero logits give ln V exactly; rows of dl sum to 0;
# torch.nn.functional.cross_entropy (ignore_index=-1); finite differences.
# --------------------------------------------------------------------------
def logsumexp(l):
    mx = np.max(l, axis=-1, keepdims=True)
    return (mx + np.log(np.sum(np.exp(l - mx), axis=-1, keepdims=True)))[..., 0]


def cross_entropy(logits, targets):
    """logits [N, V] float64, targets [N] int (< 0: not counted). Returns (loss, lse)."""
    targets = np.asarray(targets)
    lse = logsumexp(logits)
    rows = np.nonzero(targets >= 0)[0]
    if rows.size == 0:
        return 0.0, lse
    picked = logits[rows, targets[rows]]
    return float(np.sum(lse[rows] - picked) / rows.size), lse


def cross_entropy_bwd(logits, targets, lse):
    """dl = (softmax(l) - onehot(y)) / |S| on counted rows, 0 on the others."""
    targets = np.asarray(targets)
    rows = np.nonzero(targets >= 0)[0]
    g = np.zeros_like(logits)
    if rows.size == 0:
        return g
    g[rows] = np.exp(logits[rows] - lse[rows, None])
    g[rows, targets[rows]] -= 1.0
    return g / rows.size


# --------------------------------------------------------------------------
# Token embedding, untied from the head ("nanochat explainer", Modern
# architecture choices: untied embeddings).
# --------------------------------------------------------------------------
def embedding(E, tokens):
    return E[tokens]


def embedding_bwd(dx, tokens, vocab):
    """dE[v] = sum over positions n with tokens[n] == v of dx[n], n ascending.

    Written as a plain loop over positions so that its order is the
    definition's; rows for ids that never occur stay exactly 0.
    """
    dx = dx.reshape(-1, dx.shape[-1])
    tok = np.asarray(tokens).reshape(-1)
    dE = np.zeros((vocab, dx.shape[-1]), dtype=F64)
    order = np.argsort(tok, kind="stable")
    sorted_tok = tok[order]
    bounds = np.flatnonzero(np.diff(sorted_tok)) + 1
    starts = np.concatenate([[0], bounds])
    ends = np.concatenate([bounds, [tok.size]])
    for s, e in zip(starts, ends):
        if e > s:
            rows = order[s:e]
            acc = np.zeros(dx.shape[-1], dtype=F64)
            for n in rows:
                acc += dx[n]
            dE[sorted_tok[s]] = acc
    return dE
