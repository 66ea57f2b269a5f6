"""Float64 oracle of one optimizer step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix ("nanochat explainer", The Full Pipeline -> Pretraining),
as settings: optimizer groups Muon (layer matrices) and AdamW (E, W_lm);
learning rate warmed up, then cosine-decayed; global gradient-norm bound 1.0;
weight decay 0.1.  "Karpathy Built a Full ChatGPT Clone in 8,000
Lines of Code" (What the Community Is Saying) attributes Muon to Bernstein,
in Keller Jordan's implementation, and has AdamW handle the embeddings.  The
pages give no further detail; the rest follows the optimizers' published
descriptions and the plainest readings:

* groups: AdamW for E and W_lm; Muon for every weight tensor of the layers
  (W_qkv taken as one [3*H*hd, d] matrix, W_o, W_1, W_2);
* schedule: lr(s) = peak * (s + 1) / warmup for s < warmup, then
  peak * (f + (1 - f) * (1 + cos(pi * p)) / 2) with p = (s - warmup) /
  max(1, total - warmup) and f the final fraction; one multiplier for both
  groups, each with its own peak;
* clipping: one global L2 norm over all gradients; every gradient is
  multiplied by min(1, clip / (norm + 1e-6));
* weight decay: decoupled (theta <- theta - lr * wd * theta), both groups;
* AdamW (Loshchilov and Hutter, "Decoupled Weight Decay Regularization"):
  m = b1 m + (1 - b1) g, v = b2 v + (1 - b2) g^2, bias-corrected by
  1 - b^t, theta <- theta - lr (m_hat / (sqrt(v_hat) + eps) + wd theta);
* Muon (Jordan et al., "Muon: An optimizer for hidden layers in neural
  networks", 2024): momentum buffer B = mu B + G, Nesterov update U = G +
  mu B, O = NS5(U) (the quintic Newton-Schulz orthogonalisation of U / |U|_F
  with (a, b, c) = (3.4445, -4.7750, 2.0315), run on the wide orientation),
  W <- W - lr (sqrt(max(1, rows / cols)) O + wd W);
* state: fp32 master weights (here float64) from which the bf16 parameters
  are re-derived after every step.

Pin status: every function is pinned in tests/test_oracle_optim.py (closed
forms of the schedule, of the clipped norm and of AdamW under a constant
gradient, and NS5 against the scalar polynomial applied to the singular
values of a matrix built from random orthogonal factors).
"""

import math

import numpy as np

F64 = np.float64

NS_COEFFS = (3.4445, -4.7750, 2.0315)


def cosine_lr(step, peak, warmup, total, final_frac):
    """Learning rate of optimizer step `step` (0-based)."""
    if step < warmup:
        return peak * (step + 1) / warmup
    p = (step - warmup) / max(1, total - warmup)
    p = min(max(p, 0.0), 1.0)
    return peak * (final_frac + (1.0 - final_frac) * 0.5 * (1.0 + math.cos(math.pi * p)))


def clip_scale(grads, clip):
    """(global L2 norm of all gradient arrays, the factor that clips it)."""
    sq = sum(float(np.sum(np.asarray(g, dtype=F64) ** 2)) for g in grads)
    norm = math.sqrt(sq)
    return norm, min(1.0, clip / (norm + 1e-6))


def adamw_update(theta, g, m, v, t, lr, b1, b2, eps, wd):
    """One AdamW step at step count t (1-based); returns (theta, m, v)."""
    m = b1 * m + (1.0 - b1) * g
    v = b2 * v + (1.0 - b2) * g * g
    m_hat = m / (1.0 - b1 ** t)
    v_hat = v / (1.0 - b2 ** t)
    theta = theta - lr * (m_hat / (np.sqrt(v_hat) + eps) + wd * theta)
    return theta, m, v


def newton_schulz5(U, steps=5):
    """Quintic Newton-Schulz orthogonalisation of U (2-D): starting from
    X = U / |U|_F (transposed to the wide orientation), repeat
    X <- a X + (b A + c A A) X with A = X X^T; each step maps every singular
    value s of X to a s + b s^3 + c s^5 and keeps the singular vectors."""
    a, b, c = NS_COEFFS
    X = np.asarray(U, dtype=F64)
    X = X / (np.linalg.norm(X) + 1e-7)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    for _ in range(steps):
        A = X @ X.T
        X = a * X + (b * A + c * (A @ A)) @ X
    return X.T if tall else X


def muon_update(W, G, buf, lr, mu, wd, steps=5):
    """One Muon step of the matrix W [rows, cols]; returns (W, buf)."""
    buf = mu * buf + G
    U = G + mu * buf
    O = newton_schulz5(U, steps)
    rows, cols = W.shape
    W = W - lr * (math.sqrt(max(1.0, rows / cols)) * O + wd * W)
    return W, buf


ADAMW_TENSORS = ("E", "W_lm")


def is_adamw(name):
    """AdamW group: the embedding and the unembedding; Muon for the rest."""
    return name in ADAMW_TENSORS


def optimizer_step(master, grads, state, hp, step):
    """One optimizer step over all tensors.

    master: dict name -> float64 array (the master weights), updated copies
    are returned.  grads: dict name -> gradient.  state: dict with 'm', 'v'
    (AdamW tensors) and 'buf' (Muon tensors), each a dict name -> array
    (missing entries start at zero).  hp: dict with lr_adamw, lr_muon,
    warmup, total, final_frac, clip, wd, beta1, beta2, eps, momentum,
    ns_steps.  Returns (master, state, grad_norm, lr multiplier)."""
    names = list(master)
    norm, s = clip_scale([grads[n] for n in names], hp["clip"])
    mult = cosine_lr(step, 1.0, hp["warmup"], hp["total"], hp["final_frac"])
    new_master, new_state = {}, {"m": {}, "v": {}, "buf": {}}
    for n in names:
        th = np.asarray(master[n], dtype=F64)
        g = np.asarray(grads[n], dtype=F64) * s
        if is_adamw(n):
            m = state["m"].get(n, np.zeros_like(th))
            v = state["v"].get(n, np.zeros_like(th))
            th, m, v = adamw_update(th, g, m, v, step + 1, hp["lr_adamw"] * mult, hp["beta1"], hp["beta2"],
                                    hp["eps"], hp["wd"])
            new_state["m"][n], new_state["v"][n] = m, v
        else:
            b = state["buf"].get(n, np.zeros_like(th))
            th, b = muon_update(th, g, b, hp["lr_muon"] * mult, hp["momentum"], hp["wd"], hp["ns_steps"])
            new_state["buf"][n] = b
        new_master[n] = th
    return new_master, new_state, norm, mult
