"""The bench's FLOP accounting, checked by counting on the CPU.

bench.py reports MFU from model FLOPs per token: three times the forward
matmul FLOPs ("nanochat explainer", Modern architecture choices, for the
layers: QKV and output projections, a two-matrix MLP, an untied LM head) plus
causal attention, and beside it the PaLM-convention count (every query against
all T keys).  Here both are recounted from first principles: every linear
layer's multiply-adds enumerated from the model's shapes, and the causal
(query, key) pairs of a sequence summed key by key.
"""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _cfg(depth, d, heads, hd, ff, vocab, T):
    return dict(d_model=d, n_heads=heads, head_dim=hd, d_ff=ff, vocab=vocab, depth=depth, seq_len=T)


def _counted(c, causal):
    """FLOPs of one fwd+bwd sequence divided by its tokens, counted term by term."""
    d, H, hd, F, V, L, T = (c[k] for k in ("d_model", "n_heads", "head_dim", "d_ff", "vocab", "depth", "seq_len"))
    # (in, out) of every linear layer a token passes through
    layers = []
    for _ in range(L):
        layers += [(d, 3 * H * hd), (H * hd, d), (d, F), (F, d)]
    layers.append((d, V))
    fwd_lin = sum(2 * i * o for i, o in layers) * T
    # query t attends to keys 0..t (causal) or to all T keys; QK^T and PV
    # each take 2 hd FLOPs per (query, key) pair and head
    pairs = sum((t + 1) if causal else T for t in range(T))
    fwd_att = L * H * pairs * 2 * (2 * hd)
    return 3 * (fwd_lin + fwd_att) / T


def test_model_flops_match_the_count():
    for c in (_cfg(2, 128, 2, 64, 512, 512, 64), _cfg(3, 192, 3, 64, 768, 1000, 97)):
        assert abs(bench.model_flops_per_token(c) - _counted(c, causal=True)) <= 1e-9 * _counted(c, True)


def test_palm_flops_match_the_count():
    # the PaLM count is 6 N for the matmul weights plus 12 L H hd T, i.e. the
    # same enumeration with every query against all T keys
    for c in (_cfg(2, 128, 2, 64, 512, 512, 64), _cfg(3, 192, 3, 64, 768, 1000, 97)):
        assert abs(bench.palm_flops_per_token(c) - _counted(c, causal=False)) <= 1e-9 * _counted(c, False)


def test_depth20_figures():
    c = _cfg(20, 1280, 10, 128, 5120, 65536, 2048)
    assert bench.model_flops_per_token(c) == 3_177_338_880
    assert bench.palm_flops_per_token(c) == 3_491_758_080
