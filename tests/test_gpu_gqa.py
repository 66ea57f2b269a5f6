"""GPU parity of grouped-query and multi-query attention (n_kv_heads <
n_heads) against the float64 oracle, whose grouped attention is pinned in
tests/test_oracle_model.py: the training step (loss and every gradient,
the bars of tests/test_gpu_model.py) and prefill + decode (logits, the
bars of tests/test_gpu_infer.py).
"""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import banner, pack, rel_l2, to_dev, to_np, unpack

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import bwd_step_amd  # noqa: E402
from bwd_step_amd import ops  # noqa: E402

TOL = {"bf16": (1e-2, 3e-2), "fp32": (1e-4, 1e-4)}
LOGIT_TOL = {"fp32": 1e-4, "bf16": 2e-2}
CFGS = {
    # 4 query heads of 64 sharing 2 key/value heads; T ragged for the tiles
    "gqa": oracle.derive_config(2, vocab=512, seq_len=96, d_model=256, n_heads=4, head_dim=64, d_ff=512,
                                n_kv_heads=2),
    # multi-query: 2 heads of 128 sharing one
    "mqa": oracle.derive_config(2, vocab=576, seq_len=70, d_model=256, n_heads=2, head_dim=128, d_ff=320,
                                n_kv_heads=1),
}


def make(cfg, B, dt, seed):
    shapes = oracle.param_shapes(cfg)
    params = synth.weights(shapes, seed=seed, bf16=(dt == "bf16"))
    tok, tgt = synth.uniform_tokens(B, cfg.seq_len, cfg.vocab, seed=seed)
    model = bwd_step_amd.Model(cfg.depth, vocab=cfg.vocab, seq_len=cfg.seq_len, max_batch=B, dtype=dt,
                               d_model=cfg.d_model, n_heads=cfg.n_heads, head_dim=cfg.head_dim, d_ff=cfg.d_ff,
                               n_kv_heads=cfg.n_kv_heads)
    return model, shapes, params, to_dev(pack(params, shapes), dt), tok, tgt


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
@pytest.mark.parametrize("which", ["gqa", "mqa"])
def test_grouped_step_matches_oracle(dt, which):
    cfg = CFGS[which]
    banner(f"training step {which} {dt} (H {cfg.n_heads}, kv heads {cfg.kv_heads})")
    model, shapes, params, flat, tok, tgt = make(cfg, 2, dt, seed=40)
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    grads = torch.empty(model.param_count, dtype=torch.float32, device="cuda")
    model.forward_backward(flat, to_dev(tok), to_dev(tgt), loss, grads)
    assert model.check() == 0
    ref_loss, ref_grads = oracle.forward_backward(cfg, params, tok, tgt)
    tl, tg = TOL[dt]
    assert abs(loss.item() - ref_loss) <= tl * abs(ref_loss), (loss.item(), ref_loss)
    g = unpack(to_np(grads), shapes)
    worst = max((rel_l2(g[n], ref_grads[n]), n) for n, _ in shapes)
    print(f"worst {worst}", flush=True)
    assert worst[0] < tg, worst


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
@pytest.mark.parametrize("which", ["gqa", "mqa"])
def test_grouped_prefill_decode_matches_forward(dt, which):
    cfg = CFGS[which]
    banner(f"prefill + decode {which} {dt}")
    B, Tp, steps, max_len = 2, 30, 5, 128
    model, shapes, params, flat, tok, _ = make(cfg, B, dt, seed=41)
    ref = oracle.forward_logits(cfg, params, tok[:, : Tp + steps])
    es = 2 if dt == "bf16" else 4
    # the cache holds kv_heads heads per layer
    assert model.kv_cache_bytes(B, max_len) == cfg.depth * 2 * B * cfg.kv_heads * max_len * cfg.head_dim * es
    cache = torch.zeros(model.kv_cache_bytes(B, max_len) // es,
                        dtype=torch.bfloat16 if dt == "bf16" else torch.float32, device="cuda")
    ws = torch.zeros(model.decode_workspace_bytes(B, max_len), dtype=torch.uint8, device="cuda")
    logits = torch.empty(B, cfg.vocab, dtype=torch.float32, device="cuda")
    model.prefill(flat, to_dev(np.ascontiguousarray(tok[:, :Tp])), cache, B, max_len, logits)
    assert model.check() == 0
    worst = max(rel_l2(to_np(logits)[b], ref[b, Tp - 1]) for b in range(B))
    for k in range(steps):
        t = Tp + k
        model.decode(flat, to_dev(np.ascontiguousarray(tok[:, t])), to_dev(np.full(B, t, np.int32)), cache,
                     max_len, ws, logits)
        assert ops.status(ws) == 0
        worst = max(worst, max(rel_l2(to_np(logits)[b], ref[b, t]) for b in range(B)))
    print(f"worst logits rel-L2 {worst:.3g}", flush=True)
    assert worst < LOGIT_TOL[dt]
