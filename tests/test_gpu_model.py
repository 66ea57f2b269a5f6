"""GPU parity of the whole training step (nc_forward_backward, nc_forward_logits)
against the float64 oracle.

Tolerances: loss within 1e-2 relative and every gradient tensor within 3e-2
relative L2 on the bf16 path; both within 1e-4 on the fp32 debug path.
The tiny model is checked in full, ragged shapes exercise partial tiles, the
depth-20 and depth-26 widths are checked at two layers and at full depth
(20 and 26 layers) on one sequence of 2048, and the full depth-20 bench
configuration is checked through properties that hold at any size plus
oracle losses of sampled sequences.
"""

import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import banner, pack, prep, rel_l2, to_dev, to_np, unpack

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import bwd_step_amd  # noqa: E402

TOL = {"bf16": (1e-2, 3e-2), "fp32": (1e-4, 1e-4)}


def setup(cfg, B, dt, seed=0, zipf=False):
    shapes = oracle.param_shapes(cfg)
    params = synth.weights(shapes, seed=seed, bf16=(dt == "bf16"))
    if zipf:
        tok, tgt = synth.zipf_tokens(B, cfg.seq_len, cfg.vocab, seed=seed)
    else:
        tok, tgt = synth.uniform_tokens(B, cfg.seq_len, cfg.vocab, seed=seed)
    model = bwd_step_amd.Model(cfg.depth, vocab=cfg.vocab, seq_len=cfg.seq_len, max_batch=B, dtype=dt,
                               d_model=cfg.d_model, n_heads=cfg.n_heads, head_dim=cfg.head_dim, d_ff=cfg.d_ff)
    flat = to_dev(pack(params, shapes), dt)
    return model, shapes, params, flat, to_dev(tok), to_dev(tgt), tok, tgt


def run_step(model, flat, tok_d, tgt_d, accumulate=False, grads=None):
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    if grads is None:
        grads = torch.empty(model.param_count, dtype=torch.float32, device="cuda")
    model.forward_backward(flat, tok_d, tgt_d, loss, grads, accumulate=accumulate)
    assert model.check() == 0
    return loss, grads


def compare(cfg, dt, loss, grads, shapes, ref_loss, ref_grads):
    tl, tg = TOL[dt]
    assert abs(loss - ref_loss) / abs(ref_loss) < tl, (loss, ref_loss)
    g = unpack(grads, shapes)
    worst = []
    for name, _ in shapes:
        e = rel_l2(g[name], ref_grads[name])
        worst.append((e, name))
        assert e < tg, (name, e)
    return max(worst)


TINY = oracle.derive_config(2, vocab=512, seq_len=64, d_model=128, n_heads=2, head_dim=64, d_ff=512)
RAGGED = oracle.derive_config(3, vocab=576, seq_len=100, d_model=192, n_heads=3, head_dim=64, d_ff=320)
# d = 640, d_ff = 2560: every bf16 product with a k-contiguous A runs the
# 64-deep pair loop (the forward ones, the LM-head logits, the input
# gradients on transposed weights), with ragged row tiles (272 tokens) and a
# ragged LM-head column tile (V = 1152: its last tile is moved back by one
# 128-column softmax segment)
MID = oracle.derive_config(2, vocab=1152, seq_len=136, d_model=640, n_heads=5, head_dim=128, d_ff=2560)
LONG = oracle.derive_config(1, vocab=640, seq_len=600, d_model=256, n_heads=2, head_dim=128, d_ff=512)


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
@pytest.mark.parametrize("which,B", [("tiny", 2), ("ragged", 3), ("mid", 2), ("long", 1)])
def test_step_matches_oracle_small(dt, which, B):
    cfg = {"tiny": TINY, "ragged": RAGGED, "mid": MID, "long": LONG}[which]
    banner(f"step {which} {dt} B={B}")
    model, shapes, params, flat, tok_d, tgt_d, tok, tgt = setup(cfg, B, dt)
    loss, grads = run_step(model, flat, tok_d, tgt_d)
    ref_loss, ref_grads = oracle.forward_backward(cfg, params, tok, tgt)
    worst = compare(cfg, dt, loss.item(), to_np(grads), shapes, ref_loss, ref_grads)
    print(f"worst rel-L2 {worst}", flush=True)


def test_step_deterministic_and_accumulate():
    banner("step determinism + accumulate (tiny, bf16)")
    model, shapes, params, flat, tok_d, tgt_d, tok, tgt = setup(TINY, 2, "bf16", seed=1)
    l1, g1 = run_step(model, flat, tok_d, tgt_d)
    l2, g2 = run_step(model, flat, tok_d, tgt_d)
    assert l1.item() == l2.item()
    assert torch.equal(g1, g2)  # bitwise: no floating-point atomics anywhere
    g3 = g1.clone()
    run_step(model, flat, tok_d, tgt_d, accumulate=True, grads=g3)
    assert torch.allclose(g3, 2 * g1, rtol=1e-6, atol=0)


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
def test_forward_logits_and_causality(dt):
    banner(f"forward_logits {dt}")
    model, shapes, params, flat, tok_d, tgt_d, tok, tgt = setup(TINY, 2, dt, seed=2)
    logits = torch.empty(2, TINY.seq_len, TINY.vocab, dtype=torch.float32, device="cuda")
    model.forward_logits(flat, tok_d, logits)
    assert model.check() == 0
    ref = oracle.forward_logits(TINY, params, tok)
    assert rel_l2(to_np(logits), ref) < (1e-4 if dt == "fp32" else 2e-2)
    # changing tokens after position t0 leaves logits at positions <= t0 bitwise unchanged
    t0 = 37
    tok2 = tok.copy()
    tok2[:, t0 + 1:] = (tok2[:, t0 + 1:] + 11) % TINY.vocab
    logits2 = torch.empty_like(logits)
    model.forward_logits(flat, to_dev(tok2), logits2)
    assert torch.equal(logits[:, : t0 + 1], logits2[:, : t0 + 1])
    assert not torch.equal(logits[:, t0 + 1:], logits2[:, t0 + 1:])


def test_token_range_status():
    banner("step with an out-of-range token")
    model, shapes, params, flat, tok_d, tgt_d, tok, tgt = setup(TINY, 1, "bf16", seed=3)
    bad = tok.copy()
    bad[0, 5] = TINY.vocab + 3
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    grads = torch.empty(model.param_count, dtype=torch.float32, device="cuda")
    model.forward_backward(flat, to_dev(bad), tgt_d, loss, grads)
    assert model.check() == 4
    assert model.check() == 0


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
@pytest.mark.parametrize("depth_widths,zipf", [(20, False), (26, True)])
def test_step_real_widths_two_layers(dt, depth_widths, zipf):
    # depth-20 / depth-26 widths (d 1280 / 1664, 128-wide heads, V 65536), two layers, one sequence of 2048
    full = oracle.derive_config(depth_widths)
    cfg = oracle.derive_config(2, d_model=full.d_model, n_heads=full.n_heads, d_ff=full.d_ff)
    banner(f"step widths of depth {depth_widths}, 2 layers, B=1, {dt}, zipf={zipf}")
    model, shapes, params, flat, tok_d, tgt_d, tok, tgt = setup(cfg, 1, dt, seed=4, zipf=zipf)
    loss, grads = run_step(model, flat, tok_d, tgt_d)
    g = to_np(grads)
    ref_loss, ref_grads = oracle.forward_backward(cfg, params, tok, tgt)
    worst = compare(cfg, dt, loss.item(), g, shapes, ref_loss, ref_grads)
    print(f"worst rel-L2 {worst}", flush=True)


def test_full_depth20_bench_config_properties():
    """Depth 20, d 1280, V 65536, B 32 x T 2048 (the bench workload).

    The oracle cannot run a whole step at this size, so: (a) two runs give
    bitwise-identical gradients; (b) the batch loss is the mean of the 32
    per-sequence losses (fp32 sums only, 1e-5) and the batch gradient the
    mean of the per-sequence gradients to the bf16 tolerance (the B=32 and B=1
    runs sum in different fp32 orders, after which the two runs' bf16
    roundings decorrelate); (c) a sampled sequence's loss matches the oracle's
    forward; (d) the init loss is near ln V + sigma^2/2 for logits of variance
    0.02^2 * d.
    """
    cfg = oracle.derive_config(20)
    B = 32
    banner("full depth-20 step B=32 (bench configuration)")
    model, shapes, params, flat, tok_d, tgt_d, tok, tgt = setup(cfg, B, "bf16", seed=0)
    loss, grads = run_step(model, flat, tok_d, tgt_d)
    loss2, grads2 = run_step(model, flat, tok_d, tgt_d)
    assert torch.equal(grads, grads2) and loss.item() == loss2.item()
    del grads2
    L = loss.item()
    assert math.isfinite(L)
    assert abs(L - (math.log(cfg.vocab) + 0.02 ** 2 * cfg.d_model / 2)) < 0.05
    acc = torch.zeros_like(grads)
    per = []
    one = bwd_step_amd.Model(20, max_batch=1, dtype="bf16")
    for b in range(B):
        lb, _ = run_step(one, flat, tok_d[b:b + 1].contiguous(), tgt_d[b:b + 1].contiguous(),
                         accumulate=(b > 0), grads=acc)
        per.append(lb.item())
    assert abs(L - float(np.mean(per))) / L < 1e-5
    acc /= B
    gn = unpack(to_np(grads), shapes)
    an = unpack(to_np(acc), shapes)
    errs = {name: rel_l2(gn[name], an[name]) for name, _ in shapes}
    print("batch-linearity rel-L2: max %.2e (%s)" % max((v, k) for k, v in errs.items()), flush=True)
    assert max(errs.values()) < 3e-2
    p64 = {k: v.astype(np.float64) for k, v in params.items()}
    ref = oracle.forward(cfg, p64, tok[31:32], tgt[31:32])
    assert abs(per[31] - ref) / ref < 1e-2, (per[31], ref)


_FULL = {}


def _full_depth20_reference():
    """Oracle loss and gradients of one 2048-token sequence at full depth 20 (computed once)."""
    if not _FULL:
        cfg = oracle.derive_config(20)
        shapes = oracle.param_shapes(cfg)
        params = synth.weights(shapes, seed=5, bf16=True)  # bf16-representable: feeds both paths exactly
        tok, tgt = synth.uniform_tokens(1, cfg.seq_len, cfg.vocab, seed=5)
        p64 = {k: v.astype(np.float64) for k, v in params.items()}
        ref_loss, ref_grads = oracle.forward_backward(cfg, p64, tok, tgt)
        _FULL.update(cfg=cfg, shapes=shapes, params=params, tok=tok, tgt=tgt, loss=ref_loss, grads=ref_grads)
    return _FULL


def _full_depth_run(R, depth, mode):
    """One step of the full-depth model on R's sequence; mode is "fp32", "bf16"
    (sublayer outputs added to the fp32 residual stream as bf16) or
    "bf16-resid32" (added as fp32 in the projection epilogue)."""
    dt = "fp32" if mode == "fp32" else "bf16"
    cfg, shapes = R["cfg"], R["shapes"]
    model = bwd_step_amd.Model(depth, max_batch=1, dtype=dt)
    if mode == "bf16-resid32":
        model.set_residual_fp32(True)
    flat = to_dev(pack(R["params"], shapes), dt)
    loss, grads = run_step(model, flat, to_dev(R["tok"]), to_dev(R["tgt"]))
    worst = compare(cfg, dt, loss.item(), to_np(grads), shapes, R["loss"], R["grads"])
    print(f"{mode}: loss rel err {abs(loss.item() - R['loss']) / R['loss']:.3g}, worst grad rel-L2 {worst}", flush=True)
    return worst


@pytest.mark.timeout(600)
@pytest.mark.parametrize("mode", ["bf16", "bf16-resid32", "fp32"])
def test_full_depth20_one_sequence_matches_oracle(mode):
    """All 20 layers at the real widths, one sequence of 2048: every gradient tensor."""
    banner(f"full depth-20, B=1, {mode}, against the oracle")
    _full_depth_run(_full_depth20_reference(), 20, mode)


_FULL26 = {}


def _full_depth26_reference():
    """Oracle loss and gradients of one 2048-token sequence at full depth 26
    (d 1664, 13 heads of 128, F 6656, V 65536), Zipf(1.1) ids (computed once)."""
    if not _FULL26:
        cfg = oracle.derive_config(26)
        shapes = oracle.param_shapes(cfg)
        params = synth.weights(shapes, seed=6, bf16=True)
        tok, tgt = synth.zipf_tokens(1, cfg.seq_len, cfg.vocab, seed=6)
        p64 = {k: v.astype(np.float64) for k, v in params.items()}
        ref_loss, ref_grads = oracle.forward_backward(cfg, p64, tok, tgt)
        _FULL26.update(cfg=cfg, shapes=shapes, params=params, tok=tok, tgt=tgt, loss=ref_loss, grads=ref_grads)
    return _FULL26


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", ["bf16", "bf16-resid32", "fp32"])
def test_full_depth26_one_sequence_matches_oracle(mode):
    """All 26 layers at the depth-26 widths, one Zipf(1.1) sequence of 2048:
    every gradient tensor.  The bf16 addend of the residual stream is kept
    only while its worst gradient error after 26 layers stays within 2e-2."""
    banner(f"full depth-26, B=1, Zipf ids, {mode}, against the oracle")
    worst = _full_depth_run(_full_depth26_reference(), 26, mode)
    if mode == "bf16":
        assert worst[0] <= 2e-2, worst


def test_nonfinite_loss_status():
    """An infinite LM-head weight makes the loss non-finite: nc_check reports
    NC_ERR_NONFINITE (5) and clears the word."""
    banner("step with an infinite weight: non-finite loss status")
    model, shapes, params, flat, tok_d, tgt_d, tok, tgt = setup(TINY, 1, "bf16", seed=7)
    lm_off = [o for n, o, _, _ in model.layout() if n == "W_lm"][0]
    flat[lm_off + 3] = float("inf")
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    grads = torch.empty(model.param_count, dtype=torch.float32, device="cuda")
    model.forward_backward(flat, tok_d, tgt_d, loss, grads)
    assert model.check() == 5
    assert not math.isfinite(loss.item())
    assert model.check() == 0


@pytest.mark.parametrize("which,B", [("tiny", 2), ("ragged", 3), ("mid", 2), ("long", 1)])
def test_poisoned_workspace_gives_identical_results(which, B):
    """With the workspace NaN-filled before the step, loss and gradients are
    bitwise those of a normal step: no kernel reads workspace memory it did
    not write in the same call (mid: stored-dS columns past the sequence,
    moved-back GEMM tiles; ragged: partial tiles everywhere; long: 600
    tokens at head_dim 128, so the dQ kernel's 256-query tiles meet key
    blocks whose dS chunks the dK/dV kernel never stores)."""
    cfg = {"tiny": TINY, "ragged": RAGGED, "mid": MID, "long": LONG}[which]
    banner(f"poisoned workspace, {which} bf16 B={B}")
    model, shapes, params, flat, tok_d, tgt_d, tok, tgt = setup(cfg, B, "bf16", seed=8)
    l1, g1 = run_step(model, flat, tok_d, tgt_d)
    logits = torch.empty(B, cfg.seq_len, cfg.vocab, dtype=torch.float32, device="cuda")
    model.forward_logits(flat, tok_d, logits)
    model.poison_workspace(True)
    l2, g2 = run_step(model, flat, tok_d, tgt_d)
    logits2 = torch.empty_like(logits)
    model.forward_logits(flat, tok_d, logits2)
    model.poison_workspace(False)
    assert l1.item() == l2.item()
    assert torch.equal(g1, g2)
    assert torch.equal(logits, logits2)
