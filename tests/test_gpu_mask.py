"""GPU parity of the loss mask (negative targets are not counted) and of the
in-library gradient accumulation (nc_forward_backward_accum) against the
float64 oracle, whose masked cross-entropy is pinned in
tests/test_oracle_ops.py and tests/test_oracle_model.py.

Tolerances as for the unmasked step: loss within 1e-2 relative and every
gradient tensor within 3e-2 relative L2 on the bf16 path, 1e-4 on the fp32
path.  Accumulated and single-call steps over the same sequences differ
only in summation order (and, through a different split-K choice for the
smaller microbatch, in which bf16 roundings the input gradients take):
1e-5 relative on the loss; relative L2 on the gradients 2e-3 on the small
models (bf16 operands), 1e-5 on the fp32 path, and 1e-2 at depth 20, where
each embedding row's gradient is the sum of about one token's bf16-rounded
input gradient, so roundings of 2^-9 do not average out.
"""

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
from bwd_step_amd import ops  # noqa: E402

TOL = {"bf16": (1e-2, 3e-2), "fp32": (1e-4, 1e-4)}
TINY = oracle.derive_config(2, vocab=512, seq_len=64, d_model=128, n_heads=2, head_dim=64, d_ff=512)
RAGGED = oracle.derive_config(3, vocab=576, seq_len=100, d_model=192, n_heads=3, head_dim=64, d_ff=320)


def masked(tgt, seed, frac):
    rng = np.random.default_rng(seed)
    t = tgt.copy()
    t[rng.random(t.shape) < frac] = -1
    return t


def setup(cfg, B, dt, seed, max_batch=None):
    shapes = oracle.param_shapes(cfg)
    params = synth.weights(shapes, seed=seed, bf16=(dt == "bf16"))
    tok, tgt = synth.uniform_tokens(B, cfg.seq_len, cfg.vocab, seed=seed)
    model = bwd_step_amd.Model(cfg.depth, vocab=cfg.vocab, seq_len=cfg.seq_len, max_batch=max_batch or B, dtype=dt,
                               d_model=cfg.d_model, n_heads=cfg.n_heads, head_dim=cfg.head_dim, d_ff=cfg.d_ff)
    return model, shapes, params, to_dev(pack(params, shapes), dt), tok, tgt


def step(model, flat, tok, tgt):
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    grads = torch.empty(model.param_count, dtype=torch.float32, device="cuda")
    model.forward_backward(flat, to_dev(tok), to_dev(tgt), loss, grads)
    assert model.check() == 0
    return loss.item(), grads


def compare(dt, loss, grads, shapes, ref_loss, ref_grads):
    tl, tg = TOL[dt]
    assert abs(loss - ref_loss) <= tl * abs(ref_loss), (loss, ref_loss)
    g = unpack(to_np(grads), shapes)
    worst = max((rel_l2(g[n], ref_grads[n]), n) for n, _ in shapes)
    assert worst[0] < tg, worst
    return worst


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
@pytest.mark.parametrize("which,B,frac", [("tiny", 2, 0.4), ("ragged", 3, 0.7)])
def test_masked_step_matches_oracle(dt, which, B, frac):
    cfg = TINY if which == "tiny" else RAGGED
    banner(f"masked step {which} {dt} B={B} frac={frac}")
    model, shapes, params, flat, tok, tgt = setup(cfg, B, dt, seed=20)
    t = masked(tgt, 21, frac)
    t[-1, :] = -1  # one whole sequence outside the loss
    loss, grads = step(model, flat, tok, t)
    ref_loss, ref_grads = oracle.forward_backward(cfg, params, tok, t)
    print(f"worst {compare(dt, loss, grads, shapes, ref_loss, ref_grads)}", flush=True)


def test_all_masked_gives_zero():
    banner("every target masked (tiny, bf16)")
    model, shapes, params, flat, tok, tgt = setup(TINY, 2, "bf16", seed=22)
    loss, grads = step(model, flat, tok, np.full_like(tgt, -1))
    assert loss == 0.0
    assert int(torch.count_nonzero(grads)) == 0


def test_target_out_of_range_still_flagged():
    banner("target >= vocab sets the status (tiny, bf16)")
    model, shapes, params, flat, tok, tgt = setup(TINY, 1, "bf16", seed=23)
    bad = tgt.copy()
    bad[0, 3] = TINY.vocab
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    grads = torch.empty(model.param_count, dtype=torch.float32, device="cuda")
    model.forward_backward(flat, to_dev(tok), to_dev(bad), loss, grads)
    assert model.check() == 4
    assert model.check() == 0


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
@pytest.mark.parametrize("which,B,n_micro", [("tiny", 4, 2), ("ragged", 3, 3)])
def test_accumulated_step_matches_oracle_and_single_call(dt, which, B, n_micro):
    cfg = TINY if which == "tiny" else RAGGED
    banner(f"accumulated step {which} {dt} B={B} n_micro={n_micro}")
    model, shapes, params, flat, tok, tgt = setup(cfg, B, dt, seed=24)
    t = masked(tgt, 25, 0.3)
    t[0, :] = -1  # microbatches with different counts
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    grads = torch.empty(model.param_count, dtype=torch.float32, device="cuda")
    model.forward_backward_accum(flat, to_dev(tok), to_dev(t), n_micro, loss, grads)
    assert model.check() == 0
    ref_loss, ref_grads = oracle.forward_backward(cfg, params, tok, t)
    worst = compare(dt, loss.item(), grads, shapes, ref_loss, ref_grads)
    l1, g1 = step(model, flat, tok, t)
    assert abs(loss.item() - l1) <= 1e-5 * abs(l1), (loss.item(), l1)
    e = rel_l2(to_np(grads), to_np(g1))
    print(f"worst vs oracle {worst}; accumulated vs single call {e:.3g}", flush=True)
    assert e < (2e-3 if dt == "bf16" else 1e-5)


def test_lmhead_op_masked_matches_oracle():
    banner("LM head + CE op with masked ids (N 300, d 64, V 1024, fp32 and bf16)")
    N, d, V = 300, 64, 1024
    rng = np.random.default_rng(26)
    z = rng.standard_normal((N, d)).astype(np.float32)
    W = (0.1 * rng.standard_normal((V, d))).astype(np.float32)
    y = rng.integers(0, V, N).astype(np.int32)
    y[rng.random(N) < 0.5] = -1
    for dt, tl, tg in (("fp32", 1e-5, 1e-4), ("bf16", 1e-4, 3e-2)):
        zz, WW = prep(z, dt), prep(W, dt)
        loss, dz, dW, ws = ops.lmhead_ce_fwd_bwd(to_dev(zz, dt), to_dev(WW, dt), to_dev(y))
        assert ops.status(ws) == 0
        l = zz.astype(np.float64) @ WW.astype(np.float64).T
        ref, lse = oracle.ops.cross_entropy(l, y)
        G = oracle.ops.cross_entropy_bwd(l, y, lse)
        assert abs(loss.item() - ref) <= tl * abs(ref)
        assert rel_l2(to_np(dz), G @ WW.astype(np.float64)) < tg
        assert rel_l2(to_np(dW), G.T @ zz.astype(np.float64)) < tg
        assert np.all(to_np(dz)[y < 0] == 0.0)


def test_accumulation_full_depth20_bench_config():
    # the bench workload (depth 20, 32 x 2048) as 2 microbatches of 16 against one call of 32
    banner("depth 20, B = 32: accumulated (2 x 16) vs single call")
    cfg = oracle.derive_config(20)
    model = bwd_step_amd.Model(20, vocab=cfg.vocab, seq_len=cfg.seq_len, max_batch=32, dtype="bf16")
    shapes = [(n, (r, c)) for n, _, r, c in model.layout()]
    gen = torch.Generator(device="cuda").manual_seed(27)
    flat = (0.02 * torch.randn(model.param_count, generator=gen, device="cuda")).to(torch.bfloat16)
    tok, tgt = synth.uniform_tokens(32, cfg.seq_len, cfg.vocab, seed=27)
    t = masked(tgt, 28, 0.25)
    tok_d, t_d = to_dev(tok), to_dev(t)
    loss1 = torch.empty((), dtype=torch.float32, device="cuda")
    g1 = torch.empty(model.param_count, dtype=torch.float32, device="cuda")
    model.forward_backward(flat, tok_d, t_d, loss1, g1)
    assert model.check() == 0
    loss2 = torch.empty_like(loss1)
    g2 = torch.empty_like(g1)
    model.forward_backward_accum(flat, tok_d, t_d, 2, loss2, g2)
    assert model.check() == 0
    assert abs(loss2.item() - loss1.item()) <= 1e-5 * abs(loss1.item())
    a, b = to_np(g1), to_np(g2)
    for name, off, r, c in model.layout():
        e = rel_l2(b[off:off + r * c], a[off:off + r * c])
        assert e < 1e-2, (name, e)
    # at init the logits are ~N(0, 0.02^2 d) (unit-rms z), so the loss is about ln V + 0.02^2 d / 2
    assert abs(loss1.item() - (np.log(cfg.vocab) + 0.02 ** 2 * cfg.d_model / 2)) < 0.02
