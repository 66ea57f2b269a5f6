"""GPU parity of the optimizer step (nc_optim_init, nc_optim_step) against the
float64 oracle (oracle/optim.py).

Tolerances, on the update of each tensor (new master minus old master),
relative L2: AdamW tensors 1e-5 on both paths (fp32 arithmetic end to end);
Muon tensors 1e-4 on the fp32 path and 3e-2 on the bf16 path, whose
Newton-Schulz operands are rounded to bf16 (8-bit mantissa) between the fp32
accumulations of every product.  The gradient norm is accumulated in fp64
and returned in fp32: 1e-6 relative.  The small models are checked in full
over several steps (warmup, then decay), including tall and wide matrices
and widths that are not multiples of the GEMM tile; the depth-20 parameter
set is checked on its norm, a sampled block of the embedding and two layer
matrices, at full size.
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
from oracle import optim  # noqa: E402

TINY = oracle.derive_config(2, vocab=512, seq_len=64, d_model=128, n_heads=2, head_dim=64, d_ff=512)
RAGGED = oracle.derive_config(3, vocab=576, seq_len=100, d_model=192, n_heads=3, head_dim=64, d_ff=320)

HP = dict(lr_adamw=3e-3, lr_muon=0.02, beta1=0.9, beta2=0.95, eps=1e-8, momentum=0.95, weight_decay=0.1,
          clip=1.0, final_frac=0.1, warmup_steps=2, total_steps=6, ns_steps=5)
TOL_MUON = {"fp32": 1e-4, "bf16": 3e-2}
TOL_ADAMW = 1e-5


def oracle_hp(hp):
    return dict(lr_adamw=hp["lr_adamw"], lr_muon=hp["lr_muon"], warmup=hp["warmup_steps"],
                total=hp["total_steps"], final_frac=hp["final_frac"], clip=hp["clip"], wd=hp["weight_decay"],
                beta1=hp["beta1"], beta2=hp["beta2"], eps=hp["eps"], momentum=hp["momentum"],
                ns_steps=hp["ns_steps"])


def model_for(cfg, dt):
    return bwd_step_amd.Model(cfg.depth, vocab=cfg.vocab, seq_len=cfg.seq_len, max_batch=1, dtype=dt,
                              d_model=cfg.d_model, n_heads=cfg.n_heads, head_dim=cfg.head_dim, d_ff=cfg.d_ff)


def buffers(model):
    state = torch.empty(model.optim_state_bytes() // 4, dtype=torch.float32, device="cuda")
    ws = torch.empty(model.optim_workspace_bytes(), dtype=torch.uint8, device="cuda")
    return state, ws


def grads_for(shapes, seed, scale):
    rng = np.random.default_rng(seed)
    return {n: (scale * rng.standard_normal(s)).astype(np.float32) for n, s in shapes}


def state_views(model, state, shapes):
    """(masters, {name: (m, v)} of AdamW tensors, {name: buf} of Muon tensors) as numpy."""
    P = model.param_count
    st = to_np(state)
    masters = unpack(st[:P], shapes)
    adam, buf, off = {}, {}, P
    for n, s in shapes:
        k = int(np.prod(s))
        if optim.is_adamw(n):
            adam[n] = (st[off:off + k].reshape(s), st[off + k:off + 2 * k].reshape(s))
            off += 2 * k
        else:
            buf[n] = st[off:off + k].reshape(s)
            off += k
    assert off * 4 == model.optim_state_bytes()
    return masters, adam, buf


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
@pytest.mark.parametrize("which,gscale", [("tiny", 1.0), ("ragged", 1e-4)])
def test_optim_steps_match_oracle(dt, which, gscale):
    # gscale 1.0: the gradient norm is far above the clip; 1e-4: below it (no clipping)
    cfg = TINY if which == "tiny" else RAGGED
    banner(f"optimizer {which} {dt} gscale={gscale}")
    shapes = oracle.param_shapes(cfg)
    model = model_for(cfg, dt)
    params = synth.weights(shapes, seed=7, bf16=(dt == "bf16"))
    flat = to_dev(pack(params, shapes), dt)
    state, ws = buffers(model)
    model.optim_init(flat, state)
    gnorm = torch.empty((), dtype=torch.float32, device="cuda")

    ref_master = {n: np.asarray(params[n], dtype=np.float64) for n, _ in shapes}
    ref_state = {"m": {}, "v": {}, "buf": {}}
    ohp = oracle_hp(HP)
    for step in range(4):
        g = grads_for(shapes, 100 + step, gscale)
        model.optim_step(step, to_dev(pack(g, shapes)), flat, state, ws, grad_norm=gnorm, **HP)
        torch.cuda.synchronize()
        prev = ref_master
        ref_master, ref_state, ref_norm, _ = optim.optimizer_step(ref_master, g, ref_state, ohp, step)
        assert abs(gnorm.item() - ref_norm) <= 1e-6 * ref_norm, (gnorm.item(), ref_norm)
        masters, adam, buf = state_views(model, state, shapes)
        worst = []
        for n, _ in shapes:
            # compare the step's update from the oracle's previous masters
            e = rel_l2(masters[n] - prev[n], ref_master[n] - prev[n])
            tol = TOL_ADAMW if optim.is_adamw(n) else TOL_MUON[dt]
            worst.append((e, n))
            assert e < tol, (step, n, e)
            if optim.is_adamw(n):
                assert rel_l2(adam[n][0], ref_state["m"][n]) < 1e-6, (step, n)
                assert rel_l2(adam[n][1], ref_state["v"][n]) < 1e-6, (step, n)
            else:
                assert rel_l2(buf[n], ref_state["buf"][n]) < 1e-6, (step, n)
        print(f"step {step} |g| {gnorm.item():.6g} worst {max(worst)}", flush=True)
        # the model's parameters are the masters in its element type
        p = to_np(flat)
        m = pack(masters, shapes)
        want = synth.bf16_round(m) if dt == "bf16" else m.astype(np.float32)
        np.testing.assert_array_equal(p.astype(np.float32), want)
        # the next step starts from where the GPU stands (errors do not compound)
        ref_master = {n: masters[n].astype(np.float64) for n, _ in shapes}


def test_optim_deterministic_and_ns_steps_zero():
    banner("optimizer determinism, ns_steps=0 (tiny, bf16)")
    cfg = TINY
    shapes = oracle.param_shapes(cfg)
    model = model_for(cfg, "bf16")
    params = synth.weights(shapes, seed=8, bf16=True)
    g = to_dev(pack(grads_for(shapes, 5, 0.5), shapes))
    outs = []
    for _ in range(2):
        flat = to_dev(pack(params, shapes), "bf16")
        state, ws = buffers(model)
        model.optim_init(flat, state)
        model.optim_step(0, g, flat, state, ws, **HP)
        model.optim_step(1, g, flat, state, ws, **HP)
        torch.cuda.synchronize()
        outs.append((flat.clone(), state.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    # no Newton-Schulz iteration: the Muon update is the normalised Nesterov momentum itself
    hp0 = dict(HP, ns_steps=0, weight_decay=0.0)
    flat = to_dev(pack(params, shapes), "bf16")
    state, ws = buffers(model)
    model.optim_init(flat, state)
    model.optim_step(0, g, flat, state, ws, **hp0)
    torch.cuda.synchronize()
    masters, _, _ = state_views(model, state, shapes)
    ref, _, _, _ = optim.optimizer_step({n: np.asarray(params[n], np.float64) for n, _ in shapes},
                                        unpack(to_np(g), shapes), {"m": {}, "v": {}, "buf": {}},
                                        oracle_hp(hp0), 0)
    for n, _ in shapes:
        p0 = np.asarray(params[n], np.float64)
        assert rel_l2(masters[n] - p0, ref[n] - p0) < (TOL_ADAMW if optim.is_adamw(n) else 1e-2), n


def test_training_steps_lower_the_loss():
    # forward/backward, then the optimizer, on one fixed batch: the loss falls
    banner("fwd+bwd+optimizer loop (tiny, bf16)")
    cfg = TINY
    shapes = oracle.param_shapes(cfg)
    model = bwd_step_amd.Model(cfg.depth, vocab=cfg.vocab, seq_len=cfg.seq_len, max_batch=2, dtype="bf16",
                               d_model=cfg.d_model, n_heads=cfg.n_heads, head_dim=cfg.head_dim, d_ff=cfg.d_ff)
    params = synth.weights(shapes, seed=9, bf16=True)
    tok, tgt = synth.uniform_tokens(2, cfg.seq_len, cfg.vocab, seed=9)
    flat = to_dev(pack(params, shapes), "bf16")
    tok_d, tgt_d = to_dev(tok), to_dev(tgt)
    state, ws = buffers(model)
    model.optim_init(flat, state)
    loss = torch.empty((), dtype=torch.float32, device="cuda")
    grads = torch.empty(model.param_count, dtype=torch.float32, device="cuda")
    hp = dict(HP, warmup_steps=1, total_steps=100, final_frac=1.0)
    losses = []
    for step in range(6):
        model.forward_backward(flat, tok_d, tgt_d, loss, grads)
        losses.append(loss.item())
        model.optim_step(step, grads, flat, state, ws, **hp)
        assert model.check() == 0
    print(f"losses {losses}", flush=True)
    assert all(np.isfinite(losses))
    assert losses[-1] < losses[0] - 0.05, losses


def test_optim_full_depth20_sampled():
    # the depth-20 parameter set (561M parameters) at full size: global norm,
    # a block of embedding rows (AdamW) and two layer matrices (Muon), one
    # square and one tall, against the oracle in float64
    cfg = oracle.derive_config(20)
    banner("optimizer depth 20, full size, bf16")
    model = bwd_step_amd.Model(20, vocab=cfg.vocab, seq_len=cfg.seq_len, max_batch=1, dtype="bf16")
    lay = {n: (off, r, c) for n, off, r, c in model.layout()}
    P = model.param_count
    gen = torch.Generator(device="cuda").manual_seed(11)
    flat = (0.02 * torch.randn(P, generator=gen, device="cuda")).to(torch.bfloat16)
    grads = 1e-3 * torch.randn(P, generator=gen, device="cuda")
    state, ws = buffers(model)
    model.optim_init(flat, state)
    flat0 = flat.clone()  # the step rewrites flat
    gnorm = torch.empty((), dtype=torch.float32, device="cuda")
    hp = dict(HP, warmup_steps=1, total_steps=10)
    model.optim_step(0, grads, flat, state, ws, grad_norm=gnorm, **hp)
    torch.cuda.synchronize()
    g_host = grads.cpu().numpy()
    norm, s = optim.clip_scale(np.array_split(g_host, 64), hp["clip"])
    assert abs(gnorm.item() - norm) <= 1e-6 * norm, (gnorm.item(), norm)
    assert s < 1.0  # this gradient is clipped
    mult = optim.cosine_lr(0, 1.0, hp["warmup_steps"], hp["total_steps"], hp["final_frac"])

    def tensor(buf, name):
        off, r, c = lay[name]
        return to_np(buf[off:off + r * c]).reshape(r, c)

    # AdamW: embedding rows 1000..1255 (elementwise, so a block is exact)
    off, r, c = lay["E"]
    rows = slice(1000 * c, 1256 * c)
    w0 = to_np(flat0[off:off + r * c][rows])
    w1 = to_np(state[off:off + r * c][rows])
    ref, _, _ = optim.adamw_update(w0, g_host[off:off + r * c][rows].astype(np.float64) * s, 0.0, 0.0, 1,
                                   hp["lr_adamw"] * mult, hp["beta1"], hp["beta2"], hp["eps"],
                                   hp["weight_decay"])
    assert rel_l2(w1 - w0, ref - w0) < TOL_ADAMW
    # Muon: layer 7's W_o [1280, 1280] and W_1 [5120, 1280]
    for name in ("layers.7.W_o", "layers.7.W_1"):
        w0 = tensor(flat0, name)
        w1 = tensor(state, name)
        off, r, c = lay[name]
        g = g_host[off:off + r * c].reshape(r, c).astype(np.float64) * s
        ref, _ = optim.muon_update(w0, g, np.zeros((r, c)), hp["lr_muon"] * mult, hp["momentum"],
                                   hp["weight_decay"], hp["ns_steps"])
        e = rel_l2(w1 - w0, ref - w0)
        print(f"{name} update rel-L2 {e:.3g}", flush=True)
        assert e < TOL_MUON["bf16"], (name, e)
