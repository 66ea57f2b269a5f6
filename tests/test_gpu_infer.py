"""GPU parity of inference with a KV cache (nc_prefill, nc_decode).

The oracle of decoding is the definition itself: the logits a token gets
from the cache equal the forward logits at its position of the whole
sequence (oracle.forward_logits, whose causality is pinned bitwise in
tests/test_oracle_model.py).  Tolerance on each logits row, relative L2:
1e-4 on the fp32 path, 2e-2 on the bf16 path (as for nc_forward_logits).
"""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import banner, pack, rel_l2, to_dev, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import bwd_step_amd  # noqa: E402
from bwd_step_amd import ops  # noqa: E402

TOL = {"fp32": 1e-4, "bf16": 2e-2}
TINY = oracle.derive_config(2, vocab=512, seq_len=64, d_model=128, n_heads=2, head_dim=64, d_ff=512)
RAGGED = oracle.derive_config(3, vocab=576, seq_len=100, d_model=192, n_heads=3, head_dim=64, d_ff=320)
SMALLHD = oracle.derive_config(2, vocab=256, seq_len=48, d_model=64, n_heads=2, head_dim=32, d_ff=128)


def setup(cfg, B, dt, seed):
    shapes = oracle.param_shapes(cfg)
    params = synth.weights(shapes, seed=seed, bf16=(dt == "bf16"))
    tok, _ = synth.uniform_tokens(B, cfg.seq_len, cfg.vocab, seed=seed)
    model = bwd_step_amd.Model(cfg.depth, vocab=cfg.vocab, seq_len=cfg.seq_len, max_batch=B, dtype=dt,
                               d_model=cfg.d_model, n_heads=cfg.n_heads, head_dim=cfg.head_dim, d_ff=cfg.d_ff)
    return model, params, to_dev(pack(params, shapes), dt), tok


def buffers(model, B, max_len, dt):
    es = 2 if dt == "bf16" else 4
    cache = torch.zeros(model.kv_cache_bytes(B, max_len) // es, dtype=torch.bfloat16 if dt == "bf16" else
                        torch.float32, device="cuda")
    ws = torch.zeros(model.decode_workspace_bytes(B, max_len), dtype=torch.uint8, device="cuda")  # status word 0
    return cache, ws


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
@pytest.mark.parametrize("which,B,Tp,steps,max_len", [("tiny", 2, 20, 6, 64), ("ragged", 3, 37, 9, 300),
                                                      ("smallhd", 2, 5, 4, 48)])
def test_prefill_then_decode_matches_forward(dt, which, B, Tp, steps, max_len):
    cfg = {"tiny": TINY, "ragged": RAGGED, "smallhd": SMALLHD}[which]
    if which == "smallhd" and dt == "bf16":
        pytest.skip("the bf16 training kernels (used by prefill) take head_dim 64 or 128")
    banner(f"prefill {Tp} + decode {steps} {which} {dt} B={B} max_len={max_len}")
    model, params, flat, tok = setup(cfg, B, dt, seed=30)
    ref = oracle.forward_logits(cfg, params, tok[:, : Tp + steps])
    cache, ws = buffers(model, B, max_len, dt)
    logits = torch.empty(B, cfg.vocab, dtype=torch.float32, device="cuda")
    model.prefill(flat, to_dev(np.ascontiguousarray(tok[:, :Tp])), cache, B, max_len, logits)
    assert model.check() == 0
    worst = max(rel_l2(to_np(logits)[b], ref[b, Tp - 1]) for b in range(B))
    assert worst < TOL[dt], ("prefill", worst)
    for k in range(steps):
        t = Tp + k
        model.decode(flat, to_dev(np.ascontiguousarray(tok[:, t])), to_dev(np.full(B, t, np.int32)), cache,
                     max_len, ws, logits)
        assert ops.status(ws) == 0
        e = max(rel_l2(to_np(logits)[b], ref[b, t]) for b in range(B))
        worst = max(worst, e)
        assert e < TOL[dt], (t, e)
    print(f"worst logits rel-L2 {worst:.3g}", flush=True)


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
def test_ragged_positions_and_slots(dt):
    # two sequences prefilled separately into slots 0 and 1 with different
    # lengths, then decoded together at different positions
    cfg = TINY
    banner(f"ragged positions {dt}")
    model, params, flat, tok = setup(cfg, 2, dt, seed=31)
    lens = [11, 30]
    max_len = 64
    cache, ws = buffers(model, 2, max_len, dt)
    logits = torch.empty(2, cfg.vocab, dtype=torch.float32, device="cuda")
    one = torch.empty(1, cfg.vocab, dtype=torch.float32, device="cuda")
    for b, L in enumerate(lens):
        model.prefill(flat, to_dev(np.ascontiguousarray(tok[b:b + 1, :L])), cache, 2, max_len, one, slot0=b)
        assert model.check() == 0
    refs = [oracle.forward_logits(cfg, params, tok[b:b + 1, : lens[b] + 5])[0] for b in range(2)]
    for k in range(5):
        pos = np.array([lens[0] + k, lens[1] + k], np.int32)
        model.decode(flat, to_dev(np.array([tok[0, pos[0]], tok[1, pos[1]]], np.int32)), to_dev(pos), cache,
                     max_len, ws, logits)
        assert ops.status(ws) == 0
        for b in range(2):
            e = rel_l2(to_np(logits)[b], refs[b][pos[b]])
            assert e < TOL[dt], (k, b, e)


def test_decode_position_out_of_range_sets_status():
    banner("decode at a position beyond the cache")
    model, params, flat, tok = setup(TINY, 1, "bf16", seed=32)
    cache, ws = buffers(model, 1, 16, "bf16")
    logits = torch.empty(1, TINY.vocab, dtype=torch.float32, device="cuda")
    model.decode(flat, to_dev(tok[:, 0].copy()), to_dev(np.array([16], np.int32)), cache, 16, ws, logits)
    assert ops.status(ws) == 4
    assert ops.status(ws) == 0


def test_decode_batch_above_one_pass_of_skinny_rows():
    # 20 sequences: the skinny products run their rows in two passes (16 + 4)
    cfg = TINY
    banner("decode with 20 sequences (bf16)")
    B, Tp, max_len = 20, 7, 32
    model, params, flat, tok = setup(cfg, B, "bf16", seed=33)
    ref = oracle.forward_logits(cfg, params, tok[:, : Tp + 2])
    cache, ws = buffers(model, B, max_len, "bf16")
    logits = torch.empty(B, cfg.vocab, dtype=torch.float32, device="cuda")
    model.prefill(flat, to_dev(np.ascontiguousarray(tok[:, :Tp])), cache, B, max_len, logits)
    for k in range(2):
        t = Tp + k
        model.decode(flat, to_dev(np.ascontiguousarray(tok[:, t])), to_dev(np.full(B, t, np.int32)), cache,
                     max_len, ws, logits)
        assert ops.status(ws) == 0
        e = max(rel_l2(to_np(logits)[b], ref[b, t]) for b in range(B))
        assert e < TOL["bf16"], (t, e)


def test_decode_full_depth20_matches_oracle_and_graph_replay():
    # depth 20 at full width: a 300-token prompt, then 3 decoded tokens,
    # against the oracle's forward logits of the whole 303-token sequence;
    # then the same decode step captured in a HIP graph and replayed
    cfg = oracle.derive_config(20)
    banner("depth 20: prefill 300 + decode 3 (bf16) vs oracle; graph replay")
    shapes = oracle.param_shapes(cfg)
    params = synth.weights(shapes, seed=34, bf16=True)
    tok, _ = synth.uniform_tokens(1, 303, cfg.vocab, seed=34)
    model = bwd_step_amd.Model(20, vocab=cfg.vocab, seq_len=cfg.seq_len, max_batch=1, dtype="bf16")
    flat = to_dev(pack(params, shapes), "bf16")
    max_len = 2048
    cache, ws = buffers(model, 1, max_len, "bf16")
    logits = torch.empty(1, cfg.vocab, dtype=torch.float32, device="cuda")
    model.prefill(flat, to_dev(np.ascontiguousarray(tok[:, :300])), cache, 1, max_len, logits)
    assert model.check() == 0
    out = [to_np(logits)[0]]
    for t in (300, 301, 302):
        model.decode(flat, to_dev(tok[:, t].copy()), to_dev(np.array([t], np.int32)), cache, max_len, ws, logits)
        assert ops.status(ws) == 0
        out.append(to_np(logits)[0])
    ref = oracle.forward_logits(cfg, params, tok)[0]
    for i, t in enumerate((299, 300, 301, 302)):
        e = rel_l2(out[i], ref[t])
        print(f"position {t}: logits rel-L2 {e:.3g}", flush=True)
        assert e < TOL["bf16"], (t, e)
    # graph capture of one decode step (position 302 again: same key and value rewritten)
    tk = to_dev(tok[:, 302].copy())
    ps = to_dev(np.array([302], np.int32))
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        model.set_stream(s)
        with torch.cuda.graph(g, stream=s):
            model.decode(flat, tk, ps, cache, max_len, ws, logits)
    model.set_stream()
    for _ in range(3):
        logits.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert rel_l2(to_np(logits)[0], out[3]) < 1e-6
