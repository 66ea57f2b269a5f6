"""GPU check of nc_decode_static, the decode step that allocates nothing
(its scratch is a static device array of the library).

It runs the same kernels as nc_decode, so its logits and cache writes must
equal nc_decode's bitwise; checked on two calls in a row, the second with
fewer sequences (the array keeps the first call's contents), plus the
status word of an out-of-range position and the host-side size limit.
"""

import ctypes

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
from bwd_step_amd import lib  # noqa: E402

CFG = oracle.derive_config(3, vocab=576, seq_len=100, d_model=192, n_heads=3, head_dim=64, d_ff=320)
P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731


def decode_static(model, flat, tok, pos, cache, max_len, logits, status):
    model.set_stream()
    return lib().nc_decode_static(model._h, P(flat), P(tok), P(pos), tok.shape[0], P(cache), max_len, P(logits),
                                  P(status))


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_decode_static_matches_decode(dt):
    banner(f"nc_decode_static against nc_decode, {dt}")
    B, Tp, max_len = 4, 29, 100
    shapes = oracle.param_shapes(CFG)
    params = synth.weights(shapes, seed=40, bf16=(dt == "bf16"))
    tok, _ = synth.uniform_tokens(B, CFG.seq_len, CFG.vocab, seed=40)
    model = bwd_step_amd.Model(CFG.depth, vocab=CFG.vocab, seq_len=CFG.seq_len, max_batch=B, dtype=dt,
                               d_model=CFG.d_model, n_heads=CFG.n_heads, head_dim=CFG.head_dim, d_ff=CFG.d_ff)
    flat = to_dev(pack(params, shapes), dt)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    es = 2 if dt == "bf16" else 4
    cache = torch.zeros(model.kv_cache_bytes(B, max_len) // es, dtype=tdt, device="cuda")
    logits = torch.empty(B, CFG.vocab, dtype=torch.float32, device="cuda")
    model.prefill(flat, to_dev(np.ascontiguousarray(tok[:, :Tp])), cache, B, max_len, logits)
    assert model.check() == 0
    ref = oracle.forward_logits(CFG, params, tok[:, :Tp + 1])
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for nb in (B, 2):  # the second call has fewer sequences than the first
        c_ws = cache[: model.kv_cache_bytes(nb, max_len) // es].clone()
        c_st = c_ws.clone()
        ws = torch.zeros(model.decode_workspace_bytes(nb, max_len), dtype=torch.uint8, device="cuda")
        t_d = to_dev(np.ascontiguousarray(tok[:nb, Tp]))
        pos = torch.full((nb,), Tp, dtype=torch.int32, device="cuda")
        out_ws = torch.empty(nb, CFG.vocab, dtype=torch.float32, device="cuda")
        out_st = torch.full((nb, CFG.vocab), float("nan"), dtype=torch.float32, device="cuda")
        model.decode(flat, t_d, pos, c_ws, max_len, ws, out_ws)
        status.fill_(7)  # the call clears it
        assert decode_static(model, flat, t_d, pos, c_st, max_len, out_st, status) == 0
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert bwd_step_amd.ops.status(ws) == 0
        assert torch.equal(out_ws, out_st), f"batch {nb}: logits differ"
        assert torch.equal(c_ws, c_st), f"batch {nb}: cache writes differ"
        if nb == B:
            # the cache slots of B sequences are laid out [slot][head][pos]; a
            # smaller batch views the first slots, so compare against the
            # oracle on the full batch only
            err = max(rel_l2(to_np(out_st[b]), ref[b, Tp]) for b in range(nb))
            print(f"batch {nb}: worst logits rel-L2 vs oracle {err:.3g}", flush=True)
            assert err < (2e-2 if dt == "bf16" else 1e-4)


def test_decode_static_status_and_size_limit():
    banner("nc_decode_static: out-of-range position status, scratch size limit")
    B, max_len = 2, 64
    shapes = oracle.param_shapes(CFG)
    params = synth.weights(shapes, seed=41, bf16=True)
    model = bwd_step_amd.Model(CFG.depth, vocab=CFG.vocab, seq_len=CFG.seq_len, max_batch=B, dtype="bf16",
                               d_model=CFG.d_model, n_heads=CFG.n_heads, head_dim=CFG.head_dim, d_ff=CFG.d_ff)
    flat = to_dev(pack(params, shapes), "bf16")
    cache = torch.zeros(model.kv_cache_bytes(B, max_len) // 2, dtype=torch.bfloat16, device="cuda")
    logits = torch.empty(B, CFG.vocab, dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    t_d = torch.tensor([1, 2], dtype=torch.int32, device="cuda")
    pos = torch.tensor([3, max_len], dtype=torch.int32, device="cuda")  # the second is past the cache
    assert decode_static(model, flat, t_d, pos, cache, max_len, logits, status) == 0
    torch.cuda.synchronize()
    assert int(status.item()) == 1
    pos = torch.tensor([3, 4], dtype=torch.int32, device="cuda")
    assert decode_static(model, flat, t_d, pos, cache, max_len, logits, status) == 0
    torch.cuda.synchronize()
    assert int(status.item()) == 0  # cleared by the call
    # a step that needs more than the static array is refused before any launch
    big = model.decode_workspace_bytes(64, 65536)
    assert big > bwd_step_amd._nc.DECODE_SCRATCH_BYTES
    assert decode_static(model, flat, torch.zeros(64, dtype=torch.int32, device="cuda"),
                         torch.zeros(64, dtype=torch.int32, device="cuda"), cache, 65536,
                         torch.empty(64, CFG.vocab, device="cuda"), status) == 3
