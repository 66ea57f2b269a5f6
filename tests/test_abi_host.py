"""CPU tests of the C-ABI boundary: the library loads, exports every symbol
include/nc.h declares, and validates configurations and arguments on the host
(before any GPU work), with the depth dial and parameter layout the pages fix.
No compute call is made here.
"""

import ctypes
import os
import re

import pytest

import oracle
from bwd_step_amd import _nc
from bwd_step_amd._nc import NcConfig, lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nc.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_nc.LIB_PATH), reason="libnc.so not built")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nc_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound():
    names = header_functions()
    assert len(names) >= 20
    l = lib()
    for n in names:
        assert hasattr(l, n), n
    assert sorted(_nc.SIGNATURES) == names


def make(depth=2, **kw):
    args = dict(depth=depth, d_model=0, n_heads=0, head_dim=0, d_ff=0, vocab=512, seq_len=64, max_batch=2,
                rope_base=0.0, norm_eps=0.0, dtype=0)
    args.update(kw)
    return NcConfig(**args)


def init(cfg):
    h = ctypes.c_void_p()
    rc = lib().nc_init(ctypes.byref(cfg), None, ctypes.byref(h))
    return rc, h


def test_depth_dial_resolution():
    rc, h = init(make(depth=20, vocab=65536, seq_len=2048))
    assert rc == 0
    out = NcConfig()
    assert lib().nc_get_config(h, ctypes.byref(out)) == 0
    assert (out.d_model, out.n_heads, out.head_dim, out.d_ff) == (1280, 10, 128, 5120)
    assert out.rope_base == 10000.0 and out.norm_eps == pytest.approx(1e-6)
    assert lib().nc_param_count(h) == 560_988_160
    lib().nc_destroy(h)


@pytest.mark.parametrize("kw,code", [
    (dict(depth=0), 1),
    (dict(d_model=100), 1),
    (dict(head_dim=24, d_model=128, n_heads=2), 1),
    (dict(head_dim=48, d_model=192, n_heads=4, dtype=1), 1),
    (dict(vocab=500), 1),
    (dict(seq_len=0), 1),
    (dict(max_batch=0), 1),
    (dict(dtype=5), 1),
    (dict(head_dim=32, n_heads=4, d_model=128), 7),  # bf16 attention kernels: hd 64 or 128
])
def test_init_rejects_bad_configs(kw, code):
    rc, h = init(make(**kw))
    assert rc == code
    assert not h.value


def test_init_null_pointers():
    h = ctypes.c_void_p()
    assert lib().nc_init(None, None, ctypes.byref(h)) == 2
    assert lib().nc_init(ctypes.byref(make()), None, None) == 2


def test_fp32_accepts_small_power_of_two_head_dims():
    rc, h = init(make(head_dim=32, n_heads=4, d_model=128, dtype=1))
    assert rc == 0
    lib().nc_destroy(h)


def test_layout_matches_oracle_order_and_shapes():
    rc, h = init(make(depth=3, d_model=128, n_heads=2, head_dim=64, d_ff=512))
    assert rc == 0
    n = lib().nc_param_layout(h, None, 0)
    arr = (_nc.NcTensorDesc * n)()
    assert lib().nc_param_layout(h, arr, n) == n
    cfg = oracle.derive_config(3, vocab=512, seq_len=64, d_model=128, n_heads=2, head_dim=64, d_ff=512)
    shapes = oracle.param_shapes(cfg)
    assert n == len(shapes)
    off = 0
    for a, (name, shape) in zip(arr, shapes):
        assert a.name.decode() == name
        assert (a.rows, a.cols) == shape
        assert a.offset == off
        off += shape[0] * shape[1]
    assert lib().nc_param_count(h) == off == oracle.param_count(cfg)
    lib().nc_destroy(h)


def test_workspace_sizes_and_host_errors():
    rc, h = init(make())
    assert rc == 0
    assert lib().nc_workspace_bytes(h, 1) > 0
    assert lib().nc_workspace_bytes(h, 2) > lib().nc_workspace_bytes(h, 1)
    assert lib().nc_workspace_bytes(h, 0) == 0
    assert lib().nc_workspace_bytes(h, 3) == 0  # above max_batch
    fake = ctypes.c_void_p(0x1000)
    # no workspace attached: rejected on the host
    assert lib().nc_forward_backward(h, fake, fake, fake, 1, fake, fake, 0) == 3
    assert lib().nc_forward_backward(h, None, fake, fake, 1, fake, fake, 0) == 2
    assert lib().nc_forward_backward(h, fake, fake, fake, 3, fake, fake, 0) == 8
    assert lib().nc_forward_backward(h, fake, fake, fake, 1, fake, fake, 2) == 8
    assert lib().nc_forward_logits(h, fake, fake, 0, fake) == 8
    # gradient accumulation: no workspace yet, then bad counts
    assert lib().nc_forward_backward_accum(h, fake, fake, fake, 2, 1, fake, fake) == 3
    assert lib().nc_forward_backward_accum(h, fake, fake, fake, 0, 1, fake, fake) == 8
    assert lib().nc_forward_backward_accum(h, fake, fake, fake, 2, 3, fake, fake) == 8
    assert lib().nc_forward_backward_accum(h, fake, None, fake, 2, 1, fake, fake) == 2
    assert lib().nc_set_workspace(h, ctypes.c_void_p(0x1001), 4096) == 8  # misaligned
    lib().nc_destroy(h)


def test_op_argument_validation():
    fake = ctypes.c_void_p(0x1000)
    # contiguous dimension not a multiple of 8
    assert lib().nc_gemm(fake, 12, 1, fake, 12, 1, fake, 16, 16, 16, 12, 0, 0, None, 0, None) == 8
    assert lib().nc_gemm(None, 16, 1, fake, 16, 1, fake, 16, 16, 16, 16, 0, 0, None, 0, None) == 2
    assert lib().nc_attention_fwd_bwd(*([fake] * 8), 1, 2, 16, 32, 10000.0, 1e-6, 0, fake, 1 << 20, None) == 7
    assert lib().nc_attention_fwd_bwd(*([fake] * 8), 1, 2, 16, 64, 10000.0, 1e-6, 0, fake, 16, None) == 3
    assert lib().nc_lmhead_ce_fwd_bwd(fake, fake, fake, 0, 64, 64, fake, fake, fake, 0, fake, 1 << 20, None) == 8
    assert lib().nc_rmsnorm_fwd(fake, fake, fake, 4, 6, 1e-6, 0, None) == 8
    assert lib().nc_embedding_bwd(fake, fake, fake, 4, 8, 16, 0, fake, 0, None) == 3
    assert lib().nc_attention_workspace_bytes(2, 2, 64, 64, 0) > 0
    assert lib().nc_lmhead_ce_workspace_bytes(100, 64, 512, 0) > 0


def test_strerror_covers_codes():
    for c in range(9):
        assert lib().nc_strerror(c)
    assert lib().nc_strerror(99) == b"unknown status"


def test_optim_sizes_and_host_errors():
    cfg = make()
    rc, h = init(cfg)
    assert rc == 0
    P = lib().nc_param_count(h)
    n_e = n_lm = 512 * 128
    # masters, AdamW moments (2x) of E and W_lm, Muon momentum (1x) of the rest
    assert lib().nc_optim_state_bytes(h) == 4 * (2 * P + n_e + n_lm)
    assert lib().nc_optim_state_bytes(None) == 0 and lib().nc_optim_workspace_bytes(None) == 0
    need = lib().nc_optim_workspace_bytes(h)
    assert need > 0
    fake = ctypes.c_void_p(0x1000)
    good = dict(lr_adamw=3e-3, lr_muon=0.02, beta1=0.9, beta2=0.95, eps=1e-8, momentum=0.95, weight_decay=0.1,
                clip=1.0, final_frac=0.0, warmup_steps=1, total_steps=10, ns_steps=5)

    def step(step_=0, ws=need, null=None, **over):
        c = _nc.NcOptimConfig(**dict(good, **over))
        args = [h, ctypes.byref(c), step_, fake, fake, fake, fake, ws, None]
        if null is not None:
            args[null] = None
        return lib().nc_optim_step(*args)

    # every case is rejected on the host, before anything is enqueued
    assert step(ws=need - 1) == 3
    assert step(step_=-1) == 8
    for bad in (dict(beta1=1.0), dict(beta2=-0.1), dict(eps=0.0), dict(momentum=1.0), dict(clip=0.0),
                dict(final_frac=1.5), dict(warmup_steps=0), dict(total_steps=0), dict(ns_steps=-1),
                dict(lr_muon=-1.0), dict(weight_decay=-0.1)):
        assert step(**bad) == 8, bad
    for i in (0, 1, 3, 4, 5, 6):
        assert step(null=i) == 2, i
    c = _nc.NcOptimConfig(**good)
    odd = ctypes.c_void_p(0x1008)  # 8-byte aligned only
    assert lib().nc_optim_step(h, ctypes.byref(c), 0, odd, fake, fake, fake, need, None) == 8
    assert lib().nc_optim_step(h, ctypes.byref(c), 0, fake, fake, odd, fake, need, None) == 8
    assert lib().nc_optim_init(h, None, fake) == 2
    assert lib().nc_optim_init(h, fake, None) == 2
    lib().nc_destroy(h)


def test_kv_cache_size_matches_the_pages_example():
    # "nanochat explainer", Inference & KV Cache: 16 layers, 16 heads, head
    # dim 64, sequence 2048 hold 128 MB of keys and values (bf16, one sequence)
    g = {}
    for line in open(os.path.join(ROOT, "tests", "golden", "kv_cache_size.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            g[k] = int(v)
    rc, h = init(make(depth=g["layers"], d_model=g["heads"] * g["head_dim"], n_heads=g["heads"],
                      head_dim=g["head_dim"], vocab=512, seq_len=g["seq"]))
    assert rc == 0
    assert lib().nc_kv_cache_bytes(h, 1, g["seq"]) == g["mha_bytes"]
    assert lib().nc_kv_cache_bytes(h, 3, g["seq"]) == 3 * g["mha_bytes"]
    assert lib().nc_kv_cache_bytes(h, 0, g["seq"]) == 0
    assert lib().nc_kv_cache_bytes(h, 1, 70000) == 0
    assert lib().nc_decode_workspace_bytes(h, 4, 2048) > 0
    rc, hm = init(make(depth=g["layers"], d_model=g["heads"] * g["head_dim"], n_heads=g["heads"],
                       head_dim=g["head_dim"], vocab=512, seq_len=g["seq"], n_kv_heads=g["mqa_kv_heads"]))
    assert rc == 0
    assert lib().nc_kv_cache_bytes(hm, 1, g["seq"]) == g["mqa_bytes"]
    assert g["mha_bytes"] == 16 * g["mqa_bytes"]
    lib().nc_destroy(hm)
    fake = ctypes.c_void_p(0x1000)
    # prefill: len beyond seq_len, slots beyond the cache, no workspace
    assert lib().nc_prefill(h, fake, fake, 1, g["seq"] + 1, fake, 1, g["seq"] + 1, 0, fake) == 8
    assert lib().nc_prefill(h, fake, fake, 2, 16, fake, 2, 64, 1, fake) == 8
    assert lib().nc_prefill(h, fake, fake, 1, 16, fake, 1, 64, 0, fake) == 3
    assert lib().nc_prefill(h, None, fake, 1, 16, fake, 1, 64, 0, fake) == 2
    # decode: workspace too small or misaligned
    need = lib().nc_decode_workspace_bytes(h, 2, 64)
    assert lib().nc_decode(h, fake, fake, fake, 2, fake, 64, fake, need - 1, fake) == 3
    assert lib().nc_decode(h, fake, fake, fake, 2, fake, 64, ctypes.c_void_p(0x1010), need, fake) == 8
    assert lib().nc_decode(h, fake, fake, None, 2, fake, 64, fake, need, fake) == 2
    lib().nc_destroy(h)


def test_grouped_query_layout_and_config_checks():
    cfg = oracle.derive_config(2, vocab=512, seq_len=64, d_model=256, n_heads=4, head_dim=64, d_ff=512, n_kv_heads=2)
    rc, h = init(make(depth=2, d_model=256, n_heads=4, head_dim=64, d_ff=512, n_kv_heads=2))
    assert rc == 0
    out = NcConfig()
    assert lib().nc_get_config(h, ctypes.byref(out)) == 0
    assert out.n_kv_heads == 2
    n = lib().nc_param_layout(h, None, 0)
    arr = (_nc.NcTensorDesc * n)()
    lib().nc_param_layout(h, arr, n)
    assert [(a.name.decode(), a.rows, a.cols) for a in arr] == [(k, r, c) for k, (r, c) in oracle.param_shapes(cfg)]
    assert lib().nc_param_count(h) == oracle.param_count(cfg)
    lib().nc_destroy(h)
    # n_kv_heads must divide n_heads; 0 means n_heads
    assert init(make(depth=2, d_model=256, n_heads=4, head_dim=64, n_kv_heads=3))[0] == 1
    rc, h = init(make(depth=2, d_model=256, n_heads=4, head_dim=64))
    out = NcConfig()
    lib().nc_get_config(h, ctypes.byref(out))
    assert out.n_kv_heads == 4
    lib().nc_destroy(h)


def test_library_binds_to_torchs_hip_runtime():
    # loading libnc.so before torch would bind it to another libamdhip64 than
    # the one torch's streams and allocations belong to; lib() imports torch first
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from bwd_step_amd import _nc\n"
            "_nc.lib()\n"
            "print(len({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))\n" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"
