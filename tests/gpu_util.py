"""Helpers for the GPU parity tests (imported by tests only; not a test module)."""

import numpy as np

import synth


def torch_dtype(name):
    import torch
    return torch.bfloat16 if name == "bf16" else torch.float32


def prep(x, name):
    """Input values as the GPU path sees them (bf16 inputs are pre-rounded)."""
    x = np.asarray(x, dtype=np.float32)
    return synth.bf16_round(x) if name == "bf16" else x


def to_dev(x, name=None, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is None and name is not None:
        dtype = torch_dtype(name)
    return t.to("cuda", dtype=dtype) if dtype is not None else t.to("cuda")


def to_np(t):
    import torch
    return t.detach().to("cpu", dtype=torch.float64).numpy() if t.is_floating_point() else t.cpu().numpy()


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def pack(params, shapes):
    """Flat parameter vector in the documented order (E, per-layer W_qkv, W_o, W_1, W_2, W_lm)."""
    return np.concatenate([np.asarray(params[n], dtype=np.float32).reshape(-1) for n, _ in shapes])


def unpack(flat, shapes):
    out, off = {}, 0
    for n, s in shapes:
        k = int(np.prod(s))
        out[n] = flat[off:off + k].reshape(s)
        off += k
    return out


def banner(msg):
    print(f"\n[gpu] {msg}", flush=True)
