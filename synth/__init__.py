"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

Holds none of the model's arithmetic: only random draws, the token-id
distributions and the round-to-bfloat16 used to prepare inputs.  Every draw
comes from a numpy PCG64 stream keyed by (seed, stream id), so each tensor is
reproducible on its own regardless of which other tensors are drawn.

Workload shapes follow the pages' model family: ids < 65536 (a 2^16
vocabulary), sequences of 2048 positions, weights ~ N(0, 0.02).
"""

import numpy as np

# stream ids: parameters use 1000 + their index in the ordered parameter list
STREAM_TOKENS = 1
STREAM_UPSTREAM = 2
STREAM_HIDDEN = 3
STREAM_Q, STREAM_K, STREAM_V, STREAM_DO = 11, 12, 13, 14
STREAM_PARAM_BASE = 1000


def rng(seed, stream):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def bf16_round(x):
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    NaN and infinities are not expected in synthetic inputs and are not handled.
    """
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32)
    r = u + np.uint32(0x7FFF)
    r += (u >> np.uint32(16)) & np.uint32(1)
    r &= np.uint32(0xFFFF0000)
    return r.view(np.float32).reshape(a.shape)


def normal(shape, seed, stream, std=1.0):
    return (rng(seed, stream).standard_normal(size=shape, dtype=np.float32) * np.float32(std))


def weights(shapes, seed=0, std=0.02, bf16=False):
    """Dict name -> float32 array ~ N(0, std); shapes is an ordered (name, shape) list."""
    out = {}
    for i, (name, shape) in enumerate(shapes):
        w = normal(shape, seed, STREAM_PARAM_BASE + i, std)
        out[name] = bf16_round(w) if bf16 else w
    return out


def uniform_tokens(B, T, V, seed=0, stream=STREAM_TOKENS):
    """Draw B x (T+1) ids uniform in [0, V); return (tokens, targets) shifted by one."""
    ids = rng(seed, stream).integers(0, V, size=(B, T + 1), dtype=np.int64).astype(np.int32)
    return np.ascontiguousarray(ids[:, :-1]), np.ascontiguousarray(ids[:, 1:])


def zipf_probs(V, s=1.1):
    """p(id) proportional to (id + 1)^(-s) for id in [0, V), truncated to V."""
    k = np.arange(1, V + 1, dtype=np.float64)
    w = k ** (-s)
    return w / w.sum()


def zipf_tokens(B, T, V, s=1.1, seed=0, stream=STREAM_TOKENS):
    """Zipf(s) ids truncated to [0, V), by inverse CDF in float64; shifted by one."""
    cdf = np.cumsum(zipf_probs(V, s))
    cdf[-1] = 1.0
    u = rng(seed, stream).random(size=(B, T + 1))
    ids = np.searchsorted(cdf, u, side="right").astype(np.int32)
    ids = np.minimum(ids, V - 1)
    return np.ascontiguousarray(ids[:, :-1]), np.ascontiguousarray(ids[:, 1:])


def upstream(shape, seed=0, stream=STREAM_UPSTREAM):
    """An upstream gradient ~ N(0, 1) for op-level backward checks."""
    return normal(shape, seed, stream)
