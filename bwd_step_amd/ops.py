"""Operation-level wrappers over the C ABI (argument marshalling only).

Each function takes torch CUDA tensors, allocates the outputs and the
operation's workspace with torch, and calls the matching nc_* entry point on
the current stream.
"""

import ctypes

from ._nc import NC_BF16, check, lib


def _t():
    import torch
    return torch


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _s():
    return ctypes.c_void_p(_t().cuda.current_stream().cuda_stream)


def _code(t):
    torch = _t()
    if t.dtype == torch.bfloat16:
        return 0
    if t.dtype == torch.float32:
        return 1
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ws(nbytes):
    torch = _t()
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device="cuda")


def status(ws):
    """Read and clear the status word of an op workspace (synchronises)."""
    return int(lib().nc_op_status(_p(ws), _s()))


def rmsnorm_fwd(x, eps=1e-6, dtype=NC_BF16):
    torch = _t()
    N, d = x.shape
    y = torch.empty(N, d, dtype=torch.bfloat16 if dtype == NC_BF16 else torch.float32, device=x.device)
    r = torch.empty(N, dtype=torch.float32, device=x.device)
    check(lib().nc_rmsnorm_fwd(_p(x), _p(y), _p(r), N, d, eps, dtype, _s()), "nc_rmsnorm_fwd")
    return y, r


def rmsnorm_bwd(dy, y, r, dx=None, accumulate=False, want_lp=False):
    torch = _t()
    N, d = dy.shape
    if dx is None:
        dx = torch.empty(N, d, dtype=torch.float32, device=dy.device)
    lp = torch.empty_like(y) if want_lp else None
    check(lib().nc_rmsnorm_bwd(_p(dy), _p(y), _p(r), _p(dx), _p(lp), N, d, int(accumulate), _code(y), _s()),
          "nc_rmsnorm_bwd")
    return (dx, lp) if want_lp else dx


def embedding_fwd(E, tokens, ws=None):
    torch = _t()
    V, d = E.shape
    N = tokens.numel()
    x = torch.empty(N, d, dtype=torch.float32, device=E.device)
    ws = _ws(256) if ws is None else ws
    check(lib().nc_embedding_fwd(_p(E), _p(tokens), _p(x), N, d, V, _code(E), _p(ws), _s()), "nc_embedding_fwd")
    return x, ws


def embedding_bwd(dx, tokens, V, dE=None, accumulate=False):
    torch = _t()
    N, d = dx.shape
    if dE is None:
        dE = torch.empty(V, d, dtype=torch.float32, device=dx.device)
    nb = int(lib().nc_embedding_bwd_workspace_bytes(N, d, V))
    ws = _ws(nb)
    check(lib().nc_embedding_bwd(_p(dx), _p(tokens), _p(dE), N, d, V, int(accumulate), _p(ws), nb, _s()),
          "nc_embedding_bwd")
    return dE


def gemm(A, a_kmajor, B, b_kmajor, M, N, K, C=None, beta=0):
    """C[i,j] (+)= sum_k A(i,k) B(j,k); see nc_gemm in include/nc.h."""
    torch = _t()
    if C is None:
        C = torch.empty(M, N, dtype=torch.float32, device=A.device)
    dt = _code(A)
    nb = int(lib().nc_gemm_workspace_bytes(M, N, K, dt))
    ws = _ws(nb) if nb else None
    lda, ldb = A.shape[1], B.shape[1]
    check(lib().nc_gemm(_p(A), lda, int(a_kmajor), _p(B), ldb, int(b_kmajor), _p(C), C.shape[1], M, N, K,
                        int(beta), dt, _p(ws), nb, _s()), "nc_gemm")
    return C


def attention_fwd_bwd(q, k, v, dout, rope_base=10000.0, eps=1e-6, ws=None):
    """q, k, v, dout: [B, T, H, hd] (bf16 or fp32). Returns (out, dq, dk, dv).

    ws: an optional workspace of at least nc_attention_workspace_bytes (reused
    across calls, e.g. by a benchmark loop); one is allocated otherwise."""
    torch = _t()
    B, T, H, hd = q.shape
    dt = _code(q)
    out = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nb = int(lib().nc_attention_workspace_bytes(B, H, T, hd, dt))
    if ws is None or ws.numel() < nb:
        ws = _ws(nb)
    check(lib().nc_attention_fwd_bwd(_p(q), _p(k), _p(v), _p(dout), _p(out), _p(dq), _p(dk), _p(dv), B, H, T, hd,
                                     rope_base, eps, dt, _p(ws), nb, _s()), "nc_attention_fwd_bwd")
    return out, dq, dk, dv


def lmhead_ce_fwd_bwd(z, W, y, ws=None):
    """z: [N, d], W: [V, d], y: int32 [N].  Returns (loss, dz, dW, ws)."""
    torch = _t()
    N, d = z.shape
    V = W.shape[0]
    dt = _code(z)
    loss = torch.empty((), dtype=torch.float32, device=z.device)
    dz = torch.empty(N, d, dtype=torch.float32, device=z.device)
    dW = torch.empty(V, d, dtype=torch.float32, device=z.device)
    nb = int(lib().nc_lmhead_ce_workspace_bytes(N, d, V, dt))
    if ws is None or ws.numel() < nb:
        ws = _ws(nb)
    check(lib().nc_lmhead_ce_fwd_bwd(_p(z), _p(W), _p(y), N, d, V, _p(loss), _p(dz), _p(dW), dt, _p(ws), nb, _s()),
          "nc_lmhead_ce_fwd_bwd")
    return loss, dz, dW, ws
