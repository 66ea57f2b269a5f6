"""GPU parity of each operation entry point against the float64 oracle.

Inputs are seeded (synth); bf16 inputs are pre-rounded so that both sides
consume identical values.  Tolerances: relative L2 3e-2 for bf16 gradients
(1e-2 for forward values), 1e-4 on the fp32 path, tighter where the
operation does no low-precision rounding.  Shapes span several tiles and
ragged tails.
"""

import numpy as np
import pytest

import synth
from oracle import ops as O
from gpu_util import banner, prep, rel_l2, to_dev, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import bwd_step_amd  # noqa: E402
from bwd_step_amd import ops  # noqa: E402

DTS = ["bf16", "fp32"]
CODE = {"bf16": 0, "fp32": 1}


# ------------------------------------------------------------------ RMSNorm
@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("N,d", [(300, 1280), (7, 128), (33, 1664)])
def test_rmsnorm_fwd_bwd(dt, N, d):
    banner(f"rmsnorm {dt} N={N} d={d}")
    eps = 1e-6
    x = synth.normal((N, d), 0, 21) * 3.0
    y, r = ops.rmsnorm_fwd(to_dev(x), eps, CODE[dt])
    yo, ro = O.rmsnorm(x.astype(np.float64), eps)
    assert rel_l2(to_np(r), ro) < 1e-6
    assert rel_l2(to_np(y), yo) < (4e-3 if dt == "bf16" else 1e-6)
    # backward on identical inputs: y in the path's element type, r fp32
    dy = synth.normal((N, d), 0, 22)
    y_in = prep(yo, dt)
    r_in = ro.astype(np.float32)
    dxo = O.rmsnorm_bwd(dy.astype(np.float64), y_in.astype(np.float64), r_in.astype(np.float64))
    dx, lp = ops.rmsnorm_bwd(to_dev(dy), to_dev(y_in, dt), to_dev(r_in), want_lp=True)
    assert rel_l2(to_np(dx), dxo) < 1e-5
    assert rel_l2(to_np(lp), dxo) < (4e-3 if dt == "bf16" else 1e-5)
    base = synth.normal((N, d), 0, 23)
    dx2 = ops.rmsnorm_bwd(to_dev(dy), to_dev(y_in, dt), to_dev(r_in), dx=to_dev(base), accumulate=True)
    assert rel_l2(to_np(dx2), dxo + base) < 1e-5


# ------------------------------------------------------------------ embedding
@pytest.mark.parametrize("dt", DTS)
def test_embedding_fwd_exact_and_range_status(dt):
    banner(f"embedding fwd {dt}")
    V, d, N = 1000, 256, 777
    E = prep(synth.normal((V, d), 0, 31), dt)
    tok, _ = synth.uniform_tokens(1, N, V, seed=3)
    x, ws = ops.embedding_fwd(to_dev(E, dt), to_dev(tok.reshape(-1)))
    assert ops.status(ws) == 0
    np.testing.assert_array_equal(to_np(x), E[tok.reshape(-1)].astype(np.float64))
    bad = tok.reshape(-1).copy()
    bad[5], bad[9] = -1, V
    x, ws = ops.embedding_fwd(to_dev(E, dt), to_dev(bad))
    assert ops.status(ws) == 4  # NC_ERR_TOKEN_RANGE, ids clamped, no fault
    assert ops.status(ws) == 0  # cleared by the read


@pytest.mark.parametrize("kind,V,d,N", [("uniform", 1000, 256, 777), ("zipf", 65536, 64, 5000),
                                        ("uniform", 65536, 1280, 4096)])
def test_embedding_bwd_matches_oracle_and_is_deterministic(kind, V, d, N):
    banner(f"embedding bwd {kind} V={V} d={d} N={N}")
    if kind == "uniform":
        tok, _ = synth.uniform_tokens(1, N, V, seed=4)
    else:
        tok, _ = synth.zipf_tokens(1, N, V, seed=4)
    tok = tok.reshape(-1)
    dx = synth.normal((N, d), 0, 32)
    ref = O.embedding_bwd(dx.astype(np.float64), tok, V)
    dE = ops.embedding_bwd(to_dev(dx), to_dev(tok), V)
    got = to_np(dE)
    assert rel_l2(got, ref) < 1e-6
    absent = np.setdiff1d(np.arange(V), tok)
    assert np.all(got[absent] == 0.0)
    again = to_np(ops.embedding_bwd(to_dev(dx), to_dev(tok), V))
    assert np.array_equal(got, again)  # bitwise reproducible
    base = synth.normal((V, d), 0, 33)
    acc = to_np(ops.embedding_bwd(to_dev(dx), to_dev(tok), V, dE=to_dev(base), accumulate=True))
    assert rel_l2(acc, ref + base) < 1e-6


# ------------------------------------------------------------------ GEMM
LAYOUTS = [(1, 1), (1, 0), (0, 1), (0, 0)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("ak,bk", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(296, 264, 200), (8, 8, 8), (512, 256, 64)])
def test_gemm_layouts(dt, ak, bk, M, N, K):
    banner(f"gemm {dt} ak={ak} bk={bk} {M}x{N}x{K}")
    A = prep(synth.normal((M, K), 1, 41), dt)
    B = prep(synth.normal((N, K), 1, 42), dt)
    Ast = A if ak else np.ascontiguousarray(A.T)
    Bst = B if bk else np.ascontiguousarray(B.T)
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    C = ops.gemm(to_dev(Ast, dt), ak, to_dev(Bst, dt), bk, M, N, K)
    assert rel_l2(to_np(C), ref) < 1e-5
    C0 = synth.normal((M, N), 1, 43)
    C1 = ops.gemm(to_dev(Ast, dt), ak, to_dev(Bst, dt), bk, M, N, K, C=to_dev(C0), beta=1)
    assert rel_l2(to_np(C1), ref + C0) < 1e-5


@pytest.mark.parametrize("ak,bk", [(0, 0), (1, 0)])
def test_gemm_split_k_bf16(ak, bk):
    # few output tiles and a long reduction: partial sums over K splits, reduced in order
    M, N, K = 256, 264, 8200
    banner(f"gemm split-K ak={ak} bk={bk} {M}x{N}x{K}")
    A = prep(synth.normal((M, K), 2, 41), "bf16")
    B = prep(synth.normal((N, K), 2, 42), "bf16")
    Ast = A if ak else np.ascontiguousarray(A.T)
    Bst = B if bk else np.ascontiguousarray(B.T)
    assert bwd_step_amd.lib().nc_gemm_workspace_bytes(M, N, K, 0) > 0
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    C = ops.gemm(to_dev(Ast, "bf16"), ak, to_dev(Bst, "bf16"), bk, M, N, K)
    assert rel_l2(to_np(C), ref) < 1e-5


@pytest.mark.parametrize("ak,bk", [(1, 1), (1, 0)])
@pytest.mark.parametrize("M,N,K", [(300, 520, 704), (4104, 4360, 640), (264, 264, 9280), (256, 392, 640)])
def test_gemm_pair_loop_bf16(ak, bk, M, N, K):
    # Both operands k-contiguous with K a multiple of 64 of at least 640: the
    # 64-deep pair loop (ak=1, bk=0 runs the 32-deep loop on the same shapes).
    # Ragged M and N (the last tile-row and tile-column are moved back inside
    # the operands and write only what the tile before them left); 306 tiles
    # (some workgroups run two, the second prefetched under the first);
    # K = 9280 splits over K into chunks of 1152 with a last chunk of one
    # pair; N = 392 moves the last tile-column back by 120 columns.
    banner(f"gemm pair loop ak={ak} bk={bk} {M}x{N}x{K}")
    A = prep(synth.normal((M, K), 2, 44), "bf16")
    B = prep(synth.normal((N, K), 2, 45), "bf16")
    Ast = A if ak else np.ascontiguousarray(A.T)
    Bst = B if bk else np.ascontiguousarray(B.T)
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    C = ops.gemm(to_dev(Ast, "bf16"), ak, to_dev(Bst, "bf16"), bk, M, N, K)
    assert rel_l2(to_np(C), ref) < 1e-5
    C0 = synth.normal((M, N), 1, 46)
    C1 = ops.gemm(to_dev(Ast, "bf16"), ak, to_dev(Bst, "bf16"), bk, M, N, K, C=to_dev(C0), beta=1)
    assert rel_l2(to_np(C1), ref + C0) < 1e-5


# ------------------------------------------------------------------ attention
def attention_oracle(q, k, v, do, base, eps):
    """q, k, v, do: [B, T, H, hd] float64 -> out, dq, dk, dv in the same layout."""
    tr = lambda a: np.ascontiguousarray(a.transpose(0, 2, 1, 3))
    q, k, v, do = tr(q), tr(k), tr(v), tr(do)
    T, hd = q.shape[2], q.shape[3]
    cos, sin = O.rope_angles(T, hd, base)
    qh, rq = O.qknorm_rope(q, cos, sin, eps)
    kh, rk = O.qknorm_rope(k, cos, sin, eps)
    o, _ = O.attention(qh, kh, v)
    dqh, dkh, dv = O.attention_bwd(do, qh, kh, v, o)
    dq = O.qknorm_rope_bwd(dqh, qh, rq, cos, sin)
    dk = O.qknorm_rope_bwd(dkh, kh, rk, cos, sin)
    return tr(o), tr(dq), tr(dk), tr(dv)


@pytest.mark.parametrize("dt,hd", [("bf16", 128), ("bf16", 64), ("fp32", 128), ("fp32", 32)])
# T = 300: a second, partial 256-query tile of the head_dim-128 dQ kernel;
# T = 513: one key past a 512 boundary (a nearly empty last block everywhere)
@pytest.mark.parametrize("B,H,T", [(2, 2, 200), (1, 3, 64), (1, 1, 1), (1, 2, 300), (1, 1, 513)])
def test_attention_fwd_bwd(dt, hd, B, H, T):
    banner(f"attention {dt} hd={hd} B={B} H={H} T={T}")
    shp = (B, T, H, hd)
    q, k, v, do = (prep(synth.normal(shp, 5, s), dt) for s in (synth.STREAM_Q, synth.STREAM_K,
                                                               synth.STREAM_V, synth.STREAM_DO))
    ref = attention_oracle(*(a.astype(np.float64) for a in (q, k, v, do)), 10000.0, 1e-6)
    got = ops.attention_fwd_bwd(*(to_dev(a, dt) for a in (q, k, v, do)))
    tol_o, tol_g = (1e-2, 3e-2) if dt == "bf16" else (1e-4, 1e-4)
    names = ["out", "dq", "dk", "dv"]
    for n, g, r in zip(names, got, ref):
        err = rel_l2(to_np(g), r)
        assert err < (tol_o if n == "out" else tol_g), (n, err)


@pytest.mark.timeout(900)
def test_attention_full_size_all_heads():
    # the attention microbenchmark shape; the oracle runs every one of the
    # 160 (b, h) pairs (one sequence at a time, all its heads together)
    B, H, T, hd = 16, 10, 2048, 128
    banner(f"attention bf16 full size B={B} H={H} T={T} hd={hd}, all {B * H} (b, h) pairs")
    shp = (B, T, H, hd)
    arrs = [prep(synth.normal(shp, 0, s), "bf16") for s in (synth.STREAM_Q, synth.STREAM_K,
                                                          synth.STREAM_V, synth.STREAM_DO)]
    got = [to_np(t) for t in ops.attention_fwd_bwd(*(to_dev(a, "bf16") for a in arrs))]
    worst = {n: 0.0 for n in ["out", "dq", "dk", "dv"]}
    for b in range(B):
        sub = [a[b:b + 1].astype(np.float64) for a in arrs]
        ref = attention_oracle(*sub, 10000.0, 1e-6)
        for h in range(H):
            for n, g, r in zip(["out", "dq", "dk", "dv"], got, ref):
                err = rel_l2(g[b:b + 1, :, h:h + 1], r[:, :, h:h + 1])
                worst[n] = max(worst[n], err)
                assert err < (1e-2 if n == "out" else 3e-2), (b, h, n, err)
    print("worst rel-L2 per output over the 160 pairs:", worst, flush=True)


# ------------------------------------------------------------------ LM head + CE
def ce_oracle(z, W, y):
    l = z @ W.T
    loss, lse = O.cross_entropy(l, y)
    g = O.cross_entropy_bwd(l, y, lse)
    return loss, g @ W, g.T @ z


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("N,d,V", [(300, 128, 1024), (16384 + 300, 64, 512), (200, 64, 576),
                                   (16384 + 700, 64, 1024)])
def test_lmhead_ce(dt, N, d, V):
    banner(f"lmhead_ce {dt} N={N} d={d} V={V}")
    z = prep(synth.normal((N, d), 6, synth.STREAM_HIDDEN), dt)
    W = prep(synth.normal((V, d), 6, 51, std=0.2), dt)
    y = synth.rng(6, 52).integers(0, V, N).astype(np.int32)
    lo, dzo, dWo = ce_oracle(z.astype(np.float64), W.astype(np.float64), y)
    loss, dz, dW, ws = ops.lmhead_ce_fwd_bwd(to_dev(z, dt), to_dev(W, dt), to_dev(y))
    assert ops.status(ws) == 0
    assert abs(loss.item() - lo) / lo < (1e-5 if dt == "fp32" else 1e-4)
    tol = 3e-2 if dt == "bf16" else 1e-4
    assert rel_l2(to_np(dz), dzo) < tol
    assert rel_l2(to_np(dW), dWo) < tol


def test_lmhead_ce_target_range_status():
    N, d, V = 64, 64, 512
    banner("lmhead_ce target out of range")
    z = prep(synth.normal((N, d), 7, 3), "bf16")
    W = prep(synth.normal((V, d), 7, 4, std=0.1), "bf16")
    y = np.zeros(N, dtype=np.int32)
    y[3] = V + 5
    _, _, _, ws = ops.lmhead_ce_fwd_bwd(to_dev(z, "bf16"), to_dev(W, "bf16"), to_dev(y))
    assert ops.status(ws) == 4


@pytest.mark.timeout(900)
def test_lmhead_ce_benchmark_shape():
    """The LM-head + cross-entropy microbenchmark shape: N 32768 x d 1280 x
    V 65536 in bf16 (z ~ N(0,1), W ~ N(0,0.02), uniform targets), three
    token chunks.  The oracle runs in chunks of 2048 rows (each chunk's
    softmax is the definition's; the mean over all N rows rescales each
    chunk's gradient): the loss, dz on every row, dW on 320 sampled
    vocabulary rows.
    """
    N, d, V = 32768, 1280, 65536
    banner(f"lmhead_ce bf16 benchmark shape N={N} d={d} V={V}")
    z = prep(synth.normal((N, d), 8, synth.STREAM_HIDDEN), "bf16")
    W = prep(synth.normal((V, d), 8, 53, std=0.02), "bf16")
    y = synth.rng(8, 54).integers(0, V, N).astype(np.int32)
    loss, dz, dW, ws = ops.lmhead_ce_fwd_bwd(to_dev(z, "bf16"), to_dev(W, "bf16"), to_dev(y))
    assert ops.status(ws) == 0
    got_dz, got_dW = to_np(dz), to_np(dW)
    del dz, dW
    cols = np.sort(synth.rng(8, 55).choice(V, 320, replace=False))
    z64, W64 = z.astype(np.float64), W.astype(np.float64)
    tot, ref_dWs = 0.0, np.zeros((cols.size, d))
    dz_err_num, dz_den = 0.0, 0.0
    for c0 in range(0, N, 2048):
        zc, yc = z64[c0:c0 + 2048], y[c0:c0 + 2048]
        l = zc @ W64.T
        lc, lse = O.cross_entropy(l, yc)
        tot += lc * zc.shape[0]
        g = O.cross_entropy_bwd(l, yc, lse) * (zc.shape[0] / N)
        del l
        dzc = g @ W64
        dz_err_num += float(np.sum((got_dz[c0:c0 + 2048] - dzc) ** 2))
        dz_den += float(np.sum(dzc ** 2))
        ref_dWs += g[:, cols].T @ zc
    ref_loss = tot / N
    assert abs(loss.item() - ref_loss) / ref_loss < 1e-4, (loss.item(), ref_loss)
    dz_err = (dz_err_num / dz_den) ** 0.5
    dW_err = rel_l2(got_dW[cols], ref_dWs)
    print(f"loss {loss.item():.6f} (oracle {ref_loss:.6f}); dz rel-L2 {dz_err:.2e}; "
          f"dW rel-L2 on 320 rows {dW_err:.2e}", flush=True)
    assert dz_err < 3e-2
    assert dW_err < 3e-2
