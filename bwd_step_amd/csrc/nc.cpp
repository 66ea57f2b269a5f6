// Host runtime behind include/nc.h: configuration and depth dial, flat
// parameter layout, workspace plan, and the forward/backward launch schedule
// of one training step.  No device memory is allocated here; every buffer is
// a slice of the caller's workspace.
//
// Model ("nanochat explainer", Modern architecture choices; The 'One Dial'
// Design -> How dimensions are derived; The Full Pipeline -> Pretraining):
//   x = E[tok]; per layer: a = rho(x); qkv = a W_qkv^T; qh, kh = RoPE(rho_hd(q, k));
//   o = causal attention; x += o W_o^T; m = rho(x); u = m W_1^T; g = relu(u)^2;
//   x += g W_2^T;  finally z = rho(x), logits = z W_lm^T, mean cross-entropy.
// Residual stream and every gradient are fp32; GEMM operands and saved
// activations use the configured element type.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/nc.h"
#include "common.h"
#include "kernels.h"

using namespace nc;

namespace {

// Tokens per LM-head chunk: up to 16384, and the chunk's G ([chunk][V] in the
// GEMM operand type) below 2 GiB, the reach of the GEMM's buffer loads.
inline int ce_chunk(int N, int V, int dtype) {
  const size_t es = dtype == NC_BF16 ? 2 : 4;
  const size_t cap = ((size_t)0x7fff0000 / ((size_t)V * es)) / 256 * 256;
  return (int)std::min<size_t>({(size_t)N, (size_t)16384, std::max<size_t>(cap, 256)});
}


inline size_t al(size_t b) { return (b + 255) & ~(size_t)255; }
// Longest KV cache (positions) the inference entry points accept.
constexpr int kMaxCacheLen = 1 << 16;

// LM-head chunk scratch besides G: fp32 path, the fp32 logits (the bf16 path
// writes its logits into G).
size_t ce_aux_bytes(size_t chunk, size_t V, int dtype) {
  if (dtype == NC_BF16) return 0;
  return chunk * V * 4;
}

struct Desc {
  std::string name;
  uint64_t offset;
  int rows, cols;
};

struct Plan {
  int batch = 0;
  size_t status = 0;
  // per-layer saved activations: offsets inside layer 0, plus the layer stride
  size_t a1, r1, qkv, rq, rk, O, lse, m, r2, g, layer_stride;
  size_t layers_base;
  // step-global buffers
  size_t wT = 0;  // bf16: one weight matrix transposed, rewritten before each input-gradient product
  size_t x, z, rf, dx, dx_lp, tmp_d, du, dO, dqkv, dqk32, gq_dk, gq_dv, Dbuf, dsT, rope, logits, G, loss_rows,
      splitk, embed_ws;
  uint64_t splitk_bytes = 0;
  size_t total;
};

}  // namespace

// Per-kernel-class GPU timing: HIP events recorded on the launch stream
// around each launcher call, with the algorithmic FLOPs / HBM bytes of that
// call.  Off by default.
enum ProfClass {
  PC_GEMM, PC_ATTN_FWD, PC_ATTN_BWD, PC_RMS_FWD, PC_RMS_BWD, PC_QK_FWD, PC_QK_BWD,
  PC_EMB_FWD, PC_EMB_BWD, PC_CE, PC_OTHER, PC_COUNT
};
static const char* kProfNames[PC_COUNT] = {"gemm", "attn_fwd", "attn_bwd", "rmsnorm_fwd", "rmsnorm_bwd",
                                           "qknorm_rope_fwd", "qknorm_rope_bwd", "embed_fwd", "embed_bwd",
                                           "ce_rows", "other"};

struct Prof {
  bool on = false;
  struct Rec {
    int cls;
    hipEvent_t a, b;
    double flops, bytes;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  hipEvent_t get() {
    if (used < pool.size()) return pool[used++];
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    pool.push_back(e);
    ++used;
    return e;
  }
  void clear() {
    recs.clear();
    used = 0;
  }
  ~Prof() {
    for (hipEvent_t e : pool) (void)hipEventDestroy(e);
  }
};

struct nc_ctx {
  nc_config cfg;
  hipStream_t stream;
  std::vector<Desc> layout;
  uint64_t nparams;
  char* ws = nullptr;
  uint64_t ws_bytes = 0;
  Prof prof;
  bool poison = false;  // nc_debug_poison_workspace
  bool resid_fp32 = false;  // nc_set_residual_fp32
  // Backward: the weight-gradient products run on a second stream (created
  // on first use, default priority), ordered against the main stream by
  // events, so that they fill the compute units the input-gradient chain
  // leaves idle.  Serial while the per-launch profiler is on.
  hipStream_t side = nullptr;
  hipEvent_t ev_main = nullptr, ev_b2 = nullptr, ev_b4 = nullptr, ev_b6 = nullptr, ev_b8 = nullptr, ev_all = nullptr;
  ~nc_ctx() {
    for (hipEvent_t e : {ev_main, ev_b2, ev_b4, ev_b6, ev_b8, ev_all})
      if (e) (void)hipEventDestroy(e);
    if (side) (void)hipStreamDestroy(side);
  }
};

namespace {

int validate(nc_config* c) {
  if (c->depth < 1) return NC_ERR_CONFIG;
  if (c->d_model == 0) c->d_model = 64 * c->depth;
  if (c->head_dim == 0) c->head_dim = 128;
  if (c->n_heads == 0) c->n_heads = c->d_model / c->head_dim;
  if (c->d_ff == 0) c->d_ff = 4 * c->d_model;
  if (c->rope_base == 0.f) c->rope_base = 10000.f;
  if (c->norm_eps == 0.f) c->norm_eps = 1e-6f;
  if (c->d_model <= 0 || c->d_model % 64) return NC_ERR_CONFIG;
  if (c->d_ff <= 0 || c->d_ff % 64) return NC_ERR_CONFIG;
  if (c->head_dim != 16 && c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128) return NC_ERR_CONFIG;
  if (c->n_heads < 1) return NC_ERR_CONFIG;
  if (c->n_kv_heads == 0) c->n_kv_heads = c->n_heads;
  if (c->n_kv_heads < 1 || c->n_heads % c->n_kv_heads) return NC_ERR_CONFIG;
  if (c->vocab < 64 || c->vocab % 64) return NC_ERR_CONFIG;
  if (c->seq_len < 1 || c->max_batch < 1) return NC_ERR_CONFIG;
  if (!(c->rope_base > 1.f) || !(c->norm_eps > 0.f)) return NC_ERR_CONFIG;
  if (c->dtype != NC_BF16 && c->dtype != NC_FP32) return NC_ERR_CONFIG;
  if ((uint64_t)c->max_batch * c->seq_len > (1ull << 30)) return NC_ERR_CONFIG;
  if (c->dtype == NC_BF16 && c->head_dim != 64 && c->head_dim != 128) return NC_ERR_UNSUPPORTED;
  // the bf16 head_dim-128 attention backward stores dS per (b, h) as one [Tp][Tp] block
  if (c->dtype == NC_BF16 && c->head_dim == 128 && attn_ds_pad(c->seq_len) > kMaxDsPad) return NC_ERR_UNSUPPORTED;
  return NC_OK;
}

Plan make_plan(const nc_config& c, int batch) {
  Plan p;
  p.batch = batch;
  const size_t N = (size_t)batch * c.seq_len;
  const size_t d = c.d_model, hh = (size_t)c.n_heads * c.head_dim, F = c.d_ff, V = c.vocab, H = c.n_heads;
  const size_t hk = (size_t)c.n_kv_heads * c.head_dim, nq = hh + 2 * hk;  // QKV width
  const bool grouped = c.n_kv_heads != c.n_heads;
  const size_t es = c.dtype == NC_BF16 ? 2 : 4;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o += al(bytes); return r; };
  p.status = take(256);
  p.x = take(N * d * 4);
  p.z = take(N * d * es);
  p.rf = take(N * 4);
  p.dx = take(N * d * 4);
  p.dx_lp = take(N * d * es);
  p.tmp_d = take(N * d * 4);
  p.du = take(N * F * es);
  p.wT = c.dtype == NC_BF16 ? take(std::max(std::max(std::max(F * d, d * hh), nq * d), V * d) * 2) : 0;
  p.dO = take(N * hh * es);
  p.dqkv = take(N * nq * es);
  p.dqk32 = take(N * (hh + hk) * 4);
  // grouped-query attention: per-query-head dk (fp32) and dv before the group sums
  p.gq_dk = grouped ? take(N * hh * 4) : 0;
  p.gq_dv = grouped ? take(N * hh * es) : 0;
  p.Dbuf = take(N * H * 4);
  p.dsT = take(attn_ds_bytes(batch, (int)H, c.seq_len, c.head_dim, c.dtype));  // the attention backward's dS
  p.rope = take((size_t)c.seq_len * c.head_dim * 4);
  const size_t chunk = (size_t)ce_chunk((int)N, (int)V, c.dtype);
  p.logits = take(ce_aux_bytes(chunk, V, c.dtype));
  p.G = take(chunk * V * es);
  p.loss_rows = take(N * 4);
  uint64_t sk = 0;
  const int n = (int)N;
  sk = std::max(sk, gemm_ws_bytes((int)nq, (int)d, n, c.dtype));
  sk = std::max(sk, gemm_ws_bytes((int)d, (int)hh, n, c.dtype));
  sk = std::max(sk, gemm_ws_bytes((int)F, (int)d, n, c.dtype));
  sk = std::max(sk, gemm_ws_bytes((int)d, (int)F, n, c.dtype));
  sk = std::max(sk, gemm_ws_bytes((int)chunk, (int)d, (int)V, c.dtype));
  sk = std::max(sk, gemm_ws_bytes((int)V, (int)d, (int)chunk, c.dtype));
  p.splitk = take(sk);
  p.splitk_bytes = sk;
  p.embed_ws = take(embed_bwd_ws_bytes(n, (int)d, (int)V));
  // per-layer saved activations
  p.layers_base = o;
  size_t lo = 0;
  auto ltake = [&](size_t bytes) { size_t r = lo; lo += al(bytes); return r; };
  p.a1 = ltake(N * d * es);
  p.r1 = ltake(N * 4);
  p.qkv = ltake(N * nq * es);
  p.rq = ltake(N * H * 4);
  p.rk = ltake(N * c.n_kv_heads * 4);
  p.O = ltake(N * hh * es);
  p.lse = ltake(N * H * 4);
  p.m = ltake(N * d * es);
  p.r2 = ltake(N * 4);
  p.g = ltake(N * F * es);
  p.layer_stride = lo;
  o += lo * c.depth;
  p.total = o;
  return p;
}

void build_layout(nc_ctx* x) {
  const nc_config& c = x->cfg;
  const uint64_t d = c.d_model, hh = (uint64_t)c.n_heads * c.head_dim, F = c.d_ff, V = c.vocab;
  const uint64_t hk = (uint64_t)c.n_kv_heads * c.head_dim;
  uint64_t off = 0;
  auto add = [&](const std::string& n, uint64_t r, uint64_t cl) {
    x->layout.push_back({n, off, (int)r, (int)cl});
    off += r * cl;
  };
  add("E", V, d);
  for (int l = 0; l < c.depth; ++l) {
    const std::string p = "layers." + std::to_string(l) + ".";
    add(p + "W_qkv", hh + 2 * hk, d);  // query heads, then key heads, then value heads
    add(p + "W_o", d, hh);
    add(p + "W_1", F, d);
    add(p + "W_2", d, F);
  }
  add("W_lm", V, d);
  x->nparams = off;
}

__global__ void clear_status_kernel(int* s) { *s = 0; }

// Debug: fill n 16-byte words with all-ones bytes (NaN as fp32 and bf16).
__global__ void poison_kernel(uint4* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(~0u, ~0u, ~0u, ~0u);
}

// With poisoning on, every byte of the workspace past the status block is
// made NaN before a call, so a kernel that read workspace memory it had not
// written would change the result.
int maybe_poison(nc_ctx* ctx, const Plan& P) {
  if (!ctx->poison || P.total <= 256) return NC_OK;
  const size_t n = (P.total - 256) / 16;
  poison_kernel<<<2048, 256, 0, ctx->stream>>>((uint4*)(ctx->ws + 256), n);
  return hipGetLastError() == hipSuccess ? NC_OK : NC_ERR_HIP;
}

int clear_status(void* ws, hipStream_t s) {
  clear_status_kernel<<<1, 1, 0, s>>>((int*)ws);
  return hipGetLastError() == hipSuccess ? NC_OK : NC_ERR_HIP;
}

// The second stream of the backward and its events (see nc_ctx).
int ensure_side(nc_ctx* x) {
  if (x->side) return NC_OK;
  hipStream_t st = nullptr;
  if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return NC_ERR_HIP;
  for (hipEvent_t* e : {&x->ev_main, &x->ev_b2, &x->ev_b4, &x->ev_b6, &x->ev_b8, &x->ev_all})
    if (hipEventCreateWithFlags(e, hipEventDisableTiming) != hipSuccess) {
      (void)hipStreamDestroy(st);
      return NC_ERR_HIP;
    }
  x->side = st;
  return NC_OK;
}
// Work enqueued on `to` after this call starts only once the work enqueued
// on `from` so far has finished (nothing when both are one stream).
int order_after(hipEvent_t e, hipStream_t from, hipStream_t to) {
  if (from == to) return NC_OK;
  if (hipEventRecord(e, from) != hipSuccess) return NC_ERR_HIP;
  return hipStreamWaitEvent(to, e, 0) == hipSuccess ? NC_OK : NC_ERR_HIP;
}
// Record e on `from` now; a later wait_for(e, to) orders `to` after it.
int mark(hipEvent_t e, hipStream_t from, hipStream_t to) {
  if (from == to) return NC_OK;
  return hipEventRecord(e, from) == hipSuccess ? NC_OK : NC_ERR_HIP;
}
int wait_for(hipEvent_t e, hipStream_t from, hipStream_t to) {
  if (from == to) return NC_OK;
  return hipStreamWaitEvent(to, e, 0) == hipSuccess ? NC_OK : NC_ERR_HIP;
}

int read_status(void* ws, hipStream_t s) {
  int v = 0;
  if (hipMemcpyAsync(&v, ws, sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess) return NC_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return NC_ERR_HIP;
  if (clear_status(ws, s) != NC_OK) return NC_ERR_HIP;
  if (v & nc::kStatusTokenRange) return NC_ERR_TOKEN_RANGE;
  if (v & nc::kStatusNonFinite) return NC_ERR_NONFINITE;
  return NC_OK;
}

#define TRY(x)                   \
  do {                           \
    int rc_ = (x);               \
    if (rc_) return rc_;         \
  } while (0)

// Run a launcher call; when profiling, bracket it with events on stream s.
#define PROF(P, cls, fl, by, call)                                         \
  do {                                                                     \
    Prof* p_ = (P);                                                        \
    hipEvent_t e0_ = nullptr;                                              \
    if (p_ && p_->on && (e0_ = p_->get())) (void)hipEventRecord(e0_, s);   \
    TRY(call);                                                             \
    if (e0_) {                                                             \
      hipEvent_t e1_ = p_->get();                                          \
      if (e1_) {                                                           \
        (void)hipEventRecord(e1_, s);                                      \
        p_->recs.push_back({(cls), e0_, e1_, (double)(fl), (double)(by)}); \
      }                                                                    \
    }                                                                      \
  } while (0)

inline double gflops(const GemmCall& g) { return 2.0 * g.M * (double)g.N * g.K; }
// Algorithmic HBM bytes of one GEMM call: each operand read once, the output
// (and whatever the epilogue reads) once; split-K partials are not counted.
inline double gbytes(const GemmCall& g) {
  const double es = g.dtype == NC_BF16 ? 2.0 : 4.0, mn = (double)g.M * g.N;
  double out = 0.0;
  switch (g.epi) {
    case EPI_F32: out = (g.e.beta ? 8.0 : 4.0) * mn; break;   // fp32 store (accumulate: read + write)
    case EPI_F32_ACC: out = 8.0 * mn; break;
    case EPI_RESID: out = 8.0 * mn; break;                     // fp32 residual read + write
    case EPI_LP: case EPI_RELU2: out = es * mn; break;
    case EPI_DRELU2: out = 2.0 * es * mn; break;               // g read, du written
    default: break;
  }
  return es * ((double)g.M * g.K + (double)g.N * g.K) + out;
}

GemmCall mk(const void* A, long lda, bool ak, const void* B, long ldb, bool bk, int M, int N, int K, int dtype) {
  GemmCall g;
  g.A = A; g.lda = lda; g.a_k = ak;
  g.B = B; g.ldb = ldb; g.b_k = bk;
  g.M = M; g.N = N; g.K = K;
  g.dtype = dtype;
  return g;
}

// LM head + cross-entropy over tokens in chunks: loss_rows, dz (fp32, [N,d]),
// dW (fp32 [V,d]; overwritten or accumulated).  G and the scratch `aux`
// (ce_aux_bytes) are chunk-sized.  bf16: the logits GEMM writes bf16 logits
// into G, ce_finish turns them into G in place (with the fp32 target logits
// from z and W); fp32: fp32 logits, then ce_rows.  wT (bf16, optional, V*d
// elements): W is transposed into it once so that dz = G W reads both
// operands k-contiguous.
int lmhead_ce(const void* z, const void* W, const int32_t* y, int N, int d, int V, float* loss_rows, float* dz,
              float* dW, int accumulate, int dtype, float* aux, void* G, float* splitk, uint64_t splitk_bytes,
              int* status, hipStream_t s, Prof* pf, void* wT = nullptr) {
  const size_t es = dtype == NC_BF16 ? 2 : 4;
  const int chunk = ce_chunk(N, V, dtype);
  if (wT && dtype == NC_BF16) TRY(launch_transpose_bf16(W, V, d, d, wT, V, s));
  for (int c0 = 0; c0 < N; c0 += chunk) {
    const int rows = std::min(chunk, N - c0);
    const char* zc = (const char*)z + (size_t)c0 * d * es;
    GemmCall lg = mk(zc, d, true, W, d, true, rows, V, d, dtype);
    if (dtype == NC_BF16) {
      lg.epi = EPI_LP; lg.e.c_lp = G; lg.e.ld_lp = V;
      PROF(pf, PC_GEMM, gflops(lg), gbytes(lg), launch_gemm(lg, s));
      PROF(pf, PC_CE, 0, (double)rows * V * 4 + (double)rows * d * 4,
           launch_ce_finish(zc, d, W, d, d, y + c0, G, V, loss_rows + c0, rows, V, status, s));
    } else {
      lg.epi = EPI_F32; lg.e.c32 = aux; lg.e.ldc = V; lg.e.beta = 0;
      PROF(pf, PC_GEMM, gflops(lg), gbytes(lg), launch_gemm(lg, s));
      PROF(pf, PC_CE, 0, (double)rows * V * (4 + es),
           launch_ce_rows(aux, V, y + c0, G, V, loss_rows + c0, rows, V, dtype, status, s));
    }
    GemmCall gw = mk(G, V, false, zc, d, false, V, d, rows, dtype);
    gw.epi = EPI_F32; gw.e.c32 = dW; gw.e.ldc = d; gw.e.beta = (c0 > 0 || accumulate) ? 1 : 0;
    gw.splitk_ws = splitk; gw.splitk_bytes = splitk_bytes;
    PROF(pf, PC_GEMM, gflops(gw), gbytes(gw), launch_gemm(gw, s));
    GemmCall gz = (wT && dtype == NC_BF16) ? mk(G, V, true, wT, V, true, rows, d, V, dtype)
                                           : mk(G, V, true, W, d, false, rows, d, V, dtype);
    gz.epi = EPI_F32; gz.e.c32 = dz + (size_t)c0 * d; gz.e.ldc = d; gz.e.beta = 0;
    gz.splitk_ws = splitk; gz.splitk_bytes = splitk_bytes;
    PROF(pf, PC_GEMM, gflops(gz), gbytes(gz), launch_gemm(gz, s));
  }
  return NC_OK;
}

// Forward over batch sequences of T tokens (T <= seq_len; the plan is sized
// for seq_len), saving what the backward and the cache fill read.
int run_forward(nc_ctx* ctx, const Plan& P, const void* params, const int32_t* tokens, int batch, int T) {
  const nc_config& c = ctx->cfg;
  hipStream_t s = ctx->stream;
  char* W = ctx->ws;
  const int N = batch * T, d = c.d_model, H = c.n_heads, hd = c.head_dim, hh = H * hd, F = c.d_ff;
  const int Hk = c.n_kv_heads, hk = Hk * hd, nq = hh + 2 * hk;
  const int V = c.vocab, dt = c.dtype;
  const size_t es = dt == NC_BF16 ? 2 : 4;
  const char* prm = (const char*)params;
  int* status = (int*)(W + P.status);
  float* x = (float*)(W + P.x);
  float* cs = (float*)(W + P.rope);

  Prof* pf = &ctx->prof;
  const double pairs = (double)batch * H * T * (T + 1) / 2.0;  // causal (query, key) pairs
  PROF(pf, PC_EMB_FWD, 0, (double)N * d * (es + 4) + N * 4.0, launch_embed_fwd(prm, tokens, x, N, d, V, dt, status, s));
  PROF(pf, PC_OTHER, 0, 0, launch_rope_table(cs, T, hd, c.rope_base, s));
  // bf16 path: the output projections store their sublayer output y in bf16
  // and the next RMSNorm adds it to the fp32 stream x (x += y, then the norm);
  // fp32 path, and bf16 with nc_set_residual_fp32: the projections add their
  // fp32 accumulators into x in their epilogue.
  void* ybuf = W + P.dx_lp;
  const void* pend = nullptr;
  auto norm = [&](void* out, float* r) -> int {
    if (pend) {
      const void* res = pend;
      pend = nullptr;
      PROF(pf, PC_RMS_FWD, 0, (double)N * d * (4 + 2 + 4 + es) + N * 4.0,
           launch_rmsnorm_add_fwd(x, res, out, r, N, d, c.norm_eps, s));
      return NC_OK;
    }
    PROF(pf, PC_RMS_FWD, 0, (double)N * d * (4 + es) + N * 4.0, launch_rmsnorm_fwd(x, out, r, N, d, c.norm_eps, dt, s));
    return NC_OK;
  };
  auto proj_out = [&](GemmCall& g) {
    if (dt == NC_BF16 && !ctx->resid_fp32) {
      g.epi = EPI_LP; g.e.c_lp = ybuf; g.e.ld_lp = d;
      pend = ybuf;
    } else {
      g.epi = EPI_RESID; g.e.c32 = x; g.e.ldc = d;
    }
  };
  for (int l = 0; l < c.depth; ++l) {
    char* L = W + P.layers_base + (size_t)l * P.layer_stride;
    const char* Wqkv = prm + ctx->layout[1 + 4 * l].offset * es;
    const char* Wo = prm + ctx->layout[2 + 4 * l].offset * es;
    const char* W1 = prm + ctx->layout[3 + 4 * l].offset * es;
    const char* W2 = prm + ctx->layout[4 + 4 * l].offset * es;
    void* a1 = L + P.a1;
    char* qkv = L + P.qkv;
    TRY(norm(a1, (float*)(L + P.r1)));
    GemmCall g1 = mk(a1, d, true, Wqkv, d, true, N, nq, d, dt);
    g1.epi = EPI_LP; g1.e.c_lp = qkv; g1.e.ld_lp = nq;
    PROF(pf, PC_GEMM, gflops(g1), gbytes(g1), launch_gemm(g1, s));
    PROF(pf, PC_QK_FWD, 0, 2.0 * N * (hh + hk) * es + N * (H + Hk) * 4.0, launch_qknorm_rope_fwd(qkv, nq, qkv + hh * es, nq, qkv, nq, qkv + hh * es, nq,
                               (float*)(L + P.rq), (float*)(L + P.rk), cs, N, H, hd, T, c.norm_eps, dt, s, Hk));
    AttnArgs a;
    a.q = qkv; a.ldq = nq;
    a.k = qkv + hh * es; a.ldk = nq;
    a.v = qkv + (hh + hk) * es; a.ldv = nq;
    a.G = H / Hk;
    a.o = L + P.O; a.ldo = hh;
    a.lse = (float*)(L + P.lse);
    a.B = batch; a.H = H; a.T = T;
    PROF(pf, PC_ATTN_FWD, 4.0 * hd * pairs, 0, launch_attn_fwd(a, hd, dt, s));
    GemmCall g2 = mk(L + P.O, hh, true, Wo, hh, true, N, d, hh, dt);
    proj_out(g2);
    PROF(pf, PC_GEMM, gflops(g2), gbytes(g2), launch_gemm(g2, s));
    TRY(norm(L + P.m, (float*)(L + P.r2)));
    GemmCall g3 = mk(L + P.m, d, true, W1, d, true, N, F, d, dt);
    g3.epi = EPI_RELU2; g3.e.c_lp = L + P.g; g3.e.ld_lp = F;
    PROF(pf, PC_GEMM, gflops(g3), gbytes(g3), launch_gemm(g3, s));
    GemmCall g4 = mk(L + P.g, F, true, W2, F, true, N, d, F, dt);
    proj_out(g4);
    PROF(pf, PC_GEMM, gflops(g4), gbytes(g4), launch_gemm(g4, s));
  }
  TRY(norm(W + P.z, (float*)(W + P.rf)));
  return NC_OK;
}

// The count of counted targets (launch_count_targets) must be in the status
// block before the first microbatch; `last` writes the loss of the step.
int run_backward(nc_ctx* ctx, const Plan& P, const void* params, const int32_t* tokens, const int32_t* targets,
                 int batch, float* loss, float* grads, int accumulate, bool last) {
  const nc_config& c = ctx->cfg;
  hipStream_t s = ctx->stream;
  char* W = ctx->ws;
  const int N = batch * c.seq_len, d = c.d_model, H = c.n_heads, hd = c.head_dim, hh = H * hd, F = c.d_ff;
  const int Hk = c.n_kv_heads, hk = Hk * hd, nq = hh + 2 * hk;
  const int V = c.vocab, dt = c.dtype;
  const size_t es = dt == NC_BF16 ? 2 : 4;
  const char* prm = (const char*)params;
  int* status = (int*)(W + P.status);
  float* dx = (float*)(W + P.dx);
  void* dx_lp = W + P.dx_lp;
  float* tmp = (float*)(W + P.tmp_d);
  float* splitk = P.splitk ? (float*)(W + P.splitk) : nullptr;
  float* cs = (float*)(W + P.rope);
  const Desc& lm = ctx->layout.back();

  Prof* pf = &ctx->prof;
  const double pairs = (double)batch * H * c.seq_len * (c.seq_len + 1) / 2.0;
  const double rms_bwd_bytes = (double)N * d * (4 + es + 4 + 4 + es) + N * 4.0;
  TRY(lmhead_ce(W + P.z, prm + lm.offset * es, targets, N, d, V, (float*)(W + P.loss_rows), tmp,
                grads + lm.offset, accumulate, dt, (float*)(W + P.logits), W + P.G, splitk, P.splitk_bytes, status, s,
                pf, dt == NC_BF16 ? W + P.wT : nullptr));
  PROF(pf, PC_OTHER, 0, 0, launch_loss_sum((float*)(W + P.loss_rows), N, status, s));
  if (last) PROF(pf, PC_OTHER, 0, 0, launch_loss_final(loss, status, s));
  PROF(pf, PC_RMS_BWD, 0, rms_bwd_bytes - (double)N * d * 4,
       launch_rmsnorm_bwd(tmp, W + P.z, (float*)(W + P.rf), dx, dx_lp, N, d, 0, dt, s));

  // The input gradients of the MLP and QKV projections feed only the RMSNorm
  // backward: bf16 path, stored in bf16 (tmp as a bf16 [N, d] buffer); fp32
  // path, fp32.
  auto dgrad_out = [&](GemmCall& g) {
    if (dt == NC_BF16) {
      g.epi = EPI_LP; g.e.c_lp = tmp; g.e.ld_lp = d;
    } else {
      g.epi = EPI_F32; g.e.c32 = tmp; g.e.ldc = d;
    }
  };
  auto norm_bwd = [&](const void* y, const float* r) -> int {
    if (dt == NC_BF16) {
      PROF(pf, PC_RMS_BWD, 0, rms_bwd_bytes - (double)N * d * 2,
           launch_rmsnorm_bwd_lpdy(tmp, y, r, dx, dx_lp, N, d, 1, s));
    } else {
      PROF(pf, PC_RMS_BWD, 0, rms_bwd_bytes, launch_rmsnorm_bwd(tmp, y, r, dx, dx_lp, N, d, 1, dt, s));
    }
    return NC_OK;
  };
  // Weight gradients (dW = dy^T x: W_2, W_1, W_o, W_qkv) go to the second
  // stream s2.  Each reads a saved activation and a gradient buffer that the
  // main stream rewrites later: dx_lp (read by dW_2, then dW_o; rewritten by
  // the two RMSNorm backwards), du (dW_1; rewritten by the next layer's
  // MLP input gradient) and dqkv (dW_qkv; rewritten by the next layer's
  // attention backward), so the main stream waits for the product that
  // reads a buffer before it rewrites it.  The split-K workspace is used on
  // s2 only (after the LM head, which precedes the first fork).
  hipStream_t s2 = s;
  if (!pf->on) {
    TRY(ensure_side(ctx));
    s2 = ctx->side;
  }
  for (int l = c.depth - 1; l >= 0; --l) {
    const bool first = l == c.depth - 1;
    char* L = W + P.layers_base + (size_t)l * P.layer_stride;
    const Desc& dqkv_d = ctx->layout[1 + 4 * l];
    const Desc& do_d = ctx->layout[2 + 4 * l];
    const Desc& d1_d = ctx->layout[3 + 4 * l];
    const Desc& d2_d = ctx->layout[4 + 4 * l];
    const char* Wqkv = prm + dqkv_d.offset * es;
    const char* Wo = prm + do_d.offset * es;
    const char* W1 = prm + d1_d.offset * es;
    const char* W2 = prm + d2_d.offset * es;
    const int beta = accumulate ? 1 : 0;
    char* qkv = L + P.qkv;
    char* dqkv = W + P.dqkv;
    float* dqk32 = (float*)(W + P.dqk32);

    // MLP: du = (dx W_2) * 2 relu(u), with relu(u) = sqrt(g); dW_2 = dx^T g; dm = du W_1; dW_1 = du^T m
    // bf16: the product reads W_2 transposed, so that both operands are
    // k-contiguous (the pair loop and its staged ReLU²-backward epilogue)
    // dW_2 (s2) reads dx_lp as the main stream has it now
    TRY(order_after(ctx->ev_main, s, s2));
    GemmCall b2 = mk(dx_lp, d, false, L + P.g, F, false, d, F, N, dt);
    b2.epi = EPI_F32; b2.e.c32 = grads + d2_d.offset; b2.e.ldc = F; b2.e.beta = beta; b2.splitk_ws = splitk; b2.splitk_bytes = P.splitk_bytes;
    PROF(pf, PC_GEMM, gflops(b2), gbytes(b2), launch_gemm(b2, s2));
    TRY(mark(ctx->ev_b2, s2, s));
    GemmCall b1 = mk(dx_lp, d, true, W2, F, false, N, F, d, dt);
    if (dt == NC_BF16) {
      TRY(launch_transpose_bf16(W2, d, F, F, W + P.wT, d, s));
      b1 = mk(dx_lp, d, true, W + P.wT, d, true, N, F, d, dt);
    }
    b1.epi = EPI_DRELU2; b1.e.c_lp = W + P.du; b1.e.ld_lp = F; b1.e.aux = L + P.g; b1.e.ld_aux = F;
    if (!first) TRY(wait_for(ctx->ev_b4, s2, s));  // the previous layer's dW_1 has read du
    PROF(pf, PC_GEMM, gflops(b1), gbytes(b1), launch_gemm(b1, s));
    // dW_1 (s2) reads du
    TRY(order_after(ctx->ev_main, s, s2));
    GemmCall b4 = mk(W + P.du, F, false, L + P.m, d, false, F, d, N, dt);
    b4.epi = EPI_F32; b4.e.c32 = grads + d1_d.offset; b4.e.ldc = d; b4.e.beta = beta; b4.splitk_ws = splitk; b4.splitk_bytes = P.splitk_bytes;
    PROF(pf, PC_GEMM, gflops(b4), gbytes(b4), launch_gemm(b4, s2));
    TRY(mark(ctx->ev_b4, s2, s));
    GemmCall b3 = mk(W + P.du, F, true, W1, d, false, N, d, F, dt);
    if (dt == NC_BF16) {
      TRY(launch_transpose_bf16(W1, F, d, d, W + P.wT, F, s));
      b3 = mk(W + P.du, F, true, W + P.wT, F, true, N, d, F, dt);
    }
    dgrad_out(b3);
    PROF(pf, PC_GEMM, gflops(b3), gbytes(b3), launch_gemm(b3, s));
    TRY(wait_for(ctx->ev_b2, s2, s));  // dW_2 has read dx_lp
    TRY(norm_bwd(L + P.m, (float*)(L + P.r2)));

    // attention output projection: dO = dx W_o; dW_o = dx^T O
    GemmCall b5 = mk(dx_lp, d, true, Wo, hh, false, N, hh, d, dt);
    if (dt == NC_BF16) {
      TRY(launch_transpose_bf16(Wo, d, hh, hh, W + P.wT, d, s));
      b5 = mk(dx_lp, d, true, W + P.wT, d, true, N, hh, d, dt);
    }
    b5.epi = EPI_LP; b5.e.c_lp = W + P.dO; b5.e.ld_lp = hh;
    // dW_o (s2) reads the new dx_lp
    TRY(order_after(ctx->ev_main, s, s2));
    GemmCall b6 = mk(dx_lp, d, false, L + P.O, hh, false, d, hh, N, dt);
    b6.epi = EPI_F32; b6.e.c32 = grads + do_d.offset; b6.e.ldc = hh; b6.e.beta = beta; b6.splitk_ws = splitk; b6.splitk_bytes = P.splitk_bytes;
    PROF(pf, PC_GEMM, gflops(b6), gbytes(b6), launch_gemm(b6, s2));
    TRY(mark(ctx->ev_b6, s2, s));
    PROF(pf, PC_GEMM, gflops(b5), gbytes(b5), launch_gemm(b5, s));

    AttnArgs a;
    a.q = qkv; a.ldq = nq;
    a.k = qkv + hh * es; a.ldk = nq;
    a.v = qkv + (hh + hk) * es; a.ldv = nq;
    a.o = L + P.O; a.ldo = hh;
    a.dout = W + P.dO; a.lddo = hh;
    a.lse = (float*)(L + P.lse);
    a.Dbuf = (float*)(W + P.Dbuf);
    a.dsT = W + P.dsT; a.tpad = attn_ds_pad(c.seq_len);
    // bf16, head_dim 128: the dQ kernel finishes q's QK-norm + RoPE backward
    // and writes dq straight into dqkv (the pass below then handles k, unless
    // the dK/dV kernel does as well)
    const bool q_fused = dt == NC_BF16 && hd == 128;
    if (q_fused) {
      a.dq_pre = dqkv; a.lddq_pre = nq;
      a.rq = (const float*)(L + P.rq);
      a.cs = cs;
    }
    a.dq32 = dqk32; a.lddq = hh + hk;
    a.B = batch; a.H = H; a.T = c.seq_len;
    a.G = H / Hk;
    // with q finished by the dQ kernel and no key groups, the dK/dV kernel
    // finishes k's QK-norm + RoPE backward too and writes the gradient w.r.t.
    // the pre-norm k (bf16) into the k columns of dqkv: no separate pass
    const bool k_lp = q_fused && a.G == 1;
    if (a.G == 1) {
      a.dk32 = dqk32 + hh; a.lddk = hh + hk;
      if (k_lp) { a.dk_lp = dqkv + hh * es; a.lddk_lp = nq; a.rk = (const float*)(L + P.rk); }
      a.dv = dqkv + (hh + hk) * es; a.lddv = nq;
    } else {  // per query head first, then the sums over each group
      a.dk32 = (float*)(W + P.gq_dk); a.lddk = hh;
      a.dv = W + P.gq_dv; a.lddv = hh;
    }
    if (!first) TRY(wait_for(ctx->ev_b8, s2, s));  // the previous layer's dW_qkv has read dqkv
    PROF(pf, PC_ATTN_BWD, 8.0 * hd * pairs, 0, launch_attn_bwd(a, hd, dt, s));
    if (a.G > 1)
      PROF(pf, PC_OTHER, 0, (double)N * hh * (4 + es) + (double)N * hk * (4 + es),
           launch_kv_group_sum((float*)(W + P.gq_dk), hh, W + P.gq_dv, hh, dqk32 + hh, hh + hk,
                               dqkv + (hh + hk) * es, nq, N, Hk, a.G, hd, dt, s));
    if (!k_lp)
      PROF(pf, PC_QK_BWD, 0, (double)N * ((q_fused ? 0 : hh) + hk) * (4 + 2 * es) + (double)N * ((q_fused ? 0 : H) + Hk) * 4,
           launch_qknorm_rope_bwd(dqk32, hh + hk, dqk32 + hh, hh + hk, qkv, nq, qkv + hh * es, nq,
                                  (float*)(L + P.rq), (float*)(L + P.rk), dqkv, nq, dqkv + hh * es, nq, cs, N, H,
                                  hd, c.seq_len, dt, s, Hk, q_fused));

    // QKV projection: da = dqkv W_qkv; dW_qkv = dqkv^T a (s2, reads dqkv)
    TRY(order_after(ctx->ev_main, s, s2));
    GemmCall b8 = mk(dqkv, nq, false, L + P.a1, d, false, nq, d, N, dt);
    b8.epi = EPI_F32; b8.e.c32 = grads + dqkv_d.offset; b8.e.ldc = d; b8.e.beta = beta; b8.splitk_ws = splitk; b8.splitk_bytes = P.splitk_bytes;
    PROF(pf, PC_GEMM, gflops(b8), gbytes(b8), launch_gemm(b8, s2));
    TRY(mark(ctx->ev_b8, s2, s));
    GemmCall b7 = mk(dqkv, nq, true, Wqkv, d, false, N, d, nq, dt);
    if (dt == NC_BF16) {
      TRY(launch_transpose_bf16(Wqkv, nq, d, d, W + P.wT, nq, s));
      b7 = mk(dqkv, nq, true, W + P.wT, nq, true, N, d, nq, dt);
    }
    dgrad_out(b7);
    PROF(pf, PC_GEMM, gflops(b7), gbytes(b7), launch_gemm(b7, s));
    TRY(wait_for(ctx->ev_b6, s2, s));  // dW_o has read dx_lp
    TRY(norm_bwd(L + P.a1, (float*)(L + P.r1)));
  }
  // every weight gradient is complete before the main stream goes on (the
  // caller's next work, a next microbatch's forward rewriting the saved
  // activations they read)
  TRY(order_after(ctx->ev_all, s2, s));
  PROF(pf, PC_EMB_BWD, 0, (double)N * d * 4 + (double)V * d * 4 * (accumulate ? 2 : 1) + N * 4.0,
       launch_embed_bwd(dx, tokens, grads, N, d, V, accumulate, W + P.embed_ws, s));
  return NC_OK;
}

}  // namespace

namespace {
// ---------------------------------------------------------------- inference
// KV cache: per layer K then V, each [cache_batch][n_kv_heads][max_len][hd].
uint64_t kv_layer_elems(const nc_config& c, int cache_batch, int max_len) {
  return (uint64_t)cache_batch * c.n_kv_heads * max_len * c.head_dim;
}

struct DecodePlan {
  size_t x = 0, qkv = 0, qhat = 0, o = 0, g = 0, cs = 0, part_o = 0, part_ml = 0, total = 0;
};
DecodePlan decode_plan(const nc_config& c, int batch, int max_len) {
  DecodePlan p;
  const size_t es = c.dtype == NC_BF16 ? 2 : 4;
  const size_t B = batch, d = c.d_model, hh = (size_t)c.n_heads * c.head_dim, F = c.d_ff;
  const size_t nq = hh + 2 * (size_t)c.n_kv_heads * c.head_dim;
  const size_t nchunk = (max_len + kDecodeKeys - 1) / kDecodeKeys;
  size_t o = 0;
  auto take = [&](size_t b) { size_t r = o; o += al(b); return r; };
  take(256);  // status block
  p.x = take(B * d * 4);
  p.qkv = take(B * nq * es);
  p.qhat = take(B * hh * es);
  p.o = take(B * hh * es);
  p.g = take(B * F * es);
  p.cs = take((size_t)max_len * c.head_dim * 4);
  p.part_o = take(B * c.n_heads * nchunk * c.head_dim * 4);
  p.part_ml = take(B * c.n_heads * nchunk * 2 * 4);
  p.total = o;
  return p;
}

// One decode step on the buffers of plan D inside w (device), with the
// status word at `status`; the caller has checked every argument.
int decode_run(nc_ctx* ctx, const DecodePlan& D, const void* params, const int32_t* tokens, const int32_t* pos,
               int batch, void* cache, int max_len, char* w, int* status, float* logits) {
  const nc_config& c = ctx->cfg;
  hipStream_t s = ctx->stream;
  const int d = c.d_model, H = c.n_heads, hd = c.head_dim, hh = H * hd, F = c.d_ff, V = c.vocab, dt = c.dtype;
  const int Hk = c.n_kv_heads, nq = hh + 2 * Hk * hd;
  const size_t es = dt == NC_BF16 ? 2 : 4;
  float* x = (float*)(w + D.x);
  float* cs = (float*)(w + D.cs);
  const char* prm = (const char*)params;
  const uint64_t le = kv_layer_elems(c, batch, max_len);
  TRY(launch_rope_table(cs, max_len, hd, c.rope_base, s));
  TRY(launch_embed_fwd(prm, tokens, x, batch, d, V, dt, status, s));
  auto gemv = [&](const void* in, long ldin, const char* Wt, int N, int K, int epi, float* c32, void* clp, long ld,
                  float norm_eps) {
    SkinnyOut o;
    o.c32 = c32;
    o.c_lp = clp;
    o.ld = ld;
    return launch_skinny(in, ldin, Wt, K, batch, N, K, epi, o, dt, s, norm_eps);
  };
  // the RMSNorms before the QKV, MLP and LM-head products are fused into them (x fp32)
  const float ne = c.norm_eps;
  for (int l = 0; l < c.depth; ++l) {
    const char* Wqkv = prm + ctx->layout[1 + 4 * l].offset * es;
    const char* Wo = prm + ctx->layout[2 + 4 * l].offset * es;
    const char* W1 = prm + ctx->layout[3 + 4 * l].offset * es;
    const char* W2 = prm + ctx->layout[4 + 4 * l].offset * es;
    char* kc = (char*)cache + (size_t)l * 2 * le * es;
    TRY(gemv(x, d, Wqkv, nq, d, EPI_LP, nullptr, w + D.qkv, nq, ne));
    DecodeQkArgs q;
    q.qkv = w + D.qkv; q.ldqkv = nq; q.qhat = w + D.qhat;
    q.kc = kc; q.vc = kc + le * es; q.pos = pos; q.max_len = max_len; q.status = status;
    TRY(launch_decode_qk(q, cs, batch, H, Hk, hd, c.norm_eps, dt, s));
    TRY(launch_decode_attn(w + D.qhat, q.kc, q.vc, pos, batch, H, Hk, hd, max_len, (float*)(w + D.part_o),
                           (float*)(w + D.part_ml), w + D.o, dt, s));
    TRY(gemv(w + D.o, hh, Wo, d, hh, EPI_RESID, x, nullptr, d, 0.f));
    TRY(gemv(x, d, W1, F, d, EPI_RELU2, nullptr, w + D.g, F, ne));
    TRY(gemv(w + D.g, F, W2, d, F, EPI_RESID, x, nullptr, d, 0.f));
  }
  return gemv(x, d, prm + ctx->layout.back().offset * es, V, d, EPI_F32, logits, nullptr, V, ne);
}

// Device scratch of nc_decode_static: one array per GPU, held until the
// process ends.  Host code never uses the symbol's name as an address (in
// host code it is only a stand-in); the address of each device's copy comes
// from hipGetSymbolAddress, looked up once per device (with that device
// current) and kept.
static __device__ __attribute__((aligned(256))) unsigned char scratch[NC_DECODE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch[kMaxDevices] = {};

int decode_scratch(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return NC_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return NC_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return NC_ERR_HIP;
    g_scratch[dev] = (char*)ptr;
  }
  *out = g_scratch[dev];
  return NC_OK;
}
}  // namespace

// =================================================================== C ABI
extern "C" {

const char* nc_strerror(int st) {
  switch (st) {
    case NC_OK: return "ok";
    case NC_ERR_CONFIG: return "invalid configuration";
    case NC_ERR_NULL: return "null pointer argument";
    case NC_ERR_WORKSPACE: return "workspace missing or too small";
    case NC_ERR_TOKEN_RANGE: return "token or target id outside [0, vocab)";
    case NC_ERR_NONFINITE: return "non-finite loss";
    case NC_ERR_HIP: return "HIP runtime error";
    case NC_ERR_UNSUPPORTED: return "unsupported shape for the GPU kernels";
    case NC_ERR_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

int nc_init(const nc_config* cfg, void* stream, nc_ctx** out) {
  if (!cfg || !out) return NC_ERR_NULL;
  *out = nullptr;
  nc_config c = *cfg;
  const int rc = validate(&c);
  if (rc) return rc;
  nc_ctx* x = new nc_ctx();
  x->cfg = c;
  x->stream = (hipStream_t)stream;
  build_layout(x);
  *out = x;
  return NC_OK;
}

void nc_destroy(nc_ctx* ctx) { delete ctx; }

int nc_get_config(const nc_ctx* ctx, nc_config* out) {
  if (!ctx || !out) return NC_ERR_NULL;
  *out = ctx->cfg;
  return NC_OK;
}

int nc_set_stream(nc_ctx* ctx, void* stream) {
  if (!ctx) return NC_ERR_NULL;
  ctx->stream = (hipStream_t)stream;
  return NC_OK;
}

uint64_t nc_param_count(const nc_ctx* ctx) { return ctx ? ctx->nparams : 0; }

int nc_param_layout(const nc_ctx* ctx, nc_tensor_desc* out, int cap) {
  if (!ctx) return -NC_ERR_NULL;
  const int n = (int)ctx->layout.size();
  for (int i = 0; i < n && i < cap && out; ++i) {
    memset(&out[i], 0, sizeof(nc_tensor_desc));
    strncpy(out[i].name, ctx->layout[i].name.c_str(), sizeof(out[i].name) - 1);
    out[i].offset = ctx->layout[i].offset;
    out[i].rows = ctx->layout[i].rows;
    out[i].cols = ctx->layout[i].cols;
  }
  return n;
}

uint64_t nc_workspace_bytes(const nc_ctx* ctx, int batch) {
  if (!ctx || batch < 1 || batch > ctx->cfg.max_batch) return 0;
  return make_plan(ctx->cfg, batch).total;
}

int nc_set_workspace(nc_ctx* ctx, void* dev_ptr, uint64_t bytes) {
  if (!ctx || !dev_ptr) return NC_ERR_NULL;
  if ((uintptr_t)dev_ptr & 255) return NC_ERR_ARG;
  ctx->ws = (char*)dev_ptr;
  ctx->ws_bytes = bytes;
  return clear_status(dev_ptr, ctx->stream);
}

int nc_forward_backward(nc_ctx* ctx, const void* params, const int32_t* tokens, const int32_t* targets, int batch,
                        float* loss, float* grads, int accumulate) {
  if (!ctx) return NC_ERR_NULL;
  if (!params || !tokens || !targets || !loss || !grads) return NC_ERR_NULL;
  if (batch < 1 || batch > ctx->cfg.max_batch || (accumulate != 0 && accumulate != 1)) return NC_ERR_ARG;
  if (!ctx->ws) return NC_ERR_WORKSPACE;
  const Plan P = make_plan(ctx->cfg, batch);
  if (ctx->ws_bytes < P.total) return NC_ERR_WORKSPACE;
  TRY(maybe_poison(ctx, P));
  TRY(launch_count_targets(targets, (long)batch * ctx->cfg.seq_len, (int*)(ctx->ws + P.status), ctx->stream));
  TRY(run_forward(ctx, P, params, tokens, batch, ctx->cfg.seq_len));
  return run_backward(ctx, P, params, tokens, targets, batch, loss, grads, accumulate, true);
}

int nc_forward_backward_accum(nc_ctx* ctx, const void* params, const int32_t* tokens, const int32_t* targets,
                              int n_micro, int micro_batch, float* loss, float* grads) {
  if (!ctx) return NC_ERR_NULL;
  if (!params || !tokens || !targets || !loss || !grads) return NC_ERR_NULL;
  if (n_micro < 1 || micro_batch < 1 || micro_batch > ctx->cfg.max_batch) return NC_ERR_ARG;
  if (!ctx->ws) return NC_ERR_WORKSPACE;
  const Plan P = make_plan(ctx->cfg, micro_batch);
  if (ctx->ws_bytes < P.total) return NC_ERR_WORKSPACE;
  const long T = ctx->cfg.seq_len;
  TRY(maybe_poison(ctx, P));
  // one count over the whole step: every microbatch is scaled by 1 / (counted targets of the step)
  TRY(launch_count_targets(targets, (long)n_micro * micro_batch * T, (int*)(ctx->ws + P.status), ctx->stream));
  for (int m = 0; m < n_micro; ++m) {
    const size_t o = (size_t)m * micro_batch * T;
    TRY(run_forward(ctx, P, params, tokens + o, micro_batch, (int)T));
    TRY(run_backward(ctx, P, params, tokens + o, targets + o, micro_batch, loss, grads, m > 0 ? 1 : 0,
                     m == n_micro - 1));
  }
  return NC_OK;
}

int nc_forward_logits(nc_ctx* ctx, const void* params, const int32_t* tokens, int batch, float* logits) {
  if (!ctx) return NC_ERR_NULL;
  if (!params || !tokens || !logits) return NC_ERR_NULL;
  if (batch < 1 || batch > ctx->cfg.max_batch) return NC_ERR_ARG;
  if (!ctx->ws) return NC_ERR_WORKSPACE;
  const Plan P = make_plan(ctx->cfg, batch);
  if (ctx->ws_bytes < P.total) return NC_ERR_WORKSPACE;
  TRY(maybe_poison(ctx, P));
  TRY(run_forward(ctx, P, params, tokens, batch, ctx->cfg.seq_len));
  const nc_config& c = ctx->cfg;
  const size_t es = c.dtype == NC_BF16 ? 2 : 4;
  const int N = batch * c.seq_len;
  GemmCall lg = mk(ctx->ws + P.z, c.d_model, true, (const char*)params + ctx->layout.back().offset * es, c.d_model,
                   true, N, c.vocab, c.d_model, c.dtype);
  lg.epi = EPI_F32; lg.e.c32 = logits; lg.e.ldc = c.vocab; lg.e.beta = 0;
  return launch_gemm(lg, ctx->stream);
}

uint64_t nc_kv_cache_bytes(const nc_ctx* ctx, int cache_batch, int max_len) {
  if (!ctx || cache_batch < 1 || max_len < 1 || max_len > kMaxCacheLen) return 0;
  const size_t es = ctx->cfg.dtype == NC_BF16 ? 2 : 4;
  return (uint64_t)ctx->cfg.depth * 2 * kv_layer_elems(ctx->cfg, cache_batch, max_len) * es;
}


uint64_t nc_decode_workspace_bytes(const nc_ctx* ctx, int batch, int max_len) {
  if (!ctx || batch < 1 || max_len < 1 || max_len > kMaxCacheLen) return 0;
  return decode_plan(ctx->cfg, batch, max_len).total;
}

int nc_prefill(nc_ctx* ctx, const void* params, const int32_t* tokens, int batch, int len, void* cache,
               int cache_batch, int max_len, int slot0, float* logits) {
  if (!ctx) return NC_ERR_NULL;
  if (!params || !tokens || !cache || !logits) return NC_ERR_NULL;
  const nc_config& c = ctx->cfg;
  if (batch < 1 || batch > c.max_batch || len < 1 || len > c.seq_len || max_len < len ||
      max_len > kMaxCacheLen || slot0 < 0 || cache_batch < slot0 + batch)
    return NC_ERR_ARG;
  if (!ctx->ws) return NC_ERR_WORKSPACE;
  const Plan P = make_plan(c, batch);
  if (ctx->ws_bytes < P.total) return NC_ERR_WORKSPACE;
  hipStream_t s = ctx->stream;
  const size_t es = c.dtype == NC_BF16 ? 2 : 4;
  TRY(run_forward(ctx, P, params, tokens, batch, len));
  const uint64_t le = kv_layer_elems(c, cache_batch, max_len);
  for (int l = 0; l < c.depth; ++l) {
    char* kc = (char*)cache + (size_t)l * 2 * le * es;
    TRY(launch_cache_fill(ctx->ws + P.layers_base + (size_t)l * P.layer_stride + P.qkv, batch, len, c.n_heads,
                          c.n_kv_heads, c.head_dim, kc, kc + le * es, max_len, slot0, c.dtype, s));
  }
  // logits of each sequence's last position: rows len-1, 2 len-1, ... of z
  SkinnyOut o;
  o.c32 = logits;
  o.ld = c.vocab;
  return launch_skinny(ctx->ws + P.z + (size_t)(len - 1) * c.d_model * es, (long)len * c.d_model,
                       (const char*)params + ctx->layout.back().offset * es, c.d_model, batch, c.vocab, c.d_model,
                       EPI_F32, o, c.dtype, s);
}

int nc_decode(nc_ctx* ctx, const void* params, const int32_t* tokens, const int32_t* pos, int batch, void* cache,
              int max_len, void* workspace, uint64_t ws_bytes, float* logits) {
  if (!ctx) return NC_ERR_NULL;
  if (!params || !tokens || !pos || !cache || !workspace || !logits) return NC_ERR_NULL;
  if (batch < 1 || max_len < 1 || max_len > kMaxCacheLen) return NC_ERR_ARG;
  if ((uintptr_t)workspace & 255) return NC_ERR_ARG;
  const DecodePlan D = decode_plan(ctx->cfg, batch, max_len);
  if (ws_bytes < D.total) return NC_ERR_WORKSPACE;
  // the status word is the workspace's first word
  return decode_run(ctx, D, params, tokens, pos, batch, cache, max_len, (char*)workspace, (int*)workspace, logits);
}

int nc_decode_static(nc_ctx* ctx, const void* params, const int32_t* tokens, const int32_t* pos, int batch,
                     void* cache, int max_len, float* logits, int* status) {
  if (!ctx) return NC_ERR_NULL;
  if (!params || !tokens || !pos || !cache || !logits || !status) return NC_ERR_NULL;
  if (batch < 1 || max_len < 1 || max_len > kMaxCacheLen) return NC_ERR_ARG;
  const DecodePlan D = decode_plan(ctx->cfg, batch, max_len);
  if (D.total > NC_DECODE_SCRATCH_BYTES) return NC_ERR_WORKSPACE;
  char* w = nullptr;
  TRY(decode_scratch(&w));
  // this call's status word starts at zero (a kernel, not a memset: the call
  // may be captured in a graph)
  TRY(clear_status(status, ctx->stream));
  return decode_run(ctx, D, params, tokens, pos, batch, cache, max_len, w, status, logits);
}

int nc_check(nc_ctx* ctx) {
  if (!ctx) return NC_ERR_NULL;
  if (!ctx->ws) return NC_ERR_WORKSPACE;
  return read_status(ctx->ws, ctx->stream);
}

int nc_debug_poison_workspace(nc_ctx* ctx, int on) {
  if (!ctx) return NC_ERR_NULL;
  if (on != 0 && on != 1) return NC_ERR_ARG;
  ctx->poison = on != 0;
  return NC_OK;
}

int nc_set_residual_fp32(nc_ctx* ctx, int on) {
  if (!ctx) return NC_ERR_NULL;
  if (on != 0 && on != 1) return NC_ERR_ARG;
  ctx->resid_fp32 = on != 0;
  return NC_OK;
}

int nc_profile_enable(nc_ctx* ctx, int on) {
  if (!ctx) return NC_ERR_NULL;
  if (on != 0 && on != 1) return NC_ERR_ARG;
  if (hipStreamSynchronize(ctx->stream) != hipSuccess) return NC_ERR_HIP;
  ctx->prof.clear();
  ctx->prof.on = on != 0;
  return NC_OK;
}

int nc_profile_read(nc_ctx* ctx, nc_prof_entry* out, int cap) {
  if (!ctx) return -NC_ERR_NULL;
  if (hipStreamSynchronize(ctx->stream) != hipSuccess) return -NC_ERR_HIP;
  double ms[PC_COUNT] = {}, fl[PC_COUNT] = {}, by[PC_COUNT] = {};
  int64_t n[PC_COUNT] = {};
  for (const auto& r : ctx->prof.recs) {
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) return -NC_ERR_HIP;
    ms[r.cls] += t;
    fl[r.cls] += r.flops;
    by[r.cls] += r.bytes;
    n[r.cls] += 1;
  }
  for (int i = 0; i < PC_COUNT && i < cap && out; ++i) {
    memset(&out[i], 0, sizeof(nc_prof_entry));
    strncpy(out[i].name, kProfNames[i], sizeof(out[i].name) - 1);
    out[i].launches = n[i];
    out[i].ms = ms[i];
    out[i].flops = fl[i];
    out[i].bytes = by[i];
  }
  return PC_COUNT;
}

int nc_op_status(void* workspace, void* stream) {
  if (!workspace) return NC_ERR_NULL;
  return read_status(workspace, (hipStream_t)stream);
}

// ------------------------------------------------------------------- ops
static size_t attn_ws_parts(int B, int H, int T, int hd, int dtype, size_t* off) {
  const size_t N = (size_t)B * T, hh = (size_t)H * hd;
  const size_t es = dtype == NC_BF16 ? 2 : 4;
  size_t o = 0;
  auto take = [&](size_t b) { size_t r = o; o += al(b); return r; };
  off[0] = take(256);            // status
  off[1] = take(N * hh * es);    // qh
  off[2] = take(N * hh * es);    // kh
  off[3] = take(N * H * 4);      // rq
  off[4] = take(N * H * 4);      // rk
  off[5] = take(N * H * 4);      // lse
  off[6] = take(N * H * 4);      // D
  off[7] = take(N * hh * 4);     // dqh fp32
  off[8] = take(N * hh * 4);     // dkh fp32
  off[9] = take((size_t)T * hd * 4);  // rope table
  off[10] = take(attn_ds_bytes(B, H, T, hd, dtype));  // dS of the backward (bf16, head_dim 128)
  return o;
}

uint64_t nc_attention_workspace_bytes(int B, int H, int T, int hd, int dtype) {
  if (B < 1 || H < 1 || T < 1 || (hd != 16 && hd != 32 && hd != 64 && hd != 128)) return 0;
  size_t off[11];
  return attn_ws_parts(B, H, T, hd, dtype, off);
}

int nc_attention_fwd_bwd(const void* q, const void* k, const void* v, const void* dout, void* out, void* dq, void* dk,
                         void* dv, int B, int H, int T, int hd, float rope_base, float eps, int dtype, void* workspace,
                         uint64_t ws_bytes, void* stream) {
  if (!q || !k || !v || !dout || !out || !dq || !dk || !dv || !workspace) return NC_ERR_NULL;
  if (B < 1 || H < 1 || T < 1 || (hd != 16 && hd != 32 && hd != 64 && hd != 128) || !(rope_base > 1.f) ||
      !(eps > 0.f))
    return NC_ERR_ARG;
  if (dtype != NC_BF16 && dtype != NC_FP32) return NC_ERR_ARG;
  if (dtype == NC_BF16 && hd != 64 && hd != 128) return NC_ERR_UNSUPPORTED;
  if (dtype == NC_BF16 && hd == 128 && attn_ds_pad(T) > kMaxDsPad) return NC_ERR_UNSUPPORTED;
  size_t off[11];
  if (ws_bytes < attn_ws_parts(B, H, T, hd, dtype, off)) return NC_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)workspace;
  const int N = B * T, hh = H * hd;
  float* cs = (float*)(w + off[9]);
  TRY(launch_rope_table(cs, T, hd, rope_base, s));
  TRY(launch_qknorm_rope_fwd(q, hh, k, hh, w + off[1], hh, w + off[2], hh, (float*)(w + off[3]), (float*)(w + off[4]),
                             cs, N, H, hd, T, eps, dtype, s));
  AttnArgs a;
  a.q = w + off[1]; a.ldq = hh;
  a.k = w + off[2]; a.ldk = hh;
  a.v = v; a.ldv = hh;
  a.o = out; a.ldo = hh;
  a.dout = dout; a.lddo = hh;
  a.lse = (float*)(w + off[5]);
  a.Dbuf = (float*)(w + off[6]);
  a.dq32 = (float*)(w + off[7]); a.lddq = hh;
  a.dk32 = (float*)(w + off[8]); a.lddk = hh;
  a.dv = dv; a.lddv = hh;
  a.dsT = w + off[10]; a.tpad = attn_ds_pad(T);
  a.B = B; a.H = H; a.T = T;
  const bool q_fused = dtype == NC_BF16 && hd == 128;  // the dQ kernel writes dq itself
  if (q_fused) {
    a.dq_pre = dq; a.lddq_pre = hh;
    a.rq = (const float*)(w + off[3]);
    a.cs = cs;
    // and the dK/dV kernel that of k, writing dk w.r.t. the pre-norm k
    a.dk_lp = dk; a.lddk_lp = hh;
    a.rk = (const float*)(w + off[4]);
  }
  TRY(launch_attn_fwd(a, hd, dtype, s));
  TRY(launch_attn_bwd(a, hd, dtype, s));
  if (q_fused) return NC_OK;
  return launch_qknorm_rope_bwd(a.dq32, hh, a.dk32, hh, w + off[1], hh, w + off[2], hh, (float*)(w + off[3]),
                                (float*)(w + off[4]), dq, hh, dk, hh, cs, N, H, hd, T, dtype, s, 0, q_fused);
}

static size_t ce_ws_parts(int N, int d, int V, int dtype, size_t* off) {
  const size_t chunk = (size_t)ce_chunk(N, V, dtype);
  const size_t es = dtype == NC_BF16 ? 2 : 4;
  size_t o = 0;
  auto take = [&](size_t b) { size_t r = o; o += al(b); return r; };
  off[0] = take(256);
  off[1] = take(ce_aux_bytes(chunk, (size_t)V, dtype));
  off[2] = take(chunk * V * es);
  off[3] = take((size_t)N * 4);
  off[4] = take(std::max(gemm_ws_bytes((int)chunk, d, V, dtype), gemm_ws_bytes(V, d, (int)chunk, dtype)));
  // bf16: W transposed once, so that dz = G W reads both operands k-contiguous
  // (the same product as in the training step)
  off[5] = take(dtype == NC_BF16 ? (size_t)V * d * 2 : 0);
  return o;
}

uint64_t nc_lmhead_ce_workspace_bytes(int N, int d, int V, int dtype) {
  if (N < 1 || d < 8 || d % 8 || V < 8 || V % 8) return 0;
  size_t off[6];
  return ce_ws_parts(N, d, V, dtype, off);
}

int nc_lmhead_ce_fwd_bwd(const void* z, const void* W, const int32_t* y, int N, int d, int V, float* loss, float* dz,
                         float* dW, int dtype, void* workspace, uint64_t ws_bytes, void* stream) {
  if (!z || !W || !y || !loss || !dz || !dW || !workspace) return NC_ERR_NULL;
  if (N < 1 || d < 8 || d % 8 || V < 8 || V % 8) return NC_ERR_ARG;
  if (dtype != NC_BF16 && dtype != NC_FP32) return NC_ERR_ARG;
  size_t off[6];
  if (ws_bytes < ce_ws_parts(N, d, V, dtype, off)) return NC_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)workspace;
  int* status = (int*)w;
  const int chunk = ce_chunk(N, V, dtype);
  const uint64_t sk_bytes = std::max(gemm_ws_bytes(chunk, d, V, dtype), gemm_ws_bytes(V, d, chunk, dtype));
  float* sk = sk_bytes ? (float*)(w + off[4]) : nullptr;
  TRY(launch_count_targets(y, N, status, s));
  TRY(lmhead_ce(z, W, y, N, d, V, (float*)(w + off[3]), dz, dW, 0, dtype, (float*)(w + off[1]), w + off[2], sk,
                sk_bytes, status, s, nullptr, dtype == NC_BF16 ? w + off[5] : nullptr));
  TRY(launch_loss_sum((float*)(w + off[3]), N, status, s));
  return launch_loss_final(loss, status, s);
}

int nc_rmsnorm_fwd(const float* x, void* y, float* r, int N, int d, float eps, int dtype, void* stream) {
  if (N == 0) return NC_OK;
  if (!x || !y || !r) return NC_ERR_NULL;
  if (N < 0 || d < 4 || d % 4 || !(eps > 0.f) || (dtype != NC_BF16 && dtype != NC_FP32)) return NC_ERR_ARG;
  return launch_rmsnorm_fwd(x, y, r, N, d, eps, dtype, (hipStream_t)stream);
}

int nc_rmsnorm_bwd(const float* dy, const void* y, const float* r, float* dx, void* dx_lp, int N, int d,
                   int accumulate, int dtype, void* stream) {
  if (N == 0) return NC_OK;
  if (!dy || !y || !r || !dx) return NC_ERR_NULL;
  if (N < 0 || d < 4 || d % 4 || (accumulate != 0 && accumulate != 1) || (dtype != NC_BF16 && dtype != NC_FP32))
    return NC_ERR_ARG;
  return launch_rmsnorm_bwd(dy, y, r, dx, dx_lp, N, d, accumulate, dtype, (hipStream_t)stream);
}

int nc_embedding_fwd(const void* E, const int32_t* tokens, float* x, int N, int d, int V, int dtype, void* workspace,
                     void* stream) {
  if (N == 0) return NC_OK;
  if (!E || !tokens || !x || !workspace) return NC_ERR_NULL;
  if (N < 0 || d < 4 || d % 4 || V < 1 || (dtype != NC_BF16 && dtype != NC_FP32)) return NC_ERR_ARG;
  return launch_embed_fwd(E, tokens, x, N, d, V, dtype, (int*)workspace, (hipStream_t)stream);
}

uint64_t nc_embedding_bwd_workspace_bytes(int N, int d, int V) {
  if (N < 0 || d < 4 || d % 4 || V < 1) return 0;
  return embed_bwd_ws_bytes(N, d, V);
}

int nc_embedding_bwd(const float* dx, const int32_t* tokens, float* dE, int N, int d, int V, int accumulate,
                     void* workspace, uint64_t ws_bytes, void* stream) {
  if (!dE || (N > 0 && (!dx || !tokens || !workspace))) return NC_ERR_NULL;
  if (N < 0 || d < 4 || d % 4 || V < 1 || (accumulate != 0 && accumulate != 1)) return NC_ERR_ARG;
  if (ws_bytes < embed_bwd_ws_bytes(N, d, V)) return NC_ERR_WORKSPACE;
  return launch_embed_bwd(dx, tokens, dE, N, d, V, accumulate, workspace, (hipStream_t)stream);
}

uint64_t nc_gemm_workspace_bytes(int M, int N, int K, int dtype) {
  if (M < 0 || N < 0 || K < 0) return 0;
  return gemm_ws_bytes(M, N, K, dtype);
}

int nc_gemm(const void* A, int lda, int a_kmajor, const void* B, int ldb, int b_kmajor, float* C, int ldc, int M,
            int N, int K, int beta, int dtype, void* workspace, uint64_t ws_bytes, void* stream) {
  if (!A || !B || !C) return NC_ERR_NULL;
  if (M < 0 || N < 0 || K < 0 || (beta != 0 && beta != 1) || (dtype != NC_BF16 && dtype != NC_FP32)) return NC_ERR_ARG;
  if (a_kmajor != 0 && a_kmajor != 1) return NC_ERR_ARG;
  if (b_kmajor != 0 && b_kmajor != 1) return NC_ERR_ARG;
  // the contiguous dimension of each operand must be a multiple of 8 (16-byte loads)
  if ((a_kmajor ? K : M) % 8 || (b_kmajor ? K : N) % 8 || N % 4) return NC_ERR_ARG;
  if (lda < (a_kmajor ? K : M) || ldb < (b_kmajor ? K : N) || ldc < N || lda % 8 || ldb % 8 || ldc % 4)
    return NC_ERR_ARG;
  GemmCall g = mk(A, lda, a_kmajor, B, ldb, b_kmajor, M, N, K, dtype);
  g.epi = EPI_F32; g.e.c32 = C; g.e.ldc = ldc; g.e.beta = beta;
  const uint64_t need = gemm_ws_bytes(M, N, K, dtype);
  if (need && workspace && ws_bytes >= need) {
    g.splitk_ws = (float*)workspace;
    g.splitk_bytes = ws_bytes;
  }
  return launch_gemm(g, (hipStream_t)stream);
}

}  // extern "C"

// ------------------------------------------------------------------ optimizer
namespace {

constexpr int kNormBlocks = 1024;
// At most kMuonBatch Muon matrices (kernels.h) share one batched launch,
// which bounds the workspace: the depth-20 model has 40 matrices of
// 1280 x 5120.

bool optim_is_adamw(const Desc& t) { return t.name == "E" || t.name == "W_lm"; }

// Muon matrices of one wide-orientation shape [r, cc] (r <= cc), in layout order.
struct MuonGroup {
  int r = 0, cc = 0;
  std::vector<int> members;  // indices into the layout
};

// State (fp32 elements): masters [nparams], then per tensor in layout order
// its AdamW moments (2 x size) or its Muon momentum (1 x size).
struct OptimPlan {
  std::vector<uint64_t> aux;  // per tensor: element offset of its first state array
  std::vector<MuonGroup> groups;
  uint64_t state_elems = 0;
  // workspace (bytes): norm partials, scalars, and per batch of up to
  // kMuonBatch matrices the iterates X0 / X1 [r, cc], the Gram matrices
  // A = X X^T and B = b A + c A A [r, r] (element type)
  size_t partials = 0, scalars = 0, X0 = 0, X1 = 0, A = 0, B2 = 0, total = 0;
};

OptimPlan optim_plan(const nc_ctx* x) {
  OptimPlan p;
  uint64_t o = x->nparams;
  size_t max_x = 0, max_a = 0;
  for (size_t ti = 0; ti < x->layout.size(); ++ti) {
    const Desc& t = x->layout[ti];
    const uint64_t n = (uint64_t)t.rows * t.cols;
    p.aux.push_back(o);
    o += optim_is_adamw(t) ? 2 * n : n;
    if (optim_is_adamw(t)) continue;
    const int r = std::min(t.rows, t.cols), cc = std::max(t.rows, t.cols);
    MuonGroup* g = nullptr;
    for (MuonGroup& q : p.groups)
      if (q.r == r && q.cc == cc) g = &q;
    if (!g) {
      p.groups.push_back(MuonGroup{r, cc, {}});
      g = &p.groups.back();
    }
    g->members.push_back((int)ti);
  }
  for (const MuonGroup& g : p.groups) {
    const size_t nb = std::min<size_t>(g.members.size(), kMuonBatch);
    max_x = std::max(max_x, nb * g.r * g.cc);
    max_a = std::max(max_a, nb * g.r * g.r);
  }
  p.state_elems = o;
  const size_t es = x->cfg.dtype == NC_BF16 ? 2 : 4;
  size_t w = 0;
  auto take = [&](size_t b) { size_t r = w; w += al(b); return r; };
  p.partials = take(std::max(kNormBlocks, kMuonBatch * kMuonBlocks) * sizeof(double));
  p.scalars = take((4 + kMuonBatch) * sizeof(float));  // grad norm, clip factor, 1/|U|_F per member
  p.X0 = take(max_x * es);
  p.X1 = take(max_x * es);
  p.A = take(max_a * es);
  p.B2 = take(max_a * es);
  p.total = w;
  return p;
}

// Schedule multiplier of step s (the formula nc.h states).
double optim_lr_mult(const nc_optim_config& c, int s) {
  if (s < c.warmup_steps) return (s + 1.0) / c.warmup_steps;
  double p = (double)(s - c.warmup_steps) / std::max(1, c.total_steps - c.warmup_steps);
  p = std::min(1.0, std::max(0.0, p));
  return c.final_frac + (1.0 - c.final_frac) * 0.5 * (1.0 + std::cos(M_PI * p));
}

bool optim_config_ok(const nc_optim_config& c) {
  auto in01 = [](float v) { return v >= 0.f && v < 1.f; };
  return c.lr_adamw >= 0.f && c.lr_muon >= 0.f && in01(c.beta1) && in01(c.beta2) && c.eps > 0.f &&
         in01(c.momentum) && c.weight_decay >= 0.f && c.clip > 0.f && c.final_frac >= 0.f && c.final_frac <= 1.f &&
         c.warmup_steps >= 1 && c.total_steps >= c.warmup_steps && c.ns_steps >= 0;
}

}  // namespace

extern "C" {

uint64_t nc_optim_state_bytes(const nc_ctx* ctx) {
  if (!ctx) return 0;
  return optim_plan(ctx).state_elems * 4;
}

uint64_t nc_optim_workspace_bytes(const nc_ctx* ctx) {
  if (!ctx) return 0;
  return optim_plan(ctx).total;
}

int nc_optim_init(nc_ctx* ctx, const void* params, void* state) {
  if (!ctx || !params || !state) return NC_ERR_NULL;
  const OptimPlan p = optim_plan(ctx);
  float* st = (float*)state;
  TRY(launch_widen(st, params, ctx->nparams, ctx->cfg.dtype, ctx->stream));
  return launch_zero(st + ctx->nparams, p.state_elems - ctx->nparams, ctx->stream);
}

int nc_optim_step(nc_ctx* ctx, const nc_optim_config* cfg, int step, const float* grads, void* params, void* state,
                  void* workspace, uint64_t ws_bytes, float* grad_norm) {
  if (!ctx || !cfg || !grads || !params || !state || !workspace) return NC_ERR_NULL;
  if (step < 0 || !optim_config_ok(*cfg)) return NC_ERR_ARG;
  auto misaligned = [](const void* q) { return ((uintptr_t)q & 15) != 0; };
  if (misaligned(grads) || misaligned(params) || misaligned(state) || misaligned(workspace)) return NC_ERR_ARG;
  const OptimPlan P = optim_plan(ctx);
  if (ws_bytes < P.total) return NC_ERR_WORKSPACE;
  hipStream_t s = ctx->stream;
  const int dt = ctx->cfg.dtype;
  const size_t es = dt == NC_BF16 ? 2 : 4;
  char* W = (char*)workspace;
  float* st = (float*)state;
  double* partials = (double*)(W + P.partials);
  float* sc = (float*)(W + P.scalars);  // [0] |g|, [1] clip factor, [2] 1/|U|_F
  const double mult = optim_lr_mult(*cfg, step);

  // global gradient norm and clip factor
  TRY(launch_sumsq(grads, ctx->nparams, partials, kNormBlocks, s));
  TRY(launch_norm_finish(partials, kNormBlocks, 1, cfg->clip, 0, sc, sc + 1, s));
  if (grad_norm) {
    if (hipMemcpyAsync(grad_norm, sc, sizeof(float), hipMemcpyDeviceToDevice, s) != hipSuccess) return NC_ERR_HIP;
  }

  const double t = step + 1.0;
  const float bc1 = (float)(1.0 - std::pow((double)cfg->beta1, t));
  const float bc2 = (float)(1.0 - std::pow((double)cfg->beta2, t));
  const float lr_a = (float)(cfg->lr_adamw * mult), lr_m = (float)(cfg->lr_muon * mult);
  const float a = 3.4445f, b = -4.7750f, c = 2.0315f;  // quintic Newton-Schulz coefficients
  // AdamW tensors
  for (size_t ti = 0; ti < ctx->layout.size(); ++ti) {
    const Desc& d = ctx->layout[ti];
    if (!optim_is_adamw(d)) continue;
    const size_t n = (size_t)d.rows * d.cols;
    float* m1 = st + P.aux[ti];
    TRY(launch_adamw(st + d.offset, m1, m1 + n, grads + d.offset, (char*)params + d.offset * es, n, sc + 1, lr_a,
                     cfg->beta1, cfg->beta2, cfg->eps, cfg->weight_decay, bc1, bc2, dt, s));
  }
  // Muon, per batch of same-shape matrices: the momentum (and the norms of
  // the Nesterov updates), each update normalised into its slot of X0 (wide
  // orientation [r, cc]), ns_steps batched iterations X <- a X + (b A +
  // c A A) X with A = X X^T as three products whose epilogues form the
  // combinations, then every member's weight update from its slot.
  float* inv = sc + 4;
  for (const MuonGroup& grp : P.groups) {
    const int r = grp.r, cc = grp.cc;
    const long xs = (long)r * cc, as = (long)r * r;  // elements per member
    for (size_t b0 = 0; b0 < grp.members.size(); b0 += kMuonBatch) {
      MuonBatch mb;
      mb.n = (int)std::min<size_t>(kMuonBatch, grp.members.size() - b0);
      mb.r = r;
      mb.cc = cc;
      for (int k = 0; k < mb.n; ++k) {
        const int ti = grp.members[b0 + k];
        const Desc& d = ctx->layout[ti];
        mb.tall[k] = d.rows > d.cols;
        mb.adj[k] = (float)std::sqrt(std::max(1.0, (double)d.rows / d.cols));
        mb.off[k] = d.offset;
        mb.buf[k] = P.aux[ti];
      }
      const int nb = mb.n;
      char* X = W + P.X0;
      char* Xn = W + P.X1;
      char* A = W + P.A;
      char* B2 = W + P.B2;
      TRY(launch_muon_momentum(grads, st, mb, sc + 1, cfg->momentum, partials, s));
      TRY(launch_norm_finish(partials, kMuonBlocks, nb, 0.f, 1, nullptr, inv, s));
      TRY(launch_ns_init(grads, st, mb, sc + 1, cfg->momentum, inv, X, dt, s));
      for (int it = 0; it < cfg->ns_steps; ++it) {
        // A = X X^T
        GemmCall g1 = mk(X, cc, true, X, cc, true, r, r, cc, dt);
        g1.batch = nb; g1.a_bstride = xs; g1.b_bstride = xs;
        g1.epi = EPI_LP; g1.e.c_lp = A; g1.e.ld_lp = r; g1.sym = true;
        TRY(launch_gemm(g1, s));
        // B = b A + c A A (A is symmetric: its rows are its columns; so is B)
        GemmCall g2 = mk(A, r, true, A, r, true, r, r, r, dt);
        g2.batch = nb; g2.a_bstride = as; g2.b_bstride = as;
        g2.epi = EPI_AXPBY; g2.e.c_lp = B2; g2.e.ld_lp = r; g2.e.aux = A; g2.e.ld_aux = r;
        g2.e.alpha = b; g2.e.beta_f = c; g2.sym = true;
        TRY(launch_gemm(g2, s));
        // X' = a X + B X
        GemmCall g3 = mk(B2, r, true, X, cc, false, r, cc, r, dt);
        g3.batch = nb; g3.a_bstride = as; g3.b_bstride = xs;
        g3.epi = EPI_AXPBY; g3.e.c_lp = Xn; g3.e.ld_lp = cc; g3.e.aux = X; g3.e.ld_aux = cc;
        g3.e.alpha = a; g3.e.beta_f = 1.f;
        TRY(launch_gemm(g3, s));
        std::swap(X, Xn);
      }
      TRY(launch_muon_apply(st, params, X, mb, lr_m, cfg->weight_decay, dt, s));
    }
  }
  return 0;
}

}  // extern "C"
