// Internal launch API between the host runtime (nc.cpp) and the kernels.
// Every launcher enqueues on stream `s` and returns 0 or an nc_status code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nc {

// ---- GEMM epilogues
enum { EPI_F32 = 0, EPI_RESID = 1, EPI_LP = 2, EPI_RELU2 = 3, EPI_DRELU2 = 4,
       EPI_F32_ACC = 5 /* internal to the GEMM: EPI_F32 with beta = 1 */,
       EPI_AXPBY = 7 /* c_lp = alpha * aux + beta * acc, aux and c_lp in the element type */ };

struct EpiArgs {
  float* c32 = nullptr;  // EPI_F32 (beta selects store / accumulate), EPI_RESID
  long ldc = 0;
  int beta = 0;
  long split_stride = 0;    // elements between split-K partial slices
  void* c_lp = nullptr;     // EPI_LP / EPI_RELU2 (g = relu(u)^2) / EPI_DRELU2 (du)
  void* c_lp2 = nullptr;    // unused
  long ld_lp = 0;
  const void* aux = nullptr;  // EPI_DRELU2: g
  long ld_aux = 0;
  // EPI_AXPBY: the two coefficients (aux is read at the output's position)
  float alpha = 0.f, beta_f = 1.f;
};

struct GemmCall {
  const void* A = nullptr;
  long lda = 0;
  bool a_k = true;
  const void* B = nullptr;
  long ldb = 0;
  bool b_k = true;
  int M = 0, N = 0, K = 0;
  int epi = EPI_F32;
  EpiArgs e;
  int dtype = 0;
  float* splitk_ws = nullptr;  // fp32 partials for split-K (EPI_F32 only); may be null
  uint64_t splitk_bytes = 0;   // its size: a split that does not fit is not used
  // Batched products (EPI_F32 without accumulation, EPI_LP, EPI_AXPBY; no
  // split-K): matrix b uses A + b * a_bstride and B + b * b_bstride
  // (elements) and writes rows [b * M, (b + 1) * M) of the output (and reads
  // the same rows of aux), so consecutive outputs are M rows apart.
  int batch = 1;
  long a_bstride = 0, b_bstride = 0;
  // The result is symmetric (M == N; EPI_LP, or EPI_AXPBY with a symmetric
  // aux): only the tiles on and above the diagonal are computed, each
  // off-diagonal one stored twice (transposed).
  bool sym = false;
};

// dst[c][r] = src[r][c] for a bf16 matrix of R rows and C columns (row
// strides lds, ldd in elements).
int launch_transpose_bf16(const void* src, int R, int C, long lds, void* dst, long ldd, hipStream_t s);
int launch_gemm(const GemmCall& g, hipStream_t s);
int gemm_splits(int M, int N, int K, int dtype);
uint64_t gemm_ws_bytes(int M, int N, int K, int dtype);

// ---- norms
int launch_rmsnorm_fwd(const float* x, void* y, float* r, int N, int d, float eps, int dtype, hipStream_t s);
int launch_rmsnorm_bwd(const float* dy, const void* y, const float* r, float* dx, void* dx_lp, int N, int d,
                       int accumulate, int dtype, hipStream_t s);
// bf16 path: x += res (bf16) then the norm (the residual update fused in)
int launch_rmsnorm_add_fwd(float* x, const void* res, void* y, float* r, int N, int d, float eps, hipStream_t s);
// bf16 path: the backward with a bf16 dy
int launch_rmsnorm_bwd_lpdy(const void* dy, const void* y, const float* r, float* dx, void* dx_lp, int N, int d,
                            int accumulate, hipStream_t s);
int launch_rope_table(float* cs, int T, int hd, float base, hipStream_t s);
// q has H heads, k has Hk (0: H) heads.
int launch_qknorm_rope_fwd(const void* q_in, int ldq_in, const void* k_in, int ldk_in, void* q_out, int ldq_out,
                           void* k_out, int ldk_out, float* rq, float* rk, const float* cs, int N, int H, int hd,
                           int T, float eps, int dtype, hipStream_t s, int Hk = 0);
// k_only: only the k tensor (the q part was finished by the attention backward)
int launch_qknorm_rope_bwd(const float* dq, int lddq, const float* dk, int lddk, const void* qh, int ldq,
                           const void* kh, int ldk, const float* rq, const float* rk, void* dq_out, int ldq_out,
                           void* dk_out, int ldk_out, const float* cs, int N, int H, int hd, int T, int dtype,
                           hipStream_t s, int Hk = 0, bool k_only = false);

// ---- embedding
int launch_embed_fwd(const void* E, const int32_t* tok, float* x, int N, int d, int V, int dtype, int* status,
                     hipStream_t s);
uint64_t embed_bwd_ws_bytes(int N, int d, int V);
int launch_embed_bwd(const float* dx, const int32_t* tok, float* dE, int N, int d, int V, int accumulate, void* ws,
                     hipStream_t s);

// ---- attention.  Element (b, t, h, e) of tensor X is X[(b*T + t) * ldX + h*hd + e].
struct AttnArgs {
  const void* q = nullptr; long ldq = 0;
  const void* k = nullptr; long ldk = 0;
  const void* v = nullptr; long ldv = 0;
  void* o = nullptr; long ldo = 0;          // forward output (read by the backward)
  const void* dout = nullptr; long lddo = 0;
  float* lse = nullptr;                     // [B*H][T], natural log
  float* Dbuf = nullptr;                    // [B*H][T]
  float* dq32 = nullptr; long lddq = 0;     // fp32 grads w.r.t. the rotated q, k
  float* dk32 = nullptr; long lddk = 0;
  void* dv = nullptr; long lddv = 0;        // grad w.r.t. v, element type
  int B = 0, H = 0, T = 0;
  int G = 1;  // query heads per key/value head: head h reads K/V head h / G (grouped-query attention)
              // dk32 / dv stay per query head (the caller sums each group)
  float scale = 0.f, scale_log2 = 0.f;      // set by the launchers
  // bf16, head_dim 128: -dS^T of every (b, h) as a [tpad][tpad] matrix (key
  // rows, query columns), written by the dK/dV kernel and read by dQ
  void* dsT = nullptr;
  long tpad = 0;  // attn_ds_pad(T)
  // bf16, head_dim 128: the dQ kernel finishes the QK-norm + RoPE backward
  // of q itself and writes dq w.r.t. the pre-norm q (bf16) here instead of
  // dq32: rq = 1/rms of q [N][H], cs = the RoPE table (cos, sin per pair)
  void* dq_pre = nullptr; long lddq_pre = 0;
  const float* rq = nullptr;
  const float* cs = nullptr;
  // bf16, head_dim 128: the dK/dV kernel writes dk (w.r.t. the rotated k)
  // in bf16 here instead of dk32; with rk as well (1/rms of k [N][H], no
  // key groups) it finishes the QK-norm + RoPE backward of k itself and
  // writes the gradient w.r.t. the pre-norm k there (cs as for q)
  void* dk_lp = nullptr; long lddk_lp = 0;
  const float* rk = nullptr;
};
// Rows (and columns) of each (b, h) block of the stored dS: T rounded up to
// 128.  A block is addressed through one buffer resource (32-bit offsets), so
// T is at most kMaxDsPad on that path.
inline long attn_ds_pad(int T) { return ((long)T + 127) / 128 * 128; }
constexpr long kMaxDsPad = 32640;
// Bytes of the stored dS for the attention backward (0 where none is stored).
inline uint64_t attn_ds_bytes(int B, int H, int T, int hd, int dtype) {
  if (dtype != 0 || hd != 128) return 0;
  const uint64_t tp = (uint64_t)attn_ds_pad(T);
  return (uint64_t)B * H * tp * tp * 2;
}
int launch_attn_fwd(AttnArgs p, int hd, int dtype, hipStream_t s);
int launch_attn_bwd(AttnArgs p, int hd, int dtype, hipStream_t s);
// dk (fp32 [N, Hk*hd], ld ldk) and dv (element type, ld ldv) of the key/value
// heads = sums over each head's G query heads of dk_q / dv_q ([N, Hk*G*hd]).
int launch_kv_group_sum(const float* dk_q, long ldq_k, const void* dv_q, long ldq_v, float* dk, long ldk, void* dv,
                        long ldv, long N, int Hk, int G, int hd, int dtype, hipStream_t s);

// ---- cross-entropy
// A negative target leaves its row out of the loss (loss row 0, G row 0); a
// target >= V sets kStatusTokenRange.  Rows are scaled by 1 / count, count =
// the number of counted targets of the whole step (0 counted: scale 0).
//
// The 256-byte status block at the start of a workspace holds the device
// status word, the count of counted targets and the loss-sum accumulator.
__host__ __device__ inline int* blk_count(int* status) { return status + 4; }
__host__ __device__ inline double* blk_loss_acc(int* status) { return reinterpret_cast<double*>(status + 8); }
// count = number of y[i] >= 0 over n ids; loss accumulator = 0
int launch_count_targets(const int32_t* y, long n, int* status, hipStream_t s);
// Finish the cross-entropy of a chunk from its bf16 logits (logits_G [rows]
// [ld], overwritten in place by G = (softmax - onehot) / count) and the loss
// rows; z [rows][ldz] and W [V][ldw] (bf16, width d) give the fp32 target logits.
int launch_ce_finish(const void* z, long ldz, const void* W, long ldw, int d, const int32_t* tgt, void* logits_G,
                     long ld, float* loss_rows, int rows, int V, int* status, hipStream_t s);
int launch_ce_rows(const float* logits, long ldl, const int32_t* tgt, void* G, long ldg, float* loss_rows, int rows,
                   int V, int dtype, int* status, hipStream_t s);
// loss accumulator += sum of the n loss rows (fixed order)
int launch_loss_sum(const float* v, int n, int* status, hipStream_t s);
// *out = accumulator / count (0 if count is 0); a non-finite result sets kStatusNonFinite
int launch_loss_final(float* out, int* status, hipStream_t s);

// ---- inference (k_infer.hip)
// Skinny products for a few rows (decode): out[m][n] = sum_k x[m][k] W[n][k],
// W [N, K] k-contiguous, x [M, ldx]; epilogues EPI_F32 / EPI_RESID (c32),
// EPI_LP / EPI_RELU2 (c_lp, element type); rows beyond kSkinnyM run in
// further passes.  K, ldx, ldw multiples of 16 bytes' worth of elements.
constexpr int kSkinnyM = 16;
struct SkinnyOut {
  float* c32 = nullptr;
  void* c_lp = nullptr;
  long ld = 0;
};
// norm_eps > 0: x is the fp32 residual stream [M, ldx] and the product takes
// its RMS-normalised rows (the forward's parameter-free RMSNorm, fused).
int launch_skinny(const void* x, long ldx, const void* W, long ldw, int M, int N, int K, int epi, SkinnyOut o,
                  int dtype, hipStream_t s, float norm_eps = 0.f);
struct DecodeQkArgs {
  const void* qkv = nullptr;  // [B, 3hh]: q | k | v
  long ldqkv = 0;
  void* qhat = nullptr;       // [B, hh]
  void* kc = nullptr;         // this layer's K cache [slot][Hk][max_len][hd]
  void* vc = nullptr;         // this layer's V cache
  const int32_t* pos = nullptr;
  int max_len = 0;
  int* status = nullptr;      // position outside [0, max_len): kStatusTokenRange
};
// q has H heads, k and v Hk (the cache holds Hk heads)
int launch_decode_qk(const DecodeQkArgs& a, const float* cs, int B, int H, int Hk, int hd, float eps, int dtype,
                     hipStream_t s);
// Attention of qhat [B, hh] against cached keys 0 .. pos[b]; out [B, hh].
// part_o: B*H*nchunk*hd floats, part_ml: B*H*nchunk*2 (nchunk = ceil(max_len / kDecodeKeys)).
constexpr int kDecodeKeys = 64;
// query head h reads cache head h / (H / Hk)
int launch_decode_attn(const void* qhat, const void* kc, const void* vc, const int32_t* pos, int B, int H, int Hk,
                       int hd, int max_len, float* part_o, float* part_ml, void* out, int dtype, hipStream_t s);
// qkv rows [H q heads | Hk k heads | Hk v heads]; the cache holds Hk heads
int launch_cache_fill(const void* qkv, int B, int T, int H, int Hk, int hd, void* kc, void* vc, int max_len,
                      int slot0, int dtype, hipStream_t s);

// ---- optimizer (k_optim.hip)
// Vectors are fp32 with 16-byte aligned starts and lengths that are multiples
// of 4 (every tensor of the layout is a multiple of 64 elements).
// partials[b] = sum of squares of block b's fixed chunk of x (nblk blocks)
int launch_sumsq(const float* x, size_t n, double* partials, int nblk, hipStream_t s);
// Per group g of nblk partials (ngroups groups): mode 0: out0 = sqrt(sum)
// (may be null), out1 = min(1, clip / (sqrt(sum) + 1e-6)); mode 1:
// out1[g] = 1 / (sqrt(sum) + 1e-7)
int launch_norm_finish(const double* partials, int nblk, int ngroups, float clip, int mode, float* out0,
                       float* out1, hipStream_t s);
int launch_adamw(float* w, float* m, float* v, const float* g, void* param, size_t n, const float* clip_scale,
                 float lr, float b1, float b2, float eps, float wd, float bc1, float bc2, int dtype, hipStream_t s);

// Up to kMuonBatch Muon matrices sharing one wide orientation [r, cc]
// (r <= cc), processed together.  A member is either [r, cc] or, when
// tall, [cc, r] (then its Newton-Schulz iterate is the transpose).
constexpr int kMuonBatch = 40;
constexpr int kMuonBlocks = 64;  // reduction blocks per member
struct MuonBatch {
  int n = 0;
  int r = 0, cc = 0;
  int tall[kMuonBatch];
  float adj[kMuonBatch];      // sqrt(max(1, rows / cols))
  uint64_t off[kMuonBatch];   // element offset in the flat layout (grads, params, masters)
  uint64_t buf[kMuonBatch];   // element offset of the momentum in the state
};
// Per member: buf = mu buf + g * clip; partials of |g * clip + mu buf|^2
// (kMuonBlocks per member, member-major)
int launch_muon_momentum(const float* grads, float* state, const MuonBatch& mb, const float* clip_scale, float mu,
                         double* partials, hipStream_t s);
// Per member: X_k = (g * clip + mu buf) * inv[k] in the wide orientation
// (element type dtype, members r * cc apart)
int launch_ns_init(const float* grads, const float* state, const MuonBatch& mb, const float* clip_scale, float mu,
                   const float* inv, void* X, int dtype, hipStream_t s);
// Per member: w -= lr (adj O + wd w) with O = X_k in the member's own
// orientation; param = w
int launch_muon_apply(float* state, void* params, const void* X, const MuonBatch& mb, float lr, float wd, int dtype,
                      hipStream_t s);
int launch_widen(float* out, const void* in, size_t n, int dtype, hipStream_t s);
int launch_zero(float* p, size_t n, hipStream_t s);

}  // namespace nc
