// Optimizer-step kernels ("nanochat explainer", The Full Pipeline ->
// Pretraining, where the optimizer is outlined).  Settings taken from there:
//   groups        AdamW: E, W_lm;  Muon: every layer matrix
//   lr schedule   linear warmup, then cosine decay
//   grad clipping global L2 norm, bound 1.0
//   weight decay  0.1, decoupled
// AdamW follows Loshchilov and Hutter's decoupled form; Muon
// follows its published description (Jordan et al., 2024): Nesterov
// momentum, then the quintic Newton-Schulz orthogonalisation of the update,
// whose matrix products run, batched over same-shape matrices, on the MFMA
// GEMM (k_gemm.hip).
//
// The state is fp32: master weights of every parameter, AdamW moments, Muon
// momentum.  The model's parameters (bf16, or fp32 on the debug path) are
// rewritten from the masters after each step.  Every pass here is bound by
// HBM bandwidth: 16-byte vector accesses, and one launch per batch of Muon
// matrices rather than one per matrix.
//
// Reductions (the global gradient norm, the Frobenius norm of each Muon
// update) are two-level and deterministic: every block sums a fixed
// contiguous chunk in a fixed order into an fp64 partial, one block adds the
// partials in a fixed order.  The clip factor and 1/norm stay on the device.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace nc {

constexpr int kRedThreads = 256;
constexpr int kVec = 4;                                 // floats per 16-byte access
constexpr size_t kChunkQuantum = kVec * kRedThreads;  // chunk sizes are multiples of this

__device__ __forceinline__ double block_sum_f64(double v, double* sh) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
#pragma unroll
  for (int o = kRedThreads / 2; o >= 1; o >>= 1) {
    if (t < o) sh[t] += sh[t + o];
    __syncthreads();
  }
  return sh[0];
}

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
template <class T>
__device__ __forceinline__ void st4t(T* p, float4 v) {
  if constexpr (sizeof(T) == 2) {
    struct alignas(8) B4 {
      bf16 a, b, c, d;
    };
    *reinterpret_cast<B4*>(p) =
        B4{from_f32<bf16>(v.x), from_f32<bf16>(v.y), from_f32<bf16>(v.z), from_f32<bf16>(v.w)};
  } else {
    *reinterpret_cast<float4*>(p) = v;
  }
}

// Chunk of n elements per block so that nblk blocks cover them, rounded up to
// whole vector rounds of the block (so every block starts 16-byte aligned).
static size_t chunk_for(size_t n, int nblk) {
  size_t c = (n + nblk - 1) / nblk;
  return std::max<size_t>(kChunkQuantum, (c + kChunkQuantum - 1) / kChunkQuantum * kChunkQuantum);
}

// partials[b] = sum of x[i]^2 over block b's chunk [b * chunk, (b + 1) * chunk)
__global__ void __launch_bounds__(kRedThreads) sumsq_partials_kernel(const float* __restrict__ x, size_t n,
                                                                      size_t chunk, double* __restrict__ partials) {
  __shared__ double sh[kRedThreads];
  const size_t b0 = (size_t)blockIdx.x * chunk;
  const size_t b1 = b0 + chunk < n ? b0 + chunk : n;
  double acc = 0.0;
#pragma unroll 4
  for (size_t i = b0 + kVec * threadIdx.x; i < b1; i += kChunkQuantum) {
    const float4 v = ld4(x + i);
    acc += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
  }
  const double s = block_sum_f64(acc, sh);
  if (threadIdx.x == 0) partials[blockIdx.x] = s;
}

// One block per group of nblk partials: total = their sum.  mode 0 (gradient
// clipping): out0 = sqrt(total), out1 = min(1, clip / (sqrt(total) + 1e-6));
// mode 1 (Newton-Schulz normalisation): out1[group] = 1 / (sqrt(total) + 1e-7).
__global__ void __launch_bounds__(kRedThreads) norm_finish_kernel(const double* __restrict__ partials, int nblk,
                                                                   float clip, int mode, float* out0, float* out1) {
  __shared__ double sh[kRedThreads];
  const double* pg = partials + (size_t)blockIdx.x * nblk;
  double acc = 0.0;
  for (int i = threadIdx.x; i < nblk; i += kRedThreads) acc += pg[i];
  const double tot = block_sum_f64(acc, sh);
  if (threadIdx.x == 0) {
    const double nrm = sqrt(tot);
    if (mode == 0) {
      if (out0) *out0 = (float)nrm;
      *out1 = (float)fmin(1.0, (double)clip / (nrm + 1e-6));
    } else {
      out1[blockIdx.x] = (float)(1.0 / (nrm + 1e-7));
    }
  }
}

int launch_sumsq(const float* x, size_t n, double* partials, int nblk, hipStream_t s) {
  if (nblk < 1 || n % kVec) return NC_ERR_ARG;
  sumsq_partials_kernel<<<nblk, kRedThreads, 0, s>>>(x, n, chunk_for(n, nblk), partials);
  NC_LAUNCH_CHECK();
  return 0;
}

int launch_norm_finish(const double* partials, int nblk, int ngroups, float clip, int mode, float* out0,
                       float* out1, hipStream_t s) {
  if (ngroups < 1 || (mode == 0 && ngroups != 1)) return NC_ERR_ARG;
  norm_finish_kernel<<<ngroups, kRedThreads, 0, s>>>(partials, nblk, clip, mode, out0, out1);
  NC_LAUNCH_CHECK();
  return 0;
}

// ---------------------------------------------------------------- AdamW
// g <- g * clip factor; m <- b1 m + (1 - b1) g; v <- b2 v + (1 - b2) g^2;
// w <- w - lr (m / bc1 / (sqrt(v / bc2) + eps) + wd w); param <- w.
struct AdamCoef {
  float lr, b1, b2, eps, wd, bc1, bc2;
};

__device__ __forceinline__ void adam1(float& w, float& m, float& v, float g, const AdamCoef& c) {
  m = c.b1 * m + (1.0f - c.b1) * g;
  v = c.b2 * v + (1.0f - c.b2) * g * g;
  const float upd = (m / c.bc1) / (sqrtf(v / c.bc2) + c.eps) + c.wd * w;
  w = w - c.lr * upd;
}

template <class T>
__global__ void __launch_bounds__(256) adamw_kernel(float* __restrict__ w, float* __restrict__ m,
                                                    float* __restrict__ v, const float* __restrict__ g,
                                                    T* __restrict__ param, size_t n4, const float* __restrict__ cs,
                                                    AdamCoef c) {
  const float sc = *cs;
  for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < n4; q += (size_t)gridDim.x * blockDim.x) {
    const size_t i = q * kVec;
    const float4 gv = ld4(g + i);
    float4 wv = ld4(w + i), mv = ld4(m + i), vv = ld4(v + i);
    adam1(wv.x, mv.x, vv.x, gv.x * sc, c);
    adam1(wv.y, mv.y, vv.y, gv.y * sc, c);
    adam1(wv.z, mv.z, vv.z, gv.z * sc, c);
    adam1(wv.w, mv.w, vv.w, gv.w * sc, c);
    st4(m + i, mv);
    st4(v + i, vv);
    st4(w + i, wv);
    st4t(param + i, wv);
  }
}

int launch_adamw(float* w, float* m, float* v, const float* g, void* param, size_t n, const float* clip_scale,
                 float lr, float b1, float b2, float eps, float wd, float bc1, float bc2, int dtype, hipStream_t s) {
  if (n == 0) return 0;
  if (n % kVec) return NC_ERR_ARG;
  const size_t n4 = n / kVec;
  const unsigned grid = (unsigned)std::min<size_t>((n4 + 255) / 256, 8192);
  const AdamCoef c{lr, b1, b2, eps, wd, bc1, bc2};
  if (dtype == 0) adamw_kernel<bf16><<<grid, 256, 0, s>>>(w, m, v, g, (bf16*)param, n4, clip_scale, c);
  else adamw_kernel<float><<<grid, 256, 0, s>>>(w, m, v, g, (float*)param, n4, clip_scale, c);
  NC_LAUNCH_CHECK();
  return 0;
}

// ---------------------------------------------------------------- Muon
// Block (x, k): member k's chunk x.  buf <- mu buf + g * clip; the Nesterov
// update U = g * clip + mu buf (the new buf) is not stored: its squares go to
// the partials, and ns_init forms it again from g and the new buf.
__global__ void __launch_bounds__(kRedThreads) muon_momentum_kernel(const float* __restrict__ grads,
                                                                     float* __restrict__ state, MuonBatch mb,
                                                                     size_t chunk, const float* __restrict__ cs,
                                                                     float mu, double* __restrict__ partials) {
  __shared__ double sh[kRedThreads];
  const int k = blockIdx.y;
  const float sc = *cs;
  const size_t n = (size_t)mb.r * mb.cc;
  const float* g = grads + mb.off[k];
  float* buf = state + mb.buf[k];
  const size_t b0 = (size_t)blockIdx.x * chunk;
  const size_t b1 = b0 + chunk < n ? b0 + chunk : n;
  double acc = 0.0;
#pragma unroll 2
  for (size_t i = b0 + kVec * threadIdx.x; i < b1; i += kChunkQuantum) {
    const float4 gv = ld4(g + i);
    float4 bv = ld4(buf + i);
    float4 u;
    bv.x = mu * bv.x + gv.x * sc;
    bv.y = mu * bv.y + gv.y * sc;
    bv.z = mu * bv.z + gv.z * sc;
    bv.w = mu * bv.w + gv.w * sc;
    u.x = gv.x * sc + mu * bv.x;
    u.y = gv.y * sc + mu * bv.y;
    u.z = gv.z * sc + mu * bv.z;
    u.w = gv.w * sc + mu * bv.w;
    st4(buf + i, bv);
    acc += (double)u.x * u.x + (double)u.y * u.y + (double)u.z * u.z + (double)u.w * u.w;
  }
  const double s = block_sum_f64(acc, sh);
  if (threadIdx.x == 0) partials[(size_t)k * gridDim.x + blockIdx.x] = s;
}

int launch_muon_momentum(const float* grads, float* state, const MuonBatch& mb, const float* clip_scale, float mu,
                         double* partials, hipStream_t s) {
  if (mb.n < 1 || mb.n > kMuonBatch) return NC_ERR_ARG;
  const size_t n = (size_t)mb.r * mb.cc;
  if (n % kVec) return NC_ERR_ARG;
  dim3 grid(kMuonBlocks, mb.n);
  muon_momentum_kernel<<<grid, kRedThreads, 0, s>>>(grads, state, mb, chunk_for(n, kMuonBlocks), clip_scale, mu,
                                                    partials);
  NC_LAUNCH_CHECK();
  return 0;
}

// Block (x, y, k) covers the 32 x 32 tile (rows 32 y.., columns 32 x..) of
// member k's iterate X_k [r, cc] = U * inv[k] (U^T for a tall member, whose
// tile is read along U's rows and turned through LDS, so that both the reads
// and the writes are row-contiguous).
template <class T>
__global__ void __launch_bounds__(256) ns_init_kernel(const float* __restrict__ grads,
                                                      const float* __restrict__ state, MuonBatch mb,
                                                      const float* __restrict__ cs, float mu,
                                                      const float* __restrict__ inv, T* __restrict__ X) {
  __shared__ float tile[32][33];
  const int k = blockIdx.z;
  const int r = mb.r, cc = mb.cc;
  const float sc = *cs, s = inv[k];
  const float* g = grads + mb.off[k];
  const float* buf = state + mb.buf[k];
  T* Xk = X + (size_t)k * r * cc;
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  if (!mb.tall[k]) {
    for (int y = ty; y < 32; y += 8) {
      const int i = i0 + y, j = j0 + tx;
      if (i < r && j < cc) {
        const size_t e = (size_t)i * cc + j;
        Xk[e] = from_f32<T>((g[e] * sc + mu * buf[e]) * s);
      }
    }
    return;
  }
  // the member is [cc, r]: X[i][j] = U[j][i]
  for (int y = ty; y < 32; y += 8) {
    const int j = j0 + y, i = i0 + tx;
    float u = 0.f;
    if (i < r && j < cc) {
      const size_t e = (size_t)j * r + i;
      u = (g[e] * sc + mu * buf[e]) * s;
    }
    tile[y][tx] = u;
  }
  __syncthreads();
  for (int y = ty; y < 32; y += 8) {
    const int i = i0 + y, j = j0 + tx;
    if (i < r && j < cc) Xk[(size_t)i * cc + j] = from_f32<T>(tile[tx][y]);
  }
}

int launch_ns_init(const float* grads, const float* state, const MuonBatch& mb, const float* clip_scale, float mu,
                   const float* inv, void* X, int dtype, hipStream_t s) {
  if (mb.n < 1 || mb.n > kMuonBatch) return NC_ERR_ARG;
  dim3 grid((mb.cc + 31) / 32, (mb.r + 31) / 32, mb.n);
  if (dtype == 0) ns_init_kernel<bf16><<<grid, 256, 0, s>>>(grads, state, mb, clip_scale, mu, inv, (bf16*)X);
  else ns_init_kernel<float><<<grid, 256, 0, s>>>(grads, state, mb, clip_scale, mu, inv, (float*)X);
  NC_LAUNCH_CHECK();
  return 0;
}

// Block (x, y, k): the 32 x 32 tile of X_k at rows 32 y.., columns 32 x..;
// w <- w - lr (adj O + wd w) with O = X_k (the transpose for a tall member:
// the tile goes through LDS and the weights are walked along their rows).
template <class T>
__global__ void __launch_bounds__(256) muon_apply_kernel(float* __restrict__ state, T* __restrict__ params,
                                                         const T* __restrict__ X, MuonBatch mb, float lr,
                                                         float wd) {
  __shared__ float tile[32][33];
  const int k = blockIdx.z;
  const int r = mb.r, cc = mb.cc;
  const float adj = mb.adj[k];
  float* w = state + mb.off[k];
  T* prm = params + mb.off[k];
  const T* Xk = X + (size_t)k * r * cc;
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  if (!mb.tall[k]) {
    for (int y = ty; y < 32; y += 8) {
      const int i = i0 + y, j = j0 + tx;
      if (i < r && j < cc) {
        const size_t e = (size_t)i * cc + j;
        const float wn = w[e] - lr * (adj * to_f32(Xk[e]) + wd * w[e]);
        w[e] = wn;
        prm[e] = from_f32<T>(wn);
      }
    }
    return;
  }
  for (int y = ty; y < 32; y += 8) {
    const int i = i0 + y, j = j0 + tx;
    tile[y][tx] = (i < r && j < cc) ? to_f32(Xk[(size_t)i * cc + j]) : 0.f;
  }
  __syncthreads();
  // the member is [cc, r]: W[j][i] takes X[i][j]
  for (int y = ty; y < 32; y += 8) {
    const int j = j0 + y, i = i0 + tx;
    if (i < r && j < cc) {
      const size_t e = (size_t)j * r + i;
      const float wn = w[e] - lr * (adj * tile[tx][y] + wd * w[e]);
      w[e] = wn;
      prm[e] = from_f32<T>(wn);
    }
  }
}

int launch_muon_apply(float* state, void* params, const void* X, const MuonBatch& mb, float lr, float wd, int dtype,
                      hipStream_t s) {
  if (mb.n < 1 || mb.n > kMuonBatch) return NC_ERR_ARG;
  dim3 grid((mb.cc + 31) / 32, (mb.r + 31) / 32, mb.n);
  if (dtype == 0)
    muon_apply_kernel<bf16><<<grid, 256, 0, s>>>(state, (bf16*)params, (const bf16*)X, mb, lr, wd);
  else
    muon_apply_kernel<float><<<grid, 256, 0, s>>>(state, (float*)params, (const float*)X, mb, lr, wd);
  NC_LAUNCH_CHECK();
  return 0;
}

// master (fp32) <- params (element type), the state's initial weights
template <class T>
__global__ void __launch_bounds__(256) widen_kernel(float* __restrict__ out, const T* __restrict__ in, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    out[i] = to_f32(in[i]);
}

int launch_widen(float* out, const void* in, size_t n, int dtype, hipStream_t s) {
  if (n == 0) return 0;
  const unsigned grid = (unsigned)std::min<size_t>((n + 255) / 256, 16384);
  if (dtype == 0) widen_kernel<bf16><<<grid, 256, 0, s>>>(out, (const bf16*)in, n);
  else widen_kernel<float><<<grid, 256, 0, s>>>(out, (const float*)in, n);
  NC_LAUNCH_CHECK();
  return 0;
}

__global__ void __launch_bounds__(256) zero_kernel(float* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

int launch_zero(float* p, size_t n, hipStream_t s) {
  if (n == 0) return 0;
  const unsigned grid = (unsigned)std::min<size_t>((n + 255) / 256, 16384);
  zero_kernel<<<grid, 256, 0, s>>>(p, n);
  NC_LAUNCH_CHECK();
  return 0;
}

}  // namespace nc
