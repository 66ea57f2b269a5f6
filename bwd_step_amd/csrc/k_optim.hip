// Optimizer-step kernels ("nanochat explainer", The Full Pipeline ->
// Pretraining: Muon for the 2-D weights, AdamW for the embedding and the
// unembedding, cosine schedule with warmup, gradient clipping at 1.0, weight
// decay 0.1).  AdamW follows Loshchilov and Hutter's decoupled form; Muon
// follows its published description (Jordan et al., 2024): Nesterov
// momentum, then the quintic Newton-Schulz orthogonalisation of the update,
// whose matrix products run, batched over same-shape matrices, on the MFMA
// GEMM (k_gemm.hip).
//
// The state is fp32: master weights of every parameter, AdamW moments, Muon
// momentum.  The model's parameters (bf16, or fp32 on the debug path) are
// rewritten from the masters after each step.
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

// partials[b] = sum of x[i]^2 over block b's chunk [b * chunk, (b + 1) * chunk)
__global__ void __launch_bounds__(kRedThreads) sumsq_partials_kernel(const float* __restrict__ x, size_t n,
                                                                      size_t chunk, double* __restrict__ partials) {
  __shared__ double sh[kRedThreads];
  const size_t b0 = (size_t)blockIdx.x * chunk;
  const size_t b1 = b0 + chunk < n ? b0 + chunk : n;
  double acc = 0.0;
  for (size_t i = b0 + threadIdx.x; i < b1; i += kRedThreads) {
    const double v = x[i];
    acc += v * v;
  }
  const double s = block_sum_f64(acc, sh);
  if (threadIdx.x == 0) partials[blockIdx.x] = s;
}

// One block: total = sum of the partials.  mode 0 (gradient clipping):
// out0 = sqrt(total), out1 = min(1, clip / (sqrt(total) + 1e-6)); mode 1
// (Newton-Schulz normalisation): out1 = 1 / (sqrt(total) + 1e-7).
__global__ void __launch_bounds__(kRedThreads) norm_finish_kernel(const double* __restrict__ partials, int nblk,
                                                                   float clip, int mode, float* out0, float* out1) {
  __shared__ double sh[kRedThreads];
  double acc = 0.0;
  for (int i = threadIdx.x; i < nblk; i += kRedThreads) acc += partials[i];
  const double tot = block_sum_f64(acc, sh);
  if (threadIdx.x == 0) {
    const double nrm = sqrt(tot);
    if (mode == 0) {
      if (out0) *out0 = (float)nrm;
      *out1 = (float)fmin(1.0, (double)clip / (nrm + 1e-6));
    } else {
      *out1 = (float)(1.0 / (nrm + 1e-7));
    }
  }
}

int launch_sumsq(const float* x, size_t n, double* partials, int nblk, hipStream_t s) {
  if (nblk < 1) return NC_ERR_ARG;
  const size_t chunk = (n + nblk - 1) / nblk;
  sumsq_partials_kernel<<<nblk, kRedThreads, 0, s>>>(x, n, chunk > 0 ? chunk : 1, partials);
  NC_LAUNCH_CHECK();
  return 0;
}

int launch_norm_finish(const double* partials, int nblk, float clip, int mode, float* out0, float* out1,
                       hipStream_t s) {
  norm_finish_kernel<<<1, kRedThreads, 0, s>>>(partials, nblk, clip, mode, out0, out1);
  NC_LAUNCH_CHECK();
  return 0;
}

// ---------------------------------------------------------------- AdamW
// g <- g * clip factor; m <- b1 m + (1 - b1) g; v <- b2 v + (1 - b2) g^2;
// w <- w - lr (m / bc1 / (sqrt(v / bc2) + eps) + wd w); param <- w.
template <class T>
__global__ void __launch_bounds__(256) adamw_kernel(float* __restrict__ w, float* __restrict__ m,
                                                    float* __restrict__ v, const float* __restrict__ g,
                                                    T* __restrict__ param, size_t n, const float* __restrict__ cs,
                                                    float lr, float b1, float b2, float eps, float wd, float bc1,
                                                    float bc2) {
  const float sc = *cs;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const float gi = g[i] * sc;
    const float mi = b1 * m[i] + (1.0f - b1) * gi;
    const float vi = b2 * v[i] + (1.0f - b2) * gi * gi;
    const float wi = w[i];
    const float upd = (mi / bc1) / (sqrtf(vi / bc2) + eps) + wd * wi;
    const float wn = wi - lr * upd;
    m[i] = mi;
    v[i] = vi;
    w[i] = wn;
    param[i] = from_f32<T>(wn);
  }
}

int launch_adamw(float* w, float* m, float* v, const float* g, void* param, size_t n, const float* clip_scale,
                 float lr, float b1, float b2, float eps, float wd, float bc1, float bc2, int dtype, hipStream_t s) {
  if (n == 0) return 0;
  const unsigned grid = (unsigned)std::min<size_t>((n + 255) / 256, 16384);
  if (dtype == 0)
    adamw_kernel<bf16><<<grid, 256, 0, s>>>(w, m, v, g, (bf16*)param, n, clip_scale, lr, b1, b2, eps, wd, bc1, bc2);
  else
    adamw_kernel<float><<<grid, 256, 0, s>>>(w, m, v, g, (float*)param, n, clip_scale, lr, b1, b2, eps, wd, bc1,
                                             bc2);
  NC_LAUNCH_CHECK();
  return 0;
}

// ---------------------------------------------------------------- Muon
// buf <- mu buf + g * clip factor; U <- g * clip factor + mu buf (Nesterov);
// partials of sum(U^2) as in sumsq_partials_kernel.
__global__ void __launch_bounds__(kRedThreads) muon_momentum_kernel(const float* __restrict__ g,
                                                                     float* __restrict__ buf, float* __restrict__ U,
                                                                     size_t n, size_t chunk,
                                                                     const float* __restrict__ cs, float mu,
                                                                     double* __restrict__ partials) {
  __shared__ double sh[kRedThreads];
  const float sc = *cs;
  const size_t b0 = (size_t)blockIdx.x * chunk;
  const size_t b1 = b0 + chunk < n ? b0 + chunk : n;
  double acc = 0.0;
  for (size_t i = b0 + threadIdx.x; i < b1; i += kRedThreads) {
    const float gi = g[i] * sc;
    const float bi = mu * buf[i] + gi;
    const float ui = gi + mu * bi;
    buf[i] = bi;
    U[i] = ui;
    acc += (double)ui * ui;
  }
  const double s = block_sum_f64(acc, sh);
  if (threadIdx.x == 0) partials[blockIdx.x] = s;
}

int launch_muon_momentum(const float* g, float* buf, float* U, size_t n, const float* clip_scale, float mu,
                         double* partials, int nblk, hipStream_t s) {
  const size_t chunk = (n + nblk - 1) / nblk;
  muon_momentum_kernel<<<nblk, kRedThreads, 0, s>>>(g, buf, U, n, chunk > 0 ? chunk : 1, clip_scale, mu, partials);
  NC_LAUNCH_CHECK();
  return 0;
}

// X = U * inv_norm in the wide orientation: X is [rows][cols] when
// rows <= cols, else [cols][rows] (X = U^T).  32x32 tiles through LDS so
// that both the reads and the writes are row-contiguous.
template <class T>
__global__ void __launch_bounds__(256) ns_init_kernel(const float* __restrict__ U, int rows, int cols,
                                                      const float* __restrict__ inv, T* __restrict__ X, int tr) {
  __shared__ float tile[32][33];
  const float s = *inv;
  const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  if (!tr) {
    for (int y = ty; y < 32; y += 8) {
      const int r = r0 + y, c = c0 + tx;
      if (r < rows && c < cols) X[(size_t)r * cols + c] = from_f32<T>(U[(size_t)r * cols + c] * s);
    }
    return;
  }
  for (int y = ty; y < 32; y += 8) {
    const int r = r0 + y, c = c0 + tx;
    tile[y][tx] = (r < rows && c < cols) ? U[(size_t)r * cols + c] * s : 0.f;
  }
  __syncthreads();
  // X[c][r] = tile: row index of X is a column of U
  for (int y = ty; y < 32; y += 8) {
    const int c = c0 + y, r = r0 + tx;
    if (r < rows && c < cols) X[(size_t)c * rows + r] = from_f32<T>(tile[tx][y]);
  }
}

int launch_ns_init(const float* U, int rows, int cols, const float* inv_norm, void* X, int dtype, hipStream_t s) {
  dim3 grid((cols + 31) / 32, (rows + 31) / 32);
  const int tr = rows > cols;
  if (dtype == 0) ns_init_kernel<bf16><<<grid, 256, 0, s>>>(U, rows, cols, inv_norm, (bf16*)X, tr);
  else ns_init_kernel<float><<<grid, 256, 0, s>>>(U, rows, cols, inv_norm, (float*)X, tr);
  NC_LAUNCH_CHECK();
  return 0;
}

// w <- w - lr (adj O + wd w), O = X in the matrix's own orientation (X^T when
// the matrix is tall); param <- w.  32x32 tiles through LDS for the tall case.
template <class T>
__global__ void __launch_bounds__(256) muon_apply_kernel(float* __restrict__ w, T* __restrict__ param,
                                                         const T* __restrict__ X, int rows, int cols, float lr,
                                                         float adj, float wd, int tr) {
  __shared__ float tile[32][33];
  const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  if (tr) {
    // X is [cols][rows]: stage X[c0 .. c0+31][r0 .. r0+31], read it transposed
    for (int y = ty; y < 32; y += 8) {
      const int c = c0 + y, r = r0 + tx;
      tile[y][tx] = (r < rows && c < cols) ? to_f32(X[(size_t)c * rows + r]) : 0.f;
    }
    __syncthreads();
  }
  for (int y = ty; y < 32; y += 8) {
    const int r = r0 + y, c = c0 + tx;
    if (r >= rows || c >= cols) continue;
    const size_t i = (size_t)r * cols + c;
    const float o = tr ? tile[tx][y] : to_f32(X[i]);
    const float wn = w[i] - lr * (adj * o + wd * w[i]);
    w[i] = wn;
    param[i] = from_f32<T>(wn);
  }
}

int launch_muon_apply(float* w, void* param, const void* X, int rows, int cols, float lr, float adj, float wd,
                      int dtype, hipStream_t s) {
  dim3 grid((cols + 31) / 32, (rows + 31) / 32);
  const int tr = rows > cols;
  if (dtype == 0)
    muon_apply_kernel<bf16><<<grid, 256, 0, s>>>(w, (bf16*)param, (const bf16*)X, rows, cols, lr, adj, wd, tr);
  else
    muon_apply_kernel<float><<<grid, 256, 0, s>>>(w, (float*)param, (const float*)X, rows, cols, lr, adj, wd, tr);
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
