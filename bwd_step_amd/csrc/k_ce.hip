// Next-token softmax cross-entropy over one chunk of logits ("nanochat
// explainer", The Full Pipeline -> Pretraining: cross-entropy between the
// predicted logits and the actual next tokens).
//
// Per row n of the chunk: lse = log sum_v exp(l_nv) (max-subtracted, fp32),
// loss_n = lse - l_{n, y_n}, and the gradient of the mean loss
// G_nv = (exp(l_nv - lse) - [v == y_n]) / count, written in the GEMM
// operand type so that dz = G W and dW = G^T z follow directly.  The mean
// runs over the rows whose target is >= 0 (count of them over the whole
// step, on the device): a negative target is the loss mask of supervised
// fine-tuning ("nanochat explainer", Supervised Fine-Tuning: the loss
// counts the assistant's tokens only), and its row gets loss 0 and G 0.  A
// workgroup owns a row: pass 1 keeps a per-thread online (max, sum), merged
// across the workgroup; pass 2 re-reads the row (now L2/MALL-resident) and
// writes G.  The mean loss is reduced over all rows in a fixed order.
// bf16 path: the row statistics come from the LM-head GEMM epilogue instead
// (per 128-column segment), and G overwrites the bf16 logits (ce_finish).
#include "common.h"
#include "kernels.h"

namespace nc {

__device__ __forceinline__ void online_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  s = s * expf(m - mn) + s2 * expf(m2 - mn);
  m = mn;
}

__device__ __forceinline__ float inv_count(const int* count) {
  const int c = *count;
  return c > 0 ? 1.0f / (float)c : 0.f;
}

template <class T>
__global__ void __launch_bounds__(256) ce_row_kernel(const float* __restrict__ logits, long ldl,
                                                     const int32_t* __restrict__ tgt, T* __restrict__ G, long ldg,
                                                     float* __restrict__ loss_rows, int V, int* __restrict__ status) {
  const int row = blockIdx.x;
  const float* l = logits + (size_t)row * ldl;
  T* gr = G + (size_t)row * ldg;
  int y = tgt[row];
  if (y < 0) {  // not counted
    if (threadIdx.x == 0) loss_rows[row] = 0.f;
    for (int c = threadIdx.x * 4; c < V; c += 1024) {
      if constexpr (sizeof(T) == 2) *reinterpret_cast<u32x2*>(gr + c) = u32x2{0u, 0u};
      else *reinterpret_cast<f32x4*>(gr + c) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  const float inv_n = inv_count(blk_count(status));
  float m = -INFINITY, s = 0.f;
  for (int c = threadIdx.x * 4; c < V; c += 1024) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(l + c);
    const float mx = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
    const float mn = fmaxf(m, mx);
    s = s * expf(m - mn) + expf(v.x - mn) + expf(v.y - mn) + expf(v.z - mn) + expf(v.w - mn);
    m = mn;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    online_merge(m, s, m2, s2);
  }
  __shared__ float sm[4], ss[4];
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sm[wv] = m; ss[wv] = s; }
  __syncthreads();
  m = sm[0]; s = ss[0];
  for (int w = 1; w < 4; ++w) online_merge(m, s, sm[w], ss[w]);
  const float lse = m + logf(s);
  if (y >= V) {
    if (threadIdx.x == 0) atomicOr(status, kStatusTokenRange);
    y = V - 1;
  }
  if (threadIdx.x == 0) loss_rows[row] = lse - l[y];
  for (int c = threadIdx.x * 4; c < V; c += 1024) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(l + c);
    float g0 = expf(v.x - lse), g1 = expf(v.y - lse), g2 = expf(v.z - lse), g3 = expf(v.w - lse);
    if (y >= c && y < c + 4) {
      const int q = y - c;
      g0 -= q == 0; g1 -= q == 1; g2 -= q == 2; g3 -= q == 3;
    }
    if constexpr (sizeof(T) == 2) {
      u32x2 w;
      w.x = pack_bf16x2(g0 * inv_n, g1 * inv_n);
      w.y = pack_bf16x2(g2 * inv_n, g3 * inv_n);
      *reinterpret_cast<u32x2*>(gr + c) = w;
    } else {
      *reinterpret_cast<f32x4*>(gr + c) = f32x4{g0 * inv_n, g1 * inv_n, g2 * inv_n, g3 * inv_n};
    }
  }
}

int launch_ce_rows(const float* logits, long ldl, const int32_t* tgt, void* G, long ldg, float* loss_rows, int rows,
                   int V, int dtype, int* status, hipStream_t s) {
  if (rows == 0) return 0;
  if (dtype == 0)
    ce_row_kernel<bf16><<<rows, 256, 0, s>>>(logits, ldl, tgt, (bf16*)G, ldg, loss_rows, V, status);
  else
    ce_row_kernel<float><<<rows, 256, 0, s>>>(logits, ldl, tgt, (float*)G, ldg, loss_rows, V, status);
  NC_LAUNCH_CHECK();
  return 0;
}

// Finish a chunk from the partials of the LM-head GEMM epilogue (bf16 path):
// a workgroup per row combines the (max, sum exp) pairs of its 128-column
// segments into lse, writes loss_n = lse - l_{n, y_n} (fp32 target logit
// from the epilogue), then overwrites the row's bf16 logits in place with
// G_nv = (exp(l_nv - lse) - [v == y_n]) / count (zeros for a row that is
// not counted).
__global__ void __launch_bounds__(256) ce_finish_kernel(const float* __restrict__ part, int nseg,
                                                        const float* __restrict__ tlog,
                                                        const int32_t* __restrict__ tgt, bf16* __restrict__ LG,
                                                        long ld, float* __restrict__ loss_rows, int V,
                                                        int* __restrict__ status) {
  const int row = blockIdx.x;
  bf16* g = LG + (size_t)row * ld;
  int y = tgt[row];
  if (y < 0) {  // not counted
    if (threadIdx.x == 0) loss_rows[row] = 0.f;
    for (int c = threadIdx.x * 8; c < V; c += 2048) *reinterpret_cast<u32x4*>(g + c) = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const float inv_n = inv_count(blk_count(status));
  const float* pr = part + (size_t)row * nseg * 2;
  float m = -INFINITY, s = 0.f;
  for (int k = threadIdx.x; k < nseg; k += 256) online_merge(m, s, pr[2 * k], pr[2 * k + 1]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    online_merge(m, s, m2, s2);
  }
  const bool y_ok = y < V;
  if (!y_ok) y = V - 1;
  // the clamped target of an out-of-range id has no fp32 logit: read the
  // stored one before the row is overwritten
  const float ty = y_ok ? tlog[row] : to_f32(g[y]);
  __shared__ float sm[4], ss[4];
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sm[wv] = m; ss[wv] = s; }
  __syncthreads();
  m = sm[0]; s = ss[0];
  for (int w = 1; w < 4; ++w) online_merge(m, s, sm[w], ss[w]);
  const float lse = m + logf(s);
  if (threadIdx.x == 0) {
    loss_rows[row] = lse - ty;
    if (!y_ok) atomicOr(status, kStatusTokenRange);
  }
  for (int c = threadIdx.x * 8; c < V; c += 2048) {
    u32x4 w = *reinterpret_cast<const u32x4*>(g + c);
    float v[8] = {bf16lo_to_f32(w.x), bf16hi_to_f32(w.x), bf16lo_to_f32(w.y), bf16hi_to_f32(w.y),
                  bf16lo_to_f32(w.z), bf16hi_to_f32(w.z), bf16lo_to_f32(w.w), bf16hi_to_f32(w.w)};
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (expf(v[e] - lse) - (c + e == y ? 1.f : 0.f)) * inv_n;
    w.x = pack_bf16x2(v[0], v[1]);
    w.y = pack_bf16x2(v[2], v[3]);
    w.z = pack_bf16x2(v[4], v[5]);
    w.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<u32x4*>(g + c) = w;
  }
}

int launch_ce_finish(const float* part, int nseg, const float* tlog, const int32_t* tgt, void* logits_G, long ld,
                     float* loss_rows, int rows, int V, int* status, hipStream_t s) {
  if (rows == 0) return 0;
  if (V % 8 || ld % 8) return NC_ERR_ARG;
  ce_finish_kernel<<<rows, 256, 0, s>>>(part, nseg, tlog, tgt, (bf16*)logits_G, ld, loss_rows, V, status);
  NC_LAUNCH_CHECK();
  return 0;
}

// count = number of ids >= 0 (one workgroup, integer: exact in any order);
// the loss accumulator starts at 0.
__global__ void __launch_bounds__(1024) count_targets_kernel(const int32_t* __restrict__ y, long n,
                                                             int* __restrict__ status) {
  __shared__ int part[1024];
  int c = 0;
  for (long i = threadIdx.x; i < n; i += 1024) c += y[i] >= 0;
  part[threadIdx.x] = c;
  __syncthreads();
  for (int off = 512; off >= 1; off >>= 1) {
    if ((int)threadIdx.x < off) part[threadIdx.x] += part[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    *blk_count(status) = part[0];
    *blk_loss_acc(status) = 0.0;
  }
}

int launch_count_targets(const int32_t* y, long n, int* status, hipStream_t s) {
  count_targets_kernel<<<1, 1024, 0, s>>>(y, n, status);
  NC_LAUNCH_CHECK();
  return 0;
}

// Loss accumulator += sum of n values in a fixed order (one workgroup, fp64).
__global__ void __launch_bounds__(1024) loss_sum_kernel(const float* __restrict__ v, int n, int* __restrict__ status) {
  __shared__ double part[1024];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 1024) s += (double)v[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int off = 512; off >= 1; off >>= 1) {
    if ((int)threadIdx.x < off) part[threadIdx.x] += part[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) *blk_loss_acc(status) += part[0];
}

__global__ void loss_final_kernel(float* __restrict__ out, int* __restrict__ status) {
  const int c = *blk_count(status);
  const float r = c > 0 ? (float)(*blk_loss_acc(status) / c) : 0.f;
  *out = r;
  if (!isfinite(r)) atomicOr(status, kStatusNonFinite);
}

int launch_loss_sum(const float* v, int n, int* status, hipStream_t s) {
  loss_sum_kernel<<<1, 1024, 0, s>>>(v, n, status);
  NC_LAUNCH_CHECK();
  return 0;
}

int launch_loss_final(float* out, int* status, hipStream_t s) {
  loss_final_kernel<<<1, 1, 0, s>>>(out, status);
  NC_LAUNCH_CHECK();
  return 0;
}

}  // namespace nc
