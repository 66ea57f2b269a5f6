// RMSNorm and QK-norm + RoPE kernels (forward and backward).
//
// RMSNorm, parameter-free ("nanochat explainer", Modern architecture
// choices): y = x * r with r = 1/sqrt(mean(x^2) + eps); backward
// dx = r * (dy - y * mean(dy * y)).  One wavefront per row; the row's sum of
// squares is a wavefront butterfly reduction; statistics stay in fp32.
//
// QK-norm then RoPE ("nanochat explainer", Modern architecture choices;
// Architecture Choices -> RoPE Intuition): each head vector u of length hd is
// RMS-normalised and element i is paired with i + hd/2 and rotated by
// t * base^(-2i/hd), t being the position inside the sequence.  A lane owns
// one (i, i + hd/2) pair, so the rotation needs no data exchange and the norm
// is a reduction over hd/2 lanes.
#include "common.h"
#include "kernels.h"

namespace nc {

// --------------------------------------------------------------- RMSNorm
// With `res` (bf16 [N, d], the previous sublayer's output): x += res first
// (the residual update of the stream, written back to x), then the norm.
template <class T>
__global__ void __launch_bounds__(256) rmsnorm_fwd_kernel(float* __restrict__ x, const bf16* __restrict__ res,
                                                          T* __restrict__ y, float* __restrict__ r, int N, int d,
                                                          float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;
  f32x4* xr = reinterpret_cast<f32x4*>(x + (size_t)row * d);
  const int nc4 = d >> 2;
  float ss = 0.f;
  for (int c = lane; c < nc4; c += 64) {
    f32x4 v = xr[c];
    if (res) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(res + (size_t)row * d + 4 * c);
      v += f32x4{bf16lo_to_f32(w.x), bf16hi_to_f32(w.x), bf16lo_to_f32(w.y), bf16hi_to_f32(w.y)};
      xr[c] = v;
    }
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  const float rr = 1.0f / sqrtf(ss / (float)d + eps);
  if (lane == 0) r[row] = rr;
  T* yr = y + (size_t)row * d;
  for (int c = lane; c < nc4; c += 64) {
    f32x4 v = xr[c];
    if constexpr (sizeof(T) == 2) {
      u32x2 w;
      w.x = pack_bf16x2(v.x * rr, v.y * rr);
      w.y = pack_bf16x2(v.z * rr, v.w * rr);
      *reinterpret_cast<u32x2*>(yr + 4 * c) = w;
    } else {
      *reinterpret_cast<f32x4*>(yr + 4 * c) = v * rr;
    }
  }
}

template <class T>
__device__ __forceinline__ f32x4 load4(const T* p) {
  if constexpr (sizeof(T) == 2) {
    u32x2 w = *reinterpret_cast<const u32x2*>(p);
    return f32x4{bf16lo_to_f32(w.x), bf16hi_to_f32(w.x), bf16lo_to_f32(w.y), bf16hi_to_f32(w.y)};
  } else {
    return *reinterpret_cast<const f32x4*>(p);
  }
}

template <class T>
__device__ __forceinline__ void store4(T* p, f32x4 v) {
  if constexpr (sizeof(T) == 2) {
    u32x2 w;
    w.x = pack_bf16x2(v.x, v.y);
    w.y = pack_bf16x2(v.z, v.w);
    *reinterpret_cast<u32x2*>(p) = w;
  } else {
    *reinterpret_cast<f32x4*>(p) = v;
  }
}

// dy in TD (fp32, or bf16 when the producing GEMM stored bf16)
template <class T, class TD>
__global__ void __launch_bounds__(256) rmsnorm_bwd_kernel(const TD* __restrict__ dy, const T* __restrict__ y,
                                                          const float* __restrict__ r, float* __restrict__ dx,
                                                          T* __restrict__ dx_lp, int N, int d, int accumulate) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;
  const size_t base = (size_t)row * d;
  const int nc4 = d >> 2;
  float dot = 0.f;
  for (int c = lane; c < nc4; c += 64) {
    f32x4 g = load4(dy + base + 4 * c);
    f32x4 v = load4(y + base + 4 * c);
    dot += g.x * v.x + g.y * v.y + g.z * v.z + g.w * v.w;
  }
  dot = wave_sum(dot) / (float)d;
  const float rr = r[row];
  for (int c = lane; c < nc4; c += 64) {
    f32x4 g = load4(dy + base + 4 * c);
    f32x4 v = load4(y + base + 4 * c);
    f32x4 o = (g - v * dot) * rr;
    f32x4* dp = reinterpret_cast<f32x4*>(dx + base + 4 * c);
    if (accumulate) o += *dp;
    *dp = o;
    if (dx_lp) store4(dx_lp + base + 4 * c, o);
  }
}

// The same two kernels with the row held in registers (NCH 16-byte chunks of
// the row per lane, d <= 256 * NCH): every input is read from memory once,
// instead of once for the statistic and again for the output.  At most 64
// VGPRs (eight wavefronts per SIMD), so that enough loads stay in flight.
template <class T, int NCH>
__global__ void __launch_bounds__(256, 8) rmsnorm_fwd_reg_kernel(float* __restrict__ x, const bf16* __restrict__ res,
                                                              T* __restrict__ y, float* __restrict__ r, int N, int d,
                                                              float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;
  f32x4* xr = reinterpret_cast<f32x4*>(x + (size_t)row * d);
  const int nc4 = d >> 2;
  f32x4 v[NCH];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int c = lane + 64 * k;
    v[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (c < nc4) {
      v[k] = xr[c];
      if (res) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(res + (size_t)row * d + 4 * c);
        v[k] += f32x4{bf16lo_to_f32(w.x), bf16hi_to_f32(w.x), bf16lo_to_f32(w.y), bf16hi_to_f32(w.y)};
        xr[c] = v[k];
      }
    }
    ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
  }
  ss = wave_sum(ss);
  const float rr = 1.0f / sqrtf(ss / (float)d + eps);
  if (lane == 0) r[row] = rr;
  T* yr = y + (size_t)row * d;
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int c = lane + 64 * k;
    if (c < nc4) store4(yr + 4 * c, v[k] * rr);
  }
}

template <class T, class TD, int NCH>
__global__ void __launch_bounds__(256, 8) rmsnorm_bwd_reg_kernel(const TD* __restrict__ dy, const T* __restrict__ y,
                                                              const float* __restrict__ r, float* __restrict__ dx,
                                                              T* __restrict__ dx_lp, int N, int d, int accumulate) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;
  const size_t base = (size_t)row * d;
  const int nc4 = d >> 2;
  f32x4 gk[NCH], vk[NCH];
  float dot = 0.f;
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int c = lane + 64 * k;
    gk[k] = vk[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (c < nc4) {
      gk[k] = load4(dy + base + 4 * c);
      vk[k] = load4(y + base + 4 * c);
    }
    dot += gk[k].x * vk[k].x + gk[k].y * vk[k].y + gk[k].z * vk[k].z + gk[k].w * vk[k].w;
  }
  dot = wave_sum(dot) / (float)d;
  const float rr = r[row];
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int c = lane + 64 * k;
    if (c < nc4) {
      f32x4 o = (gk[k] - vk[k] * dot) * rr;
      f32x4* dp = reinterpret_cast<f32x4*>(dx + base + 4 * c);
      if (accumulate) o += *dp;
      *dp = o;
      if (dx_lp) store4(dx_lp + base + 4 * c, o);
    }
  }
}

template <class T>
int rmsnorm_fwd_t(float* x, const void* res, void* y, float* r, int N, int d, float eps, hipStream_t s) {
  if (N == 0) return 0;
  const unsigned grid = (unsigned)((N + 3) / 4);
  const bf16* rs = (const bf16*)res;
  switch ((d + 255) / 256) {
    case 1: rmsnorm_fwd_reg_kernel<T, 1><<<grid, 256, 0, s>>>(x, rs, (T*)y, r, N, d, eps); break;
    case 2: rmsnorm_fwd_reg_kernel<T, 2><<<grid, 256, 0, s>>>(x, rs, (T*)y, r, N, d, eps); break;
    case 3: rmsnorm_fwd_reg_kernel<T, 3><<<grid, 256, 0, s>>>(x, rs, (T*)y, r, N, d, eps); break;
    case 4: rmsnorm_fwd_reg_kernel<T, 4><<<grid, 256, 0, s>>>(x, rs, (T*)y, r, N, d, eps); break;
    case 5: rmsnorm_fwd_reg_kernel<T, 5><<<grid, 256, 0, s>>>(x, rs, (T*)y, r, N, d, eps); break;
    case 6: rmsnorm_fwd_reg_kernel<T, 6><<<grid, 256, 0, s>>>(x, rs, (T*)y, r, N, d, eps); break;
    case 7: rmsnorm_fwd_reg_kernel<T, 7><<<grid, 256, 0, s>>>(x, rs, (T*)y, r, N, d, eps); break;
    case 8: rmsnorm_fwd_reg_kernel<T, 8><<<grid, 256, 0, s>>>(x, rs, (T*)y, r, N, d, eps); break;
    default: rmsnorm_fwd_kernel<T><<<grid, 256, 0, s>>>(x, rs, (T*)y, r, N, d, eps); break;
  }
  NC_LAUNCH_CHECK();
  return 0;
}

int launch_rmsnorm_fwd(const float* x, void* y, float* r, int N, int d, float eps, int dtype, hipStream_t s) {
  return dtype == 0 ? rmsnorm_fwd_t<bf16>(const_cast<float*>(x), nullptr, y, r, N, d, eps, s)
                    : rmsnorm_fwd_t<float>(const_cast<float*>(x), nullptr, y, r, N, d, eps, s);
}

int launch_rmsnorm_add_fwd(float* x, const void* res, void* y, float* r, int N, int d, float eps, hipStream_t s) {
  return rmsnorm_fwd_t<bf16>(x, res, y, r, N, d, eps, s);
}

template <class T, class TD>
int rmsnorm_bwd_t(const void* dy, const void* y, const float* r, float* dx, void* dx_lp, int N, int d, int acc,
                  hipStream_t s) {
  if (N == 0) return 0;
  const unsigned grid = (unsigned)((N + 3) / 4);
  const TD* g = (const TD*)dy;
  const T* yy = (const T*)y;
  T* lp = (T*)dx_lp;
  switch ((d + 255) / 256) {
    case 1: rmsnorm_bwd_reg_kernel<T, TD, 1><<<grid, 256, 0, s>>>(g, yy, r, dx, lp, N, d, acc); break;
    case 2: rmsnorm_bwd_reg_kernel<T, TD, 2><<<grid, 256, 0, s>>>(g, yy, r, dx, lp, N, d, acc); break;
    case 3: rmsnorm_bwd_reg_kernel<T, TD, 3><<<grid, 256, 0, s>>>(g, yy, r, dx, lp, N, d, acc); break;
    case 4: rmsnorm_bwd_reg_kernel<T, TD, 4><<<grid, 256, 0, s>>>(g, yy, r, dx, lp, N, d, acc); break;
    case 5: rmsnorm_bwd_reg_kernel<T, TD, 5><<<grid, 256, 0, s>>>(g, yy, r, dx, lp, N, d, acc); break;
    case 6: rmsnorm_bwd_reg_kernel<T, TD, 6><<<grid, 256, 0, s>>>(g, yy, r, dx, lp, N, d, acc); break;
    case 7: rmsnorm_bwd_reg_kernel<T, TD, 7><<<grid, 256, 0, s>>>(g, yy, r, dx, lp, N, d, acc); break;
    case 8: rmsnorm_bwd_reg_kernel<T, TD, 8><<<grid, 256, 0, s>>>(g, yy, r, dx, lp, N, d, acc); break;
    default: rmsnorm_bwd_kernel<T, TD><<<grid, 256, 0, s>>>(g, yy, r, dx, lp, N, d, acc); break;
  }
  NC_LAUNCH_CHECK();
  return 0;
}

int launch_rmsnorm_bwd(const float* dy, const void* y, const float* r, float* dx, void* dx_lp, int N, int d,
                       int accumulate, int dtype, hipStream_t s) {
  return dtype == 0 ? rmsnorm_bwd_t<bf16, float>(dy, y, r, dx, dx_lp, N, d, accumulate, s)
                    : rmsnorm_bwd_t<float, float>(dy, y, r, dx, dx_lp, N, d, accumulate, s);
}

int launch_rmsnorm_bwd_lpdy(const void* dy, const void* y, const float* r, float* dx, void* dx_lp, int N, int d,
                            int accumulate, hipStream_t s) {
  return rmsnorm_bwd_t<bf16, bf16>(dy, y, r, dx, dx_lp, N, d, accumulate, s);
}

// --------------------------------------------------------------- RoPE table
// cos/sin of t * base^(-2i/hd) for t < T, i < hd/2, evaluated in double so
// that large angles (t up to thousands of radians) keep full fp32 accuracy.
__global__ void rope_table_kernel(float* __restrict__ cs, int T, int half, double log2_base, int hd) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * half) return;
  const int t = idx / half, i = idx - t * half;
  const double theta = exp2(-(2.0 * i / hd) * log2_base);
  double sn, c;
  sincos((double)t * theta, &sn, &c);
  cs[2 * idx] = (float)c;
  cs[2 * idx + 1] = (float)sn;
}

int launch_rope_table(float* cs, int T, int hd, float base, hipStream_t s) {
  const int half = hd / 2;
  const int n = T * half;
  if (n == 0) return 0;
  rope_table_kernel<<<(n + 255) / 256, 256, 0, s>>>(cs, T, half, log2((double)base), hd);
  NC_LAUNCH_CHECK();
  return 0;
}

// --------------------------------------------------------------- QK-norm + RoPE
// Vectors are (token n, head h) of one tensor; `which` (blockIdx.y) selects
// the q or the k tensor.  Element (n, h, e) of tensor w lives at
// ptr[w][n * ld[w] + h * hd + e].
struct QkArgs {
  const void* in[2];
  void* out[2];
  int ld_in[2];
  int ld_out[2];
  float* r[2];  // [N, heads]
  int heads[2];  // q heads, k heads (fewer with grouped-query attention)
};

// A lane owns 4 consecutive pairs (i .. i+3, i+HALF .. i+HALF+3), so a
// vector of hd = 2*HALF elements takes HALF/4 lanes and loads are 8 bytes
// (bf16) or 16 bytes (fp32) wide.
template <int HALF>
struct QkLanes {
  static constexpr int LPV = HALF / 4;   // lanes per vector
  static constexpr int VPW = 64 / LPV;   // vectors per wavefront
};

template <class T, int HALF>
__global__ void __launch_bounds__(256) qknorm_rope_fwd_kernel(QkArgs a, const float* __restrict__ cs, int N, int H,
                                                              int Tseq, float eps) {
  constexpr int LPV = QkLanes<HALF>::LPV, VPW = QkLanes<HALF>::VPW;
  const int w = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int vec = (blockIdx.x * 4 + (threadIdx.x >> 6)) * VPW + lane / LPV;
  const int i = (lane % LPV) * 4;
  const int Hw = a.heads[w];  // heads of this tensor (H >= Hw sizes the grid)
  const bool ok = vec < N * Hw;
  const int n = ok ? vec / Hw : 0, h = ok ? vec - (vec / Hw) * Hw : 0;
  const T* src = (const T*)a.in[w] + (size_t)n * a.ld_in[w] + h * (2 * HALF);
  // the RoPE table entries first, so that their latency overlaps that of the
  // row loads instead of following the reduction
  const int t = n % Tseq;
  const f32x4* csp = reinterpret_cast<const f32x4*>(cs + 2 * (t * HALF + i));
  const f32x4 cs01 = csp[0], cs23 = csp[1];  // (cos, sin) of pairs i, i+1 | i+2, i+3
  f32x4 u0 = ok ? load4(src + i) : f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 u1 = ok ? load4(src + i + HALF) : f32x4{0.f, 0.f, 0.f, 0.f};
  float ss = u0.x * u0.x + u0.y * u0.y + u0.z * u0.z + u0.w * u0.w + u1.x * u1.x + u1.y * u1.y + u1.z * u1.z +
             u1.w * u1.w;
#pragma unroll
  for (int o = LPV / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
  const float rr = 1.0f / sqrtf(ss / (float)(2 * HALF) + eps);
  if (!ok) return;
  const f32x4 c{cs01.x, cs01.z, cs23.x, cs23.z}, sn{cs01.y, cs01.w, cs23.y, cs23.w};
  const f32x4 y0 = u0 * rr, y1 = u1 * rr;
  T* dst = (T*)a.out[w] + (size_t)n * a.ld_out[w] + h * (2 * HALF);
  store4(dst + i, y0 * c - y1 * sn);
  store4(dst + i + HALF, y0 * sn + y1 * c);
  if (i == 0) a.r[w][vec] = rr;
}

// bf16 rows with HALF a multiple of 8: the same, with 8 pairs per lane so
// that every row access is 16 bytes per lane (HALF / 8 lanes per vector).
template <int HALF>
__global__ void __launch_bounds__(256) qknorm_rope_fwd16_kernel(QkArgs a, const float* __restrict__ cs, int N, int H,
                                                                int Tseq, float eps) {
  constexpr int LPV = HALF / 8, VPW = 64 / LPV;
  const int w = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int vec = (blockIdx.x * 4 + (threadIdx.x >> 6)) * VPW + lane / LPV;
  const int i = (lane % LPV) * 8;
  const int Hw = a.heads[w];
  const bool ok = vec < N * Hw;
  const int n = ok ? vec / Hw : 0, h = ok ? vec - (vec / Hw) * Hw : 0;
  const bf16* src = (const bf16*)a.in[w] + (size_t)n * a.ld_in[w] + h * (2 * HALF);
  const int t = n % Tseq;
  const f32x4* csp = reinterpret_cast<const f32x4*>(cs + 2 * (t * HALF + i));
  f32x4 cv[4];  // (cos, sin) of pairs i .. i + 7
#pragma unroll
  for (int e = 0; e < 4; ++e) cv[e] = csp[e];
  const u32x4 z{0u, 0u, 0u, 0u};
  const u32x4 w0 = ok ? *reinterpret_cast<const u32x4*>(src + i) : z;
  const u32x4 w1 = ok ? *reinterpret_cast<const u32x4*>(src + i + HALF) : z;
  float u0[8], u1[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    u0[2 * e] = bf16lo_to_f32(w0[e]);
    u0[2 * e + 1] = bf16hi_to_f32(w0[e]);
    u1[2 * e] = bf16lo_to_f32(w1[e]);
    u1[2 * e + 1] = bf16hi_to_f32(w1[e]);
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(u0[e], u0[e], fmaf(u1[e], u1[e], ss));
#pragma unroll
  for (int o = LPV / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
  const float rr = 1.0f / sqrtf(ss / (float)(2 * HALF) + eps);
  if (!ok) return;
  u32x4 o0, o1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f32x4 c2 = cv[e];  // pairs i + 2e (c2.x, c2.y) and i + 2e + 1 (c2.z, c2.w)
    const float a0 = u0[2 * e] * rr, b0 = u1[2 * e] * rr, a1 = u0[2 * e + 1] * rr, b1 = u1[2 * e + 1] * rr;
    o0[e] = pack_bf16x2(a0 * c2.x - b0 * c2.y, a1 * c2.z - b1 * c2.w);
    o1[e] = pack_bf16x2(a0 * c2.y + b0 * c2.x, a1 * c2.w + b1 * c2.z);
  }
  bf16* dst = (bf16*)a.out[w] + (size_t)n * a.ld_out[w] + h * (2 * HALF);
  *reinterpret_cast<u32x4*>(dst + i) = o0;
  *reinterpret_cast<u32x4*>(dst + i + HALF) = o1;
  if (i == 0) a.r[w][vec] = rr;
}

// Backward: dv (fp32, gradient w.r.t. the rotated normalised vector), v the
// saved rotated normalised vector, r its saved 1/rms.  du = r (dy - y mean(dy y))
// with dy = R^T dv and y = R^T v.
struct QkBwdArgs {
  const float* dv[2];
  int ld_dv[2];
  const void* v[2];
  int ld_v[2];
  const float* r[2];
  void* du[2];
  int ld_du[2];
  int heads[2];
};

template <class T, int HALF>
__global__ void __launch_bounds__(256) qknorm_rope_bwd_kernel(QkBwdArgs a, const float* __restrict__ cs, int N,
                                                              int H, int Tseq, int w0) {
  constexpr int LPV = QkLanes<HALF>::LPV, VPW = QkLanes<HALF>::VPW;
  const int w = w0 + blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int vec = (blockIdx.x * 4 + (threadIdx.x >> 6)) * VPW + lane / LPV;
  const int i = (lane % LPV) * 4;
  const int Hw = a.heads[w];  // heads of this tensor (H >= Hw sizes the grid)
  const bool ok = vec < N * Hw;
  const int n = ok ? vec / Hw : 0, h = ok ? vec - (vec / Hw) * Hw : 0;
  const int t = n % Tseq;
  const f32x4* csp = reinterpret_cast<const f32x4*>(cs + 2 * (t * HALF + i));
  const f32x4 cs01 = csp[0], cs23 = csp[1];
  const f32x4 c{cs01.x, cs01.z, cs23.x, cs23.z}, sn{cs01.y, cs01.w, cs23.y, cs23.w};
  const float* gp = a.dv[w] + (size_t)n * a.ld_dv[w] + h * (2 * HALF);
  const T* vv = (const T*)a.v[w] + (size_t)n * a.ld_v[w] + h * (2 * HALF);
  const f32x4 z{0.f, 0.f, 0.f, 0.f};
  const f32x4 g0 = ok ? *reinterpret_cast<const f32x4*>(gp + i) : z;
  const f32x4 g1 = ok ? *reinterpret_cast<const f32x4*>(gp + i + HALF) : z;
  const f32x4 v0 = ok ? load4(vv + i) : z, v1 = ok ? load4(vv + i + HALF) : z;
  // R^T: rotation by -phi
  const f32x4 dy0 = g0 * c + g1 * sn, dy1 = g1 * c - g0 * sn;
  const f32x4 y0 = v0 * c + v1 * sn, y1 = v1 * c - v0 * sn;
  const f32x4 pr = dy0 * y0 + dy1 * y1;
  float dot = pr.x + pr.y + pr.z + pr.w;
#pragma unroll
  for (int o = LPV / 2; o >= 1; o >>= 1) dot += __shfl_xor(dot, o, 64);
  dot /= (float)(2 * HALF);
  if (!ok) return;
  const float rr = a.r[w][vec];
  T* out = (T*)a.du[w] + (size_t)n * a.ld_du[w] + h * (2 * HALF);
  store4(out + i, (dy0 - y0 * dot) * rr);
  store4(out + i + HALF, (dy1 - y1 * dot) * rr);
}

template <class T>
static int qk_fwd_dispatch(const QkArgs& a, const float* cs, int N, int H, int hd, int Tseq, float eps,
                           hipStream_t s) {
  const int vecs = N * H;
  if (vecs == 0) return 0;
  const int half = hd / 2;
  if constexpr (sizeof(T) == 2) {
    if (half == 64 || half == 32) {
      const int vpb16 = 4 * (64 / (half / 8));
      dim3 g16((vecs + vpb16 - 1) / vpb16, 2);
      if (half == 64) qknorm_rope_fwd16_kernel<64><<<g16, 256, 0, s>>>(a, cs, N, H, Tseq, eps);
      else qknorm_rope_fwd16_kernel<32><<<g16, 256, 0, s>>>(a, cs, N, H, Tseq, eps);
      NC_LAUNCH_CHECK();
      return 0;
    }
  }
  const int vpb = 4 * (64 / (half / 4));
  dim3 grid((vecs + vpb - 1) / vpb, 2);
  switch (half) {
    case 64: qknorm_rope_fwd_kernel<T, 64><<<grid, 256, 0, s>>>(a, cs, N, H, Tseq, eps); break;
    case 32: qknorm_rope_fwd_kernel<T, 32><<<grid, 256, 0, s>>>(a, cs, N, H, Tseq, eps); break;
    case 16: qknorm_rope_fwd_kernel<T, 16><<<grid, 256, 0, s>>>(a, cs, N, H, Tseq, eps); break;
    case 8: qknorm_rope_fwd_kernel<T, 8><<<grid, 256, 0, s>>>(a, cs, N, H, Tseq, eps); break;
    default: return 7;
  }
  NC_LAUNCH_CHECK();
  return 0;
}

template <class T>
static int qk_bwd_dispatch(const QkBwdArgs& a, const float* cs, int N, int H, int hd, int Tseq, hipStream_t s,
                           bool k_only) {
  const int vecs = N * (k_only ? a.heads[1] : H);
  if (vecs == 0) return 0;
  const int half = hd / 2;
  const int vpb = 4 * (64 / (half / 4));
  dim3 grid((vecs + vpb - 1) / vpb, k_only ? 1 : 2);
  const int w0 = k_only ? 1 : 0;
  switch (half) {
    case 64: qknorm_rope_bwd_kernel<T, 64><<<grid, 256, 0, s>>>(a, cs, N, H, Tseq, w0); break;
    case 32: qknorm_rope_bwd_kernel<T, 32><<<grid, 256, 0, s>>>(a, cs, N, H, Tseq, w0); break;
    case 16: qknorm_rope_bwd_kernel<T, 16><<<grid, 256, 0, s>>>(a, cs, N, H, Tseq, w0); break;
    case 8: qknorm_rope_bwd_kernel<T, 8><<<grid, 256, 0, s>>>(a, cs, N, H, Tseq, w0); break;
    default: return 7;
  }
  NC_LAUNCH_CHECK();
  return 0;
}

int launch_qknorm_rope_fwd(const void* q_in, int ldq_in, const void* k_in, int ldk_in, void* q_out, int ldq_out,
                           void* k_out, int ldk_out, float* rq, float* rk, const float* cs, int N, int H, int hd,
                           int T, float eps, int dtype, hipStream_t s, int Hk) {
  QkArgs a;
  a.heads[0] = H; a.heads[1] = Hk > 0 ? Hk : H;
  a.in[0] = q_in; a.in[1] = k_in;
  a.out[0] = q_out; a.out[1] = k_out;
  a.ld_in[0] = ldq_in; a.ld_in[1] = ldk_in;
  a.ld_out[0] = ldq_out; a.ld_out[1] = ldk_out;
  a.r[0] = rq; a.r[1] = rk;
  return dtype == 0 ? qk_fwd_dispatch<bf16>(a, cs, N, H, hd, T, eps, s)
                    : qk_fwd_dispatch<float>(a, cs, N, H, hd, T, eps, s);
}

int launch_qknorm_rope_bwd(const float* dq, int lddq, const float* dk, int lddk, const void* qh, int ldq,
                           const void* kh, int ldk, const float* rq, const float* rk, void* dq_out, int ldq_out,
                           void* dk_out, int ldk_out, const float* cs, int N, int H, int hd, int T, int dtype,
                           hipStream_t s, int Hk, bool k_only) {
  QkBwdArgs a;
  a.heads[0] = H; a.heads[1] = Hk > 0 ? Hk : H;
  a.dv[0] = dq; a.dv[1] = dk;
  a.ld_dv[0] = lddq; a.ld_dv[1] = lddk;
  a.v[0] = qh; a.v[1] = kh;
  a.ld_v[0] = ldq; a.ld_v[1] = ldk;
  a.r[0] = rq; a.r[1] = rk;
  a.du[0] = dq_out; a.du[1] = dk_out;
  a.ld_du[0] = ldq_out; a.ld_du[1] = ldk_out;
  return dtype == 0 ? qk_bwd_dispatch<bf16>(a, cs, N, H, hd, T, s, k_only)
                    : qk_bwd_dispatch<float>(a, cs, N, H, hd, T, s, k_only);
}

}  // namespace nc
