// Inference kernels ("nanochat explainer", Inference & KV Cache): prefill
// runs the prompt through the training forward and fills the cache with
// every layer's keys and values; decode runs one new token per sequence,
// appending its key and value and attending to the cached ones.
//
// Cache layout, per layer: K, then V, each [slot][head][position][hd] in the
// element type, so the keys of one (sequence, head) are one contiguous
// stream for the decode attention.
//
// Decode is bound by HBM bandwidth (every weight is read once per step for
// a handful of tokens), so its products are skinny GEMMs that stream each
// weight row once with 16-byte loads while the few activation rows sit in
// LDS, rather than MFMA tiles that would be mostly padding.
#include "common.h"
#include "kernels.h"

namespace nc {

// 16 bytes of T as floats: 8 bf16 or 4 fp32.
template <class T>
struct V16 {
  static constexpr int P = 16 / sizeof(T);
};
__device__ __forceinline__ void ld16f(const bf16* p, float* f) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
  f[0] = bf16lo_to_f32(w.x); f[1] = bf16hi_to_f32(w.x);
  f[2] = bf16lo_to_f32(w.y); f[3] = bf16hi_to_f32(w.y);
  f[4] = bf16lo_to_f32(w.z); f[5] = bf16hi_to_f32(w.z);
  f[6] = bf16lo_to_f32(w.w); f[7] = bf16hi_to_f32(w.w);
}
__device__ __forceinline__ void ld16f(const float* p, float* f) {
  const f32x4 v = *reinterpret_cast<const f32x4*>(p);
  f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
}

// ---------------------------------------------------------------- skinny GEMM
// out[m][n] = sum_k x[m][k] W[n][k] for m < M <= MB.  One wavefront per
// output row n streams W's row (k-contiguous) once; the x rows are staged in
// LDS in chunks of KC so that the four wavefronts of a workgroup share them.
template <class T, int MB>
struct SkinnyCfg {
  static constexpr int P = V16<T>::P;
  static constexpr int KC = (32768 / (MB * (int)sizeof(T))) / (64 * P) * (64 * P);
};

template <class T, int MB, int EPI>
__global__ void __launch_bounds__(256) skinny_kernel(const T* __restrict__ x, long ldx, const T* __restrict__ W,
                                                     long ldw, int M, int N, int K, SkinnyOut o) {
  constexpr int P = SkinnyCfg<T, MB>::P, KC = SkinnyCfg<T, MB>::KC;
  __shared__ __attribute__((aligned(16))) T xs[MB * KC];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + wv;
  float acc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) acc[m] = 0.f;
  for (int k0 = 0; k0 < K; k0 += KC) {
    const int kc = min(KC, K - k0);
    __syncthreads();  // the previous chunk's readers are done
    for (int idx = threadIdx.x * P; idx < MB * KC; idx += 256 * P) {
      const int m = idx / KC, kk = idx - m * KC;
      u32x4 v{0u, 0u, 0u, 0u};
      if (m < M && kk < kc) v = *reinterpret_cast<const u32x4*>(x + (size_t)m * ldx + k0 + kk);
      *reinterpret_cast<u32x4*>(xs + idx) = v;
    }
    __syncthreads();
    if (n < N) {
      const T* wr = W + (size_t)n * ldw + k0;
#pragma unroll 4
      for (int kk = lane * P; kk < kc; kk += 64 * P) {
        float wf[P];
        ld16f(wr + kk, wf);
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          float xf[P];
          ld16f(xs + m * KC + kk, xf);
#pragma unroll
          for (int e = 0; e < P; ++e) acc[m] = fmaf(wf[e], xf[e], acc[m]);
        }
      }
    }
  }
  if (n >= N) return;  // no barrier follows
#pragma unroll
  for (int m = 0; m < MB; ++m) acc[m] = wave_sum(acc[m]);
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    if (lane != m || m >= M) continue;
    const size_t i = (size_t)m * o.ld + n;
    const float v = acc[m];
    if constexpr (EPI == EPI_F32) {
      o.c32[i] = v;
    } else if constexpr (EPI == EPI_RESID) {
      o.c32[i] += v;
    } else if constexpr (EPI == EPI_LP) {
      reinterpret_cast<T*>(o.c_lp)[i] = from_f32<T>(v);
    } else if constexpr (EPI == EPI_RELU2) {
      const float r = v > 0.f ? v : 0.f;
      reinterpret_cast<T*>(o.c_lp)[i] = from_f32<T>(r * r);
    }
  }
}

template <class T, int EPI>
static void skinny_mb(const T* x, long ldx, const T* W, long ldw, int M, int N, int K, SkinnyOut o, hipStream_t s) {
  const dim3 grid((N + 3) / 4);
  if (M <= 1) skinny_kernel<T, 1, EPI><<<grid, 256, 0, s>>>(x, ldx, W, ldw, M, N, K, o);
  else if (M <= 2) skinny_kernel<T, 2, EPI><<<grid, 256, 0, s>>>(x, ldx, W, ldw, M, N, K, o);
  else if (M <= 4) skinny_kernel<T, 4, EPI><<<grid, 256, 0, s>>>(x, ldx, W, ldw, M, N, K, o);
  else if (M <= 8) skinny_kernel<T, 8, EPI><<<grid, 256, 0, s>>>(x, ldx, W, ldw, M, N, K, o);
  else skinny_kernel<T, 16, EPI><<<grid, 256, 0, s>>>(x, ldx, W, ldw, M, N, K, o);
}

template <class T>
static int skinny_t(const T* x, long ldx, const T* W, long ldw, int M, int N, int K, int epi, SkinnyOut o,
                    hipStream_t s) {
  for (int m0 = 0; m0 < M; m0 += kSkinnyM) {
    const int mc = min(kSkinnyM, M - m0);
    SkinnyOut oc = o;
    if (oc.c32) oc.c32 += (size_t)m0 * o.ld;
    if (oc.c_lp) oc.c_lp = reinterpret_cast<T*>(oc.c_lp) + (size_t)m0 * o.ld;
    const T* xc = x + (size_t)m0 * ldx;
    switch (epi) {
      case EPI_F32: skinny_mb<T, EPI_F32>(xc, ldx, W, ldw, mc, N, K, oc, s); break;
      case EPI_RESID: skinny_mb<T, EPI_RESID>(xc, ldx, W, ldw, mc, N, K, oc, s); break;
      case EPI_LP: skinny_mb<T, EPI_LP>(xc, ldx, W, ldw, mc, N, K, oc, s); break;
      case EPI_RELU2: skinny_mb<T, EPI_RELU2>(xc, ldx, W, ldw, mc, N, K, oc, s); break;
      default: return NC_ERR_ARG;
    }
    NC_LAUNCH_CHECK();
  }
  return 0;
}

int launch_skinny(const void* x, long ldx, const void* W, long ldw, int M, int N, int K, int epi, SkinnyOut o,
                  int dtype, hipStream_t s) {
  if (M <= 0 || N <= 0) return 0;
  const int P = dtype == 0 ? 8 : 4;
  if (K % P || ldx % P || ldw % P || ((uintptr_t)x & 15) || ((uintptr_t)W & 15)) return NC_ERR_ARG;
  if (dtype == 0) return skinny_t<bf16>((const bf16*)x, ldx, (const bf16*)W, ldw, M, N, K, epi, o, s);
  return skinny_t<float>((const float*)x, ldx, (const float*)W, ldw, M, N, K, epi, o, s);
}

// ---------------------------------------------------------------- QK-norm + RoPE + cache append
// Per (sequence b, head h): q and k normalised over hd (parameter-free RMS)
// and rotated by position pos[b] (pairs (i, i + hd/2), the training
// forward's convention); q̂ goes to qhat [B, hh], k̂ and the untouched v to
// the cache at (slot b, head h, position pos[b]).  blockIdx.y: 0 q, 1 k,
// 2 v.  A lane owns 4 pairs as in the training kernel.
template <class T, int HALF>
__global__ void __launch_bounds__(256) decode_qk_kernel(DecodeQkArgs a, const float* __restrict__ cs, int B, int H,
                                                        float eps) {
  constexpr int LPV = HALF / 4, VPW = 64 / LPV;
  const int w = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int vec = (blockIdx.x * 4 + (threadIdx.x >> 6)) * VPW + lane / LPV;
  const int i = (lane % LPV) * 4;
  const bool ok = vec < B * H;
  const int b = ok ? vec / H : 0, h = ok ? vec - (vec / H) * H : 0;
  const int hh = H * 2 * HALF;
  const T* src = (const T*)a.qkv + (size_t)b * a.ldqkv + w * hh + h * (2 * HALF);
  f32x4 u0{0.f, 0.f, 0.f, 0.f}, u1{0.f, 0.f, 0.f, 0.f};
  if (ok) {
    const T* s0 = src + i;
    const T* s1 = src + i + HALF;
    u0 = f32x4{to_f32(s0[0]), to_f32(s0[1]), to_f32(s0[2]), to_f32(s0[3])};
    u1 = f32x4{to_f32(s1[0]), to_f32(s1[1]), to_f32(s1[2]), to_f32(s1[3])};
  }
  float ss = u0.x * u0.x + u0.y * u0.y + u0.z * u0.z + u0.w * u0.w + u1.x * u1.x + u1.y * u1.y + u1.z * u1.z +
             u1.w * u1.w;
#pragma unroll
  for (int o = LPV / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if (!ok) return;
  int p = a.pos[b];
  if (p < 0 || p >= a.max_len) {
    if (i == 0 && w == 0 && h == 0) atomicOr(a.status, kStatusTokenRange);
    p = p < 0 ? 0 : a.max_len - 1;
  }
  f32x4 y0 = u0, y1 = u1;
  if (w < 2) {
    const float rr = 1.0f / sqrtf(ss / (float)(2 * HALF) + eps);
    const f32x4* csp = reinterpret_cast<const f32x4*>(cs + 2 * ((size_t)p * HALF + i));
    const f32x4 cs01 = csp[0], cs23 = csp[1];
    const f32x4 c{cs01.x, cs01.z, cs23.x, cs23.z}, sn{cs01.y, cs01.w, cs23.y, cs23.w};
    const f32x4 n0 = u0 * rr, n1 = u1 * rr;
    y0 = n0 * c - n1 * sn;
    y1 = n0 * sn + n1 * c;
  }
  T* dst;
  if (w == 0) dst = (T*)a.qhat + (size_t)b * hh + h * (2 * HALF);
  else dst = (T*)(w == 1 ? a.kc : a.vc) + (((size_t)b * H + h) * a.max_len + p) * (2 * HALF);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    dst[i + e] = from_f32<T>(y0[e]);
    dst[i + HALF + e] = from_f32<T>(y1[e]);
  }
}

int launch_decode_qk(const DecodeQkArgs& a, const float* cs, int B, int H, int hd, float eps, int dtype,
                     hipStream_t s) {
  const int vpw = 64 / (hd / 8);
  const dim3 grid((B * H + 4 * vpw - 1) / (4 * vpw), 3);
#define NC_QK(HALF)                                                                                   \
  do {                                                                                                \
    if (dtype == 0) decode_qk_kernel<bf16, HALF><<<grid, 256, 0, s>>>(a, cs, B, H, eps);             \
    else decode_qk_kernel<float, HALF><<<grid, 256, 0, s>>>(a, cs, B, H, eps);                       \
  } while (0)
  switch (hd) {
    case 16: NC_QK(8); break;
    case 32: NC_QK(16); break;
    case 64: NC_QK(32); break;
    case 128: NC_QK(64); break;
    default: return NC_ERR_UNSUPPORTED;
  }
#undef NC_QK
  NC_LAUNCH_CHECK();
  return 0;
}

// ---------------------------------------------------------------- decode attention
// Split-key (flash-decoding) attention of one query per (sequence, head)
// against keys 0 .. pos[b] of the cache.  Block (c, bh) takes keys
// c*KDEC .. c*KDEC + KDEC - 1: one key per thread for the scores (log2
// domain, scaled by log2(e)/sqrt(hd)), a workgroup max and sum, then
// o = sum_j p_j v_j with threads over (key stripe, dimension) so that each
// key's value row is read contiguously.  It writes the unnormalised o, the
// max and the sum; decode_combine merges the chunks.
constexpr int kDecKeys = 256;

__device__ __forceinline__ float block_max256(float v, float* red) {
  v = wave_max(v);
  const int wv = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wv] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ __forceinline__ float block_sum256(float v, float* red) {
  v = wave_sum(v);
  const int wv = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wv] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

template <class T, int HD>
__global__ void __launch_bounds__(256) decode_attn_kernel(const T* __restrict__ qhat, const T* __restrict__ kc,
                                                          const T* __restrict__ vc, const int32_t* __restrict__ pos,
                                                          int H, int max_len, int nchunk, float scale_log2,
                                                          float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int P = V16<T>::P;
  constexpr int NST = 256 / HD;  // key stripes of the value pass
  __shared__ float qs[HD];
  __shared__ float ps[kDecKeys];
  __shared__ float red[4];
  __shared__ float acc_s[NST][HD];
  const int c = blockIdx.x, bh = blockIdx.y, b = bh / H;
  int p = pos[b];
  p = p < 0 ? 0 : (p >= max_len ? max_len - 1 : p);
  const int n = p + 1;
  const int j0 = c * kDecKeys;
  float* po = part_o + ((size_t)bh * nchunk + c) * HD;
  float* pml = part_ml + ((size_t)bh * nchunk + c) * 2;
  if (j0 >= n) {  // uniform over the block
    if (threadIdx.x == 0) {
      pml[0] = -INFINITY;
      pml[1] = 0.f;
    }
    return;
  }
  const int h = bh - b * H;
  if (threadIdx.x < HD) qs[threadIdx.x] = to_f32(qhat[(size_t)b * H * HD + h * HD + threadIdx.x]);
  __syncthreads();
  const int j = j0 + threadIdx.x;
  const size_t base = (size_t)bh * max_len;
  float sc = -INFINITY;
  if (j < n) {
    const T* kr = kc + (base + j) * HD;
    float dot = 0.f;
#pragma unroll
    for (int e0 = 0; e0 < HD; e0 += P) {
      float kf[P];
      ld16f(kr + e0, kf);
#pragma unroll
      for (int e = 0; e < P; ++e) dot = fmaf(qs[e0 + e], kf[e], dot);
    }
    sc = dot * scale_log2;
  }
  const float m = block_max256(sc, red);
  const float pj = j < n ? exp2f(sc - m) : 0.f;
  ps[threadIdx.x] = pj;
  const float l = block_sum256(pj, red);  // its barriers also publish ps
  const int cnt = min(kDecKeys, n - j0);
  const int e = threadIdx.x % HD, st = threadIdx.x / HD;
  float a = 0.f;
  for (int jj = st; jj < cnt; jj += NST) a = fmaf(ps[jj], to_f32(vc[(base + j0 + jj) * HD + e]), a);
  acc_s[st][e] = a;
  __syncthreads();
  if (threadIdx.x < HD) {
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < NST; ++q) t += acc_s[q][threadIdx.x];
    po[threadIdx.x] = t;
  }
  if (threadIdx.x == 0) {
    pml[0] = m;
    pml[1] = l;
  }
}

// Per (sequence, head): merge the chunks' (o, max, sum) and write o / sum.
template <class T, int HD>
__global__ void __launch_bounds__(128) decode_combine_kernel(const float* __restrict__ part_o,
                                                             const float* __restrict__ part_ml, int nchunk,
                                                             T* __restrict__ out, int H) {
  const int bh = blockIdx.x;
  const float* pml = part_ml + (size_t)bh * nchunk * 2;
  float M = -INFINITY;
  for (int c = 0; c < nchunk; ++c) M = fmaxf(M, pml[2 * c]);
  float L = 0.f;
  for (int c = 0; c < nchunk; ++c)
    if (pml[2 * c] != -INFINITY) L += exp2f(pml[2 * c] - M) * pml[2 * c + 1];
  const int b = bh / H, h = bh - b * H;
  for (int e = threadIdx.x; e < HD; e += 128) {
    float o = 0.f;
    for (int c = 0; c < nchunk; ++c)
      if (pml[2 * c] != -INFINITY) o += exp2f(pml[2 * c] - M) * part_o[((size_t)bh * nchunk + c) * HD + e];
    out[(size_t)b * H * HD + h * HD + e] = from_f32<T>(o / L);
  }
}

int launch_decode_attn(const void* qhat, const void* kc, const void* vc, const int32_t* pos, int B, int H, int hd,
                       int max_len, float* part_o, float* part_ml, void* out, int dtype, hipStream_t s) {
  const int nchunk = (max_len + kDecKeys - 1) / kDecKeys;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)hd);
  const dim3 grid(nchunk, B * H);
#define NC_DA(HD)                                                                                              \
  do {                                                                                                         \
    if (dtype == 0) {                                                                                          \
      decode_attn_kernel<bf16, HD><<<grid, 256, 0, s>>>((const bf16*)qhat, (const bf16*)kc, (const bf16*)vc,   \
                                                        pos, H, max_len, nchunk, scale_log2, part_o, part_ml); \
      decode_combine_kernel<bf16, HD><<<B * H, 128, 0, s>>>(part_o, part_ml, nchunk, (bf16*)out, H);           \
    } else {                                                                                                   \
      decode_attn_kernel<float, HD><<<grid, 256, 0, s>>>((const float*)qhat, (const float*)kc,                \
                                                         (const float*)vc, pos, H, max_len, nchunk,            \
                                                         scale_log2, part_o, part_ml);                         \
      decode_combine_kernel<float, HD><<<B * H, 128, 0, s>>>(part_o, part_ml, nchunk, (float*)out, H);         \
    }                                                                                                          \
  } while (0)
  switch (hd) {
    case 16: NC_DA(16); break;
    case 32: NC_DA(32); break;
    case 64: NC_DA(64); break;
    case 128: NC_DA(128); break;
    default: return NC_ERR_UNSUPPORTED;
  }
#undef NC_DA
  NC_LAUNCH_CHECK();
  return 0;
}

// ---------------------------------------------------------------- prefill cache fill
// k̂ and v of rows (b, t) of the forward's qkv buffer [B*T, 3hh] (q̂, k̂
// already normalised and rotated in place) into cache slots slot0 + b,
// positions 0 .. T-1; 16-byte units.
template <class E>
__global__ void __launch_bounds__(256) cache_fill_kernel(const E* __restrict__ qkv, int T, int H, int hd,
                                                         E* __restrict__ kc, E* __restrict__ vc, int max_len,
                                                         int slot0, long units) {
  constexpr int P = V16<E>::P;
  const long u = (long)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const int hh = H * hd, per = hh / P;
  const long row = u / (2 * per);
  const int rem = (int)(u - row * 2 * per);
  const int w = rem / per, e0 = (rem - w * per) * P;
  const int b = (int)(row / T), t = (int)(row - (long)b * T);
  const int h = e0 / hd, e = e0 - h * hd;
  const E* src = qkv + row * 3 * hh + (1 + w) * hh + e0;
  E* dst = (w ? vc : kc) + (((size_t)(slot0 + b) * H + h) * max_len + t) * hd + e;
  *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
}

int launch_cache_fill(const void* qkv, int B, int T, int H, int hd, void* kc, void* vc, int max_len, int slot0,
                      int dtype, hipStream_t s) {
  const int P = dtype == 0 ? 8 : 4;
  if (hd % P) return NC_ERR_UNSUPPORTED;
  const long units = (long)B * T * 2 * (H * hd / P);
  if (units == 0) return 0;
  const unsigned grid = (unsigned)((units + 255) / 256);
  if (dtype == 0)
    cache_fill_kernel<bf16><<<grid, 256, 0, s>>>((const bf16*)qkv, T, H, hd, (bf16*)kc, (bf16*)vc, max_len, slot0,
                                                  units);
  else
    cache_fill_kernel<float><<<grid, 256, 0, s>>>((const float*)qkv, T, H, hd, (float*)kc, (float*)vc, max_len,
                                                   slot0, units);
  NC_LAUNCH_CHECK();
  return 0;
}

}  // namespace nc
