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
// the same from 16 raw bytes already in registers
template <class T>
__device__ __forceinline__ void cvt16f(u32x4 w, float* f) {
  if constexpr (sizeof(T) == 2) {
    f[0] = bf16lo_to_f32(w.x); f[1] = bf16hi_to_f32(w.x);
    f[2] = bf16lo_to_f32(w.y); f[3] = bf16hi_to_f32(w.y);
    f[4] = bf16lo_to_f32(w.z); f[5] = bf16hi_to_f32(w.z);
    f[6] = bf16lo_to_f32(w.w); f[7] = bf16hi_to_f32(w.w);
  } else {
    f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
  }
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

// NORM: x is the fp32 residual stream and the product takes its RMS-normalised
// rows (parameter-free, 1/sqrt(mean(x^2) + eps), the norm of the training
// forward), computed by every workgroup for its M rows while staging them.
template <class T, int MB, int EPI, bool NORM>
__global__ void __launch_bounds__(256) skinny_kernel(const void* __restrict__ xv, long ldx, const T* __restrict__ W,
                                                     long ldw, int M, int N, int K, float eps, SkinnyOut o) {
  constexpr int P = SkinnyCfg<T, MB>::P, KC = SkinnyCfg<T, MB>::KC;
  __shared__ __attribute__((aligned(16))) T xs[MB * KC];
  __shared__ float rs[MB];
  __shared__ float red[4][MB];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + wv;
  // with NORM, the first NPRE 16-byte pieces of this lane's part of the
  // weight row are loaded before the norm and the staging, so the latencies
  // overlap (measured: it slows the plain products, so they skip it)
  constexpr int NPRE = NORM ? 4 : 0;
  u32x4 wpre[NPRE > 0 ? NPRE : 1];
  {
    const int k_first = min(KC, K);
    const T* wr = W + (size_t)(n < N ? n : 0) * ldw;
#pragma unroll
    for (int it = 0; it < NPRE; ++it) {
      const int kk = lane * P + it * 64 * P;
      wpre[it] = (n < N && kk < k_first) ? *reinterpret_cast<const u32x4*>(wr + kk) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  if constexpr (NORM) {
    const float* xf = (const float*)xv;
    float ssq[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      ssq[m] = 0.f;
      if (m < M)
        for (int k = threadIdx.x * 4; k < K; k += 1024) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(xf + (size_t)m * ldx + k);
          ssq[m] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        }
      ssq[m] = wave_sum(ssq[m]);
      if (lane == 0) red[wv][m] = ssq[m];
    }
    __syncthreads();
    if (threadIdx.x < MB) {
      const float t = (red[0][threadIdx.x] + red[1][threadIdx.x]) + (red[2][threadIdx.x] + red[3][threadIdx.x]);
      rs[threadIdx.x] = 1.0f / sqrtf(t / (float)K + eps);
    }
  }
  float acc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) acc[m] = 0.f;
  for (int k0 = 0; k0 < K; k0 += KC) {
    const int kc = min(KC, K - k0);
    __syncthreads();  // the previous chunk's readers are done (and rs is published)
    for (int idx = threadIdx.x * P; idx < MB * KC; idx += 256 * P) {
      const int m = idx / KC, kk = idx - m * KC;
      if constexpr (NORM) {
        float f[P];
#pragma unroll
        for (int e = 0; e < P; ++e) f[e] = 0.f;
        if (m < M && kk < kc) {
          const float* src = (const float*)xv + (size_t)m * ldx + k0 + kk;
          const float r = rs[m];
#pragma unroll
          for (int e = 0; e < P; e += 4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(src + e);
            f[e] = v.x * r; f[e + 1] = v.y * r; f[e + 2] = v.z * r; f[e + 3] = v.w * r;
          }
        }
#pragma unroll
        for (int e = 0; e < P; ++e) xs[idx + e] = from_f32<T>(f[e]);
      } else {
        u32x4 v{0u, 0u, 0u, 0u};
        if (m < M && kk < kc) v = *reinterpret_cast<const u32x4*>((const T*)xv + (size_t)m * ldx + k0 + kk);
        *reinterpret_cast<u32x4*>(xs + idx) = v;
      }
    }
    __syncthreads();
    if (n < N) {
      const T* wr = W + (size_t)n * ldw + k0;
      int kstart = lane * P;
      if (NPRE > 0 && k0 == 0) {
#pragma unroll
        for (int it = 0; it < NPRE; ++it) {
          const int kk = lane * P + it * 64 * P;
          if (kk < kc) {
            float wf[P];
            cvt16f<T>(wpre[it], wf);
#pragma unroll
            for (int m = 0; m < MB; ++m) {
              float xf[P];
              ld16f(xs + m * KC + kk, xf);
#pragma unroll
              for (int e = 0; e < P; ++e) acc[m] = fmaf(wf[e], xf[e], acc[m]);
            }
          }
        }
        kstart += NPRE * 64 * P;
      }
#pragma unroll 4
      for (int kk = kstart; kk < kc; kk += 64 * P) {
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

template <class T, int EPI, bool NORM>
static void skinny_mb(const void* x, long ldx, const T* W, long ldw, int M, int N, int K, float eps, SkinnyOut o,
                      hipStream_t s) {
  const dim3 grid((N + 3) / 4);
  if (M <= 1) skinny_kernel<T, 1, EPI, NORM><<<grid, 256, 0, s>>>(x, ldx, W, ldw, M, N, K, eps, o);
  else if (M <= 2) skinny_kernel<T, 2, EPI, NORM><<<grid, 256, 0, s>>>(x, ldx, W, ldw, M, N, K, eps, o);
  else if (M <= 4) skinny_kernel<T, 4, EPI, NORM><<<grid, 256, 0, s>>>(x, ldx, W, ldw, M, N, K, eps, o);
  else if (M <= 8) skinny_kernel<T, 8, EPI, NORM><<<grid, 256, 0, s>>>(x, ldx, W, ldw, M, N, K, eps, o);
  else skinny_kernel<T, 16, EPI, NORM><<<grid, 256, 0, s>>>(x, ldx, W, ldw, M, N, K, eps, o);
}

template <class T, bool NORM>
static int skinny_t(const void* x, long ldx, const T* W, long ldw, int M, int N, int K, int epi, float eps,
                    SkinnyOut o, hipStream_t s) {
  const size_t xes = NORM ? 4 : sizeof(T);
  for (int m0 = 0; m0 < M; m0 += kSkinnyM) {
    const int mc = min(kSkinnyM, M - m0);
    SkinnyOut oc = o;
    if (oc.c32) oc.c32 += (size_t)m0 * o.ld;
    if (oc.c_lp) oc.c_lp = reinterpret_cast<T*>(oc.c_lp) + (size_t)m0 * o.ld;
    const void* xc = (const char*)x + (size_t)m0 * ldx * xes;
    switch (epi) {
      case EPI_F32: skinny_mb<T, EPI_F32, NORM>(xc, ldx, W, ldw, mc, N, K, eps, oc, s); break;
      case EPI_RESID: skinny_mb<T, EPI_RESID, NORM>(xc, ldx, W, ldw, mc, N, K, eps, oc, s); break;
      case EPI_LP: skinny_mb<T, EPI_LP, NORM>(xc, ldx, W, ldw, mc, N, K, eps, oc, s); break;
      case EPI_RELU2: skinny_mb<T, EPI_RELU2, NORM>(xc, ldx, W, ldw, mc, N, K, eps, oc, s); break;
      default: return NC_ERR_ARG;
    }
    NC_LAUNCH_CHECK();
  }
  return 0;
}

int launch_skinny(const void* x, long ldx, const void* W, long ldw, int M, int N, int K, int epi, SkinnyOut o,
                  int dtype, hipStream_t s, float norm_eps) {
  if (M <= 0 || N <= 0) return 0;
  const bool norm = norm_eps > 0.f;
  const int P = dtype == 0 ? 8 : 4;
  if (K % P || ldx % P || ldw % P || ((uintptr_t)x & 15) || ((uintptr_t)W & 15)) return NC_ERR_ARG;
  if (dtype == 0)
    return norm ? skinny_t<bf16, true>(x, ldx, (const bf16*)W, ldw, M, N, K, epi, norm_eps, o, s)
                : skinny_t<bf16, false>(x, ldx, (const bf16*)W, ldw, M, N, K, epi, 0.f, o, s);
  return norm ? skinny_t<float, true>(x, ldx, (const float*)W, ldw, M, N, K, epi, norm_eps, o, s)
              : skinny_t<float, false>(x, ldx, (const float*)W, ldw, M, N, K, epi, 0.f, o, s);
}

// ---------------------------------------------------------------- QK-norm + RoPE + cache append
// Per (sequence b, head h): q and k normalised over hd (parameter-free RMS)
// and rotated by position pos[b] (pairs (i, i + hd/2), the training
// forward's convention); q̂ goes to qhat [B, hh], k̂ and the untouched v to
// the cache at (slot b, head h, position pos[b]).  blockIdx.y: 0 q, 1 k,
// 2 v.  A lane owns 4 pairs as in the training kernel.
template <class T, int HALF>
__global__ void __launch_bounds__(256) decode_qk_kernel(DecodeQkArgs a, const float* __restrict__ cs, int B, int H,
                                                        int Hk, float eps) {
  constexpr int LPV = HALF / 4, VPW = 64 / LPV;
  const int w = blockIdx.y;
  const int Hw = w == 0 ? H : Hk;  // heads of this tensor
  const int lane = threadIdx.x & 63;
  const int vec = (blockIdx.x * 4 + (threadIdx.x >> 6)) * VPW + lane / LPV;
  const int i = (lane % LPV) * 4;
  const bool ok = vec < B * Hw;
  const int b = ok ? vec / Hw : 0, h = ok ? vec - (vec / Hw) * Hw : 0;
  const int hh = H * 2 * HALF, hk = Hk * 2 * HALF;
  const int col0 = w == 0 ? 0 : (w == 1 ? hh : hh + hk);  // q | k | v columns of the qkv row
  const T* src = (const T*)a.qkv + (size_t)b * a.ldqkv + col0 + h * (2 * HALF);
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
  else dst = (T*)(w == 1 ? a.kc : a.vc) + (((size_t)b * Hk + h) * a.max_len + p) * (2 * HALF);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    dst[i + e] = from_f32<T>(y0[e]);
    dst[i + HALF + e] = from_f32<T>(y1[e]);
  }
}

int launch_decode_qk(const DecodeQkArgs& a, const float* cs, int B, int H, int Hk, int hd, float eps, int dtype,
                     hipStream_t s) {
  const int vpw = 64 / (hd / 8);
  const dim3 grid((B * H + 4 * vpw - 1) / (4 * vpw), 3);
#define NC_QK(HALF)                                                                                   \
  do {                                                                                                \
    if (dtype == 0) decode_qk_kernel<bf16, HALF><<<grid, 256, 0, s>>>(a, cs, B, H, Hk, eps);         \
    else decode_qk_kernel<float, HALF><<<grid, 256, 0, s>>>(a, cs, B, H, Hk, eps);                   \
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
// against keys 0 .. pos[b] of the cache.  Block (c, bh) takes the 64 keys
// c*64 .. c*64 + 63.  Scores: a key row is read by LPR = hd / (16-byte
// vector) adjacent lanes (one 16-byte load each, so a wavefront load covers
// 64 / LPR whole rows) and reduced across them; log2 domain, scaled by
// log2(e)/sqrt(hd).  Values: a thread holds two dimensions of one key
// stripe, so a wavefront reads whole value rows.  It writes the
// unnormalised o, the max and the sum; decode_combine merges the chunks.
constexpr int kDecKeys = kDecodeKeys;

template <class T, int HD>
__global__ void __launch_bounds__(256) decode_attn_kernel(const T* __restrict__ qhat, const T* __restrict__ kc,
                                                          const T* __restrict__ vc, const int32_t* __restrict__ pos,
                                                          int H, int Hk, int max_len, int nchunk, float scale_log2,
                                                          float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int P = V16<T>::P;
  constexpr int LPR = HD / P;                 // lanes per key row (scores)
  constexpr int KPI = 64 / LPR;               // key rows per wavefront load
  constexpr int KPW = kDecKeys / 4;           // keys per wavefront
  constexpr int TPR = HD / 2;                 // threads per value row (two dims each)
  constexpr int NST = 256 / TPR;              // key stripes of the value pass
  __shared__ float ss[kDecKeys];
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
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane % LPR;  // this lane's 16-byte piece of a row
  const size_t base = ((size_t)b * Hk + h / (H / Hk)) * max_len;  // this query head's cache head
  float qf[P];
  ld16f(qhat + (size_t)b * H * HD + h * HD + g * P, qf);
#pragma unroll
  for (int it = 0; it < KPW / KPI; ++it) {
    const int jl = wv * KPW + it * KPI + lane / LPR;  // key within the chunk
    const int j = j0 + jl;
    float dot = 0.f;
    if (j < n) {
      float kf[P];
      ld16f(kc + (base + j) * HD + g * P, kf);
#pragma unroll
      for (int e = 0; e < P; ++e) dot = fmaf(qf[e], kf[e], dot);
    }
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) dot += __shfl_xor(dot, o, 64);
    if (g == 0) ss[jl] = j < n ? dot * scale_log2 : -INFINITY;
  }
  __syncthreads();
  float m = -INFINITY;
#pragma unroll 8
  for (int q = 0; q < kDecKeys; ++q) m = fmaxf(m, ss[q]);
  const int cnt = min(kDecKeys, n - j0);
  const int e2 = (threadIdx.x % TPR) * 2, st = threadIdx.x / TPR;
  float a0 = 0.f, a1 = 0.f, l = 0.f;
  // this stripe's keys: independent loads, unrolled so that several are in flight
#pragma unroll 4
  for (int jj = st; jj < cnt; jj += NST) {
    const float pj = exp2f(ss[jj] - m);
    const T* vr = vc + (base + j0 + jj) * HD + e2;
    a0 = fmaf(pj, to_f32(vr[0]), a0);
    a1 = fmaf(pj, to_f32(vr[1]), a1);
  }
  if (threadIdx.x == 0)
    for (int jj = 0; jj < cnt; ++jj) l += exp2f(ss[jj] - m);
  acc_s[st][e2] = a0;
  acc_s[st][e2 + 1] = a1;
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

// Per (sequence, head): merge the chunks that hold keys (the first
// ceil((pos+1) / 64)): w_c = exp2(m_c - M), o = sum_c w_c o_c / sum_c w_c l_c.
template <class T, int HD>
__global__ void __launch_bounds__(128) decode_combine_kernel(const float* __restrict__ part_o,
                                                             const float* __restrict__ part_ml,
                                                             const int32_t* __restrict__ pos, int max_len,
                                                             int nchunk, T* __restrict__ out, int H) {
  constexpr int kMaxW = 1024;  // chunk weights kept in LDS (65536 / 64)
  __shared__ float wgt[kMaxW];
  __shared__ float red[2][2];
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh - b * H;
  const int wv = threadIdx.x >> 6;
  int p = pos[b];
  p = p < 0 ? 0 : (p >= max_len ? max_len - 1 : p);
  const int nc = min(min(nchunk, kMaxW), p / kDecKeys + 1);
  const float* pml = part_ml + (size_t)bh * nchunk * 2;
  float M = -INFINITY;
  for (int c = threadIdx.x; c < nc; c += 128) M = fmaxf(M, pml[2 * c]);
  M = wave_max(M);
  if ((threadIdx.x & 63) == 0) red[0][wv] = M;
  __syncthreads();
  M = fmaxf(red[0][0], red[0][1]);
  float L = 0.f;
  for (int c = threadIdx.x; c < nc; c += 128) {
    const float wc = exp2f(pml[2 * c] - M);
    wgt[c] = wc;
    L += wc * pml[2 * c + 1];
  }
  L = wave_sum(L);
  if ((threadIdx.x & 63) == 0) red[1][wv] = L;
  __syncthreads();  // also publishes wgt
  const float inv = 1.0f / (red[1][0] + red[1][1]);
  for (int e = threadIdx.x; e < HD; e += 128) {
    float o = 0.f;
    for (int c = 0; c < nc; ++c) o = fmaf(wgt[c], part_o[((size_t)bh * nchunk + c) * HD + e], o);
    out[(size_t)b * H * HD + h * HD + e] = from_f32<T>(o * inv);
  }
}

template <class T, int HD>
static int decode_attn_t(const void* qhat, const void* kc, const void* vc, const int32_t* pos, int B, int H,
                         int Hk, int max_len, float* part_o, float* part_ml, void* out, hipStream_t s) {
  // a wavefront's 16 keys must be whole multiples of its per-load rows
  if constexpr ((kDecKeys / 4) % (64 / (HD / V16<T>::P)) != 0) {
    return NC_ERR_UNSUPPORTED;
  } else {
    const int nchunk = (max_len + kDecKeys - 1) / kDecKeys;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)HD);
    decode_attn_kernel<T, HD><<<dim3(nchunk, B * H), 256, 0, s>>>((const T*)qhat, (const T*)kc, (const T*)vc, pos,
                                                                  H, Hk, max_len, nchunk, scale_log2, part_o,
                                                                  part_ml);
    decode_combine_kernel<T, HD><<<B * H, 128, 0, s>>>(part_o, part_ml, pos, max_len, nchunk, (T*)out, H);
    NC_LAUNCH_CHECK();
    return 0;
  }
}

int launch_decode_attn(const void* qhat, const void* kc, const void* vc, const int32_t* pos, int B, int H, int Hk,
                       int hd, int max_len, float* part_o, float* part_ml, void* out, int dtype, hipStream_t s) {
  if (Hk < 1 || H % Hk) return NC_ERR_ARG;
#define NC_DA(HD)                                                                                    \
  return dtype == 0 ? decode_attn_t<bf16, HD>(qhat, kc, vc, pos, B, H, Hk, max_len, part_o, part_ml, out, s) \
                    : decode_attn_t<float, HD>(qhat, kc, vc, pos, B, H, Hk, max_len, part_o, part_ml, out, s)
  switch (hd) {
    case 16: NC_DA(16);
    case 32: NC_DA(32);
    case 64: NC_DA(64);
    case 128: NC_DA(128);
    default: return NC_ERR_UNSUPPORTED;
  }
#undef NC_DA
}

// ---------------------------------------------------------------- prefill cache fill
// k̂ and v of rows (b, t) of the forward's qkv buffer [B*T, H*hd + 2*Hk*hd]
// (q̂, k̂ already normalised and rotated in place) into cache slots
// slot0 + b, positions 0 .. T-1; 16-byte units.
template <class E>
__global__ void __launch_bounds__(256) cache_fill_kernel(const E* __restrict__ qkv, int T, int H, int Hk, int hd,
                                                         E* __restrict__ kc, E* __restrict__ vc, int max_len,
                                                         int slot0, long units) {
  constexpr int P = V16<E>::P;
  const long u = (long)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const int hh = H * hd, hk = Hk * hd, per = hk / P;
  const long row = u / (2 * per);
  const int rem = (int)(u - row * 2 * per);
  const int w = rem / per, e0 = (rem - w * per) * P;
  const int b = (int)(row / T), t = (int)(row - (long)b * T);
  const int h = e0 / hd, e = e0 - h * hd;
  const E* src = qkv + row * (hh + 2 * hk) + hh + w * hk + e0;
  E* dst = (w ? vc : kc) + (((size_t)(slot0 + b) * Hk + h) * max_len + t) * hd + e;
  *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
}

int launch_cache_fill(const void* qkv, int B, int T, int H, int Hk, int hd, void* kc, void* vc, int max_len,
                      int slot0, int dtype, hipStream_t s) {
  const int P = dtype == 0 ? 8 : 4;
  if (hd % P) return NC_ERR_UNSUPPORTED;
  const long units = (long)B * T * 2 * (Hk * hd / P);
  if (units == 0) return 0;
  const unsigned grid = (unsigned)((units + 255) / 256);
  if (dtype == 0)
    cache_fill_kernel<bf16><<<grid, 256, 0, s>>>((const bf16*)qkv, T, H, Hk, hd, (bf16*)kc, (bf16*)vc, max_len,
                                                  slot0, units);
  else
    cache_fill_kernel<float><<<grid, 256, 0, s>>>((const float*)qkv, T, H, Hk, hd, (float*)kc, (float*)vc, max_len,
                                                   slot0, units);
  NC_LAUNCH_CHECK();
  return 0;
}

}  // namespace nc
